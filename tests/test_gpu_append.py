"""GPU cache append (mla_cache_append) against the fp64 write-side oracle.

Rows: each element is an fp32-accumulated dot product over d_model, rounded once to bf16
(the rotary part also turned through an fp32 rotation), so it must lie within one bf16 step
of the fp64 value: |gpu - ref| <= 2^-8 |ref| + 1e-6 max|row|.  Lengths, block-table entries
and the page count are integers and must match exactly; every cache row the append does not
write must be bit-identical before and after.  The end-to-end case appends a sequence's
tokens one decode step at a time on the GPU and then decodes on the GPU, against the oracle's
append and decode of the same tokens.
"""

import math

import numpy as np
import pytest

from oracle import mla_oracle as O
from mlra_latent_kv_amd import inputs as I

pytestmark = pytest.mark.gpu


def note(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module", autouse=True)
def built_library():
    import os
    from mlra_latent_kv_amd import binding as B
    if not os.path.exists(B.LIB_PATH):
        from mlra_latent_kv_amd import build
        build.build()
    B.load()


def _dev(a, dtype="bf16"):
    import torch
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _params(B, d_model, dc, row, paged, max_pages=0, capacity=0, bt_stride=0):
    from mlra_latent_kv_amd import binding as Bd
    p = Bd.MlaAppendParams()
    p.batch, p.d_model, p.d_latent, p.d_rope = B, d_model, dc, 64
    p.page_size = 64 if paged else 0
    p.max_pages_per_seq, p.capacity, p.dtype = max_pages, capacity, Bd.MLA_BF16
    p.latent_stride_tok = p.rope_stride_tok = row
    p.latent_stride_seq = p.rope_stride_seq = row * (64 if paged else capacity)
    p.block_table_stride = bt_stride
    p.rope_theta = 10000.0
    return p


def run_append(inp, seqlens, cache, block_table, free, paged, dc):
    """The GPU append on copies of the given state; returns (cache, seqlens, block_table,
    pages_used) read back."""
    import torch
    from mlra_latent_kv_amd import binding as Bd
    B, d_model = inp["hidden"].shape
    row = dc + 64
    c = _dev(cache)
    sl = torch.tensor(np.asarray(seqlens, np.int32), device="cuda")
    bt = None if block_table is None else torch.tensor(np.asarray(block_table, np.int32), device="cuda")
    fr = torch.tensor(np.asarray(free, np.int32) if len(free) else np.zeros(1, np.int32), device="cuda")
    used = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    p = _params(B, d_model, dc, row, paged, max_pages=0 if bt is None else bt.shape[1],
                capacity=0 if paged else cache.shape[1],
                bt_stride=0 if bt is None else bt.shape[1])
    ws = torch.empty(Bd.append_workspace_size(p), dtype=torch.uint8, device="cuda")
    Bd.mla_cache_append(p, _dev(inp["hidden"]), _dev(inp["w_dkv"]), _dev(inp["w_kr"]),
                        c.data_ptr(), c.data_ptr() + dc * 2, sl, bt, fr, len(free), used, ws)
    torch.cuda.synchronize()
    return (c.view(torch.int16).cpu().numpy().view(np.uint16), sl.cpu().numpy(),
            None if bt is None else bt.cpu().numpy(), int(used.item()))


def check_against_oracle(inp, seqlens, cache, block_table, free, paged, dc, what):
    got_cache, got_len, got_bt, got_used = run_append(inp, seqlens, cache, block_table, free,
                                                      paged, dc)
    ref = O.cache_append(I.to_f64(inp["hidden"], "bf16"), I.to_f64(inp["w_dkv"], "bf16"),
                         I.to_f64(inp["w_kr"], "bf16"), seqlens, block_table, free,
                         theta=10000.0, page_size=64 if paged else 0,
                         capacity=None if paged else cache.shape[1])
    assert np.array_equal(got_len, ref["seqlens"]), (what, got_len, ref["seqlens"])
    assert got_used == ref["pages_used"], (what, got_used, ref["pages_used"])
    if paged:
        assert np.array_equal(got_bt, ref["block_table"]), what
    touched = np.zeros(cache.shape[:2], bool)
    worst = 0.0
    for b, wh in enumerate(ref["where"]):
        if wh is None:
            continue
        touched[wh] = True
        g = I.to_f64(got_cache[wh], "bf16")
        r = ref["rows"][b]
        err = np.abs(g - r)
        bound = 2.0 ** -8 * np.abs(r) + 1e-6 * np.abs(r).max()
        assert np.all(err <= bound), (what, b, float((err / np.maximum(bound, 1e-300)).max()))
        worst = max(worst, float((err / np.maximum(np.abs(r), 1e-30)).max()))
    assert np.array_equal(got_cache[~touched], cache[~touched]), (what, "a row not written changed")
    note(f"  {what}: {int(touched.sum())} rows written, pages used {got_used}, "
         f"worst relative element error {worst:.2e}")


@pytest.mark.parametrize("dc", [512, 128], ids=["latent512", "latent128"])
@pytest.mark.parametrize("d_model", [256, 4096])
def test_append_paged_matches_oracle(d_model, dc):
    """Sequences whose token starts a page (t = 0, 64, 128), ends one (t = 63) or sits
    mid-page, with a shuffled free list: once with pages to spare and once with too few (the
    last sequences that need a page are left untouched)."""
    rng = np.random.default_rng(d_model + dc)
    lens = [0, 5, 64, 63, 128, 700, 1, 191, 192, 33] * 4
    B = len(lens)
    inp = I.make_append_inputs(d_model, dc, B, seed=11 + dc)
    row = dc + 64
    max_pages = 12
    P = 220
    perm = rng.permutation(P)
    bt = np.full((B, max_pages), -1, np.int64)
    k = 0
    for b, L in enumerate(lens):  # pages already holding tokens 0 .. L-1
        for j in range(-(-L // 64)):
            bt[b, j] = perm[k]
            k += 1
    cache = I.to_storage(rng.standard_normal((P, 64, row)).astype(np.float32), "bf16")
    free = list(perm[k:])
    need = sum(1 for L in lens if L % 64 == 0)
    check_against_oracle(inp, lens, cache, bt, free, True, dc, f"paged d_model={d_model} dc={dc}")
    check_against_oracle(inp, lens, cache, bt, free[:need - 3], True, dc,
                         f"paged d_model={d_model} dc={dc}, 3 pages short")


def test_append_contiguous_matches_oracle():
    """Contiguous cache [B, capacity, row]: rows go to (b, t); a full sequence is untouched."""
    rng = np.random.default_rng(3)
    lens = [0, 1, 31, 32, 99, 100, 63]
    cap = 100
    inp = I.make_append_inputs(512, 512, len(lens), seed=5)
    cache = I.to_storage(rng.standard_normal((len(lens), cap, 576)).astype(np.float32), "bf16")
    check_against_oracle(inp, lens, cache, None, [], False, 512, "contiguous")


def test_append_batch_of_one_and_no_free_pages():
    rng = np.random.default_rng(4)
    inp = I.make_append_inputs(256, 512, 1, seed=6)
    cache = I.to_storage(rng.standard_normal((4, 64, 576)).astype(np.float32), "bf16")
    bt = np.full((1, 4), -1, np.int64)
    check_against_oracle(inp, [0], cache, bt, [], True, 512, "B=1, empty free list")
    check_against_oracle(inp, [0], cache, bt, [2], True, 512, "B=1, one free page")


@pytest.mark.parametrize("wname", ["mla_bf16_paged_b64_h32_l1k-32k", "mlra4_bf16_b32_h32_l8192"])
def test_append_steps_then_decode(wname):
    """End to end on the GPU: three sequences start empty in a shuffled pool; each decode step
    appends one token per sequence with mla_cache_append (pages taken from the free list as
    they fill), for 150 steps, then the decode step reads the cache.  Against the oracle's
    append of the same tokens (its stored rotary keys turned back to raw keys, as the decode
    oracle takes them) and its decode."""
    import torch
    from mlra_latent_kv_amd import binding as Bd
    w = I.WORKLOADS[wname]
    B, steps, d_model = 3, 150, 512
    rng = np.random.default_rng(9)
    pool_pages = 12
    free = list(rng.permutation(pool_pages))
    row = w.row
    pool = torch.zeros((pool_pages, 64, row), dtype=torch.bfloat16, device="cuda")
    bt = torch.full((B, 4), -1, dtype=torch.int32, device="cuda")
    sl = torch.zeros(B, dtype=torch.int32, device="cuda")
    fr = torch.tensor(np.asarray(free, np.int32), device="cuda")
    used = torch.zeros(1, dtype=torch.int32, device="cuda")
    p = _params(B, d_model, w.d_c, row, True, max_pages=4, bt_stride=4)
    ws = torch.empty(Bd.append_workspace_size(p), dtype=torch.uint8, device="cuda")
    hs = [I.make_append_inputs(d_model, w.d_c, B, seed=100 + s) for s in range(steps)]
    wdk, wkr = _dev(hs[0]["w_dkv"]), _dev(hs[0]["w_kr"])
    head = 0
    for s in range(steps):
        Bd.mla_cache_append(p, _dev(hs[s]["hidden"]), wdk, wkr, pool.data_ptr(),
                            pool.data_ptr() + w.d_c * 2, sl, bt, fr[head:], len(free) - head,
                            used, ws)
        head += int(used.item())
    assert sl.cpu().tolist() == [steps] * B
    # the decode step over the GPU-written cache
    dec = I.make_inputs(w, seqlens=[steps] * B, q_gain=I.sharp_q_gain(w))
    from mlra_latent_kv_amd import harness as Hn
    dp = Hn.make_params(dec)
    dp.page_size, dp.max_pages_per_seq, dp.block_table_stride = 64, 4, 4
    dp.latent_stride_seq = dp.rope_stride_seq = 64 * row
    dp.num_pages = pool_pages
    out = torch.empty((B, w.heads, w.d_v), dtype=torch.bfloat16, device="cuda")
    dws = torch.empty(Bd.workspace_size(dp), dtype=torch.uint8, device="cuda")
    fn = Bd.mlra_decode if w.branches == 4 else Bd.mla_decode
    fn(dp, _dev(dec["q_nope"]), _dev(dec["q_rope"]), pool.data_ptr(), pool.data_ptr() + w.d_c * 2,
       sl, bt, _dev(dec["w_uk"]), _dev(dec["w_uv"]), out, dws)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    # the oracle's side: its own append of the same tokens, then its decode on raw keys
    f64 = lambda a: I.to_f64(a, "bf16")
    raw = np.zeros((B, steps, row))
    for s in range(steps):
        r = O.cache_append(f64(hs[s]["hidden"]), f64(hs[0]["w_dkv"]), f64(hs[0]["w_kr"]),
                           [s] * B, capacity=steps)
        rows = r["rows"]
        rows[:, w.d_c:] = O.rope(rows[:, w.d_c:], -s, w.rope_theta)  # back to the raw key
        raw[:, s] = rows
    ref = O.mla_decode(dec["q_nope"], dec["q_rope"], raw, [steps] * B, dec["w_uk"], dec["w_uv"],
                       d_rope=w.d_rope, scale=w.softmax_scale, out_scale=w.out_scale,
                       theta=w.rope_theta, to_f64=lambda a: f64(a) if a.dtype == np.uint16 else a)
    err = float(np.abs(got - ref).max())
    rel = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
    note(f"  {wname}: append x{steps} then decode: max_abs={err:.3e} rel_l2={rel:.3e}")
    assert err <= 2e-2 and rel <= 1e-2


# ----------------------------------------------------------------------------- fp8 latent
# A cache whose latent part is OCP FP8 E4M3 codes (MLA_LATENT_FP8): the append encodes each
# latent element as the nearest code of value / scale (ties to even, saturating).  The GPU row
# is accumulated in fp32, so at a rounding tie its code may be the neighbour of the code of
# the fp64 value; every code must be one of the two codes around the exact value, and almost
# all must be the nearest.

def _run_append_fp8(inp, seqlens, lat8, rope16, block_table, free, paged, dc, scale):
    import torch
    from mlra_latent_kv_amd import binding as Bd
    B, d_model = inp["hidden"].shape
    l8 = torch.from_numpy(np.ascontiguousarray(lat8)).cuda()
    r = _dev(rope16)
    sl = torch.tensor(np.asarray(seqlens, np.int32), device="cuda")
    bt = None if block_table is None else torch.tensor(np.asarray(block_table, np.int32), device="cuda")
    fr = torch.tensor(np.asarray(free, np.int32) if len(free) else np.zeros(1, np.int32), device="cuda")
    used = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    rows = 64 if paged else lat8.shape[1]
    p = _params(B, d_model, dc, dc + 64, paged, max_pages=0 if bt is None else bt.shape[1],
                capacity=0 if paged else lat8.shape[1], bt_stride=0 if bt is None else bt.shape[1])
    p.latent_stride_tok, p.latent_stride_seq = dc, dc * rows
    p.rope_stride_tok, p.rope_stride_seq = 64, 64 * rows
    p.latent_format, p.latent_scale = Bd.MLA_LATENT_FP8, scale
    ws = torch.empty(Bd.append_workspace_size(p), dtype=torch.uint8, device="cuda")
    Bd.mla_cache_append(p, _dev(inp["hidden"]), _dev(inp["w_dkv"]), _dev(inp["w_kr"]),
                        l8.data_ptr(), r.data_ptr(), sl, bt, fr, len(free), used, ws)
    torch.cuda.synchronize()
    return (l8.cpu().numpy(), r.view(torch.int16).cpu().numpy().view(np.uint16), sl.cpu().numpy(),
            None if bt is None else bt.cpu().numpy(), int(used.item()))


def _check_codes(got_codes, exact, scale, what):
    grid = I.e4m3_bits_to_f64(np.arange(0x7f, dtype=np.uint8))
    want = I.f64_to_e4m3_bits(exact / scale)
    got_v = I.e4m3_bits_to_f64(got_codes)
    want_v = I.e4m3_bits_to_f64(want)
    a = np.minimum(np.abs(exact / scale), 448.0)
    lo = grid[np.clip(np.searchsorted(grid, a, side="right") - 1, 0, 0x7e)]
    hi = grid[np.clip(np.searchsorted(grid, a, side="left"), 0, 0x7e)]
    mag = np.abs(got_v)
    assert np.all((mag == lo) | (mag == hi)), (what, "a code outside the two around the value")
    assert np.all((got_v == 0) | (np.sign(got_v) == np.sign(exact))), (what, "sign")
    frac = float(np.mean(got_v == want_v))
    note(f"  {what}: {got_codes.size} codes, nearest code in {100 * frac:.3f} %")
    assert frac > 0.99


@pytest.mark.parametrize("paged", [True, False], ids=["paged", "contiguous"])
def test_append_fp8_latent_matches_oracle(paged):
    rng = np.random.default_rng(21)
    dc = 512
    lens = [0, 5, 64, 63, 128, 1, 191, 33] * 2
    B = len(lens)
    inp = I.make_append_inputs(4096, dc, B, seed=31)
    scale = 0.01
    if paged:
        max_pages, P = 4, 60
        perm = rng.permutation(P)
        bt = np.full((B, max_pages), -1, np.int64)
        k = 0
        for b, L in enumerate(lens):
            for j in range(-(-L // 64)):
                bt[b, j] = perm[k]
                k += 1
        free, rows_shape = list(perm[k:]), (P, 64)
    else:
        bt, free, rows_shape = None, [], (B, 200)
    lat8 = rng.integers(0, 0x7e, size=rows_shape + (dc,), dtype=np.uint8)
    rope16 = I.to_storage(rng.standard_normal(rows_shape + (64,)).astype(np.float32), "bf16")
    got8, got_r, got_len, got_bt, got_used = _run_append_fp8(inp, lens, lat8, rope16, bt, free,
                                                             paged, dc, scale)
    ref = O.cache_append(I.to_f64(inp["hidden"], "bf16"), I.to_f64(inp["w_dkv"], "bf16"),
                         I.to_f64(inp["w_kr"], "bf16"), lens, bt, free, theta=10000.0,
                         page_size=64 if paged else 0, capacity=None if paged else rows_shape[1])
    assert np.array_equal(got_len, ref["seqlens"]) and got_used == ref["pages_used"]
    if paged:
        assert np.array_equal(got_bt, ref["block_table"])
    touched = np.zeros(rows_shape, bool)
    codes, exact = [], []
    for b, wh in enumerate(ref["where"]):
        if wh is None:
            continue
        touched[wh] = True
        codes.append(got8[wh])
        exact.append(ref["rows"][b][:dc])
        r = ref["rows"][b][dc:]
        g = I.to_f64(got_r[wh], "bf16")
        assert np.all(np.abs(g - r) <= 2.0 ** -8 * np.abs(r) + 1e-6 * np.abs(r).max())
    _check_codes(np.stack(codes), np.stack(exact), scale, f"fp8 append {'paged' if paged else 'contiguous'}")
    assert np.array_equal(got8[~touched], lat8[~touched]) and np.array_equal(got_r[~touched], rope16[~touched])


def test_append_fp8_steps_then_decode():
    """150 decode steps appended into an fp8-latent pool on the GPU, then the GPU decode of
    that cache; against the oracle's append of the same tokens, its latent encoded with the
    same scale by the host encoder, and its decode on the decoded values."""
    import torch
    from mlra_latent_kv_amd import binding as Bd
    from mlra_latent_kv_amd import harness as Hn
    w = I.WORKLOADS["mla_bf16_paged_b64_h32_l1k-32k"]
    B, steps, d_model, dc = 3, 150, 512, 512
    scale = 0.005
    rng = np.random.default_rng(9)
    pool_pages = 12
    free = list(rng.permutation(pool_pages))
    lat8 = torch.zeros((pool_pages, 64, dc), dtype=torch.uint8, device="cuda")
    rope = torch.zeros((pool_pages, 64, 64), dtype=torch.bfloat16, device="cuda")
    bt = torch.full((B, 4), -1, dtype=torch.int32, device="cuda")
    sl = torch.zeros(B, dtype=torch.int32, device="cuda")
    fr = torch.tensor(np.asarray(free, np.int32), device="cuda")
    used = torch.zeros(1, dtype=torch.int32, device="cuda")
    p = _params(B, d_model, dc, dc + 64, True, max_pages=4, bt_stride=4)
    p.latent_stride_tok, p.latent_stride_seq = dc, dc * 64
    p.rope_stride_tok, p.rope_stride_seq = 64, 64 * 64
    p.latent_format, p.latent_scale = Bd.MLA_LATENT_FP8, scale
    ws = torch.empty(Bd.append_workspace_size(p), dtype=torch.uint8, device="cuda")
    hs = [I.make_append_inputs(d_model, dc, B, seed=300 + s) for s in range(steps)]
    wdk, wkr = _dev(hs[0]["w_dkv"]), _dev(hs[0]["w_kr"])
    head = 0
    for s in range(steps):
        Bd.mla_cache_append(p, _dev(hs[s]["hidden"]), wdk, wkr, lat8.data_ptr(), rope.data_ptr(),
                            sl, bt, fr[head:], len(free) - head, used, ws)
        head += int(used.item())
    dec = I.make_inputs(w, seqlens=[steps] * B, q_gain=I.sharp_q_gain(w))
    dp = Hn.make_params(dec)
    dp.page_size, dp.max_pages_per_seq, dp.block_table_stride = 64, 4, 4
    dp.latent_stride_tok, dp.latent_stride_seq = dc, dc * 64
    dp.rope_stride_tok, dp.rope_stride_seq = 64, 64 * 64
    dp.num_pages = pool_pages
    dp.latent_format, dp.latent_scale = Bd.MLA_LATENT_FP8, scale
    out = torch.empty((B, w.heads, w.d_v), dtype=torch.bfloat16, device="cuda")
    dws = torch.empty(Bd.workspace_size(dp), dtype=torch.uint8, device="cuda")
    Bd.mla_decode(dp, _dev(dec["q_nope"]), _dev(dec["q_rope"]), lat8.data_ptr(), rope.data_ptr(),
                  sl, bt, _dev(dec["w_uk"]), _dev(dec["w_uv"]), out, dws)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    f64 = lambda a: I.to_f64(a, "bf16")
    raw = np.zeros((B, steps, dc + 64))
    for s in range(steps):
        r = O.cache_append(f64(hs[s]["hidden"]), f64(hs[0]["w_dkv"]), f64(hs[0]["w_kr"]),
                           [s] * B, capacity=steps)
        rows = r["rows"]
        rows[:, :dc] = I.e4m3_bits_to_f64(I.f64_to_e4m3_bits(rows[:, :dc] / scale)) * scale
        rows[:, dc:] = O.rope(rows[:, dc:], -s, w.rope_theta)  # back to the raw key
        raw[:, s] = rows
    ref = O.mla_decode(dec["q_nope"], dec["q_rope"], raw, [steps] * B, dec["w_uk"], dec["w_uv"],
                       d_rope=64, scale=w.softmax_scale, out_scale=w.out_scale,
                       theta=w.rope_theta, to_f64=lambda a: f64(a) if a.dtype == np.uint16 else a)
    err = float(np.abs(got - ref).max())
    rel = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
    note(f"  fp8 append x{steps} then decode: max_abs={err:.3e} rel_l2={rel:.3e}")
    assert err <= 2e-2 and rel <= 1e-2
