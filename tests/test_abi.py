"""C-ABI library: loads, exports every declared symbol, and rejects bad arguments on the host
(each call below fails validation before any HIP call, so no GPU is needed)."""

import ctypes
import os
import subprocess

import pytest

from mlra_latent_kv_amd import binding as B
from mlra_latent_kv_amd import inputs as I
from mlra_latent_kv_amd.harness import make_params

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        from mlra_latent_kv_amd import build
        build.build()
    return B.load()


def test_exports_every_declared_symbol(lib):
    declared = B.header_functions()
    assert set(declared) == {"mla_workspace_size", "mla_num_splits", "mla_decode", "mlra_decode",
                             "mla_decode_timed", "mlra_decode_timed", "mla_rope_rotate",
                             "mla_status_str"}
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    for name in declared:
        assert name in exported, name
        assert hasattr(lib, name)


def test_params_struct_layout_matches_header():
    # 12 int32, 5 int64, 3 float -> 48 + 40 + 12 = 100, padded to 104
    assert ctypes.sizeof(B.MlaParams) == 104
    assert B.MlaParams.latent_stride_tok.offset == 48
    assert B.MlaParams.softmax_scale.offset == 88


def params_for(wname, **over):
    w = I.WORKLOADS[wname]
    inp = I.make_inputs(w, seqlens=[5, 7])
    p = make_params(inp)
    for k, v in over.items():
        setattr(p, k, v)
    return p


FAKE = 1 << 20  # non-NULL, 256-aligned; never dereferenced because validation fails first


def call(lib, p, fn="mla_decode", ws_bytes=1 << 40, **ptr):
    args = dict(q_nope=FAKE, q_rope=FAKE, latent=FAKE, rope=FAKE, seqlens=FAKE, block_table=FAKE,
                w_uk=FAKE, w_uv=FAKE, out=FAKE, workspace=FAKE)
    args.update(ptr)
    return getattr(lib, fn)(ctypes.byref(p), *args.values(), ws_bytes, None)


@pytest.mark.parametrize("over,status", [
    (dict(dtype=7), 5),
    (dict(batch=0), 2),
    (dict(d_rope=63), 2),
    (dict(max_seqlen=-1), 2),
    (dict(num_splits=-2), 2),
    (dict(page_size=16), 3),
    (dict(d_latent=256), 3),
    (dict(num_heads=48), 3),
    (dict(d_nope=64), 3),
    (dict(latent_stride_tok=500), 2),
    (dict(latent_stride_tok=580), 6),
    (dict(softmax_scale=float("nan")), 2),
    (dict(rope_theta=0.0), 2),
    (dict(num_splits=1000), 2),
])
def test_invalid_params_rejected(lib, over, status):
    p = params_for("mla_bf16_b32_h128_l4096", **over)
    assert call(lib, p) == status
    n = ctypes.c_size_t(0)
    st = lib.mla_workspace_size(ctypes.byref(p), ctypes.byref(n))
    assert st == status or (status in (1, 4, 6) and st == 0)


def test_branch_count_per_entry_point(lib):
    assert call(lib, params_for("mla_bf16_b32_h128_l4096"), fn="mlra_decode") == 3
    assert call(lib, params_for("mlra4_bf16_b32_h32_l8192"), fn="mla_decode") == 3


@pytest.mark.parametrize("name", ["q_nope", "q_rope", "latent", "rope", "seqlens", "w_uk", "w_uv",
                                  "out", "workspace"])
def test_null_pointer_rejected(lib, name):
    assert call(lib, params_for("mla_bf16_b32_h128_l4096"), **{name: None}) == 1


def test_paged_needs_block_table(lib):
    p = params_for("mla_bf16_paged_b64_h32_l1k-32k")
    assert call(lib, p, block_table=None) == 1
    p.max_pages_per_seq = 0
    assert call(lib, p) == 2


def test_workspace_and_alignment(lib):
    p = params_for("mla_bf16_b32_h128_l4096")
    need = B.workspace_size(p)
    assert call(lib, p, ws_bytes=need - 1) == 4
    assert call(lib, p, latent=FAKE + 8) == 6
    assert call(lib, p, workspace=FAKE + 64) == 6
    assert call(lib, p, w_uk=FAKE + 2) == 6     # bf16 weights need 16-byte alignment


def test_rope_rotate_validation(lib):
    f = lib.mla_rope_rotate
    assert f(FAKE, 64, FAKE, 10, 63, 1e4, 1, None) == 2
    assert f(FAKE, 32, FAKE, 10, 64, 1e4, 1, None) == 2
    assert f(FAKE, 64, FAKE, 10, 64, 1e4, 3, None) == 5
    assert f(None, 64, FAKE, 10, 64, 1e4, 1, None) == 1
    assert f(None, 64, None, 0, 64, 1e4, 1, None) == 0     # empty: nothing to do
    assert f(FAKE + 1, 64, FAKE, 10, 64, 1e4, 1, None) == 6


def test_status_strings(lib):
    for s in range(8):
        assert lib.mla_status_str(s).decode().startswith(B.STATUS[s])
    assert lib.mla_status_str(99).decode() == "unknown mla_status"


@pytest.mark.parametrize("wname", I.WORKLOAD_ORDER)
@pytest.mark.parametrize("forced", [0, 3])
def test_workspace_layout(lib, wname, forced):
    w = I.WORKLOADS[wname]
    lens = [w.seqlen] * 3
    inp = I.make_inputs(w, seqlens=[1, 2, 3]) if w.seqlen > 5000 else I.make_inputs(w, seqlens=lens)
    p = make_params(inp)
    p.max_seqlen = w.seqlen
    pages = (w.seqlen + 63) // 64
    if w.paged:
        p.max_pages_per_seq = p.block_table_stride = pages
    forced = min(forced, pages)
    p.num_splits = forced
    S = B.num_splits(p)
    wide = w.dtype == "bf16" and w.branches == 1 and w.heads % 128 == 0
    wg_per_item = w.heads // 128 if wide else w.heads // 32 if w.dtype == "bf16" else w.heads
    target = max(1, -(-(256 if wide else 512) // wg_per_item))
    Bn, H, dc = 3, w.heads, w.d_c
    if forced:
        assert S == -(-pages // -(-pages // forced))
        cap = Bn * S
    else:
        assert S == min(pages, target)
        cap = max(target, Bn)
    slots = -(-cap // 8) * 8
    al = lambda x: (x + 255) // 256 * 256
    # plan (header, dispatch table, split offsets), queries, per-item partials (element type
    # on the bf16 path), (m, l) in fp32, and the fp32 merged latent
    exp = al(16 + 16 * slots + 4 * (Bn + 1)) + al(Bn * H * w.row * w.elem_bytes) + \
        al(cap * H * dc * w.elem_bytes) + al(cap * w.branches * H * 2 * 4) + \
        (al(Bn * H * dc * 4) if w.elem_bytes == 4 else 0)
    assert B.workspace_size(p) == exp


def test_split_bounds(lib):
    # bf16 MLA with H % 128 == 0: one workgroup per (work item, 128 heads), 256 items target
    p = params_for("mla_bf16_b32_h128_l4096", batch=32, max_seqlen=4096)
    assert B.num_splits(p) == 64         # one sequence may take up to all of its 64 pages
    p = params_for("mla_bf16_paged_b4_h128_l131072", batch=4, max_seqlen=131072,
                   max_pages_per_seq=2048, block_table_stride=2048)
    assert B.num_splits(p) == 256        # bounded by the item target
    p.num_splits = 7
    assert B.num_splits(p) == 7
    p.num_splits = 600                   # 4 pages per item: 512 items
    assert B.num_splits(p) == 512
    p.num_splits = 1000                  # 3 pages per item: 683 > 512 items
    with pytest.raises(B.MlaError):
        B.num_splits(p)
    # 32-head groups (two workgroups per CU): 512 items target
    p = params_for("mla_bf16_paged_b64_h32_l1k-32k", batch=64, max_seqlen=32768,
                   max_pages_per_seq=512, block_table_stride=512)
    assert B.num_splits(p) == 512
    p = params_for("mlra4_bf16_b32_h32_l8192", batch=32, max_seqlen=8192)
    assert B.num_splits(p) == 128
    p.num_splits = 129                   # more splits than pages
    with pytest.raises(B.MlaError):
        B.num_splits(p)


def test_plan_code_under_host_sanitizers(tmp_path):
    exe = tmp_path / "plan_fuzz"
    src = [os.path.join(ROOT, "tests", "plan_fuzz.cpp"),
           os.path.join(ROOT, "mlra_latent_kv_amd", "csrc", "plan.cpp")]
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "mlra_latent_kv_amd", "csrc"), *src, "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "accepted" in r.stdout


def test_plan_checker_rejects_wrong_plans():
    """The GPU tests judge the device's split plan with test_gpu_parity.check_plan; here that
    checker is shown to reject plans with a plausible mistake (pages per item one too many or
    one too few, a shifted item, a wrong split offset, a missed empty slot), on a plan built
    from its definition."""
    import numpy as np
    from test_gpu_parity import check_plan
    w = I.WORKLOADS["mla_bf16_b32_h128_l4096"]          # wide kernel: XCD-major slots
    lens = [0, 1, 64, 65, 4000, 0, 129, 3000, 77, 2048]
    target, slots, max_seqlen = 256, 256, 4000

    def build(c, forced=0):
        pages = [-(-min(L, max_seqlen) // 64) for L in lens]
        n = [-(-p // c) for p in pages]
        so = np.concatenate([[0], np.cumsum(n)]).astype(np.int64)
        W = int(so[-1]); per = -(-W // 8)
        work = np.full((slots, 4), -1, np.int64)
        work[:, 1:3] = 0
        for s_ in range(slots):
            x, g = s_ % 8, s_ // 8
            item = x * per + g if g < per else W
            if item < W:
                b = int(np.searchsorted(so, item, side="right") - 1)
                t0 = (item - so[b]) * c * 64
                work[s_] = (b, t0, min(lens[b], t0 + c * 64), item)
        return {"items": W, "pages": c, "slots": slots, "target": 0 if forced else target,
                "work": work, "split_off": so}

    good = build(1)                                      # 151 pages fit 256 items at c = 1
    check_plan(good, w, lens, max_seqlen, 0)
    check_plan(build(13, forced=5), w, lens, max_seqlen, 5)  # ceil(63 / 5) pages per item
    bad = []
    bad.append(build(2))                                 # not the smallest fitting c
    bad.append(build(12, forced=5))                      # forced page count off by one
    p = build(1); p["work"] = p["work"].copy(); p["work"][0, 1] += 64; bad.append(p)
    p = build(1); p["split_off"] = p["split_off"].copy(); p["split_off"][3] += 1; bad.append(p)
    p = build(1); p["work"] = p["work"].copy()
    p["work"][np.where(p["work"][:, 0] < 0)[0][0]] = (0, 0, 1, 0); bad.append(p)
    for i, p in enumerate(bad):
        with pytest.raises(AssertionError):
            check_plan(p, w, lens, max_seqlen, 5 if i == 1 else 0)
