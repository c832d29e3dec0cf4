"""GPU prefill (mla_prefill: many new tokens per sequence, un-absorbed; MLA and MLRA-4)
against the fp64 oracle's prefill, which computes the same causal definition as the
multi-token decode (token i at position L - s_q + i sees tokens 0 .. L - s_q + i).  Cases
cover contiguous and paged caches, lengths that are not multiples of the 32-token key tiles,
the 64-token pages or the 256-token query and projection blocks, L < s_q (rows that see
nothing are exactly zero), the default and the sharp query distributions, agreement with
the absorbed decode path at small s_q, and the full-size prefill workloads on sampled rows.
Bounds as for the decode (max-abs 2e-2, rel-L2 1e-2, worst per-row rel-L2 5e-2).
"""

import numpy as np
import pytest

from oracle import mla_oracle as O
from mlra_latent_kv_amd import inputs as I
from test_gpu_parity import assert_close, note

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def built_library():
    import os
    from mlra_latent_kv_amd import binding as B
    if not os.path.exists(B.LIB_PATH):
        from mlra_latent_kv_amd import build
        build.build()
    B.load()


def oracle_prefill(inp, batches=None, heads=None):
    w = inp["workload"]
    return O.mla_prefill(inp["q_nope"], inp["q_rope"], inp["cache"], inp["seqlens"], inp["w_uk"],
                         inp["w_uv"], num_queries=inp["num_queries"], d_rope=w.d_rope,
                         scale=inp["softmax_scale"], out_scale=inp["out_scale"],
                         theta=inp["rope_theta"], page_size=inp["page_size"],
                         block_table=inp["block_table"], to_f64=lambda a: I.to_f64(a, w.dtype),
                         batches=batches, heads=heads)


def gpu_prefill(inp):
    import torch
    from mlra_latent_kv_amd import harness as H
    case = H.to_device(inp, prefill=True)
    out = H.run_prefill(case)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), case


H128 = I.WORKLOADS["mla_bf16_b32_h128_l4096"]
H32P = I.WORKLOADS["mla_bf16_paged_b64_h32_l1k-32k"]
PREFILL = I.PREFILL_WORKLOADS["prefill_bf16_b1_h128_l4096"]

CASES = [
    # (id, workload, s_q, lengths)
    ("h128_contig_sq200", H128, 200, [300, 129]),
    ("h32_paged_sq130", H32P, 130, [700, 64, 1, 130, 257]),
    ("h32_paged_sq1", H32P, 1, [700, 64, 1, 33]),
    ("h128_contig_sq33_tails", H128, 33, [33, 95, 161]),
    ("h32_paged_sq257", H32P, 257, [257, 300, 2]),
]


@pytest.mark.parametrize("cid,w,sq,lens", CASES, ids=[c[0] for c in CASES])
def test_prefill_matches_oracle(cid, w, sq, lens):
    for sharp in (False, True):
        inp = I.make_inputs(w, seed=5, seqlens=lens, num_queries=sq,
                            q_gain=I.sharp_q_gain(w) if sharp else 1.0)
        got, _ = gpu_prefill(inp)
        ref = oracle_prefill(inp)
        assert got.shape == ref.shape == (len(lens), sq * w.heads, w.d_v)
        for b, L in enumerate(lens):
            dead = max(0, sq - L)  # query tokens before the sequence's first token
            assert not got[b, : dead * w.heads].any(), "a token that sees nothing is not zero"
        assert_close(got, ref, "bf16", f"{cid} sharp={sharp}")


@pytest.mark.parametrize("sq", [1, 4, 16])
def test_prefill_agrees_with_absorbed_decode(sq):
    """The un-absorbed prefill and the absorbed multi-token decode compute one definition; on
    the same inputs they agree to within the rounding of their different bf16 operands."""
    import torch
    from mlra_latent_kv_amd import harness as H
    inp = I.make_inputs(H32P, seed=12, seqlens=[640, 70, 17], num_queries=sq,
                        q_gain=I.sharp_q_gain(H32P))
    pre, _ = gpu_prefill(inp)
    case = H.to_device(inp)
    dec = case.run()
    torch.cuda.synchronize()
    dec = dec.float().cpu().numpy().astype(np.float64)
    assert_close(pre, dec, "bf16", f"prefill vs absorbed decode s_q={sq}")
    assert_close(pre, oracle_prefill(inp), "bf16", f"prefill vs oracle s_q={sq}")


ODD = I.Workload("prefill_odd_b3_h5", batch=3, heads=5, branches=1, d_nope=128, d_v=128,
                 d_cb=512, d_rope=64, dtype="bf16", paged=False, seqlen=600, out_scale=0.5, seed=31)
ODD_PAGED = I.Workload("prefill_odd_paged_b2_h7", batch=2, heads=7, branches=1, d_nope=128,
                       d_v=128, d_cb=512, d_rope=64, dtype="bf16", paged=True, seqlen=400, seed=32)


@pytest.mark.parametrize("w,sq,lens", [(ODD, 300, [600, 257, 1]), (ODD_PAGED, 515, [400, 515])],
                         ids=["b3_h5_contig", "b2_h7_paged"])
def test_prefill_head_counts_off_the_grid_groups(w, sq, lens):
    """Head counts and batches whose (sequence, head) pairs do not fill whole groups of eight
    (15 and 14 pairs: the attention grid's padding workgroups return at once), an odd
    out_scale, three query blocks (a lone middle block) and a sequence shorter than s_q."""
    for sharp in (False, True):
        inp = I.make_inputs(w, seed=7, seqlens=lens, num_queries=sq,
                            q_gain=I.sharp_q_gain(w) if sharp else 1.0)
        got, _ = gpu_prefill(inp)
        assert_close(got, oracle_prefill(inp), "bf16", f"{w.name} sq={sq} sharp={sharp}")


MLRA4 = I.WORKLOADS["mlra4_bf16_b32_h32_l8192"]
MLRA4_PAGED = I.Workload("prefill_mlra4_paged_b3_h32", batch=3, heads=32, branches=4, d_nope=128,
                         d_v=128, d_cb=128, d_rope=64, dtype="bf16", paged=True, seqlen=700,
                         out_scale=0.5, seed=33)


@pytest.mark.parametrize("w,sq,lens", [(MLRA4, 200, [300, 129]), (MLRA4, 33, [33, 95, 161]),
                                       (MLRA4_PAGED, 257, [700, 257, 2])],
                         ids=["mlra4_sq200", "mlra4_sq33_tails", "mlra4_paged_sq257"])
def test_prefill_mlra_matches_oracle(w, sq, lens):
    """MLRA-4: four 128-wide branches per head, each with its own up-projected keys and
    values, query and softmax, the shared rotary score, and the scaled branch sum; distinct
    per-branch queries (default and sharp).  The projection's tile loop is uneven here: 384
    and 1152 tiles of 256 tokens over one workgroup per CU (on 256 CUs, 1 or 2 and 4 or 5
    tiles each)."""
    for sharp in (False, True):
        inp = I.make_inputs(w, seed=5, seqlens=lens, num_queries=sq,
                            q_gain=I.sharp_q_gain(w) if sharp else 1.0)
        got, _ = gpu_prefill(inp)
        ref = oracle_prefill(inp)
        assert got.shape == ref.shape == (len(lens), sq * w.heads, w.d_v)
        for b, L in enumerate(lens):
            dead = max(0, sq - L)
            assert not got[b, : dead * w.heads].any(), "a token that sees nothing is not zero"
        assert_close(got, ref, "bf16", f"{w.name} sq={sq} sharp={sharp}")


@pytest.mark.parametrize("sq", [1, 4, 16])
def test_prefill_mlra_agrees_with_absorbed_decode(sq):
    """The un-absorbed MLRA-4 prefill and the absorbed multi-token mlra_decode compute one
    definition."""
    import torch
    from mlra_latent_kv_amd import harness as H
    inp = I.make_inputs(MLRA4, seed=12, seqlens=[640, 70, 17], num_queries=sq,
                        q_gain=I.sharp_q_gain(MLRA4))
    pre, _ = gpu_prefill(inp)
    case = H.to_device(inp)
    dec = case.run()
    torch.cuda.synchronize()
    dec = dec.float().cpu().numpy().astype(np.float64)
    assert_close(pre, dec, "bf16", f"mlra4 prefill vs absorbed decode s_q={sq}")
    assert_close(pre, oracle_prefill(inp), "bf16", f"mlra4 prefill vs oracle s_q={sq}")


def test_prefill_mlra_full_size_sampled():
    """The MLRA-4 prefill workload (one sequence of 4096 new tokens, 32 heads, four branches)
    at full size, sharp queries, on sampled rows across the query blocks and heads."""
    w = I.PREFILL_WORKLOADS["prefill_mlra4_bf16_b1_h32_l4096"]
    inp = I.make_inputs(w, num_queries=w.seqlen, q_gain=I.sharp_q_gain(w))
    got, _ = gpu_prefill(inp)
    tokens = [0, 1, 31, 32, 255, 256, 2047, 2048, 4095]
    heads = [0, 7, 16, 31]
    rows = [i * w.heads + h for i in tokens for h in heads]
    ref = oracle_prefill(inp, heads=rows)
    assert_close(got[:, rows], ref, "bf16", "mlra4 prefill full size sampled")


SHARD = I.WORKLOADS["mlra_shard_bf16_b32_h32_l8192"]


@pytest.mark.parametrize("sq,lens", [(200, [300, 129]), (33, [33, 95, 161])],
                         ids=["shard_sq200", "shard_sq33_tails"])
def test_prefill_mlra_shard_matches_oracle(sq, lens):
    """One MLRA branch cached on its own (rows [c_b (128) | k_rope (64)], the tensor-parallel
    shard), default and sharp queries."""
    for sharp in (False, True):
        inp = I.make_inputs(SHARD, seed=5, seqlens=lens, num_queries=sq,
                            q_gain=I.sharp_q_gain(SHARD) if sharp else 1.0)
        got, _ = gpu_prefill(inp)
        assert_close(got, oracle_prefill(inp), "bf16", f"shard sq={sq} sharp={sharp}")


def test_prefill_mlra_shards_sum_to_mlra4():
    """Tensor-parallel MLRA-4 prefill on one GPU: each branch's prefill on its own, reading its
    [c_b | k_rope] columns out of the MLRA-4 rows (latent pointer offset by 128 b, rotary
    pointer by 512, row stride 576) with its query, W_UK / W_UV blocks and out_scale 0.5, sums
    to the one-call MLRA-4 prefill ("[ICLR 2025] MLRA…", sections 2.1 and 4)."""
    import torch
    from mlra_latent_kv_amd import binding as B
    from mlra_latent_kv_amd import harness as Hn
    from test_gpu_parity import rel_l2
    inp = I.make_inputs(MLRA4, seed=14, seqlens=[300, 77], num_queries=150,
                        q_gain=I.sharp_q_gain(MLRA4))
    full, case = gpu_prefill(inp)
    total = torch.zeros(case.out.shape, dtype=torch.float32, device=case.out.device)
    esz = case.cache.element_size()
    for br in range(4):
        p = case.params.copy()
        p.num_branches, p.d_latent = 1, 128
        ws = torch.empty(B.prefill_workspace_size(p), dtype=torch.uint8, device=case.out.device)
        out = torch.empty_like(case.out)
        qn = case.q_nope[:, :, br:br + 1].contiguous()
        B.mla_prefill(p, qn, case.q_rope, case.cache.data_ptr() + 128 * br * esz,
                      case.cache.data_ptr() + 512 * esz, case.seqlens, None, case.w_uk[br],
                      case.w_uv[br], out, ws)
        torch.cuda.synchronize()
        total += out.float()
    got = total.cpu().numpy().astype(np.float64)
    assert_close(got, oracle_prefill(inp), "bf16", "sum of 4 shard prefills vs oracle")
    assert rel_l2(got, full) < 5e-3, rel_l2(got, full)


def test_prefill_empty_sequences_write_zeros():
    inp = I.make_inputs(H128, seed=3, seqlens=[0, 0], num_queries=40, max_seqlen=64)
    got, _ = gpu_prefill(inp)
    assert not got.any()


def test_prefill_full_size_sampled():
    """The prefill workload (one sequence of 4096 new tokens, 128 heads) at full size, sharp
    queries, on sampled rows: the first and last token, tokens at the 32-, 64- and 128-token
    block edges (256-token query blocks), for heads of every 32-head quarter."""
    w = PREFILL
    inp = I.make_inputs(w, num_queries=w.seqlen, q_gain=I.sharp_q_gain(w))
    got, _ = gpu_prefill(inp)
    tokens = [0, 1, 31, 32, 63, 64, 127, 128, 255, 256, 2047, 2048, 4000, 4095]
    heads = [0, 45, 77, 127]
    rows = [i * w.heads + h for i in tokens for h in heads]
    ref = oracle_prefill(inp, heads=rows)
    note(f"  sampled {len(rows)} rows")
    assert_close(got[:, rows], ref, "bf16", "prefill full size sampled")


def test_prefill_timed_matches_untimed():
    """mla_prefill_timed records its three events around the two kernels and writes the same
    output, bitwise, as mla_prefill; a second call into the same workspace and output (every
    byte of both rewritten) gives the same bytes again."""
    import torch
    import bench
    from mlra_latent_kv_amd import harness as Hn
    inp = I.make_inputs(H32P, seed=21, seqlens=[300, 77], num_queries=150,
                        q_gain=I.sharp_q_gain(H32P))
    case = Hn.to_device(inp, prefill=True)
    plain = Hn.run_prefill(case).clone()
    ev = bench.HipEvents()
    e = ev.create(3)
    stream = torch.cuda.current_stream().cuda_stream
    timed = Hn.run_prefill(case, stream=stream, events=e)
    torch.cuda.synchronize()
    assert torch.equal(plain.view(torch.int16), timed.view(torch.int16))
    proj, attn = ev.ms(e[0], e[1]), ev.ms(e[1], e[2])
    note(f"  projection {1e3 * proj:.1f} us, attention {1e3 * attn:.1f} us")
    assert proj > 0.0 and attn > 0.0
    ev.destroy(e)


def test_prefill_rejects_unsupported():
    """The folded-query form has no prefill (the prefill up-projects keys itself)."""
    from mlra_latent_kv_amd import binding as B
    from mlra_latent_kv_amd import harness as H
    inp = I.make_inputs(MLRA4, seed=1, seqlens=[10], num_queries=4)
    p = H.make_params(inp, flags=B.MLA_FLAG_QUERY_LATENT)
    with pytest.raises(B.MlaError, match="UNSUPPORTED"):
        B.prefill_workspace_size(p)
