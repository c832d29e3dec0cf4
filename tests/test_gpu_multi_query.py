"""GPU decode with several query tokens per sequence (num_queries = s_q > 1) against the fp64
oracle: token i sits at L - s_q + i and attends causally.  The (token, head) rows reach
every kernel family: the fp32 path, the 32-head kernel (MLA, MLRA-4, one MLRA branch) and the
128-row kernel, which s_q = 4 tokens of 32 heads reach as one row quad per work item (one
token per wave).  Lengths include L < s_q (rows that see nothing are zero), L = s_q, page
boundaries, and forced one-page splits, so some work items lie wholly past a token's limit.
Bounds as for one query token (max-abs 2e-2, rel-L2 1e-2 for bf16; 1e-5 for fp32, and the
worst per-row rel-L2).
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


def oracle_multi(inp, batches=None, heads=None, **kw):
    w = inp["workload"]
    return O.mla_decode(inp["q_nope"], inp["q_rope"], inp["cache"], inp["seqlens"], inp["w_uk"],
                        inp["w_uv"], d_rope=w.d_rope, scale=inp["softmax_scale"],
                        out_scale=inp["out_scale"], theta=inp["rope_theta"],
                        page_size=inp["page_size"], block_table=inp["block_table"],
                        to_f64=lambda a: I.to_f64(a, w.dtype), batches=batches, heads=heads,
                        num_queries=inp["num_queries"], **kw)


def gpu_multi(inp, num_splits=0):
    import torch
    from mlra_latent_kv_amd import harness as H
    case = H.to_device(inp, num_splits=num_splits)
    out = case.run()
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), case


F32_MLRA = I.Workload("mlra4_f32_small", batch=1, heads=4, branches=4, d_nope=16, d_v=16, d_cb=16,
                      d_rope=8, dtype="f32", paged=False, seqlen=64, out_scale=0.5, seed=77)

CASES = [
    # (id, workload, s_q, lengths, forced splits)
    ("f32_mla_sq3", I.WORKLOADS["tiny_mla_f32_b1_h4_l64"], 3, [64, 2, 3, 40], 0),
    ("f32_mlra_sq2", F32_MLRA, 2, [64, 1, 33], 0),
    ("paged_h32_sq2", I.WORKLOADS["mla_bf16_paged_b64_h32_l1k-32k"], 2, [300, 1, 2, 65, 777], 0),
    ("paged_h32_sq4_wide", I.WORKLOADS["mla_bf16_paged_b64_h32_l1k-32k"], 4,
     [300, 1, 4, 65, 777, 130], 0),
    ("paged_h32_sq4_wide_page_splits", I.WORKLOADS["mla_bf16_paged_b64_h32_l1k-32k"], 4,
     [65, 129, 66, 3], 3),
    ("h128_sq2_wide", I.WORKLOADS["mla_bf16_b32_h128_l4096"], 2, [700, 1, 2, 130], 0),
    ("h128_sq2_wide_page_splits", I.WORKLOADS["mla_bf16_b32_h128_l4096"], 2, [65, 128, 129], 3),
    ("mlra4_sq2", I.WORKLOADS["mlra4_bf16_b32_h32_l8192"], 2, [513, 1, 2, 200], 0),
    ("mlra4_sq3_page_splits", I.WORKLOADS["mlra4_bf16_b32_h32_l8192"], 3, [65, 130, 2], 3),
    ("shard_sq3", I.WORKLOADS["mlra_shard_bf16_b32_h32_l8192"], 3, [640, 63, 2, 65], 0),
]


@pytest.mark.parametrize("cid,w,sq,lens,splits", CASES, ids=[c[0] for c in CASES])
def test_multi_query_matches_oracle(cid, w, sq, lens, splits):
    for sharp in (False, True):
        inp = I.make_inputs(w, seed=9, seqlens=lens, num_queries=sq,
                            q_gain=I.sharp_q_gain(w) if sharp else 1.0)
        got, _ = gpu_multi(inp, splits)
        ref = oracle_multi(inp)
        assert got.shape == ref.shape == (len(lens), sq * w.heads, w.d_v)
        # rows of tokens that see nothing are exactly zero
        for b, L in enumerate(lens):
            for i in range(sq):
                if L - sq + 1 + i <= 0:
                    assert not np.any(got[b, i * w.heads:(i + 1) * w.heads]), (cid, b, i)
        assert_close(got, ref, w.dtype, f"{cid} {'sharp' if sharp else 'default'}")


@pytest.mark.parametrize("cid", ["paged_h32_sq4_wide", "mlra4_sq2"])
def test_multi_query_negative_controls(cid):
    """The tolerance separates the causal rule from its plausible mistakes: every token
    seeing the whole cache, and token i seeing one token fewer (planted in the oracle)."""
    _, w, sq, lens, splits = next(c for c in CASES if c[0] == cid)
    inp = I.make_inputs(w, seed=9, seqlens=lens, num_queries=sq, q_gain=I.sharp_q_gain(w))
    got, _ = gpu_multi(inp, splits)
    from test_gpu_parity import rel_l2
    # not causal: each token's rows = the one-token decode of the whole cache
    H = w.heads
    full = np.concatenate([O.mla_decode(inp["q_nope"][:, i * H:(i + 1) * H],
                                        inp["q_rope"][:, i * H:(i + 1) * H], inp["cache"],
                                        inp["seqlens"], inp["w_uk"], inp["w_uv"],
                                        d_rope=w.d_rope, scale=inp["softmax_scale"],
                                        out_scale=inp["out_scale"], theta=inp["rope_theta"],
                                        page_size=inp["page_size"],
                                        block_table=inp["block_table"],
                                        to_f64=lambda a: I.to_f64(a, w.dtype))
                           for i in range(sq)], axis=1)
    live = [b for b, L in enumerate(lens) if L > sq]
    d = rel_l2(got[live], full[live])
    note(f"  {cid}: against the non-causal oracle rel_l2={d:.3e}")
    assert d > 0.02
    shorter = dict(inp, seqlens=np.maximum(np.asarray(inp["seqlens"]) - 1, 0))
    d2 = rel_l2(got[live], oracle_multi(shorter)[live])
    note(f"  {cid}: against the one-short oracle rel_l2={d2:.3e}")
    assert d2 > 0.02


def test_multi_query_variants():
    """Several query tokens with the gate and with the folded query (their inputs gain the
    token axis too)."""
    import torch
    from mlra_latent_kv_amd import harness as H
    w = I.WORKLOADS["mlra4_bf16_b32_h32_l8192"]
    inp = I.make_inputs(w, seed=9, seqlens=[513, 2, 200], num_queries=2,
                        q_gain=I.sharp_q_gain(w))
    var = I.make_variant_inputs(inp)
    case = H.to_device(inp)
    dev = case.out.device
    g = H.run_variant(case, gate=H._to_dev(var["gate"], w.dtype, dev))
    q = H.run_variant(case, q_latent=H._to_dev(var["q_latent"], w.dtype, dev), latent_out=True)
    torch.cuda.synchronize()
    f = lambda t: t.float().cpu().numpy().astype(np.float64)
    assert_close(f(g), oracle_multi(inp, gate=var["gate"]), "bf16", "mlra4 s_q=2 gated")
    ref_q = O.mla_decode(var["q_latent"], inp["q_rope"], inp["cache"], inp["seqlens"], None, None,
                         d_rope=64, scale=inp["softmax_scale"], out_scale=0.5, theta=1e4,
                         to_f64=lambda a: I.to_f64(a, "bf16"), q_latent=True, latent_out=True,
                         branches=4, d_cb=128, num_queries=2)
    from test_gpu_variants import check
    check(f(q), ref_q, "bf16", "mlra4 s_q=2 folded query + latent output")


def test_multi_query_full_size_sampled():
    """The paged variable-length workload (64 sequences of 1k-32k tokens, H = 32) with s_q = 4
    query tokens, sharp query: 128 query rows per sequence run on the 128-row kernel, one
    token per wave.  Sampled rows of every token, the longest and the shortest sequence."""
    w = I.WORKLOADS["mla_bf16_paged_b64_h32_l1k-32k"]
    note("  generating mla_bf16_paged_b64_h32_l1k-32k with 4 query tokens")
    inp = I.make_inputs(w, num_queries=4, q_gain=I.sharp_q_gain(w))
    lens = [int(x) for x in inp["seqlens"]]
    bs = [0, int(np.argmax(lens)), int(np.argmin(lens)), 40]
    hs = [0, 31, 32, 63, 64, 95, 96, 127]
    got, _ = gpu_multi(inp)
    ref = oracle_multi(inp, batches=bs, heads=hs)
    assert np.all(np.isfinite(got))
    assert_close(got[np.ix_(bs, hs)], ref, "bf16", "paged varlen s_q=4 full size")
