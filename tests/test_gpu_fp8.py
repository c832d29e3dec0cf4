"""GPU decode over an fp8 latent cache (MLA_LATENT_FP8: OCP E4M3 codes with one per-tensor
scale, the rotary key in bf16) against the fp64 oracle run on the values that cache holds
(decoded codes times the scale).  The kernels widen the codes to bf16 exactly and fold the
scale into the query and output scales, so the bound is the bf16 one (max-abs 2e-2, rel-L2
1e-2, worst row 5e-2): the quantisation error of the cache itself lies in the inputs, not in
the comparison.  Covers the 32-head kernel's three shapes (MLA, MLRA-4, one MLRA branch), 128
heads (which the fp8 latent runs on the 32-head kernel), paged and contiguous caches, ragged
and one-page splits, several query tokens, the gate, and the paged variable-length workload at
full size on sampled outputs.
"""

import numpy as np
import pytest

from oracle import mla_oracle as O
from mlra_latent_kv_amd import inputs as I
from test_gpu_parity import assert_close, note, rel_l2

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def built_library():
    import os
    from mlra_latent_kv_amd import binding as B
    if not os.path.exists(B.LIB_PATH):
        from mlra_latent_kv_amd import build
        build.build()
    B.load()


def _f64(a):
    return a if a.dtype == np.float64 else I.to_f64(a, "bf16")


def oracle_fp8(inp, batches=None, heads=None, latent_scale=None, **kw):
    """The oracle on the cache's values (latent = decoded codes x scale, rotary key bf16)."""
    w = inp["workload"]
    cache = I.oracle_cache(inp)
    if latent_scale is not None:  # a planted wrong scale
        cache[..., :w.d_c] *= latent_scale / inp["latent_scale"]
    return O.mla_decode(inp["q_nope"], inp["q_rope"], cache, inp["seqlens"], inp["w_uk"],
                        inp["w_uv"], d_rope=w.d_rope, scale=inp["softmax_scale"],
                        out_scale=inp["out_scale"], theta=inp["rope_theta"],
                        page_size=inp["page_size"], block_table=inp["block_table"],
                        to_f64=_f64, batches=batches, heads=heads,
                        num_queries=inp.get("num_queries", 1), **kw)


def gpu_fp8(inp, num_splits=0):
    import torch
    from mlra_latent_kv_amd import harness as H
    case = H.to_device(inp, num_splits=num_splits)
    assert case.latent8 is not None and case.params.latent_format == 1
    out = case.run()
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), case


CASES = [
    # (id, workload, lengths, forced splits, query tokens)
    ("paged_h32", "mla_bf16_paged_b64_h32_l1k-32k", [300, 1, 0, 65, 777], 0, 1),
    ("paged_h32_page_splits", "mla_bf16_paged_b64_h32_l1k-32k", [129, 64, 200], 4, 1),
    ("h128_contiguous", "mla_bf16_b32_h128_l4096", [700, 1, 0, 130], 0, 1),
    ("mlra4", "mlra4_bf16_b32_h32_l8192", [513, 2, 0, 200], 0, 1),
    ("shard", "mlra_shard_bf16_b32_h32_l8192", [640, 63, 0, 5], 0, 1),
    ("paged_h32_sq2", "mla_bf16_paged_b64_h32_l1k-32k", [300, 1, 2, 65], 0, 2),
    ("mlra4_sq3", "mlra4_bf16_b32_h32_l8192", [65, 130, 2], 3, 3),
]


@pytest.mark.parametrize("cid,wname,lens,splits,sq", CASES, ids=[c[0] for c in CASES])
def test_fp8_latent_matches_oracle(cid, wname, lens, splits, sq):
    w = I.WORKLOADS[wname]
    for sharp in (False, True):
        inp = I.make_inputs(w, seed=13, seqlens=lens, num_queries=sq, latent_format="fp8",
                            q_gain=I.sharp_q_gain(w) if sharp else 1.0)
        got, _ = gpu_fp8(inp, splits)
        assert_close(got, oracle_fp8(inp), "bf16", f"fp8 {cid} {'sharp' if sharp else 'default'}")


def test_fp8_latent_controls():
    """The scale is applied (a planted scale x 1.25 in the oracle is told apart), and the fp8
    result sits near the bf16-cache result at the distance the quantisation of the cache
    gives (reported, bounded loosely: E4M3 keeps 3 mantissa bits)."""
    import torch
    from mlra_latent_kv_amd import harness as H
    w = I.WORKLOADS["mla_bf16_paged_b64_h32_l1k-32k"]
    lens = [300, 65, 777]
    inp = I.make_inputs(w, seed=13, seqlens=lens, latent_format="fp8", q_gain=I.sharp_q_gain(w))
    got, _ = gpu_fp8(inp)
    wrong = rel_l2(got, oracle_fp8(inp, latent_scale=1.25 * inp["latent_scale"]))
    note(f"  against a planted scale x1.25: rel_l2={wrong:.3e}")
    assert wrong > 0.05
    plain = dict(inp, latent_format="")
    case = H.to_device(plain)
    ref16 = case.run()
    torch.cuda.synchronize()
    q = rel_l2(got, ref16.float().cpu().numpy().astype(np.float64))
    note(f"  fp8 latent against the bf16 cache it was quantised from: rel_l2={q:.3e}")
    assert 1e-3 < q < 0.2


def test_fp8_latent_with_gate():
    import torch
    from mlra_latent_kv_amd import harness as H
    w = I.WORKLOADS["mlra4_bf16_b32_h32_l8192"]
    inp = I.make_inputs(w, seed=13, seqlens=[513, 2, 200], latent_format="fp8",
                        q_gain=I.sharp_q_gain(w))
    var = I.make_variant_inputs(inp)
    case = H.to_device(inp)
    g = H.run_variant(case, gate=H._to_dev(var["gate"], "bf16", case.out.device))
    lo = H.run_variant(case, latent_out=True)
    torch.cuda.synchronize()
    f = lambda t: t.float().cpu().numpy().astype(np.float64)
    assert_close(f(g), oracle_fp8(inp, gate=var["gate"]), "bf16", "fp8 mlra4 gated")
    from test_gpu_variants import check
    check(f(lo), oracle_fp8(inp, latent_out=True), "bf16", "fp8 mlra4 latent output")


def test_fp8_latent_full_size_sampled():
    """The paged variable-length workload (64 sequences of 1k-32k tokens) with an fp8 latent,
    sharp query, on sampled outputs including the longest and the shortest sequence."""
    w = I.WORKLOADS["mla_bf16_paged_b64_h32_l1k-32k"]
    note("  generating mla_bf16_paged_b64_h32_l1k-32k with an fp8 latent")
    inp = I.make_inputs(w, latent_format="fp8", q_gain=I.sharp_q_gain(w))
    lens = [int(x) for x in inp["seqlens"]]
    bs = [0, int(np.argmax(lens)), int(np.argmin(lens)), 21]
    hs = [0, 15, 16, 31]
    got, _ = gpu_fp8(inp)
    assert np.all(np.isfinite(got))
    assert_close(got[np.ix_(bs, hs)], oracle_fp8(inp, batches=bs, heads=hs), "bf16",
                 "fp8 paged varlen full size")
