"""GPU decode variants against the fp64 oracle: the gated output (mla_decode_gated /
mlra_decode_gated), the folded query (MLA_FLAG_QUERY_LATENT) and the latent output
(MLA_FLAG_OUTPUT_LATENT), alone and combined, on every kernel family (fp32 SIMT, the 128-head
kernel, the 32-head kernel on MLA, MLRA-4 and one MLRA branch), at small ragged sizes and at a
full size on sampled outputs.  Same bounds as the plain decode (max-abs 2e-2, rel-L2 1e-2 for
bf16; 1e-5 for fp32, and the worst per-(sequence, head) row), since each variant adds at most
one fp32 multiply before the final rounding; a latent output is checked on the same relative
bounds with max-abs scaled to its magnitude.
"""

import numpy as np
import pytest

from oracle import mla_oracle as O
from mlra_latent_kv_amd import inputs as I
from test_gpu_parity import ROW_TOL, TOL, note, rel_l2, worst_row_rel_l2

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def built_library():
    import os
    from mlra_latent_kv_amd import binding as B
    if not os.path.exists(B.LIB_PATH):
        from mlra_latent_kv_amd import build
        build.build()
    B.load()


def oracle_variant(inp, var, *, gate=False, q_latent=False, latent_out=False, batches=None,
                   heads=None):
    dt = inp["dtype"]
    w = inp["workload"]
    return O.mla_decode(var["q_latent"] if q_latent else inp["q_nope"], inp["q_rope"],
                        inp["cache"], inp["seqlens"], None if q_latent else inp["w_uk"],
                        None if latent_out else inp["w_uv"], d_rope=w.d_rope,
                        scale=inp["softmax_scale"], out_scale=inp["out_scale"],
                        theta=inp["rope_theta"], page_size=inp["page_size"],
                        block_table=inp["block_table"], to_f64=lambda a: I.to_f64(a, dt),
                        batches=batches, heads=heads, gate=var["gate"] if gate else None,
                        q_latent=q_latent, latent_out=latent_out, branches=w.branches,
                        d_cb=w.d_cb)


def check(got, ref, dtype, what):
    max_abs, rel = TOL[dtype]
    scale = max(1.0, float(np.abs(ref).max()) / 0.5) if dtype == "bf16" else 1.0
    err = float(np.abs(got - ref).max())
    rl = rel_l2(got, ref)
    row = worst_row_rel_l2(got, ref)
    note(f"  {what}: max_abs={err:.3e} rel_l2={rl:.3e} worst_row_rel_l2={row:.3e}")
    assert np.all(np.isfinite(got))
    assert err <= max_abs * scale and rl <= rel and row <= ROW_TOL[dtype], (what, err, rl, row)


F32_MLRA = I.Workload("mlra4_f32_small", batch=1, heads=4, branches=4, d_nope=16, d_v=16, d_cb=16,
                      d_rope=8, dtype="f32", paged=False, seqlen=64, out_scale=0.5, seed=77)

CASES = {
    # workload, sequence lengths (ragged tails, an empty and a one-token sequence), splits
    "tiny_mla_f32_b1_h4_l64": (I.WORKLOADS["tiny_mla_f32_b1_h4_l64"], [64, 1, 0, 37], 0),
    "mlra4_f32_small": (F32_MLRA, [64, 3, 50], 1),
    "mla_bf16_b32_h128_l4096": (I.WORKLOADS["mla_bf16_b32_h128_l4096"], [700, 1, 0, 130], 0),
    "mla_bf16_paged_b64_h32_l1k-32k": (I.WORKLOADS["mla_bf16_paged_b64_h32_l1k-32k"],
                                       [300, 65, 1, 0, 777], 3),
    "mlra4_bf16_b32_h32_l8192": (I.WORKLOADS["mlra4_bf16_b32_h32_l8192"], [513, 2, 0, 200], 0),
    "mlra_shard_bf16_b32_h32_l8192": (I.WORKLOADS["mlra_shard_bf16_b32_h32_l8192"],
                                      [640, 63, 0, 5], 0),
}
VARIANTS = {
    "gate": dict(gate=True),
    "query_latent": dict(q_latent=True),
    "output_latent": dict(latent_out=True),
    "query_latent+gate": dict(q_latent=True, gate=True),
    "query_latent+output_latent": dict(q_latent=True, latent_out=True),
}


def _device_variant(case, var, dt, gate=False, q_latent=False, latent_out=False):
    from mlra_latent_kv_amd import harness as H
    dev = case.out.device
    return H.run_variant(case, gate=H._to_dev(var["gate"], dt, dev) if gate else None,
                         q_latent=H._to_dev(var["q_latent"], dt, dev) if q_latent else None,
                         latent_out=latent_out)


@pytest.mark.parametrize("vname", list(VARIANTS))
@pytest.mark.parametrize("cname", list(CASES))
def test_variant_matches_oracle(cname, vname):
    """Each variant on each kernel family, default and sharp queries; the plain call on the
    same device inputs afterwards still matches the plain oracle (the variants leave no state
    behind)."""
    import torch
    from mlra_latent_kv_amd import harness as H
    w, lens, splits = CASES[cname]
    kw = VARIANTS[vname]
    for sharp in (False, True):
        inp = I.make_inputs(w, seed=5, seqlens=lens,
                            q_gain=I.sharp_q_gain(w) if sharp else 1.0)
        var = I.make_variant_inputs(inp)
        case = H.to_device(inp, num_splits=splits)
        out = _device_variant(case, var, w.dtype, **kw)
        torch.cuda.synchronize()
        got = out.float().cpu().numpy().astype(np.float64)
        ref = oracle_variant(inp, var, **kw)
        assert got.shape == ref.shape
        check(got, ref, w.dtype, f"{cname} {vname} {'sharp' if sharp else 'default'}")
        if sharp:
            plain = case.run()
            torch.cuda.synchronize()
            check(plain.float().cpu().numpy().astype(np.float64),
                  O.mla_decode(inp["q_nope"], inp["q_rope"], inp["cache"], inp["seqlens"],
                               inp["w_uk"], inp["w_uv"], d_rope=w.d_rope,
                               scale=inp["softmax_scale"], out_scale=inp["out_scale"],
                               theta=inp["rope_theta"], page_size=inp["page_size"],
                               block_table=inp["block_table"],
                               to_f64=lambda a: I.to_f64(a, w.dtype)),
                  w.dtype, f"{cname} plain after {vname}")


@pytest.mark.parametrize("cname", ["mlra4_bf16_b32_h32_l8192", "mla_bf16_b32_h128_l4096"])
def test_variant_negative_controls(cname):
    """The tolerance separates each variant from the plain step it modifies: the gated output
    against the ungated oracle, the folded-query output against the oracle of the unfolded
    query, the latent output against the oracle's latent output with branches 0 and 1 swapped
    (MLRA) or with its halves swapped (MLA)."""
    import torch
    from mlra_latent_kv_amd import harness as H
    w, lens, splits = CASES[cname]
    inp = I.make_inputs(w, seed=5, seqlens=lens, q_gain=I.sharp_q_gain(w))
    var = I.make_variant_inputs(inp)
    case = H.to_device(inp, num_splits=splits)
    g = _device_variant(case, var, w.dtype, gate=True)
    q = _device_variant(case, var, w.dtype, q_latent=True)
    lo = _device_variant(case, var, w.dtype, latent_out=True)
    torch.cuda.synchronize()
    f = lambda t: t.float().cpu().numpy().astype(np.float64)
    nz = [b for b, L in enumerate(lens) if L > 0]
    assert rel_l2(f(g)[nz], oracle_variant(inp, var)[nz]) > 0.2
    assert rel_l2(f(q)[nz], oracle_variant(inp, var)[nz]) > 0.2
    ref_lo = oracle_variant(inp, var, latent_out=True)
    half = ref_lo.shape[-1] // 2 if w.branches == 1 else w.d_cb
    swapped = ref_lo.copy()
    swapped[..., :half], swapped[..., half:2 * half] = ref_lo[..., half:2 * half], ref_lo[..., :half]
    assert rel_l2(f(lo)[nz], swapped[nz]) > 0.2


def test_gated_mlra4_full_size_sampled():
    """Gated MLRA-4 at its full size (32 sequences of 8192 tokens), sharp query, in the launch
    configuration of the plain call, on sampled (sequence, head) outputs; then the folded query
    with the latent output at the same size."""
    import torch
    from mlra_latent_kv_amd import harness as H
    w = I.WORKLOADS["mlra4_bf16_b32_h32_l8192"]
    note("  generating mlra4_bf16_b32_h32_l8192")
    inp = I.requery(I.make_inputs(w), I.sharp_q_gain(w))
    var = I.make_variant_inputs(inp)
    case = H.to_device(inp)
    bs, hs = [0, 17, 31], [0, 13, 31]
    g = _device_variant(case, var, w.dtype, gate=True)
    ql = _device_variant(case, var, w.dtype, q_latent=True, latent_out=True)
    torch.cuda.synchronize()
    f = lambda t: t.float().cpu().numpy().astype(np.float64)[np.ix_(bs, hs)]
    check(f(g), oracle_variant(inp, var, gate=True, batches=bs, heads=hs), "bf16",
          "mlra4 full size gated")
    check(f(ql), oracle_variant(inp, var, q_latent=True, latent_out=True, batches=bs, heads=hs),
          "bf16", "mlra4 full size folded query + latent output")
