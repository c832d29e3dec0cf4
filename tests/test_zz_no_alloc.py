"""mla_decode_noalloc (the allocation-free variant, static scratch) against mla_decode (caller
workspace) through the C ABI: two calls in a row on one GPU, the second with a smaller input,
each bit-identical to mla_decode on the same inputs and within the oracle tolerance."""

import numpy as np
import pytest

from oracle import mla_oracle as O
from mlra_latent_kv_amd import inputs as I

pytestmark = pytest.mark.gpu


def _oracle(inp):
    w = inp["workload"]
    return O.mla_decode(inp["q_nope"], inp["q_rope"], inp["cache"], inp["seqlens"], inp["w_uk"],
                        inp["w_uv"], d_rope=w.d_rope, scale=w.softmax_scale,
                        out_scale=w.out_scale, theta=w.rope_theta, page_size=inp["page_size"],
                        block_table=inp["block_table"], to_f64=lambda a: I.to_f64(a, "bf16"))


def test_noalloc_matches_workspace_entry_point_twice():
    import torch
    from mlra_latent_kv_amd import binding as B
    from mlra_latent_kv_amd import harness as H
    cases = [
        # first call: the 128-head kernel, contiguous cache
        ("mla_bf16_b32_h128_l4096", [4000, 700, 64, 1, 2048, 0, 999, 3000]),
        # second call, smaller: the 32-head kernel, paged cache
        ("mla_bf16_paged_b64_h32_l1k-32k", [130, 5, 64]),
    ]
    for wname, lens in cases:
        w = I.WORKLOADS[wname]
        inp = I.make_inputs(w, seqlens=lens, q_gain=I.sharp_q_gain(w))
        case = H.to_device(inp)
        assert B.workspace_size(case.params) <= B.NOALLOC_SCRATCH_BYTES
        case.run()
        out = torch.full_like(case.out, float("nan"))
        B.mla_decode_noalloc(case.params, case.q_nope, case.q_rope, case.latent_ptr,
                             case.rope_ptr, case.seqlens, case.block_table, case.w_uk, case.w_uv,
                             out)
        torch.cuda.synchronize()
        print(f"  {wname} B={len(lens)}: noalloc == mla_decode: {torch.equal(out, case.out)}",
              flush=True)
        assert torch.equal(out, case.out), wname
        got = out.float().cpu().numpy().astype(np.float64)
        ref = _oracle(inp)
        err = float(np.abs(got - ref).max())
        rel = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
        assert err <= 2e-2 and rel <= 1e-2, (wname, err, rel)
