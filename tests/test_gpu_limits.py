"""GPU decode at the sizes the boundary allows beyond the named workloads, against the fp64
oracle on sampled (sequence, head) outputs:
  * many sequences (1500: the device plan's per-thread scans run several passes, every
    sequence gets one work item because the batch alone exceeds the item target, and the
    merge covers 1500 rows);
  * one sequence of 2^20 tokens (a 1.2 GB paged pool, 16384 pages through the block table)
    with the automatic plan, and the same cache with the largest forced split count (512
    splits, the merge's longest split list);
  * the largest query-token count (16) on a short cache.
Same bounds as the named workloads (max-abs 2e-2, rel-L2 1e-2, worst row 5e-2).
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


def _oracle(inp, bs, hs):
    w = inp["workload"]
    return O.mla_decode(inp["q_nope"], inp["q_rope"], inp["cache"], inp["seqlens"], inp["w_uk"],
                        inp["w_uv"], d_rope=w.d_rope, scale=inp["softmax_scale"],
                        out_scale=inp["out_scale"], theta=inp["rope_theta"],
                        page_size=inp["page_size"], block_table=inp["block_table"],
                        to_f64=lambda a: I.to_f64(a, w.dtype), batches=bs, heads=hs,
                        num_queries=inp.get("num_queries", 1))


def _run(inp, num_splits=0):
    import torch
    from mlra_latent_kv_amd import harness as H
    case = H.to_device(inp, num_splits=num_splits)
    out = case.run()
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), case


def test_many_sequences():
    from mlra_latent_kv_amd import harness as H
    w = I.WORKLOADS["mla_bf16_paged_b64_h32_l1k-32k"]
    rng = np.random.default_rng(17)
    lens = rng.integers(0, 300, 1500)
    lens[[0, 700, 1499]] = [0, 1, 299]
    note("  generating 1500 sequences")
    inp = I.make_inputs(w, seqlens=lens.tolist(), q_gain=I.sharp_q_gain(w))
    got, case = _run(inp)
    plan = H.read_plan(case)
    nonempty = int((lens > 0).sum())
    assert plan["items"] == nonempty and plan["pages"] == -(-int(lens.max()) // 64), plan["items"]
    assert np.all(np.isfinite(got)) and not np.any(got[lens == 0])
    bs = [1, 2, 700, 1001, 1499]
    hs = [0, 17, 31]
    assert_close(got[np.ix_(bs, hs)], _oracle(inp, bs, hs), "bf16", "1500 sequences")


def test_one_sequence_of_a_million_tokens():
    """The automatic plan (256 items of 64 pages), then the largest forced split count (512
    items of 32 pages, the merge's longest split list), on the same cache."""
    from mlra_latent_kv_amd import harness as H
    w = I.WORKLOADS["mla_bf16_paged_b4_h128_l131072"]
    L = 1 << 20
    note(f"  generating one sequence of {L} tokens")
    inp = I.make_inputs(w, seqlens=[L], q_gain=I.sharp_q_gain(w))
    hs = [0, 77, 127]
    ref = _oracle(inp, [0], hs)
    for forced in (0, 512):
        got, case = _run(inp, forced)
        plan = H.read_plan(case)
        note(f"  plan: {plan['items']} items of {plan['pages']} pages")
        assert plan["items"] == (512 if forced else 256)
        assert np.all(np.isfinite(got))
        assert_close(got[np.ix_([0], hs)], ref, "bf16",
                     f"2^20 tokens, {'512 splits' if forced else 'automatic plan'}")
        del case


def test_sixteen_query_tokens():
    """num_queries = 16 (the largest) on 32 heads: 512 query rows, four row quads on the
    128-row kernel; lengths below, at and above 16."""
    w = I.WORKLOADS["mla_bf16_paged_b64_h32_l1k-32k"]
    inp = I.make_inputs(w, seqlens=[5, 16, 300, 1000], num_queries=16, q_gain=I.sharp_q_gain(w))
    got, _ = _run(inp)
    assert got.shape == (4, 512, 128)
    hs = [0, 31, 100, 255, 256, 400, 480, 511]
    assert_close(got[:, hs], _oracle(inp, None, hs), "bf16", "16 query tokens")
