"""Pins for the fp64 oracle, independent of the oracle itself.

Each test checks the oracle against something it does not share: closed forms,
hand-worked examples, a pure-Python brute force with a different softmax and
rotation formulation, PyTorch's scaled-dot-product attention (fp64, CPU), or
invariants the pages' method must satisfy.  The last block plants mistakes in
the oracle (on the CPU) and checks that some pin catches each one.
"""

import cmath
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import mla_oracle as O
from mlra_latent_kv_amd import inputs as I

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rel_l2(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def small_case(w, seed=7, seqlens=(37,), **kw):
    """Workload-shaped inputs with small batch/length, decoded to fp64."""
    inp = I.make_inputs(w, seed=seed, seqlens=list(seqlens), **kw)
    return inp


def run_oracle(inp, **kw):
    dt = inp["dtype"]
    return O.mla_decode(inp["q_nope"], inp["q_rope"], inp["cache"], inp["seqlens"], inp["w_uk"],
                        inp["w_uv"], d_rope=inp["workload"].d_rope, scale=inp["softmax_scale"],
                        out_scale=inp["out_scale"], theta=inp["rope_theta"],
                        page_size=inp["page_size"], block_table=inp["block_table"],
                        to_f64=lambda a: I.to_f64(a, dt), **kw)


# ----------------------------------------------------------------------------- RoPE pins

def test_rope_frequencies_closed_form():
    # 10000^(-2i/d): d=4 -> 1, 1/100 ; d=8 -> 1, 1/10, 1/100, 1/1000
    assert np.allclose(O.rope_frequencies(4, 10000.0), [1.0, 0.01], rtol=1e-15, atol=0)
    assert np.allclose(O.rope_frequencies(8, 10000.0), [1.0, 0.1, 0.01, 0.001], rtol=1e-15, atol=0)


def test_rope_d2_is_rotation_matrix():
    # d_rope = 2: one pair with frequency 1, so pos p rotates by p radians counter-clockwise.
    rng = np.random.default_rng(0)
    for p in [0, 1, 2, 5, 1000]:
        x = rng.standard_normal(2)
        R = np.array([[math.cos(p), -math.sin(p)], [math.sin(p), math.cos(p)]])
        assert np.allclose(O.rope(x, p), R @ x, rtol=0, atol=1e-14)


def test_rope_matches_complex_multiplication():
    # (x_2i + j x_2i+1) * exp(j pos theta_i) -- an independent formulation
    rng = np.random.default_rng(1)
    d, theta = 64, 10000.0
    x = rng.standard_normal((5, d))
    pos = np.array([0, 1, 63, 4095, 131071])
    got = O.rope(x, pos, theta)
    for r in range(5):
        for i in range(d // 2):
            z = complex(x[r, 2 * i], x[r, 2 * i + 1]) * cmath.exp(1j * pos[r] * theta ** (-2.0 * i / d))
            assert abs(got[r, 2 * i] - z.real) < 1e-9 and abs(got[r, 2 * i + 1] - z.imag) < 1e-9


def test_rope_identity_norm_relative_composition():
    rng = np.random.default_rng(2)
    d = 64
    q, k = rng.standard_normal(d), rng.standard_normal(d)
    assert np.array_equal(O.rope(q, 0), q)
    for p in [1, 77, 131071]:
        assert abs(np.linalg.norm(O.rope(q, p)) - np.linalg.norm(q)) < 1e-12
    # inner product depends only on the position difference (the relative-position property
    # the pages say decoupled RoPE keeps: qian.cx post; yololab section 解耦旋轉位置編碼)
    base = O.rope(q, 1000) @ O.rope(k, 990)
    for shift in [-990, 5, 30000]:
        assert abs(O.rope(q, 1000 + shift) @ O.rope(k, 990 + shift) - base) < 1e-9
    assert np.allclose(O.rope(O.rope(q, 17), 25), O.rope(q, 42), atol=1e-12)


# ----------------------------------------------------------------------------- softmax pins

def test_softmax_sums_to_one_and_matches_scipy():
    from scipy.special import softmax as sp_softmax
    rng = np.random.default_rng(3)
    s = rng.standard_normal((4, 100)) * 30
    p = O.softmax(s)
    assert np.allclose(p.sum(-1), 1.0, atol=1e-14)
    assert np.allclose(p, sp_softmax(s, axis=-1), rtol=1e-13, atol=0)


# ----------------------------------------------------------------------------- hand-worked examples

def test_hand_example_mla_content_only():
    """Two tokens, identity up-projections, rope part zero.

    c_0 = (1,0), c_1 = (0,1); q_nope = (a, 0) with scale*a = ln 3 so the scores are
    (ln 3, 0), the probabilities (3/4, 1/4) and (W_UV = I) the output (3/4, 1/4).
    """
    scale = 0.5
    a = math.log(3.0) / scale
    qn = np.array([[[a, 0.0]]])            # [H=1, NB=1, d_nope=2]
    qr = np.zeros((1, 2))                  # [H, d_rope=2]
    rows = np.array([[1.0, 0.0, 0.0, 0.0],
                     [0.0, 1.0, 0.0, 0.0]])  # [L=2, d_c=2 | d_rope=2]
    eye = np.eye(2)[None, None]
    out = O.attend_unabsorbed(qn, qr, rows, eye, eye, d_rope=2, scale=scale, out_scale=1.0,
                              theta=10000.0)
    assert np.allclose(out, [[0.75, 0.25]], rtol=0, atol=1e-15)


def test_hand_example_rope_only_pins_positions():
    """Content part zero; d_rope = 2 (frequency 1), raw keys (1,0) at positions 0 and 1.

    Rotated keys: (1,0) and (cos1, sin1).  The query (1,0) is rotated at position L-1 = 1,
    giving (cos1, sin1); scores (scale 1) are cos 1 and 1, so
    p_1 / p_0 = exp(1 - cos 1).  With V = c = e_0, e_1 the output is (p_0, p_1).
    A query rotated at position L, a sign error in the rotation, or a dropped rope term
    all change this.
    """
    qn = np.zeros((1, 1, 2))
    qr = np.array([[1.0, 0.0]])
    rows = np.array([[1.0, 0.0, 1.0, 0.0],
                     [0.0, 1.0, 1.0, 0.0]])
    eye = np.eye(2)[None, None]
    out = O.attend_unabsorbed(qn, qr, rows, eye, eye, d_rope=2, scale=1.0, out_scale=1.0,
                              theta=10000.0)
    r = math.exp(1.0 - math.cos(1.0))
    assert np.allclose(out, [[1.0 / (1.0 + r), r / (1.0 + r)]], rtol=0, atol=1e-15)


def test_hand_example_mlra4_scaled_branch_sum():
    """Four branches of width 1, identity (1x1) projections, rope zero, L = 2.

    Branch b: c_{b,0} = 1, c_{b,1} = 0, scale*q_b = ln r_b with r = 1,2,3,4, so
    p_{b,0} = r_b/(1+r_b) and o_b = p_{b,0}.  out = 0.5 * (1/2 + 2/3 + 3/4 + 4/5) = 163/120.
    """
    scale = 0.25
    r = [1.0, 2.0, 3.0, 4.0]
    qn = np.array([[[math.log(x) / scale] for x in r]])   # [H=1, NB=4, d_nope=1]
    qr = np.zeros((1, 2))
    rows = np.array([[1.0, 1.0, 1.0, 1.0, 0.0, 0.0],
                     [0.0, 0.0, 0.0, 0.0, 0.0, 0.0]])
    one = np.ones((4, 1, 1, 1))
    out = O.attend_unabsorbed(qn, qr, rows, one, one, d_rope=2, scale=scale, out_scale=0.5,
                              theta=10000.0)
    assert abs(out[0, 0] - float(Fraction(163, 120))) < 1e-15


# ----------------------------------------------------------------------------- brute force

def _rotate_py(x, pos, theta):
    d = len(x)
    out = []
    for i in range(d // 2):
        z = complex(x[2 * i], x[2 * i + 1]) * cmath.exp(1j * pos * theta ** (-2.0 * i / d))
        out += [z.real, z.imag]
    return out


def brute_force(qn, qr, rows, w_uk, w_uv, d_rope, scale, out_scale, theta):
    """Scalar loops, math.fsum, softmax as p_t = 1 / sum_j exp(s_j - s_t)."""
    NB, H, dn, dcb = w_uk.shape
    dv = w_uv.shape[-1]
    L = len(rows)
    res = []
    for h in range(H):
        qrot = _rotate_py(list(qr[h]), L - 1, theta)
        acc = [[] for _ in range(dv)]
        for br in range(NB):
            scores, vals = [], []
            for t in range(L):
                c = [float(v) for v in rows[t][br * dcb:(br + 1) * dcb]]
                K = [math.fsum(float(w_uk[br, h, n, j]) * c[j] for j in range(dcb)) for n in range(dn)]
                V = [math.fsum(float(w_uv[br, h, j, v]) * c[j] for j in range(dcb)) for v in range(dv)]
                krot = _rotate_py([float(v) for v in rows[t][NB * dcb:NB * dcb + d_rope]], t, theta)
                s = scale * (math.fsum(float(qn[h, br, n]) * K[n] for n in range(dn))
                             + math.fsum(qrot[i] * krot[i] for i in range(d_rope)))
                scores.append(s)
                vals.append(V)
            for t in range(L):
                p = 1.0 / math.fsum(math.exp(sj - scores[t]) for sj in scores)
                for v in range(dv):
                    acc[v].append(p * vals[t][v])
        res.append([out_scale * math.fsum(a) for a in acc])
    return np.array(res)


@pytest.mark.parametrize("shape", [
    dict(H=4, NB=1, dn=16, dcb=32, dr=8, dv=16, L=64, out_scale=1.0),     # tiny workload dims
    dict(H=2, NB=4, dn=3, dcb=5, dr=4, dv=6, L=9, out_scale=0.5),         # MLRA-4, non-square
    dict(H=3, NB=1, dn=7, dcb=4, dr=2, dv=5, L=1, out_scale=1.0),         # single token
])
def test_brute_force_matches_oracle(shape):
    rng = np.random.default_rng(11)
    H, NB, dn, dcb, dr, dv, L = (shape[k] for k in ("H", "NB", "dn", "dcb", "dr", "dv", "L"))
    qn = rng.standard_normal((H, NB, dn))
    qr = rng.standard_normal((H, dr))
    rows = rng.standard_normal((L, NB * dcb + dr))
    w_uk = rng.standard_normal((NB, H, dn, dcb)) / math.sqrt(dcb)
    w_uv = rng.standard_normal((NB, H, dcb, dv)) / math.sqrt(dcb)
    kw = dict(d_rope=dr, scale=0.3, out_scale=shape["out_scale"], theta=10000.0)
    got = O.attend_unabsorbed(qn, qr, rows, w_uk, w_uv, **kw)
    ref = brute_force(qn, qr, rows, w_uk, w_uv, dr, 0.3, shape["out_scale"], 10000.0)
    assert rel_l2(got, ref) < 1e-12


# ----------------------------------------------------------------------------- library routine

def sdpa_reference(qn, qr, rows, w_uk, w_uv, d_rope, scale, out_scale, theta):
    """Explicitly up-projected keys/values fed to torch's scaled_dot_product_attention (fp64, CPU)."""
    import torch
    import torch.nn.functional as F
    NB, H, dn, dcb = w_uk.shape
    L = rows.shape[0]
    krot = O.rope(rows[:, NB * dcb:NB * dcb + d_rope], np.arange(L), theta)
    out = np.zeros((H, w_uv.shape[-1]))
    for h in range(H):
        qrot = O.rope(qr[h], L - 1, theta)
        for br in range(NB):
            c = rows[:, br * dcb:(br + 1) * dcb]
            K = np.concatenate([c @ w_uk[br, h].T, krot], axis=1)
            V = c @ w_uv[br, h]
            qq = np.concatenate([qn[h, br], qrot])
            o = F.scaled_dot_product_attention(
                torch.from_numpy(qq)[None, None, None, :], torch.from_numpy(K)[None, None],
                torch.from_numpy(V)[None, None], scale=scale)
            out[h] += o[0, 0, 0].numpy()
    return out_scale * out


@pytest.mark.parametrize("wname", ["tiny_mla_f32_b1_h4_l64", "mla_bf16_b32_h128_l4096",
                                   "mlra4_bf16_b32_h32_l8192"])
def test_oracle_matches_torch_sdpa(wname):
    w = I.WORKLOADS[wname]
    inp = small_case(w, seqlens=(70,))
    dt = w.dtype
    rows = O.sequence_rows(inp["cache"], 0, 70, 0, None, lambda a: I.to_f64(a, dt))
    qn, qr = I.to_f64(inp["q_nope"], dt)[0], I.to_f64(inp["q_rope"], dt)[0]
    w_uk, w_uv = I.to_f64(inp["w_uk"], dt), I.to_f64(inp["w_uv"], dt)
    heads = list(range(min(w.heads, 8)))
    got = O.attend_unabsorbed(qn, qr, rows, w_uk, w_uv, d_rope=w.d_rope, scale=w.softmax_scale,
                              out_scale=w.out_scale, theta=w.rope_theta, heads=heads)
    ref = sdpa_reference(qn[heads], qr[heads], rows, w_uk[:, heads], w_uv[:, heads], w.d_rope,
                         w.softmax_scale, w.out_scale, w.rope_theta)
    assert rel_l2(got, ref) < 1e-12


# ----------------------------------------------------------------------------- identities

@pytest.mark.parametrize("wname", I.WORKLOAD_ORDER)
def test_absorbed_equals_unabsorbed(wname):
    """Matrix absorption is exact by associativity (yololab, section 矩陣吸收)."""
    w = I.WORKLOADS[wname]
    inp = small_case(w, seqlens=(1, 65, 130), q_gain=I.sharp_q_gain(w))
    heads = list(range(min(w.heads, 6)))
    a = run_oracle(inp, heads=heads)
    b = run_oracle(inp, heads=heads, absorbed=True)
    assert rel_l2(b, a) < 1e-12


def test_zero_query_gives_uniform_mean_of_values():
    w = I.WORKLOADS["mlra4_bf16_b32_h32_l8192"]
    inp = small_case(w, seqlens=(50,))
    inp["q_nope"][:] = 0
    inp["q_rope"][:] = 0
    out = run_oracle(inp, heads=[0, 5])[0]
    rows = I.to_f64(inp["cache"][0, :50], "bf16")
    w_uv = I.to_f64(inp["w_uv"], "bf16")
    for j, h in enumerate([0, 5]):
        exp = sum(rows[:, br * 128:(br + 1) * 128].mean(axis=0) @ w_uv[br, h] for br in range(4))
        assert rel_l2(out[j], 0.5 * exp) < 1e-13


def test_single_token_returns_its_value():
    w = I.WORKLOADS["mla_bf16_b32_h128_l4096"]
    inp = small_case(w, seqlens=(1, 1), q_gain=50.0)
    out = run_oracle(inp, heads=[3])
    for b in range(2):
        c0 = I.to_f64(inp["cache"][b, 0, :512], "bf16")
        exp = c0 @ I.to_f64(inp["w_uv"][0, 3], "bf16")
        assert rel_l2(out[b, 0], exp) < 1e-13


def test_needle_with_huge_logit():
    """One token's logit exceeds the others by ~800: the output is that token's value
    (exp(-800) underflows to 0), which needs the max-subtraction to stay finite."""
    rng = np.random.default_rng(5)
    H, dn, dcb, dr, dv, L = 1, 8, 8, 4, 8, 40
    rows = rng.standard_normal((L, dcb + dr)) * 0.01
    u = np.zeros(dcb)
    u[0] = 1.0
    rows[17, :dcb] = u
    w_uk = np.eye(dcb)[None, None]
    w_uv = rng.standard_normal((1, 1, dcb, dv))
    qn = np.zeros((1, 1, dn))
    qn[0, 0, 0] = 800.0
    out = O.attend_unabsorbed(qn, np.zeros((1, dr)), rows, w_uk, w_uv, d_rope=dr, scale=1.0,
                              out_scale=1.0, theta=10000.0)
    assert np.all(np.isfinite(out))
    assert rel_l2(out[0], u @ w_uv[0, 0]) < 1e-12


def test_probabilities_sum_to_one():
    w = I.WORKLOADS["mlra4_bf16_b32_h32_l8192"]
    inp = small_case(w, seqlens=(33,), q_gain=I.sharp_q_gain(w))
    rows = O.sequence_rows(inp["cache"], 0, 33, 0, None, lambda a: I.to_f64(a, "bf16"))
    _, p = O.attend_unabsorbed(I.to_f64(inp["q_nope"], "bf16")[0], I.to_f64(inp["q_rope"], "bf16")[0],
                               rows, I.to_f64(inp["w_uk"], "bf16"), I.to_f64(inp["w_uv"], "bf16"),
                               d_rope=64, scale=w.softmax_scale, out_scale=0.5, theta=1e4,
                               heads=[0, 1], return_probs=True)
    assert np.allclose(p.sum(-1), 1.0, atol=1e-14)
    assert (p >= 0).all()


def test_zero_length_gives_zeros():
    w = I.WORKLOADS["mla_bf16_b32_h128_l4096"]
    inp = small_case(w, seqlens=(0, 3))
    out = run_oracle(inp, heads=[0, 1])
    assert np.all(out[0] == 0) and np.any(out[1] != 0)


def test_paged_equals_contiguous():
    w = I.WORKLOADS["mla_bf16_paged_b64_h32_l1k-32k"]
    lens = (1, 64, 65, 200)
    a = run_oracle(I.make_inputs(w, seed=9, seqlens=lens, paged=True), heads=[0, 7])
    b = run_oracle(I.make_inputs(w, seed=9, seqlens=lens, paged=False), heads=[0, 7])
    assert np.array_equal(a, b)


# ----------------------------------------------------------------------------- MLRA reductions

def _mlra_small(seed=21, L=45):
    w = I.WORKLOADS["mlra4_bf16_b32_h32_l8192"]
    inp = I.make_inputs(w, seed=seed, seqlens=[L], q_gain=I.sharp_q_gain(w))
    dt = "bf16"
    qn = I.to_f64(inp["q_nope"], dt)[0]
    qr = I.to_f64(inp["q_rope"], dt)[0]
    rows = I.to_f64(inp["cache"][0, :L], dt)
    return w, qn, qr, rows, I.to_f64(inp["w_uk"], dt), I.to_f64(inp["w_uv"], dt)


def test_mlra_one_live_branch_equals_mla_on_that_branch():
    w, qn, qr, rows, wk, wv = _mlra_small()
    kw = dict(d_rope=64, scale=w.softmax_scale, theta=1e4, heads=[2])
    wv0 = wv.copy()
    wv0[1:] = 0
    got = O.attend_unabsorbed(qn, qr, rows, wk, wv0, out_scale=0.5, **kw)
    mla_rows = np.concatenate([rows[:, :128], rows[:, 512:]], axis=1)
    ref = O.attend_unabsorbed(qn[:, :1], qr, mla_rows, wk[:1], wv[:1], out_scale=1.0, **kw)
    assert rel_l2(got, 0.5 * ref) < 1e-13


def test_mlra_identical_branches_double_one_branch():
    w, qn, qr, rows, wk, wv = _mlra_small()
    rows4 = rows.copy()
    for br in range(1, 4):
        rows4[:, br * 128:(br + 1) * 128] = rows[:, :128]
    wk4 = np.repeat(wk[:1], 4, axis=0)
    wv4 = np.repeat(wv[:1], 4, axis=0)
    qn4 = np.repeat(qn[:, :1], 4, axis=1)
    kw = dict(d_rope=64, scale=w.softmax_scale, theta=1e4, heads=[0, 9])
    got = O.attend_unabsorbed(qn4, qr, rows4, wk4, wv4, out_scale=0.5, **kw)
    one = O.attend_unabsorbed(qn[:, :1], qr, np.concatenate([rows[:, :128], rows[:, 512:]], 1),
                              wk[:1], wv[:1], out_scale=1.0, **kw)
    assert rel_l2(got, 2.0 * one) < 1e-13


def test_mlra_branch_permutation_invariance():
    w, qn, qr, rows, wk, wv = _mlra_small()
    perm = [2, 0, 3, 1]
    rows_p = rows.copy()
    for nb, ob in enumerate(perm):
        rows_p[:, nb * 128:(nb + 1) * 128] = rows[:, ob * 128:(ob + 1) * 128]
    kw = dict(d_rope=64, scale=w.softmax_scale, out_scale=0.5, theta=1e4, heads=[1, 30])
    a = O.attend_unabsorbed(qn, qr, rows, wk, wv, **kw)
    b = O.attend_unabsorbed(qn[:, perm], qr, rows_p, wk[perm], wv[perm], **kw)
    assert rel_l2(b, a) < 1e-13


# ----------------------------------------------------------------------------- pages' figures

def test_workload_shapes_match_pages_figures():
    g = json.load(open(os.path.join(GOLDEN, "pages_figures.json")))
    p3 = g["latent_compression_page3"]
    w3 = I.WORKLOADS["mla_bf16_paged_b64_h32_l1k-32k"]
    assert w3.heads * w3.d_nope == p3["d_model"] == p3["heads"] * p3["head_dim"]
    assert w3.d_c == p3["d_latent"] == g["latent_compression_interview"]["d_latent"]
    assert round(p3["d_model"] / w3.d_c) == p3["compression_approx"]
    # latent+rope row vs an MHA K+V row at the same shape
    assert w3.row / (2 * w3.heads * w3.d_nope) <= g["mla_cache_fraction_of_mha"]["at_most"]
    # one MLRA-4 branch shard streams (d_cb + d_rope) per token = 1.5 head dims
    w4 = I.WORKLOADS["mlra4_bf16_b32_h32_l8192"]
    assert (w4.d_cb + w4.d_rope) / w4.d_v == g["mlra_per_device_kv_load"]["per_device_load"]
    assert w4.branches == g["mlra_per_device_kv_load"]["mlra_tp_ways"]


# ----------------------------------------------------------------------------- planted mistakes

def _pins_pass():
    """Run the pins that exercise attend_unabsorbed; False if any fails."""
    checks = [test_hand_example_mla_content_only, test_hand_example_rope_only_pins_positions,
              test_hand_example_mlra4_scaled_branch_sum, test_needle_with_huge_logit,
              lambda: test_brute_force_matches_oracle(
                  dict(H=2, NB=4, dn=3, dcb=5, dr=4, dv=6, L=9, out_scale=0.5)),
              lambda: test_oracle_matches_torch_sdpa("tiny_mla_f32_b1_h4_l64")]
    with np.errstate(all="ignore"):
        for c in checks:
            try:
                c()
            except (AssertionError, ValueError):
                return False
    return True


def test_pins_pass_unplanted():
    assert _pins_pass()


@pytest.mark.parametrize("mistake", ["rope_sign", "query_at_L", "no_rope_term", "no_max_sub",
                                     "w_uv_transposed", "softmax_unnormalised"])
def test_planted_mistake_is_caught(monkeypatch, mistake):
    real_rope, real_softmax = O.rope, O.softmax
    if mistake == "rope_sign":
        monkeypatch.setattr(O, "rope", lambda x, pos, theta=1e4: real_rope(x, -np.asarray(pos), theta))
    elif mistake == "query_at_L":
        monkeypatch.setattr(O, "rope", lambda x, pos, theta=1e4: real_rope(
            x, np.asarray(pos) + (1 if np.ndim(pos) == 0 else 0), theta))
    elif mistake == "no_rope_term":
        monkeypatch.setattr(O, "rope", lambda x, pos, theta=1e4: 0.0 * real_rope(x, pos, theta))
    elif mistake == "no_max_sub":
        monkeypatch.setattr(O, "softmax", lambda s: np.exp(s) / np.exp(s).sum(-1, keepdims=True))
    elif mistake == "w_uv_transposed":
        real = O.attend_unabsorbed

        def bad(qn, qr, rows, w_uk, w_uv, **kw):
            return real(qn, qr, rows, w_uk, np.swapaxes(w_uv, -1, -2), **kw)
        monkeypatch.setattr(O, "attend_unabsorbed", bad)
    elif mistake == "softmax_unnormalised":
        monkeypatch.setattr(O, "softmax", lambda s: np.exp(s - s.max(-1, keepdims=True)))
    assert not _pins_pass()


# ----------------------------------------------------------------------------- write-side pins
# c_KV = h W_DKV and k_rope = RoPE(h W_KR, t) at the token's own position t ("超越 GQA 的推理
# 革命…MLA…", sections 鍵值聯合低秩壓縮 and 解耦旋轉位置編碼); the new token goes to t = L_b.

def _append_case(B=5, d_model=7, d_c=4, d_r=2, seed=11):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((B, d_model)), rng.standard_normal((d_model, d_c)),
            rng.standard_normal((d_model, d_r)))


def test_append_hand_example_page_allocation():
    """Worked by hand, page size 64.  Lengths [64, 5, 0, 128, 63]: sequences 0, 2 and 3 start
    a page (64, 0 and 128 are multiples of 64) and take free pages 11, 4, 9 in batch order, at
    block-table columns 1, 0, 2; sequence 1 writes slot 5 of its page 0 and sequence 4 slot 63
    of its page 5.  With only one free page, sequences 2 and 3 are not written."""
    h, wd, wk = _append_case()
    bt = np.full((5, 4), -1)
    bt[0, 0], bt[1, 0], bt[3, 0], bt[3, 1], bt[4, 0] = 2, 0, 1, 3, 5
    r = O.cache_append(h, wd, wk, [64, 5, 0, 128, 63], bt, [11, 4, 9], page_size=64)
    assert r["where"] == [(11, 0), (0, 5), (4, 0), (9, 0), (5, 63)]
    assert list(r["seqlens"]) == [65, 6, 1, 129, 64] and r["pages_used"] == 3
    want = bt.copy()
    want[0, 1], want[2, 0], want[3, 2] = 11, 4, 9
    assert np.array_equal(r["block_table"], want) and np.array_equal(bt[0], [2, -1, -1, -1])
    r = O.cache_append(h, wd, wk, [64, 5, 0, 128, 63], bt, [11], page_size=64)
    assert r["where"] == [(11, 0), (0, 5), None, None, (5, 63)]
    assert list(r["seqlens"]) == [65, 6, 0, 128, 64] and r["pages_used"] == 1
    assert list(r["written"]) == [True, True, False, False, True]
    want = bt.copy()
    want[0, 1] = 11
    assert np.array_equal(r["block_table"], want)
    # contiguous: the row goes to (b, t); a full sequence is left untouched
    r = O.cache_append(h[:3], wd, wk, [3, 0, 8], capacity=8)
    assert r["where"] == [(0, 3), (1, 0), None] and list(r["seqlens"]) == [4, 1, 8]
    # a sequence whose page is missing (negative entry) or whose row is full is not written;
    # it still counts in the page ranks when its token starts a page
    bt2 = np.full((3, 2), -1)
    bt2[0, 0], bt2[1, 0], bt2[1, 1] = 7, 8, 9
    r = O.cache_append(h[:3], wd, wk, [65, 128, 64], bt2, [3, 6], page_size=64)
    assert r["where"] == [None, None, (6, 0)] and list(r["seqlens"]) == [65, 128, 65]
    assert r["pages_used"] == 2 and r["block_table"][2, 1] == 6


def test_append_one_hot_hidden_selects_weight_rows():
    """h = e_j picks row j of each down-projection; with d_r = 2 (one pair, frequency 1) the
    rotary part is row j of W_KR turned by t radians counter-clockwise."""
    _, wd, wk = _append_case(d_model=6)
    for j, t in [(0, 0), (3, 1), (5, 77), (2, 4095)]:
        row = O.latent_rows(np.eye(6)[j][None], wd, wk, [t])[0]
        assert np.array_equal(row[:4], wd[j])
        R = np.array([[math.cos(t), -math.sin(t)], [math.sin(t), math.cos(t)]])
        assert np.allclose(row[4:], R @ wk[j], rtol=0, atol=1e-12)


def test_append_brute_force_scalar():
    """Pure-Python scalar loops (math.fsum dot products, complex-number rotation) against the
    NumPy rows, several positions and a d_r = 8 rotary part."""
    rng = np.random.default_rng(5)
    n, d_model, d_c, d_r = 4, 9, 6, 8
    h = rng.standard_normal((n, d_model))
    wd = rng.standard_normal((d_model, d_c))
    wk = rng.standard_normal((d_model, d_r))
    pos = [0, 1, 63, 131071]
    got = O.latent_rows(h, wd, wk, pos, theta=10000.0)
    for i in range(n):
        c = [math.fsum(h[i, k] * wd[k, j] for k in range(d_model)) for j in range(d_c)]
        raw = [math.fsum(h[i, k] * wk[k, j] for k in range(d_model)) for j in range(d_r)]
        rot = []
        for p in range(d_r // 2):
            z = complex(raw[2 * p], raw[2 * p + 1]) * cmath.exp(1j * pos[i] * 10000.0 ** (-2 * p / d_r))
            rot += [z.real, z.imag]
        assert np.allclose(got[i], c + rot, rtol=1e-12, atol=1e-12)


def test_append_rows_are_linear_in_the_hidden_state():
    h, wd, wk = _append_case(B=2, d_model=9, d_c=5, d_r=4)
    pos = [17, 17]
    a = O.latent_rows(h[:1] + 2.0 * h[1:], wd, wk, pos[:1])
    b = O.latent_rows(h[:1], wd, wk, pos[:1]) + 2.0 * O.latent_rows(h[1:], wd, wk, pos[1:])
    assert np.allclose(a, b, rtol=1e-13, atol=1e-13)


def _append_then_decode(w, L, rng, patch=None):
    """Decode output of a cache built by appending L tokens one step at a time into an empty,
    shuffled paged pool (stored rotary keys turned back by their positions, since the decode
    oracle takes raw keys), and of the same tokens' raw rows laid out contiguously."""
    d_model = 24
    h = rng.standard_normal((L, d_model)) / math.sqrt(d_model)
    wd = rng.standard_normal((d_model, w.d_c)) / math.sqrt(d_model)
    wk = rng.standard_normal((d_model, w.d_rope)) / math.sqrt(d_model)
    pages = -(-L // 64)
    free = list(rng.permutation(pages + 3))
    pool = np.zeros((pages + 3, 64, w.row))
    bt = np.full((1, pages), -1)
    seqlen = [0]
    for t in range(L):
        r = O.cache_append(h[t:t + 1], wd, wk, seqlen, bt, free, page_size=64)
        pg, slot = r["where"][0]
        pool[pg, slot] = r["rows"][0]
        bt, seqlen, free = r["block_table"], list(r["seqlens"]), free[r["pages_used"]:]
    assert seqlen == [L]
    raw_pool = pool.copy()
    for t in range(L):  # decode takes raw keys: undo the rotation at each token's position
        pg, slot = bt[0, t // 64], t % 64
        raw_pool[pg, slot, w.d_c:] = O.rope(pool[pg, slot, w.d_c:], -t, w.rope_theta)
    direct = np.concatenate([h @ wd, h @ wk], axis=1)[None]
    qn = rng.standard_normal((1, w.heads, w.branches, w.d_nope))
    qr = rng.standard_normal((1, w.heads, w.d_rope))
    wuk = rng.standard_normal((w.branches, w.heads, w.d_nope, w.d_cb)) / math.sqrt(w.d_cb)
    wuv = rng.standard_normal((w.branches, w.heads, w.d_cb, w.d_v)) / math.sqrt(w.d_cb)
    kw = dict(d_rope=w.d_rope, scale=w.softmax_scale, out_scale=w.out_scale, theta=w.rope_theta)
    a = O.mla_decode(qn, qr, raw_pool, [L], wuk, wuv, page_size=64, block_table=bt, **kw)
    b = O.mla_decode(qn, qr, direct, [L], wuk, wuv, **kw)
    return a, b


@pytest.mark.parametrize("wname", ["tiny_mla_f32_b1_h4_l64", "mlra4_f32_like"])
def test_append_then_decode_equals_direct_cache(wname):
    """Appending tokens one decode step at a time (positions 0, 1, ..., pages taken from a
    shuffled free list as each page fills) gives the cache the decode step reads: its output
    equals that of the same tokens' rows written directly."""
    w = (I.WORKLOADS["tiny_mla_f32_b1_h4_l64"] if wname.startswith("tiny") else
         I.Workload("mlra4_f32_like", batch=1, heads=2, branches=4, d_nope=4, d_v=3, d_cb=4,
                    d_rope=4, dtype="f32", paged=True, seqlen=150, out_scale=0.5))
    a, b = _append_then_decode(w, 150, np.random.default_rng(3))
    assert rel_l2(a, b) < 1e-12


def _append_pins_pass():
    checks = [test_append_hand_example_page_allocation,
              test_append_one_hot_hidden_selects_weight_rows, test_append_brute_force_scalar,
              lambda: test_append_then_decode_equals_direct_cache("tiny_mla_f32_b1_h4_l64")]
    with np.errstate(all="ignore"):
        for c in checks:
            try:
                c()
            except (AssertionError, ValueError, IndexError):
                return False
    return True


def test_append_pins_pass_unplanted():
    assert _append_pins_pass()


@pytest.mark.parametrize("mistake", ["position_plus_one", "not_rotated", "reverse_allocation",
                                     "length_not_bumped", "kr_from_dkv_columns"])
def test_append_planted_mistake_is_caught(monkeypatch, mistake):
    real_rows, real_append = O.latent_rows, O.cache_append
    if mistake == "position_plus_one":
        monkeypatch.setattr(O, "latent_rows", lambda h, wd, wk, pos, theta=1e4: real_rows(
            h, wd, wk, np.asarray(pos) + 1, theta))
    elif mistake == "not_rotated":
        monkeypatch.setattr(O, "latent_rows", lambda h, wd, wk, pos, theta=1e4: real_rows(
            h, wd, wk, np.zeros_like(np.asarray(pos)), theta))
    elif mistake == "kr_from_dkv_columns":
        monkeypatch.setattr(O, "latent_rows", lambda h, wd, wk, pos, theta=1e4: real_rows(
            h, wd, np.asarray(wd)[:, :np.asarray(wk).shape[1]], pos, theta))
    elif mistake == "reverse_allocation":
        def bad(h, wd, wk, lens, bt=None, free=(), **kw):
            lens = list(lens)
            order = list(range(len(lens)))[::-1]  # allocate to the last sequences first
            res = real_append(np.asarray(h)[order], wd, wk, [lens[i] for i in order],
                              None if bt is None else np.asarray(bt)[order], free, **kw)
            inv = np.argsort(order)
            res["rows"], res["seqlens"] = res["rows"][inv], res["seqlens"][inv]
            res["where"] = [res["where"][i] for i in inv]
            res["written"] = res["written"][inv]
            if res["block_table"] is not None:
                res["block_table"] = res["block_table"][inv]
            return res
        monkeypatch.setattr(O, "cache_append", bad)
    elif mistake == "length_not_bumped":
        def bad(*a, **kw):
            res = real_append(*a, **kw)
            res["seqlens"] = np.asarray(a[3])
            return res
        monkeypatch.setattr(O, "cache_append", bad)
    assert not _append_pins_pass()


# ----------------------------------------------------------------------------- variant pins
# Gated output (the MLRA page, section 4: gated attention on MLRA-4) and the folded forms of
# matrix absorption (the yololab page, section 矩陣吸收: W_UK folded into the query's
# projection; W_UV left to the output projection, so the step returns latent-space output).

def test_sigmoid_closed_forms_and_library():
    from scipy.special import expit
    assert O.sigmoid(0.0) == 0.5
    assert abs(O.sigmoid(math.log(3.0)) - 0.75) < 1e-16
    assert abs(O.sigmoid(-math.log(3.0)) - 0.25) < 1e-16
    x = np.concatenate([np.linspace(-40, 40, 801), [-800.0, 800.0, -1e-300, 1e-300]])
    with np.errstate(over="raise"):
        got = O.sigmoid(x)
    assert np.allclose(got, expit(x), rtol=1e-15, atol=0)
    assert np.allclose(O.sigmoid(x) + O.sigmoid(-x), 1.0, rtol=0, atol=4.5e-16)  # two ulps of 1


def test_hand_example_gated_mlra4():
    """The scaled branch sum 163/120 (four width-1 branches) times sigmoid(ln 3) = 3/4, and
    gate 0 halves it: 163/160 and 163/240."""
    scale = 0.25
    r = [1.0, 2.0, 3.0, 4.0]
    qn = np.array([[[math.log(x) / scale] for x in r]])
    qr = np.zeros((1, 2))
    rows = np.array([[1.0, 1.0, 1.0, 1.0, 0.0, 0.0], [0.0] * 6])
    one = np.ones((4, 1, 1, 1))
    kw = dict(d_rope=2, scale=scale, out_scale=0.5, theta=10000.0)
    g3 = O.attend_unabsorbed(qn, qr, rows, one, one, gate=np.array([[math.log(3.0)]]), **kw)
    g0 = O.attend_unabsorbed(qn, qr, rows, one, one, gate=np.zeros((1, 1)), **kw)
    assert abs(g3[0, 0] - float(Fraction(163, 160))) < 1e-15
    assert abs(g0[0, 0] - float(Fraction(163, 240))) < 1e-15


def _brute_gated(qn, qr, rows, w_uk, w_uv, gate, d_rope, scale, out_scale, theta):
    """brute_force's output times 1 / (1 + e^-g), elementwise, in scalar Python."""
    out = brute_force(qn, qr, rows, w_uk, w_uv, d_rope, scale, out_scale, theta)
    return np.array([[o / (1.0 + math.exp(-float(g))) for o, g in zip(orow, grow)]
                     for orow, grow in zip(out, gate)])


@pytest.mark.parametrize("NB", [1, 4])
def test_gate_brute_force(NB):
    rng = np.random.default_rng(31 + NB)
    H, dn, dcb, dr, dv, L = 3, 4, 5, 4, 6, 11
    qn, qr = rng.standard_normal((H, NB, dn)), rng.standard_normal((H, dr))
    rows = rng.standard_normal((L, NB * dcb + dr))
    w_uk = rng.standard_normal((NB, H, dn, dcb))
    w_uv = rng.standard_normal((NB, H, dcb, dv))
    gate = 3.0 * rng.standard_normal((H, dv))
    kw = dict(d_rope=dr, scale=0.3, out_scale=0.5 if NB == 4 else 1.0, theta=10000.0)
    got = O.attend_unabsorbed(qn, qr, rows, w_uk, w_uv, gate=gate, **kw)
    ref = _brute_gated(qn, qr, rows, w_uk, w_uv, gate, dr, 0.3, kw["out_scale"], 1e4)
    assert rel_l2(got, ref) < 1e-12


def test_gate_limits():
    """A gate of +40 leaves the output (to 1 part in 1e17), -40 removes it."""
    w, qn, qr, rows, wk, wv = _mlra_small()
    kw = dict(d_rope=64, scale=w.softmax_scale, out_scale=0.5, theta=1e4, heads=[3, 17])
    plain = O.attend_unabsorbed(qn, qr, rows, wk, wv, **kw)
    up = O.attend_unabsorbed(qn, qr, rows, wk, wv, gate=np.full((32, 128), 40.0), **kw)
    down = O.attend_unabsorbed(qn, qr, rows, wk, wv, gate=np.full((32, 128), -40.0), **kw)
    assert rel_l2(up, plain) < 1e-15
    assert np.abs(down).max() < 1e-17 * np.abs(plain).max() + 1e-300


def _fold_query_py(qn, w_uk):
    """q_lat[h, b*dcb + j] = sum_n q_nope[h, b, n] W_UK[b, h, n, j], as scalar sums."""
    NB, H, dn, dcb = w_uk.shape
    return np.array([[math.fsum(float(qn[h, b, n]) * float(w_uk[b, h, n, j]) for n in range(dn))
                      for b in range(NB) for j in range(dcb)] for h in range(H)])


@pytest.mark.parametrize("NB", [1, 4])
def test_folded_query_equals_unabsorbed(NB):
    """Folding W_UK into the query projection (q_lat = W_UK^T q_nope, here made by scalar
    sums) and scoring q_lat . c gives the same step as the explicitly up-projected keys."""
    rng = np.random.default_rng(41 + NB)
    H, dn, dcb, dr, dv, L = 3, 6, 5, 4, 7, 13
    qn, qr = rng.standard_normal((H, NB, dn)), rng.standard_normal((H, dr))
    rows = rng.standard_normal((L, NB * dcb + dr))
    w_uk = rng.standard_normal((NB, H, dn, dcb))
    w_uv = rng.standard_normal((NB, H, dcb, dv))
    kw = dict(d_rope=dr, scale=0.3, out_scale=0.5 if NB == 4 else 1.0, theta=10000.0)
    ref = brute_force(qn, qr, rows, w_uk, w_uv, dr, 0.3, kw["out_scale"], 1e4)
    got = O.attend_unabsorbed(None, qr, rows, None, w_uv, q_latent=_fold_query_py(qn, w_uk), **kw)
    assert rel_l2(got, ref) < 1e-12


def test_latent_output_single_token_and_uniform():
    """L = 1 returns out_scale times the token's latent; with zero queries every token weighs
    1/L and the output is out_scale times the latent mean (per branch slice)."""
    rng = np.random.default_rng(5)
    NB, H, dn, dcb, dr, L = 4, 2, 3, 5, 4, 9
    rows = rng.standard_normal((L, NB * dcb + dr))
    qn, qr = rng.standard_normal((H, NB, dn)), rng.standard_normal((H, dr))
    w_uk = rng.standard_normal((NB, H, dn, dcb))
    kw = dict(d_rope=dr, scale=0.7, out_scale=0.5, theta=1e4, latent_out=True, w_uv=None)
    one = O.attend_unabsorbed(qn, qr, rows[:1], w_uk, **kw)
    assert np.array_equal(one, np.tile(0.5 * rows[0, :NB * dcb], (H, 1)))
    uni = O.attend_unabsorbed(np.zeros_like(qn), np.zeros_like(qr), rows, w_uk, **kw)
    mean = np.array([math.fsum(rows[t, j] for t in range(L)) / L for j in range(NB * dcb)])
    assert np.allclose(uni, np.tile(0.5 * mean, (H, 1)), rtol=1e-14, atol=1e-15)


@pytest.mark.parametrize("NB", [1, 4])
def test_latent_output_times_w_uv_equals_unabsorbed(NB):
    """The latent output contracted with each branch's W_UV (scalar sums) and added over the
    branches is the plain step's output."""
    rng = np.random.default_rng(51 + NB)
    H, dn, dcb, dr, dv, L = 2, 4, 6, 2, 5, 10
    qn, qr = rng.standard_normal((H, NB, dn)), rng.standard_normal((H, dr))
    rows = rng.standard_normal((L, NB * dcb + dr))
    w_uk = rng.standard_normal((NB, H, dn, dcb))
    w_uv = rng.standard_normal((NB, H, dcb, dv))
    kw = dict(d_rope=dr, scale=0.4, out_scale=0.5 if NB == 4 else 1.0, theta=1e4)
    lat = O.attend_unabsorbed(qn, qr, rows, w_uk, None, latent_out=True, **kw)
    proj = np.array([[math.fsum(float(lat[h, b * dcb + j]) * float(w_uv[b, h, j, v])
                                for b in range(NB) for j in range(dcb)) for v in range(dv)]
                     for h in range(H)])
    ref = brute_force(qn, qr, rows, w_uk, w_uv, dr, 0.4, kw["out_scale"], 1e4)
    assert rel_l2(proj, ref) < 1e-12


def test_latent_output_rejects_gate():
    rng = np.random.default_rng(0)
    with pytest.raises(ValueError):
        O.attend_unabsorbed(rng.standard_normal((1, 1, 2)), np.zeros((1, 2)),
                            rng.standard_normal((3, 6)), rng.standard_normal((1, 1, 2, 4)), None,
                            d_rope=2, scale=1.0, out_scale=1.0, theta=1e4, latent_out=True,
                            gate=np.zeros((1, 4)))


def test_variant_batch_entry_matches_per_sequence():
    """mla_decode passes the variants through per sequence (stored bf16 inputs; gate
    [B, H, d_v], folded query [B, H, NB*d_cb], latent output)."""
    w = I.WORKLOADS["mlra4_bf16_b32_h32_l8192"]
    inp = I.make_inputs(w, seed=3, seqlens=[70, 1, 33])
    f64 = lambda a: I.to_f64(a, "bf16")
    qn, qr, wk, wv = f64(inp["q_nope"]), f64(inp["q_rope"]), f64(inp["w_uk"]), f64(inp["w_uv"])
    gate = I.to_storage(np.random.default_rng(2).standard_normal((3, w.heads, w.d_v)), "bf16")
    qlat = I.to_storage(np.einsum("bhkn,khnj->bhkj", qn, wk).reshape(3, w.heads, 4 * w.d_cb),
                        "bf16")
    kw = dict(d_rope=64, scale=w.softmax_scale, out_scale=0.5, theta=1e4, heads=[0, 31],
              to_f64=f64)
    args = (inp["cache"], inp["seqlens"])
    got_g = O.mla_decode(inp["q_nope"], inp["q_rope"], *args, inp["w_uk"], inp["w_uv"],
                         gate=gate, **kw)
    got_q = O.mla_decode(qlat, inp["q_rope"], *args, None, inp["w_uv"], q_latent=True, **kw)
    got_l = O.mla_decode(inp["q_nope"], inp["q_rope"], *args, inp["w_uk"], None,
                         latent_out=True, **kw)
    one = dict(d_rope=64, scale=w.softmax_scale, out_scale=0.5, theta=1e4, heads=[0, 31])
    for b, L in enumerate(inp["seqlens"]):
        rows = f64(inp["cache"][b, :L])
        a = O.attend_unabsorbed(qn[b], qr[b], rows, wk, wv, **one)
        assert rel_l2(got_g[b], a * O.sigmoid(f64(gate)[b, [0, 31]])) < 1e-13
        aq = O.attend_unabsorbed(None, qr[b], rows, None, wv, q_latent=f64(qlat)[b], **one)
        assert np.array_equal(got_q[b], aq) and rel_l2(aq, a) < 2e-2
        lat = O.attend_unabsorbed(qn[b], qr[b], rows, wk, None, latent_out=True, **one)
        assert np.array_equal(got_l[b], lat)


def _variant_pins_pass():
    checks = [test_hand_example_gated_mlra4, lambda: test_gate_brute_force(4),
              test_latent_output_single_token_and_uniform,
              lambda: test_folded_query_equals_unabsorbed(4),
              lambda: test_latent_output_times_w_uv_equals_unabsorbed(4)]
    with np.errstate(all="ignore"):
        for c in checks:
            try:
                c()
            except (AssertionError, ValueError, IndexError):
                return False
    return True


def test_variant_pins_pass_unplanted():
    assert _variant_pins_pass()


@pytest.mark.parametrize("mistake", ["sigmoid_sign", "gate_before_scale_as_add",
                                     "folded_query_branch0", "latent_out_branch_sum"])
def test_variant_planted_mistake_is_caught(monkeypatch, mistake):
    real = O.attend_unabsorbed
    if mistake == "sigmoid_sign":
        real_sig = O.sigmoid
        monkeypatch.setattr(O, "sigmoid", lambda x: real_sig(-np.asarray(x)))
    elif mistake == "gate_before_scale_as_add":
        def bad(*a, gate=None, **kw):
            out = real(*a, **kw)
            return out if gate is None else out + O.sigmoid(gate)
        monkeypatch.setattr(O, "attend_unabsorbed", bad)
    elif mistake == "folded_query_branch0":
        def bad(*a, q_latent=None, **kw):
            if q_latent is not None:
                d = q_latent.shape[1]
                nb = kw.get("branches") or (a[4].shape[0] if a[4] is not None else 1)
                q_latent = np.tile(q_latent[:, : d // nb], (1, nb))
            return real(*a, q_latent=q_latent, **kw)
        monkeypatch.setattr(O, "attend_unabsorbed", bad)
    elif mistake == "latent_out_branch_sum":
        def bad(*a, latent_out=False, **kw):
            out = real(*a, latent_out=latent_out, **kw)
            if latent_out:
                nb = a[3].shape[0]
                d = out.shape[1] // nb
                out = np.tile(out.reshape(out.shape[0], nb, d).sum(1), (1, nb))
            return out
        monkeypatch.setattr(O, "attend_unabsorbed", bad)
    assert not _variant_pins_pass()


# ----------------------------------------------------------------------------- several query tokens
# s_q new tokens per sequence decoded in one step (the compute-heavier regime of the yololab
# page, section 繁榮背後的代價): token i sits at L - s_q + i and attends causally.

def _brute_multi(qn, qr, rows, w_uk, w_uv, sq, d_rope, scale, out_scale, theta):
    """Scalar loops over the whole cache with an explicit causal mask: query token i scores
    every token t < L and drops those with t > L - s_q + i (weight exactly 0), its rotary part
    at position L - s_q + i; softmax as 1 / sum_j exp(s_j - s_t) over the kept tokens."""
    NB, Hw, dn, dcb = w_uk.shape
    dv = w_uv.shape[-1]
    L = len(rows)
    res = []
    for r in range(sq * Hw):
        i, h = divmod(r, Hw)
        pos = L - sq + i
        kept = [t for t in range(L) if t <= pos]
        if not kept:
            res.append([0.0] * dv)
            continue
        qrot = _rotate_py(list(qr[r]), pos, theta)
        acc = [[] for _ in range(dv)]
        for br in range(NB):
            scores, vals = {}, {}
            for t in kept:
                c = [float(v) for v in rows[t][br * dcb:(br + 1) * dcb]]
                K = [math.fsum(float(w_uk[br, h, n, j]) * c[j] for j in range(dcb)) for n in range(dn)]
                krot = _rotate_py([float(v) for v in rows[t][NB * dcb:NB * dcb + d_rope]], t, theta)
                scores[t] = scale * (math.fsum(float(qn[r, br, n]) * K[n] for n in range(dn))
                                     + math.fsum(qrot[k] * krot[k] for k in range(d_rope)))
                vals[t] = [math.fsum(float(w_uv[br, h, j, v]) * c[j] for j in range(dcb))
                           for v in range(dv)]
            for t in kept:
                p = 1.0 / math.fsum(math.exp(scores[j] - scores[t]) for j in kept)
                for v in range(dv):
                    acc[v].append(p * vals[t][v])
        res.append([out_scale * math.fsum(a) for a in acc])
    return np.array(res)


@pytest.mark.parametrize("NB,sq,L", [(1, 2, 7), (4, 3, 6), (1, 4, 2), (1, 3, 3)])
def test_multi_query_brute_force(NB, sq, L):
    """Against the masked brute force, including L < s_q (the first rows see nothing) and
    L = s_q (the first row sees one token)."""
    rng = np.random.default_rng(61 + 10 * NB + sq)
    Hw, dn, dcb, dr, dv = 2, 3, 4, 4, 5
    qn = rng.standard_normal((1, sq * Hw, NB, dn))
    qr = rng.standard_normal((1, sq * Hw, dr))
    cache = rng.standard_normal((1, L, NB * dcb + dr))
    w_uk = rng.standard_normal((NB, Hw, dn, dcb))
    w_uv = rng.standard_normal((NB, Hw, dcb, dv))
    kw = dict(d_rope=dr, scale=0.4, out_scale=0.5 if NB == 4 else 1.0, theta=1e4)
    got = O.mla_decode(qn, qr, cache, [L], w_uk, w_uv, num_queries=sq, **kw)[0]
    ref = _brute_multi(qn[0], qr[0], cache[0], w_uk, w_uv, sq, dr, 0.4, kw["out_scale"], 1e4)
    assert np.abs(got - ref).max() <= 1e-12 * max(1.0, np.abs(ref).max())


def test_multi_query_hand_example():
    """One head, width-1 latent, rope zero, W_UK = 1/3, W_UV = 1, cache values (3, -1), so
    the keys are (1, -1/3); L = 2, s_q = 2.  Query 0 sees token 0 only and returns its value
    3 exactly; query 1 = -3 ln3 / 4 has logits (-3 ln3 / 4, ln3 / 4), weights (1/4, 3/4) and
    output 3/4 - 3/4 = 0."""
    qn = np.array([[[[5.0]], [[-0.75 * math.log(3.0)]]]])  # [B=1, s_q*H=2, NB=1, d_nope=1]
    qr = np.zeros((1, 2, 2))
    cache = np.array([[[3.0, 0.0, 0.0], [-1.0, 0.0, 0.0]]])
    w_uk = np.array([[[[1.0 / 3.0]]]])
    w_uv = np.ones((1, 1, 1, 1))
    out = O.mla_decode(qn, qr, cache, [2], w_uk, w_uv, d_rope=2, scale=1.0, num_queries=2)[0]
    assert out[0, 0] == 3.0
    assert abs(out[1, 0]) < 1e-15


def test_multi_query_last_row_is_plain_decode_and_causality():
    """The last query token's rows equal the one-token decode of the same cache; a change to
    cache rows past L_i leaves query i's rows unchanged and changes the later ones."""
    w = I.WORKLOADS["mlra4_bf16_b32_h32_l8192"]
    inp = I.make_inputs(w, seed=8, seqlens=[40])
    f64 = lambda a: I.to_f64(a, "bf16")
    sq = 3
    rng = np.random.default_rng(1)
    qn = rng.standard_normal((1, sq * w.heads, 4, 128)) / math.sqrt(128)
    qr = rng.standard_normal((1, sq * w.heads, 64)) / 8.0
    cache = f64(inp["cache"])
    wk, wv = f64(inp["w_uk"]), f64(inp["w_uv"])
    kw = dict(d_rope=64, scale=w.softmax_scale, out_scale=0.5, theta=1e4)
    heads = [0, 31, 32, 63, 64, 95]
    multi = O.mla_decode(qn, qr, cache, [40], wk, wv, num_queries=sq, heads=heads, **kw)[0]
    last = O.mla_decode(qn[:, 2 * 32:], qr[:, 2 * 32:], cache, [40], wk, wv, heads=[0, 31], **kw)[0]
    assert np.array_equal(multi[4:], last)
    changed = cache.copy()
    changed[0, 38] += 1.0                  # L_i = 38, 39, 40: queries 1 and 2 see token 38
    after = O.mla_decode(qn, qr, changed, [40], wk, wv, num_queries=sq, heads=heads, **kw)[0]
    assert np.array_equal(after[:2], multi[:2])        # query 0 sees tokens 0..37
    assert not np.allclose(after[2:], multi[2:])       # queries 1, 2 see token 38


def _multi_pins_pass():
    checks = [lambda: test_multi_query_brute_force(4, 3, 6), lambda: test_multi_query_brute_force(1, 4, 2),
              test_multi_query_hand_example, test_multi_query_last_row_is_plain_decode_and_causality]
    with np.errstate(all="ignore"):
        for c in checks:
            try:
                c()
            except (AssertionError, ValueError, IndexError):
                return False
    return True


def test_multi_pins_pass_unplanted():
    assert _multi_pins_pass()


@pytest.mark.parametrize("mistake", ["not_causal", "query_rotated_one_late", "off_by_one_limit"])
def test_multi_planted_mistake_is_caught(monkeypatch, mistake):
    real_rows = O.sequence_rows
    if mistake == "not_causal":
        # every query token sees the whole cache (its rotary position stays L_i - 1)
        def bad(cache, b, L, *a, **k):
            return real_rows(cache, b, np.shape(cache)[1] if np.ndim(cache) == 3 else L, *a, **k)
        monkeypatch.setattr(O, "sequence_rows", bad)
    elif mistake == "query_rotated_one_late":
        real_rope = O.rope
        monkeypatch.setattr(O, "rope", lambda x, pos, theta=1e4: real_rope(
            x, pos if np.ndim(pos) else pos + 1, theta))
    elif mistake == "off_by_one_limit":
        def bad(cache, b, L, *a, **k):
            return real_rows(cache, b, max(0, L - 1) if L else 0, *a, **k)
        monkeypatch.setattr(O, "sequence_rows", bad)
    assert not _multi_pins_pass()


# ----------------------------------------------------------------------------- fp8 latent storage
# OCP FP8 E4M3 ("e4m3fn"): the storage format of an fp8 latent cache.  The decode feeds the
# oracle the exact cached values; pinned here against the format's closed forms and a brute
# force over its grid.

def test_e4m3_decode_closed_forms():
    d = I.e4m3_bits_to_f64
    cases = {0x00: 0.0, 0x38: 1.0, 0x7e: 448.0, 0x08: 2.0 ** -6, 0x01: 2.0 ** -9,
             0x07: 7 * 2.0 ** -9, 0xc0: -2.0, 0x3c: 1.5, 0x46: 3.5, 0xfe: -448.0}
    for code, val in cases.items():
        assert d(np.array([code], np.uint8))[0] == val, hex(code)
    assert np.isnan(d(np.array([0x7f, 0xff], np.uint8))).all()
    neg0 = d(np.array([0x80], np.uint8))[0]
    assert neg0 == 0.0 and math.copysign(1.0, neg0) < 0
    v = d(np.arange(0x7f, dtype=np.uint8))
    assert np.all(np.diff(v) > 0)        # codes 0 .. 0x7e increase strictly
    assert len(set(v.tolist())) == 127


def test_e4m3_encode_is_nearest_with_ties_to_even():
    grid = I.e4m3_bits_to_f64(np.arange(0x7f, dtype=np.uint8))
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.standard_normal(3000) * 30, rng.standard_normal(1000) * 0.01,
                        (grid[:-1] + grid[1:]) / 2, -(grid[:-1] + grid[1:]) / 2,
                        [500.0, -1e6, 0.0]])
    got = I.e4m3_bits_to_f64(I.f64_to_e4m3_bits(x))
    for xi, gi in zip(x, got):
        a = min(abs(xi), 448.0)
        dist = np.abs(grid - a)
        best = np.flatnonzero(dist == dist.min())
        k = best[0] if len(best) == 1 else best[best % 2 == 0][0]  # tie: the even code
        assert abs(gi) == grid[k] and (gi == 0 or math.copysign(1.0, gi) == math.copysign(1.0, xi)), (xi, gi)


def test_e4m3_round_trip_and_saturation():
    codes = np.array([c for c in range(256) if c not in (0x7f, 0xff)], np.uint8)
    v = I.e4m3_bits_to_f64(codes)
    assert np.array_equal(I.e4m3_bits_to_f64(I.f64_to_e4m3_bits(v)), v)
    assert I.e4m3_bits_to_f64(I.f64_to_e4m3_bits(np.array([1e9, -1e9])) ).tolist() == [448.0, -448.0]


# ----------------------------------------------------------------------------- prefill
# The s_q newest tokens of each sequence attend causally over the cache, up-projected once per
# head (the interview Q&A's 核心机制 step 3, in the many-query regime of the yololab page's
# 繁榮背後的代價 section).  O.mla_prefill computes all query tokens of a head at once; it is
# pinned against the scalar masked brute force, the per-row decode oracle (itself pinned
# above, for MLA and for the four MLRA branches), an exact first-token form, causality and
# the one-live-branch reduction.

def _prefill_case(sq, L, Hw=2, dn=3, dc=4, dr=4, dv=5, seed=0):
    rng = np.random.default_rng(seed + 100 * sq + L)
    qn = rng.standard_normal((1, sq * Hw, 1, dn))
    qr = rng.standard_normal((1, sq * Hw, dr))
    cache = rng.standard_normal((1, max(L, 1), dc + dr))
    w_uk = rng.standard_normal((1, Hw, dn, dc))
    w_uv = rng.standard_normal((1, Hw, dc, dv))
    return qn, qr, cache, w_uk, w_uv


@pytest.mark.parametrize("sq,L", [(2, 7), (4, 2), (3, 3), (5, 9), (1, 4)])
def test_prefill_brute_force(sq, L):
    """Against the scalar masked brute force, with L < s_q (early rows see nothing), L = s_q
    (the first row sees one token) and s_q = 1 (a plain decode)."""
    qn, qr, cache, w_uk, w_uv = _prefill_case(sq, L)
    got = O.mla_prefill(qn, qr, cache, [L], w_uk, w_uv, num_queries=sq, d_rope=4, scale=0.4,
                        out_scale=0.7, theta=1e4)[0]
    ref = _brute_multi(qn[0], qr[0], cache[0, :L], w_uk, w_uv, sq, 4, 0.4, 0.7, 1e4)
    assert np.abs(got - ref).max() <= 1e-12 * max(1.0, np.abs(ref).max())


def test_prefill_equals_per_row_decode_paged():
    """Workload dimensions (128 heads, latent 512, rope 64, bf16 values, paged, shuffled), two
    sequences of different lengths, a sample of query rows: equal to the per-row multi-query
    decode oracle to fp64 rounding."""
    w = I.WORKLOADS["mla_bf16_paged_b4_h128_l131072"]
    sq = 6
    inp = I.make_inputs(w, seed=3, seqlens=[70, 9])
    f64 = lambda a: I.to_f64(a, "bf16")
    rng = np.random.default_rng(2)
    qn = rng.standard_normal((2, sq * w.heads, 1, 128)) / math.sqrt(128)
    qr = rng.standard_normal((2, sq * w.heads, 64)) / 8.0
    kw = dict(d_rope=64, scale=w.softmax_scale, out_scale=1.0, theta=1e4,
              page_size=inp["page_size"], block_table=inp["block_table"], to_f64=f64)
    rows = [0, 127, 128 + 5, 3 * 128 + 64, 5 * 128 + 127]
    a = O.mla_prefill(qn, qr, inp["cache"], inp["seqlens"], inp["w_uk"], inp["w_uv"],
                      num_queries=sq, heads=rows, **kw)
    b = O.mla_decode(qn, qr, inp["cache"], inp["seqlens"], inp["w_uk"], inp["w_uv"],
                     num_queries=sq, heads=rows, **kw)
    assert np.abs(a - b).max() <= 1e-12 * np.abs(b).max()


def test_prefill_first_token_is_its_value():
    """L = s_q: query token 0 sees token 0 alone, its weight is exactly 1, and its output is
    out_scale * c_0 W_UV for every head."""
    sq = L = 4
    qn, qr, cache, w_uk, w_uv = _prefill_case(sq, L, Hw=3)
    out = O.mla_prefill(qn, qr, cache, [L], w_uk, w_uv, num_queries=sq, d_rope=4, scale=0.9,
                        out_scale=0.5, theta=1e4)[0]
    for h in range(3):
        exp = 0.5 * cache[0, 0, :4] @ w_uv[0, h]
        assert np.abs(out[h] - exp).max() <= 1e-14 * max(1.0, np.abs(exp).max())


def test_prefill_causality():
    """A change to cache row t changes exactly the query rows at positions >= t."""
    sq, L = 5, 8
    qn, qr, cache, w_uk, w_uv = _prefill_case(sq, L)
    kw = dict(num_queries=sq, d_rope=4, scale=0.4, theta=1e4)
    base = O.mla_prefill(qn, qr, cache, [L], w_uk, w_uv, **kw)[0]
    t = 5                                  # positions of the query tokens: 3 .. 7
    changed = cache.copy()
    changed[0, t] += 1.0
    after = O.mla_prefill(qn, qr, changed, [L], w_uk, w_uv, **kw)[0]
    for r in range(sq * 2):
        pos = L - sq + r // 2
        if pos < t:
            assert np.array_equal(after[r], base[r])
        else:
            assert not np.allclose(after[r], base[r])


def _mlra_prefill_case(sq, L, Hw=2, NB=4, dn=3, dcb=4, dr=4, dv=5, seed=0):
    rng = np.random.default_rng(seed + 1000 + 100 * sq + L)
    qn = rng.standard_normal((1, sq * Hw, NB, dn))
    qr = rng.standard_normal((1, sq * Hw, dr))
    cache = rng.standard_normal((1, max(L, 1), NB * dcb + dr))
    w_uk = rng.standard_normal((NB, Hw, dn, dcb))
    w_uv = rng.standard_normal((NB, Hw, dcb, dv))
    return qn, qr, cache, w_uk, w_uv


@pytest.mark.parametrize("sq,L", [(3, 7), (4, 2), (1, 5)])
def test_prefill_mlra_equals_per_row_decode(sq, L):
    """Four branches (MLRA): equal to the per-row multi-query decode oracle, whose branch sum
    is pinned above (hand-worked 163/120 example, one-live-branch and identical-branch
    reductions), to fp64 rounding."""
    qn, qr, cache, w_uk, w_uv = _mlra_prefill_case(sq, L)
    kw = dict(num_queries=sq, d_rope=4, scale=0.4, out_scale=0.5, theta=1e4)
    a = O.mla_prefill(qn, qr, cache, [L], w_uk, w_uv, **kw)
    b = O.mla_decode(qn, qr, cache, [L], w_uk, w_uv, **kw)
    assert np.abs(a - b).max() <= 1e-12 * max(1.0, np.abs(b).max())


def test_prefill_mlra_one_live_branch_is_mla_on_it():
    """Branches 0, 1 and 3 with zero W_UV contribute nothing: the result is the one-branch
    prefill of branch 2 alone (its latent slice, its query, its weights) times out_scale."""
    sq, L = 4, 6
    qn, qr, cache, w_uk, w_uv = _mlra_prefill_case(sq, L)
    w_uv = w_uv.copy()
    w_uv[[0, 1, 3]] = 0.0
    kw = dict(num_queries=sq, d_rope=4, scale=0.4, theta=1e4)
    got = O.mla_prefill(qn, qr, cache, [L], w_uk, w_uv, out_scale=0.5, **kw)
    one = np.concatenate([cache[:, :, 8:12], cache[:, :, 16:]], axis=-1)
    ref = O.mla_prefill(qn[:, :, 2:3], qr, one, [L], w_uk[2:3], w_uv[2:3], out_scale=0.5, **kw)
    assert np.abs(got - ref).max() <= 1e-12 * max(1.0, np.abs(ref).max())


def _prefill_pins_pass():
    checks = [lambda: test_prefill_brute_force(2, 7), lambda: test_prefill_brute_force(4, 2),
              test_prefill_first_token_is_its_value, test_prefill_causality,
              lambda: test_prefill_mlra_equals_per_row_decode(3, 7),
              test_prefill_mlra_one_live_branch_is_mla_on_it]
    with np.errstate(all="ignore"):
        for c in checks:
            try:
                c()
            except (AssertionError, ValueError, IndexError):
                return False
    return True


def test_prefill_pins_pass_unplanted():
    assert _prefill_pins_pass()


@pytest.mark.parametrize("mistake,old,new", [
    ("not_causal", "np.arange(L)[None, :] > pos[:, None]", "np.zeros((sq, L), dtype=bool)"),
    ("mask_off_by_one", "np.arange(L)[None, :] > pos[:, None]", "np.arange(L)[None, :] >= pos[:, None]"),
    ("queries_at_last_position", "q_r = rope(qr[b, h::Hw], pos, theta)",
     "q_r = rope(qr[b, h::Hw], np.full(sq, L - 1), theta)"),
    ("values_from_keys", "V = c @ W_UV[br, h]", "V = (c @ W_UK[br, h].T)[:, :1] * np.ones((1, d_v))"),
    ("branch_query_of_branch_0", "q_n = qn[b, h::Hw, br]", "q_n = qn[b, h::Hw, 0]"),
    ("latent_slice_of_branch_0", "c = lat[:, br * d_cb:(br + 1) * d_cb]", "c = lat[:, :d_cb]"),
    ("keys_of_branch_0", "K = c @ W_UK[br, h].T", "K = c @ W_UK[0, h].T"),
    ("branches_not_summed", "O[seen] += softmax(S[seen]) @ V", "O[seen] = softmax(S[seen]) @ V"),
])
def test_prefill_planted_mistake_is_caught(monkeypatch, mistake, old, new):
    """Each mistake is planted in a copy of the oracle's prefill, on the CPU."""
    import inspect
    import textwrap
    src = textwrap.dedent(inspect.getsource(O.mla_prefill))
    assert old in src
    ns = dict(vars(O))
    exec(src.replace(old, new), ns)
    monkeypatch.setattr(O, "mla_prefill", ns["mla_prefill"])
    assert not _prefill_pins_pass()
