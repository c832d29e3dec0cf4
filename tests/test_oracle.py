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
