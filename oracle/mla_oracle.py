"""fp64 CPU oracle for MLA / MLRA-4 decode attention over a latent KV cache.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports, calls or links
this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may use it. It shares no code with the
HIP path and does not import ``mlra_latent_kv_amd``.

What it computes is the plain, *un-absorbed* definition of one decode step:
read each token's compressed latent from the cache and explicitly
up-project it to per-head keys and values; add the decoupled rotary term;
then run ordinary softmax attention. For MLRA each branch attends on its own
and the branch outputs are summed with a scale.  Sources (page title, section):

* "MLA (Multi-head Latent Attention) 是什么" (interview Q&A), section
  "核心机制", step 3 "计算": at inference the latent is read from the cache,
  up-projected with W_K_up / W_V_up to full keys and values, and attended with
  the query.
* "超越 GQA 的推理革命…MLA…" (yololab), section "鍵值聯合低秩壓縮": one joint
  latent c_KV per token is cached, and restored by an up-projection when
  scores are computed; section "解耦旋轉位置編碼": the position part is a
  separate uncompressed key carrying RoPE that joins the score directly.
* "多头潜在注意力机制…" (yunthe), section 二.1: attention is
  Softmax(Q K^T / sqrt(d)) V.
* "[ICLR 2025] MLRA…" (wispaper), section 2.1: the KV projection is split into
  independent branches, each with its own latent head; each branch computes
  its own attention output; the final output is a weighted sum of the
  branch outputs. Section 2.2 gives a variance-calibration scale whose
  formula is lost from the page; the scale is taken as the ``out_scale``
  argument (0.5 for four branches).
* RoPE follows RoFormer (cited in the interview Q&A's references): pairs
  (x_{2i}, x_{2i+1}) rotate by angle pos * theta^(-2i/d_rope).

Readings where the pages are silent (each is an argument, not hidden):
  the softmax scale is an argument (default 1/sqrt(d_nope + d_rope));
  the cached rope key is rotated at its own position t, the query at L - 1;
  one q_nope per (head, branch) and one q_rope per head shared by branches;
  L = 0 gives a zero output.

Layouts (the library's ABI layouts):
  q_nope [B, H, NB, d_nope]; q_rope [B, H, d_rope] (un-rotated);
  cache rows [c_KV (NB*d_cb) | k_rope_raw (d_rope)], contiguous [B, Lmax, row]
  or paged pool [P, page, row] addressed through block_table [B, pages];
  w_uk [NB, H, d_nope, d_cb]  (K_{h,b,t} = w_uk[b,h] @ c_{b,t});
  w_uv [NB, H, d_cb, d_v]     (V_{h,b,t} = w_uv[b,h]^T @ c_{b,t});
  output [B, H, d_v].
"""

from __future__ import annotations

from typing import Callable, Iterable, Optional

import numpy as np

F64 = np.float64


def _as_f64(a) -> np.ndarray:
    return np.asarray(a, dtype=F64)


# ----------------------------------------------------------------------------- RoPE

def rope_frequencies(d_rope: int, theta: float) -> np.ndarray:
    """theta_i = theta^(-2i/d_rope), i = 0 .. d_rope/2 - 1 (RoFormer)."""
    i = np.arange(d_rope // 2, dtype=F64)
    return np.power(F64(theta), -2.0 * i / d_rope)


def rope(x, pos, theta: float = 10000.0) -> np.ndarray:
    """Rotate consecutive pairs (x_{2i}, x_{2i+1}) of the last axis by pos * theta_i.

    ``pos`` broadcasts against ``x.shape[:-1]``. Angles and the rotation are fp64.
    """
    x = _as_f64(x)
    d = x.shape[-1]
    ang = np.asarray(pos, dtype=F64)[..., None] * rope_frequencies(d, theta)
    c, s = np.cos(ang), np.sin(ang)
    xe, xo = x[..., 0::2], x[..., 1::2]
    out = np.empty(np.broadcast_shapes(x.shape, ang.shape[:-1] + (d,)), dtype=F64)
    out[..., 0::2] = xe * c - xo * s
    out[..., 1::2] = xe * s + xo * c
    return out


# ----------------------------------------------------------------------------- cache access

def sequence_rows(cache, b: int, L: int, page_size: int = 0, block_table=None,
                  to_f64: Callable = _as_f64) -> np.ndarray:
    """Rows 0..L-1 of sequence b in logical order, as fp64 [L, row].

    Contiguous cache: cache[b, t].  Paged: cache[block_table[b, t // page], t % page].
    """
    if L == 0:
        return np.zeros((0, cache.shape[-1]), dtype=F64)
    if not page_size:
        return to_f64(cache[b, :L])
    npg = (L + page_size - 1) // page_size
    pages = np.asarray(block_table[b, :npg], dtype=np.int64)
    if (pages < 0).any() or (pages >= cache.shape[0]).any():
        raise IndexError("block table entry out of range for a used page")
    rows = cache[pages].reshape(npg * page_size, cache.shape[-1])[:L]
    return to_f64(rows)


# ----------------------------------------------------------------------------- attention

def softmax(s: np.ndarray) -> np.ndarray:
    """Plain softmax along the last axis, max-subtracted, fp64."""
    e = np.exp(s - s.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def attend_unabsorbed(q_nope, q_rope, rows, w_uk, w_uv, *, d_rope: int, scale: float,
                      out_scale: float, theta: float, heads: Optional[Iterable[int]] = None,
                      return_probs: bool = False):
    """One sequence, un-absorbed.

    q_nope [H, NB, d_nope], q_rope [H, d_rope] (raw), rows [L, NB*d_cb + d_rope] (rope raw),
    w_uk [NB, H, d_nope, d_cb], w_uv [NB, H, d_cb, d_v].  Returns out [len(heads), d_v]
    (and probabilities [len(heads), NB, L] if ``return_probs``).
    """
    q_nope, q_rope, rows = _as_f64(q_nope), _as_f64(q_rope), _as_f64(rows)
    NB, H, d_nope, d_cb = w_uk.shape
    d_v = w_uv.shape[-1]
    heads = list(range(H)) if heads is None else list(heads)
    L = rows.shape[0]
    out = np.zeros((len(heads), d_v), dtype=F64)
    probs = np.zeros((len(heads), NB, L), dtype=F64)
    if L == 0:
        return (out, probs) if return_probs else out
    lat = rows[:, : NB * d_cb]
    k_rot = rope(rows[:, NB * d_cb: NB * d_cb + d_rope], np.arange(L), theta)  # keys at position t
    for j, h in enumerate(heads):
        q_rot = rope(q_rope[h], L - 1, theta)                                   # query at L - 1
        rope_score = k_rot @ q_rot
        acc = np.zeros(d_v, dtype=F64)
        for br in range(NB):
            c = lat[:, br * d_cb:(br + 1) * d_cb]                               # [L, d_cb]
            K = c @ _as_f64(w_uk[br, h]).T                                      # [L, d_nope] up-projected keys
            V = c @ _as_f64(w_uv[br, h])                                        # [L, d_v] up-projected values
            s = scale * (K @ q_nope[h, br] + rope_score)
            p = softmax(s)
            probs[j, br] = p
            acc += p @ V
        out[j] = out_scale * acc
    return (out, probs) if return_probs else out


def attend_absorbed(q_nope, q_rope, rows, w_uk, w_uv, *, d_rope: int, scale: float,
                    out_scale: float, theta: float, heads: Optional[Iterable[int]] = None):
    """Same step with W_UK folded into the query and W_UV applied after attention.

    By associativity q.(W_UK c) = (W_UK^T q).c and sum_t p_t (W_UV^T c_t) = W_UV^T (sum_t p_t c_t),
    which is the matrix absorption of the yololab page (section "矩陣吸收").  In exact
    arithmetic it equals ``attend_unabsorbed``; it is an oracle cross-check only.
    """
    q_nope, q_rope, rows = _as_f64(q_nope), _as_f64(q_rope), _as_f64(rows)
    NB, H, d_nope, d_cb = w_uk.shape
    d_v = w_uv.shape[-1]
    heads = list(range(H)) if heads is None else list(heads)
    L = rows.shape[0]
    out = np.zeros((len(heads), d_v), dtype=F64)
    if L == 0:
        return out
    lat = rows[:, : NB * d_cb]
    k_rot = rope(rows[:, NB * d_cb: NB * d_cb + d_rope], np.arange(L), theta)
    for j, h in enumerate(heads):
        q_rot = rope(q_rope[h], L - 1, theta)
        rope_score = k_rot @ q_rot
        for br in range(NB):
            c = lat[:, br * d_cb:(br + 1) * d_cb]
            q_lat = _as_f64(w_uk[br, h]).T @ q_nope[h, br]                     # [d_cb]
            p = softmax(scale * (c @ q_lat + rope_score))
            o_lat = p @ c                                                       # [d_cb]
            out[j] += o_lat @ _as_f64(w_uv[br, h])
        out[j] *= out_scale
    return out


def mla_decode(q_nope, q_rope, cache, seqlens, w_uk, w_uv, *, d_rope: int, scale: float,
               out_scale: float = 1.0, theta: float = 10000.0, page_size: int = 0,
               block_table=None, to_f64: Callable = _as_f64,
               batches: Optional[Iterable[int]] = None, heads: Optional[Iterable[int]] = None,
               absorbed: bool = False) -> np.ndarray:
    """Decode step for a batch: out [len(batches), len(heads), d_v] in fp64.

    ``to_f64`` decodes stored cache rows (fp32 or bf16 bits) to float64; it is
    applied to one sequence's rows at a time.  ``batches`` / ``heads`` select
    a sample of outputs (each output is computed on its own, so a sample costs
    only its share).
    """
    w_uk, w_uv = to_f64(w_uk), to_f64(w_uv)
    qn, qr = to_f64(q_nope), to_f64(q_rope)
    B, H = qn.shape[0], qn.shape[1]
    batches = list(range(B)) if batches is None else list(batches)
    heads = list(range(H)) if heads is None else list(heads)
    f = attend_absorbed if absorbed else attend_unabsorbed
    out = np.zeros((len(batches), len(heads), w_uv.shape[-1]), dtype=F64)
    for i, b in enumerate(batches):
        L = int(seqlens[b])
        rows = sequence_rows(cache, b, L, page_size, block_table, to_f64)
        out[i] = f(qn[b], qr[b], rows, w_uk, w_uv, d_rope=d_rope, scale=scale,
                   out_scale=out_scale, theta=theta, heads=heads)
    return out
