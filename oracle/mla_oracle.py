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

Write side (``latent_rows``, ``cache_append``): at write time each new token's
hidden state is compressed into the joint latent by a down-projection
("超越 GQA 的推理革命…MLA…", section "鍵值聯合低秩壓縮", 寫入時（壓縮）), and the
position part is a separate uncompressed key that carries RoPE (same page,
section "解耦旋轉位置編碼"); MLRA's branches are column blocks of the same
projection ("[ICLR 2025] MLRA…", section 2.1), so the row is computed alike.

Several query tokens per step (``mla_decode(num_queries=s_q)``; the yololab page,
section "繁榮背後的代價…", names the compute-heavy regime that several query rows against one
cache read lead to): each new token attends causally over the cache, which already holds it.
``mla_prefill`` computes the same definition for many new tokens at once (the un-absorbed
prefill: keys and values up-projected once per head, all query tokens scored against them).

Variants of the decode step (``attend_unabsorbed`` / ``mla_decode`` keywords):
* gated output ("[ICLR 2025] MLRA…", section 4: MLRA-4 combined with gated attention):
  each head's output, after the scaled branch sum, is multiplied elementwise by
  sigmoid(gate), the gate logits [B, H, d_v] being an input;
* folded query ("超越 GQA 的推理革命…MLA…", section "矩陣吸收": the key up-projection is
  absorbed into the query's projection): the query arrives as a latent-space vector per
  branch, scored directly against c_KV;
* latent output (same section, the value side): W_UV is left to the output projection it
  can be folded into, and the step returns out_scale times the per-branch attention
  outputs in latent space, side by side.

Readings where the pages are silent (each is an argument, not hidden):
  the gate is a logistic sigmoid of given logits, applied after out_scale and the branch
  sum, one value per output element; a gate and a latent output are not combined;
  with s_q > 1 new tokens per step, query token i sits at L - s_q + i and sees the tokens up
  to itself (the usual causal rule among the new tokens), its rotary query rotated there;
  the cache stores the rotary key already rotated at its own position t;
  a decode step appends its token at t = L_b, then L_b becomes t + 1;
  a sequence whose new token starts a page takes the next entry of a free-page
  list, in batch order; when the list runs out that sequence is not written;
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


def sigmoid(x) -> np.ndarray:
    """Logistic function 1 / (1 + e^-x), fp64, written so that neither branch overflows."""
    x = _as_f64(x)
    e = np.exp(-np.abs(x))
    return np.where(x >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def attend_unabsorbed(q_nope, q_rope, rows, w_uk, w_uv, *, d_rope: int, scale: float,
                      out_scale: float, theta: float, heads: Optional[Iterable[int]] = None,
                      return_probs: bool = False, gate=None, q_latent=None,
                      latent_out: bool = False, branches: Optional[int] = None,
                      d_cb: Optional[int] = None):
    """One sequence, un-absorbed.

    q_nope [H, NB, d_nope], q_rope [H, d_rope] (raw), rows [L, NB*d_cb + d_rope] (rope raw),
    w_uk [NB, H, d_nope, d_cb], w_uv [NB, H, d_cb, d_v].  Returns out [len(heads), d_v]
    (and probabilities [len(heads), NB, L] if ``return_probs``).

    Variants (the MLRA page's gated attention, section 4; the yololab page's folding of the
    up-projections into the neighbouring projections, section "矩陣吸收"):
      gate [H, d_v]: the head's output is multiplied elementwise by sigmoid(gate) after the
        branch sum (gate logits are an input; the projection that makes them is the model's);
      q_latent [H, NB*d_cb]: the query arrives already in latent space, W_UK having been folded
        into the query projection offline, so the content score is q_latent_b . c_b and w_uk
        is not used (may be None);
      latent_out: W_UV is left to a folded output projection, so the result is the attention
        output in latent space, out_scale * [o_0 | ... | o_{NB-1}] with o_b = sum_t p_bt c_bt,
        [len(heads), NB*d_cb]; w_uv is not used (may be None).  Not combined with a gate (the
        gate acts on the up-projected d_v vector).
    ``branches`` / ``d_cb`` give NB and d_cb when neither weight is passed.
    """
    q_rope, rows = _as_f64(q_rope), _as_f64(rows)
    if w_uk is not None:
        NB, H, d_nope, d_cb = w_uk.shape
    elif w_uv is not None:
        NB, H, d_cb = w_uv.shape[:3]
    else:
        NB, H = int(branches), q_rope.shape[0]
    if latent_out and gate is not None:
        raise ValueError("a gate acts on the up-projected output; latent_out has none")
    d_out = NB * d_cb if latent_out else w_uv.shape[-1]
    heads = list(range(H)) if heads is None else list(heads)
    L = rows.shape[0]
    out = np.zeros((len(heads), d_out), dtype=F64)
    probs = np.zeros((len(heads), NB, L), dtype=F64)
    if L == 0:
        return (out, probs) if return_probs else out
    lat = rows[:, : NB * d_cb]
    k_rot = rope(rows[:, NB * d_cb: NB * d_cb + d_rope], np.arange(L), theta)  # keys at position t
    for j, h in enumerate(heads):
        q_rot = rope(q_rope[h], L - 1, theta)                                   # query at L - 1
        rope_score = k_rot @ q_rot
        acc = np.zeros(d_out, dtype=F64)
        for br in range(NB):
            c = lat[:, br * d_cb:(br + 1) * d_cb]                               # [L, d_cb]
            if q_latent is None:
                K = c @ _as_f64(w_uk[br, h]).T                                  # [L, d_nope] up-projected keys
                content = K @ _as_f64(q_nope)[h, br]
            else:
                content = c @ _as_f64(q_latent)[h, br * d_cb:(br + 1) * d_cb]   # folded query
            p = softmax(scale * (content + rope_score))
            probs[j, br] = p
            if latent_out:
                acc[br * d_cb:(br + 1) * d_cb] = p @ c                          # latent-space output
            else:
                V = c @ _as_f64(w_uv[br, h])                                    # [L, d_v] up-projected values
                acc += p @ V
        out[j] = out_scale * acc
        if gate is not None:
            out[j] *= sigmoid(_as_f64(gate)[h])
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
               absorbed: bool = False, gate=None, q_latent: bool = False,
               latent_out: bool = False, branches: Optional[int] = None,
               d_cb: Optional[int] = None, num_queries: int = 1) -> np.ndarray:
    """Decode step for a batch: out [len(batches), len(heads), d_v] in fp64.

    ``to_f64`` decodes stored cache rows (fp32 or bf16 bits) to float64; it is
    applied to one sequence's rows at a time.  ``batches`` / ``heads`` select
    a sample of outputs (each output is computed on its own, so a sample costs
    only its share).  ``gate`` [B, H, d_v], ``q_latent`` (then ``q_nope`` holds the folded
    latent query [B, H, NB*d_cb] and ``w_uk`` may be None) and ``latent_out`` (then ``w_uv`` may
    be None and the output is [.., .., NB*d_cb]) select the variants of ``attend_unabsorbed``.

    ``num_queries`` = s_q > 1: several new tokens per sequence are decoded in one step (the
    cache already holds all of them).  The query rows are then [B, s_q * H, ...], row
    i * H + h being head h of query token i, which sits at position L - s_q + i and attends
    causally to the tokens up to and including itself: L_i = L - s_q + 1 + i of them (none
    when L_i <= 0, giving a zero output).  ``heads`` then selects such rows.
    """
    w_uk = None if w_uk is None else to_f64(w_uk)
    w_uv = None if w_uv is None else to_f64(w_uv)
    qn, qr = to_f64(q_nope), to_f64(q_rope)
    g = None if gate is None else to_f64(gate)
    B, H = qn.shape[0], qn.shape[1]
    batches = list(range(B)) if batches is None else list(batches)
    heads = list(range(H)) if heads is None else list(heads)
    variant = g is not None or q_latent or latent_out
    if absorbed and variant:
        raise ValueError("the absorbed cross-check covers the plain decode only")
    if w_uk is not None:
        nb, dcb = w_uk.shape[0], w_uk.shape[3]
    elif w_uv is not None:
        nb, dcb = w_uv.shape[0], w_uv.shape[2]
    else:
        nb, dcb = int(branches), int(d_cb)
    d_out = nb * dcb if latent_out else w_uv.shape[-1]
    out = np.zeros((len(batches), len(heads), d_out), dtype=F64)
    sq = int(num_queries)
    if sq < 1 or H % sq:
        raise ValueError("num_queries must be >= 1 and divide the query rows")
    if sq > 1:
        if absorbed:
            raise ValueError("the absorbed cross-check covers one query token")
        Hw = H // sq  # heads per query token (the weights' head count)
        out = np.zeros((len(batches), len(heads), d_out), dtype=F64)
        for i, b in enumerate(batches):
            L = int(seqlens[b])
            for j, r in enumerate(heads):
                qi, h = divmod(r, Hw)
                Li = max(0, L - sq + 1 + qi)  # causal: tokens 0 .. L - s_q + qi
                rows = sequence_rows(cache, b, Li, page_size, block_table, to_f64)
                out[i, j] = attend_unabsorbed(
                    None if q_latent else qn[b, qi * Hw:(qi + 1) * Hw], qr[b, qi * Hw:(qi + 1) * Hw],
                    rows, w_uk, w_uv, d_rope=d_rope, scale=scale, out_scale=out_scale,
                    theta=theta, heads=[h],
                    gate=None if g is None else g[b, qi * Hw:(qi + 1) * Hw],
                    q_latent=qn[b, qi * Hw:(qi + 1) * Hw] if q_latent else None,
                    latent_out=latent_out, branches=nb, d_cb=dcb)[0]
        return out
    for i, b in enumerate(batches):
        L = int(seqlens[b])
        rows = sequence_rows(cache, b, L, page_size, block_table, to_f64)
        if absorbed:
            out[i] = attend_absorbed(qn[b], qr[b], rows, w_uk, w_uv, d_rope=d_rope, scale=scale,
                                     out_scale=out_scale, theta=theta, heads=heads)
        else:
            out[i] = attend_unabsorbed(
                None if q_latent else qn[b], qr[b], rows, w_uk, w_uv, d_rope=d_rope,
                scale=scale, out_scale=out_scale, theta=theta, heads=heads,
                gate=None if g is None else g[b], q_latent=qn[b] if q_latent else None,
                latent_out=latent_out, branches=nb, d_cb=dcb)
    return out


def mla_prefill(q_nope, q_rope, cache, seqlens, w_uk, w_uv, *, num_queries: int, d_rope: int,
                scale: float, out_scale: float = 1.0, theta: float = 10000.0, page_size: int = 0,
                block_table=None, to_f64: Callable = _as_f64,
                batches: Optional[Iterable[int]] = None,
                heads: Optional[Iterable[int]] = None) -> np.ndarray:
    """Prefill: the s_q newest tokens of each sequence attend causally over its cache, computed
    the un-absorbed way for all of a head's query tokens at once.

    The yololab page (section "繁榮背後的代價…") names the regime in which many query rows
    meet one cache read; the interview Q&A ("MLA … 是什么", 核心机制 step 3) gives the
    un-absorbed step itself: the cached latents are up-projected to full keys K = c W_UK^T and
    values V = c W_UV once per head, and every query row is scored against them.  Same
    definition, inputs and layouts as ``mla_decode(num_queries=s_q)``: query rows
    [B, s_q * H, ...] with row i * H + h = head h of query token i, which sits at position
    L - s_q + i (rotary part rotated there) and sees tokens 0 .. L - s_q + i; a row that sees no
    token is zero.  With NB latent branches (MLRA, "[ICLR 2025] MLRA…", sections 2.1 and 2.2)
    branch b has its own keys K_b = c_b W_UK[b]^T and values V_b = c_b W_UV[b] from its slice
    c_b of the latent, its own query q_nope[.., b, :] and its own softmax; every branch adds the
    same rotary score, and the head's output is out_scale times the sum of the branch outputs.
    Returns [len(batches), len(rows), d_v]; ``heads`` selects query rows.
    """
    W_UK, W_UV = to_f64(w_uk), to_f64(w_uv)
    NB, Hw, d_nope, d_cb = W_UK.shape
    d_v = W_UV.shape[-1]
    qn, qr = to_f64(q_nope), to_f64(q_rope)
    B, R = qn.shape[0], qn.shape[1]
    sq = int(num_queries)
    if sq < 1 or R != sq * Hw:
        raise ValueError("query rows must be s_q times the weights' heads")
    batches = list(range(B)) if batches is None else list(batches)
    sel = list(range(R)) if heads is None else list(heads)
    out = np.zeros((len(batches), len(sel), d_v), dtype=F64)
    for i, b in enumerate(batches):
        L = int(seqlens[b])
        rows = sequence_rows(cache, b, L, page_size, block_table, to_f64)   # [L, d_c + d_rope]
        if L == 0:
            continue
        lat = rows[:, :NB * d_cb]
        k_rot = rope(rows[:, NB * d_cb:NB * d_cb + d_rope], np.arange(L), theta)  # keys at t
        pos = L - sq + np.arange(sq)                                           # query positions
        mask = np.arange(L)[None, :] > pos[:, None]                            # [s_q, L] future
        seen = pos >= 0                                                        # sees >= 1 token
        for h in sorted({r % Hw for r in sel}):
            q_r = rope(qr[b, h::Hw], pos, theta)                               # [s_q, d_rope]
            O = np.zeros((sq, d_v), dtype=F64)
            for br in range(NB):
                c = lat[:, br * d_cb:(br + 1) * d_cb]                          # [L, d_cb]
                K = c @ W_UK[br, h].T                                          # [L, d_nope]
                V = c @ W_UV[br, h]                                            # [L, d_v]
                q_n = qn[b, h::Hw, br]                                         # [s_q, d_nope]
                S = scale * (q_n @ K.T + q_r @ k_rot.T)                        # [s_q, L]
                S[mask] = -np.inf
                if seen.any():
                    O[seen] += softmax(S[seen]) @ V
            for j, r in enumerate(sel):
                if r % Hw == h:
                    out[i, j] = out_scale * O[r // Hw]
    return out


# ----------------------------------------------------------------------------- write side

def latent_rows(hidden, w_dkv, w_kr, positions, theta: float = 10000.0) -> np.ndarray:
    """Cache rows [c_KV | k_rope] of new tokens, fp64.

    c_KV = h W_DKV, the joint low-rank latent made at write time ("超越 GQA 的推理革命…MLA…",
    section "鍵值聯合低秩壓縮"); k_rope = RoPE(h W_KR, t), the separate uncompressed key that
    carries the position (same page, section "解耦旋轉位置編碼"), rotated at the token's own
    position t as the cache stores it.  hidden [n, d_model], w_dkv [d_model, d_c],
    w_kr [d_model, d_r], positions [n] -> [n, d_c + d_r].
    """
    h = _as_f64(hidden)
    c = h @ _as_f64(w_dkv)
    k = rope(h @ _as_f64(w_kr), np.asarray(positions, dtype=np.int64), theta)
    return np.concatenate([c, k], axis=-1)


def cache_append(hidden, w_dkv, w_kr, seqlens, block_table=None, free_pages=(), *,
                 theta: float = 10000.0, page_size: int = 0, capacity: Optional[int] = None):
    """One decode step's cache write for a batch (fp64 rows, exact integer bookkeeping).

    Sequence b's new token goes to position t = seqlens[b] and the length becomes t + 1.
    Paged cache (page_size > 0): when t starts a page (t % page_size == 0) the sequence needs
    a new page; the k-th such sequence in batch order takes free_pages[k] and it is entered at
    block_table[b, t // page_size]; otherwise the row goes to the page already there.
    Contiguous cache: the row goes to cache[b, t], t < capacity.  A sequence is not written
    and keeps its length when the free list has no k-th page for it, or when t lies outside
    the cache (t < 0, a block-table column past the row, a missing page, t >= capacity).
    pages_used = min(sequences needing a page, len(free_pages)).

    Returns dict(rows [B, row] fp64, where [B] (page, slot) or (b, t) of each written row
    (None if not written), seqlens [B], block_table (copy, updated), pages_used, written [B]).
    """
    lens = [int(x) for x in np.asarray(seqlens).reshape(-1)]
    B = len(lens)
    rows = latent_rows(hidden, w_dkv, w_kr, [max(t, 0) for t in lens], theta)
    bt = None if block_table is None else np.array(block_table, dtype=np.int64, copy=True)
    where, written, new_lens, used = [None] * B, [False] * B, list(lens), 0
    free = [int(x) for x in free_pages]
    # the page ranks count every sequence whose token starts a page, in batch order
    for b, t in enumerate(lens):
        if t < 0:
            continue  # outside the cache: not written
        if page_size:
            j = t // page_size
            if t % page_size == 0:
                k = used
                used += 1
                if k >= len(free) or j >= bt.shape[1]:
                    continue  # no free page left, or the block-table row is full
                bt[b, j] = free[k]
            elif j >= bt.shape[1] or bt[b, j] < 0:
                continue  # the page for position t is missing
            where[b] = (int(bt[b, j]), t % page_size)
        else:
            if capacity is not None and t >= capacity:
                continue  # past the contiguous cache's rows
            where[b] = (b, t)
        written[b] = True
        new_lens[b] = t + 1
    return dict(rows=rows, where=where, seqlens=np.array(new_lens, dtype=np.int64),
                block_table=bt, pages_used=min(used, len(free)), written=np.array(written))
