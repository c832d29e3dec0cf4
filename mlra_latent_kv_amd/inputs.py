"""Workload table and seeded synthetic inputs for MLA / MLRA-4 decode.

This module only draws random numbers and lays them out in memory; it holds
none of the attention arithmetic. Both the fp64 CPU oracle (via the tests) and
the HIP path consume what it produces, so the two sides see identical inputs.

Shapes follow the pages' description of a latent KV cache: one compressed
latent vector per token plus one decoupled rotary key per token ("Multi-Head
Latent Attention explained", sections on joint low-rank KV compression and on
decoupled RoPE); MLRA splits the latent into independent branches
("Multi-Head Low-Rank Attention" blog, section 2.1).

Storage layout of one cache row: ``[c_KV (d_c) | k_rope (d_r)]`` with
``d_c = branches * d_cb``.  The rope columns hold the *raw* (un-rotated) key;
the GPU harness rotates them in place with ``mla_rope_rotate`` and the oracle
rotates them itself, so the two sides rotate independently.

Value distribution: every tensor is drawn from N(0, 1) / sqrt(fan_in) with
fan_in = the tensor's own feature dimension (latent: d_cb, rope keys and
query rope part: d_r, query latent part: d_nope, both up-projections: d_cb),
then rounded to the storage dtype (fp32, or bf16 with round-to-nearest-even).
Unused cache rows (the tail of a partially filled page, or rows past a
sequence's length in a contiguous cache) are filled with +/-``poison`` so
that any read past the end of a sequence shows up in the output.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import numpy as np

PAGE = 64  # tokens per page of the paged latent cache


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    heads: int
    branches: int          # 1 = MLA, 4 = MLRA-4
    d_nope: int            # per-head query/key "content" dim before absorption
    d_v: int               # per-head value / output dim
    d_cb: int              # latent dim per branch (d_c = branches * d_cb)
    d_rope: int            # decoupled rotary key dim
    dtype: str             # "f32" | "bf16"  (storage; accumulation is fp32)
    paged: bool
    seqlen: int            # fixed context length, or the upper bound when seqlen_lo is set
    seqlen_lo: Optional[int] = None  # variable lengths ~ U{seqlen_lo..seqlen}
    out_scale: float = 1.0
    rope_theta: float = 10000.0
    seed: int = 0

    @property
    def d_c(self) -> int:
        return self.branches * self.d_cb

    @property
    def row(self) -> int:
        return self.d_c + self.d_rope

    @property
    def softmax_scale(self) -> float:
        # 1/sqrt of the query-key dot-product length before absorption.
        return 1.0 / math.sqrt(self.d_nope + self.d_rope)

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny_mla_f32_b1_h4_l64", batch=1, heads=4, branches=1, d_nope=16, d_v=16,
                 d_cb=32, d_rope=8, dtype="f32", paged=False, seqlen=64, seed=1001),
        Workload("mla_bf16_b32_h128_l4096", batch=32, heads=128, branches=1, d_nope=128, d_v=128,
                 d_cb=512, d_rope=64, dtype="bf16", paged=False, seqlen=4096, seed=1002),
        Workload("mla_bf16_paged_b64_h32_l1k-32k", batch=64, heads=32, branches=1, d_nope=128,
                 d_v=128, d_cb=512, d_rope=64, dtype="bf16", paged=True, seqlen=32768,
                 seqlen_lo=1024, seed=1003),
        Workload("mlra4_bf16_b32_h32_l8192", batch=32, heads=32, branches=4, d_nope=128, d_v=128,
                 d_cb=128, d_rope=64, dtype="bf16", paged=False, seqlen=8192, out_scale=0.5,
                 seed=1004),
        Workload("mla_bf16_paged_b4_h128_l131072", batch=4, heads=128, branches=1, d_nope=128,
                 d_v=128, d_cb=512, d_rope=64, dtype="bf16", paged=True, seqlen=131072, seed=1005),
    ]
}
WORKLOAD_ORDER = list(WORKLOADS)


# ----------------------------------------------------------------------------- storage formats

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round-to-nearest-even); returns uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + bias) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    x = np.asarray(x, dtype=np.float32)
    return x.copy() if dtype == "f32" else f32_to_bf16_bits(x)


def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of a stored fp32 array or bf16 bit array."""
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    return bf16_bits_to_f32(a).astype(np.float64)


# ----------------------------------------------------------------------------- generator

def draw_seqlens(w: Workload, batch: int, rng: np.random.Generator) -> np.ndarray:
    if w.seqlen_lo is None:
        return np.full(batch, w.seqlen, dtype=np.int32)
    return rng.integers(w.seqlen_lo, w.seqlen, size=batch, endpoint=True).astype(np.int32)


def sharp_q_gain(w: Workload, target_logit_std: float = 2.0) -> float:
    """Gain on the query that makes the attention logits' std about ``target_logit_std``.

    Under the default distribution the logit of one head/branch is
    softmax_scale * (q_nope.K + q_rope.k_rope) with variance
    softmax_scale^2 * (1/d_cb + 1/d_rope): the attention is then nearly
    uniform, which would let a kernel that ignores the query pass a loose
    tolerance.  The "sharp" variant multiplies the query by this gain.
    """
    sigma0 = w.softmax_scale * math.sqrt(1.0 / w.d_cb + 1.0 / w.d_rope)
    return target_logit_std / sigma0


def make_inputs(
    w: Workload,
    *,
    seed: Optional[int] = None,
    batch: Optional[int] = None,
    seqlens: Optional[Sequence[int]] = None,
    paged: Optional[bool] = None,
    q_gain: float = 1.0,
    poison: float = 1.0e4,
    shuffle_pages: bool = True,
    max_seqlen: Optional[int] = None,
) -> dict:
    """Draw one seeded input set for workload ``w``.

    Overrides (``batch``, ``seqlens``, ``paged``, ``q_gain``) give the small and
    "sharp" parity cases at a workload's exact feature dimensions.

    Returns a dict of NumPy arrays in storage format (float32, or uint16 bf16
    bits) plus metadata:

    * ``q_nope``  [B, H, NB, d_nope]   (one vector per head, replicated over branches)
    * ``q_rope``  [B, H, d_rope]       un-rotated
    * ``cache``   contiguous [B, Lmax, d_c + d_rope] or paged pool [P, 64, d_c + d_rope];
                  rope columns are the raw (un-rotated) keys
    * ``row_pos`` int32 [rows of cache]: logical position of every cache row, -1 if unused
    * ``seqlens`` int32 [B]
    * ``block_table`` int32 [B, max_pages] (paged only, -1 = no page), else None
    * ``w_uk``    [NB, H, d_nope, d_cb];  ``w_uv`` [NB, H, d_cb, d_v]
    """
    seed = w.seed if seed is None else seed
    paged = w.paged if paged is None else paged
    kids = np.random.SeedSequence(seed).spawn(8)
    r_qn, r_qr, r_lat, r_kr, r_wk, r_wv, r_len, r_perm = (np.random.default_rng(k) for k in kids)

    if seqlens is not None:
        lens = np.asarray(seqlens, dtype=np.int32)
        B = len(lens)
    else:
        B = w.batch if batch is None else batch
        lens = draw_seqlens(w, B, r_len)
    H, NB, dn, dv, dcb, dr = w.heads, w.branches, w.d_nope, w.d_v, w.d_cb, w.d_rope
    dc = NB * dcb
    row = dc + dr
    st = np.float32 if w.dtype == "f32" else np.uint16

    def normal(rng, shape, fan_in, gain=1.0):
        return rng.standard_normal(shape, dtype=np.float32) * np.float32(gain / math.sqrt(fan_in))

    qn = normal(r_qn, (B, H, 1, dn), dn, q_gain)
    q_nope = to_storage(np.broadcast_to(qn, (B, H, NB, dn)), w.dtype)
    q_rope = to_storage(normal(r_qr, (B, H, dr), dr, q_gain), w.dtype)
    w_uk = to_storage(normal(r_wk, (NB, H, dn, dcb), dcb), w.dtype)
    w_uv = to_storage(normal(r_wv, (NB, H, dcb, dv), dcb), w.dtype)

    Lmax = int(max(int(lens.max(initial=0)), 1)) if max_seqlen is None else int(max_seqlen)
    if int(lens.max(initial=0)) > Lmax:
        raise ValueError("seqlens exceed max_seqlen")

    def poison_rows(n):
        p = np.empty((n, row), dtype=np.float32)
        p[:, 0::2] = poison
        p[:, 1::2] = -poison
        return to_storage(p, w.dtype)

    def logical_rows(b):
        L = int(lens[b])
        lat = normal(r_lat, (L, NB, dcb), dcb).reshape(L, dc)
        kr = normal(r_kr, (L, dr), dr)
        return to_storage(np.concatenate([lat, kr], axis=1), w.dtype)

    if not paged:
        cache = np.empty((B, Lmax, row), dtype=st)
        row_pos = np.full((B, Lmax), -1, dtype=np.int32)
        for b in range(B):
            L = int(lens[b])
            cache[b, :L] = logical_rows(b)
            cache[b, L:] = poison_rows(Lmax - L)
            row_pos[b, :L] = np.arange(L, dtype=np.int32)
        block_table = None
    else:
        npages = [(int(L) + PAGE - 1) // PAGE for L in lens]
        P = int(sum(npages))
        max_pages = max((Lmax + PAGE - 1) // PAGE, 1)
        perm = r_perm.permutation(P).astype(np.int32) if shuffle_pages else np.arange(P, dtype=np.int32)
        cache = np.empty((max(P, 1), PAGE, row), dtype=st)
        cache[:] = poison_rows(1)[0]
        row_pos = np.full((max(P, 1), PAGE), -1, dtype=np.int32)
        block_table = np.full((B, max_pages), -1, dtype=np.int32)
        off = 0
        for b in range(B):
            L = int(lens[b])
            rows = logical_rows(b)
            for j in range(npages[b]):
                pg = int(perm[off + j])
                block_table[b, j] = pg
                n = min(PAGE, L - j * PAGE)
                cache[pg, :n] = rows[j * PAGE: j * PAGE + n]
                row_pos[pg, :n] = np.arange(j * PAGE, j * PAGE + n, dtype=np.int32)
            off += npages[b]

    return dict(
        workload=w, dtype=w.dtype, paged=paged, page_size=PAGE if paged else 0,
        q_nope=q_nope, q_rope=q_rope, cache=cache, row_pos=row_pos.reshape(-1),
        seqlens=lens, block_table=block_table, w_uk=w_uk, w_uv=w_uv,
        max_seqlen=Lmax, softmax_scale=w.softmax_scale, out_scale=w.out_scale,
        rope_theta=w.rope_theta,
    )


def cache_bytes(w: Workload, seqlens: np.ndarray) -> int:
    """Algorithmic latent-cache bytes one decode step reads: every cached row once."""
    return int(np.asarray(seqlens, dtype=np.int64).sum()) * w.row * w.elem_bytes
