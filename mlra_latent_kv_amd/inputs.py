"""Workload table and seeded synthetic inputs for MLA / MLRA-4 decode.

This module only draws random numbers and lays them out in memory; it holds
none of the attention arithmetic. Both the fp64 CPU oracle (via the tests) and
the HIP path consume what it produces, so the two sides see identical inputs.

Shapes follow the pages' description of a latent KV cache: one compressed
latent vector per token plus one decoupled rotary key per token ("超越 GQA 的推理
革命…MLA…", sections 鍵值聯合低秩壓縮 and 解耦旋轉位置編碼); MLRA splits the latent
into independent branches, each with its own latent head ("[ICLR 2025] MLRA…",
section 2.1).

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
        # one branch of MLRA-4 on its own, as each GPU of a 4-way tensor-parallel group runs it:
        # rows [c_b (128) | k_rope (64)]; out_scale 0.5 makes the four shards' outputs sum to
        # the MLRA-4 output ("[ICLR 2025] MLRA…", sections 1 and 4)
        Workload("mlra_shard_bf16_b32_h32_l8192", batch=32, heads=32, branches=1, d_nope=128,
                 d_v=128, d_cb=128, d_rope=64, dtype="bf16", paged=False, seqlen=8192,
                 out_scale=0.5, seed=1006),
    ]
}
WORKLOAD_ORDER = list(WORKLOADS)

# Prefill workloads (mla_prefill): every token of the sequence is new, s_q = seqlen query tokens
# per sequence attend causally over the cache that holds them (the many-query regime of the
# yololab MLA page, section 繁榮背後的代價), with the decode workloads' feature dims.
PREFILL_WORKLOADS = {
    w.name: w
    for w in [
        Workload("prefill_bf16_b1_h128_l4096", batch=1, heads=128, branches=1, d_nope=128,
                 d_v=128, d_cb=512, d_rope=64, dtype="bf16", paged=False, seqlen=4096, seed=1007),
        Workload("prefill_bf16_paged_b4_h32_l4096", batch=4, heads=32, branches=1, d_nope=128,
                 d_v=128, d_cb=512, d_rope=64, dtype="bf16", paged=True, seqlen=4096, seed=1008),
        Workload("prefill_mlra4_bf16_b1_h32_l4096", batch=1, heads=32, branches=4, d_nope=128,
                 d_v=128, d_cb=128, d_rope=64, dtype="bf16", paged=False, seqlen=4096,
                 out_scale=0.5, seed=1009),
        # one MLRA branch cached on its own (the 4-way tensor-parallel shard of the workload
        # above, at four sequences): rows [c_b (128) | k_rope (64)], out_scale 0.5
        Workload("prefill_mlra_shard_bf16_b4_h32_l4096", batch=4, heads=32, branches=1,
                 d_nope=128, d_v=128, d_cb=128, d_rope=64, dtype="bf16", paged=False,
                 seqlen=4096, out_scale=0.5, seed=1010),
    ]
}


# ----------------------------------------------------------------------------- storage formats

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round-to-nearest-even); returns uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + bias) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


E4M3_MAX = 448.0  # largest finite OCP FP8 E4M3 ("e4m3fn") value


def e4m3_bits_to_f64(b: np.ndarray) -> np.ndarray:
    """Exact value of OCP FP8 E4M3 codes (1 sign, 4 exponent bits with bias 7, 3 mantissa
    bits; exponent 0 is subnormal, 2^-6 * m / 8; code 0x7f / 0xff is NaN; no infinities)."""
    b = np.asarray(b, dtype=np.uint8).astype(np.int64)
    sign = np.where(b & 0x80, -1.0, 1.0)
    e, m = (b >> 3) & 15, b & 7
    mag = np.where(e == 0, np.ldexp(m / 8.0, -6), np.ldexp(1.0 + m / 8.0, e - 7))
    return np.where((e == 15) & (m == 7), np.nan, sign * mag)


def f64_to_e4m3_bits(x: np.ndarray) -> np.ndarray:
    """Round to the nearest OCP FP8 E4M3 value (ties to the even code), saturating at
    +-448; returns uint8 codes.  Inputs must be finite."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), E4M3_MAX)
    # the code grid below 2^-6 is subnormal with spacing 2^-9; above, 3 mantissa bits
    e = np.floor(np.log2(np.maximum(a, np.ldexp(1.0, -6))))
    step = np.ldexp(1.0, (e - 3).astype(np.int64))
    q = np.round(a / step) * step  # np.round: half to even on the grid index
    grid = e4m3_bits_to_f64(np.arange(0x7f, dtype=np.uint8))  # 0 .. 448, increasing
    idx = np.searchsorted(grid, q)
    assert np.all(grid[np.minimum(idx, 0x7e)] == q), "rounded value off the E4M3 grid"
    return (idx.astype(np.uint8) | np.where(x < 0, 0x80, 0).astype(np.uint8)).astype(np.uint8)


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


def _streams(seed: int):
    """The eight independent child streams of one input set, in draw order: q_nope, q_rope,
    latent rows, raw rotary keys, W_UK, W_UV, lengths, page permutation."""
    kids = np.random.SeedSequence(seed).spawn(8)
    return tuple(np.random.default_rng(k) for k in kids)


def _normal(rng, shape, fan_in, gain=1.0):
    return rng.standard_normal(shape, dtype=np.float32) * np.float32(gain / math.sqrt(fan_in))


def _queries(w: Workload, B: int, r_qn, r_qr, q_gain: float, num_queries: int = 1):
    """q_nope [B, s_q * H, NB, d_nope] (an independent vector per query token, head and
    branch: each MLRA branch has its own latent head, so its absorbed query differs) and
    q_rope [B, s_q * H, d_rope]; s_q = num_queries new tokens per sequence, token-major."""
    rows = num_queries * w.heads
    qn = _normal(r_qn, (B, rows, w.branches, w.d_nope), w.d_nope, q_gain)
    qr = _normal(r_qr, (B, rows, w.d_rope), w.d_rope, q_gain)
    return to_storage(qn, w.dtype), to_storage(qr, w.dtype)


def requery(inp: dict, q_gain: float) -> dict:
    """The same input set with its queries redrawn at gain ``q_gain`` (same seed, so the
    same standard normals times a different gain); the cache and weights are shared, not
    copied."""
    w = inp["workload"]
    r = _streams(inp["seed"])
    out = dict(inp)
    out["q_nope"], out["q_rope"] = _queries(w, len(inp["seqlens"]), r[0], r[1], q_gain,
                                            inp.get("num_queries", 1))
    out["q_gain"] = q_gain
    return out


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
    num_queries: int = 1,
    latent_format: str = "",
) -> dict:
    """Draw one seeded input set for workload ``w``.

    ``num_queries`` = s_q new tokens per sequence decoded in one step: the queries get
    s_q * H rows (token-major); everything else is unchanged.

    ``latent_format="fp8"`` (bf16 workloads): the latent part of the cache is also stored as
    OCP FP8 E4M3 codes ``latent8`` (the cache's row layout with d_c bytes per row) with one
    per-tensor scale ``latent_scale`` = max |latent| / 448 over the stored rows, so that
    latent = decode(latent8) * latent_scale; unused rows hold the NaN code.  The rotary
    columns stay in ``cache`` (bf16).  ``oracle_cache`` gives the values the cache holds.

    Overrides (``batch``, ``seqlens``, ``paged``, ``q_gain``) give the small and
    "sharp" parity cases at a workload's exact feature dimensions.

    Returns a dict of NumPy arrays in storage format (float32, or uint16 bf16
    bits) plus metadata:

    * ``q_nope``  [B, H, NB, d_nope]   (an independent vector per head and branch)
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
    r_qn, r_qr, r_lat, r_kr, r_wk, r_wv, r_len, r_perm = _streams(seed)

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

    normal = _normal
    q_nope, q_rope = _queries(w, B, r_qn, r_qr, q_gain, num_queries)
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

    extra = {}
    if latent_format == "fp8":
        if w.dtype != "bf16":
            raise ValueError("an fp8 latent goes with the bf16 workloads")
        lat = to_f64(cache[..., :dc], w.dtype).reshape(-1, dc)
        used = row_pos.reshape(-1) >= 0
        amax = float(np.abs(lat[used]).max()) if used.any() else 1.0
        scale = np.float32(amax / E4M3_MAX if amax > 0 else 1.0)
        codes = np.full(lat.shape, 0x7F, dtype=np.uint8)  # NaN code on unused rows
        codes[used] = f64_to_e4m3_bits(lat[used] / np.float64(scale))
        extra = dict(latent8=codes.reshape(cache.shape[:-1] + (dc,)), latent_scale=float(scale))
    elif latent_format:
        raise ValueError(f"unknown latent format {latent_format!r}")
    return dict(
        **extra, latent_format=latent_format,
        workload=w, seed=seed, q_gain=q_gain, num_queries=num_queries,
        dtype=w.dtype, paged=paged, page_size=PAGE if paged else 0,
        q_nope=q_nope, q_rope=q_rope, cache=cache, row_pos=row_pos.reshape(-1),
        seqlens=lens, block_table=block_table, w_uk=w_uk, w_uv=w_uv,
        max_seqlen=Lmax, softmax_scale=w.softmax_scale, out_scale=w.out_scale,
        rope_theta=w.rope_theta,
    )


def oracle_cache(inp: dict) -> np.ndarray:
    """The values the input set's cache holds, as float64 rows [latent | raw rotary key]: the
    stored bf16 / fp32 rows, or, with an fp8 latent, its decoded codes times the scale next
    to the stored rotary columns."""
    w = inp["workload"]
    c = to_f64(inp["cache"], w.dtype)
    if inp.get("latent_format") == "fp8":
        c = c.copy()
        c[..., :w.d_c] = e4m3_bits_to_f64(inp["latent8"]) * np.float64(inp["latent_scale"])
    return c


def cache_bytes(w: Workload, seqlens: np.ndarray, latent_format: str = "") -> int:
    """Algorithmic latent-cache bytes one decode step reads: every cached row once (with an
    fp8 latent, 1 byte per latent element next to the bf16 rotary key)."""
    per = w.d_c + w.d_rope * w.elem_bytes if latent_format == "fp8" else w.row * w.elem_bytes
    return int(np.asarray(seqlens, dtype=np.int64).sum()) * per


# ----------------------------------------------------------------------------- write side

def make_variant_inputs(inp: dict, *, seed: Optional[int] = None, gate_std: float = 2.0) -> dict:
    """Seeded extra inputs of the decode step's variants, for the input set ``inp``:

    * ``gate``      [B, H, d_v] gate logits, N(0, gate_std^2), so sigmoid(gate) spans most of
                    (0, 1);
    * ``q_latent``  [B, H, NB * d_cb] a latent-space query (the form the query takes once W_UK is
                    folded into the query projection), N(0, 1) / sqrt(d_cb) times the input
                    set's query gain: the spread of W_UK^T q_nope under the default draw.
    Storage format as ``make_inputs`` (uint16 bf16 bits or float32).
    """
    w = inp["workload"]
    B = len(inp["seqlens"])
    seed = inp["seed"] + 7919 if seed is None else seed
    r_g, r_q = (np.random.default_rng(k) for k in np.random.SeedSequence(seed).spawn(2))
    rows = inp.get("num_queries", 1) * w.heads
    gate = r_g.standard_normal((B, rows, w.d_v), dtype=np.float32) * np.float32(gate_std)
    q_lat = _normal(r_q, (B, rows, w.branches * w.d_cb), w.d_cb, inp.get("q_gain", 1.0))
    return {"gate": to_storage(gate, w.dtype), "q_latent": to_storage(q_lat, w.dtype)}


def make_append_inputs(d_model: int, d_latent: int, batch: int, *, seed: int = 2001,
                       d_rope: int = 64) -> dict:
    """Seeded new-token hidden states and down-projections for a cache append: hidden
    [B, d_model], w_dkv [d_model, d_latent], w_kr [d_model, d_rope], each N(0,1)/sqrt(d_model)
    (fan_in = d_model), rounded to bf16 (uint16 bits)."""
    r_h, r_d, r_k = (np.random.default_rng(k) for k in np.random.SeedSequence(seed).spawn(3))
    return dict(hidden=to_storage(_normal(r_h, (batch, d_model), d_model), "bf16"),
                w_dkv=to_storage(_normal(r_d, (d_model, d_latent), d_model), "bf16"),
                w_kr=to_storage(_normal(r_k, (d_model, d_rope), d_model), "bf16"))
