"""Device plumbing for tests and the benchmark: upload a seeded input set, write the rotary
keys with ``mla_rope_rotate``, build ``mla_params``, allocate out/workspace (PyTorch owns
the memory) and call the library.  No attention arithmetic happens here.
"""

from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch

from . import binding as B
from .inputs import PAGE


def _to_dev(a: np.ndarray, dtype: str, device) -> torch.Tensor:
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


@dataclasses.dataclass
class DeviceCase:
    params: B.MlaParams
    q_nope: torch.Tensor
    q_rope: torch.Tensor
    cache: torch.Tensor          # rows [c_KV | k_rope], rope columns rotated on the device
    seqlens: torch.Tensor
    block_table: Optional[torch.Tensor]
    w_uk: torch.Tensor
    w_uv: torch.Tensor
    out: torch.Tensor
    workspace: torch.Tensor
    branches: int
    latent8: Optional[torch.Tensor] = None  # fp8 latent codes (MLA_LATENT_FP8), else None

    @property
    def latent_ptr(self) -> int:
        return self.cache.data_ptr() if self.latent8 is None else self.latent8.data_ptr()

    @property
    def rope_ptr(self) -> int:
        return self.cache.data_ptr() + self.params.d_latent * self.params.num_branches * self.cache.element_size()

    def run(self, stream=None, params: Optional[B.MlaParams] = None, out=None, workspace=None,
            events=None):
        p = self.params if params is None else params
        fn = B.mlra_decode if self.branches == 4 else B.mla_decode
        fn(p, self.q_nope, self.q_rope, self.latent_ptr, self.rope_ptr, self.seqlens,
           self.block_table, self.w_uk, self.w_uv, self.out if out is None else out,
           self.workspace if workspace is None else workspace, stream=stream, events=events)
        return self.out if out is None else out


def run_variant(case: "DeviceCase", *, gate=None, q_latent=None, latent_out: bool = False,
                stream=None) -> torch.Tensor:
    """One call of a decode variant on ``case``'s inputs: ``gate`` (device tensor [B, H, d_v])
    selects the gated entry point, ``q_latent`` (device tensor [B, H, NB*d_cb]) passes a folded
    query with MLA_FLAG_QUERY_LATENT (W_UK not passed), ``latent_out`` sets
    MLA_FLAG_OUTPUT_LATENT (W_UV not passed) and returns [B, H, NB*d_cb].  Returns a new
    output tensor."""
    p = case.params.copy()
    if q_latent is not None:
        p.flags |= B.MLA_FLAG_QUERY_LATENT
    if latent_out:
        p.flags |= B.MLA_FLAG_OUTPUT_LATENT
    width = p.num_branches * p.d_latent if latent_out else p.d_v
    rows = max(p.num_queries, 1) * p.num_heads
    out = torch.empty((p.batch, rows, width), dtype=case.out.dtype, device=case.out.device)
    qn = case.q_nope if q_latent is None else q_latent
    w_uk = None if q_latent is not None else case.w_uk
    w_uv = None if latent_out else case.w_uv
    args = (p, qn, case.q_rope, case.latent_ptr, case.rope_ptr, case.seqlens, case.block_table,
            w_uk, w_uv)
    if gate is not None:
        fn = B.mlra_decode_gated if case.branches == 4 else B.mla_decode_gated
        fn(*args, gate, out, case.workspace, stream=stream)
    else:
        fn = B.mlra_decode if case.branches == 4 else B.mla_decode
        fn(*args, out, case.workspace, stream=stream)
    return out


def make_params(inp: dict, num_splits: int = 0, flags: int = 0) -> B.MlaParams:
    w = inp["workload"]
    cache = inp["cache"]
    row = w.row
    p = B.MlaParams()
    p.batch = len(inp["seqlens"])
    p.num_heads = w.heads
    p.num_branches = w.branches
    p.d_nope, p.d_v, p.d_latent, p.d_rope = w.d_nope, w.d_v, w.d_cb, w.d_rope
    p.max_seqlen = int(inp["max_seqlen"])
    p.num_splits = num_splits
    p.dtype = B.MLA_BF16 if w.dtype == "bf16" else B.MLA_F32
    p.flags = flags
    p.num_queries = int(inp.get("num_queries", 1))
    p.latent_stride_tok = p.rope_stride_tok = row
    if inp["paged"]:
        p.page_size = PAGE
        bt = inp["block_table"]
        p.max_pages_per_seq = bt.shape[1]
        p.block_table_stride = bt.shape[1]
        p.latent_stride_seq = p.rope_stride_seq = PAGE * row
        p.num_pages = cache.shape[0]
    else:
        p.page_size = 0
        p.latent_stride_seq = p.rope_stride_seq = cache.shape[1] * row
    p.softmax_scale = inp["softmax_scale"]
    p.out_scale = inp["out_scale"]
    p.rope_theta = inp["rope_theta"]
    if inp.get("latent_format") == "fp8":
        # E4M3 codes in their own [rows, d_c] array: the latent strides count bytes
        p.latent_format = B.MLA_LATENT_FP8
        p.latent_scale = inp["latent_scale"]
        lat_rows = inp["latent8"].shape[-2]  # tokens per sequence (contiguous) or per page
        p.latent_stride_tok = w.d_c
        p.latent_stride_seq = lat_rows * w.d_c
    return p


def to_device(inp: dict, device="cuda", num_splits: int = 0, stream=None,
              flags: int = 0, prefill: bool = False) -> DeviceCase:
    w = inp["workload"]
    dt = w.dtype
    dev = torch.device(device)
    cache = _to_dev(inp["cache"], dt, dev)
    row_pos = torch.from_numpy(inp["row_pos"]).to(dev)
    n_rows = row_pos.numel()
    # the cache stores each rotary key already rotated at its own position
    B.mla_rope_rotate(cache.data_ptr() + w.d_c * cache.element_size(), w.row, row_pos, n_rows,
                      w.d_rope, w.rope_theta, B.MLA_BF16 if dt == "bf16" else B.MLA_F32,
                      stream=stream)
    params = make_params(inp, num_splits, flags)
    # prefill=True: the workspace of mla_prefill (up-projected keys and values)
    ws_bytes = B.prefill_workspace_size(params) if prefill else B.workspace_size(params)
    bt = inp["block_table"]
    case = DeviceCase(
        params=params,
        q_nope=_to_dev(inp["q_nope"], dt, dev),
        q_rope=_to_dev(inp["q_rope"], dt, dev),
        cache=cache,
        seqlens=torch.from_numpy(np.asarray(inp["seqlens"], np.int32)).to(dev),
        block_table=None if bt is None else torch.from_numpy(bt).to(dev),
        w_uk=_to_dev(inp["w_uk"], dt, dev),
        w_uv=_to_dev(inp["w_uv"], dt, dev),
        out=torch.empty((len(inp["seqlens"]), int(inp.get("num_queries", 1)) * w.heads, w.d_v),
                        dtype=torch.bfloat16 if dt == "bf16" else torch.float32, device=dev),
        workspace=torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev),
        branches=w.branches,
        latent8=(torch.from_numpy(np.ascontiguousarray(inp["latent8"])).to(dev)
                 if inp.get("latent_format") == "fp8" else None),
    )
    return case


def run_prefill(case: DeviceCase, stream=None, out=None, events=None) -> torch.Tensor:
    """mla_prefill on a case made with ``to_device(.., prefill=True)``: the case's queries are
    its s_q tokens per sequence; returns out [B, s_q * H, d_v]."""
    o = case.out if out is None else out
    B.mla_prefill(case.params, case.q_nope, case.q_rope, case.latent_ptr, case.rope_ptr,
                  case.seqlens, case.block_table, case.w_uk, case.w_uv, o, case.workspace,
                  stream=stream, events=events)
    return o


def read_plan(case: DeviceCase) -> dict:
    """The split plan the last call left at the start of the workspace (layout documented in
    include/mla_decode.h): item count W, pages per item c (0 for the stream plan), dispatch
    slots, item target (0 when the split count was forced), the device-check error word
    (bits, first bad sequence, its first bad block-table column), the per-slot table
    [slots, 4] = (b, t_begin, t_end, item) of each slot's first item, slot_end [slots], the
    item table [W, 4] = (b, t_begin, t_end, slot) and split_off [B + 1].  Synchronises with
    the device."""
    ws = case.workspace
    hdr = ws[:32].view(torch.int32).cpu().numpy()
    W, slots, cap = int(hdr[0]), int(hdr[2]), int(hdr[7])
    off = 32
    work = ws[off:off + 16 * slots].view(torch.int32).cpu().numpy().reshape(slots, 4)
    off += 16 * slots
    slot_end = ws[off:off + 4 * slots].view(torch.int32).cpu().numpy()
    off += 4 * slots
    items = ws[off:off + 16 * cap].view(torch.int32).cpu().numpy().reshape(cap, 4)[:W]
    off += 16 * cap
    split_off = ws[off:off + 4 * (case.params.batch + 1)].view(torch.int32).cpu().numpy()
    return {"items": W, "pages": int(hdr[1]), "slots": slots, "target": int(hdr[3]),
            "err_bits": int(hdr[4]), "err_seq": int(hdr[5]), "err_page": int(hdr[6]),
            "items_cap": cap, "work": work, "slot_end": slot_end, "item_table": items,
            "split_off": split_off}
