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

    @property
    def latent_ptr(self) -> int:
        return self.cache.data_ptr()

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


def make_params(inp: dict, num_splits: int = 0) -> B.MlaParams:
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
    p.latent_stride_tok = p.rope_stride_tok = row
    if inp["paged"]:
        p.page_size = PAGE
        bt = inp["block_table"]
        p.max_pages_per_seq = bt.shape[1]
        p.block_table_stride = bt.shape[1]
        p.latent_stride_seq = p.rope_stride_seq = PAGE * row
    else:
        p.page_size = 0
        p.latent_stride_seq = p.rope_stride_seq = cache.shape[1] * row
    p.softmax_scale = inp["softmax_scale"]
    p.out_scale = inp["out_scale"]
    p.rope_theta = inp["rope_theta"]
    return p


def to_device(inp: dict, device="cuda", num_splits: int = 0, stream=None) -> DeviceCase:
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
    params = make_params(inp, num_splits)
    ws_bytes = B.workspace_size(params)
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
        out=torch.empty((len(inp["seqlens"]), w.heads, w.d_v),
                        dtype=torch.bfloat16 if dt == "bf16" else torch.float32, device=dev),
        workspace=torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev),
        branches=w.branches,
    )
    return case


def read_plan(case: DeviceCase) -> dict:
    """The split plan the last call left at the start of the workspace (layout documented in
    include/mla_decode.h): item count W, pages per item c, dispatch slots, item target (0 when
    the split count was forced), the dispatch table [slots, 4] = (b, t_begin, t_end, item)
    and split_off [B + 1].  Synchronises with the device."""
    ws = case.workspace
    hdr = ws[:16].view(torch.int32).cpu().numpy()
    slots = int(hdr[2])
    work = ws[16:16 + 16 * slots].view(torch.int32).cpu().numpy().reshape(slots, 4)
    off = 16 + 16 * slots
    split_off = ws[off:off + 4 * (case.params.batch + 1)].view(torch.int32).cpu().numpy()
    return {"items": int(hdr[0]), "pages": int(hdr[1]), "slots": slots, "target": int(hdr[3]),
            "work": work, "split_off": split_off}
