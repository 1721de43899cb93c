"""One layer's chunked-prefill-with-past step, as a sequence of libcp calls.

Order of the calls (the cache is read by attention before the chunk's rows
are appended, so a ring never loses keys the chunk's first rows still need):

    rope(Q, K) -> [snapshot] -> attention (+ selected row) -> append -> [rollback]

Q and K are rotated by one launch, and the attention writes the last real row into
the selection as it writes the output (a tiny append also updates seen in the
same launch as its copy).

``static_append=True`` models a caller whose append always writes all C rows
(a fixed-shape graph): the ring is protected by the padded-append snapshot and
rollback ([cactus] "Fix").  Otherwise only the n_valid real rows are appended.
Every step runs in libcp's kernels; this module only sequences the calls.
"""
from dataclasses import dataclass
from typing import Optional

import torch

from . import cp


@dataclass
class StepBuffers:
    """Preallocated outputs and scratch of one step (reused across steps)."""
    q_rot: torch.Tensor
    k_rot: torch.Tensor
    out: torch.Tensor
    sel: torch.Tensor
    workspace: Optional[torch.Tensor] = None
    snap: Optional[cp.Snapshot] = None


def make_buffers(cache: cp.KVCache, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                 mask: Optional[torch.Tensor] = None, window: int = 0,
                 static_append: bool = False, flags: int = 0) -> StepBuffers:
    B, H, C, D = q.shape
    ws = cp.attn_workspace_bytes(cache, q, k, v, mask=mask, window=window, flags=flags)
    bufs = StepBuffers(q_rot=torch.empty_like(q), k_rot=torch.empty_like(k),
                       out=torch.empty_like(q),
                       sel=torch.empty((B, H, D), dtype=q.dtype, device=q.device))
    if ws:
        bufs.workspace = torch.empty(ws, dtype=torch.uint8, device=q.device)
    if static_append:
        bufs.snap = cp.Snapshot(torch.empty(max(cp.snapshot_bytes(cache, C), 1),
                                            dtype=torch.uint8, device=q.device))
    return bufs


def chunk_step(cache: cp.KVCache, q, k, v, cos, sin, n_valid, bufs: StepBuffers,
               mask: Optional[torch.Tensor] = None, window: int = 0,
               static_append: bool = False, flags: int = 0):
    """Run the whole hot path of one layer for one chunk; returns (out, selected row)."""
    cp.rope_qk_chunk(q, k, cos, sin, q_out=bufs.q_rot, k_out=bufs.k_rot)
    if static_append:
        cp.kv_snapshot_padded_append(cache, q.shape[2], n_valid, bufs.snap)
    cp.attn_chunk_with_past(cache, bufs.q_rot, bufs.k_rot, v, n_valid=n_valid, mask=mask,
                            window=window, out=bufs.out, workspace=bufs.workspace, flags=flags,
                            select_out=bufs.sel)
    cp.kv_append(cache, bufs.k_rot, v, None if static_append else n_valid)
    if static_append:
        cp.kv_rollback_padded_append(cache, bufs.snap)
    return bufs.out, bufs.sel
