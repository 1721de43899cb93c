"""One layer's chunked-prefill-with-past step, as a sequence of libcp calls.

Order of the calls (the cache is read by attention before the chunk's rows
are appended, so a ring never loses keys the chunk's first rows still need):

    rope(Q, K) -> [snapshot] -> attention (+ selected row) -> append -> [rollback]

Q and K are rotated by one launch, and the attention writes the last real row into
the selection as it writes the output.  A global cache takes the chunk's K/V in the
RoPE launch (slots the attention does not read) and the attention advances seen.  A
ring cache takes the padded-append snapshot in the RoPE launch and the append with
its rollback in one launch after the attention: RoPE+snapshot -> attention (+ split
merge) -> append+rollback.

``static_append=True`` models a caller whose append always writes all C rows
(a fixed-shape graph): the ring is protected by the padded-append snapshot and
rollback ([cactus] "Fix").  A ring takes that form in every case (with all rows real
it saves nothing; with pad rows the live region equals the exact append of the real
rows).  Every step runs in libcp's kernels; this module only sequences the calls.

The tail of a prompt (fewer real tokens than a chunk) runs either as one padded
chunk or token by token -- one-token steps, the decode contract of [TICO]
"Runtime behavior" -- chosen by `pad_tail` ([cactus] "Fix": pad from the measured
breakeven, with a kill switch that forces token by token).
"""
import dataclasses
import os
from dataclasses import dataclass
from typing import List, Optional

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
    if static_append or (cache.ring and cache.cap > C + cache.sink):
        bufs.snap = cp.Snapshot(torch.empty(max(cp.snapshot_bytes(cache, C), 1),
                                            dtype=torch.uint8, device=q.device))
    return bufs


# Queries of at least this many bytes would be rotated by the attention as it loads
# them (cp_attn_args q_cos / q_sin: the rotated copy never goes to memory and the RoPE
# launch rotates the keys only).  None: never.  Measured on MI355X (same box, the step
# and the attention alone): the long-context workload's attention 1104 -> 1112 us and
# its step 1956 -> 1967 us, the Llama-8B-like layer's attention 114 -> 123 us -- every
# workgroup reads its rows' tables at its start (for the long-context layer about 64 MB
# from L2 at once) and rotates in fp64 before its first tile, which costs more than the
# RoPE launch saves.  So the RoPE launch keeps rotating Q.
ROPE_Q_IN_ATTENTION_BYTES = None


def rope_q_in_attention(q: torch.Tensor) -> bool:
    return (ROPE_Q_IN_ATTENTION_BYTES is not None and
            q.numel() * q.element_size() >= ROPE_Q_IN_ATTENTION_BYTES)


# Balanced key splits (cp_attn_args flag CP_ATTN_BALANCE) cost a plan launch and a merge
# launch (about 8 + 9 us on MI355X) and pay off when one sequence's past dominates the
# batch: on the Llama-8B-like batch (16 pasts uniform in [0, 4095], the longest 2.5x the
# mean) the attention call went 112.2 -> 97.5 us.  A batch of equal pasts gains nothing.
BALANCE_SKEW = 1.5


def attn_flags_for(seen_host) -> int:
    """Attention flags for a batch whose past lengths the host knows (its copy of seen):
    CP_ATTN_BALANCE when the longest past exceeds BALANCE_SKEW times the mean."""
    seen_host = list(seen_host)
    if len(seen_host) < 2:
        return 0
    mean = sum(seen_host) / len(seen_host)
    return cp.ATTN_BALANCE if max(seen_host) > BALANCE_SKEW * max(mean, 1.0) else 0


def chunk_step(cache: cp.KVCache, q, k, v, cos, sin, n_valid, bufs: StepBuffers,
               mask: Optional[torch.Tensor] = None, window: int = 0,
               static_append: bool = False, flags: int = 0, max_seen: int = 0):
    """Run the whole hot path of one layer for one chunk; returns (out, selected row).

    max_seen: 0, or an upper bound on every sequence's seen known on the host (the
    attention sizes its key splits from it instead of from the cache capacity).

    A global cache takes the fused form: the RoPE launch also writes the chunk's K/V
    rows past seen (slots this chunk's attention does not read), and the attention call
    advances seen afterwards -- the same cache bytes and outputs as RoPE, attention,
    append in sequence, without the append's launches.  A ring cache (whose append
    evicts rows the attention still reads) appends after the attention: the RoPE
    launch takes the padded-append snapshot, and one launch appends and rolls back
    (the same bytes as the separate snapshot, append of all C rows and rollback).  A
    padded global append takes the same form.  A ring whose window cannot take a
    padded append (cap <= C + sink) appends its real rows with cp_kv_append."""
    # large chunks: the attention rotates Q as it loads it
    fold = rope_q_in_attention(q)
    qr, q_in, q_rope = (None, q, (cos, sin)) if fold else (q, bufs.q_rot, None)
    attn = lambda fl: cp.attn_chunk_with_past(  # noqa: E731
        cache, q_in, bufs.k_rot, v, n_valid=n_valid, mask=mask, window=window, out=bufs.out,
        workspace=bufs.workspace, flags=fl, select_out=bufs.sel, q_rope=q_rope,
        max_seen=max_seen)
    if not cache.ring and not static_append:
        cp.rope_qk_append_chunk(cache, qr, k, v, cos, sin, n_valid, q_out=bufs.q_rot,
                                k_out=bufs.k_rot)
        attn(flags | cp.ATTN_ADVANCE_SEEN)
        return bufs.out, bufs.sel
    C = q.shape[2]
    if static_append or cache.cap > C + cache.sink:
        cp.rope_qk_snapshot_chunk(cache, qr, k, cos, sin, n_valid, bufs.snap, q_out=bufs.q_rot,
                                  k_out=bufs.k_rot)
        attn(flags)
        cp.kv_append_rollback(cache, bufs.k_rot, v, bufs.snap)
        return bufs.out, bufs.sel
    if fold:
        cp.rope_chunk(k, cos, sin, out=bufs.k_rot)
    else:
        cp.rope_qk_chunk(q, k, cos, sin, q_out=bufs.q_rot, k_out=bufs.k_rot)
    attn(flags)
    cp.kv_append(cache, bufs.k_rot, v, n_valid)
    return bufs.out, bufs.sel


# ------------------------------------------------------------- prompt tails

# Smallest tail that runs as one padded chunk.  [cactus] "Fix" and its review sweep
# table: on an Apple M4 Pro the padded chunk won from 9 tail tokens (PAGES_PAD_FROM).
# The same sweep on MI355X (`bench.py --tail-sweep`, a 512-window ring holding 1023
# positions, C 128, H8/KV1 D256) measured a one-token step at ~20.5 us and a padded
# 128-row chunk at ~31.5 us, so padding wins from 2 tail tokens there.
PAGES_PAD_FROM = 9
PAD_FROM = 2
KILL_SWITCH = "CP_DISABLE_PREFILL_TAIL_PAD"


def pad_tail(n_tail: int, pad_from: int = PAD_FROM) -> bool:
    """Tail policy: True runs a tail of n_tail real tokens as one padded chunk, False token
    by token.  The environment variable CP_DISABLE_PREFILL_TAIL_PAD=1 (any value but
    empty or 0) forces token by token.  `pad_from` is the hardware's breakeven: the
    default is the one measured on MI355X; PAGES_PAD_FROM is the pages' own."""
    if os.environ.get(KILL_SWITCH, "") not in ("", "0"):
        return False
    return n_tail >= pad_from


@dataclass
class TokenSteps:
    """Per-token inputs of a tail (what a decode loop receives per step) and the
    one-token step buffers: each token has its own output and selection, the rotated
    q/k and the workspace are shared."""
    q: List[torch.Tensor]
    k: List[torch.Tensor]
    v: List[torch.Tensor]
    cos: List[torch.Tensor]
    sin: List[torch.Tensor]
    bufs: List[StepBuffers]
    ones: torch.Tensor


def token_steps(cache: cp.KVCache, q, k, v, cos, sin, n_tail: int, window: int = 0) -> TokenSteps:
    """Split rows [0, n_tail) of a chunk's inputs into one-token steps (token j sits at
    position seen + j, so it takes row j of the chunk's tables)."""
    B, H, C, D = q.shape
    if not 0 < n_tail <= C:
        raise ValueError("n_tail must be in [1, C]")
    row = lambda t, j: t[:, :, j:j + 1].contiguous()
    trow = lambda t, j: t[:, j:j + 1].contiguous()
    qs = [row(q, j) for j in range(n_tail)]
    ks = [row(k, j) for j in range(n_tail)]
    vs = [row(v, j) for j in range(n_tail)]
    base = make_buffers(cache, qs[0], ks[0], vs[0], window=window)
    bufs = [dataclasses.replace(base, out=torch.empty_like(qs[0]),
                                sel=torch.empty_like(base.sel)) for _ in range(n_tail)]
    return TokenSteps(qs, ks, vs, [trow(cos, j) for j in range(n_tail)],
                      [trow(sin, j) for j in range(n_tail)], bufs,
                      torch.ones(B, dtype=torch.int32, device=q.device))


def scalar_tail(cache: cp.KVCache, steps: TokenSteps, window: int = 0):
    """The tail token by token: per token RoPE -> attention over past + 1 key (C = 1)
    -> append of one row.  Returns the per-token outputs [B, H, 1, D] and the last
    token's selection."""
    for j in range(len(steps.q)):
        chunk_step(cache, steps.q[j], steps.k[j], steps.v[j], steps.cos[j], steps.sin[j],
                   steps.ones, steps.bufs[j], window=window)
    return [b.out for b in steps.bufs], steps.bufs[-1].sel


def prefill_tail(cache: cp.KVCache, q, k, v, cos, sin, n_valid, n_tail: int,
                 chunk_bufs: StepBuffers, steps: TokenSteps, mask=None, window: int = 0,
                 static_append: bool = False, pad_from: int = PAD_FROM):
    """Run a prompt tail of n_tail real tokens (n_valid holds n_tail per sequence) by the
    tail policy.  Returns ("padded", out [B, H, C, D], sel) or ("scalar", [out per
    token], sel)."""
    if pad_tail(n_tail, pad_from):
        out, sel = chunk_step(cache, q, k, v, cos, sin, n_valid, chunk_bufs, mask=mask,
                              window=window, static_append=static_append)
        return "padded", out, sel
    outs, sel = scalar_tail(cache, steps, window=window)
    return "scalar", outs, sel


# ------------------------------------------------------------ whole prompts

@dataclass
class PromptChunks:
    """A prompt cut into chunks of C rows (the last one padded), with each chunk's
    inputs contiguous and its step buffers: what a chunked-prefill loop feeds its chunk
    graph ([SKaiNET] "Change (additive)": one fixed-C graph called per chunk)."""
    C: int
    n_valid: List[torch.Tensor]
    q: List[torch.Tensor]
    k: List[torch.Tensor]
    v: List[torch.Tensor]
    cos: List[torch.Tensor]
    sin: List[torch.Tensor]
    bufs: List[StepBuffers]


def prompt_chunks(cache: cp.KVCache, q, k, v, cos, sin, C: int, window: int = 0,
                  static_append: bool = False) -> PromptChunks:
    """Cut prompt tensors q [B, H, P, D], k, v [B, nKV, P, D], cos/sin [Bt, P, D] (row p at
    position seen + p) into ceil(P / C) chunks of C rows; the last chunk's missing rows
    are zero padding."""
    B, H, P, D = q.shape
    n = (P + C - 1) // C

    def piece(t, c):
        lo, hi = c * C, min(P, (c + 1) * C)
        out = torch.zeros(t.shape[:-2] + (C, t.shape[-1]), dtype=t.dtype, device=t.device)
        out[..., :hi - lo, :] = t[..., lo:hi, :]
        return out

    pc = PromptChunks(C, [], [], [], [], [], [], [])
    for c in range(n):
        pc.q.append(piece(q, c))
        pc.k.append(piece(k, c))
        pc.v.append(piece(v, c))
        pc.cos.append(piece(cos, c))
        pc.sin.append(piece(sin, c))
        pc.n_valid.append(torch.full((B,), min(C, P - c * C), dtype=torch.int32,
                                     device=q.device))
    base = make_buffers(cache, pc.q[0], pc.k[0], pc.v[0], window=window,
                        static_append=static_append)
    pc.bufs = [dataclasses.replace(base, out=torch.empty_like(pc.q[0]),
                                   sel=torch.empty_like(base.sel)) for _ in range(n)]
    return pc


def prefill(cache: cp.KVCache, pc: PromptChunks, window: int = 0,
            static_append: bool = False, seen_start: Optional[int] = None):
    """Run a whole prompt chunk after chunk (the cache grows as it goes); returns the last
    chunk's selection (the prompt's last real row).  seen_start: the largest seen before
    the prompt, when the host knows it -- chunk c then passes seen_start + c * C as the
    attention's bound on seen (at least 1: 0 means no bound)."""
    for c in range(len(pc.q)):
        ms = 0 if seen_start is None else max(1, seen_start + c * pc.C)
        chunk_step(cache, pc.q[c], pc.k[c], pc.v[c], pc.cos[c], pc.sin[c], pc.n_valid[c],
                   pc.bufs[c], window=window, static_append=static_append, max_seen=ms)
    return pc.bufs[-1].sel


def choose_chunk(prompt_len: int, step_us: dict) -> int:
    """Chunk-size selection: the C of a measured table {C: microseconds per chunk step}
    that minimises ceil(prompt_len / C) * step_us[C] (a padded last chunk costs a whole
    step; `bench.py --chunk-sweep` measures the table on this GPU).  Ties go to the
    smaller C (less padding)."""
    if prompt_len <= 0 or not step_us:
        raise ValueError("need a positive prompt length and a non-empty table")
    return min(sorted(step_us), key=lambda c: ((prompt_len + c - 1) // c) * step_us[c])
