"""Thin Python binding of libcp (C ABI in include/cp.h).

Argument marshalling only: torch tensors are checked for device, dtype and
layout and passed as raw device pointers together with torch's current HIP
stream.  Every step of the path runs in libcp's HIP kernels; nothing here
computes.  Importing this module loads the library and raises ImportError if
it has not been built (``python -m chunked_prefill_attention_rope_amd.build``).
"""
import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcp.so")

OK, ERR_ARG, ERR_SHAPE, ERR_DTYPE, ERR_WINDOW, ERR_STATE, ERR_WORKSPACE, ERR_HIP = (
    0, -1, -2, -3, -4, -5, -6, -7)
ERR_SCRATCH = -8
ATTN_SCRATCH_BYTES = 64 << 20  # CP_ATTN_SCRATCH_BYTES
DEV_OVERFLOW, DEV_NVALID, DEV_MASK_LD, DEV_ROLLBACK, DEV_SEEN = 1, 2, 4, 8, 16
F32, BF16 = 0, 1
ATTN_NO_SPLIT, ATTN_FORCE_GENERIC, ATTN_FULL_TILES, ATTN_ADVANCE_SEEN = 1, 2, 4, 8
ATTN_BALANCE = 16


def ATTN_SPLITS(n: int) -> int:
    """CP_ATTN_SPLITS(n): force n key splits (bits 8..15 of the flags)."""
    return (int(n) & 0xFF) << 8
ABI_VERSION = 4

if not os.path.exists(LIB_PATH):
    raise ImportError(f"libcp.so is not built ({LIB_PATH}); run "
                      "`python -m chunked_prefill_attention_rope_amd.build`")
_lib = ctypes.CDLL(LIB_PATH)


class CacheDesc(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("seen", ctypes.c_void_p),
                ("status", ctypes.c_void_p), ("B", ctypes.c_int32), ("nKV", ctypes.c_int32),
                ("cap", ctypes.c_int32), ("D", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("ring", ctypes.c_int32), ("sink", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class SnapshotDesc(ctypes.Structure):
    _fields_ = [("buf", ctypes.c_void_p), ("bytes", ctypes.c_size_t),
                ("cache_k", ctypes.c_void_p), ("C", ctypes.c_int32), ("armed", ctypes.c_int32)]


class AttnArgs(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("k_new", ctypes.c_void_p), ("v_new", ctypes.c_void_p),
                ("out", ctypes.c_void_p), ("n_valid", ctypes.c_void_p), ("mask", ctypes.c_void_p),
                ("mask_ld", ctypes.c_int64), ("mask_head_stride", ctypes.c_int64),
                ("mask_batch_stride", ctypes.c_int64), ("workspace", ctypes.c_void_p),
                ("workspace_bytes", ctypes.c_size_t), ("H", ctypes.c_int32),
                ("C", ctypes.c_int32), ("window", ctypes.c_int32), ("scale", ctypes.c_float),
                ("flags", ctypes.c_uint32), ("reserved", ctypes.c_int32),
                ("select_out", ctypes.c_void_p), ("q_cos", ctypes.c_void_p),
                ("q_sin", ctypes.c_void_p), ("q_tables", ctypes.c_int32),
                ("max_seen", ctypes.c_int32)]


_vp, _i = ctypes.c_void_p, ctypes.c_int
_P = ctypes.POINTER
_SIGS = {
    "cp_status_str": (ctypes.c_char_p, [_i]),
    "cp_abi_version": (_i, []),
    "cp_struct_size": (ctypes.c_size_t, [_i]),
    "cp_rope_chunk": (_i, [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _vp]),
    "cp_rope_qk_chunk": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _vp]),
    "cp_kv_append": (_i, [_P(CacheDesc), _vp, _vp, _i, _vp, _vp]),
    "cp_kv_advance": (_i, [_P(CacheDesc), _i, _vp, _vp]),
    "cp_rope_qk_append_chunk": (_i, [_P(CacheDesc), _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i,
                                     _i, _vp, _vp]),
    "cp_rope_qk_snapshot_chunk": (_i, [_P(CacheDesc), _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i,
                                       _vp, _P(SnapshotDesc), _vp]),
    "cp_kv_append_rollback": (_i, [_P(CacheDesc), _vp, _vp, _i, _P(SnapshotDesc), _vp]),
    "cp_snapshot_bytes": (ctypes.c_size_t, [_P(CacheDesc), _i]),
    "cp_kv_snapshot_padded_append": (_i, [_P(CacheDesc), _i, _vp, _P(SnapshotDesc), _vp]),
    "cp_kv_rollback_padded_append": (_i, [_P(CacheDesc), _P(SnapshotDesc), _vp]),
    "cp_attn_workspace_bytes": (ctypes.c_size_t, [_P(CacheDesc), _P(AttnArgs)]),
    "cp_attn_chunk_with_past": (_i, [_P(CacheDesc), _P(AttnArgs), _vp]),
    "cp_attn_chunk_with_past_noalloc": (_i, [_P(CacheDesc), _P(AttnArgs), _vp]),
    "cp_build_mask": (_i, [_vp, ctypes.c_int64, _P(CacheDesc), _vp, _i, _i, _i, _vp]),
    "cp_select_row": (_i, [_vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _vp]),
    "cp_gdn_workspace_bytes": (ctypes.c_size_t, [_i, _i, _i, _i, _i]),
    "cp_gdn_chunk_prefill": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _vp,
                                  ctypes.c_size_t, _vp]),
}
for _name, (_res, _args) in _SIGS.items():
    _f = getattr(_lib, _name)
    _f.restype = _res
    _f.argtypes = _args

for _which, _cls in enumerate((CacheDesc, SnapshotDesc, AttnArgs)):
    if _lib.cp_struct_size(_which) != ctypes.sizeof(_cls):
        raise ImportError(f"libcp ABI mismatch for {_cls.__name__}")
if _lib.cp_abi_version() != ABI_VERSION:
    raise ImportError("libcp ABI version mismatch")


class CpError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {_lib.cp_status_str(code).decode()} ({code})")


def _check(code: int, where: str):
    if code != OK:
        raise CpError(code, where)


def status_str(code: int) -> str:
    return _lib.cp_status_str(code).decode()


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _dev(t: torch.Tensor, name: str) -> int:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _opt(t: Optional[torch.Tensor], name: str, dtype=None):
    if t is None:
        return None
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}")
    return _dev(t, name)


# --------------------------------------------------------------------- RoPE

def rope_chunk(x: torch.Tensor, cos: torch.Tensor, sin: torch.Tensor,
               out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """cp_rope_chunk: x [B, Hx, C, D]; cos/sin fp32 [Bt, C, D]; out may be x."""
    if out is None:
        out = torch.empty_like(x)
    B, Hx, C, D = x.shape
    if out.shape != x.shape or out.dtype != x.dtype:
        raise ValueError("out must match x")
    _check(_lib.cp_rope_chunk(_dev(x, "x"), _dev(out, "out"), _opt(cos, "cos", torch.float32),
                              _opt(sin, "sin", torch.float32), B, Hx, C, D, cos.shape[0],
                              _dtype_code(x), _stream()), "cp_rope_chunk")
    return out


def rope_qk_chunk(q: torch.Tensor, k: torch.Tensor, cos: torch.Tensor, sin: torch.Tensor,
                  q_out: Optional[torch.Tensor] = None,
                  k_out: Optional[torch.Tensor] = None):
    """cp_rope_qk_chunk: q [B, H, C, D] and k [B, nKV, C, D] rotated by one launch."""
    if q_out is None:
        q_out = torch.empty_like(q)
    if k_out is None:
        k_out = torch.empty_like(k)
    B, H, C, D = q.shape
    if k.shape[0] != B or k.shape[2:] != q.shape[2:] or k.dtype != q.dtype:
        raise ValueError("k must be [B, nKV, C, D] of q's dtype")
    if q_out.shape != q.shape or q_out.dtype != q.dtype or k_out.shape != k.shape \
            or k_out.dtype != k.dtype:
        raise ValueError("outputs must match their inputs")
    _check(_lib.cp_rope_qk_chunk(_dev(q, "q"), _dev(q_out, "q_out"), _dev(k, "k"),
                                 _dev(k_out, "k_out"), _opt(cos, "cos", torch.float32),
                                 _opt(sin, "sin", torch.float32), B, H, k.shape[1], C, D,
                                 cos.shape[0], _dtype_code(q), _stream()), "cp_rope_qk_chunk")
    return q_out, k_out


# ----------------------------------------------------------------- KV cache

class KVCache:
    """A caller-owned external KV cache (device tensors) and its C descriptor.

    k, v: [B, nKV, cap, D]; seen: int32 [B] (positions absorbed); ring/sink as
    in cp_cache; status: optional int32 [1] collecting CP_DEV_* bits.
    """

    def __init__(self, k: torch.Tensor, v: torch.Tensor, seen: torch.Tensor, ring: int = 0,
                 sink: int = 0, status: Optional[torch.Tensor] = None):
        if k.shape != v.shape or k.dtype != v.dtype or k.dim() != 4:
            raise ValueError("k and v must be [B, nKV, cap, D] of one dtype")
        if seen.dtype != torch.int32 or seen.shape != (k.shape[0],):
            raise ValueError("seen must be int32 [B]")
        if status is not None and status.dtype != torch.int32:
            raise ValueError("status must be int32")
        self.k, self.v, self.seen, self.status = k, v, seen, status
        self.ring, self.sink = int(ring), int(sink)
        B, nKV, cap, D = k.shape
        self.desc = CacheDesc(_dev(k, "k"), _dev(v, "v"), _dev(seen, "seen"),
                              _opt(status, "status"), B, nKV, cap, D, _dtype_code(k),
                              self.ring, self.sink, 0)

    @property
    def B(self):
        return self.desc.B

    @property
    def nKV(self):
        return self.desc.nKV

    @property
    def cap(self):
        return self.desc.cap

    @property
    def D(self):
        return self.desc.D


def rope_qk_append_chunk(cache: KVCache, q: Optional[torch.Tensor], k: torch.Tensor,
                         v: torch.Tensor, cos: torch.Tensor, sin: torch.Tensor,
                         n_valid: Optional[torch.Tensor] = None,
                         q_out: Optional[torch.Tensor] = None,
                         k_out: Optional[torch.Tensor] = None):
    """cp_rope_qk_append_chunk: rotate q (None: keys only) and k, and write rows
    [0, n_valid[b]) of the rotated k and of v past seen in a global cache (seen is not
    advanced)."""
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t is None:
            continue
        if t.dtype != cache.k.dtype or t.shape[0] != cache.B or t.shape[3] != cache.k.shape[3]:
            raise ValueError(f"{name} must be [B, heads, C, D] in the cache's dtype")
    if k.shape != v.shape or k.shape[1] != cache.k.shape[1]:
        raise ValueError("k and v must be [B, nKV, C, D]")
    if q is not None and q_out is None:
        q_out = torch.empty_like(q)
    if k_out is None:
        k_out = torch.empty_like(k)
    C = k.shape[2]
    _check(_lib.cp_rope_qk_append_chunk(
        ctypes.byref(cache.desc), _opt(q, "q"), _opt(q_out, "q_out"), _dev(k, "k"),
        _dev(k_out, "k_out"), _dev(v, "v"), _opt(cos, "cos", torch.float32),
        _opt(sin, "sin", torch.float32), q.shape[1] if q is not None else 0, C, cos.shape[0],
        _opt(n_valid, "n_valid", torch.int32), _stream()), "cp_rope_qk_append_chunk")
    return q_out, k_out


def kv_advance(cache: KVCache, C: int, n_rows: Optional[torch.Tensor] = None) -> None:
    """cp_kv_advance: seen[b] += n_rows[b] (C when None), as cp_kv_append would."""
    _check(_lib.cp_kv_advance(ctypes.byref(cache.desc), C, _opt(n_rows, "n_rows", torch.int32),
                              _stream()), "cp_kv_advance")


def kv_append(cache: KVCache, k_new: torch.Tensor, v_new: torch.Tensor,
              n_rows: Optional[torch.Tensor] = None) -> None:
    """cp_kv_append: append rows [0, n_rows[b]) (all C rows when None)."""
    C = k_new.shape[2]
    _check(_lib.cp_kv_append(ctypes.byref(cache.desc), _dev(k_new, "k_new"),
                             _dev(v_new, "v_new"), C, _opt(n_rows, "n_rows", torch.int32),
                             _stream()), "cp_kv_append")


def snapshot_bytes(cache: KVCache, C: int) -> int:
    return int(_lib.cp_snapshot_bytes(ctypes.byref(cache.desc), int(C)))


class Snapshot:
    """Caller-owned snapshot buffer (uint8 device tensor) and its descriptor."""

    def __init__(self, buf: torch.Tensor):
        self.buf = buf
        self.desc = SnapshotDesc(_dev(buf, "buf"), buf.numel() * buf.element_size(), None, 0, 0)

    @property
    def armed(self):
        return bool(self.desc.armed)


def kv_snapshot_padded_append(cache: KVCache, C: int, n_valid: Optional[torch.Tensor],
                              snap: Optional[Snapshot] = None) -> Snapshot:
    """cp_kv_snapshot_padded_append (allocates the buffer when snap is None)."""
    if snap is None:
        snap = Snapshot(torch.empty(snapshot_bytes(cache, C), dtype=torch.uint8,
                                    device=cache.k.device))
    _check(_lib.cp_kv_snapshot_padded_append(ctypes.byref(cache.desc), int(C),
                                             _opt(n_valid, "n_valid", torch.int32),
                                             ctypes.byref(snap.desc), _stream()),
           "cp_kv_snapshot_padded_append")
    return snap


def kv_rollback_padded_append(cache: KVCache, snap: Snapshot) -> None:
    _check(_lib.cp_kv_rollback_padded_append(ctypes.byref(cache.desc), ctypes.byref(snap.desc),
                                             _stream()), "cp_kv_rollback_padded_append")


def rope_qk_snapshot_chunk(cache: KVCache, q: Optional[torch.Tensor], k: torch.Tensor,
                           cos: torch.Tensor, sin: torch.Tensor,
                           n_valid: Optional[torch.Tensor], snap: Snapshot,
                           q_out: Optional[torch.Tensor] = None,
                           k_out: Optional[torch.Tensor] = None):
    """cp_rope_qk_snapshot_chunk: rotate q (None: keys only) and k, and take the padded-
    append snapshot into snap, in one launch."""
    if k.dtype != cache.k.dtype or k.shape[0] != cache.B or k.shape[1] != cache.nKV \
            or k.shape[3] != cache.D:
        raise ValueError("k must be [B, nKV, C, D] in the cache's dtype")
    if q is not None and (q.dtype != k.dtype or q.shape[0] != k.shape[0] or
                          q.shape[2:] != k.shape[2:]):
        raise ValueError("q must be [B, H, C, D] of k's dtype")
    if k_out is None:
        k_out = torch.empty_like(k)
    if q is not None and q_out is None:
        q_out = torch.empty_like(q)
    H = q.shape[1] if q is not None else 0
    _check(_lib.cp_rope_qk_snapshot_chunk(
        ctypes.byref(cache.desc), _opt(q, "q"), _opt(q_out, "q_out"), _dev(k, "k"),
        _dev(k_out, "k_out"), _opt(cos, "cos", torch.float32), _opt(sin, "sin", torch.float32),
        H, k.shape[2], cos.shape[0], _opt(n_valid, "n_valid", torch.int32),
        ctypes.byref(snap.desc), _stream()), "cp_rope_qk_snapshot_chunk")
    return q_out, k_out


def kv_append_rollback(cache: KVCache, k_new: torch.Tensor, v_new: torch.Tensor,
                       snap: Snapshot) -> None:
    """cp_kv_append_rollback: the padded append of all C rows and its rollback, one launch."""
    _check(_lib.cp_kv_append_rollback(ctypes.byref(cache.desc), _dev(k_new, "k_new"),
                                      _dev(v_new, "v_new"), k_new.shape[2],
                                      ctypes.byref(snap.desc), _stream()),
           "cp_kv_append_rollback")


# ---------------------------------------------------------------- attention

def _attn_args(cache, q, k_new, v_new, out, n_valid, mask, window, scale, workspace, flags,
               select_out=None, q_rope=None, max_seen=0):
    B, H, C, D = q.shape
    if scale is None:
        scale = float(torch.tensor(1.0 / D ** 0.5, dtype=torch.float32))
    mld = mhs = mbs = 0
    mptr = None
    if mask is not None:
        if mask.dtype != torch.float32 or mask.dim() != 4:
            raise ValueError("mask must be fp32 [B|1, H|1, C, ld]")
        mptr = _dev(mask, "mask")
        mld = mask.shape[3]
        mhs = mld * C if mask.shape[1] == H else 0
        mbs = mask.shape[1] * C * mld if mask.shape[0] == B else 0
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        ws_ptr, ws_bytes = _dev(workspace, "workspace"), workspace.numel() * workspace.element_size()
    qc = qs = None
    qt = 0
    if q_rope is not None:
        cos, sin = q_rope
        qc, qs, qt = _opt(cos, "q_cos", torch.float32), _opt(sin, "q_sin", torch.float32), \
            cos.shape[0]
    return AttnArgs(_dev(q, "q"), _dev(k_new, "k_new"), _dev(v_new, "v_new"),
                    _dev(out, "out") if out is not None else None,
                    _opt(n_valid, "n_valid", torch.int32), mptr, mld, mhs, mbs, ws_ptr, ws_bytes,
                    H, C, int(window), float(scale), int(flags), 0,
                    _dev(select_out, "select_out") if select_out is not None else None,
                    qc, qs, qt, int(max_seen))


def attn_workspace_bytes(cache: KVCache, q: torch.Tensor, k_new: torch.Tensor,
                         v_new: torch.Tensor, mask: Optional[torch.Tensor] = None,
                         window: int = 0, flags: int = 0, max_seen: int = 0) -> int:
    a = _attn_args(cache, q, k_new, v_new, q, None, mask, window, None, None, flags,
                   max_seen=max_seen)
    return int(_lib.cp_attn_workspace_bytes(ctypes.byref(cache.desc), ctypes.byref(a)))


def attn_chunk_with_past(cache: KVCache, q: torch.Tensor, k_new: torch.Tensor,
                         v_new: torch.Tensor, n_valid: Optional[torch.Tensor] = None,
                         mask: Optional[torch.Tensor] = None, window: int = 0,
                         scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                         workspace: Optional[torch.Tensor] = None,
                         flags: int = 0,
                         select_out: Optional[torch.Tensor] = None,
                         q_rope=None, max_seen: int = 0) -> torch.Tensor:
    """cp_attn_chunk_with_past over the cache as it stands (before the append).

    select_out [B, H, D] (optional) also receives the last real row of each (b, h).
    q_rope = (cos, sin): q is not rotated yet; the kernel rotates it with these tables.
    max_seen: 0, or the host's upper bound on every seen (sizes the key splits).
    """
    if out is None:
        out = torch.empty_like(q)
    if select_out is not None and (select_out.dtype != q.dtype or
                                   select_out.shape != (q.shape[0], q.shape[1], q.shape[3])):
        raise ValueError("select_out must be [B, H, D] of q's dtype")
    a = _attn_args(cache, q, k_new, v_new, out, n_valid, mask, window, scale, workspace, flags,
                   select_out, q_rope, max_seen)
    _check(_lib.cp_attn_chunk_with_past(ctypes.byref(cache.desc), ctypes.byref(a), _stream()),
           "cp_attn_chunk_with_past")
    return out


def attn_chunk_with_past_noalloc(cache: KVCache, q: torch.Tensor, k_new: torch.Tensor,
                                 v_new: torch.Tensor, out: torch.Tensor,
                                 n_valid: Optional[torch.Tensor] = None,
                                 mask: Optional[torch.Tensor] = None, window: int = 0,
                                 scale: Optional[float] = None, flags: int = 0,
                                 select_out: Optional[torch.Tensor] = None,
                                 q_rope=None, max_seen: int = 0) -> torch.Tensor:
    """cp_attn_chunk_with_past_noalloc: the same attention with the key-split partials in
    the library's own device array (no workspace; the caller passes its output)."""
    if select_out is not None and (select_out.dtype != q.dtype or
                                   select_out.shape != (q.shape[0], q.shape[1], q.shape[3])):
        raise ValueError("select_out must be [B, H, D] of q's dtype")
    a = _attn_args(cache, q, k_new, v_new, out, n_valid, mask, window, scale, None, flags,
                   select_out, q_rope, max_seen)
    _check(_lib.cp_attn_chunk_with_past_noalloc(ctypes.byref(cache.desc), ctypes.byref(a),
                                                _stream()), "cp_attn_chunk_with_past_noalloc")
    return out


def build_mask(cache: KVCache, n_valid: Optional[torch.Tensor], H: int, C: int, ld: int,
               window: int = 0, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """cp_build_mask: explicit fp32 mask [B, H, C, ld] from the in-kernel rule."""
    if out is None:
        out = torch.empty((cache.B, H, C, ld), dtype=torch.float32, device=cache.k.device)
    _check(_lib.cp_build_mask(_dev(out, "mask"), int(ld), ctypes.byref(cache.desc),
                              _opt(n_valid, "n_valid", torch.int32), int(H), int(C), int(window),
                              _stream()), "cp_build_mask")
    return out


def select_row(x: torch.Tensor, idx: torch.Tensor, offset: int = -1,
               out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """cp_select_row: y[b, h] = x[b, h, idx[b] + offset] (zeros out of range)."""
    B, H, C, D = x.shape
    if out is None:
        out = torch.empty((B, H, D), dtype=x.dtype, device=x.device)
    _check(_lib.cp_select_row(_dev(x, "x"), _dev(out, "out"), _opt(idx, "idx", torch.int32),
                              int(offset), B, H, C, D, _dtype_code(x), _stream()),
           "cp_select_row")
    return out


# ------------------------------------------------------- gated delta rule

def gdn_workspace_bytes(B: int, H: int, P: int, dk: int, dv: int) -> int:
    return int(_lib.cp_gdn_workspace_bytes(int(B), int(H), int(P), int(dk), int(dv)))


def gdn_chunk_prefill(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, beta: torch.Tensor,
                      alpha: torch.Tensor, state: torch.Tensor,
                      out: Optional[torch.Tensor] = None,
                      workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """cp_gdn_chunk_prefill: fp32 q, k [B,H,P,dk], v [B,H,P,dv], beta, alpha [B,H,P];
    state [B,H,dk,dv] is updated in place to the state after the last token."""
    B, H, P, dk = q.shape
    dv = v.shape[3]
    for name, t in (("q", q), ("k", k), ("v", v), ("beta", beta), ("alpha", alpha),
                    ("state", state)):
        if t.dtype != torch.float32:
            raise TypeError(f"{name} must be float32")
    if k.shape != q.shape or v.shape[:3] != q.shape[:3] or beta.shape != q.shape[:3] \
            or alpha.shape != q.shape[:3] or state.shape != (B, H, dk, dv):
        raise ValueError("inconsistent gated-delta-rule shapes")
    if out is None:
        out = torch.empty_like(v)
    if workspace is None:
        workspace = torch.empty(max(gdn_workspace_bytes(B, H, P, dk, dv), 1), dtype=torch.uint8,
                                device=q.device)
    _check(_lib.cp_gdn_chunk_prefill(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(beta, "beta"),
                                     _dev(alpha, "alpha"), _dev(state, "state"), _dev(out, "out"),
                                     B, H, P, dk, dv, _dev(workspace, "workspace"),
                                     workspace.numel() * workspace.element_size(), _stream()),
           "cp_gdn_chunk_prefill")
    return out


def raw():
    """The loaded ctypes library (for ABI tests)."""
    return _lib
