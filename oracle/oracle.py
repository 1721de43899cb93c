"""ctypes front end of the CPU oracle (``cp_oracle.c``).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  It works on numpy
arrays: fp32 data as ``float32``, bf16 data as raw ``uint16`` bit patterns.
It imports nothing from the HIP package.
"""
import ctypes
import os

import numpy as np

from . import build as _build

F32, BF16 = 0, 1
OK, EARG, EWINDOW, EOVERFLOW = 0, -1, -4, -8
MASKED = np.float32(-1e30)

_lib = None


def lib():
    global _lib
    if _lib is None:
        path = os.environ.get("CP_ORACLE_LIB")  # a mutated copy (tests/oracle_mutations.py)
        if not path:
            path = _build.LIB
            if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_build.SRC):
                _build.build()
        L = ctypes.CDLL(path)
        vp, ip, i32p = ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p
        L.orc_rope.argtypes = [vp, vp, vp, vp, ip, ip, ip, ip, ip, ip]
        L.orc_slot.argtypes = [ip, ip, ip, ip]
        L.orc_live_positions.argtypes = [ip, ip, ip, ip, i32p]
        L.orc_kv_append.argtypes = [vp, vp, i32p, vp, ip, ip, ip, ip, ip, ip, ip, vp, vp, ip, i32p]
        L.orc_padded_overevicted.argtypes = [ip, ip, ip, ip, ip, ip, i32p]
        L.orc_build_mask.argtypes = [vp, i32p, i32p, ip, ip, ip, ctypes.c_long, ip, ip, ip, ip]
        L.orc_attn.argtypes = [vp, vp, vp, vp, vp, i32p, i32p, vp, ctypes.c_long, ctypes.c_long,
                               ctypes.c_long, ip, ip, ip, ip, ip, ip, ip, ip, ip, ctypes.c_float,
                               ip, vp, vp]
        L.orc_select_row.argtypes = [vp, vp, i32p, ip, ip, ip, ip, ip]
        L.orc_gdn.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, ip, ip, ip, ip, ip]
        for f in ("orc_rope", "orc_slot", "orc_live_positions", "orc_kv_append",
                  "orc_padded_overevicted", "orc_build_mask", "orc_attn", "orc_select_row",
                  "orc_num_threads", "orc_gdn"):
            getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _dtype_code(a):
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    raise TypeError(f"oracle storage must be float32 or uint16 (bf16 bits), got {a.dtype}")


def _c(a, dt=None):
    if a is None:
        return None
    a = np.asarray(a)
    return np.ascontiguousarray(a if dt is None else a.astype(dt, copy=False))


def _check(rc, what):
    if rc < 0:
        raise ValueError(f"oracle {what} returned {rc}")
    return rc


def rope(x, cos, sin):
    """RoPE of x [B,Hx,C,D] with fp32 tables [Bt,C,D]; returns a new array."""
    x = _c(x)
    cos, sin = _c(cos, np.float32), _c(sin, np.float32)
    B, Hx, C, D = x.shape
    y = np.empty_like(x)
    _check(lib().orc_rope(_ptr(x), _ptr(y), _ptr(cos), _ptr(sin), B, Hx, C, D, cos.shape[0],
                          _dtype_code(x)), "rope")
    return y


def slot(p, cap, ring, sink):
    return lib().orc_slot(int(p), int(cap), int(ring), int(sink))


def live_positions(seen, cap, ring, sink):
    out = np.zeros(max(cap, seen) + 1, dtype=np.int32)
    n = _check(lib().orc_live_positions(int(seen), int(cap), int(ring), int(sink), _ptr(out)),
               "live_positions")
    return out[:n].copy()


def kv_append(kc, vc, seen, kn, vn, n_rows=None, ring=0, sink=0):
    """Append the chunk rows; returns (kc', vc', seen', live[B,cap] bool). Inputs untouched."""
    kc, vc = _c(kc).copy(), _c(vc).copy()
    seen = _c(seen, np.int32).copy()
    kn, vn = _c(kn), _c(vn)
    n_rows = _c(n_rows, np.int32)
    B, nKV, cap, D = kc.shape
    C = kn.shape[2]
    live = np.zeros((B, cap), dtype=np.uint8)
    rc = lib().orc_kv_append(_ptr(kc), _ptr(vc), _ptr(seen), _ptr(live), B, nKV, cap, D,
                             _dtype_code(kc), int(ring), int(sink), _ptr(kn), _ptr(vn), C,
                             _ptr(n_rows))
    if rc == EOVERFLOW:
        raise OverflowError("global cache overflow")
    _check(rc, "kv_append")
    return kc, vc, seen, live.astype(bool)


def padded_overevicted(seen, n_valid, C, cap, ring, sink):
    out = np.zeros(C + 1, dtype=np.int32)
    rc = lib().orc_padded_overevicted(int(seen), int(n_valid), int(C), int(cap), int(ring),
                                      int(sink), _ptr(out))
    if rc == EWINDOW:
        raise ValueError("window <= chunk + sink")
    n = _check(rc, "padded_overevicted")
    return out[:n].copy()


def build_mask(seen, n_valid, H, C, ld, cap, ring=0, sink=0, window=0):
    seen = _c(seen, np.int32)
    n_valid = _c(n_valid, np.int32)
    B = seen.shape[0]
    m = np.empty((B, H, C, ld), dtype=np.float32)
    _check(lib().orc_build_mask(_ptr(m), _ptr(seen), _ptr(n_valid), B, H, C, int(ld), int(cap),
                                int(ring), int(sink), int(window)), "build_mask")
    return m


def attn(q, kn, vn, kc, vc, seen, n_valid=None, mask=None, ring=0, sink=0, window=0, scale=None,
         rows=None):
    """Attention of the chunk over past + C keys; returns fp64 [B,H,C,D].

    rows: optional iterable of chunk rows to compute (the others are zeros)."""
    q, kn, vn, kc, vc = _c(q), _c(kn), _c(vn), _c(kc), _c(vc)
    seen = _c(seen, np.int32)
    n_valid = _c(n_valid, np.int32)
    B, H, C, D = q.shape
    nKV, cap = kc.shape[1], kc.shape[2]
    if scale is None:
        scale = np.float32(1.0 / np.sqrt(D))
    mld = mhs = mbs = 0
    if mask is not None:
        mask = _c(mask, np.float32)
        if mask.ndim != 4:
            raise ValueError("mask must be [B|1, H|1, C, ld]")
        mld = mask.shape[3]
        mhs = mld * C if mask.shape[1] == H else 0
        mbs = mask.shape[1] * C * mld if mask.shape[0] == B else 0
    sel = None
    if rows is not None:
        sel = np.zeros(C, dtype=np.uint8)
        sel[np.asarray(list(rows), dtype=np.int64)] = 1
    out = np.zeros((B, H, C, D), dtype=np.float64)
    _check(lib().orc_attn(_ptr(q), _ptr(kn), _ptr(vn), _ptr(kc), _ptr(vc), _ptr(seen),
                          _ptr(n_valid), _ptr(mask), mld, mhs, mbs, B, H, nKV, C, D, cap,
                          int(ring), int(sink), int(window), float(scale), _dtype_code(q),
                          _ptr(sel), _ptr(out)), "attn")
    return out


def select_row(x, idx, off=-1):
    x = _c(x, np.float64)
    idx = _c(idx, np.int32)
    B, H, C, D = x.shape
    y = np.empty((B, H, D), dtype=np.float64)
    _check(lib().orc_select_row(_ptr(x), _ptr(y), _ptr(idx), int(off), B, H, C, D), "select_row")
    return y


def gdn(q, k, v, beta, alpha, s0=None):
    """Gated delta rule, token by token in fp64 ([Kazeia] "Le kernel actuel").
    q, k [B,H,P,dk], v [B,H,P,dv], beta, alpha [B,H,P] (alpha = log of the gate),
    s0 [B,H,dk,dv] or None (zero state).  Returns (out [B,H,P,dv], state [B,H,dk,dv]),
    both fp64."""
    q, k, v = _c(q, np.float32), _c(k, np.float32), _c(v, np.float32)
    beta, alpha = _c(beta, np.float32), _c(alpha, np.float32)
    s0 = _c(s0, np.float32)
    B, H, P, dk = q.shape
    dv = v.shape[3]
    out = np.zeros((B, H, P, dv), dtype=np.float64)
    st = np.zeros((B, H, dk, dv), dtype=np.float64)
    _check(lib().orc_gdn(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(alpha), _ptr(s0),
                         _ptr(out), _ptr(st), B, H, P, dk, dv), "gdn")
    return out, st


def num_threads():
    return lib().orc_num_threads()
