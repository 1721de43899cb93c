"""The C-ABI library loads and exports every symbol include/cp.h declares, its
struct layouts match the binding, and the host-side checks reject bad calls
before anything is enqueued.  CPU only: no call here reaches a kernel launch.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "cp.h")
LIB = os.path.join(ROOT, "chunked_prefill_attention_rope_amd", "libcp.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libcp.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(cp_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_path():
    names = declared_functions()
    for required in ("cp_rope_chunk", "cp_kv_append", "cp_kv_snapshot_padded_append",
                     "cp_kv_rollback_padded_append", "cp_attn_chunk_with_past", "cp_build_mask",
                     "cp_select_row", "cp_status_str", "cp_snapshot_bytes",
                     "cp_attn_workspace_bytes"):
        assert required in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(LIB)
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


def test_no_symbol_outside_the_header_is_exported_with_cp_prefix():
    out = os.popen(f"nm -D --defined-only {LIB}").read()
    exported = sorted(set(re.findall(r"\bT (cp_[a-z_0-9]+)$", out, flags=re.M)))
    assert exported == declared_functions()


@pytest.fixture(scope="module")
def cp():
    from chunked_prefill_attention_rope_amd import cp as mod
    return mod


def test_binding_loads_and_struct_sizes_match(cp):
    lib = cp.raw()
    assert lib.cp_abi_version() == cp.ABI_VERSION
    assert lib.cp_struct_size(0) == ctypes.sizeof(cp.CacheDesc) == 64
    assert lib.cp_struct_size(1) == ctypes.sizeof(cp.SnapshotDesc)
    assert lib.cp_struct_size(2) == ctypes.sizeof(cp.AttnArgs)
    assert lib.cp_struct_size(9) == 0


def test_status_strings(cp):
    for code in range(-8, 1):
        assert cp.status_str(code) and cp.status_str(code) != "unknown status"
    assert cp.status_str(-99) == "unknown status"


FAKE = 0x1000  # never dereferenced: every call below fails validation first


def _cache(cp, **kw):
    d = dict(k=FAKE, v=FAKE, seen=FAKE, status=None, B=2, nKV=2, cap=64, D=128, dtype=cp.BF16,
             ring=0, sink=0, reserved=0)
    d.update(kw)
    return cp.CacheDesc(**d)


def test_rope_validation(cp):
    f = cp.raw().cp_rope_chunk
    assert f(None, FAKE, FAKE, FAKE, 1, 1, 1, 8, 1, cp.BF16, None) == cp.ERR_ARG
    assert f(FAKE, FAKE, FAKE, FAKE, 1, 1, 1, 7, 1, cp.BF16, None) == cp.ERR_SHAPE
    assert f(FAKE, FAKE, FAKE, FAKE, 1, 1, 1, 8, 1, 5, None) == cp.ERR_DTYPE
    assert f(FAKE, FAKE, FAKE, FAKE, 3, 1, 1, 8, 2, cp.BF16, None) == cp.ERR_ARG


def test_rope_qk_validation(cp):
    f = cp.raw().cp_rope_qk_chunk
    args = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE]
    assert f(None, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 2, 1, 4, 8, 1, cp.BF16, None) == cp.ERR_ARG
    assert f(*args, 1, 2, 1, 4, 7, 1, cp.BF16, None) == cp.ERR_SHAPE
    assert f(*args, 1, 2, 1, 4, 8, 1, 9, None) == cp.ERR_DTYPE
    assert f(*args, 2, 2, 1, 4, 8, 3, cp.BF16, None) == cp.ERR_ARG
    assert f(*args, 1, -1, 1, 4, 8, 1, cp.BF16, None) == cp.ERR_ARG
    # empty work is a no-op, pointers may be NULL
    assert f(None, None, None, None, None, None, 1, 2, 1, 0, 8, 1, cp.BF16, None) == cp.OK


def test_append_validation(cp):
    f = cp.raw().cp_kv_append
    assert f(None, FAKE, FAKE, 4, None, None) == cp.ERR_ARG
    c = _cache(cp, k=None)
    assert f(ctypes.byref(c), FAKE, FAKE, 4, None, None) == cp.ERR_ARG
    c = _cache(cp, dtype=7)
    assert f(ctypes.byref(c), FAKE, FAKE, 4, None, None) == cp.ERR_DTYPE
    c = _cache(cp)
    assert f(ctypes.byref(c), FAKE, FAKE, 65, None, None) == cp.ERR_SHAPE  # C > cap, global
    c = _cache(cp, ring=1, sink=64)
    assert f(ctypes.byref(c), FAKE, FAKE, 4, None, None) == cp.ERR_ARG  # sink >= cap
    c = _cache(cp, reserved=1)
    assert f(ctypes.byref(c), FAKE, FAKE, 4, None, None) == cp.ERR_ARG


def test_snapshot_window_guard_and_sizes(cp):
    lib = cp.raw()
    c = _cache(cp, ring=1, cap=128, sink=0)
    need = lib.cp_snapshot_bytes(ctypes.byref(c), 128)
    snap = cp.SnapshotDesc(FAKE, need, None, 0, 0)
    # [cactus] review hardening: window <= chunk + sink is rejected
    assert lib.cp_kv_snapshot_padded_append(ctypes.byref(c), 128, None, ctypes.byref(snap),
                                            None) == cp.ERR_WINDOW
    c2 = _cache(cp, ring=1, cap=132, sink=4)
    assert lib.cp_kv_snapshot_padded_append(ctypes.byref(c2), 128, None, ctypes.byref(snap),
                                            None) == cp.ERR_WINDOW
    small = cp.SnapshotDesc(FAKE, 16, None, 0, 0)
    c3 = _cache(cp, ring=1, cap=512, sink=0)
    assert lib.cp_kv_snapshot_padded_append(ctypes.byref(c3), 128, None, ctypes.byref(small),
                                            None) == cp.ERR_WORKSPACE
    assert snap.armed == 0  # nothing was armed by the failing calls
    # header (2*B int32 padded to 256) + K and V rows of B*nKV*C*D bf16
    assert lib.cp_snapshot_bytes(ctypes.byref(c3), 128) == 256 + 2 * (2 * 2 * 128 * 128 * 2)
    assert lib.cp_snapshot_bytes(None, 4) == 0


def test_fused_snapshot_and_append_rollback_validation(cp):
    lib = cp.raw()
    f = lib.cp_rope_qk_snapshot_chunk
    g = lib.cp_kv_append_rollback
    c = _cache(cp, ring=1, cap=132, sink=4)
    need = lib.cp_snapshot_bytes(ctypes.byref(c), 128)
    snap = cp.SnapshotDesc(FAKE, need, None, 0, 0)
    args = lambda C=128, **kw: [kw.get(n, FAKE) for n in ("q", "q_out", "k", "k_out", "cos",
                                                           "sin")] + [8, C, 1, None]
    # [cactus] review hardening: window <= chunk + sink is rejected, nothing armed
    assert f(ctypes.byref(c), *args(), ctypes.byref(snap), None) == cp.ERR_WINDOW
    assert snap.armed == 0
    c2 = _cache(cp, ring=1, cap=512, sink=0)
    small = cp.SnapshotDesc(FAKE, 16, None, 0, 0)
    assert f(ctypes.byref(c2), *args(), ctypes.byref(small), None) == cp.ERR_WORKSPACE
    assert f(ctypes.byref(c2), *args(k=None), ctypes.byref(snap), None) == cp.ERR_ARG
    assert f(ctypes.byref(c2), *args(), None, None) == cp.ERR_ARG
    # the fused append needs the armed snapshot of this cache for this C
    assert g(ctypes.byref(c2), FAKE, FAKE, 128, ctypes.byref(snap), None) == cp.ERR_STATE
    armed = cp.SnapshotDesc(FAKE, need, 0x2000, 128, 1)  # armed, for another cache
    assert g(ctypes.byref(c2), FAKE, FAKE, 128, ctypes.byref(armed), None) == cp.ERR_STATE
    mine = cp.SnapshotDesc(FAKE, 1 << 20, FAKE, 64, 1)  # this cache, another C
    assert g(ctypes.byref(c2), FAKE, FAKE, 128, ctypes.byref(mine), None) == cp.ERR_STATE
    assert mine.armed == 1


def test_rollback_requires_armed_matching_snapshot(cp):
    lib = cp.raw()
    c = _cache(cp, ring=1, cap=512)
    snap = cp.SnapshotDesc(FAKE, 1 << 20, None, 0, 0)
    assert lib.cp_kv_rollback_padded_append(ctypes.byref(c), ctypes.byref(snap),
                                            None) == cp.ERR_STATE
    snap = cp.SnapshotDesc(FAKE, 1 << 20, 0x2000, 16, 1)  # armed, but for another cache
    assert lib.cp_kv_rollback_padded_append(ctypes.byref(c), ctypes.byref(snap),
                                            None) == cp.ERR_STATE


def test_split_count_from_max_seen(cp):
    """Host planner: the key splits of a one-sequence chunk are counted from max_seen
    when the caller gives it (else from the capacity), two 32-key tiles per split, the
    count rounded up.  Read off the workspace size, which is splits x partial rows x
    (D bf16 + fp32 m and l)."""
    lib = cp.raw()
    c = _cache(cp, B=1, nKV=1, cap=1024, D=256)

    def ws(max_seen):
        a = cp.AttnArgs(q=FAKE, k_new=FAKE, v_new=FAKE, out=FAKE, mask=FAKE, mask_ld=1088,
                        mask_head_stride=64 * 1088, H=4, C=64, scale=0.0625, max_seen=max_seen)
        return lib.cp_attn_workspace_bytes(ctypes.byref(c), ctypes.byref(a))

    rows = 256  # two 128-row query tiles (4 heads x 32 chunk rows)
    per_split = rows * 256 * 2 + rows * 2 * 4
    assert ws(0) == 17 * per_split      # 1024 + 64 keys: 34 tiles
    assert ws(5000) == ws(0)            # a bound above the capacity changes nothing
    assert ws(800) == 14 * per_split    # 800 + 64 keys: 27 tiles, rounded up
    assert ws(1) == 2 * per_split       # 1 + 64 keys: 3 tiles


def test_attention_validation(cp):
    lib = cp.raw()
    c = _cache(cp)

    def args(**kw):
        d = dict(q=FAKE, k_new=FAKE, v_new=FAKE, out=FAKE, n_valid=None, mask=None, mask_ld=0,
                 mask_head_stride=0, mask_batch_stride=0, workspace=None, workspace_bytes=0,
                 H=8, C=16, window=0, scale=0.1, flags=0, reserved=0, q_cos=None, q_sin=None,
                 q_tables=0, max_seen=0)
        d.update(kw)
        return cp.AttnArgs(**d)

    f = lib.cp_attn_chunk_with_past
    assert f(ctypes.byref(c), ctypes.byref(args(q=None)), None) == cp.ERR_ARG
    assert f(ctypes.byref(c), ctypes.byref(args(H=7)), None) == cp.ERR_SHAPE  # H % nKV
    assert f(ctypes.byref(c), ctypes.byref(args(scale=float("nan"))), None) == cp.ERR_ARG
    assert f(ctypes.byref(c), ctypes.byref(args(mask=FAKE, mask_ld=8)), None) == cp.ERR_ARG
    assert f(ctypes.byref(c), ctypes.byref(args(C=65)), None) == cp.ERR_SHAPE
    # query tables: both or neither, one per batch or per sequence, even D
    assert f(ctypes.byref(c), ctypes.byref(args(q_cos=FAKE)), None) == cp.ERR_ARG
    assert f(ctypes.byref(c), ctypes.byref(args(q_cos=FAKE, q_sin=FAKE, q_tables=3)),
             None) == cp.ERR_ARG
    assert f(ctypes.byref(c), ctypes.byref(args(max_seen=-1)), None) == cp.ERR_ARG
    odd = _cache(cp, D=63)
    assert f(ctypes.byref(odd), ctypes.byref(args(q_cos=FAKE, q_sin=FAKE, q_tables=1)),
             None) == cp.ERR_SHAPE
    big = _cache(cp, D=512)
    assert f(ctypes.byref(big), ctypes.byref(args()), None) == cp.ERR_SHAPE
    assert lib.cp_attn_workspace_bytes(ctypes.byref(c), ctypes.byref(args(H=7))) == 0
    # the non-allocating form validates identically, before it looks at its scratch
    g = lib.cp_attn_chunk_with_past_noalloc
    assert g(ctypes.byref(c), ctypes.byref(args(q=None)), None) == cp.ERR_ARG
    assert g(ctypes.byref(c), ctypes.byref(args(H=7)), None) == cp.ERR_SHAPE
    assert g(ctypes.byref(big), ctypes.byref(args()), None) == cp.ERR_SHAPE
    # splits needing more than the fixed array are refused before any device call:
    # 64 forced splits of B=64 x 8 KV heads x 16 query tiles of 128 rows x D 256 fp32
    huge = _cache(cp, B=64, nKV=8, cap=8192, D=256)
    a = args(H=32, C=512, flags=cp.ATTN_SPLITS(64))
    assert lib.cp_attn_workspace_bytes(ctypes.byref(huge), ctypes.byref(a)) > cp.ATTN_SCRATCH_BYTES
    assert g(ctypes.byref(huge), ctypes.byref(a), None) == cp.ERR_SCRATCH


def test_select_and_mask_validation(cp):
    lib = cp.raw()
    assert lib.cp_select_row(None, FAKE, FAKE, -1, 1, 1, 1, 8, cp.BF16, None) == cp.ERR_ARG
    assert lib.cp_select_row(FAKE, FAKE, FAKE, -1, 1, 1, 1, 8, 9, None) == cp.ERR_DTYPE
    c = _cache(cp)
    assert lib.cp_build_mask(None, 8, ctypes.byref(c), None, 4, 2, 0, None) == cp.ERR_ARG
    assert lib.cp_build_mask(FAKE, 8, ctypes.byref(c), None, 0, 2, 0, None) == cp.ERR_ARG


def test_gdn_validation(cp):
    lib = cp.raw()
    f = lib.cp_gdn_chunk_prefill
    ws = cp.gdn_workspace_bytes(1, 2, 100, 64, 64)
    # per (sequence, head, chunk of 64): W, U, P, lg, K^T (fp32)
    assert ws == 1 * 2 * 2 * (64 * 64 + 64 * 64 + 64 * 64 + 64 + 64 * 64) * 4
    assert cp.gdn_workspace_bytes(1, 2, 100, 96, 64) == 0
    call = lambda **kw: f(*[kw.get(n, FAKE) for n in ("q", "k", "v", "beta", "alpha", "state", "out")],
                          kw.get("B", 1), kw.get("H", 2), kw.get("P", 100), kw.get("dk", 64),
                          kw.get("dv", 64), kw.get("ws", FAKE), kw.get("wsb", ws), None)
    assert call(dk=96) == cp.ERR_SHAPE
    assert call(dv=256) == cp.ERR_SHAPE
    assert call(B=65535, H=65535, P=1 << 20) == cp.ERR_SHAPE  # beyond one launch grid
    assert call(P=-1) == cp.ERR_ARG
    assert call(q=None) == cp.ERR_ARG
    assert call(ws=None) == cp.ERR_ARG
    assert call(q=FAKE + 4) == cp.ERR_ARG  # not 16-byte aligned
    assert call(wsb=ws - 1) == cp.ERR_WORKSPACE
    assert call(P=0, q=None, ws=None) == cp.OK  # empty prompt: nothing is read


def test_rope_qk_append_and_advance_validation(cp):
    lib = cp.raw()
    f = lib.cp_rope_qk_append_chunk
    c = _cache(cp)
    call = lambda cache=c, **kw: f(ctypes.byref(cache), *[kw.get(n, FAKE) for n in
                                   ("q", "q_out", "k", "k_out", "v", "cos", "sin")],
                                   kw.get("H", 8), kw.get("C", 16), kw.get("Bt", 1), None, None)
    assert call(cache=_cache(cp, ring=1)) == cp.ERR_ARG  # ring appends evict
    assert call(cache=_cache(cp, D=63)) == cp.ERR_SHAPE
    assert call(C=10 ** 6) == cp.ERR_SHAPE
    assert call(Bt=3) == cp.ERR_ARG
    assert call(k=None) == cp.ERR_ARG
    assert call(v=None) == cp.ERR_ARG
    assert call(H=-1) == cp.ERR_ARG
    assert call(C=0, k=None, v=None) == cp.OK
    g = lib.cp_kv_advance
    assert g(ctypes.byref(c), -1, None, None) == cp.ERR_ARG
    assert g(ctypes.byref(c), 10 ** 6, None, None) == cp.ERR_SHAPE
    assert g(ctypes.byref(c), 0, None, None) == cp.OK
