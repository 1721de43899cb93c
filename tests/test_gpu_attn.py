"""GPU parity of the chunk attention (HIP path through the C ABI vs the CPU oracle).

Tolerance: max over real rows of max_d |out - ref| / max_d |ref| <= 1e-4 (fp32
storage) or 2e-2 (bf16 storage, fp32 accumulation), ref = the oracle's fp64
result.  Identities the kernels must keep exactly (explicit vs in-kernel
mask on one key partition, determinism, selection) are checked bitwise.
"""
import numpy as np
import pytest
import torch

from chunked_prefill_attention_rope_amd import inputs as I
from oracle import oracle as O
from tests.gpu_helpers import TOL, bits, dev, real_rows_mask, rowwise_rel_err, to_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def cp():
    from chunked_prefill_attention_rope_amd import cp as mod
    return mod


def _np(t):
    return I.np_view(t)


def _setup(cp, cfg, nan_dead=True):
    t = I.make_layer(cfg, nan_dead=nan_dead)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    cache = cp.KVCache(dev(t["kc"]), dev(t["vc"]), dev(t["seen"]), ring=cfg.ring, sink=cfg.sink,
                       status=status)
    return t, cache, status


def _run(cp, cfg, t, cache, explicit=False, flags=0, workspace=True):
    q, k, v = dev(t["q"]), dev(t["k"]), dev(t["v"])
    nv = dev(t["n_valid"])
    mask = None
    if explicit:
        mask = cp.build_mask(cache, nv, cfg.H, cfg.C, cfg.mask_ld(), window=cfg.window)
    ws = None
    if workspace:
        nb = cp.attn_workspace_bytes(cache, q, k, v, mask=mask, window=cfg.window, flags=flags)
        if nb:
            ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    out = cp.attn_chunk_with_past(cache, q, k, v, n_valid=nv, mask=mask,
                                  window=0 if explicit else cfg.window, scale=cfg.scale,
                                  workspace=ws, flags=flags)
    torch.cuda.synchronize()
    return out, mask


def _oracle(cfg, t, rows=None):
    return O.attn(_np(t["q"]), _np(t["k"]), _np(t["v"]), _np(t["kc"]), _np(t["vc"]),
                  _np(t["seen"]), _np(t["n_valid"]), None, cfg.ring, cfg.sink, cfg.window,
                  cfg.scale, rows=rows)


def _check(cfg, out, ref, rows=None):
    got = to_f64(out)
    m = real_rows_mask(cfg, got.shape)
    if rows is not None:
        keep = np.zeros(cfg.C, dtype=bool)
        keep[list(rows)] = True
        m &= keep[None, None, :]
    err = rowwise_rel_err(got, ref, m)
    assert np.isfinite(got[m]).all()
    # pad rows are written as zeros
    assert (got[~real_rows_mask(cfg, got.shape)] == 0).all()
    assert err <= TOL[cfg.dtype], err
    return err


SMALL = [
    dict(name="gqa4_d64", dtype=I.BF16, B=2, H=8, nKV=2, D=64, C=40, cap=200, seen=[0, 131],
         n_valid=[40, 23]),
    dict(name="gqa4_d128", dtype=I.BF16, B=2, H=8, nKV=2, D=128, C=70, cap=400, seen=[65, 300],
         n_valid=[70, 1]),
    dict(name="gqa8_d256_ring", dtype=I.BF16, B=1, H=8, nKV=1, D=256, C=48, cap=96, ring=1,
         window=96, seen=[250], n_valid=[47]),
    dict(name="gqa2_d128_window", dtype=I.BF16, B=2, H=4, nKV=2, D=128, C=64, cap=256, window=50,
         seen=[100, 30], n_valid=[64, 60]),
    dict(name="ring_sink", dtype=I.BF16, B=2, H=4, nKV=1, D=128, C=32, cap=80, ring=1, sink=4,
         window=70, seen=[3, 400], n_valid=[32, 29]),
    dict(name="gqa3_d64", dtype=I.BF16, B=1, H=6, nKV=2, D=64, C=33, cap=128, seen=[77],
         n_valid=[30]),
    dict(name="mha_d128", dtype=I.BF16, B=1, H=2, nKV=2, D=128, C=130, cap=300, seen=[100],
         n_valid=[129]),
    dict(name="fp32_d64", dtype=I.F32, B=2, H=4, nKV=1, D=64, C=16, cap=64, seen=[48, 20],
         n_valid=[11, 16]),
    dict(name="fp32_d128_ring", dtype=I.F32, B=1, H=4, nKV=2, D=128, C=24, cap=64, ring=1,
         window=64, seen=[150], n_valid=[20]),
    dict(name="odd_d40", dtype=I.BF16, B=1, H=4, nKV=1, D=40, C=12, cap=50, seen=[9],
         n_valid=[12]),
    # a global cache with sink rows and a window that starts far past them: the sink
    # tiles must still be visited (sequence 1: the chunk's own first rows are sinks)
    dict(name="global_sink_window", dtype=I.BF16, B=2, H=4, nKV=1, D=128, C=32, cap=600,
         sink=4, window=64, seen=[500, 2], n_valid=[32, 20]),
    dict(name="global_sink_window_d256", dtype=I.BF16, B=1, H=8, nKV=1, D=256, C=24, cap=400,
         sink=2, window=40, seen=[300], n_valid=[21]),
    # 64 < C * G <= 128 at D = 128: the 128-row medium configuration (in-kernel rule)
    dict(name="medium_c32_d128", dtype=I.BF16, B=2, H=8, nKV=2, D=128, C=32, cap=2000,
         seen=[1900, 37], n_valid=[32, 20]),
    dict(name="medium_g3_window", dtype=I.BF16, B=2, H=6, nKV=2, D=128, C=40, cap=600,
         window=300, seen=[550, 100], n_valid=[40, 39]),
    # C * G <= 64: the matrix-core kernel's small-rows configuration
    dict(name="small_c16_d128", dtype=I.BF16, B=2, H=8, nKV=2, D=128, C=16, cap=300,
         seen=[100, 250], n_valid=[16, 9]),
    dict(name="small_c8_d64_window", dtype=I.BF16, B=2, H=4, nKV=1, D=64, C=8, cap=200,
         window=40, seen=[150, 3], n_valid=[8, 5]),
    dict(name="decode_d256_ring", dtype=I.BF16, B=2, H=8, nKV=1, D=256, C=1, cap=96, ring=1,
         window=96, seen=[50, 400], n_valid=[1, 1]),
]
SMALL_ROWS = SMALL[-3:]


@pytest.mark.parametrize("kw", SMALL, ids=lambda c: c["name"])
@pytest.mark.parametrize("mode", ["inkernel", "explicit"])
@pytest.mark.parametrize("kernel", ["auto", "generic"])
@pytest.mark.parametrize("split", ["split", "nosplit"])
def test_attention_matches_oracle(cp, kw, mode, kernel, split):
    kw = dict(kw)
    kw.pop("name")
    cfg = I.small(**kw)
    t, cache, status = _setup(cp, cfg)
    flags = (cp.ATTN_FORCE_GENERIC if kernel == "generic" else 0) | (
        cp.ATTN_NO_SPLIT if split == "nosplit" else 0)
    out, _ = _run(cp, cfg, t, cache, explicit=(mode == "explicit"), flags=flags)
    ref = _oracle(cfg, t)
    _check(cfg, out, ref)
    assert int(status.item()) == 0


@pytest.mark.parametrize("kw", SMALL[:6] + SMALL[10:12] + SMALL_ROWS, ids=lambda c: c["name"])
@pytest.mark.parametrize("kernel", [0, 2])
def test_explicit_mask_equals_inkernel_bitwise(cp, kw, kernel):
    """On the same key partition with the mask evaluated on every tile (no split,
    CP_ATTN_FULL_TILES), the explicit mask built from the rule and the in-kernel rule give
    identical outputs: the additive values are identical and masked terms are exact zeros."""
    kw = dict(kw)
    kw.pop("name")
    cfg = I.small(**kw)
    t, cache, _ = _setup(cp, cfg)
    flags = cp.ATTN_NO_SPLIT | cp.ATTN_FULL_TILES | kernel
    a, _ = _run(cp, cfg, t, cache, explicit=True, flags=flags)
    b, _ = _run(cp, cfg, t, cache, explicit=False, flags=flags)
    # compare values (+0 and -0 count as equal)
    assert torch.equal(a.float(), b.float())


@pytest.mark.parametrize("kw", SMALL, ids=lambda c: c["name"])
@pytest.mark.parametrize("split", ["split", "nosplit"])
def test_select_out_equals_select_row(cp, kw, split):
    """The selection written by the attention (its epilogue, or the split merge) is
    bit-identical to cp_select_row(out, n_valid, -1), including a sequence without
    real rows (zeros)."""
    kw = dict(kw)
    kw.pop("name")
    if kw["B"] > 1:
        kw["n_valid"] = [0] + list(kw["n_valid"][1:])
    cfg = I.small(**kw)
    t, cache, _ = _setup(cp, cfg)
    q, k, v = dev(t["q"]), dev(t["k"]), dev(t["v"])
    nv = dev(t["n_valid"])
    flags = cp.ATTN_NO_SPLIT if split == "nosplit" else cp.ATTN_SPLITS(3)
    nb = cp.attn_workspace_bytes(cache, q, k, v, window=cfg.window, flags=flags)
    ws = torch.empty(max(nb, 1), dtype=torch.uint8, device="cuda")
    sel = torch.full((cfg.B, cfg.H, cfg.D), 7.0, dtype=q.dtype, device="cuda")
    out = cp.attn_chunk_with_past(cache, q, k, v, n_valid=nv, window=cfg.window,
                                  scale=cfg.scale, workspace=ws, flags=flags, select_out=sel)
    ref = cp.select_row(out, nv, -1)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(sel), bits(ref))
    # n_valid NULL selects row C - 1
    sel2 = torch.zeros_like(sel)
    out2 = cp.attn_chunk_with_past(cache, q, k, v, window=cfg.window, scale=cfg.scale,
                                   workspace=ws, flags=flags, select_out=sel2)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(sel2), bits(out2[:, :, cfg.C - 1]))


@pytest.mark.parametrize("kw", SMALL[:5] + SMALL_ROWS, ids=lambda c: c["name"])
def test_run_twice_is_deterministic(cp, kw):
    kw = dict(kw)
    kw.pop("name")
    cfg = I.small(**kw)
    t, cache, _ = _setup(cp, cfg)
    a, _ = _run(cp, cfg, t, cache)
    b, _ = _run(cp, cfg, t, cache)
    np.testing.assert_array_equal(bits(a), bits(b))


def test_padded_equals_unpadded_on_real_rows(cp):
    """[cactus] "Fix": a padded chunk gives the real rows an unpadded chunk gives."""
    cfg = I.small(dtype=I.BF16, B=1, H=8, nKV=2, D=128, C=64, cap=400, seen=[300],
                  n_valid=[37])
    t, cache, _ = _setup(cp, cfg)
    full, _ = _run(cp, cfg, t, cache, flags=cp.ATTN_NO_SPLIT)
    q, k, v = (dev(t[n][:, :, :37].contiguous()) for n in ("q", "k", "v"))
    part = cp.attn_chunk_with_past(cache, q, k, v, n_valid=None, scale=cfg.scale,
                                   flags=cp.ATTN_NO_SPLIT)
    torch.cuda.synchronize()
    ref = _oracle(cfg, t)[:, :, :37]
    e1 = rowwise_rel_err(to_f64(part), ref)
    e2 = rowwise_rel_err(to_f64(full)[:, :, :37], ref)
    assert e1 <= TOL[I.BF16] and e2 <= TOL[I.BF16]
    d = rowwise_rel_err(to_f64(part), to_f64(full)[:, :, :37])
    assert d <= TOL[I.BF16]


def test_chunk_equals_sequential_decode_steps(cp):
    """[TICO] decode contract: C one-token steps, each appending its K/V, give the chunk's
    real rows (within tolerance), and leave a byte-identical cache."""
    cfg = I.small(dtype=I.BF16, B=1, H=4, nKV=1, D=128, C=24, cap=80, ring=1, window=80,
                  seen=[150], n_valid=[21])
    t, cache, _ = _setup(cp, cfg)
    q, k, v, nv = dev(t["q"]), dev(t["k"]), dev(t["v"]), dev(t["n_valid"])
    chunk = cp.attn_chunk_with_past(cache, q, k, v, n_valid=nv, window=cfg.window,
                                    scale=cfg.scale)
    cp.kv_append(cache, k, v, nv)
    torch.cuda.synchronize()
    k_chunk, v_chunk = bits(cache.k), bits(cache.v)
    # same start state, token by token
    t2, cache2, _ = _setup(cp, cfg)
    steps = []
    one = torch.ones(1, dtype=torch.int32, device="cuda")
    for i in range(21):
        sl = slice(i, i + 1)
        qi, ki, vi = (dev(t2[n][:, :, sl].contiguous()) for n in ("q", "k", "v"))
        steps.append(cp.attn_chunk_with_past(cache2, qi, ki, vi, n_valid=one, window=cfg.window,
                                             scale=cfg.scale))
        cp.kv_append(cache2, ki, vi, one)
    torch.cuda.synchronize()
    seq = torch.cat(steps, dim=2)
    d = rowwise_rel_err(to_f64(seq), to_f64(chunk)[:, :, :21])
    assert d <= TOL[I.BF16]
    ref = _oracle(cfg, t)[:, :, :21]
    assert rowwise_rel_err(to_f64(seq), ref) <= TOL[I.BF16]
    assert cache2.seen.item() == cache.seen.item() == 171
    np.testing.assert_array_equal(bits(cache2.k), k_chunk)
    np.testing.assert_array_equal(bits(cache2.v), v_chunk)


def test_mask_too_narrow_is_flagged_and_zeroed(cp):
    cfg = I.small(dtype=I.BF16, B=1, H=4, nKV=1, D=128, C=16, cap=64, seen=[40], n_valid=[16])
    t, cache, status = _setup(cp, cfg)
    mask = torch.zeros((1, 4, 16, 40), dtype=torch.float32, device="cuda")  # needs 56 columns
    out = cp.attn_chunk_with_past(cache, dev(t["q"]), dev(t["k"]), dev(t["v"]),
                                  n_valid=dev(t["n_valid"]), mask=mask, scale=cfg.scale)
    torch.cuda.synchronize()
    assert int(status.item()) & cp.DEV_MASK_LD
    assert (out.float() == 0).all()


def test_empty_chunk_and_no_real_rows(cp):
    cfg = I.small(dtype=I.BF16, B=2, H=4, nKV=1, D=128, C=16, cap=64, seen=[10, 20],
                  n_valid=[0, 0])
    t, cache, _ = _setup(cp, cfg)
    out, _ = _run(cp, cfg, t, cache)
    assert (out.float() == 0).all()
    z = torch.empty((2, 4, 0, 128), dtype=torch.bfloat16, device="cuda")
    zk = torch.empty((2, 1, 0, 128), dtype=torch.bfloat16, device="cuda")
    cp.attn_chunk_with_past(cache, z, zk, zk, scale=cfg.scale)
    torch.cuda.synchronize()


# ------------------------------------------------------ the named workloads

@pytest.mark.parametrize("name", ["c1", "c2", "c3"])
@pytest.mark.parametrize("mode", ["inkernel", "explicit"])
def test_workload_attention_full(cp, name, mode):
    cfg = I.config(name)
    t, cache, status = _setup(cp, cfg)
    out, _ = _run(cp, cfg, t, cache, explicit=(mode == "explicit"))
    _check(cfg, out, _oracle(cfg, t))
    assert int(status.item()) == 0


def test_workload_c4_full(cp):
    cfg = I.config("c4")
    t, cache, status = _setup(cp, cfg)
    out, _ = _run(cp, cfg, t, cache)
    _check(cfg, out, _oracle(cfg, t))
    assert int(status.item()) == 0


# Chunk rows of the long-context workload checked one by one against the oracle: every
# 8th row, and both sides of every 64-row boundary (a D = 128 query tile holds the 4 heads
# of a KV head times 64 chunk rows), of the 32-row accumulator groups at 31/32, and the
# first and last rows.
C5_ROWS = sorted(set(range(0, 512, 8)) | {1, 31, 32, 255, 256, 510, 511}
                 | {64 * t - 1 for t in range(1, 9)} | {64 * t for t in range(8)})


@pytest.mark.parametrize("layer", [0, 3, 5])
def test_workload_c5_path_rows(cp, layer):
    """Long context (B = 4, 32768 past, C = 512, H32/KV8 D128): one layer's whole step
    in the launch sequence the benchmark times (RoPE of Q and K, attention, append; for
    the global layer RoPE with the early append and the attention advancing seen).  Every
    sequence and head on C5_ROWS against the oracle; the selection is the last row; the
    cache ends byte-identical to the oracle's append on its live slots."""
    from chunked_prefill_attention_rope_amd import path
    cfg = I.config("c5", layer)
    t, cache, status = _setup(cp, cfg, nan_dead=(layer == 5))
    d = {n: dev(t[n]) for n in ("q", "k", "v", "cos", "sin", "n_valid")}
    bufs = path.make_buffers(cache, d["q"], d["k"], d["v"], window=cfg.window)
    out, sel = path.chunk_step(cache, d["q"], d["k"], d["v"], d["cos"], d["sin"], d["n_valid"],
                               bufs, window=cfg.window)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    qr = O.rope(_np(t["q"]), _np(t["cos"]), _np(t["sin"]))
    kr = O.rope(_np(t["k"]), _np(t["cos"]), _np(t["sin"]))
    np.testing.assert_array_equal(bits(bufs.k_rot), kr.view(np.uint8).reshape(bits(bufs.k_rot).shape))
    ref = O.attn(qr, kr, _np(t["v"]), _np(t["kc"]), _np(t["vc"]), _np(t["seen"]),
                 _np(t["n_valid"]), None, cfg.ring, cfg.sink, cfg.window, cfg.scale,
                 rows=C5_ROWS)
    got = to_f64(out)
    m = np.zeros(got.shape[:3], dtype=bool)
    m[:, :, C5_ROWS] = True
    assert m.sum() == cfg.B * cfg.H * len(C5_ROWS)
    err = rowwise_rel_err(got, ref, m)
    assert err <= TOL[I.BF16], err
    np.testing.assert_array_equal(bits(sel), bits(out[:, :, cfg.C - 1]))
    ko, vo, so, live = O.kv_append(_np(t["kc"]), _np(t["vc"]), _np(t["seen"]), kr, _np(t["v"]),
                                   _np(t["n_valid"]), cfg.ring, cfg.sink)
    assert cache.seen.cpu().tolist() == so.tolist()
    kg, vg = cache.k.cpu(), cache.v.cpu()
    for b in range(cfg.B):
        sl = torch.from_numpy(np.nonzero(live[b])[0])
        assert torch.equal(kg[b][:, sl], I.from_np(ko[b])[:, sl])
        assert torch.equal(vg[b][:, sl], I.from_np(vo[b])[:, sl])


MERGE = [
    dict(name="decode_d128_long", dtype=I.BF16, B=2, H=8, nKV=2, D=128, C=1, cap=4096,
         seen=[3000, 1500], n_valid=[1, 1]),
    dict(name="c4_d64_long", dtype=I.BF16, B=1, H=8, nKV=2, D=64, C=4, cap=3000, seen=[2900],
         n_valid=[3]),
    dict(name="decode_d256_window", dtype=I.BF16, B=1, H=8, nKV=1, D=256, C=1, cap=2048,
         window=1500, seen=[2000], n_valid=[1]),
    dict(name="decode_d128_global_sink", dtype=I.BF16, B=1, H=8, nKV=2, D=128, C=1, cap=3000,
         sink=4, window=1000, seen=[2900], n_valid=[1]),
]


@pytest.mark.parametrize("kw", MERGE, ids=lambda c: c["name"])
@pytest.mark.parametrize("mode", ["inkernel", "explicit"])
@pytest.mark.parametrize("split", ["auto", "four", "none"])
def test_decode_split_merge(cp, kw, mode, split):
    """Decode-sized chunks over a long past: repeated calls on one workspace give the same
    bits, match the oracle, and the selection is the merged row.  Four forced splits (or
    none) leave each split 24+ tiles, which selects the deep-ring small-rows configuration
    for the in-kernel rule; the planner's own choice does not."""
    kw = dict(kw)
    kw.pop("name")
    cfg = I.small(**kw)
    t, cache, status = _setup(cp, cfg)
    q, k, v = dev(t["q"]), dev(t["k"]), dev(t["v"])
    nv = dev(t["n_valid"])
    mask = None
    if mode == "explicit":
        mask = cp.build_mask(cache, nv, cfg.H, cfg.C, cfg.mask_ld(), window=cfg.window)
    window = 0 if mask is not None else cfg.window
    flags = {"auto": 0, "four": cp.ATTN_SPLITS(4), "none": cp.ATTN_NO_SPLIT}[split]
    nb = cp.attn_workspace_bytes(cache, q, k, v, mask=mask, window=window, flags=flags)
    assert (nb > 0) == (split != "none")
    ws = torch.empty(max(nb, 1), dtype=torch.uint8, device="cuda")
    sel = torch.zeros((cfg.B, cfg.H, cfg.D), dtype=q.dtype, device="cuda")
    outs = []
    for _ in range(3):
        outs.append(cp.attn_chunk_with_past(cache, q, k, v, n_valid=nv, mask=mask, window=window,
                                            scale=cfg.scale, workspace=ws, select_out=sel,
                                            flags=flags))
    torch.cuda.synchronize()
    ref = _oracle(cfg, t)
    _check(cfg, outs[0], ref)
    for o in outs[1:]:
        assert np.array_equal(bits(o), bits(outs[0]))
    assert np.array_equal(bits(sel), bits(cp.select_row(outs[0], nv, -1)))
    assert int(status.item()) == 0


@pytest.mark.parametrize("shape", [
    # (H, nKV, D, C, seen, n_valid): the matrix-core query tile holds 128 or 256 rows;
    # G = 3 or 5 leaves spare rows at its end, and C is not a multiple of the tile's
    # chunk rows, so the last query tile is ragged
    (6, 2, 64, 45, [300, 77], [45, 31]),
    (5, 1, 256, 40, [260, 129], [33, 40]),
    (6, 2, 128, 100, [350, 12], [100, 57]),
])
@pytest.mark.parametrize("splits", [5, 19])
@pytest.mark.parametrize("mode", ["inkernel", "explicit"])
def test_merge_fragment_rows(cp, shape, splits, mode):
    """The matrix-core kernel's split partials, in accumulator fragment order, on query
    tiles with spare rows (G does not divide the tile's rows) and a ragged last tile, two
    sequences, two KV heads: every real row matches the oracle, pad rows are zeros, the
    selection is the merged row, and a repeat is bit-identical."""
    H, nKV, D, C, seen, n_valid = shape
    cfg = I.small(dtype=I.BF16, B=2, H=H, nKV=nKV, D=D, C=C, cap=512, seen=seen,
                  n_valid=n_valid)
    t, cache, status = _setup(cp, cfg)
    q, k, v = dev(t["q"]), dev(t["k"]), dev(t["v"])
    nv = dev(t["n_valid"])
    mask = None
    if mode == "explicit":
        mask = cp.build_mask(cache, nv, cfg.H, cfg.C, cfg.mask_ld(), window=cfg.window)
    flags = cp.ATTN_SPLITS(splits)
    nb = cp.attn_workspace_bytes(cache, q, k, v, mask=mask, flags=flags)
    assert nb > 0
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    sel = torch.zeros((cfg.B, cfg.H, cfg.D), dtype=q.dtype, device="cuda")
    outs = [cp.attn_chunk_with_past(cache, q, k, v, n_valid=nv, mask=mask, scale=cfg.scale,
                                    workspace=ws, select_out=sel, flags=flags)
            for _ in range(2)]
    torch.cuda.synchronize()
    _check(cfg, outs[0], _oracle(cfg, t))
    assert np.array_equal(bits(outs[1]), bits(outs[0]))
    assert np.array_equal(bits(sel), bits(cp.select_row(outs[0], nv, -1)))
    assert int(status.item()) == 0


@pytest.mark.parametrize("shape", [
    # (B, H, nKV, D, C, cap, seen, n_valid, splits).  The blocks of a split call go to the
    # XCDs by (split, sequence, KV head) group; the group count decides the order:
    # 8 query tiles per group (1024 rows of 128) with 3 and 9 groups: each query tile's
    # splits on one XCD, the merge dealing whole tiles;
    (2, 8, 1, 256, 128, 800, [650, 200], [128, 77], 3),
    (3, 8, 1, 256, 128, 800, [600, 10, 333], [100, 128, 1], 3),
    # 2 query tiles, 14 groups: padded to 16; 5 groups: in order (fewer than 8)
    (1, 4, 1, 256, 64, 1024, [800], [52], 14),
    (1, 4, 1, 256, 64, 1024, [800], [52], 5),
    # 3 KV heads x 3 splits = 9 groups of 1 tile at D = 128
    (1, 12, 3, 128, 50, 900, [870], [49], 3),
])
@pytest.mark.parametrize("mode", ["inkernel", "explicit"])
def test_split_placement(cp, shape, mode):
    """Key splits in each block order of the XCD placement (tile-minor with whole tiles
    per XCD in the merge, padded groups, groups in order): every real row matches the
    oracle, pad rows are zeros, a repeat is bit-identical, and the selection is the
    merged row."""
    B, H, nKV, D, C, cap, seen, n_valid, splits = shape
    cfg = I.small(dtype=I.BF16, B=B, H=H, nKV=nKV, D=D, C=C, cap=cap, seen=seen,
                  n_valid=n_valid)
    t, cache, status = _setup(cp, cfg)
    q, k, v = dev(t["q"]), dev(t["k"]), dev(t["v"])
    nv = dev(t["n_valid"])
    mask = None
    if mode == "explicit":
        mask = cp.build_mask(cache, nv, cfg.H, cfg.C, cfg.mask_ld(), window=cfg.window)
    flags = cp.ATTN_SPLITS(splits)
    nb = cp.attn_workspace_bytes(cache, q, k, v, mask=mask, flags=flags)
    assert nb > 0
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    sel = torch.zeros((cfg.B, cfg.H, cfg.D), dtype=q.dtype, device="cuda")
    outs = [cp.attn_chunk_with_past(cache, q, k, v, n_valid=nv, mask=mask, scale=cfg.scale,
                                    workspace=ws, select_out=sel, flags=flags)
            for _ in range(2)]
    torch.cuda.synchronize()
    _check(cfg, outs[0], _oracle(cfg, t))
    assert np.array_equal(bits(outs[1]), bits(outs[0]))
    assert np.array_equal(bits(sel), bits(cp.select_row(outs[0], nv, -1)))
    assert int(status.item()) == 0


@pytest.mark.parametrize("splits", [16, 17, 33, 64])
@pytest.mark.parametrize("mode", ["inkernel", "explicit"])
def test_merge_rounds(cp, splits, mode):
    """Forced key splits on either side of the merge's per-round widths (16 splits per
    round up to 16, 32 above; 33 and 64 take two rounds): the merged output matches the
    oracle, repeats bit for bit, and the selection is the merged row.  Some splits of 64
    get no tile at all (their partials carry an empty maximum)."""
    cfg = I.small(dtype=I.BF16, B=2, H=8, nKV=2, D=128, C=16, cap=2304, seen=[2100, 700],
                  n_valid=[16, 9])
    t, cache, status = _setup(cp, cfg)
    q, k, v = dev(t["q"]), dev(t["k"]), dev(t["v"])
    nv = dev(t["n_valid"])
    mask = None
    if mode == "explicit":
        mask = cp.build_mask(cache, nv, cfg.H, cfg.C, cfg.mask_ld(), window=cfg.window)
    flags = cp.ATTN_SPLITS(splits)
    nb = cp.attn_workspace_bytes(cache, q, k, v, mask=mask, flags=flags)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    sel = torch.zeros((cfg.B, cfg.H, cfg.D), dtype=q.dtype, device="cuda")
    outs = [cp.attn_chunk_with_past(cache, q, k, v, n_valid=nv, mask=mask, scale=cfg.scale,
                                    workspace=ws, select_out=sel, flags=flags)
            for _ in range(2)]
    torch.cuda.synchronize()
    _check(cfg, outs[0], _oracle(cfg, t))
    assert np.array_equal(bits(outs[1]), bits(outs[0]))
    assert np.array_equal(bits(sel), bits(cp.select_row(outs[0], nv, -1)))
    assert int(status.item()) == 0


@pytest.mark.parametrize("max_seen", [1, 400, 800, 5000])
@pytest.mark.parametrize("mode", ["inkernel", "explicit"])
def test_max_seen_bound(cp, max_seen, mode):
    """The Gemma-270M-like chunk (seen 800, capacity 1024, 32-key tiles) with a host bound
    on seen: exact (800), loose (5000: the capacity rules), or below the real seen (1,
    400 -- it only sizes the splits, the device still divides each sequence's own live
    tiles).  Within tolerance of the oracle in every case, and bit for bit the call that
    forces the split count the bound implies: ceil(tiles / 2) for
    tiles = ceil((min(max_seen, 1024) + 64) / 32)."""
    cfg = I.config("c2")
    t, cache, status = _setup(cp, cfg)
    q, k, v = dev(t["q"]), dev(t["k"]), dev(t["v"])
    nv = dev(t["n_valid"])
    mask = None
    if mode == "explicit":
        mask = cp.build_mask(cache, nv, cfg.H, cfg.C, cfg.mask_ld())
    tiles = (min(max_seen, cfg.cap) + cfg.C + 31) // 32
    splits = (tiles + 1) // 2
    outs = []
    for flags, ms in ((0, max_seen), (cp.ATTN_SPLITS(splits), 0)):
        nb = cp.attn_workspace_bytes(cache, q, k, v, mask=mask, flags=flags, max_seen=ms)
        ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
        outs.append(cp.attn_chunk_with_past(cache, q, k, v, n_valid=nv, mask=mask,
                                            scale=cfg.scale, workspace=ws, flags=flags,
                                            max_seen=ms))
    torch.cuda.synchronize()
    _check(cfg, outs[0], _oracle(cfg, t))
    assert np.array_equal(bits(outs[0]), bits(outs[1]))
    assert int(status.item()) == 0
