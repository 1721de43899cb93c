"""Bit-exact GPU parity of the index and copy work: RoPE, KV append, padded-append
snapshot/rollback, mask materialisation and row selection (HIP path through the
C ABI vs the CPU oracle)."""
import numpy as np
import pytest
import torch

from chunked_prefill_attention_rope_amd import inputs as I
from oracle import oracle as O
from tests.gpu_helpers import bits, dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def cp():
    from chunked_prefill_attention_rope_amd import cp as mod
    return mod


def _np(t):
    return I.np_view(t)


# ---------------------------------------------------------------------- RoPE

@pytest.mark.parametrize("dtype", [I.F32, I.BF16])
@pytest.mark.parametrize("D", [8, 64, 128, 256, 12])
def test_rope_bit_exact(cp, dtype, D):
    cfg = I.small(dtype=dtype, B=3, H=5, D=D, C=19, seen=[0, 700, 33280])
    t = I.make_layer(cfg)
    assert t["cos"].shape[0] == 3  # per-sequence tables
    for x in (t["q"], t["k"]):
        y = cp.rope_chunk(dev(x), dev(t["cos"]), dev(t["sin"]))
        ref = O.rope(_np(x), _np(t["cos"]), _np(t["sin"]))
        np.testing.assert_array_equal(bits(y), ref.view(np.uint8))


def test_rope_in_place_and_shared_table(cp):
    cfg = I.small(dtype=I.BF16, B=2, H=4, D=128, C=64, seen=[800, 800])
    t = I.make_layer(cfg)
    assert t["cos"].shape[0] == 1
    x = dev(t["q"])
    cp.rope_chunk(x, dev(t["cos"]), dev(t["sin"]), out=x)
    ref = O.rope(_np(t["q"]), _np(t["cos"]), _np(t["sin"]))
    np.testing.assert_array_equal(bits(x), ref.view(np.uint8))


@pytest.mark.parametrize("dtype", [I.F32, I.BF16])
@pytest.mark.parametrize("D", [64, 256, 12])
def test_rope_qk_one_launch_matches_oracle(cp, dtype, D):
    """cp_rope_qk_chunk rotates Q and K of a chunk in one launch, bit-exact like two
    cp_rope_chunk calls (D = 12 takes the unvectorised path)."""
    cfg = I.small(dtype=dtype, B=2, H=6, nKV=2, D=D, C=23, seen=[5, 1000])
    t = I.make_layer(cfg)
    qo, ko = cp.rope_qk_chunk(dev(t["q"]), dev(t["k"]), dev(t["cos"]), dev(t["sin"]))
    for got, x in ((qo, t["q"]), (ko, t["k"])):
        ref = O.rope(_np(x), _np(t["cos"]), _np(t["sin"]))
        np.testing.assert_array_equal(bits(got), ref.view(np.uint8))
    # in place, shared table
    cfg = I.small(dtype=dtype, B=2, H=4, nKV=1, D=D, C=9, seen=[70, 70])
    t = I.make_layer(cfg)
    q, k = dev(t["q"]), dev(t["k"])
    cp.rope_qk_chunk(q, k, dev(t["cos"]), dev(t["sin"]), q_out=q, k_out=k)
    np.testing.assert_array_equal(bits(q), O.rope(_np(t["q"]), _np(t["cos"]),
                                                  _np(t["sin"])).view(np.uint8))
    np.testing.assert_array_equal(bits(k), O.rope(_np(t["k"]), _np(t["cos"]),
                                                  _np(t["sin"])).view(np.uint8))


def test_rope_empty(cp):
    x = torch.empty((0, 4, 8, 64), dtype=torch.bfloat16, device="cuda")
    cos = torch.zeros((1, 8, 64), device="cuda")
    cp.rope_chunk(x, cos, cos)
    torch.cuda.synchronize()


# ------------------------------------------------------------------ append

APPEND_CASES = [
    dict(ring=0, cap=96, sink=0, seen=[40, 0, 80], C=16, n=[16, 5, 0]),
    dict(ring=1, cap=32, sink=0, seen=[3, 30, 100], C=8, n=[8, 8, 3]),
    dict(ring=1, cap=32, sink=4, seen=[2, 31, 77], C=8, n=[8, 6, 1]),
    dict(ring=1, cap=16, sink=2, seen=[5, 40, 9], C=24, n=[24, 20, 17]),  # append longer than ring
]


@pytest.mark.parametrize("case", APPEND_CASES)
@pytest.mark.parametrize("dtype", [I.F32, I.BF16])
@pytest.mark.parametrize("D", [64, 128, 6])
def test_append_bit_exact(cp, case, dtype, D):
    cfg = I.small(dtype=dtype, B=3, H=2, nKV=2, D=D, C=case["C"], cap=case["cap"],
                  ring=case["ring"], sink=case["sink"], seen=case["seen"], n_valid=case["n"])
    t = I.make_layer(cfg)
    kc, vc = dev(t["kc"]), dev(t["vc"])
    seen = dev(t["seen"])
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    cache = cp.KVCache(kc, vc, seen, ring=cfg.ring, sink=cfg.sink, status=status)
    cp.kv_append(cache, dev(t["k"]), dev(t["v"]), dev(t["n_valid"]))
    ko, vo, so, live = O.kv_append(_np(t["kc"]), _np(t["vc"]), _np(t["seen"]), _np(t["k"]),
                                   _np(t["v"]), _np(t["n_valid"]), cfg.ring, cfg.sink)
    assert seen.cpu().tolist() == so.tolist()
    assert int(status.item()) == 0
    kg, vg = bits(kc), bits(vc)
    es = 2 if dtype == I.BF16 else 4
    for b in range(cfg.B):
        sl = np.nonzero(live[b])[0]
        np.testing.assert_array_equal(kg[b][:, sl], ko.view(np.uint8).reshape(kg.shape)[b][:, sl])
        np.testing.assert_array_equal(vg[b][:, sl], vo.view(np.uint8).reshape(vg.shape)[b][:, sl])
    assert kg.shape[-1] == D * es


@pytest.mark.parametrize("ring", [0, 1])
def test_append_large_takes_the_multi_block_path(cp, ring):
    """Appends of more than 1024 16-byte chunks per tensor copy over the whole GPU and
    update seen in a second launch; tiny ones do both in one workgroup (both paths are
    also taken by the smaller cases above)."""
    seen = [300, 0, 1200, 77] if ring else [300, 0, 500, 77]
    cfg = I.small(dtype=I.BF16, B=4, H=8, nKV=8, D=128, C=128, cap=1024 if ring else 700,
                  ring=ring, sink=4 if ring else 0, seen=seen, n_valid=[128, 100, 1, 64])
    t = I.make_layer(cfg)
    kc, vc, sd = dev(t["kc"]), dev(t["vc"]), dev(t["seen"])
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    cache = cp.KVCache(kc, vc, sd, ring=cfg.ring, sink=cfg.sink, status=status)
    cp.kv_append(cache, dev(t["k"]), dev(t["v"]), dev(t["n_valid"]))
    ko, vo, so, live = O.kv_append(_np(t["kc"]), _np(t["vc"]), _np(t["seen"]), _np(t["k"]),
                                   _np(t["v"]), _np(t["n_valid"]), cfg.ring, cfg.sink)
    assert sd.cpu().tolist() == so.tolist()
    assert int(status.item()) == 0
    kg, vg = bits(kc), bits(vc)
    for b in range(cfg.B):
        sl = np.nonzero(live[b])[0]
        np.testing.assert_array_equal(kg[b][:, sl], ko.view(np.uint8).reshape(kg.shape)[b][:, sl])
        np.testing.assert_array_equal(vg[b][:, sl], vo.view(np.uint8).reshape(vg.shape)[b][:, sl])


def test_append_all_rows_and_overflow_flag(cp):
    cfg = I.small(dtype=I.BF16, B=2, H=2, nKV=1, D=64, C=8, cap=20, seen=[10, 15],
                  n_valid=[8, 8])
    t = I.make_layer(cfg)
    kc, vc, seen = dev(t["kc"]), dev(t["vc"]), dev(t["seen"])
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    cache = cp.KVCache(kc, vc, seen, status=status)
    before = bits(kc)
    cp.kv_append(cache, dev(t["k"]), dev(t["v"]), None)  # all C rows
    assert seen.cpu().tolist() == [18, 15]  # sequence 1 would overflow: skipped
    assert int(status.item()) & cp.DEV_OVERFLOW
    after = bits(kc)
    np.testing.assert_array_equal(after[1], before[1])
    k_ref = _np(t["k"]).view(np.uint8)
    np.testing.assert_array_equal(after[0][:, 10:18], k_ref.reshape(2, 1, 8, -1)[0])


def test_append_nvalid_out_of_range_is_clamped_and_flagged(cp):
    cfg = I.small(dtype=I.F32, B=1, H=1, nKV=1, D=8, C=4, cap=16, seen=[2], n_valid=[4])
    t = I.make_layer(cfg)
    seen = dev(t["seen"])
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    cache = cp.KVCache(dev(t["kc"]), dev(t["vc"]), seen, status=status)
    cp.kv_append(cache, dev(t["k"]), dev(t["v"]), torch.tensor([9], dtype=torch.int32,
                                                                device="cuda"))
    assert seen.item() == 6 and int(status.item()) & cp.DEV_NVALID


# -------------------------------------------------------- snapshot / rollback

ROLLBACK_CASES = [  # ([cactus] review: no eviction, overshoot, eviction, sink)
    dict(name="no_evict", cap=64, sink=0, seen=[3], C=16, nv=[11]),
    dict(name="overshoot", cap=64, sink=0, seen=[50], C=16, nv=[11]),
    dict(name="evict", cap=64, sink=0, seen=[200], C=16, nv=[3]),
    dict(name="sink", cap=64, sink=4, seen=[200], C=16, nv=[9]),
    dict(name="sink_overshoot", cap=64, sink=4, seen=[55], C=16, nv=[2]),
    dict(name="all_real", cap=64, sink=0, seen=[90], C=16, nv=[16]),
    dict(name="all_pad", cap=64, sink=0, seen=[90], C=16, nv=[0]),
    dict(name="c3_primary", cap=512, sink=0, seen=[1023], C=128, nv=[127]),
    dict(name="c3_cactus", cap=512, sink=0, seen=[896], C=128, nv=[127]),
    dict(name="batch", cap=64, sink=2, seen=[10, 57, 300, 64], C=16, nv=[16, 5, 1, 9]),
    # 4 x 2 x 512 rows of 128 bytes (bf16) = 32768 chunks: the multi-block rollback
    dict(name="large", cap=1024, sink=0, seen=[5000, 1100, 700, 3000], C=512,
         nv=[300, 1, 512, 17]),
]


@pytest.mark.parametrize("case", ROLLBACK_CASES, ids=lambda c: c["name"])
@pytest.mark.parametrize("dtype", [I.F32, I.BF16])
def test_padded_append_rollback_equals_exact_append(cp, case, dtype):
    """[cactus] "Fix": snapshot -> padded append of C rows -> rollback leaves the live
    region byte-identical to an exact append of the n_valid real rows."""
    B = len(case["seen"])
    cfg = I.small(dtype=dtype, B=B, H=2, nKV=2, D=64, C=case["C"], cap=case["cap"], ring=1,
                  sink=case["sink"], seen=case["seen"], n_valid=case["nv"])
    t = I.make_layer(cfg)
    kc, vc, seen = dev(t["kc"]), dev(t["vc"]), dev(t["seen"])
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    cache = cp.KVCache(kc, vc, seen, ring=1, sink=cfg.sink, status=status)
    nv = dev(t["n_valid"])
    snap = cp.kv_snapshot_padded_append(cache, cfg.C, nv)
    assert snap.armed
    cp.kv_append(cache, dev(t["k"]), dev(t["v"]), None)
    assert seen.cpu().tolist() == [s + cfg.C for s in cfg.seen]
    cp.kv_rollback_padded_append(cache, snap)
    assert not snap.armed
    ko, vo, so, live = O.kv_append(_np(t["kc"]), _np(t["vc"]), _np(t["seen"]), _np(t["k"]),
                                   _np(t["v"]), _np(t["n_valid"]), 1, cfg.sink)
    assert seen.cpu().tolist() == so.tolist()
    assert int(status.item()) == 0
    kg, vg = bits(kc), bits(vc)
    kr = ko.view(np.uint8).reshape(kg.shape)
    vr = vo.view(np.uint8).reshape(vg.shape)
    for b in range(B):
        sl = np.nonzero(live[b])[0]
        np.testing.assert_array_equal(kg[b][:, sl], kr[b][:, sl])
        np.testing.assert_array_equal(vg[b][:, sl], vr[b][:, sl])
    # a second rollback of the same snapshot is refused on the host
    with pytest.raises(cp.CpError) as e:
        cp.kv_rollback_padded_append(cache, snap)
    assert e.value.code == cp.ERR_STATE


def test_snapshot_window_guard_touches_nothing(cp):
    cfg = I.small(dtype=I.BF16, B=1, H=1, nKV=1, D=64, C=16, cap=20, ring=1, sink=4,
                  seen=[30], n_valid=[3])
    t = I.make_layer(cfg)
    kc, seen = dev(t["kc"]), dev(t["seen"])
    cache = cp.KVCache(kc, dev(t["vc"]), seen, ring=1, sink=4)
    buf = torch.zeros(cp.snapshot_bytes(cache, 16), dtype=torch.uint8, device="cuda")
    with pytest.raises(cp.CpError) as e:
        cp.kv_snapshot_padded_append(cache, 16, dev(t["n_valid"]), cp.Snapshot(buf))
    assert e.value.code == cp.ERR_WINDOW
    assert seen.item() == 30 and (buf == 0).all()


def test_rollback_without_padded_append_is_flagged(cp):
    cfg = I.small(dtype=I.BF16, B=1, H=1, nKV=1, D=64, C=8, cap=64, ring=1, seen=[70],
                  n_valid=[3])
    t = I.make_layer(cfg)
    kc, seen = dev(t["kc"]), dev(t["seen"])
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    cache = cp.KVCache(kc, dev(t["vc"]), seen, ring=1, status=status)
    before = bits(kc)
    snap = cp.kv_snapshot_padded_append(cache, 8, dev(t["n_valid"]))
    cp.kv_rollback_padded_append(cache, snap)  # no append happened in between
    assert int(status.item()) & cp.DEV_ROLLBACK
    assert seen.item() == 70
    np.testing.assert_array_equal(bits(kc), before)


def test_global_cache_padded_append_rollback(cp):
    cfg = I.small(dtype=I.BF16, B=2, H=2, nKV=1, D=128, C=16, cap=128, seen=[7, 100],
                  n_valid=[5, 16])
    t = I.make_layer(cfg)
    kc, vc, seen = dev(t["kc"]), dev(t["vc"]), dev(t["seen"])
    cache = cp.KVCache(kc, vc, seen)
    snap = cp.kv_snapshot_padded_append(cache, 16, dev(t["n_valid"]))
    cp.kv_append(cache, dev(t["k"]), dev(t["v"]), None)
    cp.kv_rollback_padded_append(cache, snap)
    ko, vo, so, live = O.kv_append(_np(t["kc"]), _np(t["vc"]), _np(t["seen"]), _np(t["k"]),
                                   _np(t["v"]), _np(t["n_valid"]), 0, 0)
    assert seen.cpu().tolist() == so.tolist()
    kg = bits(kc)
    kr = ko.view(np.uint8).reshape(kg.shape)
    for b in range(2):
        sl = np.nonzero(live[b])[0]
        np.testing.assert_array_equal(kg[b][:, sl], kr[b][:, sl])


# -------------------------------------------------------------- mask, select

@pytest.mark.parametrize("kw", [
    dict(ring=0, cap=96, seen=[40, 0], window=0),
    dict(ring=0, cap=96, seen=[40, 70], window=9),
    dict(ring=1, cap=32, seen=[7, 90], window=32),
    dict(ring=1, cap=32, sink=3, seen=[2, 90], window=20),
    dict(ring=0, cap=96, sink=3, seen=[70, 2], window=9),
])
def test_build_mask_bit_exact(cp, kw):
    cfg = I.small(dtype=I.BF16, B=2, H=3, nKV=1, D=64, C=16, n_valid=[16, 9], **kw)
    t = I.make_layer(cfg)
    cache = cp.KVCache(dev(t["kc"]), dev(t["vc"]), dev(t["seen"]), ring=cfg.ring, sink=cfg.sink)
    ld = cfg.mask_ld() + 3
    m = cp.build_mask(cache, dev(t["n_valid"]), cfg.H, cfg.C, ld, window=cfg.window)
    ref = O.build_mask(cfg.seen, cfg.n_valid, cfg.H, cfg.C, ld, cfg.cap, cfg.ring, cfg.sink,
                       cfg.window)
    np.testing.assert_array_equal(bits(m), ref.view(np.uint8))


@pytest.mark.parametrize("dtype", [I.F32, I.BF16])
@pytest.mark.parametrize("off", [-1, 0, 2])
def test_select_row_bit_exact(cp, dtype, off):
    """cp_select_row against the oracle's orc_select_row: the selected rows are the same
    values bit for bit (both widen exactly to fp64 for the comparison, signs of zero
    included), rows outside [0, C) give zeros."""
    g = torch.Generator("cpu").manual_seed(31 + off)
    x = torch.randn((5, 4, 16, 256), generator=g).to(
        torch.float32 if dtype == I.F32 else torch.bfloat16)
    x[1, :, 0, :8] = -0.0
    idx = torch.tensor([16, 1, 0, 15, 20], dtype=torch.int32)
    y = cp.select_row(dev(x), dev(idx), off)
    torch.cuda.synchronize()
    got = y.cpu().double().numpy()
    ref = O.select_row(x.double().numpy(), idx.numpy(), off)
    np.testing.assert_array_equal(got, ref)
    np.testing.assert_array_equal(np.signbit(got), np.signbit(ref))
