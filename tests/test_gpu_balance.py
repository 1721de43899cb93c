"""Balanced key splits (CP_ATTN_BALANCE): a device-side plan cuts each sequence's keys by
its own past length.  Outputs within tolerance of the oracle on batches of unequal
lengths (the Llama-8B-like batch among them), in both mask modes, with selection and the
seen advance of an early-appended chunk; bit-identical repeats; and on equal lengths
(nothing cut) bit-identical to the unbalanced call."""
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


def _oracle(cfg, t):
    v = I.np_view
    return O.attn(v(t["q"]), v(t["k"]), v(t["v"]), v(t["kc"]), v(t["vc"]), v(t["seen"]),
                  v(t["n_valid"]), None, cfg.ring, cfg.sink, cfg.window, cfg.scale)


def _call(cp, cfg, t, cache, flags, explicit=False, sel=None):
    q, k, v, nv = dev(t["q"]), dev(t["k"]), dev(t["v"]), dev(t["n_valid"])
    mask = cp.build_mask(cache, nv, cfg.H, cfg.C, cfg.mask_ld(), window=cfg.window) \
        if explicit else None
    window = 0 if explicit else cfg.window
    nb = cp.attn_workspace_bytes(cache, q, k, v, mask=mask, window=window, flags=flags)
    ws = torch.empty(max(nb, 1), dtype=torch.uint8, device="cuda")
    out = cp.attn_chunk_with_past(cache, q, k, v, n_valid=nv, mask=mask, window=window,
                                  scale=cfg.scale, workspace=ws, flags=flags, select_out=sel)
    return out, nb


CASES = [
    # unequal pasts, D = 128 (256-row query tiles), one long sequence among short ones
    dict(name="d128_skew", B=6, H=8, nKV=2, D=128, C=96, cap=3200,
         seen=[3000, 5, 0, 700, 64, 2500], n_valid=[96, 96, 40, 1, 96, 77]),
    # D = 64 and D = 256 tiles, ragged chunks, G = 3 (spare rows in every query tile)
    dict(name="d64_g3", B=5, H=6, nKV=2, D=64, C=70, cap=2100, seen=[2000, 10, 900, 0, 1500],
         n_valid=[70, 70, 33, 70, 5]),
    dict(name="d256", B=4, H=8, nKV=2, D=256, C=48, cap=1600, seen=[1500, 3, 400, 1100],
         n_valid=[48, 20, 48, 47]),
    # sliding window over a ring: the window bounds each sequence's keys
    dict(name="ring_window", B=4, H=8, nKV=2, D=128, C=64, cap=1024, ring=1, window=1024,
         seen=[5000, 200, 1023, 40], n_valid=[64, 64, 30, 64]),
    # sequences with no real row and an empty past
    dict(name="empty_rows", B=4, H=4, nKV=1, D=128, C=80, cap=2000, seen=[1900, 0, 50, 1200],
         n_valid=[0, 80, 80, 0]),
]


@pytest.mark.parametrize("kw", CASES, ids=lambda c: c["name"])
@pytest.mark.parametrize("mode", ["inkernel", "explicit"])
def test_balanced_matches_oracle(cp, kw, mode):
    kw = dict(kw)
    kw.pop("name")
    cfg = I.small(dtype=I.BF16, **kw)
    t = I.make_layer(cfg)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    cache = cp.KVCache(dev(t["kc"]), dev(t["vc"]), dev(t["seen"]), ring=cfg.ring, sink=cfg.sink,
                       status=status)
    sel = torch.zeros((cfg.B, cfg.H, cfg.D), dtype=torch.bfloat16, device="cuda")
    outs = []
    for _ in range(2):
        out, nb = _call(cp, cfg, t, cache, cp.ATTN_BALANCE, explicit=(mode == "explicit"),
                        sel=sel)
        outs.append(out)
    torch.cuda.synchronize()
    assert nb > 0
    got = to_f64(outs[0])
    m = real_rows_mask(cfg, got.shape)
    assert rowwise_rel_err(got, _oracle(cfg, t), m) <= TOL[I.BF16]
    assert (got[~m] == 0).all()  # pad rows are zeros
    np.testing.assert_array_equal(bits(outs[1]), bits(outs[0]))
    np.testing.assert_array_equal(bits(sel), bits(cp.select_row(outs[0], dev(t["n_valid"]), -1)))
    assert int(status.item()) == 0


def test_balanced_workload_c4(cp):
    """The Llama-8B-like batch (16 pasts uniform in [0, 4095]), every output row."""
    cfg = I.config("c4")
    t = I.make_layer(cfg)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    cache = cp.KVCache(dev(t["kc"]), dev(t["vc"]), dev(t["seen"]), status=status)
    out, _ = _call(cp, cfg, t, cache, cp.ATTN_BALANCE)
    torch.cuda.synchronize()
    got = to_f64(out)
    assert rowwise_rel_err(got, _oracle(cfg, t), real_rows_mask(cfg, got.shape)) <= TOL[I.BF16]
    assert int(status.item()) == 0


def test_balanced_equal_lengths_cuts_nothing(cp):
    """Equal past lengths and as many items as the GPU holds workgroups (4 sequences x 8 KV
    heads x 8 query tiles): the plan keeps every sequence whole, so the output is the
    unbalanced call's, bit for bit.  (A smaller batch is cut to fill the GPU, as the
    unbalanced call's uniform split would.)"""
    cfg = I.small(dtype=I.BF16, B=4, H=32, nKV=8, D=128, C=512, cap=2400, seen=[1800] * 4,
                  n_valid=[512] * 4)
    t = I.make_layer(cfg)
    cache = cp.KVCache(dev(t["kc"]), dev(t["vc"]), dev(t["seen"]))
    a, _ = _call(cp, cfg, t, cache, cp.ATTN_BALANCE | cp.ATTN_NO_SPLIT)
    b, _ = _call(cp, cfg, t, cache, cp.ATTN_NO_SPLIT)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(a), bits(b))


def test_balanced_advances_seen(cp):
    """With the chunk appended early, the merge (always launched with a plan) advances seen
    by n_valid, as the unbalanced call does."""
    cfg = I.small(dtype=I.BF16, B=5, H=8, nKV=2, D=128, C=64, cap=3000,
                  seen=[2800, 3, 1000, 0, 2000], n_valid=[64, 10, 64, 64, 1])
    t = I.make_layer(cfg)
    cache = cp.KVCache(dev(t["kc"]), dev(t["vc"]), dev(t["seen"]))
    out, _ = _call(cp, cfg, t, cache, cp.ATTN_BALANCE | cp.ATTN_ADVANCE_SEEN)
    torch.cuda.synchronize()
    assert cache.seen.cpu().tolist() == [s + n for s, n in zip(cfg.seen, cfg.n_valid)]
    got = to_f64(out)
    assert rowwise_rel_err(got, _oracle(cfg, t), real_rows_mask(cfg, got.shape)) <= TOL[I.BF16]


def test_balance_flag_ignored_where_it_does_not_apply(cp):
    """Small-rows chunks (C * G <= 64), fp32 and the vector-ALU kernel run unbalanced."""
    for kw in (dict(dtype=I.BF16, B=6, H=8, nKV=2, D=128, C=4, cap=3000,
                    seen=[2900, 5, 100, 1500, 0, 2200], n_valid=[4, 4, 1, 4, 4, 2]),
               dict(dtype=I.F32, B=3, H=4, nKV=1, D=64, C=16, cap=900, seen=[800, 2, 300],
                    n_valid=[16, 9, 16])):
        cfg = I.small(**kw)
        t = I.make_layer(cfg)
        cache = cp.KVCache(dev(t["kc"]), dev(t["vc"]), dev(t["seen"]))
        out, _ = _call(cp, cfg, t, cache, cp.ATTN_BALANCE)
        torch.cuda.synchronize()
        got = to_f64(out)
        assert rowwise_rel_err(got, _oracle(cfg, t), real_rows_mask(cfg, got.shape)) <= \
            TOL[cfg.dtype]


def test_balanced_path_step_c4():
    """The Llama-8B-like layer's whole step as the benchmark runs it: the layer driver's
    flags for its skewed batch (balanced splits), RoPE with the early append, the
    balanced attention, and the merge advancing seen.  Every output row against the
    oracle, the selection is the last row, the cache ends byte-identical to the oracle's
    append on its live slots."""
    from chunked_prefill_attention_rope_amd import cp, path
    cfg = I.config("c4")
    flags = path.attn_flags_for(cfg.seen)
    assert flags == cp.ATTN_BALANCE
    t = I.make_layer(cfg)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    cache = cp.KVCache(dev(t["kc"]), dev(t["vc"]), dev(t["seen"]), status=status)
    d = {n: dev(t[n]) for n in ("q", "k", "v", "cos", "sin", "n_valid")}
    bufs = path.make_buffers(cache, d["q"], d["k"], d["v"], flags=flags)
    out, sel = path.chunk_step(cache, d["q"], d["k"], d["v"], d["cos"], d["sin"], d["n_valid"],
                               bufs, flags=flags, max_seen=max(cfg.seen))
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    v = I.np_view
    qr = O.rope(v(t["q"]), v(t["cos"]), v(t["sin"]))
    kr = O.rope(v(t["k"]), v(t["cos"]), v(t["sin"]))
    ref = O.attn(qr, kr, v(t["v"]), v(t["kc"]), v(t["vc"]), v(t["seen"]), v(t["n_valid"]), None,
                 cfg.ring, cfg.sink, cfg.window, cfg.scale)
    got = to_f64(out)
    assert rowwise_rel_err(got, ref, real_rows_mask(cfg, got.shape)) <= TOL[I.BF16]
    np.testing.assert_array_equal(bits(sel), bits(out[:, :, cfg.C - 1]))
    ko, vo, so, live = O.kv_append(v(t["kc"]), v(t["vc"]), v(t["seen"]), kr, v(t["v"]),
                                   v(t["n_valid"]), cfg.ring, cfg.sink)
    assert cache.seen.cpu().tolist() == so.tolist()
    kg, vg = bits(cache.k), bits(cache.v)
    for b in range(cfg.B):
        sl = np.nonzero(live[b])[0]
        np.testing.assert_array_equal(kg[b][:, sl], ko.view(np.uint8).reshape(kg.shape)[b][:, sl])
        np.testing.assert_array_equal(vg[b][:, sl], vo.view(np.uint8).reshape(vg.shape)[b][:, sl])


def test_balanced_many_sequences(cp):
    """More sequences than the plan kernel has threads (300 over 256): its per-sequence
    loops and prefix sums take several elements per thread.  Pasts from 0 to 2990, every
    output row against the oracle; then at the plan's limit (1024 sequences) the call is
    still balanced, and above it (1025) the flag is ignored."""
    seen = [(i * 37) % 2991 for i in range(300)]
    nvs = [64 if i % 7 else 9 for i in range(300)]
    cfg = I.small(dtype=I.BF16, B=300, H=4, nKV=1, D=128, C=64, cap=3000, seen=seen,
                  n_valid=nvs, seed=21)
    t = I.make_layer(cfg)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    cache = cp.KVCache(dev(t["kc"]), dev(t["vc"]), dev(t["seen"]), status=status)
    out, nb = _call(cp, cfg, t, cache, cp.ATTN_BALANCE)
    torch.cuda.synchronize()
    assert nb > 0
    got = to_f64(out)
    m = real_rows_mask(cfg, got.shape)
    assert rowwise_rel_err(got, _oracle(cfg, t), m) <= TOL[I.BF16]
    assert (got[~m] == 0).all()
    assert int(status.item()) == 0
    for B, planned in ((1024, True), (1025, False)):
        big = I.small(dtype=I.BF16, B=B, H=4, nKV=1, D=128, C=64, cap=64, seen=[0] * B,
                      n_valid=[64] * B, seed=22)
        tb = I.make_layer(big, nan_dead=False)
        cb = cp.KVCache(dev(tb["kc"]), dev(tb["vc"]), dev(tb["seen"]))
        q, k, v = dev(tb["q"]), dev(tb["k"]), dev(tb["v"])
        assert (cp.attn_workspace_bytes(cb, q, k, v, flags=cp.ATTN_BALANCE) > 0) == planned
