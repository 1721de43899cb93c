"""A prompt tail run token by token (one-token steps: RoPE, attention with C = 1, append
of one row) equals the same tail as one padded chunk: outputs of the real rows within the
bf16 tolerance of the oracle and of each other, the caches' live regions and seen
identical byte for byte ([cactus] "Fix": the padded tail must leave the cache as the
unpadded one; [TICO] "Runtime behavior": the one-token decode contract)."""
import numpy as np
import pytest
import torch

from chunked_prefill_attention_rope_amd import inputs as I
from oracle import oracle as O
from tests.gpu_helpers import TOL, bits, dev, rowwise_rel_err, to_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mods():
    from chunked_prefill_attention_rope_amd import cp, path
    return cp, path


CASES = [
    # sliding ring (the [cactus] setting: window = ring capacity), padded append with
    # snapshot/rollback, tails on both sides of the policy threshold
    dict(name="ring", B=1, H=8, nKV=1, D=256, C=16, cap=64, ring=1, window=64, seen=[150]),
    dict(name="ring_fresh", B=1, H=4, nKV=1, D=128, C=16, cap=48, ring=1, window=48, seen=[40]),
    dict(name="global", B=2, H=8, nKV=2, D=128, C=16, cap=200, seen=[57, 120]),
]


def _cache(cp, cfg, t):
    return cp.KVCache(dev(t["kc"]), dev(t["vc"]), dev(t["seen"]), ring=cfg.ring, sink=cfg.sink)


@pytest.mark.parametrize("case", CASES, ids=lambda c: c["name"])
@pytest.mark.parametrize("n_tail", [1, 5, 9, 15])
def test_scalar_tail_equals_padded_chunk(mods, case, n_tail):
    cp, path = mods
    kw = dict(case)
    kw.pop("name")
    cfg = I.small(dtype=I.BF16, n_valid=[n_tail] * kw["B"], **kw)
    t = I.make_layer(cfg)
    static = bool(cfg.ring)  # a ring's padded append is protected by snapshot/rollback
    q, k, v, cos, sin = (dev(t[n]) for n in ("q", "k", "v", "cos", "sin"))
    nv = dev(t["n_valid"])

    padded = _cache(cp, cfg, t)
    bufs = path.make_buffers(padded, q, k, v, window=cfg.window, static_append=static)
    out_p, sel_p = path.chunk_step(padded, q, k, v, cos, sin, nv, bufs, window=cfg.window,
                                   static_append=static)

    scalar = _cache(cp, cfg, t)
    steps = path.token_steps(scalar, q, k, v, cos, sin, n_tail, window=cfg.window)
    outs, sel_s = path.scalar_tail(scalar, steps, window=cfg.window)
    torch.cuda.synchronize()

    # the step rotates Q and K first
    qr = O.rope(I.np_view(t["q"]), I.np_view(t["cos"]), I.np_view(t["sin"]))
    kr = O.rope(I.np_view(t["k"]), I.np_view(t["cos"]), I.np_view(t["sin"]))
    ref = O.attn(qr, kr, I.np_view(t["v"]), I.np_view(t["kc"]), I.np_view(t["vc"]),
                 I.np_view(t["seen"]), I.np_view(t["n_valid"]), None, cfg.ring, cfg.sink,
                 cfg.window, cfg.scale)
    got_p = to_f64(out_p)[:, :, :n_tail]
    got_s = np.concatenate([to_f64(o) for o in outs], axis=2)
    real = np.ones(got_s.shape[:3], dtype=bool)
    assert rowwise_rel_err(got_p, ref[:, :, :n_tail], real) <= TOL[I.BF16]
    assert rowwise_rel_err(got_s, ref[:, :, :n_tail], real) <= TOL[I.BF16]
    assert rowwise_rel_err(got_s, got_p, real) <= TOL[I.BF16]
    # the selection is the last real row in both modes
    np.testing.assert_array_equal(bits(sel_p), bits(out_p[:, :, n_tail - 1]))
    np.testing.assert_array_equal(bits(sel_s), bits(outs[-1][:, :, 0]))

    # identical caches: seen and every live slot, byte for byte (and equal to the oracle's)
    assert padded.seen.cpu().tolist() == scalar.seen.cpu().tolist()
    ko, vo, so, live = O.kv_append(I.np_view(t["kc"]), I.np_view(t["vc"]), I.np_view(t["seen"]),
                                   kr, I.np_view(t["v"]), I.np_view(t["n_valid"]), cfg.ring,
                                   cfg.sink)
    assert scalar.seen.cpu().tolist() == so.tolist()
    for c in (padded, scalar):
        kg, vg = bits(c.k), bits(c.v)
        for b in range(cfg.B):
            sl = np.nonzero(live[b])[0]
            np.testing.assert_array_equal(kg[b][:, sl], ko.view(np.uint8).reshape(kg.shape)[b][:, sl])
            np.testing.assert_array_equal(vg[b][:, sl], vo.view(np.uint8).reshape(vg.shape)[b][:, sl])


def test_prefill_tail_follows_the_policy(mods, monkeypatch):
    cp, path = mods
    cfg = I.small(dtype=I.BF16, B=1, H=4, nKV=1, D=128, C=16, cap=48, ring=1, window=48,
                  seen=[30], n_valid=[3])
    t = I.make_layer(cfg)
    q, k, v, cos, sin = (dev(t[n]) for n in ("q", "k", "v", "cos", "sin"))
    nv = dev(t["n_valid"])
    monkeypatch.delenv(path.KILL_SWITCH, raising=False)

    def run(n_tail, **kw):
        c = _cache(cp, cfg, t)
        bufs = path.make_buffers(c, q, k, v, window=cfg.window, static_append=True)
        steps = path.token_steps(c, q, k, v, cos, sin, n_tail, window=cfg.window)
        n = torch.full_like(nv, n_tail)
        mode, _, _ = path.prefill_tail(c, q, k, v, cos, sin, n, n_tail, bufs, steps,
                                       window=cfg.window, static_append=True, **kw)
        return mode

    # the default is the MI355X breakeven: one token stays a decode step, two are padded
    assert run(1) == "scalar"
    assert run(3) == "padded"
    # the pages' threshold keeps tails below 9 token by token
    assert run(3, pad_from=path.PAGES_PAD_FROM) == "scalar"
    monkeypatch.setenv(path.KILL_SWITCH, "1")
    assert run(3) == "scalar"
    torch.cuda.synchronize()


@pytest.mark.parametrize("seen", [1023, 896])
def test_c3_tail_scalar_equals_padded(mods, seen):
    """The sliding-window workload at its own size ([cactus] "Problem" and the review
    hardening: the padded tail must give the scalar tail's outputs): a 512-window ring that
    has absorbed `seen` positions (1023: the ring holds 511..1022; 896: the page's
    1023-token prompt after its seventh full chunk), a 127-token tail run as one padded
    128-row chunk with snapshot/rollback and as 127 one-token steps.  Real-row outputs
    match the oracle and each other, the selections are the last real row, and both
    caches end byte-identical to the oracle's exact append of the 127 rows."""
    cp, path = mods
    cfg = I.config("c3")
    cfg.seen = [seen]
    t = I.make_layer(cfg)
    n_tail = cfg.n_valid[0]
    assert (cfg.C, cfg.cap, n_tail) == (128, 512, 127)
    q, k, v, cos, sin = (dev(t[n]) for n in ("q", "k", "v", "cos", "sin"))
    nv = dev(t["n_valid"])

    padded = _cache(cp, cfg, t)
    bufs = path.make_buffers(padded, q, k, v, window=cfg.window, static_append=True)
    out_p, sel_p = path.chunk_step(padded, q, k, v, cos, sin, nv, bufs, window=cfg.window,
                                   static_append=True)
    scalar = _cache(cp, cfg, t)
    steps = path.token_steps(scalar, q, k, v, cos, sin, n_tail, window=cfg.window)
    outs, sel_s = path.scalar_tail(scalar, steps, window=cfg.window)
    torch.cuda.synchronize()

    qr = O.rope(I.np_view(t["q"]), I.np_view(t["cos"]), I.np_view(t["sin"]))
    kr = O.rope(I.np_view(t["k"]), I.np_view(t["cos"]), I.np_view(t["sin"]))
    ref = O.attn(qr, kr, I.np_view(t["v"]), I.np_view(t["kc"]), I.np_view(t["vc"]),
                 I.np_view(t["seen"]), I.np_view(t["n_valid"]), None, cfg.ring, cfg.sink,
                 cfg.window, cfg.scale)[:, :, :n_tail]
    got_p = to_f64(out_p)
    got_s = np.concatenate([to_f64(o) for o in outs], axis=2)
    assert rowwise_rel_err(got_p[:, :, :n_tail], ref) <= TOL[I.BF16]
    assert rowwise_rel_err(got_s, ref) <= TOL[I.BF16]
    assert rowwise_rel_err(got_s, got_p[:, :, :n_tail]) <= TOL[I.BF16]
    assert (got_p[:, :, n_tail:] == 0).all()  # the pad row is written as zeros
    np.testing.assert_array_equal(bits(sel_p), bits(out_p[:, :, n_tail - 1]))
    np.testing.assert_array_equal(bits(sel_s), bits(outs[-1][:, :, 0]))

    ko, vo, so, live = O.kv_append(I.np_view(t["kc"]), I.np_view(t["vc"]), I.np_view(t["seen"]),
                                   kr, I.np_view(t["v"]), I.np_view(t["n_valid"]), cfg.ring,
                                   cfg.sink)
    assert so.tolist() == [seen + n_tail]
    assert live.sum() == 512  # a full window: every slot is live
    for c in (padded, scalar):
        assert c.seen.cpu().tolist() == so.tolist()
        np.testing.assert_array_equal(bits(c.k), ko.view(np.uint8).reshape(bits(c.k).shape))
        np.testing.assert_array_equal(bits(c.v), vo.view(np.uint8).reshape(bits(c.v).shape))
