"""Pins of the CPU oracle against what the pages and the mathematics fix.

CPU only.  Each test names the property it pins; together they are chosen so
that a dropped term, a wrong sign or index, or a transposed operand in the
oracle fails at least one of them.
"""
import json
import os

import numpy as np
import pytest
import torch

from chunked_prefill_attention_rope_amd import inputs as I
from oracle import oracle as O
from tests import bruteforce as BF

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _layer(cfg, nan_dead=True):
    t = I.make_layer(cfg, nan_dead=nan_dead)
    return {k: I.np_view(v) for k, v in t.items()}


# ----------------------------------------------------------------- RoPE pins

@pytest.mark.parametrize("dtype", [I.F32, I.BF16])
def test_rope_matches_complex_rotation(dtype):
    """Half-split RoPE == multiplying z = x[j] + i x[j+D/2] by exp(i*theta)."""
    cfg = I.small(dtype=dtype, B=2, H=3, D=32, C=9, seen=[5, 77])
    t = _layer(cfg)
    y = O.rope(t["q"], t["cos"], t["sin"])
    x = BF.bf16_bits_to_f64(t["q"])
    h2 = cfg.D // 2
    z = x[..., :h2] + 1j * x[..., h2:]
    cos = t["cos"].astype(np.float64)[:, None, :, :h2]
    sin = t["sin"].astype(np.float64)[:, None, :, :h2]
    w = z * (cos + 1j * sin)
    ref = np.concatenate([w.real, w.imag], axis=-1).astype(np.float32)
    got = BF.bf16_bits_to_f64(y).astype(np.float32)
    if dtype == I.BF16:
        ref = BF.bf16_bits_to_f64(I.np_view(torch.from_numpy(ref).to(torch.bfloat16)))
        np.testing.assert_array_equal(got, ref.astype(np.float32))
    else:
        # products are exact in fp64, so both evaluate the same rounded value
        np.testing.assert_array_equal(got, ref)


def test_rope_position_zero_is_identity():
    cfg = I.small(dtype=I.F32, B=1, H=2, D=16, C=4, seen=[0])
    t = _layer(cfg)
    y = O.rope(t["q"], t["cos"], t["sin"])
    np.testing.assert_array_equal(y[:, :, 0], t["q"][:, :, 0])
    assert not np.array_equal(y[:, :, 1], t["q"][:, :, 1])


def test_rope_preserves_pair_norm_and_relative_position():
    """|rope(x)| per pair is unchanged; <rope(q,m), rope(k,n)> depends on m-n only."""
    D = 16
    cfg = I.small(dtype=I.F32, B=1, H=1, D=D, C=1, seen=[0], base=100.0)
    rng = np.random.default_rng(3)
    q = rng.standard_normal((1, 1, 1, D)).astype(np.float32)
    k = rng.standard_normal((1, 1, 1, D)).astype(np.float32)

    def at(x, pos):
        c = I.small(dtype=I.F32, B=1, H=1, D=D, C=1, seen=[pos], base=100.0)
        cos, sin = I.rope_tables(c)
        return O.rope(x, cos.numpy(), sin.numpy()).astype(np.float64)

    h2 = D // 2
    for pos in (0, 3, 1000):
        y = at(q, pos)
        n0 = q[..., :h2].astype(np.float64) ** 2 + q[..., h2:].astype(np.float64) ** 2
        n1 = y[..., :h2] ** 2 + y[..., h2:] ** 2
        np.testing.assert_allclose(n1, n0, rtol=2e-6)
    d1 = float((at(q, 10) * at(k, 7)).sum())
    d2 = float((at(q, 503) * at(k, 500)).sum())
    d3 = float((at(q, 7) * at(k, 10)).sum())
    assert abs(d1 - d2) < 1e-4 * (abs(d1) + 1)
    assert abs(d1 - d3) > 1e-3  # the property is not vacuous
    del cfg


# ---------------------------------------------------------------- cache pins

@pytest.mark.parametrize("cap,sink", [(5, 0), (6, 2), (8, 1), (4, 0), (7, 3)])
def test_ring_live_set_and_slots_match_cursor_model(cap, sink):
    for seen in range(0, 30):
        live = O.live_positions(seen, cap, 1, sink)
        assert list(live) == BF.live_positions(seen, cap, 1, sink)
        where = BF.slot_of(seen, cap, 1, sink)
        for p in live:
            assert O.slot(p, cap, 1, sink) == where[p]


def _tiny_cache(rng, B, nKV, cap, D, dtype):
    kc = rng.standard_normal((B, nKV, cap, D)).astype(np.float32)
    vc = rng.standard_normal((B, nKV, cap, D)).astype(np.float32)
    if dtype == I.BF16:
        kc = I.np_view(torch.from_numpy(kc).to(torch.bfloat16))
        vc = I.np_view(torch.from_numpy(vc).to(torch.bfloat16))
    return kc, vc


def _bf_append(kc, vc, seen, kn, vn, n, ring, sink):
    """Brute-force append with the cursor model (independent of the oracle)."""
    kc, vc = kc.copy(), vc.copy()
    B, nKV, cap, D = kc.shape
    for b in range(B):
        s0, nb = int(seen[b]), int(n[b])
        for r in range(nb):
            p = s0 + r
            where = BF.slot_of(p + 1, cap, ring, sink)
            kc[b, :, where[p]] = kn[b, :, r]
            vc[b, :, where[p]] = vn[b, :, r]
    return kc, vc


@pytest.mark.parametrize("ring,cap,sink", [(0, 12, 0), (1, 5, 0), (1, 6, 2), (1, 8, 1)])
def test_append_matches_bruteforce_exhaustive(ring, cap, sink):
    rng = np.random.default_rng(11)
    D, nKV = 4, 2
    for C in range(0, 7):
        for seen in range(0, 14):
            if not ring and seen + C > cap:
                continue
            for nv in range(0, C + 1):
                kc, vc = _tiny_cache(rng, 1, nKV, cap, D, I.F32)
                kn, vn = _tiny_cache(rng, 1, nKV, max(C, 1), D, I.F32)
                kn, vn = kn[:, :, :C], vn[:, :, :C]
                k1, v1, s1, live = O.kv_append(kc, vc, [seen], kn, vn, [nv], ring, sink)
                k2, v2 = _bf_append(kc, vc, [seen], kn, vn, [nv], ring, sink)
                assert s1[0] == seen + nv
                lp = BF.live_positions(seen + nv, cap, ring, sink)
                where = BF.slot_of(seen + nv, cap, ring, sink)
                slots = sorted(where[p] for p in lp)
                assert sorted(np.nonzero(live[0])[0].tolist()) == slots
                np.testing.assert_array_equal(k1[:, :, slots], k2[:, :, slots])
                np.testing.assert_array_equal(v1[:, :, slots], v2[:, :, slots])


def test_global_append_overflow_rejected():
    rng = np.random.default_rng(1)
    kc, vc = _tiny_cache(rng, 1, 1, 8, 4, I.F32)
    kn, vn = _tiny_cache(rng, 1, 1, 4, 4, I.F32)
    with pytest.raises(OverflowError):
        O.kv_append(kc, vc, [6], kn, vn, [3], 0, 0)
    O.kv_append(kc, vc, [6], kn, vn, [2], 0, 0)


def test_overevicted_matches_closed_form_and_guard():
    """FIFO diff == [max(sink, Te-R), max(sink, Tp-R)), all pre-existing rows."""
    for cap in range(2, 12):
        for sink in range(0, cap):
            R = cap - sink
            for C in range(0, 9):
                for nv in range(0, C + 1):
                    for seen in range(0, 25):
                        if cap <= C + sink:
                            with pytest.raises(ValueError):
                                O.padded_overevicted(seen, nv, C, cap, 1, sink)
                            continue
                        got = O.padded_overevicted(seen, nv, C, cap, 1, sink).tolist()
                        lo = max(sink, seen + nv - R)
                        hi = max(sink, seen + C - R)
                        assert got == list(range(lo, max(lo, hi))), (cap, sink, C, nv, seen)
                        assert len(got) <= C - nv
                        assert all(p < seen for p in got)
    assert O.padded_overevicted(100, 3, 8, 16, 0, 0).size == 0


def test_padded_append_plus_restore_equals_exact_append():
    """[cactus] "Fix": padded append + reinsertion of the over-evicted rows leaves the
    live region byte-identical to an exact append (no-evict, overshoot, evict, sink)."""
    rng = np.random.default_rng(5)
    cases = [  # (cap, sink, seen, C, nv): no eviction, overshoot, eviction, sink
        (16, 0, 3, 6, 4), (16, 0, 11, 6, 4), (16, 0, 40, 6, 2), (16, 3, 40, 6, 1),
        (12, 2, 9, 5, 5), (12, 0, 12, 5, 0),
    ]
    for cap, sink, seen, C, nv in cases:
        for dtype in (I.F32, I.BF16):
            kc, vc = _tiny_cache(rng, 1, 2, cap, 8, dtype)
            kn, vn = _tiny_cache(rng, 1, 2, C, 8, dtype)
            ke, ve, se, live_e = O.kv_append(kc, vc, [seen], kn, vn, [nv], 1, sink)
            kp, vp, sp, _ = O.kv_append(kc, vc, [seen], kn, vn, [C], 1, sink)
            assert sp[0] == seen + C
            for p in O.padded_overevicted(seen, nv, C, cap, 1, sink):
                s = O.slot(p, cap, 1, sink)
                kp[:, :, s] = kc[:, :, s]
                vp[:, :, s] = vc[:, :, s]
            sl = np.nonzero(live_e[0])[0]
            np.testing.assert_array_equal(kp[:, :, sl].view(np.uint8), ke[:, :, sl].view(np.uint8))
            np.testing.assert_array_equal(vp[:, :, sl].view(np.uint8), ve[:, :, sl].view(np.uint8))


# ------------------------------------------------------------ attention pins

def _attn_case(cfg, explicit=False, nan_dead=True):
    t = _layer(cfg, nan_dead=nan_dead)
    mask = None
    if explicit:
        mask = O.build_mask(t["seen"], t["n_valid"], cfg.H, cfg.C, cfg.mask_ld(), cfg.cap,
                            cfg.ring, cfg.sink, cfg.window)
    return t, mask


CASES = [
    dict(dtype=I.F32, B=2, H=4, nKV=2, D=16, C=6, cap=24, seen=[0, 9], n_valid=[6, 4]),
    dict(dtype=I.BF16, B=2, H=6, nKV=2, D=8, C=5, cap=20, seen=[3, 12], n_valid=[2, 5]),
    dict(dtype=I.F32, B=1, H=2, nKV=1, D=8, C=4, cap=8, ring=1, window=8, seen=[19], n_valid=[3]),
    dict(dtype=I.BF16, B=2, H=4, nKV=4, D=8, C=3, cap=9, ring=1, sink=2, window=7, seen=[4, 30],
         n_valid=[3, 1]),
    dict(dtype=I.F32, B=1, H=4, nKV=1, D=12, C=6, cap=30, window=5, seen=[11], n_valid=[6]),
]


@pytest.mark.parametrize("kw", CASES)
@pytest.mark.parametrize("explicit", [False, True])
def test_attn_matches_bruteforce(kw, explicit):
    cfg = I.small(**kw)
    t, mask = _attn_case(cfg, explicit)
    got = O.attn(t["q"], t["k"], t["v"], t["kc"], t["vc"], t["seen"], t["n_valid"], mask,
                 cfg.ring, cfg.sink, cfg.window, cfg.scale)
    ref = BF.attn(t["q"], t["k"], t["v"], t["kc"], t["vc"], t["seen"], t["n_valid"], cfg.ring,
                  cfg.sink, cfg.window, cfg.scale, mask=mask)
    assert np.isfinite(got).all()
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_attn_no_past_equals_torch_causal_sdpa():
    """past = 0, all rows real, no window: textbook causal attention (library routine)."""
    cfg = I.small(dtype=I.F32, B=2, H=6, nKV=3, D=16, C=11, cap=16, seen=[0, 0],
                  n_valid=[11, 11])
    t = _layer(cfg)
    got = O.attn(t["q"], t["k"], t["v"], t["kc"], t["vc"], t["seen"], t["n_valid"], None, 0, 0,
                 0, cfg.scale)
    q = torch.from_numpy(t["q"]).double()
    k = torch.from_numpy(t["k"]).double().repeat_interleave(cfg.G, dim=1)
    v = torch.from_numpy(t["v"]).double().repeat_interleave(cfg.G, dim=1)
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True,
                                                           scale=cfg.scale)
    np.testing.assert_allclose(got, ref.numpy(), rtol=1e-10, atol=1e-12)


def test_attn_single_key_returns_value():
    """First row of an empty-past chunk sees only itself: out = v exactly."""
    cfg = I.small(dtype=I.F32, B=1, H=2, nKV=1, D=8, C=3, cap=8, seen=[0], n_valid=[3])
    t = _layer(cfg)
    got = O.attn(t["q"], t["k"], t["v"], t["kc"], t["vc"], t["seen"], t["n_valid"], None, 0, 0,
                 0, cfg.scale)
    for h in range(2):
        np.testing.assert_array_equal(got[0, h, 0], t["v"][0, 0, 0].astype(np.float64))


@pytest.mark.parametrize("kw", CASES[:4])
def test_attn_probabilities_sum_to_one_and_respect_mask(kw):
    """With V = identity rows, outputs are the softmax probabilities themselves."""
    cfg = I.small(**kw)
    t = _layer(cfg)
    B, nKV, C = cfg.B, cfg.nKV, cfg.C
    nk = cfg.cap + C
    D = nk
    # one-hot V over (past slot | chunk row) so each output column is one key's weight
    vc = np.zeros((B, nKV, cfg.cap, D), dtype=np.float32)
    vn = np.zeros((B, nKV, C, D), dtype=np.float32)
    for s in range(cfg.cap):
        vc[:, :, s, s] = 1.0
    for j in range(C):
        vn[:, :, j, cfg.cap + j] = 1.0
    q = BF.bf16_bits_to_f64(t["q"])
    Dq = q.shape[-1]
    # q/k keep their own head dim; only V is widened, so run via the brute-force shape rules
    qf = q.astype(np.float32)
    kc = BF.bf16_bits_to_f64(t["kc"]).astype(np.float32)
    kn = BF.bf16_bits_to_f64(t["k"]).astype(np.float32)
    # attention needs a shared D; embed q/k into D columns with zeros beyond Dq
    def widen(a):
        out = np.zeros(a.shape[:-1] + (D,), dtype=np.float32)
        out[..., :Dq] = a
        return out
    kc_dead = np.isnan(kc).any(-1)
    kcw = widen(np.nan_to_num(kc))
    vcw = vc.copy()
    got = O.attn(widen(qf), widen(kn), vn, kcw, vcw, t["seen"], t["n_valid"], None, cfg.ring,
                 cfg.sink, cfg.window, cfg.scale)
    for b in range(B):
        nv = int(t["n_valid"][b])
        s = np.asarray(got[b, :, :nv]).sum(-1)
        np.testing.assert_allclose(s, 1.0, rtol=0, atol=1e-12)
        assert (got[b, :, :nv] >= 0).all()
        # dead slots and future / pad chunk keys carry exactly zero weight
        dead = np.nonzero(kc_dead[b, 0])[0]
        assert (got[b, :, :nv][..., dead] == 0).all()
        for i in range(nv):
            fut = [cfg.cap + j for j in range(C) if j > i or j >= nv]
            assert (got[b, :, i][..., fut] == 0).all()
            assert (got[b, :, i, cfg.cap + i] > 0).all()


def test_attn_constant_values_give_that_value():
    cfg = I.small(dtype=I.F32, B=1, H=4, nKV=2, D=8, C=5, cap=16, seen=[7], n_valid=[5])
    t = _layer(cfg)
    vrow = np.arange(8, dtype=np.float32) - 3.5
    vc = np.broadcast_to(vrow, t["vc"].shape).copy()
    vn = np.broadcast_to(vrow, t["v"].shape).copy()
    got = O.attn(t["q"], t["k"], vn, t["kc"], vc, t["seen"], t["n_valid"], None, 0, 0, 0,
                 cfg.scale)
    np.testing.assert_allclose(got[0], np.broadcast_to(vrow, got[0].shape), rtol=0, atol=1e-14)


def test_attn_gqa_head_mapping():
    """Perturbing KV head g changes exactly the query heads g*G .. g*G+G-1."""
    cfg = I.small(dtype=I.F32, B=1, H=6, nKV=3, D=8, C=4, cap=16, seen=[6], n_valid=[4])
    t = _layer(cfg)
    base = O.attn(t["q"], t["k"], t["v"], t["kc"], t["vc"], t["seen"], t["n_valid"])
    for g in range(3):
        kc = t["kc"].copy()
        kc[0, g, :6] += 1.0
        got = O.attn(t["q"], t["k"], t["v"], kc, t["vc"], t["seen"], t["n_valid"])
        changed = [h for h in range(6) if not np.array_equal(got[0, h], base[0, h])]
        assert changed == [g * 2, g * 2 + 1]


def test_attn_window_excludes_old_keys():
    """Keys outside the window do not influence the output; keys inside do."""
    cfg = I.small(dtype=I.F32, B=1, H=2, nKV=1, D=8, C=4, cap=32, window=6, seen=[20],
                  n_valid=[4])
    t = _layer(cfg)
    base = O.attn(t["q"], t["k"], t["v"], t["kc"], t["vc"], t["seen"], t["n_valid"], window=6)
    vc = t["vc"].copy()
    vc[0, 0, 14] += 10.0  # position 14: in window of query pos 20 (20-14=6 -> out), 19? no
    got = O.attn(t["q"], t["k"], t["v"], t["kc"], vc, t["seen"], t["n_valid"], window=6)
    np.testing.assert_array_equal(got, base)  # 20 - 14 = 6 is not < 6
    vc = t["vc"].copy()
    vc[0, 0, 15] += 10.0  # 20 - 15 = 5 < 6: row 0 sees it, row 1 (pos 21) does not
    got = O.attn(t["q"], t["k"], t["v"], t["kc"], vc, t["seen"], t["n_valid"], window=6)
    assert not np.array_equal(got[0, :, 0], base[0, :, 0])
    np.testing.assert_array_equal(got[0, :, 1:], base[0, :, 1:])


# ----------------------------------------------- invariants the pages fix

def _run_chunk(t, cfg, rows):
    """Oracle chunk call restricted to chunk rows [0, rows) (unpadded)."""
    return O.attn(t["q"][:, :, :rows], t["k"][:, :, :rows], t["v"][:, :, :rows], t["kc"],
                  t["vc"], t["seen"], np.minimum(t["n_valid"], rows), None, cfg.ring, cfg.sink,
                  cfg.window, cfg.scale)


@pytest.mark.parametrize("kw", [CASES[0], CASES[1], CASES[2], CASES[3], CASES[4]])
def test_chunk_equals_sequential_decode_steps(kw):
    """[TICO] decode contract: one token per step against the external cache, the
    runtime appending each step's K/V; a chunk call equals those steps (bit-exact)."""
    cfg = I.small(**kw)
    t = _layer(cfg)
    full = O.attn(t["q"], t["k"], t["v"], t["kc"], t["vc"], t["seen"], t["n_valid"], None,
                  cfg.ring, cfg.sink, cfg.window, cfg.scale)
    for b in range(cfg.B):
        kc, vc = t["kc"][b:b + 1].copy(), t["vc"][b:b + 1].copy()
        seen = t["seen"][b:b + 1].copy()
        nv = int(t["n_valid"][b])
        for i in range(nv):
            sl = slice(i, i + 1)
            step = O.attn(t["q"][b:b + 1, :, sl], t["k"][b:b + 1, :, sl], t["v"][b:b + 1, :, sl],
                          kc, vc, seen, [1], None, cfg.ring, cfg.sink, cfg.window, cfg.scale)
            np.testing.assert_array_equal(step[0, :, 0], full[b, :, i])
            kc, vc, seen, _ = O.kv_append(kc, vc, seen, t["k"][b:b + 1, :, sl],
                                          t["v"][b:b + 1, :, sl], [1], cfg.ring, cfg.sink)


@pytest.mark.parametrize("kw", CASES)
def test_padded_equals_unpadded_on_real_rows(kw):
    """[cactus] "Fix": running the remainder as one padded chunk gives the real rows
    an unpadded chunk gives (bit-exact in the oracle)."""
    cfg = I.small(**kw)
    t = _layer(cfg)
    full = O.attn(t["q"], t["k"], t["v"], t["kc"], t["vc"], t["seen"], t["n_valid"], None,
                  cfg.ring, cfg.sink, cfg.window, cfg.scale)
    for b in range(cfg.B):
        nv = int(t["n_valid"][b])
        sub = {k: (v[b:b + 1] if k in ("q", "k", "v", "kc", "vc", "seen", "n_valid") else v)
               for k, v in t.items()}
        part = _run_chunk(sub, cfg, nv)
        np.testing.assert_array_equal(part[0, :, :nv], full[b, :, :nv])
        assert (full[b, :, nv:] == 0).all()


@pytest.mark.parametrize("kw", CASES)
def test_explicit_mask_equals_inkernel_rule(kw):
    cfg = I.small(**kw)
    t, mask = _attn_case(cfg, explicit=True)
    a = O.attn(t["q"], t["k"], t["v"], t["kc"], t["vc"], t["seen"], t["n_valid"], mask,
               cfg.ring, cfg.sink, cfg.window, cfg.scale)
    b = O.attn(t["q"], t["k"], t["v"], t["kc"], t["vc"], t["seen"], t["n_valid"], None,
               cfg.ring, cfg.sink, cfg.window, cfg.scale)
    np.testing.assert_array_equal(a, b)


def test_mask_values_and_layout():
    """[SKaiNET] mask [1, nHeads, C, past+C], 0 attends and -1e30 masks; causal band
    in the chunk columns, padded chunk columns masked."""
    m = O.build_mask([4], [3], 2, 5, 9, 16)
    assert m.shape == (1, 2, 5, 9)
    assert set(np.unique(m).tolist()) == {0.0, float(np.float32(-1e30))}
    assert (m[0, :, :, :4] == 0).all()
    chunk = m[0, 0, :, 4:]
    for i in range(5):
        for j in range(5):
            assert (chunk[i, j] == 0) == (j <= i and j < 3)


def test_select_row_is_last_real_row():
    x = np.random.default_rng(0).standard_normal((2, 3, 7, 4))
    y = O.select_row(x, np.array([5, 0], dtype=np.int32), -1)
    np.testing.assert_array_equal(y[0], x[0, :, 4])
    assert (y[1] == 0).all()  # n_valid = 0: no real row


# ------------------------------------------------------------ golden values

def test_golden_skainet_validation_case():
    """[SKaiNET] "Validation": an 852-token prompt split as an 800-position cache plus a
    52-token chunk padded to C = 64; the selected row is 51 and sits at position 851."""
    g = json.load(open(os.path.join(GOLDEN, "skainet_validation.json")))
    cfg = I.config("c2")
    assert cfg.seen[0] == g["cached"] and cfg.C == g["chunk"] and cfg.n_valid[0] == g["real"]
    assert cfg.n_valid[0] - 1 == g["select_row"]
    assert cfg.seen[0] + g["select_row"] == g["position"]
    assert cfg.seen[0] + cfg.n_valid[0] == g["prompt_tokens"]
    m = O.build_mask(cfg.seen, cfg.n_valid, cfg.H, cfg.C, cfg.mask_ld(), cfg.cap)
    assert m.shape == tuple(g["mask_shape"])


def test_golden_cactus_tail():
    """[cactus] "Problem"/"Fix" and the review sweep: tail = prompt mod 128; a padded tail
    over-evicts at most pad_count rows of a 512-window ring."""
    g = json.load(open(os.path.join(GOLDEN, "cactus_tail.json")))
    for n, tail in zip(g["sweep_prompt"], g["sweep_tail"]):
        assert n % g["chunk"] == tail
    n = g["worst_prompt"]
    full, tail = divmod(n, g["chunk"])
    assert tail == g["worst_tail"]
    seen = full * g["chunk"]
    ev = O.padded_overevicted(seen, tail, g["chunk"], g["window"], 1, 0)
    assert g["chunk"] - tail == g["pad_count"]
    assert 0 < len(ev) <= g["pad_count"]
    # they are the oldest rows that the exact (unpadded) append keeps
    kept = O.live_positions(seen + tail, g["window"], 1, 0)
    assert list(ev) == list(kept[:len(ev)])
    assert all(p < seen for p in ev)


def test_row_subset_matches_full_call():
    """Computing selected rows only returns the same bits for those rows."""
    cfg = I.small(**CASES[1])
    t = _layer(cfg)
    full = O.attn(t["q"], t["k"], t["v"], t["kc"], t["vc"], t["seen"], t["n_valid"])
    part = O.attn(t["q"], t["k"], t["v"], t["kc"], t["vc"], t["seen"], t["n_valid"], rows=[0, 3])
    np.testing.assert_array_equal(part[:, :, [0, 3]], full[:, :, [0, 3]])
    assert (part[:, :, [1, 2, 4]] == 0).all()
