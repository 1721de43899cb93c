"""cp_attn_chunk_with_past_noalloc (key-split partials in the library's own device array)
against cp_attn_chunk_with_past with a caller workspace: bit-identical outputs and
selections on two calls in a row, the second on a smaller problem (the array keeps the
first call's partials), and within tolerance of the oracle."""
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


def _case(cp, cfg, explicit):
    t = I.make_layer(cfg)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    cache = cp.KVCache(dev(t["kc"]), dev(t["vc"]), dev(t["seen"]), ring=cfg.ring, sink=cfg.sink,
                       status=status)
    q, k, v, nv = dev(t["q"]), dev(t["k"]), dev(t["v"]), dev(t["n_valid"])
    mask = cp.build_mask(cache, nv, cfg.H, cfg.C, cfg.mask_ld()) if explicit else None
    window = 0 if explicit else cfg.window
    return t, cache, status, q, k, v, nv, mask, window


def _ref_call(cp, cfg, cache, q, k, v, nv, mask, window):
    nb = cp.attn_workspace_bytes(cache, q, k, v, mask=mask, window=window)
    assert nb > 0, "the case must take the key-split path"
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    sel = torch.zeros((cfg.B, cfg.H, cfg.D), dtype=q.dtype, device="cuda")
    out = cp.attn_chunk_with_past(cache, q, k, v, n_valid=nv, mask=mask, window=window,
                                  scale=cfg.scale, workspace=ws, select_out=sel)
    return out, sel, nb


def _oracle(cfg, t):
    v = I.np_view
    return O.attn(v(t["q"]), v(t["k"]), v(t["v"]), v(t["kc"]), v(t["vc"]), v(t["seen"]),
                  v(t["n_valid"]), None, cfg.ring, cfg.sink, cfg.window, cfg.scale)


# first a larger split problem (c2: 800 cached, 52 of 64 rows, explicit mask, D 256), then
# smaller ones whose partials occupy only the front of the array
SEQUENCES = [
    [("c2", True), ("decode", False)],
    [("c3", False), ("c2", True)],
]


def _cfg(name):
    if name == "decode":
        return I.small(dtype=I.BF16, B=2, H=8, nKV=2, D=128, C=1, cap=3000, seen=[2900, 1200],
                       n_valid=[1, 1], seed=11)
    return I.config(name)


@pytest.mark.parametrize("seq", SEQUENCES, ids=lambda s: "-".join(n for n, _ in s))
def test_noalloc_matches_workspace_call(cp, seq):
    for name, explicit in seq:
        cfg = _cfg(name)
        t, cache, status, q, k, v, nv, mask, window = _case(cp, cfg, explicit)
        ref, ref_sel, need = _ref_call(cp, cfg, cache, q, k, v, nv, mask, window)
        assert need <= cp.ATTN_SCRATCH_BYTES
        out = torch.full_like(q, 3.0)
        sel = torch.full((cfg.B, cfg.H, cfg.D), 5.0, dtype=q.dtype, device="cuda")
        cp.attn_chunk_with_past_noalloc(cache, q, k, v, out, n_valid=nv, mask=mask,
                                        window=window, scale=cfg.scale, select_out=sel)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(bits(out), bits(ref))
        np.testing.assert_array_equal(bits(sel), bits(ref_sel))
        got = to_f64(out)
        err = rowwise_rel_err(got, _oracle(cfg, t), real_rows_mask(cfg, got.shape))
        assert err <= TOL[cfg.dtype], (name, err)
        assert int(status.item()) == 0


def test_noalloc_unsplit_and_refusal(cp):
    """A call that needs no key split (the array is not touched) gives the workspace
    call's bits; a forced split count whose partials exceed the array is refused with
    CP_ERR_SCRATCH and enqueues nothing (the output keeps its contents)."""
    cfg = I.small(dtype=I.BF16, B=2, H=8, nKV=2, D=128, C=300, cap=700, seen=[250, 399],
                  n_valid=[300, 177], seed=12)
    t, cache, status, q, k, v, nv, mask, window = _case(cp, cfg, False)
    ns = cp.ATTN_NO_SPLIT
    assert cp.attn_workspace_bytes(cache, q, k, v, flags=ns) == 0
    ref = cp.attn_chunk_with_past(cache, q, k, v, n_valid=nv, scale=cfg.scale, flags=ns)
    out = torch.empty_like(q)
    cp.attn_chunk_with_past_noalloc(cache, q, k, v, out, n_valid=nv, scale=cfg.scale, flags=ns)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(out), bits(ref))

    big = I.small(dtype=I.BF16, B=16, H=32, nKV=8, D=256, C=512, cap=1024, seen=[64] * 16,
                  n_valid=[512] * 16, seed=13)
    tb = I.make_layer(big, nan_dead=False)
    cb = cp.KVCache(dev(tb["kc"]), dev(tb["vc"]), dev(tb["seen"]))
    qb, kb, vb = dev(tb["q"]), dev(tb["k"]), dev(tb["v"])
    flags = cp.ATTN_SPLITS(64)
    assert cp.attn_workspace_bytes(cb, qb, kb, vb, flags=flags) > cp.ATTN_SCRATCH_BYTES
    ob = torch.full_like(qb, 7.0)
    with pytest.raises(cp.CpError) as e:
        cp.attn_chunk_with_past_noalloc(cb, qb, kb, vb, ob, scale=big.scale, flags=flags)
    assert e.value.code == cp.ERR_SCRATCH
    torch.cuda.synchronize()
    assert (ob.float() == 7.0).all()


def test_noalloc_balanced(cp):
    """Balanced key splits (CP_ATTN_BALANCE) through the array: the plan and the pieces'
    partials of the Llama-8B-like batch, then of a smaller skewed batch (the array keeps
    the first plan), each bit-identical to the workspace call and within tolerance of
    the oracle."""
    small = I.small(dtype=I.BF16, B=5, H=8, nKV=2, D=128, C=96, cap=3200,
                    seen=[3000, 5, 700, 2500, 64], n_valid=[96, 96, 40, 77, 1], seed=14)
    for cfg in (I.config("c4"), small):
        t, cache, status, q, k, v, nv, mask, window = _case(cp, cfg, False)
        flags = cp.ATTN_BALANCE
        need = cp.attn_workspace_bytes(cache, q, k, v, flags=flags)
        assert 0 < need <= cp.ATTN_SCRATCH_BYTES
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        ref = cp.attn_chunk_with_past(cache, q, k, v, n_valid=nv, scale=cfg.scale, workspace=ws,
                                      flags=flags)
        out = torch.full_like(q, 3.0)
        cp.attn_chunk_with_past_noalloc(cache, q, k, v, out, n_valid=nv, scale=cfg.scale,
                                        flags=flags)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(bits(out), bits(ref))
        got = to_f64(out)
        err = rowwise_rel_err(got, _oracle(cfg, t), real_rows_mask(cfg, got.shape))
        assert err <= TOL[cfg.dtype], (cfg.name, err)
        assert int(status.item()) == 0
