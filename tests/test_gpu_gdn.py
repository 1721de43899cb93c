"""GPU parity of the chunked gated-delta-rule prefill (HIP path through the C ABI) with
the oracle's token-by-token recurrence ([Kazeia] "Chantier 4 -- GDN chunkwise prefill").
Tolerance: fp32 storage, max over (sequence, head, token) of max_j |out - ref| / max_j
|ref| <= 1e-4; the final state alike over its rows."""
import numpy as np
import pytest
import torch

from chunked_prefill_attention_rope_amd import inputs as I
from oracle import oracle as O
from tests.gpu_helpers import dev, rowwise_rel_err, to_f64

pytestmark = pytest.mark.gpu
TOL = 1e-4


@pytest.fixture(scope="module")
def cp():
    from chunked_prefill_attention_rope_amd import cp as mod
    return mod


def _run(cp, t):
    d = {k: dev(v) for k, v in t.items()}
    st = d["state"].clone()
    out = cp.gdn_chunk_prefill(d["q"], d["k"], d["v"], d["beta"], d["alpha"], st)
    torch.cuda.synchronize()
    return out, st


def _check(cp, t):
    out, st = _run(cp, t)
    ref_o, ref_s = O.gdn(*(t[n].numpy() for n in ("q", "k", "v", "beta", "alpha", "state")))
    assert rowwise_rel_err(to_f64(out), ref_o) <= TOL
    assert rowwise_rel_err(to_f64(st), ref_s) <= TOL


@pytest.mark.parametrize("dk,dv", [(64, 64), (64, 128), (128, 64), (128, 128)])
@pytest.mark.parametrize("P", [1, 63, 64, 150])
def test_gdn_matches_token_recurrence(cp, dk, dv, P):
    cfg = I.GdnCfg("t", 2, 3, P, dk, dv, 77)
    _check(cp, I.make_gdn(cfg))


def test_gdn_many_heads(cp):
    """33 (sequence, head) pairs over five chunks, the last one ragged: the scan
    workgroups of several heads share each XCD's slots (surplus workgroups of the last
    group exit at once), and the output waves run over an odd number of chunks."""
    cfg = I.GdnCfg("t", 3, 11, 300, 128, 128, 91)
    _check(cp, I.make_gdn(cfg))


@pytest.mark.parametrize("name", ["g0", "g1"])
def test_gdn_workloads(cp, name):
    _check(cp, I.make_gdn(I.gdn_config(name)))


def test_gdn_state_carries_across_calls(cp):
    """Two calls handing the state over equal one call (the layer's cache semantics)."""
    cfg = I.GdnCfg("t", 1, 2, 200, 64, 64, 5)
    t = I.make_gdn(cfg)
    whole, st_whole = _run(cp, t)
    d = {k: dev(v) for k, v in t.items()}
    st = d["state"].clone()
    P1 = 77
    o1 = cp.gdn_chunk_prefill(*(d[n][:, :, :P1].contiguous() for n in ("q", "k", "v", "beta", "alpha")), st)
    o2 = cp.gdn_chunk_prefill(*(d[n][:, :, P1:].contiguous() for n in ("q", "k", "v", "beta", "alpha")), st)
    torch.cuda.synchronize()
    got = torch.cat([o1, o2], dim=2)
    assert rowwise_rel_err(to_f64(got), to_f64(whole)) <= TOL
    assert rowwise_rel_err(to_f64(st), to_f64(st_whole)) <= TOL


def test_gdn_empty_is_a_noop(cp):
    z = torch.empty((1, 2, 0, 64), device="cuda")
    st = torch.ones((1, 2, 64, 64), device="cuda")
    cp.gdn_chunk_prefill(z, z, z, torch.empty((1, 2, 0), device="cuda"),
                         torch.empty((1, 2, 0), device="cuda"), st)
    torch.cuda.synchronize()
    assert bool((st == 1).all())
