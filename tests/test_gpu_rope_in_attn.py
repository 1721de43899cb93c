"""RoPE of the queries folded into the attention's load of Q ([SKaiNET] "Change
(additive)": RoPE from per-position tables): the call with the raw queries and the
tables gives the bits of cp_rope_chunk(q) followed by the call with the rotated queries,
in every kernel configuration, both mask modes, split and unsplit, shared and per-sequence
tables; and the fused layer step matches the oracle."""
import numpy as np
import pytest
import torch

from chunked_prefill_attention_rope_amd import inputs as I
from oracle import oracle as O
from tests.gpu_helpers import TOL, bits, dev, real_rows_mask, rowwise_rel_err, to_f64
from tests.test_gpu_attn import SMALL

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def cp():
    from chunked_prefill_attention_rope_amd import cp as mod
    return mod


@pytest.mark.parametrize("kw", SMALL, ids=lambda c: c["name"])
@pytest.mark.parametrize("mode", ["inkernel", "explicit"])
@pytest.mark.parametrize("kernel", ["auto", "generic"])
@pytest.mark.parametrize("split", ["split", "nosplit"])
def test_rope_q_in_attention_bitwise(cp, kw, mode, kernel, split):
    kw = dict(kw)
    kw.pop("name")
    cfg = I.small(**kw)
    t = I.make_layer(cfg)
    cache = cp.KVCache(dev(t["kc"]), dev(t["vc"]), dev(t["seen"]), ring=cfg.ring, sink=cfg.sink)
    q, k, v, cos, sin = (dev(t[n]) for n in ("q", "k", "v", "cos", "sin"))
    nv = dev(t["n_valid"])
    mask = (cp.build_mask(cache, nv, cfg.H, cfg.C, cfg.mask_ld(), window=cfg.window)
            if mode == "explicit" else None)
    window = 0 if mask is not None else cfg.window
    flags = (cp.ATTN_FORCE_GENERIC if kernel == "generic" else 0) | (
        cp.ATTN_NO_SPLIT if split == "nosplit" else 0)
    nb = cp.attn_workspace_bytes(cache, q, k, v, mask=mask, window=window, flags=flags)
    ws = torch.empty(max(nb, 1), dtype=torch.uint8, device="cuda")
    qr = cp.rope_chunk(q, cos, sin)
    ref = cp.attn_chunk_with_past(cache, qr, k, v, n_valid=nv, mask=mask, window=window,
                                  scale=cfg.scale, workspace=ws, flags=flags)
    sel = torch.zeros((cfg.B, cfg.H, cfg.D), dtype=q.dtype, device="cuda")
    got = cp.attn_chunk_with_past(cache, q, k, v, n_valid=nv, mask=mask, window=window,
                                  scale=cfg.scale, workspace=ws, flags=flags, select_out=sel,
                                  q_rope=(cos, sin))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(got), bits(ref))
    np.testing.assert_array_equal(bits(sel), bits(cp.select_row(ref, nv, -1)))


@pytest.mark.parametrize("tables", ["shared", "per_sequence"])
@pytest.mark.parametrize("ring", [0, 1])
def test_fused_step_with_rope_q_in_attention(cp, tables, ring, monkeypatch):
    """The layer step with the queries rotated by the attention (forced for a small
    chunk) against the oracle and against the step with a separate RoPE of Q."""
    from chunked_prefill_attention_rope_amd import path
    seen = [300, 300] if tables == "shared" else [300, 41]
    cfg = I.small(dtype=I.BF16, B=2, H=8, nKV=2, D=128, C=64, cap=256 if ring else 512,
                  ring=ring, window=256 if ring else 0, seen=seen, n_valid=[64, 50])
    t = I.make_layer(cfg)
    assert t["cos"].shape[0] == (1 if tables == "shared" else 2)

    def run(fold):
        monkeypatch.setattr(path, "ROPE_Q_IN_ATTENTION_BYTES", 0 if fold else 1 << 62)
        cache = cp.KVCache(dev(t["kc"]), dev(t["vc"]), dev(t["seen"]), ring=cfg.ring)
        d = {n: dev(t[n]) for n in ("q", "k", "v", "cos", "sin", "n_valid")}
        bufs = path.make_buffers(cache, d["q"], d["k"], d["v"], window=cfg.window)
        out, sel = path.chunk_step(cache, d["q"], d["k"], d["v"], d["cos"], d["sin"],
                                   d["n_valid"], bufs, window=cfg.window)
        torch.cuda.synchronize()
        return out, sel, cache

    out_f, sel_f, cf = run(True)
    out_s, sel_s, cs = run(False)
    np.testing.assert_array_equal(bits(out_f), bits(out_s))
    np.testing.assert_array_equal(bits(sel_f), bits(sel_s))
    np.testing.assert_array_equal(bits(cf.k), bits(cs.k))
    np.testing.assert_array_equal(bits(cf.v), bits(cs.v))
    assert cf.seen.cpu().tolist() == cs.seen.cpu().tolist()
    qr = O.rope(I.np_view(t["q"]), I.np_view(t["cos"]), I.np_view(t["sin"]))
    kr = O.rope(I.np_view(t["k"]), I.np_view(t["cos"]), I.np_view(t["sin"]))
    ref = O.attn(qr, kr, I.np_view(t["v"]), I.np_view(t["kc"]), I.np_view(t["vc"]),
                 I.np_view(t["seen"]), I.np_view(t["n_valid"]), None, cfg.ring, cfg.sink,
                 cfg.window, cfg.scale)
    got = to_f64(out_f)
    assert rowwise_rel_err(got, ref, real_rows_mask(cfg, got.shape)) <= TOL[I.BF16]
