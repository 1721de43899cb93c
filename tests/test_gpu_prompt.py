"""A whole prompt run in chunks of any size C gives the oracle's result for the prompt as
one chunk (chunked prefill is exact: [SKaiNET] "Change (additive)" / "Validation") --
outputs within the bf16 tolerance, the final caches identical byte for byte whatever C."""
import numpy as np
import pytest
import torch

from chunked_prefill_attention_rope_amd import inputs as I
from oracle import oracle as O
from tests.gpu_helpers import TOL, bits, dev, rowwise_rel_err, to_f64

pytestmark = pytest.mark.gpu

CASES = [
    dict(name="global", B=2, H=8, nKV=2, D=128, C=40, cap=200, seen=[30, 0]),
    dict(name="ring", B=1, H=8, nKV=1, D=256, C=40, cap=64, ring=1, window=64, seen=[100]),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: c["name"])
def test_prompt_in_chunks_of_any_size(case):
    from chunked_prefill_attention_rope_amd import cp, path
    kw = dict(case)
    kw.pop("name")
    P = kw["C"]
    cfg = I.small(dtype=I.BF16, n_valid=[P] * kw["B"], **kw)
    t = I.make_layer(cfg)
    qr = O.rope(I.np_view(t["q"]), I.np_view(t["cos"]), I.np_view(t["sin"]))
    kr = O.rope(I.np_view(t["k"]), I.np_view(t["cos"]), I.np_view(t["sin"]))
    ref = O.attn(qr, kr, I.np_view(t["v"]), I.np_view(t["kc"]), I.np_view(t["vc"]),
                 I.np_view(t["seen"]), I.np_view(t["n_valid"]), None, cfg.ring, cfg.sink,
                 cfg.window, cfg.scale)
    ko, vo, so, live = O.kv_append(I.np_view(t["kc"]), I.np_view(t["vc"]), I.np_view(t["seen"]),
                                   kr, I.np_view(t["v"]), I.np_view(t["n_valid"]), cfg.ring,
                                   cfg.sink)
    q, k, v, cos, sin = (dev(t[n]) for n in ("q", "k", "v", "cos", "sin"))
    # seen_start: the host's bound on seen before the prompt (sizes the key splits only)
    ms = max(cfg.seen)
    for C, ss in ((8, None), (16, None), (33, None), (64, None), (16, ms), (33, ms)):
        cache = cp.KVCache(dev(t["kc"]), dev(t["vc"]), dev(t["seen"]), ring=cfg.ring,
                           sink=cfg.sink)
        pc = path.prompt_chunks(cache, q, k, v, cos, sin, C, window=cfg.window)
        sel = path.prefill(cache, pc, window=cfg.window, seen_start=ss)
        torch.cuda.synchronize()
        got = np.concatenate([to_f64(b.out) for b in pc.bufs], axis=2)[:, :, :P]
        assert rowwise_rel_err(got, ref) <= TOL[I.BF16], C
        np.testing.assert_array_equal(bits(sel), bits(pc.bufs[-1].out[:, :, (P - 1) % C]))
        assert cache.seen.cpu().tolist() == so.tolist()
        kg, vg = bits(cache.k), bits(cache.v)
        for b in range(cfg.B):
            sl = np.nonzero(live[b])[0]
            np.testing.assert_array_equal(kg[b][:, sl], ko.view(np.uint8).reshape(kg.shape)[b][:, sl])
            np.testing.assert_array_equal(vg[b][:, sl], vo.view(np.uint8).reshape(vg.shape)[b][:, sl])
