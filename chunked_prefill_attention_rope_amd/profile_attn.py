"""Run one workload's attention call (or whole layer step) N times, for profilers.

    python -m chunked_prefill_attention_rope_amd.profile_attn --workload c5 --layer 5 --reps 5
    python -m chunked_prefill_attention_rope_amd.profile_attn --workload c5g --C 16 --reps 5

A workload of the bandwidth sweep (c2 at batch --B, c4 or c5g at chunk --C, --explicit
for c2's mask) is built as the sweep builds it.

Eager launches on torch's current stream, inputs resident in HBM, nothing
else timed or checked: meant to sit under `rocprofv3 --kernel-trace` or
`--pmc` so that per-dispatch counters cover exactly the kernels of the path.
"""
import argparse
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import torch  # noqa: E402

from chunked_prefill_attention_rope_amd import cp, inputs as I, path  # noqa: E402


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default="c2")
    ap.add_argument("--layer", type=int, default=0)
    ap.add_argument("--reps", type=int, default=5)
    ap.add_argument("--step", action="store_true", help="whole layer step, not attention only")
    ap.add_argument("--flags", type=int, default=0)
    ap.add_argument("--B", type=int, default=None, help="sweep shape: batch (c2)")
    ap.add_argument("--C", type=int, default=None, help="sweep shape: chunk rows (c4, c5g)")
    ap.add_argument("--explicit", type=int, default=None, help="sweep shape: c2's mask (1/0)")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="instead: copy a buffer of this many bytes (counter calibration)")
    a = ap.parse_args()
    if a.copy_bytes:
        # a plain device copy of known size: reads and writes exactly copy_bytes each
        src = torch.ones(a.copy_bytes // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(a.reps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(f"profile_attn: copy of {a.copy_bytes} bytes x{a.reps} done", flush=True)
        return
    if a.B is not None or a.C is not None or a.explicit is not None or a.workload == "c5g":
        cfg = I.derived(a.workload, B=a.B, C=a.C,
                        explicit_mask=None if a.explicit is None else bool(a.explicit))
    else:
        cfg = I.config(a.workload, a.layer)
    t = I.make_layer(cfg, nan_dead=False)
    d = {k: v.to("cuda") for k, v in t.items()}
    seen0 = d["seen"].clone()
    cache = cp.KVCache(d["kc"], d["vc"], d["seen"], ring=cfg.ring, sink=cfg.sink)
    mask = None
    if cfg.explicit_mask:
        mask = cp.build_mask(cache, d["n_valid"], cfg.H, cfg.C, cfg.mask_ld())
    window = 0 if mask is not None else cfg.window
    static = bool(cfg.ring) and any(n < cfg.C for n in cfg.n_valid)
    max_seen = max(1, max(cfg.seen))  # the host's bound on seen, as the bench passes it
    # no flags given: the ones the bench passes (balanced splits for a skewed batch)
    flags = a.flags if a.flags else path.attn_flags_for(cfg.seen)
    bufs = path.make_buffers(cache, d["q"], d["k"], d["v"], mask=mask, window=window,
                             static_append=static, flags=flags)
    cp.rope_chunk(d["q"], d["cos"], d["sin"], out=bufs.q_rot)
    cp.rope_chunk(d["k"], d["cos"], d["sin"], out=bufs.k_rot)
    for _ in range(a.reps):
        if a.step:
            d["seen"].copy_(seen0)
            path.chunk_step(cache, d["q"], d["k"], d["v"], d["cos"], d["sin"], d["n_valid"],
                            bufs, mask=mask, window=window, static_append=static, flags=flags,
                            max_seen=max_seen)
        else:
            fold = path.rope_q_in_attention(d["q"])  # the step's configuration
            cp.attn_chunk_with_past(cache, d["q"] if fold else bufs.q_rot, bufs.k_rot, d["v"],
                                    n_valid=d["n_valid"], mask=mask, window=window,
                                    scale=cfg.scale, out=bufs.out, workspace=bufs.workspace,
                                    flags=flags, max_seen=max_seen,
                                    q_rope=(d["cos"], d["sin"]) if fold else None)
    torch.cuda.synchronize()
    print(f"profile_attn: {a.workload} layer {a.layer} x{a.reps} done", flush=True)


if __name__ == "__main__":
    main()
