#!/usr/bin/env python3
"""Throughput of the chunked-prefill-with-past hot path on one MI355X.

One step = one pass of the whole path of every layer of the workload over one
chunk: RoPE(Q), RoPE(K), [padded-append snapshot], attention over past + C
keys, KV append, [rollback], last-real-row selection -- all in libcp's HIP
kernels.  Inputs are seeded synthetic tensors resident in HBM before timing.

Each timed step gets its own pre-initialised `seen` array over the shared K/V
buffers, so every step does exactly the same work (same positions, same rows
written) and nothing but the path runs inside the timed region.  The K timed
steps are captured once into a HIP graph and replayed (launch amortisation);
the eager rate is reported beside it on stderr.

Prints ONE JSON line on stdout.  metric: real chunk tokens per second per
layer.  roofline: the attention call (the dominant kernel) timed alone with
HIP events over a graph of back-to-back launches, against its algorithmic
bytes or flops.  cpu_baseline: the CPU oracle timed on a bounded sample.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

from chunked_prefill_attention_rope_amd import inputs as I  # noqa: E402

METRIC = "chunk-prefill tok/s per layer; achieved TB/s or MFMA % of MI355X peak"
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0    # dense bf16 MFMA
FP32_PEAK_TFLOPS = 157.3     # fp32 vector

WORKLOADS = {
    "c1": "single fp32 layer, H4/KV1 D64, 48 cached, C16 (11 real), global, explicit mask",
    "c2": "Gemma-270M-like global layer, bf16, H4/KV1 D256, 800 cached, C64 (52 real), "
          "explicit per-head mask [1,4,64,864], select row 51",
    "c3": "sliding ring W512 holding 1023 positions, bf16, H8/KV1 D256, C128 (127 real, "
          "padded append with snapshot/rollback), in-kernel mask",
    "c4": "Llama-8B-like GQA layer, bf16, B16 H32/KV8 D128, past U[0,4095], C128, global causal",
    "c5": "long context, bf16, B4 H32/KV8 D128, 32768 past, C512, 5 sliding (W4096) + 1 global",
}


def layers_of(name):
    return [I.config(name, l) for l in range(6)] if name == "c5" else [I.config(name)]


def attended(cfg, b, i):
    """(past rows, chunk rows) attended by real row i of sequence b (in-kernel rule)."""
    seen = cfg.seen[b]
    qpos = seen + i
    L = cfg.live_count(b)
    if cfg.ring:
        R = cfg.cap - cfg.sink
        ns = min(cfg.sink, seen)
        lo = max(cfg.sink, seen - R)
    else:
        ns, lo = 0, 0
    first = qpos - cfg.window + 1 if cfg.window else -(1 << 60)
    npast = ns + max(0, seen - max(lo, first)) if L else 0
    npast = min(npast, L)
    nchunk = i + 1 if not cfg.window else min(i + 1, cfg.window)
    return npast, nchunk


def algorithmic(cfg):
    """Algorithmic HBM bytes and flops of one attention launch: Q, the chunk's K/V, the
    past K/V rows some real row attends, the output (and the explicit mask); flops
    4*D per attended (query head, key) pair of a real row."""
    es = 4 if cfg.dtype == I.F32 else 2
    B, H, nKV, C, D = cfg.B, cfg.H, cfg.nKV, cfg.C, cfg.D
    nbytes = 2 * B * H * C * D * es + 2 * B * nKV * C * D * es
    pairs = 0
    for b in range(B):
        nv = cfg.n_valid[b]
        for i in range(nv):
            npast, nchunk = attended(cfg, b, i)
            pairs += npast + nchunk
        # every real row attends a suffix of the live past (plus the sinks); row 0's
        # is the longest, so it is the union of the past rows that must be read
        if nv:
            nbytes += 2 * nKV * attended(cfg, b, 0)[0] * D * es
    if cfg.explicit_mask:
        nbytes += B * H * C * cfg.mask_ld() * 4
    flops = 4 * D * H * pairs
    return nbytes, flops


def measured_traffic(workload, flags):
    """HBM bytes per attention call from the committed rocprofv3 counter record
    (FETCH_SIZE and WRITE_SIZE scaled by the copy-kernel calibration), or None when
    none was taken for this workload or the attention sources changed since."""
    from chunked_prefill_attention_rope_amd.profiling import source_digest
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if flags or not os.path.exists(path):
        return None
    rec = json.load(open(path)).get(workload)
    if not rec or rec.get("source_sha1") != source_digest():
        return None
    return rec["bytes_per_call"]


class Layer:
    """Device inputs, per-step caches and buffers of one layer."""

    def __init__(self, cp, path, cfg, nsteps, flags=0):
        self.cfg = cfg
        # no flags given: the ones a caller that knows its past lengths would pass
        self.flags = flags if flags else path.attn_flags_for(cfg.seen)
        t = I.make_layer(cfg, nan_dead=False)
        self.host = t
        d = {k: v.to("cuda") for k, v in t.items()}
        self.d = d
        self.seen0 = d["seen"]
        self.seen_all = d["seen"].repeat(nsteps, 1).contiguous()
        self.caches = [cp.KVCache(d["kc"], d["vc"], self.seen_all[s], ring=cfg.ring,
                                  sink=cfg.sink) for s in range(nsteps)]
        self.mask = None
        if cfg.explicit_mask:
            self.mask = cp.build_mask(self.caches[0], d["n_valid"], cfg.H, cfg.C, cfg.mask_ld())
        self.static = bool(cfg.ring) and any(n < cfg.C for n in cfg.n_valid)
        self.window = 0 if cfg.explicit_mask else cfg.window
        # the host knows the past lengths it generated: the attention sizes its key
        # splits from the longest (a serving scheduler holds them the same way)
        self.max_seen = max(1, max(cfg.seen))
        self.bufs = path.make_buffers(self.caches[0], d["q"], d["k"], d["v"], mask=self.mask,
                                      window=self.window, static_append=self.static,
                                      flags=self.flags)

    def reset(self):
        self.seen_all.copy_(self.seen0.expand_as(self.seen_all))

    def step(self, path, s):
        d = self.d
        path.chunk_step(self.caches[s], d["q"], d["k"], d["v"], d["cos"], d["sin"],
                        d["n_valid"], self.bufs, mask=self.mask, window=self.window,
                        static_append=self.static, flags=self.flags, max_seen=self.max_seen)

    def attn_only(self, cp):
        """The attention call in the step's configuration (for large chunks the kernel
        rotates Q as it loads it, as the step does)."""
        from chunked_prefill_attention_rope_amd import path
        d, b = self.d, self.bufs
        fold = path.rope_q_in_attention(d["q"])
        cp.attn_chunk_with_past(self.caches[0], d["q"] if fold else b.q_rot, b.k_rot, d["v"],
                                n_valid=d["n_valid"], mask=self.mask, window=self.window,
                                scale=self.cfg.scale, out=b.out, workspace=b.workspace,
                                flags=self.flags, q_rope=(d["cos"], d["sin"]) if fold else None,
                                max_seen=self.max_seen)


def time_graph(fn, reps_inside, replays=1, warm=1):
    """Capture fn() once into a HIP graph; replay it `warm` times untimed, then `replays`
    times timed; ms per timed replay."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()  # warm the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    for _ in range(warm):  # warm replays
        g.replay()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(replays):
        g.replay()
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / replays, g


def cpu_baseline(layers, seconds):
    """The oracle as it stands, on host cores, over a bounded sample of the workload."""
    from oracle import oracle as O
    cores = O.num_threads()
    masks = [O.build_mask(l.cfg.seen, l.cfg.n_valid, l.cfg.H, l.cfg.C, l.cfg.mask_ld(),
                          l.cfg.cap, l.cfg.ring, l.cfg.sink, l.cfg.window)
             if l.cfg.explicit_mask else None for l in layers]  # caller-side input, untimed
    total_tok, total_s, reps, desc = 0, 0.0, 0, ""
    deadline = time.perf_counter() + seconds
    while True:
        for lay, mask in zip(layers, masks):
            cfg, t = lay.cfg, lay.host
            nv = I.np_view
            rows = None
            if cfg.C * max(cfg.live_count(b) for b in range(cfg.B)) > 4_000_000:
                rows = [0, cfg.C // 2, cfg.C - 1]  # sampled rows of a long-context layer
            t0 = time.perf_counter()
            qr = O.rope(nv(t["q"]), nv(t["cos"]), nv(t["sin"]))
            kr = O.rope(nv(t["k"]), nv(t["cos"]), nv(t["sin"]))
            out = O.attn(qr, kr, nv(t["v"]), nv(t["kc"]), nv(t["vc"]), nv(t["seen"]),
                         nv(t["n_valid"]), mask, cfg.ring, cfg.sink,
                         0 if mask is not None else cfg.window, cfg.scale, rows=rows)
            if rows is None:
                O.kv_append(nv(t["kc"]), nv(t["vc"]), nv(t["seen"]), kr, nv(t["v"]),
                            nv(t["n_valid"]), cfg.ring, cfg.sink)
            O.select_row(out, nv(t["n_valid"]), -1)
            total_s += time.perf_counter() - t0
            total_tok += (len(rows) * cfg.B) if rows else sum(cfg.n_valid)
            desc = (f"{len(rows)} sampled chunk rows x {cfg.B} sequences per layer (attention "
                    f"only)" if rows else "full layer step (rope, attention, append, select)")
        reps += 1
        if time.perf_counter() > deadline or reps >= 10000:
            break
    return {"value": total_tok / total_s, "unit": "tok/s", "cores": cores, "kind": "oracle",
            "sample": f"{desc}, {reps} reps over {len(layers)} layer(s), {total_s:.1f} s; "
                      f"{os.cpu_count()} host CPUs visible"}


# Bandwidth sweep: each workload's per-sequence shape at sizes where the attention can
# be HBM-bound (c2's shape batched; c4 and the c5 global layer at small chunks).
SWEEP = ([("c2", dict(B=b, explicit_mask=em)) for em in (True, False) for b in (1, 16, 64, 256)]
         + [(n, dict(C=c)) for n in ("c4", "c5g") for c in (1, 16, 32, 64)])

# Prompt-tail sweep: real tokens of a tail, run as one padded chunk or token by token.
TAIL_SWEEP = [1, 2, 3, 4, 6, 8, 9, 10, 12, 16, 24, 32, 48, 64, 96, 127]


def launch_latency_us():
    """Duration of a one-element device kernel per launch in a HIP graph (the floor any
    launch of the path pays)."""
    x = torch.zeros(1, device="cuda")
    ms, _ = time_graph(lambda: [x.add_(1.0) for _ in range(200)], 200)
    return ms * 1e3 / 200


def sweep(out_path):
    """Time the attention call alone on the SWEEP shapes; print a markdown table (and
    JSON lines to out_path).  Not the contract line: a separate measurement mode."""
    from chunked_prefill_attention_rope_amd import cp, path
    torch.cuda.set_device(0)
    lat = launch_latency_us()
    rows = []
    for name, kw in SWEEP:
        cfg = I.derived(name, **kw)
        lay = Layer(cp, path, cfg, 1, 0)
        d = lay.d
        cp.rope_qk_chunk(d["q"], d["k"], d["cos"], d["sin"], q_out=lay.bufs.q_rot,
                         k_out=lay.bufs.k_rot)
        reps = 20 if name == "c5g" else 100
        # steady state: a freshly built layer's first replays run slower (the long-context
        # caches measured 116 us per call on the first replay, 108 us after a few)
        ms, _ = time_graph(lambda: [lay.attn_only(cp) for _ in range(reps)], reps, replays=3,
                           warm=5)
        us = ms * 1e3 / reps
        nbytes, flops = algorithmic(cfg)
        row = {"shape": name, "B": cfg.B, "C": cfg.C, "G": cfg.G, "D": cfg.D,
               "mask": "explicit" if cfg.explicit_mask else "in-kernel",
               "attn_us": round(us, 3), "algorithmic_bytes": nbytes, "algorithmic_flops": flops,
               "flop_per_byte": round(flops / nbytes, 1),
               "hbm_gbs": round(nbytes / us / 1e3, 1),
               "hbm_frac": round(nbytes / us / 1e3 / HBM_PEAK_GBS, 4),
               "tflops": round(flops / us / 1e6, 1),
               "mfma_frac": round(flops / us / 1e6 / BF16_PEAK_TFLOPS, 4),
               "launch_latency_us": round(lat, 3)}
        rows.append(row)
        print(json.dumps(row), file=sys.stderr, flush=True)
        del lay
        torch.cuda.empty_cache()
    print(f"launch latency (one-element kernel in a graph): {lat:.2f} us")
    print("| shape | B | C | mask | flop/B | attention us | GB/s | % HBM | TFLOP/s | % MFMA |")
    print("|---|---:|---:|---|---:|---:|---:|---:|---:|---:|")
    for r in rows:
        print(f"| {r['shape']} | {r['B']} | {r['C']} | {r['mask']} | {r['flop_per_byte']} | "
              f"{r['attn_us']} | {r['hbm_gbs']} | {100 * r['hbm_frac']:.1f} | {r['tflops']} | "
              f"{100 * r['mfma_frac']:.1f} |")
    if out_path:
        with open(out_path, "w") as f:
            for r in rows:
                f.write(json.dumps(r) + "\n")


def tail_sweep(out_path, reps=20):
    """The [cactus] tail experiment on one layer of c3's shape (sliding ring W512 holding
    1023 positions, C128, H8/KV1 D256): a tail of n real tokens as one padded chunk step
    (snapshot, static append of 128 rows, rollback) against n one-token steps (RoPE,
    attention with C = 1, append of one row).  Each mode is a HIP graph of `reps`
    back-to-back tails; prints a markdown table and the breakeven."""
    from chunked_prefill_attention_rope_amd import cp, path
    torch.cuda.set_device(0)
    cfg = I.config("c3")
    t = I.make_layer(cfg, nan_dead=False)
    d = {k: v.to("cuda") for k, v in t.items()}
    cache = cp.KVCache(d["kc"], d["vc"], d["seen"], ring=cfg.ring, sink=cfg.sink)
    q, k, v, cos, sin = d["q"], d["k"], d["v"], d["cos"], d["sin"]
    W = cfg.window
    bufs = path.make_buffers(cache, q, k, v, window=W, static_append=True)
    rows = []
    for n in TAIL_SWEEP:
        nv = torch.full((cfg.B,), n, dtype=torch.int32, device="cuda")
        steps = path.token_steps(cache, q, k, v, cos, sin, n, window=W)
        ms_p, _ = time_graph(lambda: [path.chunk_step(cache, q, k, v, cos, sin, nv, bufs, window=W,
                                                      static_append=True)
                                      for _ in range(reps)], reps)
        ms_s, _ = time_graph(lambda: [path.scalar_tail(cache, steps, window=W)
                                      for _ in range(reps)], reps)
        row = {"n_tail": n, "padded_us": round(ms_p * 1e3 / reps, 2),
               "scalar_us": round(ms_s * 1e3 / reps, 2),
               "scalar_us_per_token": round(ms_s * 1e3 / reps / n, 2)}
        rows.append(row)
        print(json.dumps(row), file=sys.stderr, flush=True)
        del steps
    even = next((r["n_tail"] for r in rows if r["scalar_us"] > r["padded_us"]), None)
    print("| tail tokens | padded chunk us | token by token us | us per token |")
    print("|---:|---:|---:|---:|")
    for r in rows:
        print(f"| {r['n_tail']} | {r['padded_us']} | {r['scalar_us']} | {r['scalar_us_per_token']} |")
    print(f"breakeven: padding wins from {even} tail tokens on this GPU "
          f"(the pages' threshold: pad from {path.PAGES_PAD_FROM}; the default here: {path.PAD_FROM})")
    if out_path:
        with open(out_path, "w") as f:
            for r in rows:
                f.write(json.dumps(r) + "\n")


# Chunk-size sweep: a whole prompt prefilled in chunks of C on one layer of a workload's
# shape, from an empty global cache.
CHUNK_SWEEP_PROMPT = 1023
CHUNK_SWEEP_SIZES = [16, 32, 64, 128, 256, 512]
CHUNK_SWEEP_SHAPES = {
    "c2": dict(B=1, H=4, nKV=1, D=256, base=1e6),   # Gemma-270M-like
    "c4": dict(B=4, H=32, nKV=8, D=128, base=5e5),  # Llama-8B-like GQA
}


def chunk_sweep(out_path, reps=5):
    """Prefill a CHUNK_SWEEP_PROMPT-token prompt on one layer in chunks of each size (each
    rep from an empty cache), then apply the chunk-size selection to the measured
    per-chunk-step times."""
    from chunked_prefill_attention_rope_amd import cp, path
    torch.cuda.set_device(0)
    P = CHUNK_SWEEP_PROMPT
    rows = []
    for name, sh in CHUNK_SWEEP_SHAPES.items():
        cfg = I.LayerCfg(f"{name}-prompt", I.BF16, sh["B"], sh["H"], sh["nKV"], sh["D"], P,
                         P + 1, base=sh["base"], seen=[0] * sh["B"], n_valid=[P] * sh["B"],
                         seed=4242)
        t = I.make_layer(cfg, nan_dead=False)
        d = {k: v.to("cuda") for k, v in t.items()}
        seen_all = d["seen"].repeat(reps, 1).contiguous()
        caches = [cp.KVCache(d["kc"], d["vc"], seen_all[r]) for r in range(reps)]
        table = {}
        for C in CHUNK_SWEEP_SIZES:
            pc = path.prompt_chunks(caches[0], d["q"], d["k"], d["v"], d["cos"], d["sin"], C)
            seen_all.zero_()
            ms, _ = time_graph(lambda: [path.prefill(caches[r], pc) for r in range(reps)], reps)
            seen_all.zero_()
            us = ms * 1e3 / reps
            n = len(pc.q)
            table[C] = us / n
            row = {"shape": name, "prompt": P, "C": C, "chunks": n, "prefill_us": round(us, 1),
                   "us_per_chunk": round(us / n, 2), "tok_per_s": round(P / us * 1e6, 1)}
            rows.append(row)
            print(json.dumps(row), file=sys.stderr, flush=True)
            del pc
        best = path.choose_chunk(P, table)
        rows.append({"shape": name, "prompt": P, "chosen_C": best})
        del caches, d
        torch.cuda.empty_cache()
    print("| shape | C | chunks | prompt us | us per chunk | tok/s |")
    print("|---|---:|---:|---:|---:|---:|")
    for r in rows:
        if "C" in r:
            print(f"| {r['shape']} | {r['C']} | {r['chunks']} | {r['prefill_us']} | "
                  f"{r['us_per_chunk']} | {r['tok_per_s']} |")
    for r in rows:
        if "chosen_C" in r:
            print(f"chunk-size selection for a {r['prompt']}-token prompt on {r['shape']}: "
                  f"C = {r['chosen_C']}")
    if out_path:
        with open(out_path, "w") as f:
            for r in rows:
                f.write(json.dumps(r) + "\n")


def gdn_flops(B, H, P, dk, dv):
    """Algorithmic flops of a gated-delta-rule prefill: per token and head, the three
    dk x dv matrix-vector products of the recurrence (S^T k, the rank-1 update k delta^T,
    the read-out S^T q) at 2 flops per multiply-add -- the 3 S^2 multiply-adds per token
    that [Kazeia] "Le kernel actuel" counts.  The gate's scaling and the chunkwise form's
    extra intra-chunk products are not counted."""
    return 6 * B * H * P * dk * dv


def gdn_bytes(B, H, P, dk, dv):
    """Algorithmic HBM bytes: q, k, v, beta, alpha read, out written, state read and
    written once (fp32)."""
    return 4 * (B * H * P * (2 * dk + 2 * dv + 2) + 2 * B * H * dk * dv)


def gdn_bench(name, reps, cpu_seconds, with_cpu):
    """The gated-delta-rule chunkwise prefill (cp_gdn_chunk_prefill) on one workload:
    prompt tokens per second per layer, the call's roofline, the oracle's rate."""
    from chunked_prefill_attention_rope_amd import cp
    torch.cuda.set_device(0)
    cfg = I.gdn_config(name)
    t = I.make_gdn(cfg)
    d = {k: v.cuda() for k, v in t.items()}
    B, H, P, dk, dv = cfg.B, cfg.H, cfg.P, cfg.dk, cfg.dv
    st = d["state"].clone()
    out = torch.empty_like(d["v"])
    ws = torch.empty(cp.gdn_workspace_bytes(B, H, P, dk, dv), dtype=torch.uint8, device="cuda")

    def call():
        cp.gdn_chunk_prefill(d["q"], d["k"], d["v"], d["beta"], d["alpha"], st, out, ws)

    for _ in range(5):
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        call()
    e1.record()
    torch.cuda.synchronize()
    eager_ms = e0.elapsed_time(e1) / reps
    ms, _ = time_graph(lambda: [call() for _ in range(reps)], reps)
    ms /= reps
    flops, nbytes = gdn_flops(B, H, P, dk, dv), gdn_bytes(B, H, P, dk, dv)
    achieved = flops / (ms * 1e-3) / 1e12
    result = {
        "metric": "gated-delta-rule prefill tok/s per layer", "value": round(B * P / (ms * 1e-3), 1),
        "unit": "tok/s", "n_gpus": 1, "steps": reps, "warmup": 5,
        "ms_per_step": round(ms, 6), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"{name}: B={B} H={H} P={P} dk={dk} dv={dv}, chunk 64",
                   "launch": "hip-graph", "eager_ms_per_call": round(eager_ms, 6)},
        "roofline": {"bound": "alu", "achieved": round(achieved, 4), "peak": FP32_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / FP32_PEAK_TFLOPS, 5),
                     "traffic": None, "kernel": "cp_gdn_chunk_prefill (prep + scan)",
                     "avg_launch_us": round(ms * 1e3, 3), "algorithmic_flops": flops,
                     "algorithmic_bytes": nbytes,
                     "hbm_frac": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 5)},
    }
    if with_cpu:
        from oracle import oracle as O
        args = [t[n].numpy() for n in ("q", "k", "v", "beta", "alpha", "state")]
        total, reps_c = 0.0, 0
        while total < cpu_seconds and reps_c < 1000:
            t0 = time.perf_counter()
            O.gdn(*args)
            total += time.perf_counter() - t0
            reps_c += 1
        result["cpu_baseline"] = {
            "value": round(B * P * reps_c / total, 1), "unit": "tok/s",
            "cores": O.num_threads(), "kind": "oracle",
            "sample": f"whole workload, token-by-token fp64 recurrence, {reps_c} reps, "
                      f"{total:.1f} s; {os.cpu_count()} host CPUs visible"}
    print(f"[bench] {name}: gdn {ms * 1e3:.2f} us/call graph, {eager_ms * 1e3:.2f} eager",
          file=sys.stderr, flush=True)
    print(json.dumps(result), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="c5", choices=sorted(WORKLOADS))
    ap.add_argument("--eager", action="store_true", help="time eager launches, not a graph")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--attn-reps", type=int, default=200)
    ap.add_argument("--attn-flags", type=int, default=0,
                    help="CP_ATTN_* flags for the attention call (e.g. a forced split count)")
    ap.add_argument("--sweep", action="store_true",
                    help="instead: the attention alone on the bandwidth-sweep shapes")
    ap.add_argument("--sweep-out", default=None, help="JSON lines of the sweep")
    ap.add_argument("--tail-sweep", action="store_true",
                    help="instead: padded-chunk vs token-by-token prompt tails (c3's shape)")
    ap.add_argument("--chunk-sweep", action="store_true",
                    help="instead: a whole prompt in chunks of 16..512 and the chunk selection")
    ap.add_argument("--gdn", default=None, choices=["g0", "g1"],
                    help="instead: the gated-delta-rule chunkwise prefill on this workload")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU: this path has no multi-GPU mode (see DESIGN.md for "
              "how it would shard); use --gpus 1", file=sys.stderr)
        sys.exit(2)
    if args.gdn:
        gdn_bench(args.gdn, args.attn_reps, args.cpu_seconds, not args.no_cpu_baseline)
        return
    if args.sweep:
        sweep(args.sweep_out)
        return
    if args.tail_sweep:
        tail_sweep(args.sweep_out)
        return
    if args.chunk_sweep:
        chunk_sweep(args.sweep_out)
        return

    from chunked_prefill_attention_rope_amd import cp, path

    torch.cuda.set_device(0)
    K, W = args.steps, args.warmup
    layers = [Layer(cp, path, cfg, K + W, args.attn_flags) for cfg in layers_of(args.workload)]
    torch.cuda.synchronize()
    cfg0 = layers[0].cfg
    tokens_per_layer = sum(cfg0.n_valid)
    nl = len(layers)

    def run_steps(lo, hi):
        for s in range(lo, hi):
            for lay in layers:
                lay.step(path, s)

    # warmup: W eager steps
    run_steps(0, W)
    torch.cuda.synchronize()

    # eager rate over the K step slots
    for lay in layers:
        lay.reset()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    run_steps(W, W + K)
    e1.record()
    torch.cuda.synchronize()
    eager_ms = e0.elapsed_time(e1) / K

    if args.eager:
        ms_per_step = eager_ms
        mode = "eager"
    else:
        # capture the K timed steps once, reset the per-step lengths, replay once (timed)
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            run_steps(W, W + K)
        torch.cuda.synchronize()
        for lay in layers:
            lay.reset()
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        g.replay()
        t1.record()
        torch.cuda.synchronize()
        ms_per_step = t0.elapsed_time(t1) / K
        mode = "hip-graph"
        del g

    # tok/s per layer: the real tokens one layer takes per step over the mean time of one
    # layer's hot path (step time / layers); the whole stack passes value / nl tokens/s
    value = tokens_per_layer * nl / (ms_per_step * 1e-3)
    stack_tok_s = tokens_per_layer / (ms_per_step * 1e-3)

    # dominant kernel: the attention call, timed alone (graph of back-to-back launches)
    lay_dom = max(layers, key=lambda l: algorithmic(l.cfg)[1])
    R = args.attn_reps
    attn_ms, _ = time_graph(lambda: [lay_dom.attn_only(cp) for _ in range(R)], R)
    attn_ms /= R
    nbytes, flops = algorithmic(lay_dom.cfg)
    intensity = flops / nbytes
    ridge = (BF16_PEAK_TFLOPS if lay_dom.cfg.dtype == I.BF16 else FP32_PEAK_TFLOPS) * 1e12 / (
        HBM_PEAK_GBS * 1e9)
    if intensity < ridge:
        achieved = nbytes / (attn_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 5)}
    else:
        peak = BF16_PEAK_TFLOPS if lay_dom.cfg.dtype == I.BF16 else FP32_PEAK_TFLOPS
        achieved = flops / (attn_ms * 1e-3) / 1e12
        roof = {"bound": "mfma" if lay_dom.cfg.dtype == I.BF16 else "alu",
                "achieved": round(achieved, 3), "peak": peak, "unit": "TFLOP/s",
                "frac": round(achieved / peak, 5)}
    roof["traffic"] = measured_traffic(args.workload, lay_dom.flags)
    roof["kernel"] = "cp_attn_chunk_with_past"
    roof["avg_launch_us"] = round(attn_ms * 1e3, 3)
    roof["algorithmic_bytes"] = nbytes
    roof["algorithmic_flops"] = flops

    result = {
        "metric": METRIC, "value": round(value, 1), "unit": "tok/s", "n_gpus": 1, "steps": K,
        "warmup": W, "ms_per_step": round(ms_per_step, 6), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": "f32" if cfg0.dtype == I.F32 else "bf16", "data": "synthetic",
        "config": {"workload": f"{args.workload}: {WORKLOADS[args.workload]}",
                   "layers_per_step": nl, "real_tokens_per_layer": tokens_per_layer,
                   "value_is": "real tokens per layer x layers per step / step time",
                   "stack_tok_per_s": round(stack_tok_s, 1),
                   "launch": mode, "eager_ms_per_step": round(eager_ms, 6),
                   "attn_flags": lay_dom.flags,
                   "max_seen": lay_dom.max_seen},
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(layers, args.cpu_seconds)
    print(f"[bench] {args.workload}: {mode} {ms_per_step * 1e3:.2f} us/step, eager "
          f"{eager_ms * 1e3:.2f} us/step, attention {attn_ms * 1e3:.2f} us/launch",
          file=sys.stderr, flush=True)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
