"""Seeded synthetic inputs for the chunked-prefill-with-past path.

This module only draws random tensors and builds the caller-side inputs the
path consumes (per-position cos/sin tables, past lengths, the shapes of the
workloads).  It holds none of the path's arithmetic (no RoPE application, no
mask rule, no attention, no cache update), imports neither the HIP binding
nor the oracle, and is the one module both sides share.

Workloads (the shapes of the pages' workloads, data synthetic, N(0, 1)):
  c1  one fp32 layer, 4 heads / 1 KV head, D 64, 48 cached, chunk 16 with 11
      real rows, global cache, RoPE base 1e4.
  c2  Gemma-270M-like global layer ([SKaiNET] "Validation": an 800-position
      cache plus a 52-token chunk padded to C = 64, select row 51), bf16,
      4 heads / 1 KV head, D 256, base 1e6, explicit per-head mask.
  c3  sliding-window ring (window 512) that has absorbed 1023 positions, a
      127-token tail padded to C = 128 ([cactus] "Problem": a 1023-token
      prompt), bf16, 8 heads / 1 KV head, D 256, base 1e4.
  c4  Llama-8B-like GQA layer, batch 16, past lengths uniform in [0, 4095],
      C = 128, 32 heads / 8 KV heads, D 128, base 5e5.
  c5  long context, batch 4, 32768 past positions, C = 512, 32 / 8 heads,
      D 128; five sliding layers (window 4096, base 1e4) and one global
      layer (base 1e6).

The pages' own prompts, weights and bundles are not available; these seeded
tensors stand in for them.
"""
from dataclasses import dataclass
from typing import List, Optional

import numpy as np
import torch

F32, BF16 = 0, 1


@dataclass
class LayerCfg:
    name: str
    dtype: int            # F32 or BF16
    B: int
    H: int
    nKV: int
    D: int
    C: int
    cap: int
    ring: int = 0
    sink: int = 0
    window: int = 0
    base: float = 1e4
    seen: Optional[List[int]] = None     # per-sequence absorbed positions
    n_valid: Optional[List[int]] = None  # per-sequence real rows
    explicit_mask: bool = False
    select: bool = True
    seed: int = 0
    layer: int = 0

    @property
    def G(self):
        return self.H // self.nKV

    @property
    def scale(self):
        return float(np.float32(1.0 / np.sqrt(self.D)))

    def live_count(self, b):
        s = self.seen[b]
        return min(s, self.cap) if self.ring else s

    def mask_ld(self):
        return max(self.live_count(b) for b in range(self.B)) + self.C


def _c4_past(seed: int) -> List[int]:
    g = torch.Generator("cpu").manual_seed(seed)
    return [int(x) for x in torch.randint(0, 4096, (16,), generator=g)]


def config(name: str, layer: int = 0) -> LayerCfg:
    """The layer configuration of workload `name` (c1..c5); c5 has layers 0..5."""
    if name == "c1":
        return LayerCfg("c1", F32, 1, 4, 1, 64, 16, 64, base=1e4, seen=[48], n_valid=[11],
                        explicit_mask=True, seed=1001)
    if name == "c2":
        return LayerCfg("c2", BF16, 1, 4, 1, 256, 64, 1024, base=1e6, seen=[800], n_valid=[52],
                        explicit_mask=True, seed=1002)
    if name == "c3":
        return LayerCfg("c3", BF16, 1, 8, 1, 256, 128, 512, ring=1, sink=0, window=512, base=1e4,
                        seen=[1023], n_valid=[127], seed=1003)
    if name == "c4":
        return LayerCfg("c4", BF16, 16, 32, 8, 128, 128, 4224, base=5e5, seen=_c4_past(1004),
                        n_valid=[128] * 16, seed=1004)
    if name == "c5":
        if not 0 <= layer <= 5:
            raise ValueError("c5 has layers 0..5")
        if layer < 5:
            return LayerCfg("c5", BF16, 4, 32, 8, 128, 512, 4096, ring=1, sink=0, window=4096,
                            base=1e4, seen=[32768] * 4, n_valid=[512] * 4, seed=1005,
                            layer=layer)
        return LayerCfg("c5", BF16, 4, 32, 8, 128, 512, 33280, base=1e6, seen=[32768] * 4,
                        n_valid=[512] * 4, seed=1005, layer=5)
    raise ValueError(f"unknown workload {name}")


@dataclass
class GdnCfg:
    """A gated-delta-rule prefill workload ([Kazeia] "Chantier 4": head size 64 over 256
    tokens is the page's kernel test; 128-wide states over a 512-token prompt its pp512
    benchmark)."""
    name: str
    B: int
    H: int
    P: int
    dk: int
    dv: int
    seed: int


def gdn_config(name: str) -> GdnCfg:
    if name == "g0":
        return GdnCfg("g0", 1, 4, 256, 64, 64, 2001)
    if name == "g1":
        return GdnCfg("g1", 1, 16, 512, 128, 128, 2002)
    raise ValueError(f"unknown gated-delta-rule workload {name}")


def make_gdn(cfg: GdnCfg, P: Optional[int] = None):
    """Draws for a gated-delta-rule prefill (fp32, CPU): q and k N(0,1) with unit-norm keys
    (k / |k|, as the layer normalises them), v N(0,1), beta = sigmoid(N(0,1)), log-gates
    alpha = -softplus(N(0,1) - 2) (gates between about 0.3 and 1), entry state
    N(0,1) * 0.1.  Order of draws from Generator(seed): q, k, v, beta, alpha, state."""
    g = torch.Generator("cpu").manual_seed(cfg.seed)
    P = cfg.P if P is None else P
    B, H, dk, dv = cfg.B, cfg.H, cfg.dk, cfg.dv
    q = torch.randn((B, H, P, dk), generator=g)
    k = torch.randn((B, H, P, dk), generator=g)
    k = k / k.norm(dim=-1, keepdim=True)
    v = torch.randn((B, H, P, dv), generator=g)
    beta = torch.sigmoid(torch.randn((B, H, P), generator=g))
    alpha = -torch.nn.functional.softplus(torch.randn((B, H, P), generator=g) - 2)
    state = torch.randn((B, H, dk, dv), generator=g) * 0.1
    return dict(q=q, k=k, v=v, beta=beta, alpha=alpha, state=state)


def derived(name: str, B: Optional[int] = None, C: Optional[int] = None,
            explicit_mask: Optional[bool] = None) -> LayerCfg:
    """A workload's per-sequence shape at another batch or chunk size (the bandwidth
    sweep): c2 at batch B (every sequence 800 cached, 52 of 64 rows real), c4 (its 16
    seeded past lengths) and the c5 global layer at chunk C (all rows real)."""
    if name == "c2":
        cfg = config("c2")
        nb = B or cfg.B
        cfg.B, cfg.seen, cfg.n_valid = nb, [800] * nb, [52] * nb
    elif name == "c4":
        cfg = config("c4")
        c = C or cfg.C
        cfg.C, cfg.cap, cfg.n_valid = c, 4096 + c, [c] * cfg.B
    elif name == "c5g":
        cfg = config("c5", 5)
        c = C or cfg.C
        cfg.C, cfg.n_valid = c, [c] * cfg.B
    else:
        raise ValueError(f"no derived shapes of {name}")
    if explicit_mask is not None:
        cfg.explicit_mask = explicit_mask
    return cfg


def rope_tables(cfg: LayerCfg):
    """Caller-side per-position cos/sin tables [Bt, C, D] (fp32).

    Chunk row i of sequence b sits at absolute position seen[b] + i.  Angles
    are pos * base**(-2j/D) for j < D/2 in fp64, duplicated over both halves
    of the head (half-split pairing), then rounded to fp32.  Bt = 1 when all
    sequences share their positions, else B.
    """
    same = all(s == cfg.seen[0] for s in cfg.seen)
    seqs = [cfg.seen[0]] if same else list(cfg.seen)
    j = np.arange(cfg.D // 2, dtype=np.float64)
    inv = cfg.base ** (-2.0 * j / cfg.D)
    cos = np.empty((len(seqs), cfg.C, cfg.D), dtype=np.float32)
    sin = np.empty_like(cos)
    for t, s in enumerate(seqs):
        pos = (s + np.arange(cfg.C, dtype=np.float64))[:, None]
        ang = pos * inv[None, :]
        c, si = np.cos(ang), np.sin(ang)
        cos[t] = np.concatenate([c, c], axis=1).astype(np.float32)
        sin[t] = np.concatenate([si, si], axis=1).astype(np.float32)
    return torch.from_numpy(cos), torch.from_numpy(sin)


def _cast(t: torch.Tensor, dtype: int) -> torch.Tensor:
    return t if dtype == F32 else t.to(torch.bfloat16)


def dead_slots(cfg: LayerCfg, b: int) -> np.ndarray:
    """Boolean [cap]: physical slots that hold no live row for sequence b.

    A global cache holds positions [0, seen) in slots [0, seen).  A ring whose
    sequence has absorbed fewer than cap positions holds them in slots
    [0, seen); once it has absorbed cap or more, every slot is live.
    """
    dead = np.zeros(cfg.cap, dtype=bool)
    s = cfg.seen[b]
    if s < cfg.cap:
        dead[s:] = True
    return dead


def make_layer(cfg: LayerCfg, nan_dead: bool = True):
    """Draw one layer's inputs on the CPU.

    Order of draws from Generator(seed + 17 * layer): q [B,H,C,D],
    k [B,nKV,C,D], v [B,nKV,C,D], k cache [B,nKV,cap,D], v cache, all N(0,1)
    fp32, then rounded (RNE) to the storage dtype.  Dead cache slots are set
    to NaN when nan_dead, so that any read of them poisons the result.
    """
    g = torch.Generator("cpu").manual_seed(cfg.seed + 17 * cfg.layer)
    B, H, nKV, C, D, cap = cfg.B, cfg.H, cfg.nKV, cfg.C, cfg.D, cfg.cap
    q = _cast(torch.randn((B, H, C, D), generator=g), cfg.dtype)
    k = _cast(torch.randn((B, nKV, C, D), generator=g), cfg.dtype)
    v = _cast(torch.randn((B, nKV, C, D), generator=g), cfg.dtype)
    kc = _cast(torch.randn((B, nKV, cap, D), generator=g), cfg.dtype)
    vc = _cast(torch.randn((B, nKV, cap, D), generator=g), cfg.dtype)
    if nan_dead:
        for b in range(B):
            dead = torch.from_numpy(dead_slots(cfg, b))
            if dead.any():
                kc[b][:, dead] = float("nan")
                vc[b][:, dead] = float("nan")
    cos, sin = rope_tables(cfg)
    return dict(q=q, k=k, v=v, kc=kc, vc=vc, cos=cos, sin=sin,
                seen=torch.tensor(cfg.seen, dtype=torch.int32),
                n_valid=torch.tensor(cfg.n_valid if cfg.n_valid else [C] * B, dtype=torch.int32))


def small(name="tiny", dtype=BF16, B=2, H=4, nKV=2, D=64, C=16, cap=96, ring=0, sink=0, window=0,
          seen=None, n_valid=None, base=1e4, seed=7, explicit_mask=False) -> LayerCfg:
    """A small configuration for parity tests (sizes the oracle finishes in seconds)."""
    if seen is None:
        seen = [min(cap - C, 40 + 7 * b) if not ring else 50 + 31 * b for b in range(B)]
    if n_valid is None:
        n_valid = [max(1, C - 3 * b) for b in range(B)]
    return LayerCfg(name, dtype, B, H, nKV, D, C, cap, ring=ring, sink=sink, window=window,
                    base=base, seen=list(seen), n_valid=list(n_valid),
                    explicit_mask=explicit_mask, seed=seed)


def np_view(t: torch.Tensor) -> np.ndarray:
    """CPU tensor -> numpy array the oracle accepts (bf16 as uint16 bit patterns)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def from_np(a: np.ndarray) -> torch.Tensor:
    """Inverse of np_view."""
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16)
    return torch.from_numpy(a.copy())
