"""Shared helpers of the GPU parity tests (HIP path through the C-ABI vs the oracle)."""
import numpy as np
import torch

from chunked_prefill_attention_rope_amd import inputs as I

TOL = {I.F32: 1e-4, I.BF16: 2e-2}


def dev(t):
    return t.to("cuda")


def rowwise_rel_err(got, ref, rows_mask=None):
    """max over rows of max_d |got - ref| / max_d |ref|  (rows = all leading dims)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = np.abs(got - ref).max(axis=-1)
    scale = np.abs(ref).max(axis=-1)
    scale = np.where(scale == 0, 1.0, scale)
    rel = err / scale
    if rows_mask is not None:
        rel = rel[rows_mask]
    return float(rel.max()) if rel.size else 0.0


def real_rows_mask(cfg, shape):
    B, H, C = shape[:3]
    m = np.zeros((B, H, C), dtype=bool)
    for b in range(B):
        m[b, :, :cfg.n_valid[b]] = True
    return m


def to_f64(t):
    return t.detach().float().cpu().double().numpy()


def bits(t):
    """Raw bytes of a tensor (bit-exact comparisons)."""
    t = t.detach().cpu().contiguous()
    return t.view(torch.uint8).numpy() if t.dtype != torch.uint8 else t.numpy()
