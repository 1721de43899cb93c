"""Independent numpy fp64 brute force for tiny shapes (pins the C oracle).

Written separately from the oracle: the cache is modelled as a physical ring
with a write cursor (the cursor advances per appended row and wraps back to
the first non-sink slot), the live set is "whatever the cursor has not yet
overwritten", and attention builds a literal dense mask over absolute
positions and calls a dense softmax.  Only for small inputs.
"""
import numpy as np

MASKED = -1e30


def bf16_bits_to_f64(a):
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def cursor_model(seen, cap, ring, sink):
    """Return {slot: position} after writing positions 0..seen-1 with a cursor."""
    occupant = {}
    cur = 0
    for p in range(seen):
        if not ring and cur >= cap:
            raise OverflowError
        occupant[cur] = p
        cur += 1
        if ring and cur == cap:
            cur = sink
    return occupant


def live_positions(seen, cap, ring, sink):
    occ = cursor_model(seen, cap, ring, sink)
    return sorted(occ.values())


def slot_of(seen_total, cap, ring, sink):
    """position -> slot for every position still live after seen_total writes."""
    occ = cursor_model(seen_total, cap, ring, sink)
    return {p: s for s, p in occ.items()}


def attn(q, kn, vn, kc, vc, seen, n_valid, ring, sink, window, scale, mask=None):
    """Dense masked softmax attention over [live past ; chunk] keys, fp64."""
    q, kn, vn = bf16_bits_to_f64(q), bf16_bits_to_f64(kn), bf16_bits_to_f64(vn)
    kc, vc = bf16_bits_to_f64(kc), bf16_bits_to_f64(vc)
    B, H, C, D = q.shape
    nKV, cap = kc.shape[1], kc.shape[2]
    G = H // nKV
    out = np.zeros((B, H, C, D))
    for b in range(B):
        nv = C if n_valid is None else int(n_valid[b])
        past = live_positions(int(seen[b]), cap, ring, sink)
        where = slot_of(int(seen[b]), cap, ring, sink)
        kpos = np.array(past + [int(seen[b]) + j for j in range(C)], dtype=np.int64)
        real = np.array([True] * len(past) + [j < nv for j in range(C)])
        qpos = int(seen[b]) + np.arange(C)
        allowed = (kpos[None, :] <= qpos[:, None]) & real[None, :]
        if window:
            inwin = (qpos[:, None] - kpos[None, :] < window) | (kpos[None, :] < sink)
            allowed &= inwin
        for h in range(H):
            g = h // G
            K = np.concatenate([kc[b, g, [where[p] for p in past]].reshape(len(past), D),
                                kn[b, g]], axis=0)
            V = np.concatenate([vc[b, g, [where[p] for p in past]].reshape(len(past), D),
                                vn[b, g]], axis=0)
            S = float(scale) * (q[b, h] @ K.T)
            if mask is None:
                S = S + np.where(allowed, 0.0, MASKED)
            else:
                mb = mask[b if mask.shape[0] > 1 else 0, h if mask.shape[1] > 1 else 0]
                S = S + mb[:, :K.shape[0]].astype(np.float64)
            S = S - S.max(axis=1, keepdims=True)
            P = np.exp(S)
            P /= P.sum(axis=1, keepdims=True)
            O = P @ V
            O[nv:] = 0.0
            out[b, h] = O
    return out
