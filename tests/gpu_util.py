"""Helpers for the GPU parity tests: upload seeded host arrays, compare against the oracle."""
from __future__ import annotations

import numpy as np
import torch

import oracle

DEV = "cuda:0"


def dev(x: np.ndarray, fmt: str = None):
    """Host storage array -> device tensor (uint16 bf16 bits become torch.bfloat16)."""
    if x is None:
        return None
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(x).to(DEV)


def host_f64(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return oracle.decode_bf16(t.view(torch.int16).cpu().numpy().view(np.uint16))
    return t.cpu().numpy().astype(np.float64)


def values(x: np.ndarray, fmt: str) -> np.ndarray:
    """Exact float64 values of a host storage array (data only, no scales)."""
    if fmt == "bf16":
        return oracle.decode_bf16(x)
    return np.asarray(x, np.float64)


def rel_l2(got: np.ndarray, ref: np.ndarray) -> float:
    num = np.linalg.norm((got - ref).ravel())
    den = np.linalg.norm(ref.ravel())
    return float(num / den) if den > 0 else float(num)


def topk_agreement(gpu_idx, ref_idx, ref_scores, k_rows_tau_rule=1e-3):
    """Set agreement between two [..., k] index arrays with the gap rule.

    Returns (agreement fraction, number of mismatches outside the gap rule).
    ref_scores holds the oracle's float64 scores of each row.
    """
    g = gpu_idx.reshape(-1, gpu_idx.shape[-1])
    r = ref_idx.reshape(-1, ref_idx.shape[-1])
    s = ref_scores.reshape(-1, ref_scores.shape[-1])
    inter = total = bad = 0
    for row in range(g.shape[0]):
        rs = set(int(x) for x in r[row] if x >= 0)
        gs = set(int(x) for x in g[row] if x >= 0)
        inter += len(rs & gs)
        total += len(rs)
        if rs == gs:
            continue
        sel = sorted(rs, key=lambda j: s[row, j])
        tau = s[row, sel[0]]
        tol = k_rows_tau_rule * (abs(tau) if tau != 0 else np.max(np.abs(s[row][np.isfinite(s[row])])))
        for j in gs - rs:
            if not (tau - s[row, j] <= tol):
                bad += 1
        for j in rs - gs:
            if not (s[row, j] - tau <= tol):
                bad += 1
    return inter / max(total, 1), bad


def codes_close(got_codes, ref_codes, ref_vals_scaled, table):
    """Codes must match except where the exact value sits within 1e-5 (relative) of a rounding midpoint."""
    mism = got_codes != ref_codes
    if not mism.any():
        return True
    a = np.abs(ref_vals_scaled[mism])
    lo = np.abs(table[ref_codes[mism] & (0x7F if len(table) == 256 else 0x7)])
    hi = np.abs(table[got_codes[mism] & (0x7F if len(table) == 256 else 0x7)])
    mid = 0.5 * (lo + hi)
    return bool(np.all(np.abs(a - mid) <= 1e-5 * np.maximum(mid, 1e-30)))


def score_keys(x32):
    """The header's order-preserving uint32 key of float32 scores (+0 and -0 share a key)."""
    u = np.ascontiguousarray(x32, np.float32).view(np.uint32).copy()
    u[(u << np.uint32(1)) == 0] = 0
    neg = (u & np.uint32(0x80000000)) != 0
    return np.where(neg, ~u, u | np.uint32(0x80000000)).astype(np.uint32)


def host_bound(scores32, pos0, m):
    """Bound keys as the decode csa_index kernel lays them out: for each bound set, the keys of its two largest
    visible scores (0 where the set has fewer).  Sets split each run of 256 entries: the whole run when the
    cache holds more than 65536 entries, else the eight sets {e : e mod 64 in [8 r, 8 r + 8)}."""
    B, T, N = scores32.shape
    runs = 4 * ((N + 1023) // 1024)
    sets = 1 if N > 65536 else 8
    out = np.zeros((B, T, 2 * runs * sets), np.uint32)
    keys = score_keys(scores32)
    for b in range(B):
        for r in range(T):
            vis = min((pos0[b] + r) // m, N)
            for u in range(runs):
                e = np.arange(256 * u, min(256 * u + 256, vis))
                for s in range(sets):
                    sel = e if sets == 1 else e[(e % 64) // 8 == s]
                    kk = np.sort(keys[b, r, sel])[::-1]
                    j = u * sets + s
                    out[b, r, 2 * j:2 * j + min(2, len(kk))] = kk[:2]
    return out


def host_bound_prefill(scores32, pos0, m):
    """Bound keys as the tiled prefill csa_index kernel lays them out: set j is entries [32 j, 32 j + 32) when
    the cache holds at most 65536 entries, else [256 j, 256 j + 256); its two largest visible keys at 2 j and
    2 j + 1 (0 where it has fewer), every later position 0.  The row length is that of host_bound."""
    B, T, N = scores32.shape
    nb = 2 * 4 * (1 if N > 65536 else 8) * ((N + 1023) // 1024)
    size = 256 if N > 65536 else 32
    out = np.zeros((B, T, nb), np.uint32)
    keys = score_keys(scores32)
    for b in range(B):
        for r in range(T):
            vis = min((pos0[b] + r) // m, N)
            for j in range((vis + size - 1) // size):
                kk = np.sort(keys[b, r, size * j:min(size * j + size, vis)])[::-1]
                out[b, r, 2 * j:2 * j + min(2, len(kk))] = kk[:2]
    return out
