"""Float64 CPU oracle of the CSA/HCA layer step -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline leg
may import this module.  It is deliberately plain: explicit loops over entries
and query rows, numpy float64 for the inner vector algebra, no blocking, no
online softmax, no fusion.  Equations are restated from
"【论文解读】DeepSeek-V4" (wkq9411.github.io), section 一(三) "混合注意力架构：CSA + HCA"
(cited below as [CSA] / [HCA] / [details] by subsection).

Readings where the pages are silent (each is an argument here, not a constant
hidden in code): softmax scale = 1/sqrt(c); RMSNorm eps = 1e-6 with the mean over
all c dims, norm before RoPE; RoPE on adjacent pairs (2i, 2i+1) of the last r
dims with theta_i = base^(-2i/r); a compressed entry s sits at position m*s;
the window is positions t-n_win+1 .. t clipped at 0; query t sees compressed
entries s < floor(t/m); top-k ties go to the lower index and the index list is
returned in ascending order padded with -1.
"""
from __future__ import annotations

import numpy as np


# ---------------------------------------------------------------------------
# compression  ([CSA] (1) "压缩 KV Entries" and [HCA] (1))
# ---------------------------------------------------------------------------
def compress(ca, cb, za, zb, bias_a, bias_b, m, row0_pos, first_entry, num_entries):
    """Compressed entries C^Comp_i for i = first_entry .. first_entry+num_entries-1.

    [CSA] (1): for entry i and channel j the 2m logits are
    Z^a[mi+r, j] + B^a[r, j] (r < m) and Z^b[m(i-1)+r, j] + B^b[r, j]; a softmax
    over those 2m values gives S^a, S^b and C^Comp_i = sum S^a * C^a + sum S^b * C^b.
    For i = 0 the b-logits are -inf and the b-values 0.  HCA (cb is None): one
    stream, m' rows per entry, no overlap ([HCA] (1)).

    Inputs are float64 arrays [B][rows][c]; row r holds absolute position row0_pos + r.
    """
    ca = np.asarray(ca, dtype=np.float64)
    za = np.asarray(za, dtype=np.float64)
    hca = cb is None
    B, rows, c = ca.shape
    out = np.zeros((B, num_entries, c), dtype=np.float64)
    for e in range(num_entries):
        i = first_entry + e
        ra = m * i - row0_pos                     # first a-row of entry i
        logits = [za[:, ra + r, :] + bias_a[r] for r in range(m)]
        values = [ca[:, ra + r, :] for r in range(m)]
        if not hca:
            for r in range(m):
                if i == 0:
                    logits.append(np.full((B, c), -np.inf))
                    values.append(np.zeros((B, c)))
                else:
                    rb = m * (i - 1) - row0_pos + r
                    logits.append(np.asarray(zb[:, rb, :], np.float64) + bias_b[r])
                    values.append(np.asarray(cb[:, rb, :], np.float64))
        L = np.stack(logits)                      # [2m or m', B, c]
        V = np.stack(values)
        mx = np.max(L, axis=0)
        ex = np.exp(L - mx)
        S = ex / np.sum(ex, axis=0)               # softmax over the rows, per channel
        out[:, e, :] = np.sum(S * V, axis=0)
    return out


def compress_weights(za, zb, bias_a, bias_b, m, row0_pos, i):
    """The softmax weights [2m or m', B, c] of entry i (exposed for the sum-to-one pin)."""
    za = np.asarray(za, dtype=np.float64)
    ra = m * i - row0_pos
    logits = [za[:, ra + r, :] + bias_a[r] for r in range(m)]
    if zb is not None:
        for r in range(m):
            if i == 0:
                logits.append(np.full(za[:, 0, :].shape, -np.inf))
            else:
                logits.append(np.asarray(zb[:, m * (i - 1) - row0_pos + r, :], np.float64) + bias_b[r])
    L = np.stack(logits)
    ex = np.exp(L - np.max(L, axis=0))
    return ex / np.sum(ex, axis=0)


# ---------------------------------------------------------------------------
# lightning indexer  ([CSA] (2) "Lightning Indexer 稀疏选择")
# ---------------------------------------------------------------------------
def index(qI, w, kI, pos0, m, n_max=None):
    """Index scores I[b, t, s] = sum_h w[b,t,h] * ReLU(q^I[b,t,h] . K^IComp[b,s]).

    Defined for s < floor(t/m) with t = pos0[b] + row; every other s gets -inf.
    qI: [B][T][HI][cI] float64 (exact dequantized values), w: [B][T][HI],
    kI: [B][N][cI].  Returns float64 [B][T][N].
    """
    qI = np.asarray(qI, np.float64)
    kI = np.asarray(kI, np.float64)
    w = np.asarray(w, np.float64)
    B, T, HI, cI = qI.shape
    N = kI.shape[1] if n_max is None else n_max
    out = np.full((B, T, N), -np.inf)
    for b in range(B):
        for r in range(T):
            t = int(pos0[b]) + r
            vis = min(t // m, N)
            if vis == 0:
                continue
            dots = qI[b, r] @ kI[b, :vis].T               # [HI, vis]
            out[b, r, :vis] = w[b, r] @ np.maximum(dots, 0.0)
    return out


# ---------------------------------------------------------------------------
# top-k selector  ([CSA] (2), the Top-k equation for C^SprsComp_t)
# ---------------------------------------------------------------------------
def topk(scores, pos0, m, k):
    """Indices of the min(k, floor(t/m)) best visible entries, ascending, padded with -1.

    Order: larger score first; equal scores (including +0 and -0) go to the lower index.
    """
    scores = np.asarray(scores, np.float64)
    B, T, N = scores.shape
    idx = np.full((B, T, k), -1, dtype=np.int32)
    for b in range(B):
        for r in range(T):
            vis = min((int(pos0[b]) + r) // m, N)
            row = scores[b, r, :vis] + 0.0                 # -0.0 + 0.0 == +0.0
            order = sorted(range(vis), key=lambda s: (-row[s], s))
            chosen = sorted(order[:min(k, vis)])
            idx[b, r, :len(chosen)] = chosen
    return idx


# ---------------------------------------------------------------------------
# core attention pieces  ([details] (1) RMSNorm, (2) partial RoPE, (4) sink)
# ---------------------------------------------------------------------------
def rmsnorm(x, gamma=None, eps=1e-6):
    """x / sqrt(mean(x^2) + eps) * gamma over the last axis."""
    x = np.asarray(x, np.float64)
    y = x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    return y if gamma is None else y * np.asarray(gamma, np.float64)


def rope_thetas(rope_dims, base):
    return base ** (-np.arange(0, rope_dims, 2, dtype=np.float64) / rope_dims)


def rope(x, pos, rope_dims, base):
    """Rotate pairs (c-r+2i, c-r+2i+1) of the last axis by angle pos * theta_i.

    x: [..., c]; pos: scalar or array broadcastable to x.shape[:-1].
    """
    x = np.array(x, dtype=np.float64, copy=True)
    if rope_dims == 0:
        return x
    c = x.shape[-1]
    th = rope_thetas(rope_dims, base)
    ang = np.asarray(pos, np.float64)[..., None] * th          # [..., r/2]
    cs, sn = np.cos(ang), np.sin(ang)
    x0 = x[..., c - rope_dims::2].copy()
    x1 = x[..., c - rope_dims + 1::2].copy()
    x[..., c - rope_dims::2] = x0 * cs - x1 * sn
    x[..., c - rope_dims + 1::2] = x0 * sn + x1 * cs
    return x


def _core_attention(q_rows, entries, entry_pos, t, sink, gamma_q, gamma_kv, rope_dims, scale, eps, base,
                    n_given=0):
    """One query position t, all heads: o_h = RoPE_{-t}(sum_j p_hj e^_j).

    q_rows [H][c]; entries [L][c] (raw KV, except that the first n_given rows are already the prepared
    e^ = RoPE_pos(RMSNorm(e))); entry_pos [L].
    p_hj = exp(z_hj) / (sum_j' exp(z_hj') + exp(z'_h)),  z_hj = scale * q^_h . e^_j.
    """
    qh = rope(rmsnorm(q_rows, gamma_q, eps), t, rope_dims, base)          # [H][c]
    if len(entries) == 0:
        return np.zeros_like(qh)
    entries = np.asarray(entries, np.float64)
    raw = rope(rmsnorm(entries[n_given:], gamma_kv, eps), np.asarray(entry_pos)[n_given:], rope_dims, base)
    eh = np.concatenate([entries[:n_given], raw], axis=0)                 # [L][c]
    z = scale * (qh @ eh.T)                                               # [H][L]
    zs = np.asarray(sink, np.float64)[:, None]
    M = np.maximum(np.max(z, axis=1, keepdims=True), zs)
    ez = np.exp(z - M)
    denom = np.sum(ez, axis=1, keepdims=True) + np.exp(zs - M)
    o = (ez / denom) @ eh                                                 # [H][c]
    return rope(o, -t, rope_dims, base)


def _window(win_kv_b, t, pos0_b, n_win):
    """Window entries for position t: positions max(0, t-n_win+1) .. t."""
    lo = max(0, t - n_win + 1)
    rows = np.arange(lo, t + 1) - (pos0_b - n_win + 1)
    return np.asarray(win_kv_b, np.float64)[rows], np.arange(lo, t + 1, dtype=np.float64)


def attend(q, comp_kv, idx, win_kv, sink, pos0, m, n_win, rope_dims, scale, eps=1e-6, rope_base=10000.0,
           gamma_q=None, gamma_kv=None, rows=None, comp_prepared=False):
    """CSA core attention ([CSA] (3) shared key-value MQA, plus [details] (1)-(4)).

    Entries for query t: the selected compressed entries C^Comp[s] (s in idx[t],
    -1 skipped, position m*s) followed by the window tokens.  Every entry is both
    key and value.  q [B][T][H][c], comp_kv [B][N][c], idx [B][T][k],
    win_kv [B][T+n_win-1][c].  Returns float64 [B][T][H][c] (rows: optional list
    of (b, r) pairs to evaluate; the others stay zero).  comp_prepared: comp_kv
    holds the prepared e^ of each entry (its RMSNorm and RoPE at m*s already applied).
    """
    q = np.asarray(q, np.float64)
    B, T, H, c = q.shape
    out = np.zeros((B, T, H, c))
    todo = [(b, r) for b in range(B) for r in range(T)] if rows is None else rows
    for b, r in todo:
        t = int(pos0[b]) + r
        sel = [int(s) for s in idx[b, r] if s >= 0]
        ce = np.asarray(comp_kv[b, sel], np.float64).reshape(len(sel), c)
        we, wp = _window(win_kv[b], t, int(pos0[b]), n_win)
        ents = np.concatenate([ce, we], axis=0)
        epos = np.concatenate([m * np.asarray(sel, np.float64), wp])
        out[b, r] = _core_attention(q[b, r], ents, epos, t, sink, gamma_q, gamma_kv, rope_dims, scale, eps,
                                    rope_base, len(sel) if comp_prepared else 0)
    return out


def hca_attend(q, comp_kv, win_kv, sink, pos0, m_hca, n_win, rope_dims, scale, eps=1e-6, rope_base=10000.0,
               gamma_q=None, gamma_kv=None, rows=None, comp_prepared=False):
    """HCA core attention ([HCA] (2)): dense over every visible entry s < floor(t/m'), plus the window
    (comp_prepared as in attend)."""
    q = np.asarray(q, np.float64)
    B, T, H, c = q.shape
    N = comp_kv.shape[1]
    out = np.zeros((B, T, H, c))
    todo = [(b, r) for b in range(B) for r in range(T)] if rows is None else rows
    for b, r in todo:
        t = int(pos0[b]) + r
        vis = min(t // m_hca, N)
        ce = np.asarray(comp_kv[b, :vis], np.float64)
        we, wp = _window(win_kv[b], t, int(pos0[b]), n_win)
        ents = np.concatenate([ce, we], axis=0)
        epos = np.concatenate([m_hca * np.arange(vis, dtype=np.float64), wp])
        out[b, r] = _core_attention(q[b, r], ents, epos, t, sink, gamma_q, gamma_kv, rope_dims, scale, eps,
                                    rope_base, vis if comp_prepared else 0)
    return out
