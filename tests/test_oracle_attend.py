"""Pins of oracle.attend / oracle.hca_attend / rmsnorm / rope.

The strongest pin is (i): with every visible compressed entry selected and a
window that covers the whole prefix, CSA core attention must equal dense causal
attention with a sink over [visible compressed entries ; tokens 0..t], built
here with a dense mask over all (query, key) pairs and scipy's softmax.
"""
import numpy as np
import pytest
import torch
from scipy.special import softmax as sp_softmax

import oracle


def test_rmsnorm_unit_rms_and_scale_invariance():
    r = np.random.default_rng(0)
    x = r.standard_normal((10, 64)) * 5
    y = oracle.rmsnorm(x, eps=0.0)
    assert np.allclose(np.sqrt(np.mean(y * y, axis=-1)), 1.0)
    assert np.allclose(oracle.rmsnorm(3.0 * x, eps=0.0), y)
    g = r.uniform(0.5, 2, 64)
    assert np.allclose(oracle.rmsnorm(x, g, eps=0.0), y * g)


def test_rope_complex_form_and_group_property():
    r = np.random.default_rng(1)
    c, rd, base = 16, 8, 10000.0
    x = r.standard_normal((5, c))
    pos = np.array([0.0, 1.0, 7.0, 1000.0, 123456.0])
    y = oracle.rope(x, pos, rd, base)
    # independent complex-number form: pair (2i, 2i+1) of the last rd dims times e^{i pos theta_i}
    th = base ** (-(2.0 * np.arange(rd // 2)) / rd)
    z = x[:, c - rd::2] + 1j * x[:, c - rd + 1::2]
    zr = z * np.exp(1j * pos[:, None] * th)
    assert np.allclose(y[:, c - rd::2], zr.real, atol=1e-12)
    assert np.allclose(y[:, c - rd + 1::2], zr.imag, atol=1e-12)
    assert np.array_equal(y[:, :c - rd], x[:, :c - rd])                  # first c-r dims untouched
    assert np.allclose(oracle.rope(x, 0.0, rd, base), x)
    assert np.allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1))
    assert np.allclose(oracle.rope(oracle.rope(x, 5.0, rd, base), -5.0, rd, base), x, atol=1e-12)
    assert np.allclose(oracle.rope(oracle.rope(x, 3.0, rd, base), 4.0, rd, base), oracle.rope(x, 7.0, rd, base))


def _case(seed=0, n=24, m=4, c=16, H=3, rd=8, n_win=None, B=1):
    r = np.random.default_rng(seed)
    n_win = n if n_win is None else n_win
    N = n // m
    q = r.standard_normal((B, n, H, c))
    comp = r.standard_normal((B, N, c))
    win = r.standard_normal((B, n + n_win - 1, c))
    sink = r.standard_normal(H)
    return q, comp, win, sink, N, n_win


def _dense_reference(q, comp, tokens, sink, m, rd, scale, base, eps=1e-6):
    """Dense causal attention with a sink over [compressed ; tokens] using a full mask matrix."""
    n, H, c = q.shape
    N = comp.shape[0]
    keys = np.concatenate([comp, tokens], axis=0)
    kpos = np.concatenate([m * np.arange(N), np.arange(n)]).astype(np.float64)
    kh = oracle.rope(oracle.rmsnorm(keys, eps=eps), kpos, rd, base)
    t = np.arange(n)
    qh = oracle.rope(oracle.rmsnorm(q, eps=eps), t[:, None].astype(np.float64), rd, base)   # [n][H][c]
    mask = np.zeros((n, N + n), dtype=bool)
    mask[:, :N] = np.arange(N)[None, :] < (t[:, None] // m)
    mask[:, N:] = np.arange(n)[None, :] <= t[:, None]
    logits = scale * np.einsum("thc,kc->thk", qh, kh)
    logits = np.where(mask[:, None, :], logits, -np.inf)
    full = np.concatenate([logits, np.broadcast_to(sink[None, :, None], (n, H, 1))], axis=2)
    P = sp_softmax(full, axis=2)[:, :, :-1]
    o = np.einsum("thk,kc->thc", P, kh)
    return oracle.rope(o, -t[:, None].astype(np.float64), rd, base)


@pytest.mark.parametrize("seed", [0, 1])
def test_full_coverage_equals_dense_causal_attention_with_sink(seed):
    m, rd, base = 4, 8, 10000.0
    q, comp, win, sink, N, n_win = _case(seed)
    n, c = q.shape[1], q.shape[3]
    pos0 = [0]
    k = N
    scores = oracle.index(np.ones((1, n, 1, 1)), np.ones((1, n, 1)), np.ones((1, N, 1)), pos0, m)
    idx = oracle.topk(scores, pos0, m, k)                     # all visible entries
    out = oracle.attend(q, comp, idx, win, sink, pos0, m, n_win, rd, 1 / np.sqrt(c), rope_base=base)
    tokens = win[0, n_win - 1:]
    ref = _dense_reference(q[0], comp[0], tokens, sink, m, rd, 1 / np.sqrt(c), base)
    assert np.allclose(out[0], ref, rtol=1e-11, atol=1e-12)
    hca = oracle.hca_attend(q, comp, win, sink, pos0, m, n_win, rd, 1 / np.sqrt(c), rope_base=base)
    assert np.allclose(hca, out, rtol=1e-12, atol=1e-13)


def test_sink_limits():
    m, rd = 4, 8
    q, comp, win, sink, N, n_win = _case(2, n=16)
    c = q.shape[-1]
    idx = np.tile(np.arange(N, dtype=np.int32), (1, 16, 1))
    idx = np.where(idx < (np.arange(16)[None, :, None] // m), idx, -1)
    big = oracle.attend(q, comp, idx, win, np.full(3, 1e4), [0], m, n_win, rd, 1 / np.sqrt(c))
    assert np.max(np.abs(big)) < 1e-300
    none = oracle.attend(q, comp, idx, win, np.full(3, -1e4), [0], m, n_win, rd, 1 / np.sqrt(c))
    # without a sink every query's weights sum to one: check against torch SDPA with rope off
    none0 = oracle.attend(q, comp, idx, win, np.full(3, -1e4), [0], m, n_win, 0, 1 / np.sqrt(c))
    t = 9
    keys = np.concatenate([comp[0, :t // m], win[0, n_win - 1:n_win + t]], 0)
    qq = torch.from_numpy(oracle.rmsnorm(q[0, t]))[None, :, None, :]          # [1][H][1][c]
    kk = torch.from_numpy(oracle.rmsnorm(keys))[None, None].expand(1, 3, -1, -1).contiguous()
    ref = torch.nn.functional.scaled_dot_product_attention(qq, kk, kk)[0, :, 0].numpy()
    assert np.allclose(none0[0, t], ref, atol=1e-12)
    assert np.isfinite(none).all()


def test_translation_invariance_pins_output_rotation_sign():
    m, rd, base = 4, 8, 10000.0
    q, comp, win, sink, N, n_win = _case(3, n=20, n_win=8)
    c = q.shape[-1]
    r = np.random.default_rng(9)
    T = 20
    idx = np.full((1, T, 3), -1, np.int32)
    for t in range(T):
        vis = t // m
        if vis:
            ch = np.sort(r.choice(vis, size=min(3, vis), replace=False))
            idx[0, t, :len(ch)] = ch
    a = oracle.attend(q, comp, idx, win, sink, [0], m, n_win, rd, 1 / np.sqrt(c), rope_base=base)
    d = 250_000                                    # shift every position by m*d = 1,000,000
    comp2 = np.concatenate([np.zeros((1, d, c)), comp], axis=1)
    idx2 = np.where(idx >= 0, idx + d, -1)
    b = oracle.attend(q, comp2, idx2, win, sink, [m * d], m, n_win, rd, 1 / np.sqrt(c), rope_base=base)
    # window rows of the shifted run: positions m*d - n_win + 1 + j; rows below m*d were clipped at 0 before
    # and are now visible, so compare only the queries whose window never reached below position 0
    ok = np.arange(T) >= n_win - 1
    assert np.allclose(a[0, ok], b[0, ok], atol=1e-9)


def test_output_rotation_sign_has_teeth():
    """Rotating the output by +t instead of -t breaks translation invariance (so the pin above can fail)."""
    rd, base = 8, 10000.0
    r = np.random.default_rng(4)
    e = r.standard_normal((1, 16))
    for sign in (-1.0, +1.0):
        outs = []
        for shift in (0.0, 4000.0):
            t, p = 40.0 + shift, 12.0 + shift
            outs.append(oracle.rope(oracle.rope(e, p, rd, base), sign * t, rd, base))
        same = np.allclose(outs[0], outs[1], atol=1e-9)
        assert same == (sign < 0)


def test_single_entry_closed_form():
    rd, base, c, H = 8, 10000.0, 16, 2
    r = np.random.default_rng(5)
    q = r.standard_normal((1, 1, H, c))
    e = r.standard_normal((1, 1, c))
    sink = np.array([0.3, -1.2])
    t = 37
    win = np.zeros((1, 1, c))          # n_win = 1: window holds only position t ...
    win[0, 0] = r.standard_normal(c)
    # use the window entry as the single entry (no compressed entry selected)
    idx = -np.ones((1, 1, 1), np.int32)
    out = oracle.attend(q, e, idx, win, sink, [t], 4, 1, rd, 1 / np.sqrt(c), rope_base=base)
    eh = oracle.rope(oracle.rmsnorm(win[0, 0]), t, rd, base)
    for h in range(H):
        qh = oracle.rope(oracle.rmsnorm(q[0, 0, h]), t, rd, base)
        z = qh @ eh / np.sqrt(c)
        p = 1.0 / (1.0 + np.exp(sink[h] - z))                 # sigma(z - z')
        ref = oracle.rope(p * eh, -t, rd, base)
        assert np.allclose(out[0, 0, h], ref, atol=1e-13)


def test_window_clipping_and_no_compressed_entries():
    m, rd = 4, 8
    q, comp, win, sink, N, n_win = _case(6, n=8, n_win=4)
    c = q.shape[-1]
    idx = -np.ones((1, 8, 2), np.int32)
    out = oracle.attend(q, comp, idx, win, sink, [0], m, n_win, rd, 1 / np.sqrt(c))
    # query 0 sees only token 0: single-entry closed form
    eh = oracle.rope(oracle.rmsnorm(win[0, n_win - 1]), 0.0, rd, 10000.0)
    qh = oracle.rope(oracle.rmsnorm(q[0, 0, 0]), 0.0, rd, 10000.0)
    p = 1.0 / (1.0 + np.exp(sink[0] - qh @ eh / np.sqrt(c)))
    assert np.allclose(out[0, 0, 0], p * eh, atol=1e-13)


@pytest.mark.parametrize("mode", ["csa", "hca"])
def test_prepared_entries_equal_raw_entries(mode):
    """comp_prepared: handing attend the prepared e^ = RoPE_{m s}(RMSNorm_gamma(e)) of every compressed
    entry gives the raw-entry result (only the place of the preparation moves); a wrong position or a
    missing gain would break it."""
    r = np.random.default_rng(7)
    B, T, H, c, R, m, N, n_win = 2, 3, 4, 32, 8, 4, 40, 5
    q = r.standard_normal((B, T, H, c))
    comp = r.standard_normal((B, N, c))
    win = r.standard_normal((B, T + n_win - 1, c))
    sink = r.standard_normal(H)
    gk = r.uniform(0.5, 1.5, c)
    pos0 = np.array([4 * 30 + 1, 4 * 12])
    prep = oracle.rope(oracle.rmsnorm(comp, gk, 1e-6), m * np.arange(N, dtype=np.float64)[None, :], R, 1e4)
    if mode == "csa":
        idx = np.stack([np.sort(r.choice(min(int(p) // m, N), 6, replace=False)) for p in pos0])[:, None, :]
        idx = np.repeat(idx, T, axis=1)
        a = oracle.attend(q, comp, idx, win, sink, pos0, m, n_win, R, 0.3, gamma_kv=gk)
        b = oracle.attend(q, prep, idx, win, sink, pos0, m, n_win, R, 0.3, gamma_kv=gk, comp_prepared=True)
        wrong = oracle.attend(q, oracle.rmsnorm(comp, gk, 1e-6), idx, win, sink, pos0, m, n_win, R, 0.3,
                              gamma_kv=gk, comp_prepared=True)
    else:
        a = oracle.hca_attend(q, comp, win, sink, pos0, m, n_win, R, 0.3, gamma_kv=gk)
        b = oracle.hca_attend(q, prep, win, sink, pos0, m, n_win, R, 0.3, gamma_kv=gk, comp_prepared=True)
        wrong = oracle.hca_attend(q, oracle.rmsnorm(comp, gk, 1e-6), win, sink, pos0, m, n_win, R, 0.3,
                                  gamma_kv=gk, comp_prepared=True)
    assert np.allclose(a, b, rtol=0, atol=1e-12)
    assert not np.allclose(a, wrong, atol=1e-3)
