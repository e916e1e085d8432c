"""Pins of oracle.compress against hand-worked values, closed forms and invariants."""
import json
import os

import numpy as np
import pytest
from scipy.special import softmax as sp_softmax

import oracle
from oracle.csa import compress_weights

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _arr(x):
    return np.asarray(x, np.float64).reshape(1, -1, 1)


def test_hand_worked_cases():
    cases = json.load(open(os.path.join(GOLD, "compress_hand.json")))["cases"]
    for cs in cases:
        m = cs["m"]
        n = len(cs["ca"]) // m
        out = oracle.compress(_arr(cs["ca"]), _arr(cs["cb"]), _arr(cs["za"]), _arr(cs["zb"]),
                              np.asarray(cs["bias_a"], np.float64).reshape(m, 1),
                              np.asarray(cs["bias_b"], np.float64).reshape(m, 1), m, 0, 0, n)[0, :, 0]
        if "expected" in cs:
            assert np.allclose(out, cs["expected"], rtol=1e-14, atol=0), (out, cs["expected"])
        else:
            assert abs(out[1] - cs["expected_entry1"]) < 1e-14


def _rand(B=2, rows=24, c=5, m=4, seed=0):
    r = np.random.default_rng(seed)
    return [r.standard_normal((B, rows, c)) for _ in range(4)] + [r.standard_normal((m, c)) for _ in range(2)]


def test_weights_sum_to_one_per_channel():
    ca, cb, za, zb, ba, bb = _rand()
    for i in range(6):
        S = compress_weights(za, zb, ba, bb, 4, 0, i)
        assert S.shape[0] == 8
        if i == 0:
            assert np.all(S[4:] == 0.0)      # padded b-logits are -inf
        assert np.allclose(S.sum(axis=0), 1.0, atol=1e-15)
        assert np.all(S >= 0)
    S = compress_weights(za, None, ba, None, 4, 0, 3)
    assert np.allclose(S.sum(axis=0), 1.0, atol=1e-15)


def test_equal_logits_give_block_means():
    ca, cb, za, zb, _, _ = _rand()
    z0 = np.zeros_like(za)
    b0 = np.zeros((4, 5))
    out = oracle.compress(ca, cb, z0, z0, b0, b0, 4, 0, 0, 6)
    assert np.allclose(out[:, 0], ca[:, 0:4].mean(axis=1), atol=1e-14)         # i = 0: a-rows only
    for i in range(1, 6):
        ref = np.concatenate([ca[:, 4 * i:4 * i + 4], cb[:, 4 * (i - 1):4 * i]], axis=1).mean(axis=1)
        assert np.allclose(out[:, i], ref, atol=1e-14)


def test_dominant_logit_selects_its_row():
    ca, cb, za, zb, ba, bb = _rand()
    za2, zb2 = za.copy(), zb.copy()
    za2[:, 4 * 2 + 3, :] = 1e9          # entry 2: a-row r=3 dominates
    zb2[:, 4 * 3 + 1, :] = 1e9          # entry 4: b-row r=1 (token 13) dominates (a-rows 16..19 are ordinary)
    out = oracle.compress(ca, cb, za2, zb2, ba, bb, 4, 0, 0, 6)
    assert np.array_equal(out[:, 2], ca[:, 11])
    assert np.array_equal(out[:, 4], cb[:, 13])


def test_b_stream_minus_inf_reduces_to_hca_with_m_equal_m():
    ca, cb, za, zb, ba, bb = _rand()
    zneg = np.full_like(zb, -np.inf)
    csa = oracle.compress(ca, cb, za, zneg, ba, bb, 4, 0, 0, 6)
    hca = oracle.compress(ca, None, za, None, ba, None, 4, 0, 0, 6)
    assert np.allclose(csa, hca, atol=1e-15)


def test_matches_library_softmax_on_stacked_windows():
    ca, cb, za, zb, ba, bb = _rand(B=3, rows=40, c=7, m=4, seed=3)
    m = 4
    out = oracle.compress(ca, cb, za, zb, ba, bb, m, 0, 0, 10)
    # rebuild every window as one [B, 2m, c] block via reshapes, then scipy's softmax over axis 1
    za_b = za.reshape(3, 10, m, 7) + ba
    zb_b = zb.reshape(3, 10, m, 7) + bb
    ca_b = ca.reshape(3, 10, m, 7)
    cb_b = cb.reshape(3, 10, m, 7)
    zb_prev = np.concatenate([np.full((3, 1, m, 7), -np.inf), zb_b[:, :-1]], axis=1)
    cb_prev = np.concatenate([np.zeros((3, 1, m, 7)), cb_b[:, :-1]], axis=1)
    L = np.concatenate([za_b, zb_prev], axis=2)
    V = np.concatenate([ca_b, cb_prev], axis=2)
    ref = (sp_softmax(L, axis=2) * V).sum(axis=2)
    assert np.allclose(out, ref, rtol=1e-13, atol=1e-13)


def test_b_rows_come_from_previous_block_only():
    ca, cb, za, zb, ba, bb = _rand()
    base = oracle.compress(ca, cb, za, zb, ba, bb, 4, 0, 0, 6)
    cb2 = cb.copy()
    cb2[:, 8:12] += 1.0                  # b-rows of block 2
    out = oracle.compress(ca, cb2, za, zb, ba, bb, 4, 0, 0, 6)
    changed = np.abs(out - base).max(axis=(0, 2)) > 0
    assert list(changed) == [False, False, False, True, False, False]


def test_row_offset_and_first_entry():
    ca, cb, za, zb, ba, bb = _rand(rows=24)
    full = oracle.compress(ca, cb, za, zb, ba, bb, 4, 0, 0, 6)
    # hand the kernel only tokens 8..23 (row0_pos = 8) and ask for entries 3..5
    part = oracle.compress(ca[:, 8:], cb[:, 8:], za[:, 8:], zb[:, 8:], ba, bb, 4, 8, 3, 3)
    assert np.allclose(part, full[:, 3:6], atol=0)


@pytest.mark.parametrize("mm", [8, 128])
def test_hca_is_block_softmax(mm):
    r = np.random.default_rng(mm)
    ca = r.standard_normal((1, 2 * mm, 3))
    za = r.standard_normal((1, 2 * mm, 3))
    bias = r.standard_normal((mm, 3))
    out = oracle.compress(ca, None, za, None, bias, None, mm, 0, 0, 2)
    for i in range(2):
        w = sp_softmax(za[0, i * mm:(i + 1) * mm] + bias, axis=0)
        assert np.allclose(out[0, i], (w * ca[0, i * mm:(i + 1) * mm]).sum(0), atol=1e-14)
