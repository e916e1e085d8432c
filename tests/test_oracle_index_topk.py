"""Pins of oracle.index and oracle.topk: hand values, brute force, full sorts, invariants."""
import json
import os

import numpy as np
import pytest

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_index_hand_worked():
    g = json.load(open(os.path.join(GOLD, "index_topk_hand.json")))
    q = np.asarray(g["q"], np.float64)[None, None]          # [1][1][HI][cI]
    w = np.asarray(g["w"], np.float64)[None, None]
    K = np.asarray(g["K"], np.float64)[None]
    s = oracle.index(q, w, K, [g["t_full"]], g["m"])
    assert np.array_equal(s[0, 0], g["scores_full"])
    s = oracle.index(q, w, K, [g["t_partial"]], g["m"])
    assert list(s[0, 0, :2]) == g["scores_full"][:2] and s[0, 0, 2] == -np.inf


def test_topk_hand_worked():
    g = json.load(open(os.path.join(GOLD, "index_topk_hand.json")))
    for cs in g["topk_cases"]:
        sc = np.asarray(cs["scores"], np.float64)[None, None]
        n = sc.shape[-1]
        idx = oracle.topk(sc, [4 * n], 4, cs["k"])
        assert list(idx[0, 0]) == cs["expected"]


def test_index_brute_force_loops():
    r = np.random.default_rng(0)
    B, T, HI, cI, N, m = 2, 5, 3, 4, 7, 4
    q = r.standard_normal((B, T, HI, cI))
    w = r.uniform(-1, 1, (B, T, HI))
    K = r.standard_normal((B, N, cI))
    pos0 = [13, 20]
    s = oracle.index(q, w, K, pos0, m)
    for b in range(B):
        for tr in range(T):
            t = pos0[b] + tr
            for j in range(N):
                if j >= t // m:
                    assert s[b, tr, j] == -np.inf
                    continue
                tot = 0.0
                for h in range(HI):
                    d = sum(q[b, tr, h, x] * K[b, j, x] for x in range(cI))
                    tot += w[b, tr, h] * max(d, 0.0)
                assert abs(tot - s[b, tr, j]) < 1e-12


def test_index_one_head_is_relu_gemv_and_scale_invariant_ranking():
    r = np.random.default_rng(1)
    q = r.standard_normal((1, 1, 1, 16))
    K = r.standard_normal((1, 50, 16))
    s = oracle.index(q, np.ones((1, 1, 1)), K, [400], 4)
    assert np.allclose(s[0, 0], np.maximum(K[0] @ q[0, 0, 0], 0))
    q4 = r.standard_normal((1, 1, 4, 16))
    w4 = r.uniform(0, 1, (1, 1, 4))
    a = oracle.index(q4, w4, K, [400], 4)
    b = oracle.index(3.7 * q4, w4, K, [400], 4)
    assert np.allclose(b, 3.7 * a)
    assert np.array_equal(oracle.topk(a, [400], 4, 10), oracle.topk(b, [400], 4, 10))


def _ref_topk_lexsort(row, k):
    row = row + 0.0
    order = np.lexsort((np.arange(len(row)), -row))   # primary: -score, secondary: index
    return np.sort(order[:k])


def test_topk_equals_full_sort_with_duplicates():
    r = np.random.default_rng(2)
    for trial in range(20):
        n = int(r.integers(1, 300))
        row = np.round(r.standard_normal(n) * 3) / 2          # many duplicates
        row[r.random(n) < 0.2] = 0.0
        row[r.random(n) < 0.1] = -0.0
        k = int(r.integers(1, 40))
        idx = oracle.topk(row[None, None], [4 * n], 4, k)[0, 0]
        ref = _ref_topk_lexsort(row, min(k, n))
        assert list(idx[:len(ref)]) == list(ref)
        assert np.all(idx[len(ref):] == -1)


def test_topk_visibility_and_padding():
    row = np.arange(20, dtype=np.float64)[None, None]
    idx = oracle.topk(row, [9], 4, 5)        # floor(9/4) = 2 visible
    assert list(idx[0, 0]) == [0, 1, -1, -1, -1]
    idx = oracle.topk(row, [3], 4, 5)        # nothing visible
    assert list(idx[0, 0]) == [-1] * 5


def test_topk_permutation_consistency():
    r = np.random.default_rng(3)
    row = r.standard_normal(64)
    perm = r.permutation(64)
    a = oracle.topk(row[None, None], [256], 4, 8)[0, 0]
    b = oracle.topk(row[perm][None, None], [256], 4, 8)[0, 0]
    assert sorted(perm[b]) == list(a)


def test_dequantized_fp8_and_mxfp4_inputs_score_like_their_values():
    from synth import formats as sf
    r = np.random.default_rng(4)
    x = r.standard_normal((1, 40, 128)).astype(np.float32)
    q = r.standard_normal((1, 1, 2, 128)).astype(np.float32)
    codes, sc = sf.fp8_rowscale_encode(x)
    kx = oracle.dequant_rows(codes, sc, "fp8")
    assert np.max(np.abs(kx - x)) <= np.max(np.abs(x)) / 448 * 16      # within a few fp8 steps
    s_q = oracle.index(q.astype(np.float64), np.ones((1, 1, 2)), kx, [160], 4)
    s_x = oracle.index(q.astype(np.float64), np.ones((1, 1, 2)), x.astype(np.float64), [160], 4)
    assert np.corrcoef(s_q[0, 0], s_x[0, 0])[0, 1] > 0.99
    p, e = sf.mxfp4_encode(x)
    kx4 = oracle.dequant_rows(p, e, "mxfp4")
    assert kx4.shape == x.shape and np.corrcoef(kx4.ravel(), x.ravel())[0, 1] > 0.98
