"""Pins of the oracle's projections (oracle/proj.py) to facts the pages and linear algebra fix, independent of
the oracle's own formulas: a hand-computed example, the one-group case as two plain products, the group
structure (a group's intermediate sees only its own heads), and the shared latent of the two query heads."""
import numpy as np

import oracle


def test_grouped_out_proj_hand_example():
    # 2 heads of c = 1, g = 2 groups (one head each), d_g = 1, d = 1:
    # o = [3, 5]; group weights 2 and -1; final weights [10, 100] -> 3*2*10 + 5*(-1)*100 = -440
    o = np.array([[3.0, 5.0]])
    w_g = np.array([[[2.0]], [[-1.0]]])
    w_o = np.array([[10.0, 100.0]])
    out, mid = oracle.grouped_out_proj(o, w_g, w_o, 2)
    assert mid.tolist() == [[6.0, -5.0]]
    assert out.tolist() == [[-440.0]]


def test_one_group_is_two_plain_products():
    rng = np.random.default_rng(0)
    o = rng.standard_normal((3, 24))
    w1 = rng.standard_normal((1, 5, 24))
    w2 = rng.standard_normal((7, 5))
    out, mid = oracle.grouped_out_proj(o, w1, w2, 1)
    ref_mid = np.einsum("rk,nk->rn", o, w1[0])
    assert np.allclose(mid, ref_mid, rtol=1e-13, atol=1e-13)
    assert np.allclose(out, np.einsum("rk,nk->rn", ref_mid, w2), rtol=1e-12, atol=1e-12)


def test_groups_see_only_their_heads():
    """Changing the heads of group 1 leaves group 0's and group 2's intermediates exactly as they were."""
    rng = np.random.default_rng(1)
    g, heads, c, d_g = 3, 6, 4, 5
    o = rng.standard_normal((2, heads * c))
    w_g = rng.standard_normal((g, d_g, heads * c // g))
    w_o = rng.standard_normal((9, g * d_g))
    _, mid = oracle.grouped_out_proj(o, w_g, w_o, g)
    o2 = o.copy()
    per = heads * c // g
    o2[:, per:2 * per] += rng.standard_normal((2, per))
    _, mid2 = oracle.grouped_out_proj(o2, w_g, w_o, g)
    assert np.array_equal(mid[:, :d_g], mid2[:, :d_g]) and np.array_equal(mid[:, 2 * d_g:], mid2[:, 2 * d_g:])
    assert not np.allclose(mid[:, d_g:2 * d_g], mid2[:, d_g:2 * d_g])


def test_q_up_proj_shares_the_latent_and_is_linear():
    rng = np.random.default_rng(2)
    cq = rng.standard_normal((3, 16))
    w_uq, w_iuq = rng.standard_normal((8, 16)), rng.standard_normal((4, 16))
    q, qi = oracle.q_up_proj(cq, w_uq, w_iuq)
    # a unit latent picks one weight column: q[e_j] = W^UQ[:, j]
    e = np.zeros((1, 16))
    e[0, 5] = 1.0
    q1, qi1 = oracle.q_up_proj(e, w_uq, w_iuq)
    assert np.array_equal(q1[0], w_uq[:, 5]) and np.array_equal(qi1[0], w_iuq[:, 5])
    q2, qi2 = oracle.q_up_proj(2.0 * cq[:1] - cq[1:2], w_uq, w_iuq)
    assert np.allclose(q2, 2.0 * q[:1] - q[1:2], rtol=1e-12, atol=1e-12)
    assert np.allclose(qi2, 2.0 * qi[:1] - qi[1:2], rtol=1e-12, atol=1e-12)
