"""The dense projections on either side of the CSA / HCA step -- TEST INFRASTRUCTURE ONLY (float64).

"【论文解读】DeepSeek-V4" (wkq9411.github.io), section 一(三)1(2)-(3): the queries come from a shared low-rank latent
c^Q_t in R^{d_c}: the attention queries q_t = c^Q_t W^UQ (n_h heads of c) and the indexer queries q^I_t =
c^Q_t W^IUQ (n_h^I heads of c^I).  Section 一(三)1(4): the grouped output projection splits the n_h head outputs
into g groups of n_h / g consecutive heads, projects group i's concatenated outputs (c n_h / g values) to a
d_g-dim intermediate o^G'_{t,i}, and projects the concatenation of the g intermediates (g d_g values) to the
d-dim attention output; section 一(三)2(2) uses the same projections for HCA.

Weights are passed as the kernels store them, output-major: W^UQ as [c n_h][d_c] (row j = the weights of output
column j), a group's projection as [d_g][c n_h / g], the final one as [d][g d_g].  A matmul is the only primitive.
"""
from __future__ import annotations

import numpy as np


def q_up_proj(cq, w_uq, w_iuq):
    """(q, q^I) = (c^Q W^UQ, c^Q W^IUQ) for latent rows cq [rows][d_c]; weights [outputs][d_c]."""
    cq = np.asarray(cq, np.float64)
    return cq @ np.asarray(w_uq, np.float64).T, cq @ np.asarray(w_iuq, np.float64).T


def grouped_out_proj(o, w_g, w_o, g):
    """Attention output of rows o [rows][n_h c] (heads in order): o^G'_i = o^G_i W_i for each group i, then
    [o^G'_1; ...; o^G'_g] W^O.  w_g [g][d_g][n_h c / g], w_o [d][g d_g].  Returns (output [rows][d],
    intermediates [rows][g d_g])."""
    o = np.asarray(o, np.float64)
    rows, width = o.shape
    per = width // g
    mids = [o[:, i * per:(i + 1) * per] @ np.asarray(w_g[i], np.float64).T for i in range(g)]
    mid = np.concatenate(mids, axis=1)
    return mid @ np.asarray(w_o, np.float64).T, mid
