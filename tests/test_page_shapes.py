"""Shape and count pins printed on the pages (hyper-parameter table, 1M-context entry counts, lcm block)."""
import json
import math
import os

import numpy as np

import oracle
from synth import configs

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_model_table_matches_workload_configs():
    t = json.load(open(os.path.join(GOLD, "model_table.json")))
    for cfg, col in ((configs.C2, "flash"), (configs.C4, "flash"), (configs.C3, "pro"), (configs.C5, "pro")):
        p = t[col]
        assert (cfg.m, cfg.HI, cfg.cI, cfg.k, cfg.m_hca, cfg.H, cfg.c, cfg.n_win) == (
            p["m"], p["indexer_heads"], p["indexer_dim"], p["top_k"], p["m_hca"], p["query_heads"],
            p["head_dim"], p["window"])


def test_one_million_context_counts():
    g = json.load(open(os.path.join(GOLD, "page_counts.json")))
    ctx = g["context_tokens"]
    for cfg in (configs.C3, configs.C5):
        assert cfg.pos0 == ctx
        assert cfg.visible(cfg.pos0) == g["csa_candidates"] == cfg.n_comp
        assert cfg.k + cfg.n_win == g["pro"]["entries_read"]
    assert configs.C5.n_hca == g["hca_entries"] == ctx // g["m_hca"]
    assert 512 + 128 == g["flash"]["entries_read"] == configs.C2.k + configs.C2.n_win
    # the oracle's visibility rule gives exactly the printed candidate count at t = 1M
    sc = np.zeros((1, 1, g["csa_candidates"] + 5))
    idx = oracle.topk(sc[:, :, :8], [ctx], g["m"], 4)
    assert list(idx[0, 0]) == [0, 1, 2, 3]
    assert min(ctx // g["m"], sc.shape[-1]) == g["csa_candidates"]


def test_lcm_block():
    g = json.load(open(os.path.join(GOLD, "page_counts.json")))
    lcm = g["m"] * g["m_hca"] // math.gcd(g["m"], g["m_hca"])
    assert lcm == g["lcm_tokens"]
    assert lcm // g["m"] == g["csa_entries_per_lcm_block"] and lcm // g["m_hca"] == g["hca_entries_per_lcm_block"]
