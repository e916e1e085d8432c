"""Per-sequence generation of the large seeded caches in worker processes.

The full-size workloads hold up to 8 x 262,144 cache rows; drawing them one
sequence per worker keeps the host side of those tests to seconds.  Only seeded
inputs are made here (``synth.gen``); no arithmetic of the method.
"""
from __future__ import annotations

import concurrent.futures as cf
import os

import numpy as np

from synth import configs, gen


def _one(args):
    name, b = args
    cfg = configs.get_config(name)
    out = {"kv": gen.kv_cache(cfg, seqs=[b])[0]}
    ik = gen.indexer_key_cache(cfg, seqs=[b])
    out["ik"] = ik["data"][0]
    out["ik_scale"] = ik["scale"][0] if "scale" in ik else None
    if cfg.with_hca:
        out["hca"] = gen.kv_cache(cfg, seqs=[b], hca=True)[0]
    return b, out


def caches(cfg, workers: int = 8):
    """Stacked caches of every sequence: kv [B][N][c], ik (+ ik_scale) [B][N][..], hca [B][N_hca][c]."""
    B = cfg.B
    res = {}
    nproc = max(1, min(B, workers, len(os.sched_getaffinity(0))))
    with cf.ProcessPoolExecutor(max_workers=nproc) as ex:
        for b, out in ex.map(_one, [(cfg.name, b) for b in range(B)]):
            for k, v in out.items():
                if v is None:
                    res.setdefault(k, None)
                    continue
                if k not in res or res[k] is None:
                    res[k] = np.empty((B,) + v.shape, dtype=v.dtype)
                res[k][b] = v
    return res
