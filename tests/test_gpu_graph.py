"""A decode step captured in a HIP graph and replayed repeatedly matches the eager step on every replay."""
import numpy as np
import pytest
import torch

from synth import configs, gen
from tests.gpu_util import DEV, dev

pytestmark = pytest.mark.gpu


def test_graph_replay_matches_eager():
    from long_context_sparse_04_amd import api
    cfg = configs.C3.scaled(B=4, n_comp=262144)   # the Pro 1M decode shape: one bound set per run
    print("[gpu-case] graph replay of a decode step", flush=True)
    kc = gen.indexer_key_cache(cfg)
    qi, w = gen.indexer_queries(cfg)
    pos = torch.full((cfg.B,), 4 * cfg.n_comp, dtype=torch.int64, device=DEV)
    kv = dev(gen.kv_cache(cfg))
    q, win, sink = dev(gen.queries(cfg)), dev(gen.window(cfg)), dev(gen.sink(cfg))
    ik, iks, qd, qs, wd = dev(kc["data"]), dev(kc["scale"]), dev(qi["data"]), dev(qi["scale"]), dev(w)
    t = lambda ci: {k: dev(ci[k]) for k in ("ca", "cb", "za", "zb", "bias_a", "bias_b")}
    cik, ckv = t(gen.compress_inputs(cfg, indexer=True)), t(gen.compress_inputs(cfg))
    scores = torch.empty((cfg.B, 1, cfg.n_comp), device=DEV)
    idx = torch.empty((cfg.B, 1, cfg.k), dtype=torch.int32, device=DEV)
    bound = api.bound_keys(cfg.B, 1, cfg.n_comp, DEV)
    out = torch.empty((cfg.B, 1, cfg.H, cfg.c), dtype=torch.bfloat16, device=DEV)
    first = cfg.n_comp - 1
    prep = api.kv_prep(cfg.rope_dims, cfg.eps, cfg.rope_base)
    api.prepare_kv(kv, prep, pos_stride=cfg.m, out=kv)

    def step():  # the benchmark's step, launch for launch: the block's indexer key inside the index launch,
        # its KV entry (stored prepared) in the selection's launch, then the attention over the prepared cache
        api.compress_index(None, cik, cfg.m, 4 * cfg.n_comp - 8, first, qd, qs, wd, ik, iks, pos, "fp8",
                           scores=scores, bound=bound)
        api.topk_compress(scores, pos, cfg.m, cfg.k, dict(ckv, out=kv[:, first:], out_batch_stride=cfg.n_comp,
                                                          prep=prep), 4 * cfg.n_comp - 8, first, idx=idx, bound=bound)
        api.attend(q, kv, idx, win, sink, pos, cfg.m, cfg.n_win, cfg.rope_dims, cfg.scale, out=out,
                   kv_prepared=True)

    step()
    torch.cuda.synchronize()
    ref_idx, ref_out, ref_kv = idx.clone(), out.clone(), kv[:, first].clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        idx.fill_(-7)
        out.zero_()
        scores.zero_()          # eager work between replays
        kv[:, first:].zero_()   # the entry the step writes
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(idx, ref_idx), f"replay {rep}: top-k differs"
        assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16)), f"replay {rep}: output differs"
        assert torch.equal(kv[:, first].view(torch.int16), ref_kv.view(torch.int16)), f"replay {rep}: KV entry"
