#!/usr/bin/env python3
"""Benchmark of the CSA decode layer step on one MI355X.

One step = one pass of the whole CSA layer step over one decode batch:
  csa_compress_index (decode; csa_compress_pair + csa_index for prefill): the KV entry that
  completes at this step, stored prepared
  for attention, and its indexer key, quantized to the cache format)  ->
  csa_index (decode: also the selector's bound keys)  ->  csa_topk  ->  csa_attend
  (prepared compressed entries; decode reads
  raw window rows, prefill prepares the chunk's token rows first and reads them prepared)
(plus, for the workloads with an HCA layer: compress, preparation of the step's
window rows, hca_attend).

Default workload: Pro-shaped decode at 1M context (B=4, 262,144 compressed
entries, 128 heads x 512, fp8 e4m3 indexer with row scales, top-k 1024, window
128).  `value` is per-layer decode tokens/s = B / step time, inputs resident in
HBM.  Four input sets (distinct queries, and separate copies of the indexer-key
cache, 4 x 138 MB) are rotated so that no step finds its working set in the
256 MB Infinity Cache.

Prints ONE JSON line (see --help for options).
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from synth import configs, gen  # noqa: E402

METRIC = "CSA decode tokens/s at 1M ctx (Pro shape) + % HBM/MFMA roofline"
HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0, "mxfp4": 10100.0}   # dense, MI355X
NSETS = 4


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--config", default="c3", help="c3 (default), c2 or c5 (decode), c4 (chunked prefill)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--eager", action="store_true", help="launch the step's calls one by one (no HIP graph)")
    p.add_argument("--scores", default="f32", choices=("f32", "bf16"),
                   help="index-score storage between the indexer and the selector (bf16: the rounded variant)")
    p.add_argument("--kv", default="bf16", choices=("bf16", "fp8rope"),
                   help="compressed KV cache storage: bf16 rows, or the non-RoPE dims in fp8 e4m3 with a row scale "
                        "and the RoPE dims in bf16")
    p.add_argument("--paged", action="store_true",
                   help="decode across steps: tokens enter the state-cache rings (csa_decode_append, which compresses "
                        "an entry when a block completes), compressed entries live in paged pools behind a shuffled "
                        "block table, and every step advances the positions by one")
    p.add_argument("--page-tokens", type=int, default=1024, help="raw tokens per page (a power of two >= 128)")
    p.add_argument("--proj", action="store_true",
                   help="the step also runs the query up-projections from the latent (q and the indexer "
                        "queries, one launch) before it and the grouped output projection after it (decode rows: "
                        "weight-streaming kernels; prefill rows: the LDS-tiled MFMA kernel)")
    p.add_argument("--batch", type=int, default=None,
                   help="decode: run the workload with this many sequences instead of its own batch (same shapes "
                        "per sequence; each sequence's inputs are seeded by its index)")
    p.add_argument("--copy-calibration", action="store_true",
                   help="first run three plain 1 GiB device-to-device copies (reference for HBM byte counters)")
    return p.parse_args()


# ----------------------------------------------------------------------------- inputs
def _gen_seq(args):
    """Host arrays of one sequence (runs in a worker process)."""
    name, b = args
    cfg = configs.get_config(name)
    out = {
        "kv": gen.kv_cache(cfg, seqs=[b])[0],
        "ik": {k: v[0] for k, v in gen.indexer_key_cache(cfg, seqs=[b]).items()},
    }
    if cfg.with_hca:
        out["hca"] = gen.kv_cache(cfg, seqs=[b], hca=True)[0]
    return b, out


def host_inputs(cfg, seed):
    c = cfg.scaled(seed=seed)
    qi, w = gen.indexer_queries(c)
    d = {
        "q": gen.queries(c), "qi": qi, "w": w, "win": gen.window(c), "sink": gen.sink(c),
        "ckv": gen.compress_inputs(c), "cik": gen.compress_inputs(c, indexer=True),
    }
    if cfg.with_hca:
        d.update(hq=gen.queries(c, hca=True), hwin=gen.window(c, hca=True), hsink=gen.sink(c, hca=True),
                 chca=gen.compress_inputs(c, hca=True))
    return d


def _paged_setup(a, cfg, api, torch, sets, kv_cache, kv_scale, ik_data, ik_scale, hca_cache, hca_scale, prep, pos,
                 scores, bound, idx, out, hout, hca_ws, side, mixed):
    """Pools, block table, state rings and the paged decode step.  Returns (step, parts, visible, scores):
    parts(set) maps the step's launches to callables."""
    dev = pos.device
    B, N, R, m, mh, W = cfg.B, cfg.n_comp, cfg.rope_dims, cfg.m, cfg.m_hca, cfg.n_win
    P = a.page_tokens
    E, Eh = P // m, P // mh
    maxp = -(-N // E) + 1                      # the context's pages plus one page of room to grow
    n_phys = B * maxp
    g = torch.Generator(device="cpu").manual_seed(1234)
    table = torch.randperm(n_phys, generator=g).to(torch.int32).reshape(B, maxp).to(dev)
    pg = api.pages(table, P)
    cap = maxp * E
    rows = (table.to(torch.int64)[:, torch.arange(N, device=dev) // E] * E + torch.arange(N, device=dev) % E)

    def pool_of(x, per_row_shape, dtype, ent=E, n=N, rws=None):
        pool = torch.zeros((n_phys * ent,) + per_row_shape, dtype=dtype, device=dev)
        if x is not None:
            pool[(rows if rws is None else rws).reshape(-1)] = x.reshape((B * n,) + per_row_shape)
        return pool

    kv_pool = pool_of(kv_cache, tuple(kv_cache.shape[2:]), kv_cache.dtype)
    kv_spool = pool_of(kv_scale, (), torch.float32) if mixed else None
    for st in sets:   # each set keeps its own copy of the key pool (rotation past the Infinity Cache)
        st["ik_pool"] = pool_of(st["ik"], tuple(st["ik"].shape[2:]), st["ik"].dtype)
        st["iks_pool"] = None if st["ik_scale"] is None else pool_of(st["ik_scale"], tuple(st["ik_scale"].shape[2:]),
                                                                       st["ik_scale"].dtype)
    hpool = hspool = None
    if cfg.with_hca:
        nh = cfg.n_hca
        hrows = (table.to(torch.int64)[:, torch.arange(nh, device=dev) // Eh] * Eh + torch.arange(nh, device=dev) % Eh)
        hpool = pool_of(hca_cache, tuple(hca_cache.shape[2:]), hca_cache.dtype, Eh, nh, hrows)
        hspool = pool_of(hca_scale, (), torch.float32, Eh, nh, hrows) if mixed else None
    # state rings: the tail tokens' streams (synthetic N(0,1) rows) and the window rows, prepared at their
    # positions; ring row p % ring holds position p
    torch.manual_seed(4321)
    rnd = lambda shape: torch.randn(shape, device=dev).to(torch.bfloat16)
    kv_r = [rnd((B, 2 * m, cfg.c)) for _ in range(4)]
    ik_r = [rnd((B, 2 * m, cfg.cI)) for _ in range(4)]
    hc_r = [rnd((B, mh, cfg.c)) for _ in range(2)] if cfg.with_hca else None
    p0 = cfg.pos0 - W + 1
    st0 = sets[0]
    win_ring = torch.roll(api.prepare_kv(st0["win"], prep, pos_base=pos, pos_first=-(W - 1)), p0 % W, dims=1)
    hwin_ring = torch.roll(api.prepare_kv(st0["hwin"], prep, pos_base=pos, pos_first=-(W - 1)), p0 % W, dims=1) \
        if cfg.with_hca else None
    cache_fmt = "fp8rope" if mixed else None
    fmt = cfg.idx_dtype
    for st in sets:   # the step's new token rows: one row of each stream per sequence
        row = lambda d, k: None if d.get(k) is None else d[k][:, 0].contiguous()
        c, ci = st["ckv"], st["cik"]
        st["kv_job"] = dict(ca=row(c, "ca"), cb=row(c, "cb"), za=row(c, "za"), zb=row(c, "zb"), bias_a=c["bias_a"],
                            bias_b=c["bias_b"], m=m, ring_ca=kv_r[0], ring_cb=kv_r[1], ring_za=kv_r[2],
                            ring_zb=kv_r[3], out=kv_pool, out_scale=kv_spool, out_fmt=cache_fmt, prep=prep)
        st["ik_job"] = dict(ca=row(ci, "ca"), cb=row(ci, "cb"), za=row(ci, "za"), zb=row(ci, "zb"),
                            bias_a=ci["bias_a"], bias_b=ci["bias_b"], m=m, ring_ca=ik_r[0], ring_cb=ik_r[1],
                            ring_za=ik_r[2], ring_zb=ik_r[3], out=st["ik_pool"], out_scale=st["iks_pool"],
                            out_fmt=fmt if fmt in ("fp8", "mxfp4") else None)
        st["win_job"] = dict(row=st["win"][:, W - 1].contiguous(), ring=win_ring, prep=prep)
        if cfg.with_hca:
            ch = st["chca"]
            st["hc_job"] = dict(ca=row(ch, "ca"), za=row(ch, "za"), bias_a=ch["bias_a"], m=mh, ring_ca=hc_r[0],
                                ring_za=hc_r[1], out=hpool, out_scale=hspool, out_fmt=cache_fmt, prep=prep)
            st["hwin_job"] = dict(row=st["hwin"][:, W - 1].contiguous(), ring=hwin_ring, prep=prep)
    hws = None
    if cfg.with_hca:
        nb = api._lib.load().hca_attend_workspace_bytes(B, 1, cfg.H, cfg.c, maxp * Eh, W)
        hws = torch.empty(max(nb, 1), dtype=torch.uint8, device=dev)
    bnd = api.bound_keys(B, 1, cap, dev)
    sc = torch.empty((B, 1, cap), dtype=scores.dtype, device=dev)
    steps_done = [0]

    def step(st):
        main_s = torch.cuda.current_stream()
        if side is not None:
            side.wait_stream(main_s)
            with torch.cuda.stream(side):
                api.decode_append([st["hc_job"]], [st["hwin_job"]], pos, pg, stream=side)
                api.hca_attend_paged(st["hq"], hpool, hwin_ring, st["hsink"], pos, pg, mh, R, cfg.scale,
                                     maxp * Eh, cfg.eps, cfg.rope_base, out=hout, ws=hws, stream=side,
                                     kv_prepared=2, comp_scale=hspool)
        # the token's append (rings, window, the entry a block completes) inside the paged index launch
        api.append_index_paged([st["kv_job"], st["ik_job"]], st["win_job"], st["qi"], st["qi_scale"], st["w"],
                               st["ik_pool"], st["iks_pool"], pg, pos, m, fmt, cap, scores=sc, bound=bnd)
        api.topk(sc, pos, m, cfg.k, idx=idx, bound=bnd)
        api.attend_paged(st["q"], kv_pool, idx, win_ring, st["sink"], pos, pg, m, R, cfg.scale, cap, cfg.eps,
                         cfg.rope_base, out=out, kv_prepared=2, comp_scale=kv_spool)
        if side is not None:
            main_s.wait_stream(side)
        pos.add_(1)   # the next step decodes the next token
        steps_done[0] += 1

    # the step's launches one by one (timed back to back for the per-kernel figures)
    def parts(st):
        return {
            "index": lambda: api.append_index_paged([st["kv_job"], st["ik_job"]], st["win_job"], st["qi"],
                                                    st["qi_scale"], st["w"], st["ik_pool"], st["iks_pool"], pg, pos,
                                                    m, fmt, cap, scores=sc, bound=bnd),
            "topk": lambda: api.topk(sc, pos, m, cfg.k, idx=idx, bound=bnd),
            "attend": lambda: api.attend_paged(st["q"], kv_pool, idx, win_ring, st["sink"], pos, pg, m, R, cfg.scale,
                                               cap, cfg.eps, cfg.rope_base, out=out, kv_prepared=2,
                                               comp_scale=kv_spool),
        }

    def visible():
        return int(min(int(pos[0].item()) // m, cap))

    return step, parts, visible, sc


# Pro / Flash projection shapes ("【论文解读】DeepSeek-V4", section 三(二): d_c, g, d_g, d)
PROJ_SHAPES = {128: dict(d_c=1536, g=16, d_g=1024, d=7168), 64: dict(d_c=1024, g=8, d_g=1024, d=4096)}


def _with_projections(cfg, api, torch, step, out, dev):
    """Wrap a step: latent -> (q, q^I) before it, grouped output projection after it.  Returns the wrapped
    step and the two projection launches, each as (call on an input set, algorithmic bytes, FLOPs): the
    weights and the rows read once, the outputs written once; 2 FLOPs per multiply-add."""
    ps = PROJ_SHAPES[cfg.H]
    rows = cfg.B * cfg.T
    x = gen.proj_inputs(rows, ps["d_c"], cfg.H, cfg.c, cfg.HI, cfg.cI, ps["g"], ps["d_g"], ps["d"], seed=3)
    up = lambda a: torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
    cq = up(x["cq"])
    # the weights are packed once, at load time, into the projections' MFMA-tile layout
    w_uq, w_iuq, w_g, w_o = (api.pack_proj_weights(up(x[k])) for k in ("w_uq", "w_iuq", "w_g", "w_o"))
    mid = torch.empty((rows, ps["g"] * ps["d_g"]), dtype=torch.bfloat16, device=dev)
    hid = torch.empty((rows, ps["d"]), dtype=torch.bfloat16, device=dev)
    fmt = cfg.idx_dtype

    def up(st):
        api.q_up_proj(cq, w_uq, w_iuq, cfg.H, cfg.c, cfg.HI, cfg.cI, qi_fmt=fmt, q=st["q"], qi=st["qi"],
                      qi_scale=st["qi_scale"])

    def down(st):
        api.grouped_out_proj(out.view(rows, cfg.H * cfg.c), w_g, w_o, ps["g"], mid=mid, out=hid)

    def run(st):
        up(st)
        step(st)
        down(st)

    d_c, nq, ni, gd = ps["d_c"], cfg.H * cfg.c, cfg.HI * cfg.cI, ps["g"] * ps["d_g"]
    qi_row = {"f32": 4 * ni, "bf16": 2 * ni, "fp8": ni + 4 * cfg.HI, "mxfp4": ni // 2 + ni // 32}[fmt]
    up_bytes = 2 * (nq + ni) * d_c + rows * (2 * d_c + 2 * nq + qi_row)
    down_bytes = 2 * gd * nq // ps["g"] + 2 * ps["d"] * gd + rows * (2 * nq + 2 * 2 * gd + 2 * ps["d"])
    parts = {"csa_q_up_proj": (up, up_bytes, 2 * rows * d_c * (nq + ni)),
             "csa_grouped_out_proj": (down, down_bytes, 2 * rows * (nq * ps["d_g"] + gd * ps["d"]))}
    return run, parts


def source_hash(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "long_context_sparse_04_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# ----------------------------------------------------------------------------- bench
def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {a.gpus}); this build has no multi-GPU path: the decode "
              "batch shards by sequence with no exchange, so N GPUs run N independent copies of this benchmark.",
              file=sys.stderr)
        sys.exit(2)
    import torch
    from long_context_sparse_04_amd import _lib, api

    cfg = configs.get_config(a.config)
    if a.batch is not None:
        if cfg.T > 1 or a.batch < 1:
            print("--batch takes a positive batch of a decode workload", file=sys.stderr)
            sys.exit(2)
        cfg = cfg.scaled(B=a.batch)
    prefill = cfg.T > 1
    _lib.load()
    dev = "cuda:0"
    B, N = cfg.B, cfg.n_comp
    fmt = cfg.idx_dtype

    def up(x):
        if x is None:
            return None
        x = np.ascontiguousarray(x)
        if x.dtype == np.uint16:
            return torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(x).to(dev)

    t0 = time.time()
    nproc = max(1, min(B, len(os.sched_getaffinity(0)), 8))
    kv_cache = torch.empty((B, N, cfg.c), dtype=torch.bfloat16, device=dev)
    ik_rows = 64 if fmt == "mxfp4" else 128
    ik_data = torch.empty((B, N, ik_rows), dtype=torch.uint8 if fmt != "bf16" else torch.bfloat16, device=dev)
    if fmt == "bf16":
        ik_data = torch.empty((B, N, cfg.cI), dtype=torch.bfloat16, device=dev)
    ik_scale = None
    if fmt == "fp8":
        ik_scale = torch.empty((B, N), dtype=torch.float32, device=dev)
    elif fmt == "mxfp4":
        ik_scale = torch.empty((B, N, 4), dtype=torch.uint8, device=dev)
    hca_cache = torch.empty((B, cfg.n_hca, cfg.c), dtype=torch.bfloat16, device=dev) if cfg.with_hca else None
    host0 = {"kv": [None] * B, "ik_data": [None] * B, "ik_scale": [None] * B, "hca": [None] * B}
    with cf.ProcessPoolExecutor(max_workers=nproc) as ex:
        for b, out in ex.map(_gen_seq, [(cfg.name, b) for b in range(B)]):
            kv_cache[b].copy_(up(out["kv"]))
            ik_data[b].copy_(up(out["ik"]["data"]))
            if ik_scale is not None:
                ik_scale[b].copy_(up(out["ik"]["scale"]))
            if cfg.with_hca:
                hca_cache[b].copy_(up(out["hca"]))
            if b == 0 or not a.no_cpu_baseline:
                host0["kv"][b] = out["kv"]
                host0["ik_data"][b] = out["ik"]["data"]
                host0["ik_scale"][b] = out["ik"].get("scale")
                host0["hca"][b] = out.get("hca")
    # rotated sets: distinct queries (seed s), own copy of the indexer-key cache
    sets = []
    for s in range(NSETS):
        h = host_inputs(cfg, s)
        st = {k: up(v) for k, v in (("q", h["q"]), ("w", h["w"]), ("win", h["win"]), ("sink", h["sink"]))}
        st["qi"] = up(h["qi"]["data"])
        st["qi_scale"] = up(h["qi"].get("scale"))
        st["ik"] = ik_data if s == 0 else ik_data.clone()
        st["ik_scale"] = ik_scale if (s == 0 or ik_scale is None) else ik_scale.clone()
        for nm in ("ckv", "cik") + (("chca",) if cfg.with_hca else ()):
            st[nm] = {k: (up(v) if isinstance(v, np.ndarray) else v) for k, v in h[nm].items()}
        for nm in ("ckv", "cik"):
            st[nm + "_t"] = {k: st[nm][k] for k in ("ca", "cb", "za", "zb", "bias_a", "bias_b")}
        if cfg.with_hca:
            st.update(hq=up(h["hq"]), hwin=up(h["hwin"]), hsink=up(h["hsink"]))
        st["host"] = h if s == 0 else None
        sets.append(st)
    pos = torch.full((B,), cfg.pos0, dtype=torch.int64, device=dev)
    # compressed entries are stored prepared for attention (RMSNorm + RoPE at their positions, done once when
    # an entry is written); the synthetic context caches are prepared here, outside the timed region
    prep = api.kv_prep(cfg.rope_dims, cfg.eps, cfg.rope_base)
    mixed = a.kv == "fp8rope"
    kv_scale = hca_scale = None
    if mixed:   # caches in the fp8 + bf16 RoPE rows (c + R bytes) with one float32 scale per row
        kv_cache, kv_scale = api.prepare_kv(kv_cache, prep, pos_stride=cfg.m, out_fmt="fp8rope")
        if cfg.with_hca:
            hca_cache, hca_scale = api.prepare_kv(hca_cache, prep, pos_stride=cfg.m_hca, out_fmt="fp8rope")
        torch.cuda.synchronize()
    else:
        api.prepare_kv(kv_cache, prep, pos_stride=cfg.m, out=kv_cache)
        if cfg.with_hca:
            api.prepare_kv(hca_cache, prep, pos_stride=cfg.m_hca, out=hca_cache)
    cache_fmt = dict(out_fmt="fp8rope") if mixed else {}
    T = cfg.T
    # window rows: prefill (CSA) and the HCA layer also keep the token rows prepared (each row once, at its own
    # position, when it is written); rows of earlier steps are prepared here, the step's own T rows in the step
    csa_mode = 2 if T > 1 else 1
    win_new = dict(pos_base=pos, pos_first=0)
    for st in sets:
        st["pwin"] = api.prepare_kv(st["win"], prep, pos_base=pos, pos_first=-(cfg.n_win - 1)) if csa_mode == 2 \
            else st["win"]
        if cfg.with_hca:
            st["phwin"] = api.prepare_kv(st["hwin"], prep, pos_base=pos, pos_first=-(cfg.n_win - 1))
    scores = torch.empty((B, T, N), dtype=torch.bfloat16 if a.scores == "bf16" else torch.float32, device=dev)
    # the indexer also writes the selector's lower-bound keys (two per set of 256 entries, or of 32 for caches
    # of up to 65,536 entries): decode rows then take the one-launch selection, prefill rows one pruning pass
    bound = api.bound_keys(B, T, N, dev)
    idx = torch.empty((B, T, cfg.k), dtype=torch.int32, device=dev)
    out = torch.empty((B, T, cfg.H, cfg.c), dtype=torch.bfloat16, device=dev)
    hout = torch.empty_like(out) if cfg.with_hca else None
    # the HCA attention runs on its own stream, so it gets its own workspace
    hca_ws = None
    if cfg.with_hca:
        nb = _lib.load().hca_attend_workspace_bytes(B, T, cfg.H, cfg.c, cfg.n_hca, cfg.n_win)
        hca_ws = torch.empty(max(nb, 1), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    t_setup = time.time() - t0

    # decode: the entry completed by the block that ends at pos0-1; prefill: every entry of the chunk
    first, n_new = sets[0]["ckv"]["first_entry"], sets[0]["ckv"]["num_entries"]

    # the HCA layer does not depend on the CSA chain: it runs on a side stream that joins at the step's end
    # (a cross-stream join inside a HIP graph costs a few microseconds, which only work of this size repays)
    side = torch.cuda.Stream() if cfg.with_hca else None

    if a.paged:
        if prefill:
            print("--paged runs decode workloads only", file=sys.stderr)
            sys.exit(2)
        step, parts_paged, vis_now, scores_paged = _paged_setup(a, cfg, api, torch, sets, kv_cache, kv_scale, ik_data,
                                                       ik_scale, hca_cache, hca_scale, prep, pos, scores, bound, idx,
                                                       out, hout, hca_ws, side, mixed)

    def step_contiguous(st):
        main_s = torch.cuda.current_stream()
        if side is not None:
            side.wait_stream(main_s)
            with torch.cuda.stream(side):
                c = st["chca"]
                api.compress(c["ca"], None, c["za"], None, c["bias_a"], None, cfg.m_hca, c["row0_pos"],
                             c["first_entry"], c["num_entries"], out=hca_cache[:, c["first_entry"]:],
                             out_scale=hca_scale[:, c["first_entry"]:] if mixed else None,
                             out_batch_stride=cfg.n_hca, prep=prep, stream=side, **cache_fmt)
                api.prepare_kv(st["hwin"][:, cfg.n_win - 1:], prep, out=st["phwin"][:, cfg.n_win - 1:],
                               stream=side, **win_new)
                api.hca_attend(st["hq"], hca_cache, st["phwin"], st["hsink"], pos, cfg.m_hca, cfg.n_win,
                               cfg.rope_dims, cfg.scale, cfg.eps, cfg.rope_base, out=hout, ws=hca_ws, stream=side,
                               kv_prepared=2, comp_scale=hca_scale)
        c = st["cik"]
        kv_job = dict(st["ckv_t"], out=kv_cache[:, first:], out_batch_stride=N, prep=prep, **cache_fmt)
        if mixed:
            kv_job["out_scale"] = kv_scale[:, first:]
        if T == 1:
            # decode: the block's indexer key (into the key cache) is computed inside the index launch, by the
            # workgroup that scores it first
            api.compress_index(None, st["cik_t"], cfg.m, c["row0_pos"], first, st["qi"], st["qi_scale"], st["w"],
                               st["ik"], st["ik_scale"], pos, fmt, scores=scores, bound=bound)
        else:
            # prefill: every entry of the chunk, KV entry and indexer key (in the cache format), one launch
            ik_job = dict(st["cik_t"], out=st["ik"][:, first:], out_batch_stride=N,
                          out_fmt=fmt if fmt in ("fp8", "mxfp4") else None,
                          out_scale=st["ik_scale"][:, first:] if fmt in ("fp8", "mxfp4") else None)
            api.compress_pair(kv_job, ik_job, cfg.m, c["row0_pos"], first, n_new)
            if csa_mode == 2:
                api.prepare_kv(st["win"][:, cfg.n_win - 1:], prep, out=st["pwin"][:, cfg.n_win - 1:], **win_new)
            api.index(st["qi"], st["qi_scale"], st["w"], st["ik"], st["ik_scale"], pos, cfg.m, fmt, scores=scores,
                      bound=bound)
        if T == 1:   # decode: the block's KV entry rides in the selection's launch (one more workgroup per row)
            api.topk_compress(scores, pos, cfg.m, cfg.k, kv_job, c["row0_pos"], first, idx=idx, bound=bound)
        else:
            api.topk(scores, pos, cfg.m, cfg.k, idx=idx, bound=bound)
        api.attend(st["q"], kv_cache, idx, st["pwin"], st["sink"], pos, cfg.m, cfg.n_win, cfg.rope_dims, cfg.scale,
                   cfg.eps, cfg.rope_base, out=out, kv_prepared=csa_mode, comp_scale=kv_scale)
        if side is not None:
            main_s.wait_stream(side)

    if not a.paged:
        step = step_contiguous
    proj_parts = {}
    if a.proj:
        step, proj_parts = _with_projections(cfg, api, torch, step, out, dev)
    if a.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    for i in range(a.warmup):
        step(sets[i % NSETS])
    torch.cuda.synchronize()
    # one HIP graph per input set: the whole step is replayed with a single launch, so host-side
    # launch overhead does not leave the GPU idle between the step's kernels
    graphs = []
    if not a.eager:
        for s in range(NSETS):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(sets[s])
            graphs.append(g)
        for i in range(a.warmup):
            graphs[i % NSETS].replay()
        torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(a.steps):
        if graphs:
            graphs[i % NSETS].replay()
        else:
            step(sets[i % NSETS])
    end.record()
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(end) / a.steps
    # The step's launches one by one: each is timed by HIP events recorded on the launch stream around
    # back-to-back launches over the same input rotation, so that the average is the kernel's own time.
    def step_parts(st):
        if a.paged:
            return parts_paged(st)
        c = st["cik"]
        kv_job = dict(st["ckv_t"], out=kv_cache[:, first:], out_batch_stride=N, prep=prep, **cache_fmt)
        if mixed:
            kv_job["out_scale"] = kv_scale[:, first:]
        p = {}
        if T == 1:   # the step's own launches: the key-only compress + index, then top-k with the KV entry
            p["index"] = lambda: api.compress_index(None, st["cik_t"], cfg.m, c["row0_pos"], first, st["qi"],
                                                    st["qi_scale"], st["w"], st["ik"], st["ik_scale"], pos, fmt,
                                                    scores=scores, bound=bound)
            p["topk"] = lambda: api.topk_compress(scores, pos, cfg.m, cfg.k, kv_job, c["row0_pos"], first, idx=idx,
                                                  bound=bound)
        else:
            p["index"] = lambda: api.index(st["qi"], st["qi_scale"], st["w"], st["ik"], st["ik_scale"], pos, cfg.m,
                                           fmt, scores=scores, bound=bound)
            p["topk"] = lambda: api.topk(scores, pos, cfg.m, cfg.k, idx=idx, bound=bound)
        p["attend"] = lambda: api.attend(st["q"], kv_cache, idx, st["pwin"], st["sink"], pos, cfg.m, cfg.n_win,
                                         cfg.rope_dims, cfg.scale, cfg.eps, cfg.rope_base, out=out,
                                         kv_prepared=csa_mode, comp_scale=kv_scale)
        if cfg.with_hca:
            p["hca_attend"] = lambda: api.hca_attend(st["hq"], hca_cache, st["phwin"], st["hsink"], pos, cfg.m_hca,
                                                     cfg.n_win, cfg.rope_dims, cfg.scale, cfg.eps, cfg.rope_base,
                                                     out=hout, ws=hca_ws, kv_prepared=2, comp_scale=hca_scale)
        return p

    def time_call(f):   # f(i) runs one launch on input set i; the average of a.steps launches
        for i in range(NSETS):
            f(i)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for i in range(a.steps):
            f(i)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / a.steps

    def time_part(name):
        calls = [step_parts(sets[i % NSETS])[name] for i in range(max(a.steps, NSETS))]
        return time_call(lambda i: calls[i]())

    sc_t = scores_paged if a.paged else scores
    Nsc = sc_t.shape[2]
    n_read = vis_now() if a.paged else N   # paged: the visible entries of the current positions (all read)
    # index: every K^I row (+ its scales) read once, the queries / weights read once per query row; the
    # score write is booked to the selector, which reads it back
    row_bytes = {"bf16": 2 * cfg.cI, "fp8": cfg.cI + 4, "mxfp4": cfg.cI // 2 + cfg.cI // 32}[fmt]
    q_bytes = row_bytes * cfg.HI + 4 * cfg.HI
    idx_bytes = B * (n_read * row_bytes + T * q_bytes)
    score_bytes = B * T * Nsc * sc_t.element_size()
    pairs = sum(min((cfg.pos0 + r) // cfg.m, N) for r in range(T)) * B
    idx_flops = 2 * cfg.HI * cfg.cI * pairs
    # top-k: the scores read once, the index list written once
    topk_bytes = score_bytes + B * T * cfg.k * 4
    # attention: every selected / visible entry row and window row read once per query row, the queries read
    # and the outputs written once, the index list read once; FLOPs 4 c per (row, head, entry)
    comp_row = (cfg.c + cfg.rope_dims + 4) if mixed else 2 * cfg.c
    win_vis = [min(cfg.n_win, cfg.pos0 + r + 1) for r in range(T)]
    sel = [min(cfg.k, min((cfg.pos0 + r) // cfg.m, N)) for r in range(T)]
    att_bytes = B * sum(sel[r] * comp_row + win_vis[r] * 2 * cfg.c + 4 * cfg.H * cfg.c + 4 * cfg.k
                        for r in range(T))
    att_flops = B * sum(4 * cfg.c * cfg.H * (sel[r] + win_vis[r]) for r in range(T))
    if cfg.with_hca:
        hvis = [min((cfg.pos0 + r) // cfg.m_hca, cfg.n_hca) for r in range(T)]
        hcomp_row = (cfg.c + cfg.rope_dims + 4) if mixed else 2 * cfg.c
        hca_bytes = B * sum(hvis[r] * hcomp_row + win_vis[r] * 2 * cfg.c + 4 * cfg.H * cfg.c for r in range(T))
        hca_flops = B * sum(4 * cfg.c * cfg.H * (hvis[r] + win_vis[r]) for r in range(T))
    bf16_peak = MFMA_PEAK_TFLOPS["bf16"]

    def entry(name, ms, nbytes, flops, bound):
        e = {"kernel": name, "avg_us": round(ms * 1e3, 2), "bound": bound,
             "algorithmic_bytes": nbytes, "algorithmic_flops": flops}
        if bound == "hbm":
            e.update(achieved=nbytes / (ms * 1e-3) / 1e9, peak=HBM_PEAK_GBS, unit="GB/s")
        else:
            pk = MFMA_PEAK_TFLOPS[fmt] if name.startswith("csa_index") else bf16_peak
            e.update(achieved=flops / (ms * 1e-3) / 1e12, peak=pk, unit="TFLOP/s")
        e["frac"] = e["achieved"] / e["peak"]
        return e

    idx_name = ("csa_append_index_paged" if a.paged else "csa_compress_index (indexer key only)") if T == 1 \
        else "csa_index (tiled prefill)"
    idx_ms = time_part("index")
    kernels = [
        entry(idx_name, idx_ms, idx_bytes, idx_flops, "mfma" if prefill else "hbm"),
        entry("csa_topk" if (a.paged or prefill) else "csa_topk_compress (with the KV entry)", time_part("topk"),
              topk_bytes, 0, "hbm"),
        entry(("csa_attend_paged" if a.paged else "csa_attend") + " + combine", time_part("attend"), att_bytes,
              att_flops, "mfma" if prefill else "hbm"),
    ]
    if cfg.with_hca and not a.paged:
        kernels.append(entry("hca_attend", time_part("hca_attend"), hca_bytes, hca_flops, "mfma" if prefill else "hbm"))
    for pname, (pf, pbytes, pflops) in proj_parts.items():   # decode: a weight stream; prefill: MFMA-bound
        kernels.append(entry(pname, time_call(lambda i: pf(sets[i % NSETS])), pbytes, pflops,
                             "mfma" if prefill else "hbm"))
    traffic = None
    tpath = os.path.join(ROOT, "profiles", f"index_{cfg.name}_traffic.json")
    if os.path.exists(tpath) and not a.paged and not a.proj and a.batch is None:
        t = json.load(open(tpath))
        if t.get("source_hash") == source_hash("index.hip") and t.get("index_scores", "f32") == a.scores:
            traffic = t.get("hbm_bytes_per_launch")
    k0 = kernels[0]
    roofline = {"kernel": idx_name, "bound": k0["bound"], "achieved": k0["achieved"], "peak": k0["peak"],
                "unit": k0["unit"], "frac": k0["frac"], "traffic": traffic, "avg_launch_ms": idx_ms}
    if prefill:
        roofline["algorithmic_flops_per_launch"] = idx_flops
    else:
        roofline["algorithmic_bytes_per_launch"] = idx_bytes
        roofline["score_write_bytes_per_launch"] = score_bytes
    if cfg.name == configs.C3.name:
        metric = METRIC
    elif prefill:
        metric = f"CSA+HCA chunked prefill tokens/s ({cfg.name}) + % MFMA roofline"
    else:
        metric = f"CSA decode tokens/s ({cfg.name}) + % HBM roofline"

    res = {
        "metric": metric,
        "value": B * T / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"fp8": "fp8+bf16", "mxfp4": "mxfp4+bf16", "bf16": "bf16"}[fmt],
        "data": "synthetic (seeded Gaussian, synth/gen.py recipe)",
        "config": {"workload": cfg.name, "batch": B, "query_rows": T, "context": cfg.pos0, "compressed_entries": N,
                   "heads": cfg.H,
                   "head_dim": cfg.c, "indexer": f"{cfg.HI}x{cfg.cI} {fmt}", "top_k": cfg.k, "window": cfg.n_win,
                   "hca_entries": cfg.n_hca if cfg.with_hca else 0, "index_scores": a.scores, "kv_cache": a.kv,
                   "projections": "q / q^I up-projection + grouped output projection" if a.proj else "none",
                   "cache_layout": f"paged ({a.page_tokens}-token pages) + state rings, positions advancing"
                   if a.paged else "contiguous",
                   "input_sets_rotated": NSETS},
        "roofline": roofline,
        "kernels": kernels,
        "setup_s": round(t_setup, 1),
        "launch": "eager" if a.eager else "hip_graph (one graph per rotated input set)",
    }

    if not a.no_cpu_baseline:
        res["cpu_baseline"] = (cpu_baseline_prefill if prefill else cpu_baseline)(cfg, sets[0]["host"], host0)
    print(json.dumps(res), flush=True)


class _Bf16Rows:
    """Read-only view of a bf16 cache [1][N][c] that decodes only the rows indexed (plus overridden rows)."""

    def __init__(self, bits, override):
        self.bits, self.override = bits, override

    def __getitem__(self, key):
        import oracle
        b, rows = key
        out = oracle.decode_bf16(self.bits[b, rows])
        for j, r in enumerate(rows):
            if (b, int(r)) in self.override:
                out[j] = self.override[(b, int(r))]
        return out


def cpu_baseline(cfg, h, host0):
    """The float64 oracle, as it stands, on whole decode steps of the same workload (about 10 s of host work)."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = 1
    fmt = cfg.idx_dtype
    t0 = time.time()
    B = cfg.B
    pos0 = np.full(B, cfg.pos0)
    deq = lambda d, s: oracle.dequant_rows(d, s, fmt)
    ck = h["ckv"]
    f = lambda x: None if x is None else oracle.decode_bf16(x)
    new_kv = oracle.compress(f(ck["ca"]), f(ck["cb"]), f(ck["za"]), f(ck["zb"]), ck["bias_a"].astype(np.float64),
                             ck["bias_b"].astype(np.float64), cfg.m, ck["row0_pos"], ck["first_entry"], 1)
    ci = h["cik"]
    new_ik = oracle.compress(f(ci["ca"]), f(ci["cb"]), f(ci["za"]), f(ci["zb"]), ci["bias_a"].astype(np.float64),
                             ci["bias_b"].astype(np.float64), cfg.m, ci["row0_pos"], ci["first_entry"], 1)
    done = 0
    while True:  # whole decode steps (all B sequences) until >= 10 s of CPU work, bounded at ~30 s
        for b in range(B):
            kI = deq(host0["ik_data"][b], host0["ik_scale"][b])[None]
            kI[0, -1] = new_ik[b, 0]
            qI = deq(h["qi"]["data"][b:b + 1], None if h["qi"].get("scale") is None else h["qi"]["scale"][b:b + 1])
            sc = oracle.index(qI, h["w"][b:b + 1], kI, pos0[b:b + 1], cfg.m)
            sel = oracle.topk(sc, pos0[b:b + 1], cfg.m, cfg.k)
            cache = _Bf16Rows(host0["kv"][b][None], {(0, cfg.n_comp - 1): new_kv[b, 0]})
            oracle.attend(oracle.decode_bf16(h["q"][b:b + 1]), cache, sel, oracle.decode_bf16(h["win"][b:b + 1]),
                          h["sink"], pos0[b:b + 1], cfg.m, cfg.n_win, cfg.rope_dims, cfg.scale, cfg.eps,
                          cfg.rope_base)
            done += 1
        if time.time() - t0 > 10:
            break
    dt = time.time() - t0
    return {"value": done / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{done // B} full decode steps x {B} sequences (compress, index, top-k, attend) in "
                      f"float64, {dt:.1f} s"}




def cpu_baseline_prefill(cfg, h, host0):
    """The float64 oracle, as it stands, on the chunked-prefill workload: the chunk's compression once, then
    sampled query rows (index, top-k, attend, hca_attend) until about 10 s of host work, scaled to tokens/s."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = 1
    f = lambda x: None if x is None else oracle.decode_bf16(x) if x.dtype == np.uint16 else np.asarray(x, np.float64)
    t0 = time.time()
    caches = {}
    for nm, key, mm in (("ckv", "kv", cfg.m), ("cik", "ik_data", cfg.m), ("chca", "hca", cfg.m_hca)):
        ci = h[nm]
        new = oracle.compress(f(ci["ca"]), f(ci["cb"]), f(ci["za"]), f(ci["zb"]), f(ci["bias_a"]), f(ci["bias_b"]),
                              mm, ci["row0_pos"], ci["first_entry"], ci["num_entries"])[0]
        cache = oracle.decode_bf16(host0[key][0])
        cache[ci["first_entry"]:ci["first_entry"] + ci["num_entries"]] = oracle.decode_bf16(oracle.encode_bf16(new))
        caches[key] = cache
    t_comp = time.time() - t0
    qv, q, win, hq, hwin = f(h["qi"]["data"]), f(h["q"]), f(h["win"]), f(h["hq"]), f(h["hwin"])
    rng = np.random.default_rng(0)
    t1 = time.time()
    done = 0
    while time.time() - t1 < 10.0:
        r = int(rng.integers(0, cfg.T))
        t = cfg.pos0 + r
        sc = oracle.index(qv[:, r:r + 1], h["w"][:, r:r + 1], caches["ik_data"][None], [t], cfg.m)
        sel = oracle.topk(sc, [t], cfg.m, cfg.k)
        full = np.full((1, cfg.T, cfg.k), -1, np.int32)
        full[0, r] = sel[0, 0]
        oracle.attend(q, caches["kv"][None], full, win, h["sink"], [cfg.pos0], cfg.m, cfg.n_win, cfg.rope_dims,
                      cfg.scale, cfg.eps, cfg.rope_base, rows=[(0, r)])
        oracle.hca_attend(hq, caches["hca"][None], hwin, h["hsink"], [cfg.pos0], cfg.m_hca, cfg.n_win,
                          cfg.rope_dims, cfg.scale, cfg.eps, cfg.rope_base, rows=[(0, r)])
        done += 1
    t_rows = time.time() - t1
    per_token = t_rows / done + t_comp / cfg.T
    return {"value": 1.0 / per_token, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{done} sampled query rows of the {cfg.T}-row chunk (index, top-k, attend, hca_attend; "
                      f"{t_rows:.1f} s) plus the chunk's compression ({t_comp:.1f} s, amortised over {cfg.T} rows), "
                      f"float64"}


if __name__ == "__main__":
    main()
