"""GPU parity of decode across steps: the state cache (rings of the tail tokens and of the window) and the paged
compressed caches ("【论文解读】DeepSeek-V4", section 二(六) 推理框架; "DeepseekV4论文解析", its KV-cache part).

  - csa_index_paged / csa_attend_paged / hca_attend_paged on a shuffled block table (unused pages filled with
    noise) equal the contiguous calls on the same entries bit for bit: scores, bound keys, outputs; every
    kernel variant (bf16 / fp8 / MXFP4 keys; narrow raw, narrow prepared, wide; bf16 and mixed KV rows);
  - csa_decode_append's entries equal csa_compress on the same token rows bit for bit (KV prepared in bf16
    and in the mixed format, fp8 indexer keys, the HCA entry), its rings hold the token's rows, and its
    window ring holds the token's row prepared exactly as csa_prepare_kv prepares it;
  - a decode loop of several steps per sequence (append -> paged index -> top-k -> paged attention, CSA and
    HCA, crossing CSA and HCA block boundaries) against the float64 oracle computed from the token streams
    alone: every score within 2^-8 of its absolute-value scale (the keys' bf16 rounding), the selection (k
    below the visible count: exact on the GPU's own scores, the 1e-3 gap rule and >= 99.9% agreement against
    the oracle's), the outputs (rel-L2 <= 5e-3).
"""
import numpy as np
import pytest
import torch

import oracle
from synth import configs, gen
from tests.gpu_util import DEV, dev, host_f64, rel_l2, topk_agreement

pytestmark = pytest.mark.gpu
LOWP_TOL = 5e-3


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)


@pytest.fixture(scope="module")
def api():
    from long_context_sparse_04_amd import api as a
    from long_context_sparse_04_amd import _lib
    _lib.load()
    return a


def _pos(arr):
    return torch.tensor(np.asarray(arr, np.int64), device=DEV)


def make_table(rng, B, max_pages, extra=5):
    """A shuffled block table over B * max_pages + extra physical pages."""
    n_phys = B * max_pages + extra
    return rng.permutation(n_phys)[: B * max_pages].reshape(B, max_pages).astype(np.int32), n_phys


def pool_rows(table, E, N):
    """Pool row of every logical entry (b, s < N): [B][N] int64."""
    s = np.arange(N)
    return table[:, s // E].astype(np.int64) * E + s % E


def scatter(x, table, E, n_phys, seed=0):
    """Contiguous [B][N][...] -> pool [n_phys * E][...]; rows of unmapped slots hold noise."""
    if x is None:
        return None
    B, N = x.shape[0], x.shape[1]
    g = torch.Generator(device=DEV).manual_seed(seed)
    shape = (n_phys * E,) + tuple(x.shape[2:])
    if x.dtype == torch.uint8:
        pool = torch.randint(0, 120, shape, dtype=torch.uint8, device=DEV, generator=g)
    else:
        pool = (torch.rand(shape, device=DEV, generator=g) + 0.5).to(x.dtype)
    rows = torch.from_numpy(pool_rows(table, E, N).reshape(-1)).to(DEV)
    pool[rows] = x.reshape((B * N,) + tuple(x.shape[2:]))
    return pool


def ring_of(rows_by_pos, positions, n_ring):
    """[B][L][c] rows of positions[b][j] -> ring [B][n_ring][c] (row p % n_ring)."""
    B = rows_by_pos.shape[0]
    ring = torch.zeros((B, n_ring) + tuple(rows_by_pos.shape[2:]), dtype=rows_by_pos.dtype, device=DEV)
    for b in range(B):
        for j, p in enumerate(positions[b]):
            ring[b, p % n_ring] = rows_by_pos[b, j]
    return ring


# ---- paged == contiguous --------------------------------------------------------------------------------------

@pytest.mark.parametrize("name,n_comp,page_tokens", [("c3", 5037, 1024), ("c2", 3000, 128), ("c5", 2100, 4096),
                                                     ("c3", 700, 128)])
def test_index_paged_matches_contiguous(api, name, n_comp, page_tokens):
    cfg = configs.get_config(name).scaled(B=3, n_comp=n_comp)
    fmt, N, B = cfg.idx_dtype, cfg.n_comp, cfg.B
    E = page_tokens // cfg.m
    table, n_phys = make_table(np.random.default_rng(n_comp), B, -(-N // E))
    say(f"index_paged {cfg.name} fmt={fmt} N={N} page_tokens={page_tokens} pages={n_phys}")
    kc = gen.indexer_key_cache(cfg)
    qi, w = gen.indexer_queries(cfg)
    pos = _pos([4 * N, 4 * N + 3, 4 * (N // 3) + 1])
    k, ks = dev(kc["data"]), dev(kc.get("scale"))
    kp, ksp = scatter(k, table, E, n_phys, 1), scatter(ks, table, E, n_phys, 2)
    pg = api.pages(dev(table), page_tokens)
    qd, qs, wd = dev(qi["data"]), dev(qi.get("scale")), dev(w)
    bc, bp = api.bound_keys(B, 1, N, DEV), api.bound_keys(B, 1, N, DEV)
    sc = api.index(qd, qs, wd, k, ks, pos, cfg.m, fmt, bound=bc)
    sp = api.index_paged(qd, qs, wd, kp, ksp, pg, pos, cfg.m, fmt, N, bound=bp)
    torch.cuda.synchronize()
    assert torch.equal(sc.view(torch.int32), sp.view(torch.int32))
    assert torch.equal(bc, bp)


def _attend_pair(api, cfg, hca, prepared, mixed, page_tokens, seed):
    q = dev(gen.queries(cfg, hca=hca))
    cache = dev(gen.kv_cache(cfg, hca=hca))
    win = dev(gen.window(cfg, hca=hca))
    sink = dev(gen.sink(cfg, hca=hca))
    B, N, R = cfg.B, cache.shape[1], cfg.rope_dims
    ratio = cfg.m_hca if hca else cfg.m
    pos0 = [ratio * N, ratio * (N // 2) + 3, 40][:B]
    pos = _pos(pos0)
    prep = api.kv_prep(R, cfg.eps, cfg.rope_base)
    if mixed:
        comp, cscale = api.prepare_kv(cache, prep, pos_stride=ratio, out_fmt="fp8rope")
    else:
        comp, cscale = api.prepare_kv(cache, prep, pos_stride=ratio), None
    if prepared == 2:
        win = api.prepare_kv(win, prep, pos_base=pos, pos_first=-(cfg.n_win - 1))
    E = page_tokens // ratio
    table, n_phys = make_table(np.random.default_rng(seed), B, -(-N // E))
    pg = api.pages(dev(table), page_tokens)
    cp, csp = scatter(comp, table, E, n_phys, 3), scatter(cscale, table, E, n_phys, 4)
    wpos = [[p0 - cfg.n_win + 1 + j for j in range(cfg.n_win)] for p0 in pos0]
    ring = ring_of(win, wpos, cfg.n_win)
    say(f"{'hca' if hca else 'csa'}_attend_paged B={B} H={cfg.H} N={N} prepared={prepared} mixed={mixed} "
        f"page_tokens={page_tokens}")
    if hca:
        oc = api.hca_attend(q, comp, win, sink, pos, ratio, cfg.n_win, R, cfg.scale, cfg.eps, cfg.rope_base,
                            kv_prepared=prepared, comp_scale=cscale)
        op = api.hca_attend_paged(q, cp, ring, sink, pos, pg, ratio, R, cfg.scale, N, cfg.eps, cfg.rope_base,
                                  kv_prepared=prepared, comp_scale=csp)
    else:
        rng = np.random.default_rng(seed + 1)
        idx = np.full((B, 1, cfg.k), -1, np.int32)
        for b in range(B):
            vis = min(pos0[b] // cfg.m, N)
            n = min(cfg.k - 7, vis)
            idx[b, 0, :n] = np.sort(rng.choice(vis, size=n, replace=False))
        idx = dev(idx)
        oc = api.attend(q, comp, idx, win, sink, pos, cfg.m, cfg.n_win, R, cfg.scale, cfg.eps, cfg.rope_base,
                        kv_prepared=prepared, comp_scale=cscale)
        op = api.attend_paged(q, cp, idx, ring, sink, pos, pg, cfg.m, R, cfg.scale, N, cfg.eps, cfg.rope_base,
                              kv_prepared=prepared, comp_scale=csp)
    torch.cuda.synchronize()
    return oc, op


@pytest.mark.parametrize("prepared,mixed", [(1, False), (2, False), (1, True), (2, True)])
def test_attend_paged_matches_contiguous(api, prepared, mixed):
    cfg = configs.C3.scaled(B=3, n_comp=3000)
    oc, op = _attend_pair(api, cfg, False, prepared, mixed, 128 if prepared == 1 else 1024, 11 + prepared)
    assert torch.equal(oc.view(torch.int16), op.view(torch.int16))


@pytest.mark.parametrize("prepared,mixed", [(1, False), (2, False), (2, True)])
def test_hca_attend_paged_matches_contiguous(api, prepared, mixed):
    cfg = configs.C5.scaled(B=3, n_hca=700)   # H = 128: prepared 2 runs the wide variant, 1 the narrow raw one
    oc, op = _attend_pair(api, cfg, True, prepared, mixed, 1024, 21 + prepared)
    assert torch.equal(oc.view(torch.int16), op.view(torch.int16))


# ---- csa_decode_append == csa_compress / csa_prepare_kv --------------------------------------------------------

def _linear_rows(st, name, lo, hi):
    """Rows of positions [lo, hi) of stream `name` of every sequence, [B][hi - lo][w] bf16 on the device."""
    return dev(np.stack([s[name][lo[b]:hi[b]] for b, s in enumerate(st)]))


def test_decode_append_matches_compress(api):
    cfg = configs.C3.scaled(B=3)
    m, mh, R = cfg.m, cfg.m_hca, cfg.rope_dims
    # sequence 0 completes a CSA and an HCA block, 1 completes neither, 2 completes CSA entry 0 / HCA entry 0
    ts = [128 * 7, 4 * 301 + 2, 128]
    st = [gen.decode_streams(cfg, t + 1, b) for b, t in enumerate(ts)]
    bi = gen.decode_biases(cfg)
    B = cfg.B
    page_tokens = 128
    maxp = max(ts) // page_tokens + 2
    table, n_phys = make_table(np.random.default_rng(5), B, maxp)
    pg = api.pages(dev(table), page_tokens)
    E, Eh = page_tokens // m, page_tokens // mh
    prep = api.kv_prep(R, cfg.eps, cfg.rope_base)
    pos = _pos(ts)
    say(f"decode_append positions {ts}")

    def rings(names, ring):
        lo = [t - ring for t in ts]
        out = []
        for nm in names:
            rows = torch.zeros((B, ring, st[0][nm].shape[1]), dtype=torch.bfloat16, device=DEV)
            for b, t in enumerate(ts):
                for p in range(max(0, t - ring), t):
                    rows[b, p % ring] = dev(st[b][nm][p:p + 1])[0]
            out.append(rows)
        return out

    kv_r = rings(("ca", "cb", "za", "zb"), 2 * m)
    ik_r = rings(("ica", "icb", "iza", "izb"), 2 * m)
    hc_r = rings(("hca_c", "hca_z"), mh)
    tok = lambda nm: dev(np.stack([s[nm][t] for s, t in zip(st, ts)]))
    kv_pool = torch.zeros((n_phys * E, cfg.c), dtype=torch.bfloat16, device=DEV)
    mx_pool = torch.zeros((n_phys * E, cfg.c + R), dtype=torch.uint8, device=DEV)
    mx_scale = torch.zeros((n_phys * E,), dtype=torch.float32, device=DEV)
    ik_pool = torch.zeros((n_phys * E, cfg.cI), dtype=torch.uint8, device=DEV)
    ik_scale = torch.zeros((n_phys * E,), dtype=torch.float32, device=DEV)
    hc_pool = torch.zeros((n_phys * Eh, cfg.c), dtype=torch.bfloat16, device=DEV)
    win_ring = torch.zeros((B, cfg.n_win, cfg.c), dtype=torch.bfloat16, device=DEV)
    b_kv = dict(bias_a=dev(bi["bias_a"]), bias_b=dev(bi["bias_b"]))
    b_ik = dict(bias_a=dev(bi["ibias_a"]), bias_b=dev(bi["ibias_b"]))
    kv_job = dict(ca=tok("ca"), cb=tok("cb"), za=tok("za"), zb=tok("zb"), m=m, ring_ca=kv_r[0], ring_cb=kv_r[1],
                  ring_za=kv_r[2], ring_zb=kv_r[3], out=kv_pool, prep=prep, **b_kv)
    ik_job = dict(ca=tok("ica"), cb=tok("icb"), za=tok("iza"), zb=tok("izb"), m=m, ring_ca=ik_r[0], ring_cb=ik_r[1],
                  ring_za=ik_r[2], ring_zb=ik_r[3], out=ik_pool, out_scale=ik_scale, out_fmt="fp8", **b_ik)
    win_job = dict(row=tok("win"), ring=win_ring, prep=prep)
    kv_r0 = [r.clone() for r in kv_r]
    api.decode_append([kv_job, ik_job], [win_job], pos, pg)
    # the same KV entry in the mixed format, from the rings as they were
    mx_job = dict(kv_job, ring_ca=kv_r0[0], ring_cb=kv_r0[1], ring_za=kv_r0[2], ring_zb=kv_r0[3], out=mx_pool,
                  out_scale=mx_scale, out_fmt="fp8rope")
    api.decode_append([mx_job], [], pos, pg)
    hc_job = dict(ca=tok("hca_c"), za=tok("hca_z"), bias_a=dev(bi["hca_bias"]), m=mh, ring_ca=hc_r[0],
                  ring_za=hc_r[1], out=hc_pool, prep=prep)
    api.decode_append([hc_job], [], pos, pg)
    torch.cuda.synchronize()
    for b, t in enumerate(ts):
        one = lambda x: None if x is None else x[b:b + 1]
        for (job, nm, ratio, pool, psc, fmt, E_) in (
                (kv_job, ("ca", "cb", "za", "zb"), m, kv_pool, None, "bf16", E),
                (mx_job, ("ca", "cb", "za", "zb"), m, mx_pool, mx_scale, "fp8rope", E),
                (ik_job, ("ica", "icb", "iza", "izb"), m, ik_pool, ik_scale, "fp8", E),
                (hc_job, ("hca_c", None, "hca_z", None), mh, hc_pool, None, "bf16", Eh)):
            if t % ratio or t < ratio:
                continue
            i = t // ratio - 1
            lo = max(0, ratio * (i - (1 if nm[1] else 0)))
            rows = {k: (None if n is None else dev(st[b][n][lo:t][None])) for k, n in zip(("ca", "cb", "za", "zb"),
                                                                                            nm)}
            ref, ref_s = api.compress(rows["ca"], rows["cb"], rows["za"], rows["zb"], job["bias_a"], job.get("bias_b"),
                                      ratio, lo, i, 1, out_fmt=None if fmt == "bf16" else fmt, prep=job.get("prep"))
            prow = int(table[b, i // E_]) * E_ + i % E_
            got = pool[prow]
            assert torch.equal(got.contiguous().view(torch.uint8), ref[0, 0].contiguous().view(torch.uint8)), (b, fmt)
            if psc is not None:
                assert torch.equal(psc[prow], ref_s[0, 0].reshape(())), (b, fmt)
        # the token's rows now sit at ring row t % ring; the window ring holds the prepared row
        for rs, names, ring in ((kv_r, ("ca", "cb", "za", "zb"), 2 * m), (hc_r, ("hca_c", "hca_z"), mh)):
            for r_, nm in zip(rs, names):
                assert torch.equal(r_[b, t % ring].view(torch.int16), dev(st[b][nm][t:t + 1])[0].view(torch.int16))
        pw = api.prepare_kv(dev(st[b]["win"][t:t + 1][None]), prep, pos_first=t)
        assert torch.equal(win_ring[b, t % cfg.n_win].view(torch.int16), pw[0, 0].view(torch.int16))


# ---- a decode loop against the oracle --------------------------------------------------------------------------

def test_decode_loop_against_oracle(api):
    """Sequences at positions that cross CSA (every 4) and HCA (every 128) block boundaries during the loop;
    every step appends its token, then indexes, selects and attends over the paged caches and the rings."""
    cfg = configs.C2.scaled(B=2, H=64, k=64)           # bf16 indexer keys; k below every step's visible count
    m, mh, R, W = cfg.m, cfg.m_hca, cfg.rope_dims, cfg.n_win
    t0 = [764, 509]
    S = 7
    B = cfg.B
    page_tokens = 128
    L = [t + S for t in t0]
    st = [gen.decode_streams(cfg, L[b], b) for b in range(B)]
    bi = gen.decode_biases(cfg)
    dq = [gen.decode_queries(cfg, S, b) for b in range(B)]
    sink, hsink = gen.sink(cfg), gen.sink(cfg, hca=True)
    maxp = max(L) // page_tokens + 1
    table, n_phys = make_table(np.random.default_rng(9), B, maxp)
    pg = api.pages(dev(table), page_tokens)
    E, Eh = page_tokens // m, page_tokens // mh
    prep = api.kv_prep(R, cfg.eps, cfg.rope_base)
    v = oracle.decode_bf16
    say(f"decode loop t0={t0} steps={S} page_tokens={page_tokens}")

    # state before the first step: entries completed by blocks that end before t0 - 1 (the block ending at
    # t0 - 1, if any, is compressed by the first step's append), rings of the last tokens
    def n_done(t, ratio):
        return (t - 1) // ratio if t % ratio == 0 else t // ratio

    kv_pool = torch.zeros((n_phys * E, cfg.c), dtype=torch.bfloat16, device=DEV)
    ik_pool = torch.zeros((n_phys * E, cfg.cI), dtype=torch.bfloat16, device=DEV)
    hc_pool = torch.zeros((n_phys * Eh, cfg.c), dtype=torch.bfloat16, device=DEV)
    for b in range(B):
        for (names, ratio, pool, E_, pp, bias) in (
                (("ca", "cb", "za", "zb"), m, kv_pool, E, prep, (bi["bias_a"], bi["bias_b"])),
                (("ica", "icb", "iza", "izb"), m, ik_pool, E, None, (bi["ibias_a"], bi["ibias_b"])),
                (("hca_c", None, "hca_z", None), mh, hc_pool, Eh, prep, (bi["hca_bias"], None))):
            n = n_done(t0[b], ratio)
            if n == 0:
                continue
            rows = [None if nm is None else dev(st[b][nm][: ratio * n][None]) for nm in names]
            out, _ = api.compress(rows[0], rows[1], rows[2], rows[3], dev(bias[0]), dev(bias[1]), ratio, 0, 0, n,
                                  prep=pp)
            prow = torch.from_numpy(pool_rows(table[b:b + 1], E_, n)[0]).to(DEV)
            pool[prow] = out[0]

    def ring_init(names, ring):
        out = []
        for nm in names:
            r_ = torch.zeros((B, ring, st[0][nm].shape[1]), dtype=torch.bfloat16, device=DEV)
            for b in range(B):
                for p in range(max(0, t0[b] - ring), t0[b]):
                    r_[b, p % ring] = dev(st[b][nm][p:p + 1])[0]
            out.append(r_)
        return out

    kv_r = ring_init(("ca", "cb", "za", "zb"), 2 * m)
    ik_r = ring_init(("ica", "icb", "iza", "izb"), 2 * m)
    hc_r = ring_init(("hca_c", "hca_z"), mh)
    win_ring = torch.zeros((B, W, cfg.c), dtype=torch.bfloat16, device=DEV)
    hwin_ring = torch.zeros((B, W, cfg.c), dtype=torch.bfloat16, device=DEV)
    for b in range(B):   # window rows of positions t0 - W + 1 .. t0 - 1, prepared at their positions
        lo = max(0, t0[b] - W + 1)
        for nm, rg in (("win", win_ring), ("hca_win", hwin_ring)):
            pr = api.prepare_kv(dev(st[b][nm][lo:t0[b]][None]), prep, pos_first=lo)
            for j, p in enumerate(range(lo, t0[b])):
                rg[b, p % W] = pr[0, j]
    n_max = maxp * E
    n_hmax = maxp * Eh
    scores = torch.empty((B, 1, n_max), dtype=torch.float32, device=DEV)
    bd = lambda x: dev(x)
    sel_stats = []
    for s in range(S):
        ts = [t0[b] + s for b in range(B)]
        pos = _pos(ts)
        tok = lambda nm: dev(np.stack([st[b][nm][ts[b]] for b in range(B)]))
        kv_job = dict(ca=tok("ca"), cb=tok("cb"), za=tok("za"), zb=tok("zb"), bias_a=bd(bi["bias_a"]),
                      bias_b=bd(bi["bias_b"]), m=m, ring_ca=kv_r[0], ring_cb=kv_r[1], ring_za=kv_r[2],
                      ring_zb=kv_r[3], out=kv_pool, prep=prep)
        ik_job = dict(ca=tok("ica"), cb=tok("icb"), za=tok("iza"), zb=tok("izb"), bias_a=bd(bi["ibias_a"]),
                      bias_b=bd(bi["ibias_b"]), m=m, ring_ca=ik_r[0], ring_cb=ik_r[1], ring_za=ik_r[2],
                      ring_zb=ik_r[3], out=ik_pool)
        api.decode_append([kv_job, ik_job], [dict(row=tok("win"), ring=win_ring, prep=prep)], pos, pg)
        hc_job = dict(ca=tok("hca_c"), za=tok("hca_z"), bias_a=bd(bi["hca_bias"]), m=mh, ring_ca=hc_r[0],
                      ring_za=hc_r[1], out=hc_pool, prep=prep)
        api.decode_append([hc_job], [dict(row=tok("hca_win"), ring=hwin_ring, prep=prep)], pos, pg)
        q = dev(np.stack([dq[b]["q"][s:s + 1] for b in range(B)]))
        hq = dev(np.stack([dq[b]["hq"][s:s + 1] for b in range(B)]))
        qi = dev(np.stack([dq[b]["qi"]["data"][s:s + 1] for b in range(B)]))
        w = dev(np.stack([dq[b]["w"][s:s + 1] for b in range(B)]))
        api.index_paged(qi, None, w, ik_pool, None, pg, pos, m, "bf16", n_max, scores=scores)
        idx, _ = api.topk(scores, pos, m, cfg.k)
        out = api.attend_paged(q, kv_pool, idx, win_ring, dev(sink), pos, pg, m, R, cfg.scale, n_max, cfg.eps,
                               cfg.rope_base, kv_prepared=2)
        hout = api.hca_attend_paged(hq, hc_pool, hwin_ring, dev(hsink), pos, pg, mh, R, cfg.scale, n_hmax, cfg.eps,
                                    cfg.rope_base, kv_prepared=2)
        torch.cuda.synchronize()
        g_sc, g_idx, g_out, g_hout = host_f64(scores), idx.cpu().numpy(), host_f64(out), host_f64(hout)
        for b in range(B):
            t = ts[b]
            # the oracle, from the token streams alone
            f = lambda nm, lo, hi: v(st[b][nm][lo:hi])
            nv, nh = t // m, t // mh
            g3 = lambda nm, n: None if nm is None else f(nm, 0, n)[None]
            ents = oracle.compress(g3("ca", m * nv), g3("cb", m * nv), g3("za", m * nv), g3("zb", m * nv),
                                   bi["bias_a"], bi["bias_b"], m, 0, 0, nv)
            keys = oracle.compress(g3("ica", m * nv), g3("icb", m * nv), g3("iza", m * nv), g3("izb", m * nv),
                                   bi["ibias_a"], bi["ibias_b"], m, 0, 0, nv)
            keys = v(oracle.encode_bf16(keys))                    # the cache stores bf16 keys
            hents = oracle.compress(g3("hca_c", mh * nh), None, g3("hca_z", mh * nh), None, bi["hca_bias"], None,
                                    mh, 0, 0, nh)
            wl = t - W + 1
            win = np.zeros((1, W, cfg.c))
            hwin = np.zeros((1, W, cfg.c))
            ok = np.arange(wl, t + 1) >= 0
            win[0, ok] = f("win", max(0, wl), t + 1)
            hwin[0, ok] = f("hca_win", max(0, wl), t + 1)
            qv = v(dq[b]["qi"]["data"][s:s + 1])[None]
            sc_ref = oracle.index(qv, dq[b]["w"][s:s + 1][None], keys, [t], m)
            # element by element: both sides store bf16 keys of their own pooled values, which may differ by
            # one bf16 rounding per element, so a score may move by 2^-8 of sum_h w_h |q_h|.|K| (plus float32
            # accumulation)
            absref = oracle.index(np.abs(qv), dq[b]["w"][s:s + 1][None], np.abs(keys), [t], m)
            err = np.abs(g_sc[b, 0, :nv] - sc_ref[0, 0, :nv])
            assert np.all(err <= (2.0 ** -8 + 1e-5) * absref[0, 0, :nv]), (s, b, np.max(err / absref[0, 0, :nv]))
            assert np.all(np.isneginf(g_sc[b, 0, nv:n_max]))
            assert nv > cfg.k                                      # the selection is not trivial
            # the selector is exact on the GPU's own scores; against the oracle's scores every difference
            # must lie within the 1e-3 gap rule
            assert np.array_equal(g_idx[b], oracle.topk(g_sc[b:b + 1, :, :n_max], [t], m, cfg.k)[0]), (s, b)
            idx_ref = oracle.topk(sc_ref, [t], m, cfg.k)
            agree, bad = topk_agreement(g_idx[b:b + 1], idx_ref, sc_ref)
            sel_stats.append(agree)
            assert bad == 0, (s, b, agree)
            # attention on the GPU's own list (the selection is checked above), so that the two are isolated
            o_ref = oracle.attend(v(dq[b]["q"][s:s + 1])[None], ents, g_idx[b:b + 1], win, sink, [t], m, W, R,
                                  cfg.scale, cfg.eps, cfg.rope_base)
            e = rel_l2(g_out[b], o_ref[0])
            h_ref = oracle.hca_attend(v(dq[b]["hq"][s:s + 1])[None], hents, hwin, hsink, [t], mh, W, R, cfg.scale,
                                      cfg.eps, cfg.rope_base)
            eh = rel_l2(g_hout[b], h_ref[0])
            say(f"  step {s} seq {b} t={t} visible {nv}/{nh}: top-k agreement {agree:.4f}, csa rel-L2 {e:.2e}, "
                f"hca rel-L2 {eh:.2e}")
            assert e <= LOWP_TOL and eh <= LOWP_TOL, (s, b, e, eh)
    assert np.mean(sel_stats) >= 0.999, sel_stats


def test_append_index_paged_matches_separate(api):
    """csa_append_index_paged equals csa_decode_append followed by csa_index_paged bit for bit: the pools, the
    rings, the window ring, the scores and bound keys.  Sequence 0 completes an entry that a later workgroup
    scores, 1 completes none, 2 completes one in workgroup 0's range (which then also compresses the KV entry)."""
    cfg = configs.C3.scaled(B=3, n_comp=5000)
    m, R, B = cfg.m, cfg.rope_dims, 3
    ts = [4 * 4096, 4 * 3000 + 1, 4 * 700]
    page_tokens = 1024
    E = page_tokens // m
    maxp = -(-cfg.n_comp // E)
    table, n_phys = make_table(np.random.default_rng(31), B, maxp)
    pg = api.pages(dev(table), page_tokens)
    prep = api.kv_prep(R, cfg.eps, cfg.rope_base)
    bi = gen.decode_biases(cfg)
    qi, w = gen.indexer_queries(cfg)
    kc = gen.indexer_key_cache(cfg)
    rnd = lambda *shape: (torch.randn(shape, device=DEV)).to(torch.bfloat16)
    torch.manual_seed(3)
    base = dict(kv_r=[rnd(B, 2 * m, cfg.c) for _ in range(4)], ik_r=[rnd(B, 2 * m, cfg.cI) for _ in range(4)],
                win=rnd(B, cfg.n_win, cfg.c), kv_pool=rnd(n_phys * E, cfg.c),
                ik_pool=scatter(dev(kc["data"]), table, E, n_phys, 5), ik_sc=scatter(dev(kc["scale"]), table, E, n_phys, 6))
    toks = {nm: rnd(B, cfg.c if nm in ("ca", "cb", "za", "zb", "win") else cfg.cI)
            for nm in ("ca", "cb", "za", "zb", "ica", "icb", "iza", "izb", "win")}
    pos = _pos(ts)
    say(f"append_index_paged positions {ts}")
    results = []
    for fused in (False, True):
        st = {k: ([x.clone() for x in v] if isinstance(v, list) else v.clone()) for k, v in base.items()}
        kv_job = dict(ca=toks["ca"], cb=toks["cb"], za=toks["za"], zb=toks["zb"], bias_a=dev(bi["bias_a"]),
                      bias_b=dev(bi["bias_b"]), m=m, ring_ca=st["kv_r"][0], ring_cb=st["kv_r"][1],
                      ring_za=st["kv_r"][2], ring_zb=st["kv_r"][3], out=st["kv_pool"], prep=prep)
        ik_job = dict(ca=toks["ica"], cb=toks["icb"], za=toks["iza"], zb=toks["izb"], bias_a=dev(bi["ibias_a"]),
                      bias_b=dev(bi["ibias_b"]), m=m, ring_ca=st["ik_r"][0], ring_cb=st["ik_r"][1],
                      ring_za=st["ik_r"][2], ring_zb=st["ik_r"][3], out=st["ik_pool"], out_scale=st["ik_sc"],
                      out_fmt="fp8")
        win_job = dict(row=toks["win"], ring=st["win"], prep=prep)
        bound = api.bound_keys(B, 1, cfg.n_comp, DEV)
        qd, qs, wd = dev(qi["data"]), dev(qi["scale"]), dev(w)
        if fused:
            sc = api.append_index_paged([kv_job, ik_job], win_job, qd, qs, wd, st["ik_pool"], st["ik_sc"], pg, pos, m,
                                        "fp8", cfg.n_comp, bound=bound)
        else:
            api.decode_append([kv_job, ik_job], [win_job], pos, pg)
            sc = api.index_paged(qd, qs, wd, st["ik_pool"], st["ik_sc"], pg, pos, m, "fp8", cfg.n_comp, bound=bound)
        torch.cuda.synchronize()
        results.append([sc, bound, st["kv_pool"], st["ik_pool"], st["ik_sc"], st["win"]] + st["kv_r"] + st["ik_r"])
    for a_, b_ in zip(*results):
        assert torch.equal(a_.contiguous().view(torch.uint8), b_.contiguous().view(torch.uint8))


def test_paged_full_size_matches_contiguous(api):
    """The Pro 1M decode shapes in the launch configuration bench.py runs (C3: fp8 keys over 262,144 entries,
    k = 1024; C5's HCA over 8,192 entries, wide variant): paged == contiguous bit for bit.  Entries are seeded
    device noise (the equality needs no oracle)."""
    g = torch.Generator(device=DEV).manual_seed(41)
    cfg = configs.C3
    B, N, m = cfg.B, cfg.n_comp, cfg.m
    page_tokens = 1024
    E = page_tokens // m
    table, n_phys = make_table(np.random.default_rng(42), B, -(-N // E) + 1)
    pg = api.pages(dev(table), page_tokens)
    cap = table.shape[1] * E
    say(f"paged full size C3 N={N} capacity={cap}")
    keys = torch.randint(0, 120, (B, cap, cfg.cI), dtype=torch.uint8, device=DEV, generator=g)
    ksc = torch.rand((B, cap), device=DEV, generator=g) * 0.01 + 0.001
    qi, w = gen.indexer_queries(cfg)
    qd, qs, wd = dev(qi["data"]), dev(qi["scale"]), dev(w)
    pos = _pos([4 * N - 4 * 5, 4 * N, 4 * N - 1001, 4 * (N // 2)])
    bc, bp = api.bound_keys(B, 1, cap, DEV), api.bound_keys(B, 1, cap, DEV)
    sc = api.index(qd, qs, wd, keys, ksc, pos, m, "fp8", bound=bc)
    sp = api.index_paged(qd, qs, wd, scatter(keys, table, E, n_phys, 1), scatter(ksc, table, E, n_phys, 2), pg, pos,
                         m, "fp8", cap, bound=bp)
    torch.cuda.synchronize()
    assert torch.equal(sc.view(torch.int32), sp.view(torch.int32)) and torch.equal(bc, bp)
    idx, _ = api.topk(sc, pos, m, cfg.k, bound=bc)
    del keys
    kv = torch.randn((B, cap, cfg.c), device=DEV, generator=g).to(torch.bfloat16)
    win = torch.randn((B, cfg.n_win, cfg.c), device=DEV, generator=g).to(torch.bfloat16)
    q = (torch.randn((B, 1, cfg.H, cfg.c), device=DEV, generator=g) / 22.6).to(torch.bfloat16)
    sink = dev(gen.sink(cfg))
    p0 = pos.cpu().numpy()
    ring = ring_of(win, [[int(t) - cfg.n_win + 1 + j for j in range(cfg.n_win)] for t in p0], cfg.n_win)
    oc = api.attend(q, kv, idx, win, sink, pos, m, cfg.n_win, cfg.rope_dims, cfg.scale, cfg.eps, cfg.rope_base,
                    kv_prepared=1)
    op = api.attend_paged(q, scatter(kv, table, E, n_phys, 3), idx, ring, sink, pos, pg, m, cfg.rope_dims, cfg.scale,
                          cap, cfg.eps, cfg.rope_base, kv_prepared=1)
    torch.cuda.synchronize()
    assert torch.equal(oc.view(torch.int16), op.view(torch.int16))
    del kv
    c5 = configs.C5
    nh, Eh = c5.n_hca, page_tokens // c5.m_hca
    say(f"paged full size C5 HCA n={nh}")
    tb5, n5 = make_table(np.random.default_rng(43), c5.B, -(-nh // Eh))
    pg5 = api.pages(dev(tb5), page_tokens)
    hk = torch.randn((c5.B, nh, c5.c), device=DEV, generator=g).to(torch.bfloat16)
    hw = torch.randn((c5.B, c5.n_win, c5.c), device=DEV, generator=g).to(torch.bfloat16)
    hq = (torch.randn((c5.B, 1, c5.H, c5.c), device=DEV, generator=g) / 22.6).to(torch.bfloat16)
    hpos = _pos([c5.pos0 - 128 * b for b in range(c5.B)])
    hp0 = hpos.cpu().numpy()
    hring = ring_of(hw, [[int(t) - c5.n_win + 1 + j for j in range(c5.n_win)] for t in hp0], c5.n_win)
    hs = dev(gen.sink(c5, hca=True))
    oc = api.hca_attend(hq, hk, hw, hs, hpos, c5.m_hca, c5.n_win, c5.rope_dims, c5.scale, c5.eps, c5.rope_base,
                        kv_prepared=2)
    op = api.hca_attend_paged(hq, scatter(hk, tb5, Eh, n5, 4), hring, hs, hpos, pg5, c5.m_hca, c5.rope_dims, c5.scale,
                              nh, c5.eps, c5.rope_base, kv_prepared=2)
    torch.cuda.synchronize()
    assert torch.equal(oc.view(torch.int16), op.view(torch.int16))
