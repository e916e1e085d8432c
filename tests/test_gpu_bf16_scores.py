"""GPU parity of the bf16 index-score variant: csa_index / csa_compress_index writing bfloat16 scores
and csa_topk selecting from them.

The pages quantize the indexer's scores from float32 to bf16 for a faster selector and report the
recall of the resulting selection against the higher-precision one ("【论文解读】DeepSeek-V4",
section 二(四); "DeepseekV4论文解析", the inference-side list of precision choices).

Checks, on seeded inputs:
  - the bf16 scores are the float32 scores of the same call rounded to nearest even (bit-exact, via the
    oracle's encoder), and lie within half a bf16 ulp plus the float32 tolerance of the float64 oracle;
  - bound keys written with bf16 scores follow their definition on the stored bf16 values;
  - csa_topk on bf16 scores is bit-exact against the oracle's top-k of the same bf16 values, on every
    selector path (per-row, histogram split, bound keys), with ties and +0/-0;
  - the recall of the bf16-score selection against the float64 oracle's selection, reported beside
    the pages' figure, with every swapped entry inside the bf16 rounding band of the k-th score.
"""
import numpy as np
import pytest
import torch

import oracle
from synth import configs, gen
from tests.gpu_util import DEV, dev, host_bound, topk_agreement

pytestmark = pytest.mark.gpu


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


def _bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _to_bf16_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV).view(torch.bfloat16)


def _index_inputs(cfg):
    kc = gen.indexer_key_cache(cfg)
    qi, w = gen.indexer_queries(cfg)
    return kc, qi, w


def _run_index(api, cfg, kc, qi, w, pos0, score_fmt, bound=None):
    sc = api.index(dev(qi["data"]), dev(qi.get("scale")), dev(w), dev(kc["data"]), dev(kc.get("scale")),
                   _pos(pos0), cfg.m, cfg.idx_dtype, score_fmt=score_fmt, bound=bound)
    torch.cuda.synchronize()
    return sc


CASES = [
    ("f32", configs.C1, None, [0]),
    ("bf16", configs.C2, dict(B=3, n_comp=5037), [4 * 5037, 4 * 3001 + 2, 4 * 17 + 3]),
    ("fp8", configs.C3, dict(B=3, n_comp=5037), [4 * 5037, 4 * 3001 + 2, 4 * 17 + 3]),
    ("mxfp4", configs.C5, dict(B=3, n_comp=5037), [4 * 5037, 4 * 3001 + 2, 4 * 17 + 3]),
    ("prefill", configs.C4, dict(T=37, n_comp=3001, pos0=4 * 2990 - 20), None),
    ("rows", configs.C4, dict(T=5, n_comp=2100, pos0=4 * 2000 - 5), None),
]


@pytest.mark.parametrize("name,base,scale,pos0", CASES, ids=[c[0] for c in CASES])
def test_index_bf16_scores(api, name, base, scale, pos0):
    """Every index kernel (float32, per-row MFMA in the three formats, the tiled prefill kernel, the
    per-row kernel on a few rows) stores the bf16 rounding of the float32 score it computes."""
    cfg = base if scale is None else base.scaled(**scale)
    pos0 = [cfg.pos0] if pos0 is None else pos0
    say(f"index bf16 scores {name} {cfg.name} fmt={cfg.idx_dtype} B={cfg.B} T={cfg.T} N={cfg.n_comp}")
    kc, qi, w = _index_inputs(cfg)
    s32 = _run_index(api, cfg, kc, qi, w, pos0, "f32")
    s16 = _run_index(api, cfg, kc, qi, w, pos0, "bf16")
    assert s16.dtype == torch.bfloat16 and s16.shape == s32.shape
    got = _bits(s16)
    want = oracle.encode_bf16(s32.cpu().numpy().astype(np.float64))
    assert np.array_equal(got, want), np.argwhere(got != want)[:5]
    # against the float64 oracle: bf16 rounding (half an ulp, at most 2^-8 of the value: 8 significant
    # bits) plus the float32 path's own tolerance
    qv = oracle.dequant_rows(qi["data"], qi.get("scale"), cfg.idx_dtype)
    kv = oracle.dequant_rows(kc["data"], kc.get("scale"), cfg.idx_dtype)
    ref = oracle.index(qv, w, kv, pos0, cfg.m)
    absref = oracle.index(np.abs(qv), np.abs(w), np.abs(kv), pos0, cfg.m)
    g = oracle.decode_bf16(got)
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(g), fin) and np.all(g[~fin] == -np.inf)
    err = np.abs(g[fin] - ref[fin])
    assert np.all(err <= 2.0 ** -8 * np.abs(ref[fin]) + 2e-5 * absref[fin])


@pytest.mark.parametrize("fmt", ["bf16", "fp8", "mxfp4"])
def test_index_bf16_bound_keys(api, fmt):
    """Bound keys written beside bf16 scores are the per-256-entry top-2 keys of the stored bf16 values."""
    base = {"bf16": configs.C2, "fp8": configs.C3, "mxfp4": configs.C5}[fmt]
    cfg = base.scaled(B=3, n_comp=9037)
    pos0 = [4 * 9037, 4 * 5001 + 2, 4 * 300 + 3]
    say(f"index bf16 bound keys {cfg.name}")
    kc, qi, w = _index_inputs(cfg)
    bound = api.bound_keys(cfg.B, 1, cfg.n_comp, DEV)
    s16 = _run_index(api, cfg, kc, qi, w, pos0, "bf16", bound=bound)
    vals32 = oracle.decode_bf16(_bits(s16)).astype(np.float32)
    assert np.array_equal(bound.cpu().numpy().view(np.uint32), host_bound(vals32, pos0, cfg.m))


@pytest.mark.parametrize("name,n_comp", [("c3", 5037), ("c5", 3100), ("c2", 1500)])
def test_compress_index_bf16_scores_match_separate(api, name, n_comp):
    """The fused decode launch with bf16 scores writes the same caches, scores and bound keys as
    csa_compress_pair followed by csa_index with bf16 scores."""
    cfg = configs.get_config(name).scaled(B=3, n_comp=n_comp)
    fmt, N = cfg.idx_dtype, cfg.n_comp
    say(f"compress_index bf16 scores {cfg.name} fmt={fmt} N={N}")
    ckv, cik = gen.compress_inputs(cfg), gen.compress_inputs(cfg, indexer=True)
    first, r0p = N - 1, 4 * N - 8
    kc = gen.indexer_key_cache(cfg)
    qi, w = gen.indexer_queries(cfg)
    pos0 = [4 * N, 4 * N + 3, 4 * (N - 100)]
    d = lambda ci: {k: dev(ci[k]) for k in ("ca", "cb", "za", "zb", "bias_a", "bias_b")}
    prep = api.kv_prep(cfg.rope_dims, cfg.eps, cfg.rope_base)
    kv0 = dev(gen.kv_cache(cfg))
    outs = []
    for fused in (False, True):
        kv, ik = kv0.clone(), dev(kc["data"])
        iks = dev(kc.get("scale"))
        bound = api.bound_keys(cfg.B, 1, N, DEV)
        qd, qs, wd = dev(qi["data"]), dev(qi.get("scale")), dev(w)
        pkv = dict(d(ckv), out=kv[:, first:], out_batch_stride=N, prep=prep)
        if fused:
            sc = api.compress_index(pkv, d(cik), cfg.m, r0p, first, qd, qs, wd, ik, iks, _pos(pos0), fmt,
                                    bound=bound, score_fmt="bf16")
        else:
            api.compress_pair(pkv, dict(d(cik), out=ik[:, first:], out_batch_stride=N,
                                        out_scale=None if iks is None else iks[:, first:],
                                        out_fmt=None if fmt == "bf16" else fmt), cfg.m, r0p, first, 1)
            sc = api.index(qd, qs, wd, ik, iks, _pos(pos0), cfg.m, fmt, bound=bound, score_fmt="bf16")
        torch.cuda.synchronize()
        assert sc.dtype == torch.bfloat16
        outs.append((kv, ik, iks, sc, bound))
    bits = lambda t: None if t is None else (t.view(torch.int16) if t.dtype == torch.bfloat16 else
                                            t.contiguous().view(torch.uint8))
    for a_, b_ in zip(*outs):
        if a_ is not None:
            assert torch.equal(bits(a_), bits(b_))


def _topk_bf16_case(api, bits, pos0, m, k, name, bound=None):
    """Top-k of bf16 scores against the oracle's top-k of the same bf16 values (bit-exact indices;
    values are the exact float32 of each selected bf16 score)."""
    say(f"topk bf16 {name} shape={bits.shape} k={k} bound={'none' if bound is None else 'given'}")
    vals64 = oracle.decode_bf16(bits)
    if isinstance(bound, str):
        bound = host_bound(vals64.astype(np.float32), pos0, m)
    bd = None if bound is None else dev(np.ascontiguousarray(bound).view(np.int32))
    idx, vals = api.topk(_to_bf16_dev(bits), _pos(pos0), m, k, want_vals=True, bound=bd)
    torch.cuda.synchronize()
    ref = oracle.topk(vals64, pos0, m, k)
    got = idx.cpu().numpy()
    assert np.array_equal(got, ref), f"{name}: {np.argwhere(got != ref)[:5]}"
    v = vals.cpu().numpy()
    for b in range(got.shape[0]):
        for r in range(got.shape[1]):
            sel = got[b, r][got[b, r] >= 0]
            assert np.array_equal(v[b, r, :len(sel)], (vals64[b, r, sel] + 0.0).astype(np.float32))
            assert np.all(v[b, r, len(sel):] == -np.inf)


@pytest.mark.parametrize("bound", [None, "index"])
def test_topk_bf16_split_path(api, bound):
    """Split (histogram) and bound-key paths on bf16 scores: many natural ties, +0/-0 runs, ragged
    visibility, a row longer than the cache (visibility capped)."""
    rng = np.random.default_rng(31)
    N = 262144
    x = rng.standard_normal((4, 1, N))
    x[0, 0, ::7] = 0.0
    x[0, 0, 3::7] = -0.0
    bits = oracle.encode_bf16(x)
    pos0 = [4 * N, 4 * (N - 1000) + 3, 4 * 20000, 4 * N + 100]
    _topk_bf16_case(api, bits, pos0, 4, 1024, "split path", bound)


def test_topk_bf16_bound_adversarial(api):
    """Bound keys over bf16 scores: ascending scores, a bound of zeros, and keys above every score."""
    rng = np.random.default_rng(32)
    N = 100000
    x = rng.standard_normal((3, 1, N))
    x[0, 0] = np.arange(N) / N
    x[2, 0] = np.round(x[2, 0] * 4) / 4
    bits = oracle.encode_bf16(x)
    pos0 = [4 * N, 4 * N - 1, 4 * (N - 3333)]
    _topk_bf16_case(api, bits, pos0, 4, 1024, "bound: ascending / random / coarse", "index")
    nb = 8 * ((N + 1023) // 1024)
    _topk_bf16_case(api, bits, pos0, 4, 1024, "bound of zeros", np.zeros((3, 1, nb), np.uint32))
    _topk_bf16_case(api, bits, pos0, 4, 1024, "bound above the scores", np.full((3, 1, nb), 0xFFFFFFF0, np.uint32))


def test_topk_bf16_row_path_and_edges(api):
    """Per-row path (many query rows), k = 1, all-equal rows (k > number of distinct values), a row width
    that is not a multiple of 4, and a split-path all-equal row with k above the visible count."""
    rng = np.random.default_rng(33)
    s2 = oracle.encode_bf16(rng.standard_normal((2, 70, 300)))
    s2[1, :, :150] = 0
    _topk_bf16_case(api, s2, [0, 4 * 299], 4, 1, "row path k=1")
    _topk_bf16_case(api, s2, [0, 4 * 299], 4, 64, "row path k=64 with zeros")
    s3 = oracle.encode_bf16(rng.standard_normal((1, 3, 50001)))
    _topk_bf16_case(api, s3, [4 * 50001 - 2], 4, 700, "row path, odd width")
    s4 = oracle.encode_bf16(rng.standard_normal((3, 1, 40000)))
    s4[1] = oracle.encode_bf16(np.full((1, 40000), 1.5))
    _topk_bf16_case(api, s4, [4 * 40000, 4 * 40000, 4 * 100], 4, 2048, "split path all-equal, k > V")


@pytest.mark.parametrize("name,scale", [("c3", dict(B=2, n_comp=65536)), ("c2", dict(B=4)),
                                        ("c5", dict(B=2, n_comp=65536))])
def test_bf16_score_recall(api, name, scale):
    """Recall of the bf16-score selection against the float64 oracle's selection of the same entries
    (same quantized indexer inputs), next to the float32-score selection's.  Rounding to bf16 (at most
    2^-8 of a score) may swap entries whose scores lie within that band of a row's k-th score, and
    only those: every entry gained or lost must pass that gap rule.  The recall itself depends on how
    densely scores crowd the k-th one; seeded Gaussian-like inputs crowd it more than a trained
    indexer, so it is reported, not held to the pages' figure."""
    cfg = configs.get_config(name).scaled(**scale)
    N = cfg.n_comp
    pos0 = [4 * N] * cfg.B
    say(f"bf16 score recall {cfg.name} B={cfg.B} N={N} k={cfg.k}")
    kc, qi, w = _index_inputs(cfg)
    qv = oracle.dequant_rows(qi["data"], qi.get("scale"), cfg.idx_dtype)
    kv = oracle.dequant_rows(kc["data"], kc.get("scale"), cfg.idx_dtype)
    ref_scores = oracle.index(qv, w, kv, pos0, cfg.m)
    ref_sel = oracle.topk(ref_scores, pos0, cfg.m, cfg.k)
    rec, bad = {}, {}
    for sf, rule in (("f32", 1e-3), ("bf16", 2.0 ** -7 + 1e-3)):
        sc = _run_index(api, cfg, kc, qi, w, pos0, sf)
        idx, _ = api.topk(sc, _pos(pos0), cfg.m, cfg.k)
        torch.cuda.synchronize()
        rec[sf], bad[sf] = topk_agreement(idx.cpu().numpy(), ref_sel, ref_scores, rule)
    say(f"recall vs float64 selection: f32 scores {rec['f32']:.5f}  bf16 scores {rec['bf16']:.5f}")
    assert bad["f32"] == 0 and bad["bf16"] == 0, bad
    assert rec["f32"] >= 0.999


@pytest.mark.parametrize("n_comp", [65536, 5037])
def test_topk_compress_matches_separate(api, n_comp):
    """The decode step with the KV entry moved into the selection's launch (csa_compress_index with the indexer
    key alone, then csa_topk_compress) writes the same caches, scores, bound keys and selection as
    csa_compress_index with both jobs followed by csa_topk; 65,536 entries take the bound-key launch (one extra
    workgroup per row), 5,037 the row path (the entry in a launch of its own)."""
    cfg = configs.C3.scaled(B=3, n_comp=n_comp)
    fmt, N = cfg.idx_dtype, cfg.n_comp
    say(f"topk_compress {cfg.name} N={N}")
    ckv, cik = gen.compress_inputs(cfg), gen.compress_inputs(cfg, indexer=True)
    first, r0p = N - 1, 4 * N - 8
    kc = gen.indexer_key_cache(cfg)
    qi, w = gen.indexer_queries(cfg)
    pos0 = [4 * N, 4 * N + 3, 4 * (N - 100)]
    d = lambda ci: {k: dev(ci[k]) for k in ("ca", "cb", "za", "zb", "bias_a", "bias_b")}
    prep = api.kv_prep(cfg.rope_dims, cfg.eps, cfg.rope_base)
    kv0 = dev(gen.kv_cache(cfg))
    outs = []
    for fused in (False, True):
        kv, ik, iks = kv0.clone(), dev(kc["data"]), dev(kc["scale"])
        bound = api.bound_keys(cfg.B, 1, N, DEV)
        qd, qs, wd = dev(qi["data"]), dev(qi["scale"]), dev(w)
        pkv = dict(d(ckv), out=kv[:, first:], out_batch_stride=N, prep=prep)
        if fused:
            sc = api.compress_index(None, d(cik), cfg.m, r0p, first, qd, qs, wd, ik, iks, _pos(pos0), fmt, bound=bound)
            idx = api.topk_compress(sc, _pos(pos0), cfg.m, cfg.k, pkv, r0p, first, bound=bound)
        else:
            sc = api.compress_index(pkv, d(cik), cfg.m, r0p, first, qd, qs, wd, ik, iks, _pos(pos0), fmt, bound=bound)
            idx, _ = api.topk(sc, _pos(pos0), cfg.m, cfg.k, bound=bound)
        torch.cuda.synchronize()
        outs.append((kv, ik, iks, sc, bound, idx))
    for a_, b_ in zip(*outs):
        assert torch.equal(a_.contiguous().view(torch.uint8), b_.contiguous().view(torch.uint8))
