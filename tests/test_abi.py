"""The C-ABI library loads, exports every symbol include/csa.h declares, and rejects bad arguments
on the host (no device work: these calls return before any HIP runtime call)."""
import ctypes as C
import os
import re

import pytest

from long_context_sparse_04_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "csa.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        from long_context_sparse_04_amd import build
        build.build()
    return _lib.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+char\s*\*|csa_status|size_t|int64_t|int)\s+(\w+)\s*\(", text, flags=re.M)
    return set(names)


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert names == set(_lib.SIGNATURES), names ^ set(_lib.SIGNATURES)
    raw = C.CDLL(_lib.LIB_PATH)
    for n in names:
        assert hasattr(raw, n), n


def test_status_strings_and_version(lib):
    assert lib.csa_abi_version() == 7
    for code in range(6):
        s = lib.csa_status_string(code).decode()
        assert s.startswith(_lib.STATUS[code])
    assert lib.csa_status_string(99).decode() == "unknown csa_status"


DUMMY = C.c_void_p(0x1000)  # never dereferenced: validation fails before any launch


def test_compress_validation(lib):
    f = lib.csa_compress
    args = dict(ca=DUMMY, cb=DUMMY, za=DUMMY, zb=DUMMY, ba=DUMMY, bb=DUMMY, B=1, rows=8, c=128, m=4, row0=0, first=1,
                num=1, in_t=1, out=DUMMY, osc=None, out_t=1, stride=0, prep=None, stream=None)

    def call(**kw):
        a = {**args, **kw}
        return f(a["ca"], a["cb"], a["za"], a["zb"], a["ba"], a["bb"], a["B"], a["rows"], a["c"], a["m"], a["row0"],
                 a["first"], a["num"], a["in_t"], a["out"], a["osc"], a["out_t"], a["stride"], a["prep"], a["stream"])

    assert call(B=-1) == 2
    assert call(c=130) == 2
    assert call(m=0) == 2
    assert call(in_t=2) == 3
    assert call(out_t=3, c=100) == 3
    assert call(ca=None) == 1
    prep = C.byref(_lib.KvPrep(None, 1e-6, 64, 1e4))
    assert call(prep=prep, out_t=2, osc=DUMMY) == 3        # prepared entries: F32, BF16 or fp8 + bf16 RoPE
    assert call(out_t=4, osc=DUMMY) == 3                   # the fp8 + bf16 RoPE rows are prepared rows
    assert call(prep=prep, out_t=4, osc=None) == 1          # and need their scales
    assert call(prep=C.byref(_lib.KvPrep(None, 1e-6, 56, 1e4)), out_t=4, osc=DUMMY) == 3   # c - R % 16
    assert call(prep=C.byref(_lib.KvPrep(None, 1e-6, 60, 1e4))) == 3
    assert call(prep=C.byref(_lib.KvPrep(None, -1.0, 64, 1e4))) == 2
    # csa_prepare_kv
    pk = lib.csa_prepare_kv
    assert pk(DUMMY, 8, DUMMY, None, 8, 2, 8, 512, 1, 1, None, 0, 4, None, None) == 1
    assert pk(DUMMY, 8, DUMMY, None, 8, 2, 8, 510, 1, 1, None, 0, 4, prep, None) == 2
    assert pk(DUMMY, 8, DUMMY, None, 8, 2, 8, 512, 2, 1, None, 0, 4, prep, None) == 3
    assert pk(DUMMY, 4, DUMMY, None, 8, 2, 8, 512, 1, 1, None, 0, 4, prep, None) == 2   # batch stride below rows
    assert pk(DUMMY, 8, DUMMY, None, 8, 2, 8, 512, 1, 0, None, 0, 4, prep, None) == 2   # in place needs one layout
    assert pk(DUMMY, 8, DUMMY, None, 8, 0, 8, 512, 1, 1, None, 0, 4, prep, None) == 0
    assert pk(DUMMY, 8, DUMMY, None, 8, 2, 8, 512, 1, 4, None, 0, 4, prep, None) == 1   # fp8 + bf16 RoPE: scales
    assert pk(DUMMY, 8, DUMMY, None, 8, 2, 8, 512, 1, 5, None, 0, 4, prep, None) == 3
    assert call(cb=None) == 1                     # b-stream must be all or nothing
    assert call(out_t=2, osc=None) == 1           # fp8 needs the scale output
    assert call(first=2) == 2                     # entry 2 needs rows 4..11 but only 0..7 exist
    assert call(row0=1) == 2                      # entry 1's b-rows start at 0 < row0
    assert call(stride=0, num=0) == 0             # nothing to do
    assert call(B=0) == 0


def test_compress_pair_validation(lib):
    P = DUMMY

    def pair(**kw):
        a = dict(c0=512, c1=128, t0=1, t1=2, os1=P, B=4, rows=8, m=4, r0=1048568, first=262143, n=1, in_t=1)
        a.update(kw)
        return lib.csa_compress_pair(P, P, P, P, P, P, a["c0"], P, None, a["t0"], 262144, None,
                                     P, P, P, P, P, P, a["c1"], P, a["os1"], a["t1"], 262144, None,
                                     a["B"], a["rows"], a["m"], a["r0"], a["first"], a["n"], a["in_t"], None)
    assert pair(os1=None) == 1          # fp8 output of problem 1 needs its scales
    assert pair(c1=130) == 2
    assert pair(t1=3, c1=48) == 3       # MXFP4 needs a width in multiples of 32
    assert pair(r0=1048569) == 2        # entry 262143 reads rows from 1048568 on
    assert pair(in_t=2) == 3
    assert pair(n=0) == 0 and pair(B=0) == 0


def test_index_topk_attend_validation(lib):
    assert lib.csa_index(DUMMY, None, DUMMY, DUMMY, None, 1, 1, 64, 128, 1000, DUMMY, 4, 7, DUMMY, 0, None, None) == 3
    assert lib.csa_index(DUMMY, None, DUMMY, DUMMY, None, 1, 1, 48, 128, 1000, DUMMY, 4, 1, DUMMY, 0, None, None) == 3
    assert lib.csa_index(DUMMY, None, DUMMY, DUMMY, None, 1, 1, 64, 64, 1000, DUMMY, 4, 2, DUMMY, 0, None, None) == 3
    assert lib.csa_index(DUMMY, None, DUMMY, DUMMY, None, 1, 1, 64, 128, 1000, DUMMY, 4, 2, DUMMY, 0, None, None) == 1
    assert lib.csa_index(None, None, DUMMY, DUMMY, None, 1, 1, 64, 128, 1000, DUMMY, 4, 1, DUMMY, 0, None, None) == 1
    assert lib.csa_index(DUMMY, None, DUMMY, DUMMY, None, 1, 1, 64, 128, -1, DUMMY, 4, 1, DUMMY, 0, None, None) == 2
    # top-k
    nb = lib.csa_topk_workspace_bytes(4, 1, 262144, 1024)
    assert nb >= 4 * 262144 * 8
    assert lib.csa_topk_workspace_bytes(1, 4096, 17408, 512) == 0     # row path needs none
    assert lib.csa_topk(DUMMY, 0, 4, 1, 262144, DUMMY, 4, 1024, None, DUMMY, None, None, 0, None) == 4
    assert lib.csa_topk(DUMMY, 0, 4, 1, 262144, DUMMY, 4, 1024, None, DUMMY, None, DUMMY, nb - 1, None) == 4
    assert lib.csa_topk(DUMMY, 0, 4, 1, 262144, DUMMY, 4, 0, None, DUMMY, None, DUMMY, nb, None) == 2
    assert lib.csa_topk(DUMMY, 0, 4, 1, 262144, DUMMY, 4, 4096, None, DUMMY, None, DUMMY, nb, None) == 2
    assert lib.csa_topk(DUMMY, 0, 4, 1, 262144, None, 4, 1024, None, DUMMY, None, DUMMY, nb, None) == 1
    assert lib.csa_index(DUMMY, C.c_void_p(0x1002), DUMMY, DUMMY, DUMMY, 1, 1, 64, 128, 1000, DUMMY, 4, 3, DUMMY,
                         0, None, None) == 2           # MXFP4 query scales are read as aligned 32-bit words
    # bound keys: two per bound set (256 entries, or 32 for caches of up to 65536 entries; per 1024 entries
    # 8 or 64 keys), from the MFMA kernels (decode and tiled prefill) only, 8-byte aligned
    assert lib.csa_index_bound_keys(262144) == 2048 and lib.csa_index_bound_keys(1000) == 64
    assert lib.csa_index_bound_keys(65536) == 4096 and lib.csa_index_bound_keys(65537) == 520
    assert lib.csa_index_bound_keys(17408) == 1088
    assert lib.csa_index_bound_keys(0) == 0
    assert lib.csa_index(DUMMY, None, DUMMY, DUMMY, None, 1, 1, 32, 128, 1000, DUMMY, 4, 0, DUMMY, 0,
                         DUMMY, None) == 3                 # float32 path: no bound keys
    assert lib.csa_index(DUMMY, None, DUMMY, DUMMY, None, 1, 1, 64, 128, 1000, DUMMY, 4, 1, DUMMY, 0,
                         C.c_void_p(0x1004), None) == 2
    # scores: float32 or bf16 only
    assert lib.csa_index(DUMMY, None, DUMMY, DUMMY, None, 1, 1, 64, 128, 1000, DUMMY, 4, 1, DUMMY, 2, None,
                         None) == 3
    assert lib.csa_topk(DUMMY, 2, 4, 1, 262144, DUMMY, 4, 1024, None, DUMMY, None, DUMMY, nb, None) == 3
    # compress_index: the MFMA formats only, entries of m < 64 rows, the new entry inside the cache
    def ci(**kw):
        a = dict(m=4, first=1023, n=1024, qk=2, q=DUMMY, rows=8, r0=4088, st=0)
        a.update(kw)
        return lib.csa_compress_index(DUMMY, DUMMY, DUMMY, DUMMY, DUMMY, DUMMY, 512, DUMMY, None, 1, 0, None,
                                      DUMMY, DUMMY, DUMMY, DUMMY, DUMMY, DUMMY, 4, a["rows"], a["m"], a["r0"],
                                      a["first"], 1, a["q"], DUMMY, DUMMY, DUMMY, DUMMY, 64, 128, a["n"], DUMMY,
                                      a["qk"], DUMMY, a["st"], None, None)
    assert ci(qk=0) == 3 and ci(m=128) == 3
    assert ci(first=1024) == 2 and ci(first=-1) == 2
    assert ci(q=None) == 1
    assert ci(r0=4096) == 2                   # the entry reads rows before row0_pos
    assert ci(st=3) == 3
    # attend
    ws = lib.csa_attend_workspace_bytes(4, 1, 128, 512, 1024, 128)
    assert ws > 0 and lib.csa_attend_workspace_bytes(1, 4096, 64, 512, 512, 128) == 0

    def att(**kw):
        a = dict(q=DUMMY, comp=DUMMY, idx=DUMMY, win=DUMMY, sink=DUMMY, B=4, T=1, H=128, c=512, R=64, k=1024,
                 n_win=128, N=262144, pos=DUMMY, m=4, kv_t=1, out=DUMMY, out_t=1, ws=None, nb=0, prep=0, ct=None,
                 cs=None)
        a.update(kw)
        ct = a["kv_t"] if a["ct"] is None else a["ct"]
        return lib.csa_attend(a["q"], a["comp"], a["cs"], a["idx"], a["win"], a["sink"], None, None, a["B"], a["T"],
                              a["H"], a["c"], a["R"], a["k"], a["n_win"], a["N"], a["pos"], a["m"], 0.044, 1e-6, 1e4,
                              a["kv_t"], ct, a["prep"], a["out"], a["out_t"], a["ws"], a["nb"], None)
    assert att() == 4                         # decode needs the split workspace
    assert att(c=192) == 3
    assert att(R=60) == 3
    assert att(H=40) == 3                     # bf16 path: heads in multiples of 16
    assert att(kv_t=2) == 3
    assert att(k=0) == 2
    assert att(q=None, ws=DUMMY, nb=ws) == 1
    assert att(prep=3, ws=DUMMY, nb=ws) == 3 and att(prep=-1, ws=DUMMY, nb=ws) == 3   # kv_prepared is 0, 1 or 2
    # fp8 + bf16 RoPE compressed rows: bf16 queries, prepared entries, scales, c - R a multiple of 16
    assert att(ct=4, prep=1, ws=DUMMY, nb=ws) == 1
    assert att(ct=4, prep=0, cs=DUMMY, ws=DUMMY, nb=ws) == 3
    assert att(ct=4, prep=1, cs=DUMMY, R=56, ws=DUMMY, nb=ws) == 3
    assert att(ct=4, kv_t=0, prep=1, cs=DUMMY, ws=DUMMY, nb=ws) == 3
    assert att(ct=2, prep=1, cs=DUMMY, ws=DUMMY, nb=ws) == 3
    assert lib.hca_attend(DUMMY, DUMMY, None, DUMMY, DUMMY, None, None, 8, 1, 128, 512, 64, 128, 8192, DUMMY, 128, 0.044,
                          1e-6, 1e4, 1, 1, 3, DUMMY, 1, None, 0, None) == 3
    assert lib.hca_attend(DUMMY, DUMMY, None, DUMMY, DUMMY, None, None, 8, 1, 128, 512, 64, 128, 8192, DUMMY, 128, 0.044,
                          1e-6, 1e4, 1, 4, 2, DUMMY, 1, DUMMY, 1 << 30, None) == 1
    assert lib.hca_attend_workspace_bytes(8, 1, 128, 512, 8192, 128) > 0


def _pages(table=DUMMY, max_pages=4, page_tokens=1024):
    return _lib.Pages(table, max_pages, page_tokens)


def test_decode_append_validation(lib):
    """csa_decode_append: job / window shapes, the page map, the thread-count class of the jobs."""
    def job(**kw):
        a = dict(ca=DUMMY, cb=DUMMY, za=DUMMY, zb=DUMMY, bias_a=DUMMY, bias_b=DUMMY, c=512, m=4, ring_ca=DUMMY,
                 ring_cb=DUMMY, ring_za=DUMMY, ring_zb=DUMMY, out=DUMMY, out_scale=None, out_t=1, prep=None)
        a.update(kw)
        return _lib.AppendJob(**a)

    def call(jobs, wins=(), B=2, pos=DUMMY, pages=None, in_t=1):
        ja = (_lib.AppendJob * max(1, len(jobs)))(*jobs)
        wa = (_lib.WindowJob * max(1, len(wins)))(*wins)
        pg = _pages() if pages is None else pages
        return lib.csa_decode_append(ja, len(jobs), wa, len(wins), B, pos, C.byref(pg), in_t, None)

    hca = job(cb=None, zb=None, bias_b=None, ring_cb=None, ring_zb=None, m=128)
    assert call([job(), job(c=128)], B=0) == 0                   # nothing to do
    assert call([], B=2) == 2                                     # at least one job
    assert call([job(), job(), job()]) == 2                       # at most two
    assert call([job(c=130)]) == 2
    assert call([job(m=0)]) == 2
    assert call([job(), hca]) == 3                                # mixed thread-count classes
    assert call([job()], in_t=2) == 3
    assert call([job(ring_za=None)]) == 1
    assert call([job(ring_cb=None)]) == 1                         # half an overlapped job
    assert call([job(out_t=2)]) == 1                              # fp8 output needs its scales
    assert call([job(out_t=4)]) == 3                              # fp8 + bf16 RoPE needs prepared entries
    assert call([job()], pages=_pages(page_tokens=96)) == 2       # not a power of two / multiple of 128
    assert call([job()], pages=_pages(page_tokens=64)) == 2
    assert call([job()], pages=_pages(table=None)) == 1
    assert call([job()], pos=None) == 1
    assert call([job()], wins=[_lib.WindowJob(DUMMY, DUMMY, 512, 0, None)]) == 2   # empty window ring
    assert call([job()], wins=[_lib.WindowJob(None, DUMMY, 512, 128, None)]) == 1


def test_paged_index_attend_validation(lib):
    """csa_index_paged / csa_attend_paged / hca_attend_paged: formats, the page map and its coverage."""
    pg = _pages(max_pages=4, page_tokens=1024)                  # 4 pages of 256 CSA entries, 8 HCA entries
    P = C.byref(pg)

    def index(n_max=1000, qk_t=2, pages=P, HI=64, cI=128, q=DUMMY):
        return lib.csa_index_paged(q, DUMMY, DUMMY, DUMMY, DUMMY, pages, 2, HI, cI, n_max, DUMMY, 4, qk_t, DUMMY, 0,
                                   None, None)

    assert index(qk_t=0) == 3                                     # the MFMA formats only
    assert index(n_max=1025) == 2                                 # more entries than the mapped pages hold
    assert index(cI=64) == 3
    assert index(q=None) == 1
    bad = _pages(page_tokens=1000)
    assert index(pages=C.byref(bad)) == 2

    def attend(n_max=1000, kv_t=1, comp_t=1, prep=1, pages=P, m=4, k=512):
        return lib.csa_attend_paged(DUMMY, DUMMY, None, pages, DUMMY, DUMMY, DUMMY, None, None, 2, 64, 512, 64, k, 128,
                                    n_max, DUMMY, m, 0.04, 1e-6, 1e4, kv_t, comp_t, prep, DUMMY, 1, DUMMY, 1 << 30,
                                    None)

    assert attend(kv_t=0, comp_t=0) == 3                          # bf16 only
    assert attend(n_max=1025) == 2
    assert attend(comp_t=4) == 1                                  # mixed rows need their scales
    assert attend(comp_t=4, prep=0) == 3                          # ... and prepared entries
    assert attend(m=3) == 2                                       # page_tokens must be a multiple of m

    def hca(n_max=32, m_hca=128, pages=P):
        return lib.hca_attend_paged(DUMMY, DUMMY, None, pages, DUMMY, DUMMY, None, None, 2, 128, 512, 64, 128, n_max,
                                    DUMMY, m_hca, 0.04, 1e-6, 1e4, 1, 1, 2, DUMMY, 1, DUMMY, 1 << 30, None)

    assert hca(n_max=33) == 2                                     # 4 pages x 8 HCA entries
    assert hca(m_hca=2048) == 2


def test_projection_validation(lib):
    f = lib.csa_q_up_proj
    ok = lambda **kw: dict(dict(rows=4, d_c=1536, n_h=16, c=512, n_hI=64, cI=128, qi_t=2), **kw)

    def q(**kw):
        a = ok(**kw)
        return f(DUMMY, DUMMY, DUMMY, a["rows"], a["d_c"], a["n_h"], a["c"], a["n_hI"], a["cI"], DUMMY, DUMMY,
                 DUMMY, a["qi_t"], None)

    assert q(rows=0) == 0
    assert q(rows=-1) == 2
    assert q(d_c=1000) == 2                     # d_c a multiple of 32
    assert q(cI=64) == 3                        # quantized indexer queries: heads of 128
    assert q(qi_t=0) == 3
    assert f(DUMMY, None, DUMMY, 4, 1536, 16, 512, 64, 128, DUMMY, DUMMY, DUMMY, 1, None) == 1
    assert f(DUMMY, DUMMY, DUMMY, 4, 1536, 16, 512, 64, 128, DUMMY, DUMMY, None, 2, None) == 1   # fp8 scales
    odd = C.c_void_p(0x1008)
    assert f(odd, DUMMY, DUMMY, 4, 1536, 16, 512, 64, 128, DUMMY, DUMMY, None, 1, None) == 3    # 16-byte operands
    assert f(DUMMY, DUMMY, DUMMY, 4, 1536, 16, 512, 64, 128, C.c_void_p(0x1004), DUMMY, None, 1, None) == 3
    g = lib.csa_grouped_out_proj
    assert g(DUMMY, DUMMY, DUMMY, 4, 128, 512, 12, 1024, 7168, DUMMY, DUMMY, None) == 2    # g must divide n_h
    assert g(DUMMY, DUMMY, DUMMY, 4, 128, 512, 16, 1000, 7168, DUMMY, DUMMY, None) == 3    # d_g % 16
    assert g(DUMMY, DUMMY, DUMMY, -1, 128, 512, 16, 1024, 7168, DUMMY, DUMMY, None) == 2
    assert g(DUMMY, DUMMY, DUMMY, 0, 128, 512, 16, 1024, 7168, DUMMY, DUMMY, None) == 0
    assert g(DUMMY, DUMMY, DUMMY, 4, 128, 512, 16, 1024, 7168, None, DUMMY, None) == 1
    assert g(DUMMY, DUMMY, DUMMY, 4, 128, 512, 16, 1024, 7168, odd, DUMMY, None) == 3       # 16-byte mid


def test_fused_decode_entry_validation(lib):
    """csa_topk_compress and csa_append_index_paged reject bad arguments before any launch."""
    tk = lib.csa_topk_compress

    def t(**kw):
        a = dict(st=0, B=4, n=262144, m=4, k=1024, ws=1 << 30, c=512, rows=8, row0=4 * 262144 - 8, first=262143,
                 in_t=1, out=DUMMY, out_t=1)
        a.update(kw)
        return tk(DUMMY, a["st"], a["B"], a["n"], DUMMY, a["m"], a["k"], DUMMY, DUMMY, None, DUMMY, a["ws"], DUMMY,
                  DUMMY, DUMMY, DUMMY, DUMMY, DUMMY, a["c"], a["rows"], a["row0"], a["first"], a["in_t"], a["out"], None,
                  a["out_t"], 0, None, None)

    assert t(m=64) == 3                 # one 256-thread workgroup pools the entry
    assert t(st=2) == 3                 # scores f32 or bf16
    assert t(k=0) == 2
    assert t(out=None) == 1
    assert t(ws=0) == 4                 # the top-k workspace
    assert t(row0=0) == 2               # the entry's rows outside the streams
    ja = (_lib.AppendJob * 2)()
    pg = _pages()
    ai = lib.csa_append_index_paged
    # no jobs described (null stream pointers): rejected before the index checks
    assert ai(ja, None, 1, DUMMY, DUMMY, DUMMY, DUMMY, DUMMY, C.byref(pg), 2, 64, 128, 1000, DUMMY, 4, 2, DUMMY, 0,
              None, None) in (1, 2)


def test_attend_noalloc_rejects_oversize_workspace(lib):
    """csa_attend_noalloc returns CSA_ERR_WORKSPACE, without touching a device, when the decode partials would
    exceed its 64 MiB array; argument errors come first, as in csa_attend."""
    B, H, c, k, n_win = 60000, 128, 512, 1024, 128
    assert lib.csa_attend_workspace_bytes(B, 1, H, c, k, n_win) > (64 << 20)
    d = C.c_void_p(16)     # never dereferenced
    call = lambda **kw: lib.csa_attend_noalloc(d, d, None, d, d, d, None, None, kw.get("B", B), 1, H, c, 64, k, n_win,
                                               262144, kw.get("pos", d), 4, 0.04, 1e-6, 10000.0, 1, 1, 1, d, 1, None)
    assert call() == 4                      # CSA_ERR_WORKSPACE
    assert call(pos=None) == 1              # CSA_ERR_NULL before the size check
    assert call(B=0) == 0                   # nothing to do
