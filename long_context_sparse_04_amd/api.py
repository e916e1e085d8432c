"""Thin torch-facing binding of the C ABI (include/csa.h): argument marshalling only.

Every computation runs in the HIP kernels of libcsa.so; these wrappers check
that tensors are contiguous device tensors, pass their pointers and the current
stream, and raise CSAError on a non-zero status.  bf16 data travels as
torch.bfloat16 (bit patterns), fp8 / MXFP4 data as torch.uint8.
"""
from __future__ import annotations

import ctypes as C

import torch

from . import _lib
from ._lib import CSAError

FMT = {"f32": _lib.F32, "bf16": _lib.BF16, "fp8": _lib.FP8_E4M3_ROWSCALE, "mxfp4": _lib.MXFP4_E8M0_B32,
       "fp8rope": _lib.FP8_BF16_ROPE}
_TORCH_FMT = {torch.float32: "f32", torch.bfloat16: "bf16"}

_ws_cache: dict = {}


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise CSAError("tensor must live on the GPU")
    if not t.is_contiguous():
        raise CSAError("tensor must be contiguous")
    return t.data_ptr()


def _dptr(t):
    """Device address of a tensor that may be a strided view (rows at a batch stride the call is given)."""
    if t is None:
        return None
    if not t.is_cuda:
        raise CSAError("tensor must live on the GPU")
    return t.data_ptr()


def _ws_bytes(ws):
    """The size the library may use: the workspace tensor's own."""
    return 0 if ws is None else ws.numel() * ws.element_size()


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def workspace(nbytes: int, device, key: str, zero: bool = False) -> torch.Tensor | None:
    """Reusable device workspace per (key, device); zero-filled once when asked."""
    if nbytes == 0:
        return None
    k = (key, str(device))
    ws = _ws_cache.get(k)
    if ws is None or ws.numel() < nbytes:
        ws = torch.zeros(nbytes, dtype=torch.uint8, device=device) if zero else torch.empty(
            nbytes, dtype=torch.uint8, device=device)
        _ws_cache[k] = ws
    return ws


def kv_prep(rope_dims, eps=1e-6, rope_base=10000.0, gamma=None):
    """A csa_kv_prep (keep the returned object alive while the call that uses it is made)."""
    p = _lib.KvPrep(_ptr(gamma), eps, rope_dims, rope_base)
    p._gamma = gamma
    return p


def _prep_arg(prep):
    return None if prep is None else C.byref(prep)


def compress(ca, cb, za, zb, bias_a, bias_b, m, row0_pos, first_entry, num_entries, out=None, out_scale=None,
             out_fmt=None, out_batch_stride=0, prep=None, stream=None):
    """csa_compress.  ca/za (and cb/zb for CSA) are [B][rows][c] f32 or bf16 tensors; prep (kv_prep) stores the
    entries prepared for attention."""
    lib = _lib.load()
    B, rows, c = ca.shape
    in_fmt = _TORCH_FMT[ca.dtype]
    out_fmt = out_fmt or in_fmt
    dev = ca.device
    if out is None:
        if out_fmt == "f32":
            out = torch.empty((B, num_entries, c), dtype=torch.float32, device=dev)
        elif out_fmt == "bf16":
            out = torch.empty((B, num_entries, c), dtype=torch.bfloat16, device=dev)
        elif out_fmt == "fp8":
            out = torch.empty((B, num_entries, c), dtype=torch.uint8, device=dev)
            out_scale = torch.empty((B, num_entries), dtype=torch.float32, device=dev)
        elif out_fmt == "fp8rope":   # prepared entries: c - R fp8 bytes + R bf16 RoPE dims, one scale per row
            out = torch.empty((B, num_entries, c + prep.rope_dims), dtype=torch.uint8, device=dev)
            out_scale = torch.empty((B, num_entries), dtype=torch.float32, device=dev)
        else:
            out = torch.empty((B, num_entries, c // 2), dtype=torch.uint8, device=dev)
            out_scale = torch.empty((B, num_entries, c // 32), dtype=torch.uint8, device=dev)
    st = lib.csa_compress(_ptr(ca), _ptr(cb), _ptr(za), _ptr(zb), _ptr(bias_a), _ptr(bias_b), B, rows, c, m,
                          row0_pos, first_entry, num_entries, FMT[in_fmt], out.data_ptr(),
                          None if out_scale is None else out_scale.data_ptr(), FMT[out_fmt], out_batch_stride,
                          _prep_arg(prep), _stream(stream))
    _lib.check(st, "csa_compress")
    return out, out_scale


def _compress_out(B, num_entries, c, fmt, dev, rope_dims=0):
    if fmt == "f32":
        return torch.empty((B, num_entries, c), dtype=torch.float32, device=dev), None
    if fmt == "bf16":
        return torch.empty((B, num_entries, c), dtype=torch.bfloat16, device=dev), None
    if fmt == "fp8":
        return (torch.empty((B, num_entries, c), dtype=torch.uint8, device=dev),
                torch.empty((B, num_entries), dtype=torch.float32, device=dev))
    if fmt == "fp8rope":
        return (torch.empty((B, num_entries, c + rope_dims), dtype=torch.uint8, device=dev),
                torch.empty((B, num_entries), dtype=torch.float32, device=dev))
    return (torch.empty((B, num_entries, c // 2), dtype=torch.uint8, device=dev),
            torch.empty((B, num_entries, c // 32), dtype=torch.uint8, device=dev))


def compress_pair(p0, p1, m, row0_pos, first_entry, num_entries, stream=None):
    """csa_compress_pair: two compression problems (dicts with ca, cb, za, zb, bias_a, bias_b and optional out,
    out_scale, out_fmt, out_batch_stride, prep) of the same rows and entries in one launch.  Returns
    ((out0, scale0), (out1, scale1))."""
    lib = _lib.load()
    B, rows, _ = p0["ca"].shape
    in_fmt = _TORCH_FMT[p0["ca"].dtype]
    args, outs = [], []
    for p in (p0, p1):
        c = p["ca"].shape[2]
        fmt = p.get("out_fmt") or in_fmt
        out, osc = p.get("out"), p.get("out_scale")
        if out is None:
            prep = p.get("prep")
            out, osc = _compress_out(B, num_entries, c, fmt, p["ca"].device, prep.rope_dims if prep else 0)
        args += [_ptr(p["ca"]), _ptr(p.get("cb")), _ptr(p["za"]), _ptr(p.get("zb")), _ptr(p["bias_a"]),
                 _ptr(p.get("bias_b")), c, out.data_ptr(), None if osc is None else osc.data_ptr(), FMT[fmt],
                 p.get("out_batch_stride", 0), _prep_arg(p.get("prep"))]
        outs.append((out, osc))
    st = lib.csa_compress_pair(*args, B, rows, m, row0_pos, first_entry, num_entries, FMT[in_fmt], _stream(stream))
    _lib.check(st, "csa_compress_pair")
    return tuple(outs)


def compress_index(p_kv, p_ik, m, row0_pos, first_entry, q, q_scale, w, k, k_scale, pos0, fmt, scores=None,
                   bound=None, stream=None, score_fmt="f32"):
    """csa_compress_index: compress_pair(p_kv, p_ik) for entry first_entry (one per sequence) and a decode index
    (T = 1), one launch.  p_kv: dict as in compress_pair (out required: f32 / bf16, or uint8 rows in the fp8 +
    bf16 RoPE format with out_scale; optional out_batch_stride, prep); p_ik: the indexer-key streams, whose entry is written into k / k_scale at first_entry.  Returns
    the scores."""
    lib = _lib.load()
    B, rows, _ = p_ik["ca"].shape
    in_fmt = _TORCH_FMT[p_ik["ca"].dtype]
    if p_kv is None:   # the indexer key alone (the KV entry computed elsewhere, e.g. by topk_compress)
        p_kv = {"ca": None, "za": None, "bias_a": None, "out": None}
    c0 = 0 if p_kv["ca"] is None else p_kv["ca"].shape[2]
    HI = q.shape[2]
    cI = q.shape[3] * (2 if fmt == "mxfp4" else 1)
    N = k.shape[1]
    out0 = p_kv["out"]
    if scores is None:
        scores = _score_buf(B, 1, N, score_fmt, q.device)
    st = lib.csa_compress_index(
        _ptr(p_kv["ca"]), _ptr(p_kv.get("cb")), _ptr(p_kv["za"]), _ptr(p_kv.get("zb")), _ptr(p_kv["bias_a"]),
        _ptr(p_kv.get("bias_b")), c0, _dptr(out0), _dptr(p_kv.get("out_scale")),
        0 if out0 is None else (FMT["fp8rope"] if out0.dtype == torch.uint8 else FMT[_TORCH_FMT[out0.dtype]]),
        p_kv.get("out_batch_stride", 0),
        _prep_arg(p_kv.get("prep")),
        _ptr(p_ik["ca"]), _ptr(p_ik.get("cb")), _ptr(p_ik["za"]), _ptr(p_ik.get("zb")), _ptr(p_ik["bias_a"]),
        _ptr(p_ik.get("bias_b")),
        B, rows, m, row0_pos, first_entry, FMT[in_fmt],
        _ptr(q), _ptr(q_scale), _ptr(w), _ptr(k), _ptr(k_scale), HI, cI, N, _ptr(pos0), FMT[fmt], _ptr(scores),
        FMT[_TORCH_FMT[scores.dtype]], _ptr(bound), _stream(stream))
    _lib.check(st, "csa_compress_index")
    return scores


def bound_keys(B, T, n_max, device):
    """An int32 buffer [B][T][csa_index_bound_keys(n_max)] for the indexer's bound keys (uint32 bits)."""
    return torch.empty((B, T, _lib.load().csa_index_bound_keys(n_max)), dtype=torch.int32, device=device)


def _score_buf(B, T, N, score_fmt, device):
    return torch.empty((B, T, N), dtype=torch.bfloat16 if score_fmt == "bf16" else torch.float32, device=device)


def index(q, q_scale, w, k, k_scale, pos0, m, fmt, n_max=None, scores=None, stream=None, bound=None,
          score_fmt="f32"):
    """csa_index.  q [B][T][HI][row], k [B][N][row]; returns scores [B][T][N] (float32, or bf16 with
    score_fmt="bf16" / a bf16 scores tensor).  bound: optional buffer from bound_keys() that also
    receives the selector's lower-bound keys."""
    lib = _lib.load()
    B, T, HI = q.shape[0], q.shape[1], q.shape[2]
    cI = q.shape[3] * (2 if fmt == "mxfp4" else 1)
    N = k.shape[1] if n_max is None else n_max
    if scores is None:
        scores = _score_buf(B, T, N, score_fmt, q.device)
    st = lib.csa_index(_ptr(q), _ptr(q_scale), _ptr(w), _ptr(k), _ptr(k_scale), B, T, HI, cI, N, _ptr(pos0), m,
                       FMT[fmt], _ptr(scores), FMT[_TORCH_FMT[scores.dtype]], _ptr(bound), _stream(stream))
    _lib.check(st, "csa_index")
    return scores


def topk(scores, pos0, m, k, idx=None, vals=None, ws=None, stream=None, want_vals=False, bound=None):
    """csa_topk.  Returns (idx int32 [B][T][k], vals float32 or None).  bound: the keys csa_index wrote
    for these scores (optional; the same result, fewer kernels on long rows)."""
    lib = _lib.load()
    B, T, N = scores.shape
    dev = scores.device
    if idx is None:
        idx = torch.empty((B, T, k), dtype=torch.int32, device=dev)
    if vals is None and want_vals:
        vals = torch.empty((B, T, k), dtype=torch.float32, device=dev)
    nb = lib.csa_topk_workspace_bytes(B, T, N, k)
    if ws is None:
        ws = workspace(nb, dev, "topk", zero=True)
    if bound is not None and tuple(bound.shape) != (B, T, lib.csa_index_bound_keys(N)):
        raise CSAError(f"topk: bound shape {tuple(bound.shape)} does not match the scores")
    st = lib.csa_topk(_ptr(scores), FMT[_TORCH_FMT[scores.dtype]], B, T, N, _ptr(pos0), m, k, _ptr(bound),
                      _ptr(idx), _ptr(vals), _ptr(ws), _ws_bytes(ws), _stream(stream))
    _lib.check(st, "csa_topk")
    return idx, vals


def topk_compress(scores, pos0, m, k, p_kv, row0_pos, first_entry, idx=None, ws=None, bound=None, stream=None):
    """csa_topk_compress (decode rows): the selection and the KV entry first_entry of every sequence (p_kv as in
    compress_pair, out required) in one launch.  Returns idx."""
    lib = _lib.load()
    B, T, N = scores.shape
    if T != 1:
        raise CSAError("topk_compress: decode rows only (T = 1)")
    if idx is None:
        idx = torch.empty((B, 1, k), dtype=torch.int32, device=scores.device)
    nb = lib.csa_topk_workspace_bytes(B, 1, N, k)
    if ws is None:
        ws = workspace(nb, scores.device, "topk", zero=True)
    ca = p_kv["ca"]
    out = p_kv["out"]
    if out.dtype == torch.uint8:   # uint8 rows: the prepared fp8 + bf16 RoPE format, as compress_index infers it
        out_fmt = "fp8rope"
    else:
        out_fmt = p_kv.get("out_fmt") or _TORCH_FMT[out.dtype]
    prep = p_kv.get("prep")
    st = lib.csa_topk_compress(_ptr(scores), FMT[_TORCH_FMT[scores.dtype]], B, N, _ptr(pos0), m, k, _ptr(bound),
                               _ptr(idx), None, _ptr(ws), _ws_bytes(ws), _ptr(ca), _ptr(p_kv.get("cb")), _ptr(p_kv["za"]),
                               _ptr(p_kv.get("zb")), _ptr(p_kv["bias_a"]), _ptr(p_kv.get("bias_b")), ca.shape[2],
                               ca.shape[1], row0_pos, first_entry, FMT[_TORCH_FMT[ca.dtype]], _dptr(out),
                               _dptr(p_kv.get("out_scale")), FMT[out_fmt], p_kv.get("out_batch_stride", 0),
                               _prep_arg(prep), _stream(stream))
    _lib.check(st, "csa_topk_compress")
    return idx


def prepare_kv(x, prep, pos_first=0, pos_stride=1, pos_base=None, out=None, out_fmt=None, stream=None,
               out_scale=None):
    """csa_prepare_kv: rows x [B][rows][c] -> RoPE_pos(RMSNorm(x)), row j of sequence b at position
    (pos_base[b] if given) + pos_first + j * pos_stride.  out may be x itself (in place).  With
    out_fmt="fp8rope" the rows are stored as uint8 [B][rows][c + R] with float32 scales [B][rows], and
    (out, out_scale) is returned."""
    lib = _lib.load()
    B, rows, c = x.shape
    in_fmt = _TORCH_FMT[x.dtype]
    out_fmt = out_fmt or in_fmt
    mixed = out_fmt == "fp8rope"
    ob = c + prep.rope_dims if mixed else c   # output row length in elements of out's dtype
    if out is None:
        dt = torch.uint8 if mixed else (torch.float32 if out_fmt == "f32" else torch.bfloat16)
        out = torch.empty((B, rows, ob), dtype=dt, device=x.device)
    if mixed and out_scale is None:
        out_scale = torch.empty((B, rows), dtype=torch.float32, device=x.device)
    if tuple(out.shape) != (B, rows, ob):
        raise CSAError(f"prepare_kv: out shape {tuple(out.shape)} is not {(B, rows, ob)}")
    # rows of one sequence contiguous; sequences may sit at any row stride (the strides of size-1 dims are
    # whatever the tensor's maker left there, and do not matter)
    bstride = {}
    for nm, t, n in (("x", x, c), ("out", out, ob)):
        if t.stride(2) != 1 or (rows > 1 and t.stride(1) != n) or (B > 1 and t.stride(0) % n):
            raise CSAError("prepare_kv: rows must be contiguous with a whole-row batch stride")
        bstride[nm] = t.stride(0) // n if B > 1 else rows
    for t in (x, out):
        if not t.is_cuda:
            raise CSAError("tensor must live on the GPU")
    if mixed and ((rows > 1 and out_scale.stride(1) != 1) or (B > 1 and out_scale.stride(0) != bstride["out"])):
        raise CSAError("prepare_kv: out_scale must follow out's row layout")
    st = lib.csa_prepare_kv(x.data_ptr(), bstride["x"], out.data_ptr(), _ptr(out_scale), bstride["out"], B,
                            rows, c, FMT[in_fmt], FMT[out_fmt], _ptr(pos_base), pos_first, pos_stride,
                            _prep_arg(prep), _stream(stream))
    _lib.check(st, "csa_prepare_kv")
    return (out, out_scale) if mixed else out


def _comp_t(comp_kv, comp_scale, kv_fmt):
    if comp_kv.dtype == torch.uint8:   # rows in CSA_FP8_BF16_ROPE with their scales
        if comp_scale is None:
            raise CSAError("comp_kv in the fp8 + bf16 RoPE format needs comp_scale")
        return FMT["fp8rope"]
    return FMT[kv_fmt]


def attend(q, comp_kv, idx, win_kv, sink, pos0, m, n_win, rope_dims, scale, eps=1e-6, rope_base=10000.0,
           gamma_q=None, gamma_kv=None, out=None, out_fmt=None, ws=None, stream=None, kv_prepared=False,
           comp_scale=None):
    """csa_attend.  q [B][T][H][c], comp_kv [B][N][c] (or uint8 [B][N][c + R] in the fp8 + bf16 RoPE format,
    with comp_scale [B][N]), idx int32 [B][T][k], win_kv [B][T+n_win-1][c]."""
    lib = _lib.load()
    B, T, H, c = q.shape
    k = idx.shape[2]
    N = comp_kv.shape[1]
    kv_fmt = _TORCH_FMT[q.dtype]
    out_fmt = out_fmt or kv_fmt
    if out is None:
        out = torch.empty((B, T, H, c), dtype=torch.float32 if out_fmt == "f32" else torch.bfloat16, device=q.device)
    nb = lib.csa_attend_workspace_bytes(B, T, H, c, k, n_win)
    if ws is None:
        ws = workspace(nb, q.device, "attend")
    st = lib.csa_attend(_ptr(q), _ptr(comp_kv), _ptr(comp_scale), _ptr(idx), _ptr(win_kv), _ptr(sink), _ptr(gamma_q),
                        _ptr(gamma_kv), B, T, H, c, rope_dims, k, n_win, N, _ptr(pos0), m, scale, eps, rope_base,
                        FMT[kv_fmt], _comp_t(comp_kv, comp_scale, kv_fmt), int(kv_prepared), _ptr(out), FMT[out_fmt],
                        _ptr(ws), _ws_bytes(ws), _stream(stream))
    _lib.check(st, "csa_attend")
    return out


def hca_attend(q, comp_kv, win_kv, sink, pos0, m_hca, n_win, rope_dims, scale, eps=1e-6, rope_base=10000.0,
               gamma_q=None, gamma_kv=None, out=None, out_fmt=None, ws=None, stream=None, kv_prepared=False,
               comp_scale=None):
    """hca_attend: dense over every visible compressed entry s < floor(t/m_hca), plus the window."""
    lib = _lib.load()
    B, T, H, c = q.shape
    N = comp_kv.shape[1]
    kv_fmt = _TORCH_FMT[q.dtype]
    out_fmt = out_fmt or kv_fmt
    if out is None:
        out = torch.empty((B, T, H, c), dtype=torch.float32 if out_fmt == "f32" else torch.bfloat16, device=q.device)
    nb = lib.hca_attend_workspace_bytes(B, T, H, c, N, n_win)
    if ws is None:
        ws = workspace(nb, q.device, "hca")
    st = lib.hca_attend(_ptr(q), _ptr(comp_kv), _ptr(comp_scale), _ptr(win_kv), _ptr(sink), _ptr(gamma_q),
                        _ptr(gamma_kv), B, T, H, c, rope_dims, n_win, N, _ptr(pos0), m_hca, scale, eps, rope_base,
                        FMT[kv_fmt], _comp_t(comp_kv, comp_scale, kv_fmt), int(kv_prepared), _ptr(out),
                        FMT[out_fmt], _ptr(ws), _ws_bytes(ws), _stream(stream))
    _lib.check(st, "hca_attend")
    return out


# ---- decode across steps: state rings and paged compressed caches -------------------------------------------


def pages(block_table, page_tokens):
    """csa_pages for a device int32 block table [B][max_pages] (kept alive by the returned struct's owner)."""
    if block_table.dtype != torch.int32 or block_table.dim() != 2 or not block_table.is_contiguous():
        raise CSAError("pages: block_table must be a contiguous int32 [B][max_pages] tensor")
    pg = _lib.Pages(_ptr(block_table), block_table.shape[1], page_tokens)
    pg._table = block_table
    return pg


def decode_append(jobs, wins, pos, pg, stream=None):
    """csa_decode_append.  jobs: dicts with ca, cb, za, zb ([B][c] token rows; cb = zb = None for HCA), bias_a,
    bias_b, m, ring_ca, ring_cb, ring_za, ring_zb ([B][ring][c]), out, out_scale, out_fmt, prep.  wins: dicts with
    row [B][c], ring [B][n_win][c], prep (optional).  pos: device int64 [B], the token's position."""
    lib = _lib.load()
    B = pos.shape[0]
    in_fmt = _TORCH_FMT[jobs[0]["ca"].dtype]
    keep = []
    jarr = (_lib.AppendJob * max(1, len(jobs)))()
    for i, j in enumerate(jobs):
        prep = j.get("prep")
        keep.append(prep)
        jarr[i] = _lib.AppendJob(_ptr(j["ca"]), _ptr(j.get("cb")), _ptr(j["za"]), _ptr(j.get("zb")), _ptr(j["bias_a"]),
                                 _ptr(j.get("bias_b")), j["ca"].shape[1], j["m"], _ptr(j["ring_ca"]),
                                 _ptr(j.get("ring_cb")), _ptr(j["ring_za"]), _ptr(j.get("ring_zb")), _dptr(j["out"]),
                                 _dptr(j.get("out_scale")), FMT[j.get("out_fmt") or in_fmt],
                                 None if prep is None else C.pointer(prep))
    warr = (_lib.WindowJob * max(1, len(wins)))()
    for i, w in enumerate(wins):
        prep = w.get("prep")
        keep.append(prep)
        warr[i] = _lib.WindowJob(_ptr(w["row"]), _ptr(w["ring"]), w["ring"].shape[2], w["ring"].shape[1],
                                 None if prep is None else C.pointer(prep))
    st = lib.csa_decode_append(jarr, len(jobs), warr, len(wins), B, _ptr(pos), C.byref(pg), FMT[in_fmt],
                               _stream(stream))
    _lib.check(st, "csa_decode_append")


def _append_structs(jobs, wins, in_fmt):
    keep = []
    jarr = (_lib.AppendJob * max(1, len(jobs)))()
    for i, j in enumerate(jobs):
        prep = j.get("prep")
        keep.append(prep)
        jarr[i] = _lib.AppendJob(_ptr(j["ca"]), _ptr(j.get("cb")), _ptr(j["za"]), _ptr(j.get("zb")), _ptr(j["bias_a"]),
                                 _ptr(j.get("bias_b")), j["ca"].shape[1], j["m"], _ptr(j["ring_ca"]),
                                 _ptr(j.get("ring_cb")), _ptr(j["ring_za"]), _ptr(j.get("ring_zb")), _dptr(j["out"]),
                                 _dptr(j.get("out_scale")), FMT[j.get("out_fmt") or in_fmt],
                                 None if prep is None else C.pointer(prep))
    warr = (_lib.WindowJob * max(1, len(wins)))()
    for i, w in enumerate(wins):
        prep = w.get("prep")
        keep.append(prep)
        warr[i] = _lib.WindowJob(_ptr(w["row"]), _ptr(w["ring"]), w["ring"].shape[2], w["ring"].shape[1],
                                 None if prep is None else C.pointer(prep))
    return jarr, warr, keep


def append_index_paged(jobs, win, q, q_scale, w, k_pool, k_scale_pool, pg, pos0, m, fmt, n_max, scores=None,
                       bound=None, score_fmt="f32", stream=None):
    """csa_append_index_paged: decode_append(jobs = [KV job, indexer-key job into k_pool], [win]) and index_paged
    in one launch.  Returns the scores."""
    lib = _lib.load()
    B, HI = q.shape[0], q.shape[2]
    cI = q.shape[3] * (2 if fmt == "mxfp4" else 1)
    in_fmt = _TORCH_FMT[jobs[0]["ca"].dtype]
    jarr, warr, keep = _append_structs(jobs, [win] if win is not None else [], in_fmt)
    if scores is None:
        scores = _score_buf(B, 1, n_max, score_fmt, q.device)
    st = lib.csa_append_index_paged(jarr, warr if win is not None else None, FMT[in_fmt], _ptr(q), _ptr(q_scale),
                                    _ptr(w), _ptr(k_pool), _ptr(k_scale_pool), C.byref(pg), B, HI, cI, n_max,
                                    _ptr(pos0), m, FMT[fmt], _ptr(scores), FMT[_TORCH_FMT[scores.dtype]], _ptr(bound),
                                    _stream(stream))
    _lib.check(st, "csa_append_index_paged")
    return scores


def index_paged(q, q_scale, w, k_pool, k_scale_pool, pg, pos0, m, fmt, n_max, scores=None, bound=None,
                score_fmt="f32", stream=None):
    """csa_index_paged: decode rows (q [B][1][HI][row]) over the paged key pool; scores [B][1][n_max]."""
    lib = _lib.load()
    B, T, HI = q.shape[0], q.shape[1], q.shape[2]
    if T != 1:
        raise CSAError("index_paged: decode rows only (T = 1)")
    cI = q.shape[3] * (2 if fmt == "mxfp4" else 1)
    if scores is None:
        scores = _score_buf(B, 1, n_max, score_fmt, q.device)
    st = lib.csa_index_paged(_ptr(q), _ptr(q_scale), _ptr(w), _ptr(k_pool), _ptr(k_scale_pool), C.byref(pg), B, HI, cI,
                             n_max, _ptr(pos0), m, FMT[fmt], _ptr(scores), FMT[_TORCH_FMT[scores.dtype]], _ptr(bound),
                             _stream(stream))
    _lib.check(st, "csa_index_paged")
    return scores


def attend_paged(q, comp_pool, idx, win_ring, sink, pos0, pg, m, rope_dims, scale, n_max, eps=1e-6,
                 rope_base=10000.0, gamma_q=None, gamma_kv=None, out=None, ws=None, stream=None, kv_prepared=1,
                 comp_scale=None):
    """csa_attend_paged: q [B][1][H][c], comp_pool rows (bf16 [rows][c] or uint8 [rows][c + R] with comp_scale),
    idx int32 [B][1][k], win_ring [B][n_win][c] (position p at row p % n_win)."""
    lib = _lib.load()
    B, T, H, c = q.shape
    if T != 1:
        raise CSAError("attend_paged: decode rows only (T = 1)")
    k = idx.shape[2]
    n_win = win_ring.shape[1]
    if out is None:
        out = torch.empty((B, 1, H, c), dtype=torch.bfloat16, device=q.device)
    nb = lib.csa_attend_workspace_bytes(B, 1, H, c, k, n_win)
    if ws is None:
        ws = workspace(nb, q.device, "attend")
    st = lib.csa_attend_paged(_ptr(q), _ptr(comp_pool), _ptr(comp_scale), C.byref(pg), _ptr(idx), _ptr(win_ring),
                              _ptr(sink), _ptr(gamma_q), _ptr(gamma_kv), B, H, c, rope_dims, k, n_win, n_max,
                              _ptr(pos0), m, scale, eps, rope_base, FMT["bf16"],
                              _comp_t(comp_pool, comp_scale, "bf16"), int(kv_prepared), _ptr(out),
                              FMT[_TORCH_FMT[out.dtype]], _ptr(ws), _ws_bytes(ws), _stream(stream))
    _lib.check(st, "csa_attend_paged")
    return out


def hca_attend_paged(q, comp_pool, win_ring, sink, pos0, pg, m_hca, rope_dims, scale, n_max, eps=1e-6,
                     rope_base=10000.0, gamma_q=None, gamma_kv=None, out=None, ws=None, stream=None, kv_prepared=1,
                     comp_scale=None):
    """hca_attend_paged: dense over the visible entries of the paged HCA pool, window from the ring."""
    lib = _lib.load()
    B, T, H, c = q.shape
    if T != 1:
        raise CSAError("hca_attend_paged: decode rows only (T = 1)")
    n_win = win_ring.shape[1]
    if out is None:
        out = torch.empty((B, 1, H, c), dtype=torch.bfloat16, device=q.device)
    nb = lib.hca_attend_workspace_bytes(B, 1, H, c, n_max, n_win)
    if ws is None:
        ws = workspace(nb, q.device, "hca")
    st = lib.hca_attend_paged(_ptr(q), _ptr(comp_pool), _ptr(comp_scale), C.byref(pg), _ptr(win_ring), _ptr(sink),
                              _ptr(gamma_q), _ptr(gamma_kv), B, H, c, rope_dims, n_win, n_max, _ptr(pos0), m_hca, scale,
                              eps, rope_base, FMT["bf16"], _comp_t(comp_pool, comp_scale, "bf16"), int(kv_prepared),
                              _ptr(out), FMT[_TORCH_FMT[out.dtype]], _ptr(ws), _ws_bytes(ws), _stream(stream))
    _lib.check(st, "hca_attend_paged")
    return out


# ---- dense projections for decode rows ------------------------------------------------------------------------


def pack_proj_weights(w, stream=None):
    """csa_pack_proj_weights: bf16 [n][k] or [z][n][k] output-major weights -> the packed layout (same shape)."""
    lib = _lib.load()
    z, n, k = (1,) + tuple(w.shape) if w.dim() == 2 else tuple(w.shape)
    packed = torch.empty_like(w)
    st = lib.csa_pack_proj_weights(_ptr(w), _ptr(packed), z, n, k, _stream(stream))
    _lib.check(st, "csa_pack_proj_weights")
    return packed


def q_up_proj(cq, w_uq, w_iuq, n_h, c, n_hI, cI, qi_fmt="bf16", q=None, qi=None, qi_scale=None, stream=None):
    """csa_q_up_proj: cq bf16 [rows][d_c], packed weights (pack_proj_weights of [outputs][d_c]).  Returns (q [rows][n_h][c] bf16, q^I in
    qi_fmt [rows][n_hI][...], its scales or None)."""
    lib = _lib.load()
    rows, d_c = cq.shape
    dev = cq.device
    if q is None:
        q = torch.empty((rows, n_h, c), dtype=torch.bfloat16, device=dev)
    if qi is None:
        if qi_fmt == "bf16":
            qi = torch.empty((rows, n_hI, cI), dtype=torch.bfloat16, device=dev)
        elif qi_fmt == "fp8":
            qi = torch.empty((rows, n_hI, cI), dtype=torch.uint8, device=dev)
            qi_scale = torch.empty((rows, n_hI), dtype=torch.float32, device=dev) if qi_scale is None else qi_scale
        else:
            qi = torch.empty((rows, n_hI, cI // 2), dtype=torch.uint8, device=dev)
            qi_scale = torch.empty((rows, n_hI, cI // 32), dtype=torch.uint8, device=dev) if qi_scale is None \
                else qi_scale
    st = lib.csa_q_up_proj(_ptr(cq), _ptr(w_uq), _ptr(w_iuq), rows, d_c, n_h, c, n_hI, cI, _ptr(q), _ptr(qi),
                           _ptr(qi_scale), FMT[qi_fmt], _stream(stream))
    _lib.check(st, "csa_q_up_proj")
    return q, qi, qi_scale


def grouped_out_proj(o, w_g, w_o, g, mid=None, out=None, stream=None):
    """csa_grouped_out_proj: o bf16 [rows][n_h * c] (or [rows][n_h][c]), packed w_g [g][d_g][n_h c / g] and
    w_o [d][g d_g] (pack_proj_weights).
    Returns (out [rows][d], mid [rows][g d_g])."""
    lib = _lib.load()
    rows = o.shape[0]
    n_h, c = (o.shape[1], o.shape[2]) if o.dim() == 3 else (g, o.shape[1] // g)
    d_g, d = w_g.shape[1], w_o.shape[0]
    if mid is None:
        mid = torch.empty((rows, g * d_g), dtype=torch.bfloat16, device=o.device)
    if out is None:
        out = torch.empty((rows, d), dtype=torch.bfloat16, device=o.device)
    st = lib.csa_grouped_out_proj(_ptr(o), _ptr(w_g), _ptr(w_o), rows, n_h, c, g, d_g, d, _ptr(mid), _ptr(out),
                                  _stream(stream))
    _lib.check(st, "csa_grouped_out_proj")
    return out, mid
