// C ABI of the CSA / HCA step: O(1) host-side validation, then launches on the
// caller's stream.  No HIP runtime call is made before validation passes, so
// argument errors are reported without touching a device.
#include <atomic>
#include <mutex>

#include "csa_common.h"
#include "csa_internal.h"

namespace {
bool is_pow2_dim(int c) { return c == 128 || c == 256 || c == 512; }
}  // namespace

extern "C" {

const char* csa_status_string(int status) {
  switch (status) {
    case CSA_OK: return "CSA_OK";
    case CSA_ERR_NULL: return "CSA_ERR_NULL: a required pointer is NULL";
    case CSA_ERR_SHAPE: return "CSA_ERR_SHAPE: sizes are inconsistent or out of range";
    case CSA_ERR_UNSUPPORTED: return "CSA_ERR_UNSUPPORTED: this dtype / size combination is not implemented";
    case CSA_ERR_WORKSPACE: return "CSA_ERR_WORKSPACE: workspace missing or too small";
    case CSA_ERR_LAUNCH: return "CSA_ERR_LAUNCH: kernel launch failed";
    default: return "unknown csa_status";
  }
}

int csa_abi_version(void) { return 7; }

}  // extern "C"

namespace {
// checks of one compression problem; CSA_OK with `empty` set means nothing to launch
csa_status check_compress(const void* ca, const void* cb, const void* za, const void* zb, const float* bias_a,
                          const float* bias_b, int B, int rows, int c, int m, int64_t row0_pos, int64_t first_entry,
                          int num_entries, int in_t, void* out, void* out_scale, int out_t,
                          int64_t& out_batch_stride, const csa_kv_prep* prep, bool& empty) {
  empty = false;
  if (prep && (out_t != CSA_F32 && out_t != CSA_BF16 && out_t != CSA_FP8_BF16_ROPE)) return CSA_ERR_UNSUPPORTED;
  if (out_t == CSA_FP8_BF16_ROPE && (!prep || (c - prep->rope_dims) % 16 != 0)) return CSA_ERR_UNSUPPORTED;
  if (prep && (prep->rope_dims < 0 || (prep->rope_dims % 8) || prep->rope_dims > c || prep->rope_dims > 128))
    return CSA_ERR_UNSUPPORTED;
  if (prep && !(prep->eps >= 0.0f)) return CSA_ERR_SHAPE;
  if (B < 0 || rows < 0 || num_entries < 0 || m < 1 || m > 1024 || c < 4 || c > 1024 || (c & 3)) return CSA_ERR_SHAPE;
  if (in_t != CSA_F32 && in_t != CSA_BF16) return CSA_ERR_UNSUPPORTED;
  if (out_t < CSA_F32 || out_t > CSA_FP8_BF16_ROPE) return CSA_ERR_UNSUPPORTED;
  if (out_t == CSA_MXFP4_E8M0_B32 && (c % 32)) return CSA_ERR_UNSUPPORTED;
  if (B == 0 || num_entries == 0) {
    empty = true;
    return CSA_OK;
  }
  const bool overlap = cb != nullptr || zb != nullptr || bias_b != nullptr;
  if (!ca || !za || !bias_a || !out) return CSA_ERR_NULL;
  if (overlap && (!cb || !zb || !bias_b)) return CSA_ERR_NULL;
  if ((out_t == CSA_FP8_E4M3_ROWSCALE || out_t == CSA_MXFP4_E8M0_B32 || out_t == CSA_FP8_BF16_ROPE) && !out_scale)
    return CSA_ERR_NULL;
  if (first_entry < 0) return CSA_ERR_SHAPE;
  if (out_batch_stride == 0) out_batch_stride = num_entries;
  if (out_batch_stride < num_entries) return CSA_ERR_SHAPE;
  // every row the entries read must be inside [row0_pos, row0_pos + rows)
  const int64_t last = first_entry + num_entries - 1;
  const int64_t lo_entry = (overlap && first_entry > 0) ? first_entry - 1 : first_entry;
  if ((int64_t)m * lo_entry < row0_pos) return CSA_ERR_SHAPE;
  if ((int64_t)m * (last + 1) - 1 >= row0_pos + rows) return CSA_ERR_SHAPE;
  return CSA_OK;
}
}  // namespace

extern "C" {

csa_status csa_compress(const void* ca, const void* cb, const void* za, const void* zb, const float* bias_a,
                        const float* bias_b, int B, int rows, int c, int m, int64_t row0_pos, int64_t first_entry,
                        int num_entries, int in_t, void* out, void* out_scale, int out_t, int64_t out_batch_stride,
                        const csa_kv_prep* prep, void* stream) {
  bool empty;
  const csa_status st = check_compress(ca, cb, za, zb, bias_a, bias_b, B, rows, c, m, row0_pos, first_entry,
                                       num_entries, in_t, out, out_scale, out_t, out_batch_stride, prep, empty);
  if (st != CSA_OK || empty) return st;
  return launch_compress(ca, cb, za, zb, bias_a, bias_b, B, rows, c, m, row0_pos, first_entry, num_entries, in_t, out,
                         out_scale, out_t, out_batch_stride, prep, (hipStream_t)stream);
}

csa_status csa_compress_pair(const void* ca0, const void* cb0, const void* za0, const void* zb0,
                             const float* bias_a0, const float* bias_b0, int c0, void* out0, void* out_scale0,
                             int out_t0, int64_t out_batch_stride0, const csa_kv_prep* prep0, const void* ca1,
                             const void* cb1, const void* za1, const void* zb1, const float* bias_a1,
                             const float* bias_b1, int c1, void* out1, void* out_scale1, int out_t1,
                             int64_t out_batch_stride1, const csa_kv_prep* prep1, int B, int rows, int m,
                             int64_t row0_pos, int64_t first_entry, int num_entries, int in_t, void* stream) {
  bool e0, e1;
  csa_status st = check_compress(ca0, cb0, za0, zb0, bias_a0, bias_b0, B, rows, c0, m, row0_pos, first_entry,
                                 num_entries, in_t, out0, out_scale0, out_t0, out_batch_stride0, prep0, e0);
  if (st != CSA_OK) return st;
  st = check_compress(ca1, cb1, za1, zb1, bias_a1, bias_b1, B, rows, c1, m, row0_pos, first_entry, num_entries, in_t,
                      out1, out_scale1, out_t1, out_batch_stride1, prep1, e1);
  if (st != CSA_OK || e0) return st;  // both problems share B and num_entries, so both are empty or neither
  const CompressJob jobs[2] = {
      {ca0, cb0, za0, zb0, bias_a0, bias_b0, c0, out0, out_scale0, out_t0, out_batch_stride0, prep0},
      {ca1, cb1, za1, zb1, bias_a1, bias_b1, c1, out1, out_scale1, out_t1, out_batch_stride1, prep1}};
  return launch_compress_jobs(jobs, 2, B, rows, m, row0_pos, first_entry, num_entries, in_t, (hipStream_t)stream);
}

csa_status csa_prepare_kv(const void* in, int64_t in_batch_stride, void* out, void* out_scale,
                          int64_t out_batch_stride, int B, int rows, int c, int in_t, int out_t,
                          const int64_t* pos_base, int64_t pos_first, int64_t pos_stride, const csa_kv_prep* prep,
                          void* stream) {
  if (B < 0 || rows < 0 || c < 4 || c > 1024 || (c & 3)) return CSA_ERR_SHAPE;
  if ((in_t != CSA_F32 && in_t != CSA_BF16) || (out_t != CSA_F32 && out_t != CSA_BF16 && out_t != CSA_FP8_BF16_ROPE))
    return CSA_ERR_UNSUPPORTED;
  if (!prep) return CSA_ERR_NULL;
  if (prep->rope_dims < 0 || (prep->rope_dims % 8) || prep->rope_dims > c || prep->rope_dims > 128)
    return CSA_ERR_UNSUPPORTED;
  if (out_t == CSA_FP8_BF16_ROPE && (c - prep->rope_dims) % 16 != 0) return CSA_ERR_UNSUPPORTED;
  if (!(prep->eps >= 0.0f)) return CSA_ERR_SHAPE;
  if (B == 0 || rows == 0) return CSA_OK;
  if (!in || !out || (out_t == CSA_FP8_BF16_ROPE && !out_scale)) return CSA_ERR_NULL;
  if (in_batch_stride < rows || out_batch_stride < rows) return CSA_ERR_SHAPE;
  if (rows >= 2147483647 || B >= 65536) return CSA_ERR_UNSUPPORTED;
  // in place only with the same element type and the same layout
  if (in == out && (in_t != out_t || in_batch_stride != out_batch_stride)) return CSA_ERR_SHAPE;
  return launch_prepare_kv(in, in_batch_stride, out, out_scale, out_batch_stride, B, rows, c, in_t, out_t, pos_base,
                           pos_first, pos_stride, prep, (hipStream_t)stream);
}

}  // extern "C"

namespace {
// shape / dtype / pointer checks of csa_index; CSA_OK with `empty` set means nothing to launch
csa_status check_index(const void* q, const void* q_scale, const float* w, const void* k, const void* k_scale, int B,
                       int T, int HI, int cI, int64_t n_max, const int64_t* pos0, int m, int qk_t, const void* scores,
                       bool& empty) {
  empty = false;
  if (B < 0 || T < 0 || HI < 1 || cI < 1 || n_max < 0 || m < 1) return CSA_ERR_SHAPE;
  if (n_max >= ((int64_t)1 << 31)) return CSA_ERR_SHAPE;
  if ((int64_t)B * T >= 65536) return CSA_ERR_UNSUPPORTED;  // grid.y limit
  switch (qk_t) {
    case CSA_F32:
      if ((cI & 3) || cI > 512 || HI > 128 || HI * cI > 16384) return CSA_ERR_UNSUPPORTED;
      break;
    case CSA_BF16:
    case CSA_FP8_E4M3_ROWSCALE:
    case CSA_MXFP4_E8M0_B32:
      if (cI != 128 || !(HI == 16 || HI == 32 || HI == 64 || HI == 128)) return CSA_ERR_UNSUPPORTED;
      break;
    default:
      return CSA_ERR_UNSUPPORTED;
  }
  if (B == 0 || T == 0 || n_max == 0) {
    empty = true;
    return CSA_OK;
  }
  if (!q || !w || !k || !pos0 || !scores) return CSA_ERR_NULL;
  if ((qk_t == CSA_FP8_E4M3_ROWSCALE || qk_t == CSA_MXFP4_E8M0_B32) && (!q_scale || !k_scale)) return CSA_ERR_NULL;
  // the MXFP4 query scales are read as one 32-bit word per head
  if (qk_t == CSA_MXFP4_E8M0_B32 && (reinterpret_cast<uintptr_t>(q_scale) & 3)) return CSA_ERR_SHAPE;
  return CSA_OK;
}
}  // namespace

extern "C" {

int64_t csa_index_bound_keys(int64_t n_max) { return n_max > 0 ? index_bound_keys(n_max) : 0; }

csa_status csa_index(const void* q, const void* q_scale, const float* w, const void* k, const void* k_scale, int B,
                     int T, int HI, int cI, int64_t n_max, const int64_t* pos0, int m, int qk_t, void* scores,
                     int score_t, uint32_t* bound, void* stream) {
  bool empty;
  const csa_status st = check_index(q, q_scale, w, k, k_scale, B, T, HI, cI, n_max, pos0, m, qk_t, scores, empty);
  if (st != CSA_OK) return st;
  if (score_t != CSA_F32 && score_t != CSA_BF16) return CSA_ERR_UNSUPPORTED;
  // bound keys come from the MFMA kernels (per-row decode and tiled prefill)
  if (bound && qk_t == CSA_F32) return CSA_ERR_UNSUPPORTED;
  if (empty) return CSA_OK;
  if (bound && (reinterpret_cast<uintptr_t>(bound) & 7)) return CSA_ERR_SHAPE;
  return launch_index(q, q_scale, w, k, k_scale, B, T, HI, cI, n_max, pos0, m, qk_t, scores, score_t, bound,
                      (hipStream_t)stream);
}

csa_status csa_compress_index(const void* ca0, const void* cb0, const void* za0, const void* zb0,
                              const float* bias_a0, const float* bias_b0, int c0, void* out0, void* out_scale0,
                              int out_t0, int64_t out_batch_stride0, const csa_kv_prep* prep0, const void* ca1,
                              const void* cb1,
                              const void* za1, const void* zb1, const float* bias_a1, const float* bias_b1, int B,
                              int rows, int m, int64_t row0_pos, int64_t first_entry, int in_t, const void* q,
                              const void* q_scale, const float* w, void* k, void* k_scale, int HI, int cI,
                              int64_t n_max, const int64_t* pos0, int qk_t, void* scores, int score_t,
                              uint32_t* bound, void* stream) {
  if (score_t != CSA_F32 && score_t != CSA_BF16) return CSA_ERR_UNSUPPORTED;
  if (qk_t != CSA_BF16 && qk_t != CSA_FP8_E4M3_ROWSCALE && qk_t != CSA_MXFP4_E8M0_B32) return CSA_ERR_UNSUPPORTED;
  if (m >= 64) return CSA_ERR_UNSUPPORTED;  // one 256-thread workgroup pools an entry's rows
  if (n_max < 1 || first_entry < 0 || first_entry >= n_max) return CSA_ERR_SHAPE;
  bool empty;
  csa_status st = check_index(q, q_scale, w, k, k_scale, B, 1, HI, cI, n_max, pos0, m, qk_t, scores, empty);
  if (st != CSA_OK) return st;
  if (bound && (reinterpret_cast<uintptr_t>(bound) & 7)) return CSA_ERR_SHAPE;
  // the indexer key is written into the key cache at first_entry (row stride n_max per sequence)
  const int64_t krow = qk_t == CSA_BF16 ? 2 * (int64_t)cI : (qk_t == CSA_FP8_E4M3_ROWSCALE ? cI : cI / 2);
  const int64_t srow = qk_t == CSA_FP8_E4M3_ROWSCALE ? 4 : (qk_t == CSA_MXFP4_E8M0_B32 ? cI / 32 : 0);
  void* out1 = k ? static_cast<uint8_t*>(k) + first_entry * krow : nullptr;
  void* out_scale1 = k_scale ? static_cast<uint8_t*>(k_scale) + first_entry * srow : nullptr;
  int64_t bs0 = out_batch_stride0, bs1 = n_max;
  bool e0 = false, e1;
  if (out0) {  // (out0 NULL: no KV job, the indexer key alone)
    st = check_compress(ca0, cb0, za0, zb0, bias_a0, bias_b0, B, rows, c0, m, row0_pos, first_entry, 1, in_t, out0,
                        out_scale0, out_t0, bs0, prep0, e0);
    if (st != CSA_OK) return st;
    if (out_t0 != CSA_F32 && out_t0 != CSA_BF16 && out_t0 != CSA_FP8_BF16_ROPE) return CSA_ERR_UNSUPPORTED;
  }
  st = check_compress(ca1, cb1, za1, zb1, bias_a1, bias_b1, B, rows, cI, m, row0_pos, first_entry, 1, in_t, out1,
                      out_scale1, qk_t, bs1, nullptr, e1);
  if (st != CSA_OK || e0 || empty) return st;
  const CompressJob jobs[2] = {{ca0, cb0, za0, zb0, bias_a0, bias_b0, c0, out0, out_scale0, out_t0, bs0, prep0},
                               {ca1, cb1, za1, zb1, bias_a1, bias_b1, cI, out1, out_scale1, qk_t, bs1, nullptr}};
  return launch_compress_index(jobs, rows, m, row0_pos, first_entry, in_t, q, q_scale, w, k, k_scale, B, HI, cI,
                               n_max, pos0, qk_t, scores, score_t, bound, (hipStream_t)stream);
}

size_t csa_topk_workspace_bytes(int B, int T, int64_t n_max, int k) {
  if (B <= 0 || T <= 0 || n_max <= 0 || k <= 0) return 0;
  return topk_workspace_bytes(B, T, n_max, k);
}

csa_status csa_topk(const void* scores, int score_t, int B, int T, int64_t n_max, const int64_t* pos0, int m,
                    int k, const uint32_t* bound, int32_t* idx, float* vals, void* workspace, size_t ws_bytes,
                    void* stream) {
  if (score_t != CSA_F32 && score_t != CSA_BF16) return CSA_ERR_UNSUPPORTED;
  if (B < 0 || T < 0 || n_max < 0 || m < 1 || k < 1 || k > 2048) return CSA_ERR_SHAPE;
  if (n_max >= ((int64_t)1 << 31)) return CSA_ERR_SHAPE;
  if (B == 0 || T == 0) return CSA_OK;
  if (!idx || !pos0 || (n_max > 0 && !scores)) return CSA_ERR_NULL;
  const size_t need = csa_topk_workspace_bytes(B, T, n_max > 0 ? n_max : 1, k);
  if (need > 0 && (!workspace || ws_bytes < need)) return CSA_ERR_WORKSPACE;
  return launch_topk(scores, score_t, B, T, n_max, pos0, m, k, bound, idx, vals, workspace, (hipStream_t)stream);
}

// the compressed cache's format: the KV type, or fp8 + bf16 RoPE dims (bf16 MFMA path, prepared entries)
static csa_status check_comp_t(int kv_t, int comp_t, int kv_prepared, int c, int rope_dims) {
  if (comp_t == kv_t) return CSA_OK;
  if (comp_t != CSA_FP8_BF16_ROPE || kv_t != CSA_BF16 || kv_prepared < 1) return CSA_ERR_UNSUPPORTED;
  if ((c - rope_dims) % 16 != 0) return CSA_ERR_UNSUPPORTED;
  return CSA_OK;
}

static csa_status check_attend(int kv_t, int out_t, int B, int T, int H, int c, int rope_dims, int n_win, int m) {
  if (B < 0 || T < 0 || H < 1 || m < 1 || n_win < 1 || n_win > 4096) return CSA_ERR_SHAPE;
  if (!is_pow2_dim(c)) return CSA_ERR_UNSUPPORTED;
  if (rope_dims < 0 || (rope_dims % 8) || rope_dims > c || rope_dims > 128) return CSA_ERR_UNSUPPORTED;
  if (kv_t != CSA_F32 && kv_t != CSA_BF16) return CSA_ERR_UNSUPPORTED;
  if (out_t != CSA_F32 && out_t != CSA_BF16) return CSA_ERR_UNSUPPORTED;
  if (kv_t == CSA_BF16 && (H % 16)) return CSA_ERR_UNSUPPORTED;
  if ((int64_t)B * T >= 65536) return CSA_ERR_UNSUPPORTED;
  return CSA_OK;
}

size_t csa_attend_workspace_bytes(int B, int T, int H, int c, int k, int n_win) {
  if (B <= 0 || T <= 0 || H <= 0 || c <= 0 || k <= 0 || n_win <= 0) return 0;
  return attend_workspace_bytes(0, B, T, H, c, (int64_t)k, n_win);
}

// csa_attend's checks, shared by csa_attend_noalloc; sets *need to the workspace bytes the call uses
static csa_status check_csa_attend(const void* q, const void* comp_kv, const float* comp_scale, const int32_t* idx,
                                   const void* win_kv, const float* sink, int B, int T, int H, int c, int rope_dims,
                                   int k, int n_win, int64_t n_max, const int64_t* pos0, int m, int kv_t, int comp_t,
                                   int kv_prepared, const void* out, int out_t, size_t* need) {
  *need = 0;
  csa_status st = check_attend(kv_t, out_t, B, T, H, c, rope_dims, n_win, m);
  if (st != CSA_OK) return st;
  st = check_comp_t(kv_t, comp_t, kv_prepared, c, rope_dims);
  if (st != CSA_OK) return st;
  if (k < 1 || k > 2048 || n_max < 0 || n_max >= ((int64_t)1 << 31)) return CSA_ERR_SHAPE;
  if (kv_prepared < 0 || kv_prepared > 2) return CSA_ERR_UNSUPPORTED;
  if (B == 0 || T == 0) return CSA_OK;
  if (!q || !idx || !win_kv || !sink || !pos0 || !out || (n_max > 0 && !comp_kv)) return CSA_ERR_NULL;
  if (comp_t != kv_t && n_max > 0 && !comp_scale) return CSA_ERR_NULL;
  *need = csa_attend_workspace_bytes(B, T, H, c, k, n_win);
  return CSA_OK;
}

csa_status csa_attend(const void* q, const void* comp_kv, const float* comp_scale, const int32_t* idx,
                      const void* win_kv, const float* sink, const float* gamma_q, const float* gamma_kv, int B, int T,
                      int H, int c, int rope_dims, int k, int n_win, int64_t n_max, const int64_t* pos0, int m,
                      float scale, float eps, float rope_base, int kv_t, int comp_t, int kv_prepared, void* out,
                      int out_t, void* workspace, size_t ws_bytes, void* stream) {
  size_t need = 0;
  const csa_status st = check_csa_attend(q, comp_kv, comp_scale, idx, win_kv, sink, B, T, H, c, rope_dims, k, n_win,
                                         n_max, pos0, m, kv_t, comp_t, kv_prepared, out, out_t, &need);
  if (st != CSA_OK || B == 0 || T == 0) return st;
  if (need > 0 && (!workspace || ws_bytes < need)) return CSA_ERR_WORKSPACE;
  return launch_attend(0, q, comp_kv, comp_scale, comp_t != kv_t, nullptr, idx, win_kv, sink, gamma_q, gamma_kv, B, T, H, c,
                       rope_dims, k, n_win, n_max, pos0, m, scale, eps, rope_base, kv_t, kv_prepared, out, out_t,
                       workspace, (hipStream_t)stream);
}

size_t hca_attend_workspace_bytes(int B, int T, int H, int c, int64_t n_max, int n_win) {
  if (B <= 0 || T <= 0 || H <= 0 || c <= 0 || n_max < 0 || n_win <= 0) return 0;
  return attend_workspace_bytes(1, B, T, H, c, n_max, n_win);
}

csa_status hca_attend(const void* q, const void* comp_kv, const float* comp_scale, const void* win_kv,
                      const float* sink, const float* gamma_q, const float* gamma_kv, int B, int T, int H, int c,
                      int rope_dims, int n_win, int64_t n_max, const int64_t* pos0, int m_hca, float scale, float eps,
                      float rope_base, int kv_t, int comp_t, int kv_prepared, void* out, int out_t, void* workspace,
                      size_t ws_bytes, void* stream) {
  csa_status st = check_attend(kv_t, out_t, B, T, H, c, rope_dims, n_win, m_hca);
  if (st != CSA_OK) return st;
  st = check_comp_t(kv_t, comp_t, kv_prepared, c, rope_dims);
  if (st != CSA_OK) return st;
  if (n_max < 0 || n_max >= ((int64_t)1 << 24)) return CSA_ERR_SHAPE;
  if (kv_prepared < 0 || kv_prepared > 2) return CSA_ERR_UNSUPPORTED;
  if (B == 0 || T == 0) return CSA_OK;
  if (!q || !win_kv || !sink || !pos0 || !out || (n_max > 0 && !comp_kv)) return CSA_ERR_NULL;
  if (comp_t != kv_t && n_max > 0 && !comp_scale) return CSA_ERR_NULL;
  const size_t need = hca_attend_workspace_bytes(B, T, H, c, n_max, n_win);
  if (need > 0 && (!workspace || ws_bytes < need)) return CSA_ERR_WORKSPACE;
  return launch_attend(1, q, comp_kv, comp_scale, comp_t != kv_t, nullptr, nullptr, win_kv, sink, gamma_q, gamma_kv, B, T, H,
                       c, rope_dims, 1, n_win, n_max, pos0, m_hca, scale, eps, rope_base, kv_t, kv_prepared, out, out_t,
                       workspace, (hipStream_t)stream);
}


}  // extern "C"

namespace {
// a page map usable for entries at ratio r: page_tokens a power of two, a multiple of 128 and of r
csa_status check_pages(const csa_pages* pages, int ratio) {
  if (!pages || !pages->block_table) return CSA_ERR_NULL;
  const int P = pages->page_tokens;
  if (P < 128 || (P & (P - 1)) || pages->max_pages < 1) return CSA_ERR_SHAPE;
  if (ratio < 1 || P % ratio) return CSA_ERR_SHAPE;
  return CSA_OK;
}
// logical entries of a sequence must fit its table row
csa_status check_pages_cover(const csa_pages* pages, int ratio, int64_t n_max) {
  const int64_t per_page = pages->page_tokens / ratio;
  return (n_max + per_page - 1) / per_page <= pages->max_pages ? CSA_OK : CSA_ERR_SHAPE;
}
csa_status check_prep(const csa_kv_prep* prep, int c) {
  if (!prep) return CSA_OK;
  if (prep->rope_dims < 0 || (prep->rope_dims % 8) || prep->rope_dims > c || prep->rope_dims > 128)
    return CSA_ERR_UNSUPPORTED;
  if (!(prep->eps >= 0.0f)) return CSA_ERR_SHAPE;
  return CSA_OK;
}
}  // namespace

extern "C" {

}  // extern "C"

namespace {
csa_status check_append(const csa_append_job* jobs, int njobs, const csa_window_job* wins, int nwins, int B,
                        const csa_pages* pages, int in_t) {
  if (njobs < 1 || njobs > 2 || nwins < 0 || nwins > 2 || B < 0) return CSA_ERR_SHAPE;
  if (in_t != CSA_F32 && in_t != CSA_BF16) return CSA_ERR_UNSUPPORTED;
  if (B >= 65536) return CSA_ERR_UNSUPPORTED;
  if (!jobs || (nwins > 0 && !wins)) return CSA_ERR_NULL;
  for (int i = 0; i < njobs; ++i) {
    const csa_append_job& j = jobs[i];
    if (j.m < 1 || j.m > 1024 || j.c < 4 || j.c > 1024 || (j.c & 3)) return CSA_ERR_SHAPE;
    if ((j.m >= 64) != (jobs[0].m >= 64)) return CSA_ERR_UNSUPPORTED;
    if (j.out_t < CSA_F32 || j.out_t > CSA_FP8_BF16_ROPE) return CSA_ERR_UNSUPPORTED;
    if (j.prep && j.out_t != CSA_F32 && j.out_t != CSA_BF16 && j.out_t != CSA_FP8_BF16_ROPE)
      return CSA_ERR_UNSUPPORTED;
    if (j.out_t == CSA_FP8_BF16_ROPE && (!j.prep || (j.c - j.prep->rope_dims) % 16 != 0)) return CSA_ERR_UNSUPPORTED;
    if (j.out_t == CSA_MXFP4_E8M0_B32 && (j.c % 32)) return CSA_ERR_UNSUPPORTED;
    csa_status st = check_prep(j.prep, j.c);
    if (st != CSA_OK) return st;
    st = check_pages(pages, j.m);
    if (st != CSA_OK) return st;
    const bool overlap = j.cb || j.zb || j.bias_b || j.ring_cb || j.ring_zb;
    if (!j.ca || !j.za || !j.bias_a || !j.ring_ca || !j.ring_za || !j.out) return CSA_ERR_NULL;
    if (overlap && (!j.cb || !j.zb || !j.bias_b || !j.ring_cb || !j.ring_zb)) return CSA_ERR_NULL;
    if ((j.out_t == CSA_FP8_E4M3_ROWSCALE || j.out_t == CSA_MXFP4_E8M0_B32 || j.out_t == CSA_FP8_BF16_ROPE) &&
        !j.out_scale)
      return CSA_ERR_NULL;
  }
  for (int i = 0; i < nwins; ++i) {
    const csa_window_job& w = wins[i];
    if (w.c < 4 || w.c > 1024 || (w.c & 3) || w.n_win < 1 || w.n_win > 4096) return CSA_ERR_SHAPE;
    const csa_status st = check_prep(w.prep, w.c);
    if (st != CSA_OK) return st;
    if (!w.row || !w.ring) return CSA_ERR_NULL;
  }
  return CSA_OK;
}
}  // namespace

extern "C" {

csa_status csa_decode_append(const csa_append_job* jobs, int njobs, const csa_window_job* wins, int nwins, int B,
                             const int64_t* pos, const csa_pages* pages, int in_t, void* stream) {
  const csa_status st = check_append(jobs, njobs, wins, nwins, B, pages, in_t);
  if (st != CSA_OK) return st;
  if (B == 0) return CSA_OK;
  if (!pos) return CSA_ERR_NULL;
  return launch_decode_append(jobs, njobs, wins, nwins, B, pos, pages, in_t, (hipStream_t)stream);
}

}  // extern "C"
namespace {
csa_status check_index_paged(const void* q, const void* q_scale, const float* w, const void* k_pool,
                             const void* k_scale_pool, const csa_pages* pages, int B, int HI, int cI, int64_t n_max,
                             const int64_t* pos0, int m, int qk_t, void* scores, int score_t, uint32_t* bound,
                             bool& empty);
}  // namespace
extern "C" {

csa_status csa_append_index_paged(const csa_append_job* jobs, const csa_window_job* win, int in_t, const void* q,
                                  const void* q_scale, const float* w, const void* k_pool, const void* k_scale_pool,
                                  const csa_pages* pages, int B, int HI, int cI, int64_t n_max, const int64_t* pos0,
                                  int m, int qk_t, void* scores, int score_t, uint32_t* bound, void* stream) {
  csa_status st = check_append(jobs, 2, win, win ? 1 : 0, B, pages, in_t);
  if (st != CSA_OK) return st;
  if (jobs[0].m != m || jobs[1].m != m || m >= 64) return CSA_ERR_UNSUPPORTED;
  // the indexer-key job writes the key pool this call scores
  if (jobs[1].out != k_pool || jobs[1].out_scale != k_scale_pool || jobs[1].out_t != qk_t || jobs[1].c != cI ||
      jobs[1].prep)
    return CSA_ERR_SHAPE;
  if (win && (win->c % 4 || win->c / 4 > 256)) return CSA_ERR_UNSUPPORTED;  // one 256-thread workgroup
  if (jobs[0].c / 4 > 256 || jobs[1].c / 4 > 256) return CSA_ERR_UNSUPPORTED;
  bool empty;
  st = check_index_paged(q, q_scale, w, k_pool, k_scale_pool, pages, B, HI, cI, n_max, pos0, m, qk_t, scores, score_t,
                         bound, empty);
  if (st != CSA_OK || empty) return st;
  return launch_append_index_paged(jobs, win, in_t, q, q_scale, w, k_pool, k_scale_pool, pages, B, HI, cI, n_max,
                                   pos0, m, qk_t, scores, score_t, bound, (hipStream_t)stream);
}

}  // extern "C"

namespace {
csa_status check_index_paged(const void* q, const void* q_scale, const float* w, const void* k_pool,
                             const void* k_scale_pool, const csa_pages* pages, int B, int HI, int cI, int64_t n_max,
                             const int64_t* pos0, int m, int qk_t, void* scores, int score_t, uint32_t* bound,
                             bool& empty) {
  empty = false;
  if (qk_t != CSA_BF16 && qk_t != CSA_FP8_E4M3_ROWSCALE && qk_t != CSA_MXFP4_E8M0_B32) return CSA_ERR_UNSUPPORTED;
  if (score_t != CSA_F32 && score_t != CSA_BF16) return CSA_ERR_UNSUPPORTED;
  csa_status st = check_index(q, q_scale, w, k_pool, k_scale_pool, B, 1, HI, cI, n_max, pos0, m, qk_t, scores,
                              empty);
  if (st != CSA_OK) return st;
  st = check_pages(pages, m);
  if (st != CSA_OK) return st;
  st = check_pages_cover(pages, m, n_max);
  if (st != CSA_OK) return st;
  if (!empty && bound && (reinterpret_cast<uintptr_t>(bound) & 7)) return CSA_ERR_SHAPE;
  return CSA_OK;
}
}  // namespace

extern "C" {

csa_status csa_index_paged(const void* q, const void* q_scale, const float* w, const void* k_pool,
                           const void* k_scale_pool, const csa_pages* pages, int B, int HI, int cI, int64_t n_max,
                           const int64_t* pos0, int m, int qk_t, void* scores, int score_t, uint32_t* bound,
                           void* stream) {
  bool empty;
  const csa_status st = check_index_paged(q, q_scale, w, k_pool, k_scale_pool, pages, B, HI, cI, n_max, pos0, m,
                                          qk_t, scores, score_t, bound, empty);
  if (st != CSA_OK || empty) return st;
  return launch_index_paged(q, q_scale, w, k_pool, k_scale_pool, pages, B, HI, cI, n_max, pos0, m, qk_t, scores,
                            score_t, bound, (hipStream_t)stream);
}

csa_status csa_attend_paged(const void* q, const void* comp_pool, const float* comp_scale_pool,
                            const csa_pages* pages, const int32_t* idx, const void* win_ring, const float* sink,
                            const float* gamma_q, const float* gamma_kv, int B, int H, int c, int rope_dims, int k,
                            int n_win, int64_t n_max, const int64_t* pos0, int m, float scale, float eps,
                            float rope_base, int kv_t, int comp_t, int kv_prepared, void* out, int out_t,
                            void* workspace, size_t ws_bytes, void* stream) {
  csa_status st = check_attend(kv_t, out_t, B, 1, H, c, rope_dims, n_win, m);
  if (st != CSA_OK) return st;
  if (kv_t != CSA_BF16) return CSA_ERR_UNSUPPORTED;
  st = check_comp_t(kv_t, comp_t, kv_prepared, c, rope_dims);
  if (st != CSA_OK) return st;
  if (k < 1 || k > 2048 || n_max < 0 || n_max >= ((int64_t)1 << 31)) return CSA_ERR_SHAPE;
  if (kv_prepared < 0 || kv_prepared > 2) return CSA_ERR_UNSUPPORTED;
  st = check_pages(pages, m);
  if (st != CSA_OK) return st;
  st = check_pages_cover(pages, m, n_max);
  if (st != CSA_OK) return st;
  if (B == 0) return CSA_OK;
  if (!q || !idx || !win_ring || !sink || !pos0 || !out || (n_max > 0 && !comp_pool)) return CSA_ERR_NULL;
  if (comp_t != kv_t && n_max > 0 && !comp_scale_pool) return CSA_ERR_NULL;
  const size_t need = csa_attend_workspace_bytes(B, 1, H, c, k, n_win);
  if (need > 0 && (!workspace || ws_bytes < need)) return CSA_ERR_WORKSPACE;
  return launch_attend(0, q, comp_pool, comp_scale_pool, comp_t != kv_t, pages, idx, win_ring, sink, gamma_q,
                       gamma_kv, B, 1, H, c, rope_dims, k, n_win, n_max, pos0, m, scale, eps, rope_base, kv_t,
                       kv_prepared, out, out_t, workspace, (hipStream_t)stream);
}

csa_status hca_attend_paged(const void* q, const void* comp_pool, const float* comp_scale_pool,
                            const csa_pages* pages, const void* win_ring, const float* sink, const float* gamma_q,
                            const float* gamma_kv, int B, int H, int c, int rope_dims, int n_win, int64_t n_max,
                            const int64_t* pos0, int m_hca, float scale, float eps, float rope_base, int kv_t,
                            int comp_t, int kv_prepared, void* out, int out_t, void* workspace, size_t ws_bytes,
                            void* stream) {
  csa_status st = check_attend(kv_t, out_t, B, 1, H, c, rope_dims, n_win, m_hca);
  if (st != CSA_OK) return st;
  if (kv_t != CSA_BF16) return CSA_ERR_UNSUPPORTED;
  st = check_comp_t(kv_t, comp_t, kv_prepared, c, rope_dims);
  if (st != CSA_OK) return st;
  if (n_max < 0 || n_max >= ((int64_t)1 << 24)) return CSA_ERR_SHAPE;
  if (kv_prepared < 0 || kv_prepared > 2) return CSA_ERR_UNSUPPORTED;
  st = check_pages(pages, m_hca);
  if (st != CSA_OK) return st;
  st = check_pages_cover(pages, m_hca, n_max);
  if (st != CSA_OK) return st;
  if (B == 0) return CSA_OK;
  if (!q || !win_ring || !sink || !pos0 || !out || (n_max > 0 && !comp_pool)) return CSA_ERR_NULL;
  if (comp_t != kv_t && n_max > 0 && !comp_scale_pool) return CSA_ERR_NULL;
  const size_t need = hca_attend_workspace_bytes(B, 1, H, c, n_max, n_win);
  if (need > 0 && (!workspace || ws_bytes < need)) return CSA_ERR_WORKSPACE;
  return launch_attend(1, q, comp_pool, comp_scale_pool, comp_t != kv_t, pages, nullptr, win_ring, sink, gamma_q,
                       gamma_kv, B, 1, H, c, rope_dims, 1, n_win, n_max, pos0, m_hca, scale, eps, rope_base, kv_t,
                       kv_prepared, out, out_t, workspace, (hipStream_t)stream);
}


csa_status csa_q_up_proj(const void* cq, const void* w_uq, const void* w_iuq, int rows, int d_c, int n_h, int c,
                         int n_hI, int cI, void* q, void* qi, void* qi_scale, int qi_t, void* stream) {
  if (rows < 0 || d_c < 32 || (d_c % 32) || n_h < 1 || c < 1 || n_hI < 1 || cI < 1) return CSA_ERR_SHAPE;
  if (((int64_t)n_h * c) % 128 || ((int64_t)n_hI * cI) % 128) return CSA_ERR_UNSUPPORTED;
  if ((int64_t)n_h * c >= ((int64_t)1 << 28) || (int64_t)n_hI * cI >= ((int64_t)1 << 28)) return CSA_ERR_SHAPE;
  if (qi_t != CSA_BF16 && qi_t != CSA_FP8_E4M3_ROWSCALE && qi_t != CSA_MXFP4_E8M0_B32) return CSA_ERR_UNSUPPORTED;
  if (qi_t != CSA_BF16 && cI != 128) return CSA_ERR_UNSUPPORTED;
  if (rows == 0) return CSA_OK;
  if (!cq || !w_uq || !w_iuq || !q || !qi || (qi_t != CSA_BF16 && !qi_scale)) return CSA_ERR_NULL;
  // 16-byte operand loads; 8-byte bf16 / 4-byte fp8 / 2-byte MXFP4 result stores
  const uintptr_t qi_align = qi_t == CSA_BF16 ? 7 : (qi_t == CSA_FP8_E4M3_ROWSCALE ? 3 : 1);
  if ((((uintptr_t)cq | (uintptr_t)w_uq | (uintptr_t)w_iuq) & 15) || ((uintptr_t)q & 7) || ((uintptr_t)qi & qi_align))
    return CSA_ERR_UNSUPPORTED;
  return launch_q_up_proj(cq, w_uq, w_iuq, rows, d_c, n_h, c, n_hI, cI, q, qi, qi_scale, qi_t, (hipStream_t)stream);
}

csa_status csa_grouped_out_proj(const void* o, const void* w_g, const void* w_o, int rows, int n_h, int c, int g,
                                int d_g, int d, void* mid, void* out, void* stream) {
  if (rows < 0 || n_h < 1 || c < 1 || g < 1 || d_g < 1 || d < 1) return CSA_ERR_SHAPE;
  if (n_h % g) return CSA_ERR_SHAPE;
  const int64_t per = (int64_t)(n_h / g) * c;
  if (per % 32 || ((int64_t)g * d_g) % 32 || d_g % 16 || d % 16) return CSA_ERR_UNSUPPORTED;
  if (per >= ((int64_t)1 << 28) || (int64_t)g * d_g >= ((int64_t)1 << 28) || g >= 65536) return CSA_ERR_SHAPE;
  if (rows == 0) return CSA_OK;
  if (!o || !w_g || !w_o || !mid || !out) return CSA_ERR_NULL;
  if ((((uintptr_t)o | (uintptr_t)w_g | (uintptr_t)w_o | (uintptr_t)mid) & 15) || ((uintptr_t)out & 7))
    return CSA_ERR_UNSUPPORTED;   // 16-byte operand loads, 8-byte result stores
  return launch_grouped_out_proj(o, w_g, w_o, rows, n_h, c, g, d_g, d, mid, out, (hipStream_t)stream);
}


csa_status csa_topk_compress(const void* scores, int score_t, int B, int64_t n_max, const int64_t* pos0, int m,
                             int k, const uint32_t* bound, int32_t* idx, float* vals, void* workspace,
                             size_t ws_bytes, const void* ca, const void* cb, const void* za, const void* zb,
                             const float* bias_a, const float* bias_b, int c, int rows, int64_t row0_pos,
                             int64_t first_entry, int in_t, void* out, void* out_scale, int out_t,
                             int64_t out_batch_stride, const csa_kv_prep* prep, void* stream) {
  if (m >= 64) return CSA_ERR_UNSUPPORTED;  // one 256-thread workgroup pools the entry's rows
  bool empty;
  csa_status st = check_compress(ca, cb, za, zb, bias_a, bias_b, B, rows, c, m, row0_pos, first_entry, 1, in_t, out,
                                 out_scale, out_t, out_batch_stride, prep, empty);
  if (st != CSA_OK) return st;
  if (score_t != CSA_F32 && score_t != CSA_BF16) return CSA_ERR_UNSUPPORTED;
  if (B < 0 || n_max < 0 || m < 1 || k < 1 || k > 2048) return CSA_ERR_SHAPE;
  if (n_max >= ((int64_t)1 << 31)) return CSA_ERR_SHAPE;
  if (B == 0) return CSA_OK;
  if (!idx || !pos0 || (n_max > 0 && !scores)) return CSA_ERR_NULL;
  const size_t need = csa_topk_workspace_bytes(B, 1, n_max > 0 ? n_max : 1, k);
  if (need > 0 && (!workspace || ws_bytes < need)) return CSA_ERR_WORKSPACE;
  const CompressJob kv{ca, cb, za, zb, bias_a, bias_b, c, out, out_scale, out_t, out_batch_stride, prep};
  return launch_topk(scores, score_t, B, 1, n_max, pos0, m, k, bound, idx, vals, workspace, (hipStream_t)stream, &kv,
                     rows, m, row0_pos, first_entry, in_t);
}


csa_status csa_pack_proj_weights(const void* w, void* packed, int z, int n, int k, void* stream) {
  if (z < 0 || n < 0 || k < 0) return CSA_ERR_SHAPE;
  if (n % 16 || k % 32) return CSA_ERR_UNSUPPORTED;
  if ((int64_t)z * n * k >= ((int64_t)1 << 40)) return CSA_ERR_SHAPE;
  if (z == 0 || n == 0 || k == 0) return CSA_OK;
  if (!w || !packed || w == packed) return CSA_ERR_NULL;
  return launch_pack_proj_weights(w, packed, z, n, k, (hipStream_t)stream);
}

}  // extern "C"

// ---- csa_attend_noalloc: csa_attend with its workspace in a fixed device array ----------------------------------
//
// The decode split partials live in `scratch`, a file-scope device array each GPU holds for the life of the
// process.  Its device address is looked up once per device (hipGetSymbolAddress, with that device current) and
// kept; host code uses only that address, never the array's name, which on the host is a stand-in and not a
// device pointer.  Nothing here allocates.
namespace {
constexpr size_t kNoallocScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

csa_status scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return CSA_ERR_LAUNCH;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (!p) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return CSA_ERR_LAUNCH;
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return CSA_OK;
}
}  // namespace

extern "C" {

csa_status csa_attend_noalloc(const void* q, const void* comp_kv, const float* comp_scale, const int32_t* idx,
                              const void* win_kv, const float* sink, const float* gamma_q, const float* gamma_kv,
                              int B, int T, int H, int c, int rope_dims, int k, int n_win, int64_t n_max,
                              const int64_t* pos0, int m, float scale, float eps, float rope_base, int kv_t,
                              int comp_t, int kv_prepared, void* out, int out_t, void* stream) {
  size_t need = 0;
  csa_status st = check_csa_attend(q, comp_kv, comp_scale, idx, win_kv, sink, B, T, H, c, rope_dims, k, n_win, n_max,
                                   pos0, m, kv_t, comp_t, kv_prepared, out, out_t, &need);
  if (st != CSA_OK || B == 0 || T == 0) return st;
  if (need > kNoallocScratchBytes) return CSA_ERR_WORKSPACE;
  void* ws = nullptr;
  if (need > 0) {
    st = scratch_address(&ws);
    if (st != CSA_OK) return st;
  }
  return launch_attend(0, q, comp_kv, comp_scale, comp_t != kv_t, nullptr, idx, win_kv, sink, gamma_q, gamma_kv, B, T,
                       H, c, rope_dims, k, n_win, n_max, pos0, m, scale, eps, rope_base, kv_t, kv_prepared, out, out_t,
                       ws, (hipStream_t)stream);
}

}  // extern "C"
