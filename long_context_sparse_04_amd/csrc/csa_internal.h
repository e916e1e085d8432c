// Host-side launchers of the gfx950 kernels (called by the C ABI after validation).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/csa.h"

csa_status launch_compress(const void* ca, const void* cb, const void* za, const void* zb, const float* bias_a,
                           const float* bias_b, int B, int rows, int c, int m, int64_t row0_pos,
                           int64_t first_entry, int num_entries, int in_t, void* out, void* out_scale, int out_t,
                           int64_t out_bstride, const csa_kv_prep* prep, hipStream_t stream);

// one problem of a compression launch (see csa_compress_pair)
struct CompressJob {
  const void* ca;
  const void* cb;
  const void* za;
  const void* zb;
  const float* bias_a;
  const float* bias_b;
  int c;
  void* out;
  void* out_scale;
  int out_t;
  int64_t out_bstride;
  const csa_kv_prep* prep;  // NULL: store the pooled entry as it is
};
csa_status launch_compress_jobs(const CompressJob* jobs, int njobs, int B, int rows, int m, int64_t row0_pos,
                                int64_t first_entry, int num_entries, int in_t, hipStream_t stream);

csa_status launch_prepare_kv(const void* in, int64_t in_bstride, void* out, void* out_scale, int64_t out_bstride,
                             int B, int rows, int c, int in_t, int out_t, const int64_t* pos_base, int64_t pos_first,
                             int64_t pos_stride, const csa_kv_prep* prep, hipStream_t stream);

// csa_decode_append (validated): the jobs' rings and paged outputs, the window rings
csa_status launch_decode_append(const csa_append_job* jobs, int njobs, const csa_window_job* wins, int nwins, int B,
                                const int64_t* pos, const csa_pages* pages, int in_t, hipStream_t stream);

csa_status launch_index_paged(const void* q, const void* q_scale, const float* w, const void* k_pool,
                              const void* k_scale_pool, const csa_pages* pages, int B, int HI, int cI, int64_t n_max,
                              const int64_t* pos0, int m, int qk_t, void* scores, int score_t, uint32_t* bound,
                              hipStream_t stream);

// bound keys per query row written by the decode index kernel (two per bound set)
int64_t index_bound_keys(int64_t n_max);
bool use_prefill_index(int fmt, int T, int HI);
csa_status launch_index(const void* q, const void* q_scale, const float* w, const void* k, const void* k_scale,
                        int B, int T, int HI, int cI, int64_t n_max, const int64_t* pos0, int m, int qk_t,
                        void* scores, int score_t, uint32_t* bound, hipStream_t stream);

// csa_compress_pair's two problems (jobs[0]: the KV entry, jobs[1]: the indexer key, whose output is the
// key cache at first_entry) and a decode csa_index (T = 1) in one launch
csa_status launch_compress_index(const CompressJob* jobs, int rows, int m, int64_t row0_pos, int64_t first_entry,
                                 int in_t, const void* q, const void* q_scale, const float* w, const void* k,
                                 const void* k_scale, int B, int HI, int cI, int64_t n_max, const int64_t* pos0,
                                 int qk_t, void* scores, int score_t, uint32_t* bound, hipStream_t stream);

size_t topk_workspace_bytes(int B, int T, int64_t n_max, int k);
// kv (optional, decode): a KV-entry compression (entry kv_first of each sequence, rows as csa_compress) done
// inside the launch by one more workgroup per row
csa_status launch_topk(const void* scores, int score_t, int B, int T, int64_t n_max, const int64_t* pos0, int m, int k,
                       const uint32_t* bound, int32_t* idx, float* vals, void* ws, hipStream_t stream,
                       const CompressJob* kv = nullptr, int kv_rows = 0, int kv_m = 0, int64_t kv_row0 = 0,
                       int64_t kv_first = 0, int kv_in_t = 0);

// mode 0: CSA (index list), mode 1: HCA (dense range)
size_t attend_workspace_bytes(int mode, int B, int T, int H, int c, int64_t ncomp, int n_win);
// comp_mixed: comp_kv rows in CSA_FP8_BF16_ROPE with their scales in comp_scale
// pages (non-NULL, decode rows only): comp_kv / comp_scale are paged pools, win_kv a ring [B][n_win][c]
csa_status launch_attend(int mode, const void* q, const void* comp_kv, const float* comp_scale, bool comp_mixed,
                         const csa_pages* pages, const int32_t* idx, const void* win_kv,
                         const float* sink, const float* gamma_q, const float* gamma_kv, int B, int T, int H,
                         int c, int rope_dims, int k, int n_win, int64_t n_max, const int64_t* pos0, int m,
                         float scale, float eps, float rope_base, int kv_t, int kv_prepared, void* out, int out_t,
                         void* ws, hipStream_t stream);

// dense projections for decode rows (validated)
csa_status launch_q_up_proj(const void* cq, const void* w_uq, const void* w_iuq, int rows, int d_c, int n_h, int c,
                            int n_hI, int cI, void* q, void* qi, void* qi_scale, int qi_t, hipStream_t stream);
csa_status launch_grouped_out_proj(const void* o, const void* w_g, const void* w_o, int rows, int n_h, int c, int g,
                                   int d_g, int d, void* mid, void* out, hipStream_t stream);

// csa_decode_append's work for the token (two jobs: KV entry, indexer key into k_pool; optional window) fused
// into the paged decode index launch (validated)
csa_status launch_append_index_paged(const csa_append_job* jobs, const csa_window_job* win, int in_t, const void* q,
                                     const void* q_scale, const float* w, const void* k_pool,
                                     const void* k_scale_pool, const csa_pages* pages, int B, int HI, int cI,
                                     int64_t n_max, const int64_t* pos0, int m, int qk_t, void* scores, int score_t,
                                     uint32_t* bound, hipStream_t stream);
csa_status launch_pack_proj_weights(const void* w, void* packed, int z, int n, int k, hipStream_t stream);
