// csa_compress kernel: learned per-channel softmax pooling of per-token KV rows.
//
// "【论文解读】DeepSeek-V4" (wkq9411.github.io), section 一(三)1(1) "压缩 KV Entries":
// each compressed entry is a per-channel softmax-weighted sum over the m a-rows
// of its own block and the m b-rows of the previous block (block 0: no b-rows);
// section 一(三)2(1) gives the HCA form (one stream, m' rows, no overlap).
//
// Design: one workgroup (256 threads; 1024 for entries that pool 64 rows or more) per (entry,
// sequence, job), running the shared body in compress_body.h.
#include "compress_body.h"
#include "csa_common.h"
#include "csa_internal.h"

namespace {
using namespace csa_compress_body;

constexpr int kThreads = 256;

template <typename TIn, int NT>
__global__ __launch_bounds__(NT) void compress_kernel(Jobs jobs, int rows, int m, int64_t row0_pos,
                                                            int64_t first_entry) {
  __shared__ f32x4 s_m[NT], s_l[NT], s_a[NT];
  __shared__ float s_red[NT / 64];
  const Job jb = blockIdx.z ? jobs.j[1] : jobs.j[0];  // uniform select (no indexed kernel-argument copy)
  compress_one<TIn, NT>(jb, jobs.theta[blockIdx.z], blockIdx.x, blockIdx.y, rows, m, row0_pos, first_entry, s_m,
                        s_l, s_a, s_red);
}

// csa_decode_append: workgroup (b, j) serves sequence b; j < njobs is a compression problem (its
// entry, when the token completes a block, then the token's rows into the rings), j >= njobs a window
// ring.  All rows of a job's entry are loaded before compress_one's first barrier, so once it returns
// the token's rows may replace the oldest ring rows.
struct WinJob {
  const void* row;
  void* ring;
  int c, n_win, prep;
  const float* gamma;
  float eps;
  int R;
};
struct AppendArgs {
  Jobs jobs;                  // ca .. zb of each job are its rings (Job::ring > 0), out its paged pool
  const void* src[2][4];      // the token's rows of each job: ca, cb, za, zb ([B][c])
  int jm[2];                  // each job's ratio
  int njobs;
  WinJob win[2];
  double wtheta[2][64];
  const int64_t* pos;
};

template <typename TIn>
CSA_DEV void copy_row4(const TIn* src, TIn* dst, int c) {  // c / 4 chunks of 4 elements
  for (int q = threadIdx.x; q < c / 4; q += blockDim.x) {
    if constexpr (sizeof(TIn) == 4)
      reinterpret_cast<f32x4*>(dst)[q] = reinterpret_cast<const f32x4*>(src)[q];
    else
      reinterpret_cast<uint2*>(dst)[q] = reinterpret_cast<const uint2*>(src)[q];
  }
}

template <typename TIn, int NT>
__global__ __launch_bounds__(NT) void append_kernel(AppendArgs a) {
  __shared__ f32x4 s_m[NT], s_l[NT], s_a[NT];
  __shared__ float s_red[NT / 64];
  const int b = blockIdx.x;
  const int j = blockIdx.y;
  const int64_t t = a.pos[b];
  if (t < 0) return;  // (uniform) no position: nothing to store
  if (j < a.njobs) {
    const Job jb = j ? a.jobs.j[1] : a.jobs.j[0];  // uniform select
    const int m = j ? a.jm[1] : a.jm[0];
    // (uniform) an entry whose page lies past the block table's row is not stored
    if (t >= m && t % m == 0 && ((t / m - 1) >> jb.plog2) < jb.tstride)
      compress_one<TIn, NT>(jb, a.jobs.theta[j], 0, b, 0, m, 0, t / m - 1, s_m, s_l, s_a, s_red);
    const int64_t rrow = ((int64_t)b * jb.ring + t % jb.ring) * jb.c;
    const void* const* src = j ? a.src[1] : a.src[0];
    const void* dst[4] = {jb.ca, jb.cb, jb.za, jb.zb};
#pragma unroll
    for (int s = 0; s < 4; ++s)
      if (dst[s])
        copy_row4<TIn>(static_cast<const TIn*>(src[s]) + (int64_t)b * jb.c,
                       static_cast<TIn*>(const_cast<void*>(dst[s])) + rrow, jb.c);
    return;
  }
  const WinJob wj = (j - a.njobs) ? a.win[1] : a.win[0];
  const double* theta = (j - a.njobs) ? a.wtheta[1] : a.wtheta[0];
  const int c = wj.c;
  const int cg = threadIdx.x;
  const bool holder = cg < c / 4;
  const TIn* in = static_cast<const TIn*>(wj.row) + (int64_t)b * c;
  float y[4] = {0.f, 0.f, 0.f, 0.f};
  if (holder) {
    Raw4<TIn> v;
    v.load(in + 4 * cg);
#pragma unroll
    for (int q = 0; q < 4; ++q) y[q] = v.get(q);
  }
  if (wj.prep) prep_row4<NT>(y, holder, cg, c, (double)t, wj.gamma, wj.eps, wj.R, theta, s_red);
  if (!holder) return;
  TIn* out = static_cast<TIn*>(wj.ring) + ((int64_t)b * wj.n_win + t % wj.n_win) * c + 4 * cg;
  if constexpr (sizeof(TIn) == 4) {
    *reinterpret_cast<f32x4*>(out) = f32x4{y[0], y[1], y[2], y[3]};
  } else {
    uint2 o;
    o.x = pack_bf16x2(y[0], y[1]);
    o.y = pack_bf16x2(y[2], y[3]);
    *reinterpret_cast<uint2*>(out) = o;
  }
}

}  // namespace

csa_status launch_compress(const void* ca, const void* cb, const void* za, const void* zb, const float* bias_a,
                           const float* bias_b, int B, int rows, int c, int m, int64_t row0_pos,
                           int64_t first_entry, int num_entries, int in_t, void* out, void* out_scale, int out_t,
                           int64_t out_bstride, const csa_kv_prep* prep, hipStream_t stream) {
  CompressJob j{ca, cb, za, zb, bias_a, bias_b, c, out, out_scale, out_t, out_bstride, prep};
  return launch_compress_jobs(&j, 1, B, rows, m, row0_pos, first_entry, num_entries, in_t, stream);
}

void csa_compress_body::fill_jobs(const CompressJob* jobs, int njobs, Jobs& js) {
  for (int i = 0; i < njobs; ++i) {
    const csa_kv_prep* pp = jobs[i].prep;
    js.j[i] = Job{jobs[i].ca, jobs[i].cb, jobs[i].za, jobs[i].zb, jobs[i].bias_a, jobs[i].bias_b, jobs[i].c,
                  jobs[i].out, jobs[i].out_scale, jobs[i].out_t, jobs[i].out_bstride, pp ? 1 : 0,
                  pp ? pp->gamma : nullptr, pp ? pp->eps : 0.0f, pp ? pp->rope_dims : 0, 0, nullptr, 0, 0};
    const RopeTable rt = make_rope_table(pp ? pp->rope_dims : 0, pp ? pp->rope_base : 1.0f);
    for (int t = 0; t < 64; ++t) js.theta[i][t] = rt.theta[t];
  }
}

csa_status launch_compress_jobs(const CompressJob* jobs, int njobs, int B, int rows, int m, int64_t row0_pos,
                                int64_t first_entry, int num_entries, int in_t, hipStream_t stream) {
  Jobs js;
  fill_jobs(jobs, njobs, js);
  dim3 grid(num_entries, B, njobs);
  // an entry that pools many rows (HCA: m' = 128) gets 1024 threads, so that each thread walks few rows;
  // the choice depends on m only, so an entry's result does not depend on the batch
  if (m >= 64) {
    if (in_t == CSA_F32)
      hipLaunchKernelGGL((compress_kernel<float, 1024>), grid, dim3(1024), 0, stream, js, rows, m, row0_pos,
                         first_entry);
    else
      hipLaunchKernelGGL((compress_kernel<uint16_t, 1024>), grid, dim3(1024), 0, stream, js, rows, m, row0_pos,
                         first_entry);
  } else {
    if (in_t == CSA_F32)
      hipLaunchKernelGGL((compress_kernel<float, kThreads>), grid, dim3(kThreads), 0, stream, js, rows, m, row0_pos,
                         first_entry);
    else
      hipLaunchKernelGGL((compress_kernel<uint16_t, kThreads>), grid, dim3(kThreads), 0, stream, js, rows, m,
                         row0_pos, first_entry);
  }
  return hipGetLastError() == hipSuccess ? CSA_OK : CSA_ERR_LAUNCH;
}

namespace {

// csa_prepare_kv: one workgroup per (row, sequence); thread t < c/4 owns channels [4t, 4t + 4).
template <typename TIn>
__global__ __launch_bounds__(kThreads) void prepare_kernel(const TIn* __restrict__ in, int64_t in_bstride,
                                                           void* __restrict__ out, float* __restrict__ out_scale,
                                                           int64_t out_bstride, int c,
                                                           int out_t, const int64_t* __restrict__ pos_base,
                                                           int64_t pos_first, int64_t pos_stride,
                                                           const float* __restrict__ gamma, float eps, int R,
                                                           RopeTable rt) {
  __shared__ float s_red[kThreads / 64];
  const int j = blockIdx.x;
  const int b = blockIdx.y;
  const int cg = threadIdx.x;
  const bool holder = cg < (c >> 2);
  float y[4] = {0.f, 0.f, 0.f, 0.f};
  if (holder) {
    Raw4<TIn> v;
    v.load(in + ((int64_t)b * in_bstride + j) * c + 4 * cg);
#pragma unroll
    for (int q = 0; q < 4; ++q) y[q] = v.get(q);
  }
  const int64_t pos = (pos_base ? pos_base[b] : 0) + pos_first + (int64_t)j * pos_stride;
  prep_row4<kThreads>(y, holder, cg, c, (double)pos, gamma, eps, R, rt.theta, s_red);
  if (out_t == CSA_FP8_BF16_ROPE) {
    const int64_t orow = (int64_t)b * out_bstride + j;
    store_fp8_rope_row<kThreads>(y, holder, cg, c, R, static_cast<uint8_t*>(out) + orow * (c + R), out_scale + orow,
                                 s_red);
    return;
  }
  if (!holder) return;
  const int64_t o = ((int64_t)b * out_bstride + j) * c + 4 * cg;
  if (out_t == CSA_F32) {
    *reinterpret_cast<f32x4*>(static_cast<float*>(out) + o) = f32x4{y[0], y[1], y[2], y[3]};
  } else {
    uint2 pk;
    pk.x = pack_bf16x2(y[0], y[1]);
    pk.y = pack_bf16x2(y[2], y[3]);
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + o) = pk;
  }
}

}  // namespace

csa_status launch_prepare_kv(const void* in, int64_t in_bstride, void* out, void* out_scale, int64_t out_bstride,
                             int B, int rows, int c, int in_t, int out_t, const int64_t* pos_base, int64_t pos_first,
                             int64_t pos_stride, const csa_kv_prep* prep, hipStream_t stream) {
  const RopeTable rt = make_rope_table(prep->rope_dims, prep->rope_base);
  dim3 grid(rows, B);
  float* osc = static_cast<float*>(out_scale);
  if (in_t == CSA_F32)
    hipLaunchKernelGGL(prepare_kernel<float>, grid, dim3(kThreads), 0, stream, (const float*)in, in_bstride, out, osc,
                       out_bstride, c, out_t, pos_base, pos_first, pos_stride, prep->gamma, prep->eps,
                       prep->rope_dims, rt);
  else
    hipLaunchKernelGGL(prepare_kernel<uint16_t>, grid, dim3(kThreads), 0, stream, (const uint16_t*)in, in_bstride,
                       out, osc, out_bstride, c, out_t, pos_base, pos_first, pos_stride, prep->gamma, prep->eps,
                       prep->rope_dims, rt);
  return hipGetLastError() == hipSuccess ? CSA_OK : CSA_ERR_LAUNCH;
}

csa_status launch_decode_append(const csa_append_job* jobs, int njobs, const csa_window_job* wins, int nwins, int B,
                                const int64_t* pos, const csa_pages* pages, int in_t, hipStream_t stream) {
  AppendArgs a;
  a.njobs = njobs;
  a.pos = pos;
  CompressJob cj[2];
  for (int i = 0; i < njobs; ++i) {
    const csa_append_job& jb = jobs[i];
    const bool overlap = jb.cb != nullptr;
    cj[i] = CompressJob{jb.ring_ca, overlap ? jb.ring_cb : nullptr, jb.ring_za, overlap ? jb.ring_zb : nullptr,
                        jb.bias_a, overlap ? jb.bias_b : nullptr, jb.c, jb.out, jb.out_scale, jb.out_t, 0, jb.prep};
  }
  fill_jobs(cj, njobs, a.jobs);
  for (int i = 0; i < njobs; ++i) {
    const csa_append_job& jb = jobs[i];
    const bool overlap = jb.cb != nullptr;
    Job& J = a.jobs.j[i];
    J.ring = overlap ? 2 * jb.m : jb.m;
    J.table = pages->block_table;
    J.tstride = pages->max_pages;
    int plog2 = 0;
    while ((1 << plog2) < pages->page_tokens / jb.m) ++plog2;
    J.plog2 = plog2;
    a.src[i][0] = jb.ca;
    a.src[i][1] = overlap ? jb.cb : nullptr;
    a.src[i][2] = jb.za;
    a.src[i][3] = overlap ? jb.zb : nullptr;
    a.jm[i] = jb.m;
  }
  for (int i = 0; i < nwins; ++i) {
    const csa_window_job& w = wins[i];
    const csa_kv_prep* pp = w.prep;
    a.win[i] = WinJob{w.row, w.ring, w.c, w.n_win, pp ? 1 : 0, pp ? pp->gamma : nullptr, pp ? pp->eps : 0.0f,
                      pp ? pp->rope_dims : 0};
    const RopeTable rt = make_rope_table(pp ? pp->rope_dims : 0, pp ? pp->rope_base : 1.0f);
    for (int q = 0; q < 64; ++q) a.wtheta[i][q] = rt.theta[q];
  }
  dim3 grid(B, njobs + nwins);
  const bool wide = jobs[0].m >= 64;  // the thread count csa_compress uses for the same ratio
  if (wide) {
    if (in_t == CSA_F32)
      hipLaunchKernelGGL((append_kernel<float, 1024>), grid, dim3(1024), 0, stream, a);
    else
      hipLaunchKernelGGL((append_kernel<uint16_t, 1024>), grid, dim3(1024), 0, stream, a);
  } else {
    if (in_t == CSA_F32)
      hipLaunchKernelGGL((append_kernel<float, kThreads>), grid, dim3(kThreads), 0, stream, a);
    else
      hipLaunchKernelGGL((append_kernel<uint16_t, kThreads>), grid, dim3(kThreads), 0, stream, a);
  }
  return hipGetLastError() == hipSuccess ? CSA_OK : CSA_ERR_LAUNCH;
}

void csa_compress_body::fill_append(const csa_append_job* jobs, const csa_window_job* win, const csa_pages* pages,
                                    int in_t, AppendFuse& af) {
  CompressJob cj[2];
  for (int i = 0; i < 2; ++i) {
    const csa_append_job& jb = jobs[i];
    const bool overlap = jb.cb != nullptr;
    cj[i] = CompressJob{jb.ring_ca, overlap ? jb.ring_cb : nullptr, jb.ring_za, overlap ? jb.ring_zb : nullptr,
                        jb.bias_a, overlap ? jb.bias_b : nullptr, jb.c, jb.out, jb.out_scale, jb.out_t, 0, jb.prep};
  }
  fill_jobs(cj, 2, af.jobs);
  for (int i = 0; i < 2; ++i) {
    const csa_append_job& jb = jobs[i];
    const bool overlap = jb.cb != nullptr;
    Job& J = af.jobs.j[i];
    J.ring = overlap ? 2 * jb.m : jb.m;
    J.table = pages->block_table;
    J.tstride = pages->max_pages;
    int plog2 = 0;
    while ((1 << plog2) < pages->page_tokens / jb.m) ++plog2;
    J.plog2 = plog2;
    af.src[i][0] = jb.ca;
    af.src[i][1] = overlap ? jb.cb : nullptr;
    af.src[i][2] = jb.za;
    af.src[i][3] = overlap ? jb.zb : nullptr;
  }
  af.m = jobs[0].m;
  af.in_t = in_t;
  af.win_row = win ? win->row : nullptr;
  af.win_ring = win ? win->ring : nullptr;
  af.win_c = win ? win->c : 0;
  af.win_n = win ? win->n_win : 1;
  const csa_kv_prep* pp = win ? win->prep : nullptr;
  af.win_prep = pp ? 1 : 0;
  af.win_gamma = pp ? pp->gamma : nullptr;
  af.win_eps = pp ? pp->eps : 0.0f;
  af.win_R = pp ? pp->rope_dims : 0;
  const RopeTable rt = make_rope_table(pp ? pp->rope_dims : 0, pp ? pp->rope_base : 1.0f);
  for (int q = 0; q < 64; ++q) af.win_theta[q] = rt.theta[q];
}
