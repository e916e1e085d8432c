// Compression of one entry of one sequence by one workgroup of NT threads: the body shared by the
// csa_compress kernel and the fused compress-then-index launch.
//
// "【论文解读】DeepSeek-V4" (wkq9411.github.io), section 一(三)1(1) "压缩 KV Entries":
// each compressed entry is a per-channel softmax-weighted sum over the m a-rows
// of its own block and the m b-rows of the previous block (block 0: no b-rows);
// section 一(三)2(1) gives the HCA form (one stream, m' rows, no overlap).
//
// Thread tid owns channel group cg = tid % (c/4) (4 adjacent channels, one 16-byte / 8-byte load per
// row) and row slice rs = tid / (c/4); each thread runs an online softmax over its rows (branch-free,
// base-2 exponentials), the slices are merged in LDS in a fixed order, and the rs == 0 threads write
// the entry (optionally prepared for attention, or quantized).  Loads are contiguous across the
// channel groups of a row, so every row read is coalesced.
#pragma once
#include "csa_common.h"
#include "csa_internal.h"

namespace csa_compress_body {

// Raw 4-channel loads (kept as bits until use, so that a batch of loads has no
// dependent instruction between them) and their conversion to float32.
template <typename TIn>
struct Raw4;
template <>
struct Raw4<float> {
  f32x4 v;
  CSA_DEV void load(const float* p) { v = *reinterpret_cast<const f32x4*>(p); }
  CSA_DEV float get(int q) const { return v[q]; }
};
template <>
struct Raw4<uint16_t> {
  uint2 v;
  CSA_DEV void load(const uint16_t* p) { v = *reinterpret_cast<const uint2*>(p); }
  CSA_DEV float get(int q) const {
    const uint32_t w = (q < 2) ? v.x : v.y;
    return __uint_as_float((q & 1) ? (w & 0xFFFF0000u) : (w << 16));
  }
};

constexpr float kLog2e = 1.4426950408889634f;

// A row's logit in base-2 units, rounded on its own: the multiply is not contracted into a later
// subtraction (an instruction compiled without contraction is never fused), so the row holding the maximum
// has lg2 - mx = 0 exactly.
CSA_DEV float logit2(float z, float bias) {
#pragma clang fp contract(off)
  return (z + bias) * kLog2e;
}

// Online softmax state of 4 channels in base-2 units (logits scaled by log2 e).
struct Soft4 {
  float mx[4], sm[4], ac[4];
  CSA_DEV void init() {
#pragma unroll
    for (int q = 0; q < 4; ++q) { mx[q] = -INFINITY; sm[q] = 0.0f; ac[q] = 0.0f; }
  }
  // branch-free update with one row: logit lg2 (finite, base 2, from logit2) and value v; the row holding
  // the maximum gets weight exp2(0) = 1, so a logit far above the others returns its row's value bit for bit
  CSA_DEV void add(int q, float lg2, float v) {
    const float mn = fmaxf(mx[q], lg2);
    const float sc = __builtin_amdgcn_exp2f(mx[q] - mn);  // 0 while the state is empty
    const float p = __builtin_amdgcn_exp2f(lg2 - mn);
    sm[q] = fmaf(sm[q], sc, p);
    ac[q] = fmaf(ac[q], sc, p * v);
    mx[q] = mn;
  }
};

// One compression problem: its streams, biases, width and output.  A launch serves one or two of
// them (blockIdx.z), with the same batch, rows, ratio and entries, e.g. a block's KV entry and its
// indexer-key entry.
struct Job {
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
  int prep;            // store the entry prepared for attention (RMSNorm + RoPE at m * i)
  const float* gamma;
  float eps;
  int R;
  int ring;              // > 0: rows are a state ring of `ring` rows per sequence (position p at p % ring)
  const int32_t* table;  // non-NULL: the output is a paged pool (entry i of sequence b at its page's row)
  int tstride;           // block-table row length
  int plog2;             // log2 of the entries per page
};
struct Jobs {
  Job j[2];
  double theta[2][64];  // RoPE frequencies of each job
};

// Entry first_entry + e of sequence b: reads the job's rows, writes row b * out_bstride + e of its
// output.  s_m, s_l, s_a: NT f32x4 each; s_red: NT / 64 floats (LDS).
template <typename TIn, int NT>
CSA_DEV void compress_one(const Job& jb, const double* theta, int e, int b, int rows, int m, int64_t row0_pos,
                          int64_t first_entry, f32x4* s_m, f32x4* s_l, f32x4* s_a, float* s_red) {
  const TIn* __restrict__ ca = static_cast<const TIn*>(jb.ca);
  const TIn* __restrict__ cb = static_cast<const TIn*>(jb.cb);
  const TIn* __restrict__ za = static_cast<const TIn*>(jb.za);
  const TIn* __restrict__ zb = static_cast<const TIn*>(jb.zb);
  const float* __restrict__ bias_a = jb.bias_a;
  const float* __restrict__ bias_b = jb.bias_b;
  const int c = jb.c;
  void* __restrict__ out = jb.out;
  void* __restrict__ out_scale = jb.out_scale;
  const int out_t = jb.out_t;
  const int64_t out_bstride = jb.out_bstride;
  const int tid = threadIdx.x;
  const int ncg = c >> 2;
  const int nrs = NT / ncg;  // row slices (>= 1 because c <= 1024)
  const int cg = tid % ncg;
  const int rs = tid / ncg;
  const int64_t i = first_entry + e;
  const bool overlap = (cb != nullptr);
  const int nrows = (overlap && i > 0) ? 2 * m : m;  // i == 0: the b-side is -inf / 0
  const int64_t base = (int64_t)b * (jb.ring ? jb.ring : rows) * c;

  Soft4 st;
  st.init();
  if (rs < nrs) {
    // rows of this thread's slice, 4 at a time: loads issued unconditionally (rows past the end
    // are clamped to a valid row and skipped afterwards)
    constexpr int kBatch = 4;
    for (int rr0 = rs; rr0 < nrows; rr0 += kBatch * nrs) {
      Raw4<TIn> z[kBatch], v[kBatch];
      f32x4 bb[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int rr = min(rr0 + u * nrs, nrows - 1);
        const bool is_a = rr < m;
        const int rw = is_a ? rr : rr - m;
        const int64_t p = (is_a ? m * i : m * (i - 1)) + rw;  // the row's token position
        const int64_t row = jb.ring ? p % jb.ring : p - row0_pos;
        z[u].load((is_a ? za : zb) + base + row * c + 4 * cg);
        v[u].load((is_a ? ca : cb) + base + row * c + 4 * cg);
        bb[u] = *reinterpret_cast<const f32x4*>((is_a ? bias_a : bias_b) + (int64_t)rw * c + 4 * cg);
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        if (rr0 + u * nrs >= nrows) break;
#pragma unroll
        for (int q = 0; q < 4; ++q) st.add(q, logit2(z[u].get(q), bb[u][q]), v[u].get(q));
      }
    }
  }
  s_m[tid] = f32x4{st.mx[0], st.mx[1], st.mx[2], st.mx[3]};
  s_l[tid] = f32x4{st.sm[0], st.sm[1], st.sm[2], st.sm[3]};
  s_a[tid] = f32x4{st.ac[0], st.ac[1], st.ac[2], st.ac[3]};
  __syncthreads();

  // merge the row slices in a fixed order (slice 0 first)
  float y[4] = {0.f, 0.f, 0.f, 0.f};
  const bool writer = (tid < ncg);
  if (writer) {
    f32x4 M = s_m[cg];
    for (int sl = 1; sl < nrs; ++sl) {
      const f32x4 mo = s_m[sl * ncg + cg];
#pragma unroll
      for (int q = 0; q < 4; ++q) M[q] = fmaxf(M[q], mo[q]);
    }
    float L[4] = {0.f, 0.f, 0.f, 0.f}, A[4] = {0.f, 0.f, 0.f, 0.f};
    for (int sl = 0; sl < nrs; ++sl) {
      const f32x4 ms = s_m[sl * ncg + cg], ls = s_l[sl * ncg + cg], as = s_a[sl * ncg + cg];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float f = (ms[q] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(ms[q] - M[q]);  // empty slice
        L[q] = fmaf(ls[q], f, L[q]);
        A[q] = fmaf(as[q], f, A[q]);
      }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) y[q] = A[q] / L[q];
  }

  if (jb.prep) prep_row4<NT>(y, writer, cg, c, (double)m * (double)i, jb.gamma, jb.eps, jb.R, theta, s_red);
  const int64_t orow =
      jb.table ? (((int64_t)jb.table[(int64_t)b * jb.tstride + (i >> jb.plog2)] << jb.plog2) | (i & ((1 << jb.plog2) - 1)))
               : (int64_t)b * out_bstride + e;
  if (out_t == CSA_FP8_BF16_ROPE) {  // prepared entries only (checked on the host)
    store_fp8_rope_row<NT>(y, writer, cg, c, jb.R, static_cast<uint8_t*>(out) + orow * (c + jb.R),
                           static_cast<float*>(out_scale) + orow, s_red);
    return;
  }
  if (out_t == CSA_F32) {
    if (writer) *reinterpret_cast<f32x4*>(static_cast<float*>(out) + orow * c + 4 * cg) = f32x4{y[0], y[1], y[2], y[3]};
    return;
  }
  if (out_t == CSA_BF16) {
    if (writer) {
      uint2 o;
      o.x = pack_bf16x2(y[0], y[1]);
      o.y = pack_bf16x2(y[2], y[3]);
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + orow * c + 4 * cg) = o;
    }
    return;
  }
  if (out_t == CSA_FP8_E4M3_ROWSCALE) {
    // row amax over all c channels: wave maxima, then the block maximum through LDS
    float am = writer ? fmaxf(fmaxf(fabsf(y[0]), fabsf(y[1])), fmaxf(fabsf(y[2]), fabsf(y[3]))) : 0.0f;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) am = fmaxf(am, __shfl_xor(am, o, 64));
    if ((tid & 63) == 0) s_red[tid >> 6] = am;
    __syncthreads();
    am = s_red[0];
#pragma unroll
    for (int w = 1; w < NT / 64; ++w) am = fmaxf(am, s_red[w]);
    const float scale = am / 448.0f;
    if (writer) {
      uint32_t pk = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) pk |= f32_to_e4m3(scale > 0.0f ? y[q] / scale : 0.0f) << (8 * q);
      *reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(out) + orow * c + 4 * cg) = pk;
      if (tid == 0) static_cast<float*>(out_scale)[orow] = scale;
    }
    return;
  }
  // CSA_MXFP4_E8M0_B32: 8 channel groups (32 channels) share one E8M0 scale
  if (writer) {
    float am = fmaxf(fmaxf(fabsf(y[0]), fabsf(y[1])), fmaxf(fabsf(y[2]), fabsf(y[3])));
    am = fmaxf(am, __shfl_xor(am, 1, 8));
    am = fmaxf(am, __shfl_xor(am, 2, 8));
    am = fmaxf(am, __shfl_xor(am, 4, 8));
    int X = -127;
    if (am > 0.0f) {
      int ex;
      frexpf(am, &ex);  // am = f * 2^ex, f in [0.5, 1)
      X = ex - 1 - 2;
      X = X < -127 ? -127 : (X > 127 ? 127 : X);
    }
    uint32_t codes = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) codes |= f32_to_e2m1(ldexpf(y[q], -X)) << (4 * q);
    *reinterpret_cast<uint16_t*>(static_cast<uint8_t*>(out) + orow * (c / 2) + 2 * cg) = (uint16_t)codes;
    if ((cg & 7) == 0) static_cast<uint8_t*>(out_scale)[orow * (c / 32) + cg / 8] = (uint8_t)(X + 127);
  }
}


// A decode token's state-cache work (csa_decode_append) carried by another launch: the KV entry and the
// indexer key (rings in Job::ring, paged outputs in Job::table), the token's ring rows, the window row.
struct AppendFuse {
  Jobs jobs;               // j[0]: the KV entry, j[1]: the indexer key
  const void* src[2][4];   // the token's rows of each job: ca, cb, za, zb ([B][c])
  int m, in_t;
  const void* win_row;     // the window job (win_ring NULL: none)
  void* win_ring;
  int win_c, win_n, win_prep;
  const float* win_gamma;
  float win_eps;
  int win_R;
  double win_theta[64];
};

// The token's rows of a job into ring row t % ring (every thread of the block takes part).
template <typename TIn>
CSA_DEV void store_ring_rows(const Job& jb, const void* const* src, int b, int64_t t) {
  const int64_t rrow = ((int64_t)b * jb.ring + t % jb.ring) * jb.c;
  const void* dst[4] = {jb.ca, jb.cb, jb.za, jb.zb};
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    if (!dst[s]) continue;
    const TIn* from = static_cast<const TIn*>(src[s]) + (int64_t)b * jb.c;
    TIn* to = static_cast<TIn*>(const_cast<void*>(dst[s])) + rrow;
    for (int q = threadIdx.x; q < jb.c / 4; q += blockDim.x) {
      if constexpr (sizeof(TIn) == 4)
        reinterpret_cast<f32x4*>(to)[q] = reinterpret_cast<const f32x4*>(from)[q];
      else
        reinterpret_cast<uint2*>(to)[q] = reinterpret_cast<const uint2*>(from)[q];
    }
  }
}

// The token's window row into ring row t % n_win, prepared at position t when asked (every thread of the
// NT-thread block calls it: it holds barriers).  s_red: NT / 64 floats.
template <typename TIn, int NT>
CSA_DEV void store_window_row(const AppendFuse& a, int b, int64_t t, float* s_red) {
  const int c = a.win_c;
  const int cg = threadIdx.x;
  const bool holder = cg < c / 4;
  float y[4] = {0.f, 0.f, 0.f, 0.f};
  if (holder) {
    Raw4<TIn> v;
    v.load(static_cast<const TIn*>(a.win_row) + (int64_t)b * c + 4 * cg);
#pragma unroll
    for (int q = 0; q < 4; ++q) y[q] = v.get(q);
  }
  if (a.win_prep) prep_row4<NT>(y, holder, cg, c, (double)t, a.win_gamma, a.win_eps, a.win_R, a.win_theta, s_red);
  if (!holder) return;
  TIn* out = static_cast<TIn*>(a.win_ring) + ((int64_t)b * a.win_n + t % a.win_n) * c + 4 * cg;
  if constexpr (sizeof(TIn) == 4) {
    *reinterpret_cast<f32x4*>(out) = f32x4{y[0], y[1], y[2], y[3]};
  } else {
    uint2 o;
    o.x = pack_bf16x2(y[0], y[1]);
    o.y = pack_bf16x2(y[2], y[3]);
    *reinterpret_cast<uint2*>(out) = o;
  }
}

// host: device-side job descriptions (and RoPE tables) of up to two compression problems
void fill_jobs(const CompressJob* jobs, int njobs, Jobs& js);
// host: an AppendFuse from csa_decode_append's two compression jobs and optional window job
void fill_append(const csa_append_job* jobs, const csa_window_job* win, const csa_pages* pages, int in_t,
                 AppendFuse& af);

}  // namespace csa_compress_body
