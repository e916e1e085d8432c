// csa_compress kernel: learned per-channel softmax pooling of per-token KV rows.
//
// "【论文解读】DeepSeek-V4" (wkq9411.github.io), section 一(三)1(1) "压缩 KV Entries":
// each compressed entry is a per-channel softmax-weighted sum over the m a-rows
// of its own block and the m b-rows of the previous block (block 0: no b-rows);
// section 一(三)2(1) gives the HCA form (one stream, m' rows, no overlap).
//
// Design: one workgroup (256 threads) per (entry, sequence).  Thread tid owns
// channel group cg = tid % (c/4) (4 adjacent channels, one 16-byte / 8-byte load
// per row) and row slice rs = tid / (c/4); each thread runs an online softmax
// over its rows, the slices are merged in LDS in a fixed order, and the rs == 0
// threads write the entry (optionally quantized).  Loads are contiguous across
// the channel groups of a row, so every row read is coalesced.
#include "csa_common.h"
#include "csa_internal.h"

namespace {

constexpr int kThreads = 256;

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

template <typename TIn>
__global__ __launch_bounds__(kThreads) void compress_kernel(
    const TIn* __restrict__ ca, const TIn* __restrict__ cb, const TIn* __restrict__ za,
    const TIn* __restrict__ zb, const float* __restrict__ bias_a, const float* __restrict__ bias_b,
    int rows, int c, int m, int64_t row0_pos, int64_t first_entry, void* __restrict__ out,
    void* __restrict__ out_scale, int out_t, int64_t out_bstride) {
  __shared__ float s_m[kThreads][4];
  __shared__ float s_l[kThreads][4];
  __shared__ float s_a[kThreads][4];
  __shared__ float s_red[kThreads];

  const int e = blockIdx.x;
  const int b = blockIdx.y;
  const int tid = threadIdx.x;
  const int ncg = c >> 2;
  const int nrs = kThreads / ncg;  // row slices (>= 1 because c <= 1024)
  const int cg = tid % ncg;
  const int rs = tid / ncg;
  const bool active = rs < nrs;
  const int64_t i = first_entry + e;
  const bool overlap = (cb != nullptr);
  const int nrows = (overlap && i > 0) ? 2 * m : m;  // i == 0: b-side is -inf / 0
  const int64_t base = (int64_t)b * rows * c;

  float mx[4], sm[4], ac[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) { mx[q] = -INFINITY; sm[q] = 0.0f; ac[q] = 0.0f; }

  if (active) {
    // rows of this thread's slice, 8 at a time: the loads of a batch are issued unconditionally
    // (rows past the end are clamped to a valid row and masked afterwards)
    constexpr int kBatch = 8;
    for (int rr0 = rs; rr0 < nrows; rr0 += kBatch * nrs) {
      Raw4<TIn> z[kBatch], v[kBatch];
      f32x4 bb[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int rr = min(rr0 + u * nrs, nrows - 1);
        const bool is_a = rr < m;
        const int rw = is_a ? rr : rr - m;
        const int64_t row = (is_a ? m * i : m * (i - 1)) + rw - row0_pos;
        z[u].load((is_a ? za : zb) + base + row * c + 4 * cg);
        v[u].load((is_a ? ca : cb) + base + row * c + 4 * cg);
        bb[u] = *reinterpret_cast<const f32x4*>((is_a ? bias_a : bias_b) + (int64_t)rw * c + 4 * cg);
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        if (rr0 + u * nrs >= nrows) break;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float lg = z[u].get(q) + bb[u][q];
          const float val = v[u].get(q);
          if (lg > mx[q]) {
            const float sc = expf(mx[q] - lg);  // exp(-inf) = 0 on the first row
            sm[q] = sm[q] * sc + 1.0f;
            ac[q] = ac[q] * sc + val;
            mx[q] = lg;
          } else {
            const float p = expf(lg - mx[q]);
            sm[q] += p;
            ac[q] = fmaf(p, val, ac[q]);
          }
        }
      }
    }
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) { s_m[tid][q] = mx[q]; s_l[tid][q] = sm[q]; s_a[tid][q] = ac[q]; }
  __syncthreads();

  float y[4] = {0.f, 0.f, 0.f, 0.f};
  const bool writer = (tid < ncg);
  if (writer) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float M = -INFINITY;
      for (int s = 0; s < nrs; ++s) M = fmaxf(M, s_m[s * ncg + cg][q]);
      float L = 0.f, A = 0.f;
      for (int s = 0; s < nrs; ++s) {
        float ms = s_m[s * ncg + cg][q];
        if (ms == -INFINITY) continue;  // slice saw no row
        float f = expf(ms - M);
        L = fmaf(s_l[s * ncg + cg][q], f, L);
        A = fmaf(s_a[s * ncg + cg][q], f, A);
      }
      y[q] = A / L;
    }
  }

  const int64_t orow = (int64_t)b * out_bstride + e;
  if (out_t == CSA_F32) {
    if (writer) {
      f32x4 o = {y[0], y[1], y[2], y[3]};
      *reinterpret_cast<f32x4*>(static_cast<float*>(out) + orow * c + 4 * cg) = o;
    }
    return;
  }
  if (out_t == CSA_BF16) {
    if (writer) {
      uint2 o;
      o.x = (uint32_t)f32_to_bf16(y[0]) | ((uint32_t)f32_to_bf16(y[1]) << 16);
      o.y = (uint32_t)f32_to_bf16(y[2]) | ((uint32_t)f32_to_bf16(y[3]) << 16);
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + orow * c + 4 * cg) = o;
    }
    return;
  }
  if (out_t == CSA_FP8_E4M3_ROWSCALE) {
    // row amax over all c channels (fixed-order tree in LDS)
    float am = writer ? fmaxf(fmaxf(fabsf(y[0]), fabsf(y[1])), fmaxf(fabsf(y[2]), fabsf(y[3]))) : 0.0f;
    s_red[tid] = am;
    __syncthreads();
    for (int w = kThreads / 2; w > 0; w >>= 1) {
      if (tid < w) s_red[tid] = fmaxf(s_red[tid], s_red[tid + w]);
      __syncthreads();
    }
    const float scale = s_red[0] / 448.0f;
    if (writer) {
      uint32_t pk = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float v = scale > 0.0f ? y[q] / scale : 0.0f;
        pk |= f32_to_e4m3(v) << (8 * q);
      }
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
    int X;
    if (am > 0.0f) {
      int ex;
      frexpf(am, &ex);  // am = f * 2^ex, f in [0.5, 1)
      X = ex - 1 - 2;
      X = X < -127 ? -127 : (X > 127 ? 127 : X);
    } else {
      X = -127;
    }
    uint32_t codes = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) codes |= f32_to_e2m1(ldexpf(y[q], -X)) << (4 * q);
    *reinterpret_cast<uint16_t*>(static_cast<uint8_t*>(out) + orow * (c / 2) + 2 * cg) = (uint16_t)codes;
    if ((cg & 7) == 0) static_cast<uint8_t*>(out_scale)[orow * (c / 32) + cg / 8] = (uint8_t)(X + 127);
  }
}

}  // namespace

csa_status launch_compress(const void* ca, const void* cb, const void* za, const void* zb, const float* bias_a,
                           const float* bias_b, int B, int rows, int c, int m, int64_t row0_pos,
                           int64_t first_entry, int num_entries, int in_t, void* out, void* out_scale, int out_t,
                           int64_t out_bstride, hipStream_t stream) {
  dim3 grid(num_entries, B);
  if (in_t == CSA_F32) {
    hipLaunchKernelGGL(compress_kernel<float>, grid, dim3(kThreads), 0, stream, (const float*)ca, (const float*)cb,
                       (const float*)za, (const float*)zb, bias_a, bias_b, rows, c, m, row0_pos, first_entry, out,
                       out_scale, out_t, out_bstride);
  } else {
    hipLaunchKernelGGL(compress_kernel<uint16_t>, grid, dim3(kThreads), 0, stream, (const uint16_t*)ca,
                       (const uint16_t*)cb, (const uint16_t*)za, (const uint16_t*)zb, bias_a, bias_b, rows, c, m,
                       row0_pos, first_entry, out, out_scale, out_t, out_bstride);
  }
  return hipGetLastError() == hipSuccess ? CSA_OK : CSA_ERR_LAUNCH;
}
