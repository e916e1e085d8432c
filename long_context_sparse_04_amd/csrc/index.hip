// csa_index kernels: lightning-indexer scores.
//
// "【论文解读】DeepSeek-V4" (wkq9411.github.io), section 一(三)1(2): the score of
// query t against compressed indexer key s < floor(t/m) is
// sum_h w_{t,h} * ReLU(q^I_{t,h} . K^IComp_s); section 二(四) puts this QK path in
// FP4 (MXFP4) and the scores in FP32 before top-k.
//
// MFMA design (BF16 / FP8 / MXFP4, c^I = 128): one wave owns one query row's
// HI x 128 indexer queries as the A operand, held in registers for the whole
// launch (heads are MFMA rows), and streams 16-entry tiles of K^IComp straight
// from HBM into the B operand (entries are MFMA columns).  Each lane loads one
// contiguous slice of one entry row, so a wave reads 16 whole rows per tile; a
// wave loads 4 tiles at a time, double-buffered so that the next 4 are in flight
// during the MFMAs and epilogue of the current ones.  K is used exactly once,
// so there is no LDS staging.  The epilogue applies ReLU and the per-head weights
// in the MFMA output layout (lane = entry column, 4 heads per lane per 16-head
// tile), then a reduce-scatter over the 4 lane groups leaves 64 consecutive
// scores in the 64 lanes for one coalesced store.
// Row scales of the FP8 format are applied to the float32 dot products
// (w*sigma_q folded per head, sigma_k after the head sum, both positive);
// MXFP4 block scales are operands of the scaled MFMA.
#include "csa_common.h"
#include "csa_internal.h"

namespace {

constexpr int kWaves = 4;
constexpr int kTilesPerWave = 16;                      // 4 waves x 16 tiles x 16 entries = 1024 entries / WG
constexpr int kEntriesPerWG = kWaves * kTilesPerWave * 16;

template <int FMT>
struct Fmt;
template <>
struct Fmt<CSA_BF16> {
  static constexpr int kRowBytes = 256;
  static constexpr int kLaneBytes = 64;
};
template <>
struct Fmt<CSA_FP8_E4M3_ROWSCALE> {
  static constexpr int kRowBytes = 128;
  static constexpr int kLaneBytes = 32;
};
template <>
struct Fmt<CSA_MXFP4_E8M0_B32> {
  static constexpr int kRowBytes = 64;
  static constexpr int kLaneBytes = 16;
};

// A lane's 64 / 32 / 16 bytes of a 128-dim row: lane group g = lane>>4 owns the
// contiguous quarter of the row.  The same dim -> (lane, slot) map is used for
// A and B, so every dot product covers all 128 dims exactly once.
template <int FMT>
struct Frag {
  i32x4 v[Fmt<FMT>::kLaneBytes / 16];
};

template <int FMT>
CSA_DEV Frag<FMT> load_frag(const uint8_t* row, int lane) {
  Frag<FMT> f;
  const i32x4* p = reinterpret_cast<const i32x4*>(row + (lane >> 4) * Fmt<FMT>::kLaneBytes);
#pragma unroll
  for (int j = 0; j < Fmt<FMT>::kLaneBytes / 16; ++j) f.v[j] = __builtin_nontemporal_load(p + j);
  return f;
}

template <int FMT>
CSA_DEV Frag<FMT> load_frag_cached(const uint8_t* row, int lane) {
  Frag<FMT> f;
  const i32x4* p = reinterpret_cast<const i32x4*>(row + (lane >> 4) * Fmt<FMT>::kLaneBytes);
#pragma unroll
  for (int j = 0; j < Fmt<FMT>::kLaneBytes / 16; ++j) f.v[j] = p[j];
  return f;
}

CSA_DEV bf16x8 as_bf16x8(i32x4 v) { return __builtin_bit_cast(bf16x8, v); }

template <int FMT>
CSA_DEV f32x4 mfma_tile(const Frag<FMT>& a, const Frag<FMT>& b, int sa, int sb) {
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  if constexpr (FMT == CSA_BF16) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a.v[ks]), as_bf16x8(b.v[ks]), acc, 0, 0, 0);
  } else if constexpr (FMT == CSA_FP8_E4M3_ROWSCALE) {
    i32x8 av = {a.v[0][0], a.v[0][1], a.v[0][2], a.v[0][3], a.v[1][0], a.v[1][1], a.v[1][2], a.v[1][3]};
    i32x8 bv = {b.v[0][0], b.v[0][1], b.v[0][2], b.v[0][3], b.v[1][0], b.v[1][1], b.v[1][2], b.v[1][3]};
    // format 0 = fp8 E4M3 for both operands; E8M0 scale 127 = 2^0 (row scales are applied outside)
    acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, acc, 0, 0, 0, 127, 0, 127);
  } else {
    i32x8 av = {a.v[0][0], a.v[0][1], a.v[0][2], a.v[0][3], 0, 0, 0, 0};
    i32x8 bv = {b.v[0][0], b.v[0][1], b.v[0][2], b.v[0][3], 0, 0, 0, 0};
    // format 4 = fp4 e2m1; per-lane E8M0 scale of the lane's 32-element block
    acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, acc, 4, 4, 0, sa, 0, sb);
  }
  return acc;
}

template <int FMT, int NT>
__global__ __launch_bounds__(kWaves * 64) void index_mfma_kernel(
    const uint8_t* __restrict__ q, const void* __restrict__ q_scale, const float* __restrict__ w,
    const uint8_t* __restrict__ kI, const void* __restrict__ k_scale, int T, int64_t n_max,
    const int64_t* __restrict__ pos0, int m, float* __restrict__ scores) {
  constexpr int HI = NT * 16;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int row = blockIdx.y;  // b * T + r
  const int b = row / T;
  const int r = row - b * T;
  const int64_t t = pos0[b] + r;
  const int64_t vis = visible_entries(t, m, n_max);
  const int64_t wg_first = (int64_t)blockIdx.x * kEntriesPerWG;
  float* srow = scores + (int64_t)row * n_max;

  // ---- A operand: this query row's HI heads, and the per-head epilogue weights
  Frag<FMT> qa[NT];
  int qsc[NT];
  float wq[NT][4];
#pragma unroll
  for (int g = 0; g < NT; ++g) {
    const int head = 16 * g + (lane & 15);
    qa[g] = load_frag_cached<FMT>(q + ((int64_t)row * HI + head) * Fmt<FMT>::kRowBytes, lane);
    if constexpr (FMT == CSA_MXFP4_E8M0_B32)
      qsc[g] = static_cast<const uint8_t*>(q_scale)[((int64_t)row * HI + head) * 4 + (lane >> 4)];
    else
      qsc[g] = 127;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h2 = 16 * g + 4 * (lane >> 4) + i;  // head of output row i in this lane
      float wv = w[(int64_t)row * HI + h2];
      if constexpr (FMT == CSA_FP8_E4M3_ROWSCALE) wv *= static_cast<const float*>(q_scale)[(int64_t)row * HI + h2];
      wq[g][i] = wv;
    }
  }

  const uint8_t* kb = kI + (int64_t)b * n_max * Fmt<FMT>::kRowBytes;
  // wave w streams the contiguous entries [wave_first, wave_first + 16 * kTilesPerWave) in groups of
  // 4 tiles (64 entries), double-buffered: the loads of group i+1 are in flight during group i
  const int64_t wave_first = wg_first + (int64_t)wave * kTilesPerWave * 16;
  const int gl = lane >> 4;
  constexpr int NG = kTilesPerWave / 4;
  Frag<FMT> kf[2][4];
  int ksc[2][4];
  float ksf[2][4];
  auto load_group = [&](int buf, int64_t e0) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t e = e0 + 16 * u + (lane & 15);
      const int64_t el = e < n_max ? e : n_max - 1;
      kf[buf][u] = load_frag<FMT>(kb + el * Fmt<FMT>::kRowBytes, lane);
      ksc[buf][u] = 127;
      ksf[buf][u] = 1.0f;
      if constexpr (FMT == CSA_MXFP4_E8M0_B32)
        ksc[buf][u] = static_cast<const uint8_t*>(k_scale)[((int64_t)b * n_max + el) * 4 + gl];
      if constexpr (FMT == CSA_FP8_E4M3_ROWSCALE)
        ksf[buf][u] = static_cast<const float*>(k_scale)[(int64_t)b * n_max + el];
    }
  };
  if (wave_first < vis) load_group(0, wave_first);
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) {
    const int buf = gi & 1;
    const int64_t e0 = wave_first + (int64_t)gi * 64;
    if (e0 >= n_max) break;
    if (gi + 1 < NG && e0 + 64 < vis) load_group(buf ^ 1, e0 + 64);
    const int64_t eo = e0 + lane;  // entry this lane writes
    if (e0 >= vis) {               // fully masked group
      if (eo < n_max) srow[eo] = -INFINITY;
      continue;
    }
    float p[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      float part = 0.0f;
#pragma unroll
      for (int g = 0; g < NT; ++g) {
        const f32x4 acc = mfma_tile<FMT>(qa[g], kf[buf][u], qsc[g], ksc[buf][u]);
#pragma unroll
        for (int i = 0; i < 4; ++i) part = fmaf(wq[g][i], fmaxf(acc[i], 0.0f), part);
      }
      p[u] = part * ksf[buf][u];  // the FP8 row scale is positive, so it factors out of every ReLU
    }
    // reduce-scatter over the 4 lane groups: lane 16u + e ends with the sum for tile u, entry e
    const bool hi2 = gl >= 2;
    const float s0 = hi2 ? p[0] : p[2], s1 = hi2 ? p[1] : p[3];
    const float k0 = (hi2 ? p[2] : p[0]) + __shfl_xor(s0, 32, 64);
    const float k1 = (hi2 ? p[3] : p[1]) + __shfl_xor(s1, 32, 64);
    const bool odd = gl & 1;
    const float val = (odd ? k1 : k0) + __shfl_xor(odd ? k0 : k1, 16, 64);
    if (eo < n_max) srow[eo] = (eo < vis) ? val : -INFINITY;
  }
}

// float32 path: one thread per (query row, entry), FMA over dims then heads.
constexpr int kF32Threads = 256;
__global__ __launch_bounds__(kF32Threads) void index_f32_kernel(const float* __restrict__ q,
                                                                const float* __restrict__ w,
                                                                const float* __restrict__ kI, int T, int HI, int cI,
                                                                int64_t n_max, const int64_t* __restrict__ pos0,
                                                                int m, float* __restrict__ scores) {
  extern __shared__ float s_q[];  // [HI][cI]
  const int row = blockIdx.y;
  const int b = row / T;
  const int r = row - b * T;
  const int64_t t = pos0[b] + r;
  const int64_t vis = visible_entries(t, m, n_max);
  for (int i = threadIdx.x; i < HI * cI; i += kF32Threads) s_q[i] = q[(int64_t)row * HI * cI + i];
  __syncthreads();
  const int64_t s = (int64_t)blockIdx.x * kF32Threads + threadIdx.x;
  if (s >= n_max) return;
  float* out = scores + (int64_t)row * n_max + s;
  if (s >= vis) {
    *out = -INFINITY;
    return;
  }
  const float* krow = kI + ((int64_t)b * n_max + s) * cI;
  float tot = 0.0f;
  for (int h = 0; h < HI; ++h) {
    float d = 0.0f;
    for (int j = 0; j < cI; j += 4) {
      f32x4 kv = *reinterpret_cast<const f32x4*>(krow + j);
      d = fmaf(s_q[h * cI + j + 0], kv[0], d);
      d = fmaf(s_q[h * cI + j + 1], kv[1], d);
      d = fmaf(s_q[h * cI + j + 2], kv[2], d);
      d = fmaf(s_q[h * cI + j + 3], kv[3], d);
    }
    tot = fmaf(w[(int64_t)row * HI + h], fmaxf(d, 0.0f), tot);
  }
  *out = tot;
}

template <int FMT>
csa_status launch_fmt(const void* q, const void* q_scale, const float* w, const void* k, const void* k_scale, int B,
                      int T, int HI, int64_t n_max, const int64_t* pos0, int m, float* scores, hipStream_t stream) {
  dim3 grid(ceil_div(n_max, kEntriesPerWG), B * T);
  dim3 block(kWaves * 64);
#define CSA_IDX_LAUNCH(NT)                                                                                  \
  hipLaunchKernelGGL((index_mfma_kernel<FMT, NT>), grid, block, 0, stream, (const uint8_t*)q, q_scale, w, \
                     (const uint8_t*)k, k_scale, T, n_max, pos0, m, scores)
  switch (HI) {
    case 16: CSA_IDX_LAUNCH(1); break;
    case 32: CSA_IDX_LAUNCH(2); break;
    case 64: CSA_IDX_LAUNCH(4); break;
    case 128: CSA_IDX_LAUNCH(8); break;
    default: return CSA_ERR_UNSUPPORTED;
  }
#undef CSA_IDX_LAUNCH
  return hipGetLastError() == hipSuccess ? CSA_OK : CSA_ERR_LAUNCH;
}

}  // namespace

csa_status launch_index(const void* q, const void* q_scale, const float* w, const void* k, const void* k_scale,
                        int B, int T, int HI, int cI, int64_t n_max, const int64_t* pos0, int m, int qk_t,
                        float* scores, hipStream_t stream) {
  switch (qk_t) {
    case CSA_F32: {
      dim3 grid(ceil_div(n_max, kF32Threads), B * T);
      size_t lds = (size_t)HI * cI * sizeof(float);
      hipLaunchKernelGGL(index_f32_kernel, grid, dim3(kF32Threads), lds, stream, (const float*)q, w,
                         (const float*)k, T, HI, cI, n_max, pos0, m, scores);
      return hipGetLastError() == hipSuccess ? CSA_OK : CSA_ERR_LAUNCH;
    }
    case CSA_BF16:
      return launch_fmt<CSA_BF16>(q, q_scale, w, k, k_scale, B, T, HI, n_max, pos0, m, scores, stream);
    case CSA_FP8_E4M3_ROWSCALE:
      return launch_fmt<CSA_FP8_E4M3_ROWSCALE>(q, q_scale, w, k, k_scale, B, T, HI, n_max, pos0, m, scores, stream);
    case CSA_MXFP4_E8M0_B32:
      return launch_fmt<CSA_MXFP4_E8M0_B32>(q, q_scale, w, k, k_scale, B, T, HI, n_max, pos0, m, scores, stream);
    default:
      return CSA_ERR_UNSUPPORTED;
  }
}
