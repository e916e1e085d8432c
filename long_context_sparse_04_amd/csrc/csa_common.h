// Internal helpers shared by the gfx950 kernels of the CSA / HCA step.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/csa.h"

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

#define CSA_DEV __device__ __forceinline__

// ---------------------------------------------------------------- number formats
CSA_DEV float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// float32 -> bfloat16, round to nearest even (NaN stays NaN).
CSA_DEV uint16_t f32_to_bf16(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Two float32 -> packed bf16 pair (low half = lo), hardware round to nearest even.
CSA_DEV uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}
// acc + x.lo^2 + x.hi^2 for a packed bf16 pair (products are exact in float32).
CSA_DEV float sumsq_bf16x2(uint32_t w, float acc) {
  const bf16x2 x = __builtin_bit_cast(bf16x2, w);
  return __builtin_amdgcn_fdot2_f32_bf16(x, x, acc, false);
}

// float32 -> OCP fp8 E4M3, round to nearest even, saturating at +-448 (NaN -> 0x7F).
CSA_DEV uint32_t f32_to_e4m3(float x) {
  uint32_t u = __float_as_uint(x);
  uint32_t sign = (u >> 24) & 0x80u;
  float a = fabsf(x);
  if (a != a) return 0x7Fu;
  if (!(a < 448.0f)) return sign | 0x7Eu;
  uint32_t code;
  if (a < 0x1p-6f) {
    code = (uint32_t)rintf(a * 512.0f);  // multiples of 2^-9; 8 becomes the smallest normal
  } else {
    uint32_t au = __float_as_uint(a);
    int e = (int)(au >> 23) - 127;
    uint32_t mant = au & 0x7FFFFFu;
    uint32_t keep = mant >> 20, rest = mant & 0xFFFFFu;
    if (rest > 0x80000u || (rest == 0x80000u && (keep & 1u))) keep++;
    if (keep == 8u) { keep = 0u; e++; }
    code = ((uint32_t)(e + 7) << 3) | keep;
    if (code > 0x7Eu) code = 0x7Eu;
  }
  return code ? (sign | code) : 0u;
}

// |v| (already divided by the block scale) -> e2m1 code, ties to even, saturating at 6.
CSA_DEV uint32_t f32_to_e2m1(float v) {
  float a = fabsf(v);
  uint32_t code = (a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) + (a > 2.5f) + (a >= 3.5f) + (a > 5.0f);
  return (code && v < 0.0f) ? (code | 8u) : code;
}

// Order-preserving key of a float32 score (+0 and -0 map to the same key).
CSA_DEV uint32_t score_key(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u << 1) == 0u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
CSA_DEV float key_to_score(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return __uint_as_float(u);
}

// ---------------------------------------------------------------- cross-lane helpers
// The two largest of the union of two disjoint pairs (t1 >= t2, b1 >= b2), kept in (t1, t2).
CSA_DEV void top2_merge(uint32_t& t1, uint32_t& t2, uint32_t b1, uint32_t b2) {
  const uint32_t lo = min(t1, b1);
  t1 = max(t1, b1);
  t2 = max(lo, max(t2, b2));
}
template <int CTRL>
CSA_DEV uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, true);
}
// Every lane ends with the two largest keys of its 16-lane row's disjoint lane pairs: quad exchanges
// and row rotations by 4 and 8.
CSA_DEV void row16_top2(uint32_t& t1, uint32_t& t2) {
  top2_merge(t1, t2, dpp_u32<0xB1>(t1), dpp_u32<0xB1>(t2));    // quad_perm [1,0,3,2]
  top2_merge(t1, t2, dpp_u32<0x4E>(t1), dpp_u32<0x4E>(t2));    // quad_perm [2,3,0,1]
  top2_merge(t1, t2, dpp_u32<0x124>(t1), dpp_u32<0x124>(t2));  // row_ror:4
  top2_merge(t1, t2, dpp_u32<0x128>(t1), dpp_u32<0x128>(t2));  // row_ror:8
}
// Every lane ends with the two largest keys of its 8-lane half row's disjoint lane pairs: quad exchanges,
// then the half-row mirror (lane i of a half row with lane 7 - i, i.e. quad 0 with quad 1).
CSA_DEV void half_row_top2(uint32_t& t1, uint32_t& t2) {
  top2_merge(t1, t2, dpp_u32<0xB1>(t1), dpp_u32<0xB1>(t2));    // quad_perm [1,0,3,2]
  top2_merge(t1, t2, dpp_u32<0x4E>(t1), dpp_u32<0x4E>(t2));    // quad_perm [2,3,0,1]
  top2_merge(t1, t2, dpp_u32<0x141>(t1), dpp_u32<0x141>(t2));  // row_half_mirror
}
// Every lane ends with the two largest keys of its 32-lane half wave's disjoint lane pairs: the rows'
// results, then the row-pair swap.
CSA_DEV void half_wave_top2(uint32_t& t1, uint32_t& t2) {
  row16_top2(t1, t2);
  const auto a = __builtin_amdgcn_permlane16_swap(t1, t1, false, false);
  const auto c = __builtin_amdgcn_permlane16_swap(t2, t2, false, false);
  t1 = a[0]; t2 = c[0];
  top2_merge(t1, t2, a[1], c[1]);
}
// Every lane ends with the two largest keys of the wave's 64 disjoint lane pairs: the rows' results,
// then the gfx950 row-pair and half-wave swaps.
CSA_DEV void wave_top2(uint32_t& t1, uint32_t& t2) {
  row16_top2(t1, t2);
  {
    const auto a = __builtin_amdgcn_permlane16_swap(t1, t1, false, false);
    const auto c = __builtin_amdgcn_permlane16_swap(t2, t2, false, false);
    t1 = a[0]; t2 = c[0];
    top2_merge(t1, t2, a[1], c[1]);
  }
  {
    const auto a = __builtin_amdgcn_permlane32_swap(t1, t1, false, false);
    const auto c = __builtin_amdgcn_permlane32_swap(t2, t2, false, false);
    t1 = a[0]; t2 = c[0];
    top2_merge(t1, t2, a[1], c[1]);
  }
}

// DPP row operations act inside 16-lane rows.
template <int CTRL>
CSA_DEV float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}
// max / sum over the 16 lanes of a row; every lane of the row receives the result
CSA_DEV float row16_max(float v) {
  v = fmaxf(v, dpp_f32<0xB1>(v));   // quad_perm [1,0,3,2]
  v = fmaxf(v, dpp_f32<0x4E>(v));   // quad_perm [2,3,0,1]
  v = fmaxf(v, dpp_f32<0x124>(v));  // row_ror:4
  v = fmaxf(v, dpp_f32<0x128>(v));  // row_ror:8
  return v;
}
CSA_DEV float row16_sum(float v) {
  v += dpp_f32<0xB1>(v);
  v += dpp_f32<0x4E>(v);
  v += dpp_f32<0x124>(v);
  v += dpp_f32<0x128>(v);
  return v;
}
CSA_DEV float shfl_xor_f32(float v, int mask) { return __shfl_xor(v, mask, 64); }
CSA_DEV float wave_sum(float v) {
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// ---------------------------------------------------------------- RoPE
// theta_i = rope_base^(-2i/R) for the R/2 pairs, computed once on the host in double.
struct RopeTable {
  double theta[64];
};

// cos / sin of pos * theta.  The angle is formed and reduced to [-pi/4, pi/4] plus a
// quadrant in double precision (Cody-Waite style, pi/2 split into two doubles), so
// positions near 2^20 keep float32-level accuracy; sin and cos of the reduced
// argument are their Taylor series through x^9 / x^10 (truncation < 2e-9 on
// [-pi/4, pi/4]), evaluated in float32 by Horner's rule.  |pos * theta| < 2^31 * pi/2
// (positions below 2^31 with theta <= 1).
CSA_DEV void rope_cs(double pos, double theta, float& c, float& s) {
  const double pio2_hi = 1.5707963267948966;     // nearest double to pi/2
  const double pio2_lo = 6.123233995736766e-17;  // pi/2 - pio2_hi
  const double ang = pos * theta;
  const double kq = rint(ang * 0.6366197723675814);  // 2/pi
  double red = fma(-kq, pio2_hi, ang);
  red = fma(-kq, pio2_lo, red);
  const float x = (float)red, x2 = x * x;
  const float sp = fmaf(x * x2, fmaf(x2, fmaf(x2, fmaf(x2, 1.0f / 362880.0f, -1.0f / 5040.0f), 1.0f / 120.0f),
                                     -1.0f / 6.0f), x);
  const float cp = fmaf(x2, fmaf(x2, fmaf(x2, fmaf(x2, fmaf(x2, -1.0f / 3628800.0f, 1.0f / 40320.0f),
                                                   -1.0f / 720.0f), 1.0f / 24.0f), -0.5f), 1.0f);
  // angle = red + q * pi/2: odd quadrants swap sin and cos; the signs follow the quadrant
  const int q = (int)kq & 3;
  const float s1 = (q & 1) ? cp : sp, c1 = (q & 1) ? sp : cp;
  s = (q & 2) ? -s1 : s1;
  c = ((q + 1) & 2) ? -c1 : c1;
}

// RMSNorm (gain gamma, epsilon eps) and then RoPE at position pos of one c-dim row held 4 channels
// per thread: thread t < c/4 (the holder) owns channels [4t, 4t + 4) in y.  Every thread of the
// NT-thread block calls it (it holds two barriers); s_red has room for NT/64 floats.
template <int NT>
CSA_DEV void prep_row4(float* y, bool holder, int cg, int c, double pos, const float* gamma, float eps, int R,
                       const double* theta, float* s_red) {
  float ss = holder ? fmaf(y[0], y[0], fmaf(y[1], y[1], fmaf(y[2], y[2], y[3] * y[3]))) : 0.0f;
  for (int o = 32; o >= 1; o >>= 1) ss += __shfl_xor(ss, o, 64);
  if ((threadIdx.x & 63) == 0) s_red[threadIdx.x >> 6] = ss;
  __syncthreads();
  float tot = 0.0f;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) tot += s_red[w];
  __syncthreads();  // s_red is free again for the caller
  if (!holder) return;
  const float rn = 1.0f / sqrtf(tot / (float)c + eps);
  const int d = 4 * cg;
#pragma unroll
  for (int q = 0; q < 4; ++q) y[q] = gamma ? y[q] * rn * gamma[d + q] : y[q] * rn;
  const int rope_lo = c - R;
  if (d >= rope_lo) {
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      float cs, sn;
      rope_cs(pos, theta[(d + 2 * p - rope_lo) / 2], cs, sn);
      const float x0 = y[2 * p], x1 = y[2 * p + 1];
      y[2 * p] = x0 * cs - x1 * sn;
      y[2 * p + 1] = x0 * sn + x1 * cs;
    }
  }
}

// Store a prepared row held 4 channels per thread (thread t < c/4 owns channels [4t, 4t + 4)) in
// CSA_FP8_BF16_ROPE: channels below c - R as OCP e4m3 codes at byte offset d with one float32 scale
// (amax/448 of those channels, codes RNE, saturating), channels from c - R on as bf16 at byte offset
// (c - R) + 2 (d - (c - R)).  Every thread of the NT-thread block calls it (it holds a barrier); s_red
// has room for NT/64 floats.  c - R is a multiple of 16, so a thread's 4 channels lie in one part.
template <int NT>
CSA_DEV void store_fp8_rope_row(const float* y, bool holder, int cg, int c, int R, uint8_t* row, float* scale_out,
                                float* s_red) {
  const int nfp = c - R;
  const int d = 4 * cg;
  const bool fp = holder && d < nfp;
  float am = fp ? fmaxf(fmaxf(fabsf(y[0]), fabsf(y[1])), fmaxf(fabsf(y[2]), fabsf(y[3]))) : 0.0f;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) am = fmaxf(am, __shfl_xor(am, o, 64));
  if ((threadIdx.x & 63) == 0) s_red[threadIdx.x >> 6] = am;
  __syncthreads();
  am = s_red[0];
#pragma unroll
  for (int w = 1; w < NT / 64; ++w) am = fmaxf(am, s_red[w]);
  const float scale = am / 448.0f;
  if (fp) {
    uint32_t pk = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) pk |= f32_to_e4m3(scale > 0.0f ? y[q] / scale : 0.0f) << (8 * q);
    *reinterpret_cast<uint32_t*>(row + d) = pk;
  } else if (holder) {
    uint2 pk;
    pk.x = pack_bf16x2(y[0], y[1]);
    pk.y = pack_bf16x2(y[2], y[3]);
    *reinterpret_cast<uint2*>(row + nfp + 2 * (d - nfp)) = pk;
  }
  if (threadIdx.x == 0) *scale_out = scale;
}

// theta_i = rope_base^(-2i/R), i < R/2 <= 64, in double on the host
static inline RopeTable make_rope_table(int R, float base) {
  RopeTable rt;
  for (int i = 0; i < 64; ++i) rt.theta[i] = (2 * i < R) ? pow((double)base, -(double)(2 * i) / (double)R) : 0.0;
  return rt;
}

// ---------------------------------------------------------------- misc
CSA_DEV int64_t visible_entries(int64_t t, int m, int64_t n_max) {
  int64_t v = t >= 0 ? t / m : 0;
  return v < n_max ? v : n_max;
}

static inline int ceil_div(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }
