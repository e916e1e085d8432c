// Dense projections on either side of the attention step: decode rows (at most 32 per call, a weight
// stream) and prefill rows (more than 32, an LDS-tiled MFMA product).
//
// "【论文解读】DeepSeek-V4" (wkq9411.github.io), section 一(三)1(2)-(3): q = c^Q W^UQ and q^I = c^Q W^IUQ from
// one shared latent c^Q; section 一(三)1(4): the grouped output projection (g groups of n_h / g heads, each
// projected to d_g, then the g d_g intermediates projected to d).
//
// Design: with a handful of rows the product is a stream over the weights (every weight byte is read
// once, the rows stay in L2), so the kernel is HBM-bound and runs bf16 MFMA only because it is free:
// C[z][m][n] = sum_k A[z][m][k] W[z][n][k].  The weights are stored packed in MFMA tiles (csa_pack_proj_weights):
// the 16-output x 32-k tile (n / 16, k / 32) is 1 KB contiguous, lane-ordered, so that lane l's 16-byte
// load -- row / column l % 16, k-group l / 16 of a 16x16x32 MFMA -- is bytes [16 l, 16 l + 16) of it: every
// load instruction reads 1 KB of contiguous memory (an output-major row layout would give 16 half-used
// 128-byte lines per instruction, which streams far below the HBM rate).  A workgroup's 4 waves either take
// different column tiles over the whole K (the fused query launch: 128 columns, one indexer head, per
// workgroup) or share 16 columns and split K four ways, summed in LDS in a fixed order (the output
// projection: enough workgroups to keep every CU streaming).
//
// With many rows (chunked prefill) every weight tile serves many rows and the product is MFMA-bound: the
// tiled kernel below stages 256-row x 128-column x 32-k tiles of both operands in LDS (global-to-LDS loads
// into a three-stage ring, each 16-row or 16-column operand tile 1 KB in MFMA lane order, so every LDS
// read is one contiguous, conflict-free 1 KB) and gives each wave a 128 x 64 block of the output.
#include "csa_common.h"
#include "csa_internal.h"

namespace {

constexpr int kProjThreads = 256;
constexpr int kProjDecodeRows = 32;  // up to this many rows: the weight-streaming kernel
constexpr int kUnroll = 4;  // k-steps whose loads are in flight together

enum ProjEpi { kEpiBf16 = 0, kEpiFp8Head = 1, kEpiMxfp4 = 2 };

// One column segment of a launch: its weights, output and epilogue.  A launch has one or two segments
// (the fused query launch: W^UQ -> q, W^IUQ -> q^I) over the same rows and K.
struct ProjSeg {
  const uint16_t* w;   // [Z][N][K] bf16
  int64_t w_zstride;   // elements per batch
  int n;               // columns per batch
  void* c;             // output rows (row stride ldc elements; bytes for the quantized forms)
  int64_t ldc;
  int64_t c_zoff;      // column offset of batch z in the output row
  void* scale;         // fp8: float [rows][n / 128]; MXFP4: bytes [rows][n / 32]
  int epi;
  int blocks;          // workgroups of this segment along x
};
struct ProjArgs {
  const uint16_t* a;   // [rows][lda] bf16, batch z's K values start at column z * a_zoff
  int64_t lda, a_zoff;
  int rows, k;
  ProjSeg seg[2];
};

// MT: 16-row tiles of A (rows <= 16 * MT); TPW: column tiles per wave; KS: waves sharing a column group
// The body of one segment's workgroup (sg: its segment, bx: the workgroup's index in it).  s_red:
// (KS - 1) * 64 * MT * TPW f32x4 of LDS; s_amax: [4][32] floats.
template <int MT, int TPW, int KS>
__device__ __forceinline__ void proj_body(const ProjArgs& p, const ProjSeg& sg, int bx, f32x4* s_red,
                                          float (*s_amax)[32]) {
  constexpr int kGroups = 4 / KS;               // column groups per workgroup
  constexpr int kCols = 16 * TPW * kGroups;     // columns per workgroup

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int z = blockIdx.y;
  const int grp = wave / KS, ks = wave % KS;
  const int n0 = bx * kCols + grp * 16 * TPW;   // first column of this wave's tiles
  const int kg = lane >> 4, li = lane & 15;
  const int nsteps = p.k / 32;

  const uint16_t* wz = sg.w + (int64_t)z * sg.w_zstride;
  const uint16_t* az = p.a + (int64_t)z * p.a_zoff;
  // packed tiles: tile (n / 16, s) at ((n / 16) * nsteps + s) * 512 elements; this lane's 8 at 8 * lane
  const uint16_t* wrow[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t) wrow[t] = wz + (int64_t)((n0 / 16 + t) * (int64_t)nsteps) * 512 + 8 * lane;
  const uint16_t* arow[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) arow[mt] = az + (int64_t)min(16 * mt + li, p.rows - 1) * p.lda + 8 * kg;

  f32x4 acc[MT][TPW];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int t = 0; t < TPW; ++t) acc[mt][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // two register batches of kUnroll k-steps: the next batch's loads go out before this batch's MFMAs, so
  // 2 * kUnroll k-steps of weights are in flight per wave
  bf16x8 wA[kUnroll][TPW], aA[kUnroll][MT], wB[kUnroll][TPW], aB[kUnroll][MT];
  auto load_batch = [&](int s0, bf16x8 (&wf)[kUnroll][TPW], bf16x8 (&af)[kUnroll][MT]) {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int s = s0 + u * KS;
      if (s < nsteps) {  // (uniform)
#pragma unroll
        for (int t = 0; t < TPW; ++t)
          wf[u][t] = __builtin_bit_cast(bf16x8, __builtin_nontemporal_load(
                                                    reinterpret_cast<const u32x4*>(wrow[t] + 512 * (int64_t)s)));
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          af[u][mt] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(arow[mt] + 32 * s));
      }
    }
  };
  auto mfma_batch = [&](int s0, const bf16x8 (&wf)[kUnroll][TPW], const bf16x8 (&af)[kUnroll][MT]) {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      if (s0 + u * KS < nsteps) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int t = 0; t < TPW; ++t)
            acc[mt][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[u][mt], wf[u][t], acc[mt][t], 0, 0, 0);
      }
    }
  };
  constexpr int kBatch = KS * kUnroll;  // k-steps between a wave's batches
  if (ks < nsteps) {
    load_batch(ks, wA, aA);
    for (int s0 = ks;; s0 += 2 * kBatch) {
      const int s1 = s0 + kBatch;
      if (s1 < nsteps) load_batch(s1, wB, aB);
      mfma_batch(s0, wA, aA);
      if (s1 >= nsteps) break;
      if (s1 + kBatch < nsteps) load_batch(s1 + kBatch, wA, aA);
      mfma_batch(s1, wB, aB);
      if (s1 + kBatch >= nsteps) break;
    }
  }

  if constexpr (KS > 1) {  // the K-split partial sums, added in wave order
    if (ks > 0) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int t = 0; t < TPW; ++t) s_red[(((ks - 1) * MT + mt) * TPW + t) * 64 + lane] = acc[mt][t];
    }
    __syncthreads();
    if (ks > 0) return;
#pragma unroll
    for (int q = 1; q < KS; ++q)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
          const f32x4 o = s_red[(((q - 1) * MT + mt) * TPW + t) * 64 + lane];
#pragma unroll
          for (int v = 0; v < 4; ++v) acc[mt][t][v] += o[v];
        }
  }

  // lane l holds column n0 + 16 t + l % 16 of rows 16 mt + 4 (l / 16) + v
  const int64_t coff = (int64_t)z * sg.c_zoff;
  if (sg.epi == kEpiBf16) {
    uint16_t* c = static_cast<uint16_t*>(sg.c);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int m = 16 * mt + 4 * kg + v;
        if (m < p.rows) {
#pragma unroll
          for (int t = 0; t < TPW; ++t)
            c[(int64_t)m * sg.ldc + coff + n0 + 16 * t + li] =
                (uint16_t)(pack_bf16x2(acc[mt][t][v], 0.0f) & 0xFFFFu);
        }
      }
    return;
  }
  if (sg.epi == kEpiFp8Head) {  // one head = this workgroup's 128 columns (KS == 1): amax per row
    uint8_t* c = static_cast<uint8_t*>(sg.c);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        float am = 0.0f;
#pragma unroll
        for (int t = 0; t < TPW; ++t) am = fmaxf(am, fabsf(acc[mt][t][v]));
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) am = fmaxf(am, __shfl_xor(am, o, 64));
        if (li == 0) s_amax[wave][16 * mt + 4 * kg + v] = am;
      }
    }
    __syncthreads();
    const int head = (bx * kCols) / 128;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int r = 16 * mt + 4 * kg + v;
        const float am = fmaxf(fmaxf(s_amax[0][r], s_amax[1][r]), fmaxf(s_amax[2][r], s_amax[3][r]));
        const float scale = am / 448.0f;
        if (r < p.rows) {
#pragma unroll
          for (int t = 0; t < TPW; ++t)
            c[(int64_t)r * sg.ldc + n0 + 16 * t + li] =
                (uint8_t)f32_to_e4m3(scale > 0.0f ? acc[mt][t][v] / scale : 0.0f);
          if (wave == 0 && li == 0) static_cast<float*>(sg.scale)[(int64_t)r * (sg.n / 128) + head] = scale;
        }
      }
    return;
  }
  // MXFP4: a wave's 32 columns (TPW == 2) are one block: E8M0 scale floor(log2 amax) - 2, e2m1 codes,
  // element 2i in the low nibble
  uint8_t* c = static_cast<uint8_t*>(sg.c);
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int r = 16 * mt + 4 * kg + v;
      float am = fmaxf(fabsf(acc[mt][0][v]), fabsf(acc[mt][TPW - 1][v]));
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) am = fmaxf(am, __shfl_xor(am, o, 64));
      int X = -127;
      if (am > 0.0f) {
        int ex;
        frexpf(am, &ex);  // am = f * 2^ex, f in [0.5, 1)
        X = ex - 1 - 2;
        X = X < -127 ? -127 : (X > 127 ? 127 : X);
      }
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
        const uint32_t code = f32_to_e2m1(ldexpf(acc[mt][t][v], -X));
        const uint32_t up = __shfl_xor(code, 1, 64);  // the odd column's code, to the even lane
        if (r < p.rows && (li & 1) == 0)
          c[(int64_t)r * sg.ldc + (n0 + 16 * t + li) / 2] = (uint8_t)(code | (up << 4));
      }
      if (r < p.rows && li == 0) static_cast<uint8_t*>(sg.scale)[(int64_t)r * (sg.n / 32) + n0 / 32] = (uint8_t)(X + 127);
    }
}

// [Z][N][K] output-major -> packed MFMA tiles: one thread per 16-byte chunk of the packed array
__global__ __launch_bounds__(256) void proj_pack_kernel(const uint16_t* __restrict__ w, uint16_t* __restrict__ out,
                                                        int64_t chunks, int n, int k) {
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= chunks) return;
  const int nsteps = k / 32;
  const int64_t per_z = (int64_t)n * k / 8;          // chunks per batch
  const int64_t z = c / per_z;
  const int64_t rem = c - z * per_z;
  const int64_t tile = rem / 64;                     // (n / 16) * nsteps + s
  const int lane = (int)(rem % 64);
  const int64_t nt = tile / nsteps, s = tile % nsteps;
  const int64_t row = nt * 16 + (lane & 15);
  const int64_t kk = s * 32 + 8 * (lane >> 4);
  *reinterpret_cast<u32x4*>(out + 8 * c) =
      *reinterpret_cast<const u32x4*>(w + (z * n + row) * (int64_t)k + kk);
}

// Segment 0 runs the (TPW0, KS0) mapping, segment 1 the (TPW1, KS1) one: the fused query launch streams W^UQ
// four waves to 16 columns (many workgroups) and W^IUQ one head of 128 columns per workgroup (its quantizing
// epilogue needs the head in one workgroup).
template <int MT, int TPW0, int KS0, int TPW1, int KS1>
__global__ __launch_bounds__(kProjThreads) void proj_kernel(ProjArgs p) {
  constexpr int kRed0 = KS0 > 1 ? (KS0 - 1) * 64 * MT * TPW0 : 1;
  constexpr int kRed1 = KS1 > 1 ? (KS1 - 1) * 64 * MT * TPW1 : 1;
  __shared__ f32x4 s_red[kRed0 > kRed1 ? kRed0 : kRed1];
  __shared__ float s_amax[4][32];  // fp8 epilogue: per wave, per row
  if ((int)blockIdx.x < p.seg[0].blocks)  // (uniform)
    proj_body<MT, TPW0, KS0>(p, p.seg[0], (int)blockIdx.x, s_red, s_amax);
  else
    proj_body<MT, TPW1, KS1>(p, p.seg[1], (int)blockIdx.x - p.seg[0].blocks, s_red, s_amax);
}

// ---- Prefill rows: the LDS-tiled product ----
// Workgroup tile kTM rows x kTN columns (8 waves), k-steps of 32; wave w = 4 wm + wn owns rows 128 wm .. +128
// and columns 64 wn .. +64 of it (8 x 4 MFMA tiles of 16 x 16, 128 accumulator registers).  A stage holds
// the 16 A tiles (16 rows x 32 k each: lane l's 16 bytes are row l % 16, k-group l / 16) and the 16 packed
// weight tiles (16 columns x 32 k in the same lane order, as they lie in memory), 1 KB each; a ring of
// kTStages stages keeps kTStages - 1 of them in flight, which is what covers the fetch latency (the product
// is MFMA-bound only while the next stages keep arriving).  The MFMA takes the weight tile as its first
// operand, so that lane l's four results are columns 4 (l / 16) .. +4 of row l % 16 (one 8-byte store).
constexpr int kTM = 256, kTN = 256;
constexpr int kTThreads = 512;
constexpr int kTStages = 5;
constexpr int kTStageBytes = (kTM + kTN) / 16 * 1024;            // 32 KB
constexpr int kTDmaPerWave = kTStageBytes / 1024 / (kTThreads / 64);  // 4 1-KB loads per wave and stage
constexpr size_t kTLdsBytes = (size_t)kTStages * kTStageBytes;   // 160 KB
constexpr int kTGroupRows = 4;   // row tiles per group of the tile order

// the segment, batch and tile of workgroup t
struct TiledMap {
  int ntm;            // row tiles
  int ntn[2];         // column tiles per batch of each segment
  int64_t tiles0;     // tiles of segment 0
  int64_t tiles;      // all tiles
  int64_t per_xcd;    // tiles per XCD (the last XCDs may get fewer)
};

// The wave's 8 A and 4 B operand reads of one k-step in one block that waits for them once (plain loads
// with the next k-step's reads issued during the second half of this one's MFMAs measured the same).
CSA_DEV void lds_read_ab(u32x4 (&a)[8], u32x4 (&b)[4], uint32_t aaddr, uint32_t baddr) {
  asm volatile(
      "ds_read_b128 %0, %12 offset:0\n\tds_read_b128 %1, %12 offset:1024\n\t"
      "ds_read_b128 %2, %12 offset:2048\n\tds_read_b128 %3, %12 offset:3072\n\t"
      "ds_read_b128 %4, %12 offset:4096\n\tds_read_b128 %5, %12 offset:5120\n\t"
      "ds_read_b128 %6, %12 offset:6144\n\tds_read_b128 %7, %12 offset:7168\n\t"
      "ds_read_b128 %8, %13 offset:0\n\tds_read_b128 %9, %13 offset:1024\n\t"
      "ds_read_b128 %10, %13 offset:2048\n\tds_read_b128 %11, %13 offset:3072\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(a[0]), "=&v"(a[1]), "=&v"(a[2]), "=&v"(a[3]), "=&v"(a[4]), "=&v"(a[5]), "=&v"(a[6]), "=&v"(a[7]),
        "=&v"(b[0]), "=&v"(b[1]), "=&v"(b[2]), "=&v"(b[3])
      : "v"(aaddr), "v"(baddr)
      : "memory");
}

CSA_DEV uint32_t lds_byte_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

__global__ __launch_bounds__(kTThreads, 1) void proj_tiled_kernel(ProjArgs p, TiledMap mp) {
  extern __shared__ __align__(1024) uint8_t s_ring[];   // kTStages x [16 A tiles | 16 B tiles] of 1 KB

  // workgroup i runs on XCD i % 8: XCD x takes the contiguous tiles [x per_xcd, (x + 1) per_xcd); within a
  // segment and batch the tiles go in groups of kTGroupRows row tiles, row tile fastest, so that the
  // workgroups an XCD runs together share a few row tiles and a few weight tiles in its L2
  const int64_t t = (int64_t)(blockIdx.x % 8) * mp.per_xcd + blockIdx.x / 8;
  if (t >= mp.tiles) return;
  const int si = t < mp.tiles0 ? 0 : 1;
  const ProjSeg& sg = p.seg[si];
  const int64_t tt = si ? t - mp.tiles0 : t;
  const int ntn = mp.ntn[si];
  const int64_t per_z = (int64_t)ntn * mp.ntm;
  const int z = (int)(tt / per_z);
  const int64_t L = tt % per_z;
  const int64_t gsz = (int64_t)kTGroupRows * ntn;
  const int mfirst = (int)(L / gsz) * kTGroupRows;
  const int gm = min(kTGroupRows, mp.ntm - mfirst);
  const int rem = (int)(L % gsz);
  const int m0 = (mfirst + rem % gm) * kTM, n0 = (rem / gm) * kTN;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave >> 2, wn = wave & 3;
  const int li = lane & 15, kg = lane >> 4;
  const int nsteps = p.k / 32;
  const int nct = sg.n / 16;   // 16-column tiles of the segment

  // this wave's loads of a stage: 1-KB tiles 4 wave .. +4, A tiles 0..15 (waves 0-3), B tiles 16..31
  const bool is_a = wave < 4;
  const uint16_t* src[kTDmaPerWave];
#pragma unroll
  for (int j = 0; j < kTDmaPerWave; ++j) {
    const int q = kTDmaPerWave * wave + j;
    if (is_a) {
      const int row = min(m0 + 16 * q + li, p.rows - 1);
      src[j] = p.a + (int64_t)z * p.a_zoff + (int64_t)row * p.lda + 8 * kg;
    } else {
      const int ct = min(n0 / 16 + (q - 16), nct - 1);
      src[j] = sg.w + (int64_t)z * sg.w_zstride + (int64_t)ct * nsteps * 512 + 8 * lane;
    }
  }
  const int step_elems = is_a ? 32 : 512;   // elements between k-steps
  auto issue = [&](int s) {
    uint8_t* stage = s_ring + (s % kTStages) * kTStageBytes + kTDmaPerWave * wave * 1024;
#pragma unroll
    for (int j = 0; j < kTDmaPerWave; ++j)
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(src[j] + (int64_t)s * step_elems),
                                       (__attribute__((address_space(3))) void*)(stage + j * 1024), 16, 0, 0);
  };

  f32x4 acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const uint32_t ring = lds_byte_addr(s_ring);
  const uint32_t aoff = (uint32_t)(8 * wm) * 1024 + 16 * lane;
  const uint32_t boff = 16 * 1024 + (uint32_t)(4 * wn) * 1024 + 16 * lane;
#pragma unroll
  for (int s = 0; s < kTStages - 1; ++s)
    if (s < nsteps) issue(s);
  for (int s = 0; s < nsteps; ++s) {
    // stage s has landed once at most the later stages' loads are outstanding (vector memory operations
    // complete in issue order): kTStages - 2 stages after it, fewer near the end
    const int later = min(kTStages - 2, nsteps - 1 - s);
    if (later >= 3)
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(3 * kTDmaPerWave) : "memory");
    else if (later == 2)
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * kTDmaPerWave) : "memory");
    else if (later == 1)
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kTDmaPerWave) : "memory");
    else
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    // every wave's part of stage s is in; every wave is done with stage s - 1 (a bare barrier: the fence
    // of __syncthreads would wait for the later stages' loads too)
    __builtin_amdgcn_s_barrier();
    if (s + kTStages - 1 < nsteps) issue(s + kTStages - 1);   // into stage s - 1's buffer
    const uint32_t sb = ring + (uint32_t)((s % kTStages) * kTStageBytes);
    u32x4 fa[8], fb[4];
    lds_read_ab(fa, fb, sb + aoff, sb + boff);
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, fb[j]),
                                                            __builtin_bit_cast(bf16x8, fa[i]), acc[i][j], 0, 0, 0);
  }

  // lane l holds columns n0 + 64 wn + 16 j + 4 (l / 16) + v, v = 0..3, of row m0 + 128 wm + 16 i + l % 16
  const int64_t coff = (int64_t)z * sg.c_zoff;
  const int rbase = m0 + 128 * wm + li;
  const int cbase = n0 + 64 * wn + 4 * kg;
  if (sg.epi == kEpiBf16) {
    uint16_t* c = static_cast<uint16_t*>(sg.c);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = rbase + 16 * i;
      if (r < p.rows) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (cbase + 16 * j < sg.n)
            *reinterpret_cast<u32x2*>(c + (int64_t)r * sg.ldc + coff + cbase + 16 * j) =
                u32x2{pack_bf16x2(acc[i][j][0], acc[i][j][1]), pack_bf16x2(acc[i][j][2], acc[i][j][3])};
      }
    }
    return;
  }
  if (sg.epi == kEpiFp8Head) {  // a head = 128 columns = waves wn and wn ^ 1: amax per row over both
    __syncthreads();            // every wave is done with the ring, which now holds the row maxima
    float* s_amax = reinterpret_cast<float*>(s_ring);   // [4][kTM]
    uint8_t* c = static_cast<uint8_t*>(sg.c);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float am = 0.0f;
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int v = 0; v < 4; ++v) am = fmaxf(am, fabsf(acc[i][j][v]));
      am = fmaxf(am, __shfl_xor(am, 16, 64));
      am = fmaxf(am, __shfl_xor(am, 32, 64));
      if (kg == 0) s_amax[wn * kTM + 128 * wm + 16 * i + li] = am;
    }
    __syncthreads();
    const int head = (n0 + 64 * wn) / 128;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int rl = 128 * wm + 16 * i + li;
      const int r = m0 + rl;
      const float scale = fmaxf(s_amax[(wn & 2) * kTM + rl], s_amax[((wn & 2) + 1) * kTM + rl]) / 448.0f;
      if (r < p.rows && cbase < sg.n) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          uint32_t w = 0;
#pragma unroll
          for (int v = 0; v < 4; ++v)
            w |= f32_to_e4m3(scale > 0.0f ? acc[i][j][v] / scale : 0.0f) << (8 * v);
          *reinterpret_cast<uint32_t*>(c + (int64_t)r * sg.ldc + cbase + 16 * j) = w;
        }
        if ((wn & 1) == 0 && kg == 0) static_cast<float*>(sg.scale)[(int64_t)r * (sg.n / 128) + head] = scale;
      }
    }
    return;
  }
  // MXFP4: MFMA tiles 2 h and 2 h + 1 form the 32-column block h; E8M0 scale floor(log2 amax) - 2, e2m1
  // codes, element 2i in the low nibble
  uint8_t* c = static_cast<uint8_t*>(sg.c);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = rbase + 16 * i;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      float am = 0.0f;
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int v = 0; v < 4; ++v) am = fmaxf(am, fabsf(acc[i][2 * h + u][v]));
      am = fmaxf(am, __shfl_xor(am, 16, 64));
      am = fmaxf(am, __shfl_xor(am, 32, 64));
      int X = -127;
      if (am > 0.0f) {
        int ex;
        frexpf(am, &ex);  // am = f * 2^ex, f in [0.5, 1)
        X = ex - 1 - 2;
        X = X < -127 ? -127 : (X > 127 ? 127 : X);
      }
      const int col0 = n0 + 64 * wn + 32 * h;
      if (r < p.rows && col0 < sg.n) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          uint32_t w = 0;
#pragma unroll
          for (int v = 0; v < 4; ++v) w |= f32_to_e2m1(ldexpf(acc[i][2 * h + u][v], -X)) << (4 * v);
          *reinterpret_cast<uint16_t*>(c + (int64_t)r * sg.ldc + (cbase + 32 * h + 16 * u) / 2) = (uint16_t)w;
        }
        if (kg == 0) static_cast<uint8_t*>(sg.scale)[(int64_t)r * (sg.n / 32) + col0 / 32] = (uint8_t)(X + 127);
      }
    }
  }
}

// p's segments over the tiled kernel (seg[1].n == 0: one segment); z batches
csa_status launch_proj_tiled(const ProjArgs& p, int z, hipStream_t stream) {
  static bool attr_set = false;
  if (!attr_set) {
    if (hipFuncSetAttribute((const void*)proj_tiled_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)kTLdsBytes) != hipSuccess)
      return CSA_ERR_LAUNCH;
    attr_set = true;
  }
  TiledMap mp;
  mp.ntm = (p.rows + kTM - 1) / kTM;
  for (int i = 0; i < 2; ++i) mp.ntn[i] = (p.seg[i].n + kTN - 1) / kTN;
  mp.tiles0 = (int64_t)z * mp.ntn[0] * mp.ntm;
  mp.tiles = mp.tiles0 + (int64_t)z * mp.ntn[1] * mp.ntm;
  mp.per_xcd = (mp.tiles + 7) / 8;
  if (mp.per_xcd * 8 > (int64_t)INT32_MAX) return CSA_ERR_SHAPE;
  hipLaunchKernelGGL(proj_tiled_kernel, dim3((unsigned)(mp.per_xcd * 8)), dim3(kTThreads), kTLdsBytes, stream, p, mp);
  return hipGetLastError() == hipSuccess ? CSA_OK : CSA_ERR_LAUNCH;
}

template <int TPW0, int KS0, int TPW1, int KS1>
csa_status launch_proj(const ProjArgs& p, int z, hipStream_t stream) {
  if (p.rows > kProjDecodeRows) return launch_proj_tiled(p, z, stream);
  dim3 grid(p.seg[0].blocks + p.seg[1].blocks, z);
  if (p.rows <= 16)
    hipLaunchKernelGGL((proj_kernel<1, TPW0, KS0, TPW1, KS1>), grid, dim3(kProjThreads), 0, stream, p);
  else
    hipLaunchKernelGGL((proj_kernel<2, TPW0, KS0, TPW1, KS1>), grid, dim3(kProjThreads), 0, stream, p);
  return hipGetLastError() == hipSuccess ? CSA_OK : CSA_ERR_LAUNCH;
}

}  // namespace

csa_status launch_q_up_proj(const void* cq, const void* w_uq, const void* w_iuq, int rows, int d_c, int n_h, int c,
                            int n_hI, int cI, void* q, void* qi, void* qi_scale, int qi_t, hipStream_t stream) {
  ProjArgs p;
  p.a = static_cast<const uint16_t*>(cq);
  p.lda = d_c;
  p.a_zoff = 0;
  p.rows = rows;
  p.k = d_c;
  const int nq = n_h * c, ni = n_hI * cI;
  p.seg[0] = ProjSeg{static_cast<const uint16_t*>(w_uq), 0, nq, q, nq, 0, nullptr, kEpiBf16, nq / 16};
  const int epi = qi_t == CSA_FP8_E4M3_ROWSCALE ? kEpiFp8Head : (qi_t == CSA_MXFP4_E8M0_B32 ? kEpiMxfp4 : kEpiBf16);
  const int64_t ldi = qi_t == CSA_MXFP4_E8M0_B32 ? ni / 2 : ni;  // bytes for the quantized forms
  p.seg[1] = ProjSeg{static_cast<const uint16_t*>(w_iuq), 0, ni, qi, ldi, 0, qi_scale, epi, ni / 128};
  return launch_proj<1, 4, 2, 1>(p, 1, stream);
}

csa_status launch_grouped_out_proj(const void* o, const void* w_g, const void* w_o, int rows, int n_h, int c, int g,
                                   int d_g, int d, void* mid, void* out, hipStream_t stream) {
  const int per = n_h * c / g;
  ProjArgs p1;
  p1.a = static_cast<const uint16_t*>(o);
  p1.lda = (int64_t)n_h * c;
  p1.a_zoff = per;
  p1.rows = rows;
  p1.k = per;
  p1.seg[0] = ProjSeg{static_cast<const uint16_t*>(w_g), (int64_t)d_g * per, d_g, mid, (int64_t)g * d_g, d_g, nullptr,
                      kEpiBf16, d_g / 16};
  p1.seg[1] = ProjSeg{nullptr, 0, 0, nullptr, 0, 0, nullptr, kEpiBf16, 0};
  csa_status st = launch_proj<1, 4, 1, 4>(p1, g, stream);
  if (st != CSA_OK) return st;
  ProjArgs p2;
  p2.a = static_cast<const uint16_t*>(mid);
  p2.lda = (int64_t)g * d_g;
  p2.a_zoff = 0;
  p2.rows = rows;
  p2.k = g * d_g;
  p2.seg[0] = ProjSeg{static_cast<const uint16_t*>(w_o), 0, d, out, d, 0, nullptr, kEpiBf16, d / 16};
  p2.seg[1] = ProjSeg{nullptr, 0, 0, nullptr, 0, 0, nullptr, kEpiBf16, 0};
  return launch_proj<1, 4, 1, 4>(p2, 1, stream);
}

csa_status launch_pack_proj_weights(const void* w, void* packed, int z, int n, int k, hipStream_t stream) {
  const int64_t chunks = (int64_t)z * n * k / 8;
  hipLaunchKernelGGL(proj_pack_kernel, dim3((unsigned)((chunks + 255) / 256)), dim3(256), 0, stream,
                     static_cast<const uint16_t*>(w), static_cast<uint16_t*>(packed), chunks, n, k);
  return hipGetLastError() == hipSuccess ? CSA_OK : CSA_ERR_LAUNCH;
}
