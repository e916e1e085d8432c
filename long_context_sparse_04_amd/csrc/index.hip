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
#include <type_traits>

#include "compress_body.h"
#include "csa_common.h"
#include "csa_internal.h"

namespace {

constexpr int kWaves = 4;
constexpr int kTilesPerWave = 16;                      // 4 waves x 16 tiles x 16 entries = 1024 entries / WG
constexpr int kEntriesPerWG = kWaves * kTilesPerWave * 16;
// Bound keys come in runs of 256 entries (one wave's range) and a row holds four runs per 1024 entries.
constexpr int kRun = 256;
static_assert(kTilesPerWave * 16 == kRun, "a bound run is one wave's range");
constexpr int kBoundSpan = 1024;
// Workgroups per row: every run of the row's bound keys is written, so whole 1024-entry spans.
__host__ __device__ inline int64_t index_slots(int64_t n_max) {
  return (kBoundSpan / kEntriesPerWG) * ((n_max + kBoundSpan - 1) / kBoundSpan);
}

// Bound-key sets: two keys per 256 entries for caches of more than kFineBoundMax entries, otherwise two
// per 32 entries, so that a short cache still holds enough keys (2k for k up to n_max / 32).  The decode
// kernel's sets of a 256-entry run are the whole run, or its eight interleaved 32-entry sets
// {e : e mod 64 in [8 r, 8 r + 8)} (the entries one half of a 16-lane row writes; the run's two waves
// merge their halves); the tiled prefill kernel takes each 64-entry tile's halves (fine) or 4 tiles
// (coarse).  The selector uses only the keys' values.
constexpr int64_t kFineBoundMax = 65536;
__host__ __device__ inline int bound_sets(int64_t n_max) { return n_max <= kFineBoundMax ? 8 : 1; }
__host__ __device__ inline int64_t bound_keys_per_row(int64_t n_max) {
  return 2 * (kBoundSpan / kRun) * bound_sets(n_max) * ((n_max + kBoundSpan - 1) / kBoundSpan);
}
constexpr int kRing = 4;                               // tiles in flight per wave

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

// The scores' destination: float32, or bf16 rounded to nearest even (the selector's cheaper input).
struct ScoreOut {
  void* p;
  int bf16;
  CSA_DEV void store(int64_t i, float v) const {
    if (bf16)
      static_cast<uint16_t*>(p)[i] = f32_to_bf16(v);
    else
      static_cast<float*>(p)[i] = v;
  }
  CSA_DEV float stored(float v) const { return bf16 ? __uint_as_float((uint32_t)f32_to_bf16(v) << 16) : v; }
};

// Tiles in flight per wave (each of 16 entry rows), chosen by measurement; the LDS rings of the staged
// formats stay small enough for three (bf16) or four (fp8) workgroups per CU.
template <int FMT>
struct Ring;
template <>
struct Ring<CSA_BF16> {
  static constexpr int kTiles = 2;
};
template <>
struct Ring<CSA_FP8_E4M3_ROWSCALE> {
  static constexpr int kTiles = 3;
};
template <>
struct Ring<CSA_MXFP4_E8M0_B32> {
  static constexpr int kTiles = kRing;  // register ring (rows of 64 bytes: see the kernel)
};

// Swizzle of the 16-byte chunks of an entry row in a staged tile: chunk c of row e sits at position
// c ^ key(e), which spreads the 8 rows one 128-byte LDS read phase touches over all banks.
template <int RB>
CSA_DEV int tile_swz_key(int e) {
  return RB == 64 ? ((e >> 1) & 3) : (e & 7);
}

// N 16-byte LDS reads at byte addresses a[0..N) in one block that waits for them (no read outlives the
// block; outputs early-clobber so that none shares a later read's address register).  Out of the
// compiler's sight on purpose: for reads of a buffer that global-to-LDS loads also fill, it would wait
// for every outstanding load first, draining the ring of tiles in flight.
template <int N>
CSA_DEV void lds_read16(i32x4 (&o)[N], const uint32_t (&a)[N]) {
  if constexpr (N == 1) {
    asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=&v"(o[0]) : "v"(a[0]) : "memory");
  } else if constexpr (N == 2) {
    asm volatile("ds_read_b128 %0, %2\n\tds_read_b128 %1, %3\n\ts_waitcnt lgkmcnt(0)"
                 : "=&v"(o[0]), "=&v"(o[1]) : "v"(a[0]), "v"(a[1]) : "memory");
  } else {
    static_assert(N == 4, "1, 2 or 4 reads");
    asm volatile(
        "ds_read_b128 %0, %4\n\tds_read_b128 %1, %5\n\tds_read_b128 %2, %6\n\tds_read_b128 %3, %7\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3])
        : "memory");
  }
}

// The compression launch folded into a decode index launch: the step's new KV entry and indexer key of
// every sequence (entry first_entry), computed by the workgroup whose entry range holds the new key
// (before it reads any tile, so its scores see the new key) and by another early workgroup (the KV entry).
struct IndexFuse {
  csa_compress_body::Jobs jobs;  // j[0]: the KV entry, j[1]: the indexer key, written into the key cache
  int rows, m, in_t;
  int64_t row0_pos, first_entry;
};
struct NoFuse {};
// A paged key cache (csa_pages): logical entry s of sequence b is pool row table[b * tstride + (s >> plog2)]
// << plog2 | (s & (2^plog2 - 1)).
struct PageMap {
  const int32_t* table;
  int tstride;
  int plog2;
};

template <int FMT, int NT, bool FUSE, bool PAGED>
__global__ __launch_bounds__(kWaves * 64) void index_mfma_kernel(
    const uint8_t* __restrict__ q, const void* __restrict__ q_scale, const float* __restrict__ w,
    const uint8_t* __restrict__ kI, const void* __restrict__ k_scale, int T, int64_t n_max,
    const int64_t* __restrict__ pos0, int m, ScoreOut so, uint32_t* __restrict__ bound,
    std::conditional_t<FUSE, std::conditional_t<PAGED, csa_compress_body::AppendFuse, IndexFuse>, NoFuse> fz,
    PageMap pm) {
  constexpr int HI = NT * 16;
  constexpr int RB = Fmt<FMT>::kRowBytes;
  constexpr int LB = Fmt<FMT>::kLaneBytes;
  constexpr int R = Ring<FMT>::kTiles;
  constexpr int kSlots = R + 1;
  constexpr int kTileBytes = 16 * RB;
  constexpr int kDmaPerTile = kTileBytes / 1024;   // 1 KB (16 bytes per lane) per DMA instruction
  constexpr bool kScaled = FMT != CSA_BF16;
  // Rows of 128 or 256 bytes are staged through LDS: a lane's operand is 32 or 64 bytes of one row, so
  // loading it straight into registers would make every load instruction touch half- or quarter-used
  // 128-byte lines of all 16 rows.  Rows of 64 bytes (MXFP4) load their 16 bytes per lane straight into
  // registers: one instruction then covers the whole 1 KB tile.
  constexpr bool kStaged = RB > 64;
  // The tile rings, slot-major ([slot][wave][tile]).  This query row's HI indexer queries are staged in
  // the last slot when they fit there: that slot is first filled after the queries sit in registers.
  constexpr int kRingBytes = kStaged ? kSlots * kWaves * kTileBytes : 0;
  constexpr bool kQInRing = kStaged && HI * RB <= kWaves * kTileBytes;
  __shared__ __align__(16) uint8_t s_lds[kRingBytes + (kQInRing ? 0 : HI * RB)];
  uint8_t (*s_ring)[kWaves][kTileBytes] = reinterpret_cast<uint8_t (*)[kWaves][kTileBytes]>(s_lds);
  uint8_t* s_q = kQInRing ? &s_lds[R * kWaves * kTileBytes] : &s_lds[kRingBytes];
  __shared__ float s_wq[HI];                      // w (times the fp8 query row scale) per head
  __shared__ uint32_t s_qsc[HI];                  // MXFP4: the 4 E8M0 block scales of each head
  __shared__ uint32_t s_ksc[kStaged && kScaled ? kWaves : 1][kTilesPerWave * 16];  // key scale word per entry

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int gl = lane >> 4;
  // With compression work (the step's new indexer key, read by chunk fc, and its KV entry) row r's slot
  // s serves entry chunk (s + fc - r) mod the slot count: slot r (mod the count) compresses the key
  // before its tiles and slot r + 1 takes the KV entry, so the rows' compressing workgroups sit early in
  // their rows and on different XCDs and CUs (workgroup i runs on XCD i mod 8) instead of sharing one.
  const int row = blockIdx.y;  // b * T + r
  const int wslot = blockIdx.x;
  const int nslots = (int)index_slots(n_max);
  const int b = row / T;
  const int r = row - b * T;
  const int64_t srow = (int64_t)row * n_max;  // this row's first score
  const int ik_slot = row % nslots, kv_slot = (row + 1) % nslots;
  int64_t fc = 0;
  [[maybe_unused]] int64_t tf = 0, fi = 0;
  [[maybe_unused]] bool fdone = false;
  if constexpr (FUSE && PAGED) {
    tf = pos0[b];
    fi = tf / fz.m - 1;
    // (uniform) the block tf closes has an entry whose page is mapped
    fdone = tf >= fz.m && tf % fz.m == 0 && (fi >> fz.jobs.j[0].plog2) < fz.jobs.j[0].tstride;
    if (fdone) fc = fi / kEntriesPerWG;
  } else if constexpr (FUSE) {
    fc = fz.first_entry / kEntriesPerWG;
  }
  const int64_t chunk = FUSE ? ((int64_t)wslot + fc + nslots - ik_slot) % nslots : wslot;
  const int64_t wg_first = chunk * kEntriesPerWG;

  if constexpr (FUSE && PAGED) {  // decode rows only (row == b): this token's csa_decode_append work
    constexpr int kScratch = 3 * 256;
    constexpr bool kInLds = sizeof(s_lds) >= kScratch * sizeof(f32x4);
    __shared__ __align__(16) f32x4 s_cz[kInLds ? 1 : kScratch];
    __shared__ float s_czr[4];
    f32x4* cz = kInLds ? reinterpret_cast<f32x4*>(s_lds) : s_cz;
    const int64_t t = tf;
    const int m = fz.m;
    const int64_t i = fi;
    const bool done = fdone;
    const bool do_ik = done && wslot == ik_slot;  // its key, before this WG's tiles
    const bool do_kv = t >= 0 && wslot == kv_slot;
    const bool f32in = fz.in_t == CSA_F32;
    if (do_ik) {
      if (f32in) {
        csa_compress_body::compress_one<float, 256>(fz.jobs.j[1], fz.jobs.theta[1], 0, b, 0, m, 0, i, cz, cz + 256,
                                                    cz + 512, s_czr);
        csa_compress_body::store_ring_rows<float>(fz.jobs.j[1], fz.src[1], b, t);
      } else {
        csa_compress_body::compress_one<uint16_t, 256>(fz.jobs.j[1], fz.jobs.theta[1], 0, b, 0, m, 0, i, cz,
                                                       cz + 256, cz + 512, s_czr);
        csa_compress_body::store_ring_rows<uint16_t>(fz.jobs.j[1], fz.src[1], b, t);
      }
    }
    if (do_ik && do_kv) __syncthreads();  // the slice-merge scratch is used again
    if (do_kv) {
      if (f32in) {
        if (done)
          csa_compress_body::compress_one<float, 256>(fz.jobs.j[0], fz.jobs.theta[0], 0, b, 0, m, 0, i, cz,
                                                      cz + 256, cz + 512, s_czr);
        csa_compress_body::store_ring_rows<float>(fz.jobs.j[0], fz.src[0], b, t);
        if (!done) csa_compress_body::store_ring_rows<float>(fz.jobs.j[1], fz.src[1], b, t);
        if (fz.win_ring) csa_compress_body::store_window_row<float, 256>(fz, b, t, s_czr);
      } else {
        if (done)
          csa_compress_body::compress_one<uint16_t, 256>(fz.jobs.j[0], fz.jobs.theta[0], 0, b, 0, m, 0, i, cz,
                                                         cz + 256, cz + 512, s_czr);
        csa_compress_body::store_ring_rows<uint16_t>(fz.jobs.j[0], fz.src[0], b, t);
        if (!done) csa_compress_body::store_ring_rows<uint16_t>(fz.jobs.j[1], fz.src[1], b, t);
        if (fz.win_ring) csa_compress_body::store_window_row<uint16_t, 256>(fz, b, t, s_czr);
      }
    }
    if (do_ik || do_kv) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
    }
  } else if constexpr (FUSE) {  // decode rows only (row == b)
    constexpr int kScratch = 3 * 256;  // f32x4 slots of the compression's slice merge
    constexpr bool kInLds = sizeof(s_lds) >= kScratch * sizeof(f32x4);
    __shared__ __align__(16) f32x4 s_cz[kInLds ? 1 : kScratch];
    __shared__ float s_czr[4];
    f32x4* cz = kInLds ? reinterpret_cast<f32x4*>(s_lds) : s_cz;
    const bool do_ik = wslot == ik_slot;                                // chunk fc holds first_entry
    const bool do_kv = wslot == kv_slot && fz.jobs.j[0].out != nullptr;  // (no KV job: the key alone)
    if (do_ik) {
      if (fz.in_t == CSA_F32)
        csa_compress_body::compress_one<float, 256>(fz.jobs.j[1], fz.jobs.theta[1], 0, row, fz.rows, fz.m,
                                                    fz.row0_pos, fz.first_entry, cz, cz + 256, cz + 512, s_czr);
      else
        csa_compress_body::compress_one<uint16_t, 256>(fz.jobs.j[1], fz.jobs.theta[1], 0, row, fz.rows, fz.m,
                                                       fz.row0_pos, fz.first_entry, cz, cz + 256, cz + 512, s_czr);
    }
    if (do_ik && do_kv) __syncthreads();  // the slice-merge scratch is used again
    if (do_kv) {
      if (fz.in_t == CSA_F32)
        csa_compress_body::compress_one<float, 256>(fz.jobs.j[0], fz.jobs.theta[0], 0, row, fz.rows, fz.m,
                                                    fz.row0_pos, fz.first_entry, cz, cz + 256, cz + 512, s_czr);
      else
        csa_compress_body::compress_one<uint16_t, 256>(fz.jobs.j[0], fz.jobs.theta[0], 0, row, fz.rows, fz.m,
                                                       fz.row0_pos, fz.first_entry, cz, cz + 256, cz + 512, s_czr);
    }
    if (do_ik || do_kv) {
      // the new key is in memory (L2) before this workgroup reads any tile, and the scratch is free
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
    }
  }

  // Wave w streams the contiguous entries [wave_first, wave_first + 16 * kTilesPerWave) tile by tile.
  // A tile's 16 rows are contiguous in memory and arrive by direct global-to-LDS loads of 1 KB per
  // instruction (lane i -> bytes [16 i, 16 i + 16) of the instruction's span), into this wave's ring of
  // R + 1 tile buffers: the load of tile i + R is issued before tile i is used, into the buffer tile
  // i - 1 has released, so R tiles are always in flight.  The wave reads its MFMA operands back from its
  // own buffers, so no barrier is involved.
  const int64_t wave_first = wg_first + (int64_t)wave * kTilesPerWave * 16;
  // Paged keys: a 16-entry tile never straddles a page (pages hold 2^plog2 >= 32 entries), and the tile
  // of a clamped row (past n_max - 1) is the page of entry n_max - 1.  Lane j holds the pool page of this
  // wave's j-th logical page (clamped to the last one), loaded once before any tile.
  const int64_t wfp = PAGED ? wave_first >> pm.plog2 : 0;
  const int64_t pmask = PAGED ? ((int64_t)1 << pm.plog2) - 1 : 0;
  // Pages of 256 entries or more hold a wave's whole range (clamped rows included): one uniform entry.
  const bool one_page = PAGED && pm.plog2 >= 8;  // (uniform)
  int tab = 0, tab1 = 0;
  if constexpr (PAGED) {
    const int64_t lastp = (n_max - 1) >> pm.plog2;
    if (one_page) {
      const int64_t wfu = __builtin_amdgcn_readfirstlane((int)wfp);
      tab1 = __builtin_amdgcn_readfirstlane(pm.table[(int64_t)b * pm.tstride + min(wfu, lastp)]);
    } else {
      tab = pm.table[(int64_t)b * pm.tstride + min(wfp + lane, lastp)];
    }
  }
  // pool row of the clamped entry er, whose tile starts at the clamped entry ec
  auto key_row = [&](int64_t er, int64_t ec) -> int64_t {
    if constexpr (PAGED) {
      const int pg = one_page ? tab1 : __builtin_amdgcn_readlane(tab, (int)max((int64_t)0, (ec >> pm.plog2) - wfp));
      return ((int64_t)pg << pm.plog2) | (er & pmask);
    } else {
      return (int64_t)b * n_max + er;
    }
  };
  Frag<FMT> kf_reg[kStaged ? 1 : kSlots];  // register ring (unstaged rows)
  int ksc_reg[kStaged ? 1 : kSlots];
  auto issue_tile = [&](int slot, int64_t e0) {
    if constexpr (!kStaged) {
      const int64_t el = min(e0 + (lane & 15), n_max - 1);
      const int64_t kr = key_row(el, min(e0, n_max - 1));
      kf_reg[slot] = load_frag<FMT>(kI + kr * RB, lane);
      ksc_reg[slot] = static_cast<const uint8_t*>(k_scale)[kr * 4 + gl];
      return;
    }
#pragma unroll
    for (int j = 0; j < kDmaPerTile; ++j) {
      const int off = 1024 * j + 16 * lane;       // byte offset in the tile (LDS position)
      const int e = off / RB;                     // tile row
      const int pos = (off % RB) / 16;            // chunk position in the row
      const int c = pos ^ tile_swz_key<RB>(e);    // logical chunk stored there
      const int64_t er = min(e0 + e, n_max - 1);  // rows past the end re-read the last one
      __builtin_amdgcn_global_load_lds(
          (const __attribute__((address_space(1))) void*)(kI + key_row(er, min(e0, n_max - 1)) * RB + 16 * c),
          (__attribute__((address_space(3))) void*)(&s_ring[slot][wave][1024 * j]), 16, 0, 0);
    }
  };
  // the key scale words of all of the wave's entries (4 bytes each: the fp8 row scale, or the 4 E8M0
  // block scales of an MXFP4 row), 64 entries per instruction, before any tile
  if constexpr (kStaged && kScaled) {
    constexpr int kScaleLoads = kTilesPerWave * 16 / 64;
    int64_t srow[kScaleLoads];  // every row first: the page lookups are lane exchanges, kept ahead of the DMA
#pragma unroll
    for (int j = 0; j < kScaleLoads; ++j) {
      const int64_t er = min(wave_first + 64 * j + lane, n_max - 1);
      if constexpr (PAGED)
        srow[j] = ((int64_t)(one_page ? tab1 : __shfl(tab, (int)((er >> pm.plog2) - wfp), 64)) << pm.plog2) |
                  (er & pmask);
      else
        srow[j] = (int64_t)b * n_max + er;
    }
#pragma unroll
    for (int j = 0; j < kScaleLoads; ++j)
      __builtin_amdgcn_global_load_lds(
          (const __attribute__((address_space(1))) void*)(static_cast<const uint32_t*>(k_scale) + srow[j]),
          (__attribute__((address_space(3))) void*)(&s_ksc[wave][64 * j]), 4, 0, 0);
  }
  // the first R tiles go out before anything else (they do not wait for the query position; past the
  // visible range they are simply not used)
#pragma unroll
  for (int u = 0; u < R; ++u) issue_tile(u, wave_first + 16 * u);

  // ---- this row's queries and weights, loaded once per workgroup into LDS
  const int64_t t = pos0[b] + r;
  const int64_t vis = visible_entries(t, m, n_max);
  {
    const i32x4* src = reinterpret_cast<const i32x4*>(q + (int64_t)row * HI * RB);
    i32x4* dst = reinterpret_cast<i32x4*>(s_q);
#pragma unroll
    for (int i = threadIdx.x; i < HI * RB / 16; i += kWaves * 64) dst[i] = src[i];
    if (threadIdx.x < HI) {
      float wv = w[(int64_t)row * HI + threadIdx.x];
      if constexpr (FMT == CSA_FP8_E4M3_ROWSCALE)
        wv *= static_cast<const float*>(q_scale)[(int64_t)row * HI + threadIdx.x];
      s_wq[threadIdx.x] = wv;
      if constexpr (FMT == CSA_MXFP4_E8M0_B32)
        s_qsc[threadIdx.x] = reinterpret_cast<const uint32_t*>(q_scale)[(int64_t)row * HI + threadIdx.x];
    }
  }
  __syncthreads();
  // A operand (heads are MFMA rows) and the epilogue weights of the 4 heads of each lane's output rows
  Frag<FMT> qa[NT];
  int qsc[NT];
  float wq[NT][4];
#pragma unroll
  for (int g = 0; g < NT; ++g) {
    const int head = 16 * g + (lane & 15);
    const i32x4* p = reinterpret_cast<const i32x4*>(s_q + head * RB + gl * Fmt<FMT>::kLaneBytes);
#pragma unroll
    for (int j = 0; j < Fmt<FMT>::kLaneBytes / 16; ++j) qa[g].v[j] = p[j];
    qsc[g] = (FMT == CSA_MXFP4_E8M0_B32) ? (int)((s_qsc[head] >> (8 * gl)) & 0xFFu) : 127;
#pragma unroll
    for (int i = 0; i < 4; ++i) wq[g][i] = s_wq[16 * g + 4 * gl + i];  // head of output row i in this lane
  }
  if constexpr (kQInRing) __syncthreads();  // every wave holds its queries before slot R is refilled

  // tiles past the visible range are not computed (their scores are -inf)
  const int ntiles = (int)max((int64_t)0, min((int64_t)kTilesPerWave, (vis - wave_first + 15) / 16));
  // this lane's operand chunks in a staged tile: row lane & 15, logical chunks LB/16 * gl .. + LB/16 - 1
  const int te = lane & 15;
  float p[4];
  uint32_t top1 = 0u, top2 = 0u;  // this lane's two largest visible score keys (0: none)
#pragma unroll
  for (int ti = 0; ti < kTilesPerWave; ++ti) {
    const int slot = ti % kSlots;
    const int u = ti & 3;
    const int64_t e0 = wave_first + (int64_t)ti * 16;
    const bool refill = ti + R < ntiles;
    if (refill) issue_tile((ti + R) % kSlots, e0 + 16 * R);
    if (ti < ntiles) {
      Frag<FMT> kf;
      int ksc = 127;
      float ksf = 1.0f;
      if constexpr (!kStaged) {
        kf = kf_reg[slot];
        ksc = ksc_reg[slot];
      } else {
      // tile ti has landed once at most the R younger tiles' loads are outstanding (loads complete
      // in order); near the end, once none is
      if (refill)
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(R * kDmaPerTile) : "memory");
      else
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      uint32_t ka[LB / 16];
#pragma unroll
      for (int j = 0; j < LB / 16; ++j)
        ka[j] = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)&s_ring[slot][wave][0] +
                (uint32_t)(te * RB + 16 * (((LB / 16) * gl + j) ^ tile_swz_key<RB>(te)));
      lds_read16<LB / 16>(kf.v, ka);
      if constexpr (kScaled) {
        i32x4 sw[1];
        const uint32_t sa[1] = {(uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)&s_ksc[wave][16 * ti + te]};
        asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=&v"(sw[0][0]) : "v"(sa[0]) : "memory");
        if constexpr (FMT == CSA_MXFP4_E8M0_B32) ksc = (int)(((uint32_t)sw[0][0] >> (8 * gl)) & 0xFFu);
        if constexpr (FMT == CSA_FP8_E4M3_ROWSCALE) ksf = __int_as_float(sw[0][0]);
      }
      }
      float part = 0.0f;
#pragma unroll
      for (int g = 0; g < NT; ++g) {
        const f32x4 acc = mfma_tile<FMT>(qa[g], kf, qsc[g], ksc);
#pragma unroll
        for (int i = 0; i < 4; ++i) part = fmaf(wq[g][i], fmaxf(acc[i], 0.0f), part);
      }
      p[u] = part * ksf;  // the FP8 row scale is positive, so it factors out of every ReLU
    } else {
      p[u] = 0.0f;
    }
    if (u == 3) {
      // reduce-scatter over the 4 lane groups: lane 16u + e ends with the sum for tile u, entry e
      const int64_t eg = e0 - 48;  // first entry of this group of 4 tiles
      if (eg >= n_max) break;
      const bool hi2 = gl >= 2;
      const float s0 = hi2 ? p[0] : p[2], s1 = hi2 ? p[1] : p[3];
      const float k0 = (hi2 ? p[2] : p[0]) + __shfl_xor(s0, 32, 64);
      const float k1 = (hi2 ? p[3] : p[1]) + __shfl_xor(s1, 32, 64);
      const bool odd = gl & 1;
      const float val = (odd ? k1 : k0) + __shfl_xor(odd ? k0 : k1, 16, 64);
      const int64_t eo = eg + lane;  // entry this lane writes
      if (eo < n_max) so.store(srow + eo, (eo < vis) ? val : -INFINITY);
      if (eo < vis) {
        const uint32_t key = score_key(so.stored(val));  // the key of the score the selector will read
        top2 = max(top2, min(top1, key));
        top1 = max(top1, key);
      }
    }
  }
  // Lower-bound keys for the selector: the two largest visible scores of each of the wave's bound sets
  // (the whole wave, or each half of a 16-lane row: see bound_sets).  They are scores of distinct visible entries,
  // so the K-th largest key over a row's bound keys never exceeds the row's K-th largest score key.
  if (bound) {
    const int sets = bound_sets(n_max);
    const int64_t nbw = bound_keys_per_row(n_max);
    if (sets == 8) {
      half_row_top2(top1, top2);
    } else {
      wave_top2(top1, top2);
    }
    if ((lane & 7) == 0 && (sets == 8 || lane == 0)) {
      const int64_t run = wave_first / kRun;
      uint32_t* dst = bound + (int64_t)row * nbw + (run * sets + (lane >> 3)) * 2;
      dst[0] = top1;
      dst[1] = top2;
    }
  }
}

// Prefill (many query rows, bf16): the indexer is a dense contraction
// [rows x heads] x [c^I x entries].  A workgroup serves kPRows consecutive query
// rows of one sequence, kPRowsPerWave per wave, each wave holding its rows'
// HI x 128 queries in registers as MFMA A operands.  Entries stream through LDS
// in tiles of 64 rows (global_load_lds, double-buffered, 16-byte chunk c of
// entry e stored at chunk c ^ (e & 15) so that the B-operand reads of 16 entries
// hit all banks), and every tile is shared by the workgroup's kPRows rows.  The
// epilogue is the decode kernel's: weighted ReLU head sum per lane, then a
// reduce-scatter over the 4 lane groups for one coalesced 256-byte store per row
// and tile.
constexpr int kPRowsPerWave = 2;
constexpr int kPRows = kWaves * kPRowsPerWave;  // 8 query rows per workgroup
constexpr int kPTile = 64;                      // entries per LDS tile
constexpr int kPRowBytes = 256;                 // bf16 c^I = 128
constexpr int kPDmaPerWave = kPTile * kPRowBytes / 1024 / kWaves;  // 1 KB per DMA instruction: 4 per wave

template <int NT>
__global__ __launch_bounds__(kWaves * 64, 2) void index_prefill_bf16_kernel(
    const uint8_t* __restrict__ q, const float* __restrict__ w, const uint8_t* __restrict__ kI, int T,
    int64_t n_max, const int64_t* __restrict__ pos0, int m, ScoreOut so, uint32_t* __restrict__ bound) {
  constexpr int HI = NT * 16;
  __shared__ __align__(16) uint8_t s_k[2][kPTile * kPRowBytes];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // (uniform: row arithmetic in SGPRs)
  const int gl = lane >> 4;
  const int b = blockIdx.y;
  const int r_first = blockIdx.x * kPRows;
  const uint8_t* kb = kI + (int64_t)b * n_max * kPRowBytes;

  // tile DMA: instruction j of wave w fills entries 4 (w + 4 j) .. +3 of the tile; lane i writes chunk
  // position i % 16 of entry 4 (w + 4 j) + i / 16 and so loads the logical chunk stored there
  auto issue_tile = [&](int buf, int64_t e_base) {
#pragma unroll
    for (int j = 0; j < kPDmaPerWave; ++j) {
      const int e0 = 4 * (wave + 4 * j);
      const int e = e0 + (lane >> 4);
      const int64_t ge = min(e_base + e, n_max - 1);
      const uint8_t* src = kb + ge * kPRowBytes + 16 * ((lane & 15) ^ (e & 15));
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                       (__attribute__((address_space(3))) void*)(&s_k[buf][e0 * kPRowBytes]), 16,
                                       0, 0);
    }
  };

  // the rows of this wave: queries (A operands) and per-head weights
  bf16x8 qa[kPRowsPerWave][NT][4];
  float wq[kPRowsPerWave][NT][4];
  int64_t vis[kPRowsPerWave];
  bool live[kPRowsPerWave];
#pragma unroll
  for (int rr = 0; rr < kPRowsPerWave; ++rr) {
    const int r = r_first + wave * kPRowsPerWave + rr;
    live[rr] = r < T;
    const int rc = live[rr] ? r : T - 1;
    const int64_t row = (int64_t)b * T + rc;
#pragma unroll
    for (int g = 0; g < NT; ++g) {
      const int head = 16 * g + (lane & 15);
      const i32x4* src = reinterpret_cast<const i32x4*>(q + (row * HI + head) * kPRowBytes + gl * 16);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) qa[rr][g][ks] = as_bf16x8(src[4 * ks]);  // dims 32 ks + 8 gl .. +8
#pragma unroll
      for (int i = 0; i < 4; ++i) wq[rr][g][i] = w[row * HI + 16 * g + 4 * gl + i];
    }
    vis[rr] = visible_entries(pos0[b] + rc, m, n_max);
  }
  // entries up to the largest visibility of the workgroup's rows are computed; the rest are -inf
  const int r_last = min(r_first + kPRows, T) - 1;
  const int64_t vis_max = visible_entries(pos0[b] + r_last, m, n_max);
  const int ntiles = (int)((vis_max + kPTile - 1) / kPTile);

  // bound keys (optional): the two largest visible score keys of each 32-entry half tile (caches of up to
  // kFineBoundMax entries), or of each run of 4 tiles (256 entries); sets past the computed tiles get 0
  const bool fine = bound_sets(n_max) > 1;
  const int64_t nbw = bound_keys_per_row(n_max);
  uint32_t bt1[kPRowsPerWave], bt2[kPRowsPerWave];  // coarse sets: the lane's running top-2 of each row
#pragma unroll
  for (int rr = 0; rr < kPRowsPerWave; ++rr) bt1[rr] = bt2[rr] = 0u;

  if (ntiles > 0) issue_tile(0, 0);
  for (int ti = 0; ti < ntiles; ++ti) {
    const int buf = ti & 1;
    if (ti + 1 < ntiles) {
      issue_tile(buf ^ 1, (int64_t)(ti + 1) * kPTile);
      // this tile has landed once only the next tile's kPDmaPerWave loads are outstanding (vector memory
      // operations complete in issue order)
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kPDmaPerWave) : "memory");
    } else {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    __syncthreads();
    const uint8_t* tb = s_k[buf];
#pragma unroll
    for (int rr = 0; rr < kPRowsPerWave; ++rr) {
      float p[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {  // 16-entry sub-tile u: B operands from LDS, then NT x 4 MFMAs
        const int e = 16 * u + (lane & 15);
        bf16x8 kbf[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          kbf[ks] = *reinterpret_cast<const bf16x8*>(tb + e * kPRowBytes + 16 * ((4 * ks + gl) ^ (e & 15)));
        float part = 0.0f;
#pragma unroll
        for (int g = 0; g < NT; ++g) {
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[rr][g][ks], kbf[ks], acc, 0, 0, 0);
#pragma unroll
          for (int i = 0; i < 4; ++i) part = fmaf(wq[rr][g][i], fmaxf(acc[i], 0.0f), part);
        }
        p[u] = part;
      }
      // reduce-scatter over the 4 lane groups: lane 16u + e ends with the sum for sub-tile u, entry e
      const bool hi2 = gl >= 2;
      const float s0 = hi2 ? p[0] : p[2], s1 = hi2 ? p[1] : p[3];
      const float k0 = (hi2 ? p[2] : p[0]) + __shfl_xor(s0, 32, 64);
      const float k1 = (hi2 ? p[3] : p[1]) + __shfl_xor(s1, 32, 64);
      const bool odd = gl & 1;
      const float val = (odd ? k1 : k0) + __shfl_xor(odd ? k0 : k1, 16, 64);
      const int64_t eo = (int64_t)ti * kPTile + lane;
      const int64_t row = (int64_t)b * T + r_first + wave * kPRowsPerWave + rr;
      if (live[rr] && eo < n_max) so.store(row * n_max + eo, eo < vis[rr] ? val : -INFINITY);
      if (bound) {   // (wave-uniform branches)
        const uint32_t key = (eo < vis[rr]) ? score_key(so.stored(val)) : 0u;
        if (fine) {
          uint32_t t1 = key, t2 = 0u;
          half_wave_top2(t1, t2);
          if (live[rr] && (lane & 31) == 0) {
            uint32_t* dst = bound + row * nbw + (2 * (int64_t)ti + (lane >> 5)) * 2;
            dst[0] = t1;
            dst[1] = t2;
          }
        } else {
          bt2[rr] = max(bt2[rr], min(bt1[rr], key));
          bt1[rr] = max(bt1[rr], key);
          if ((ti & 3) == 3 || ti == ntiles - 1) {
            uint32_t t1 = bt1[rr], t2 = bt2[rr];
            wave_top2(t1, t2);
            if (live[rr] && lane == 0) {
              uint32_t* dst = bound + row * nbw + (int64_t)(ti >> 2) * 2;
              dst[0] = t1;
              dst[1] = t2;
            }
            bt1[rr] = bt2[rr] = 0u;
          }
        }
      }
    }
    __syncthreads();  // the buffer is refilled by the next-but-one tile
  }
  if (bound) {   // sets past the computed tiles hold no visible entry
    const int64_t done = fine ? 2 * (int64_t)ntiles : ((int64_t)ntiles + 3) / 4;
#pragma unroll
    for (int rr = 0; rr < kPRowsPerWave; ++rr) {
      if (!live[rr]) continue;
      const int64_t row = (int64_t)b * T + r_first + wave * kPRowsPerWave + rr;
      for (int64_t j = 2 * done + lane; j < nbw; j += 64) bound[row * nbw + j] = 0u;
    }
  }
  // entries past every row's visibility
#pragma unroll
  for (int rr = 0; rr < kPRowsPerWave; ++rr) {
    if (!live[rr]) continue;
    const int64_t row = (int64_t)b * T + r_first + wave * kPRowsPerWave + rr;
    for (int64_t eo = (int64_t)ntiles * kPTile + lane; eo < n_max; eo += 64) so.store(row * n_max + eo, -INFINITY);
  }
}

// float32 path: one thread per (query row, entry), FMA over dims then heads.
constexpr int kF32Threads = 256;
__global__ __launch_bounds__(kF32Threads) void index_f32_kernel(const float* __restrict__ q,
                                                                const float* __restrict__ w,
                                                                const float* __restrict__ kI, int T, int HI, int cI,
                                                                int64_t n_max, const int64_t* __restrict__ pos0,
                                                                int m, ScoreOut so) {
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
  const int64_t out = (int64_t)row * n_max + s;
  if (s >= vis) {
    so.store(out, -INFINITY);
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
  so.store(out, tot);
}

template <int FMT>
csa_status launch_fmt(const void* q, const void* q_scale, const float* w, const void* k, const void* k_scale, int B,
                      int T, int HI, int64_t n_max, const int64_t* pos0, int m, ScoreOut so, uint32_t* bound,
                      const IndexFuse* fuse, const PageMap* pages, hipStream_t stream,
                      const csa_compress_body::AppendFuse* afz = nullptr) {
  if (pages) {  // decode rows over a paged key pool (with this token's append work when afz is given)
    if (fuse || T != 1) return CSA_ERR_UNSUPPORTED;
    const dim3 grid((unsigned)index_slots(n_max), B);
    dim3 block(kWaves * 64);
#define CSA_IDX_PAGED(NT)                                                                                   \
  if (afz)                                                                                                  \
    hipLaunchKernelGGL((index_mfma_kernel<FMT, NT, true, true>), grid, block, 0, stream, (const uint8_t*)q, q_scale, \
                       w, (const uint8_t*)k, k_scale, 1, n_max, pos0, m, so, bound, *afz, *pages);          \
  else                                                                                                      \
    hipLaunchKernelGGL((index_mfma_kernel<FMT, NT, false, true>), grid, block, 0, stream, (const uint8_t*)q, q_scale, \
                       w, (const uint8_t*)k, k_scale, 1, n_max, pos0, m, so, bound, NoFuse{}, *pages)
    switch (HI) {
      case 16: CSA_IDX_PAGED(1); break;
      case 32: CSA_IDX_PAGED(2); break;
      case 64: CSA_IDX_PAGED(4); break;
      case 128: CSA_IDX_PAGED(8); break;
      default: return CSA_ERR_UNSUPPORTED;
    }
#undef CSA_IDX_PAGED
    return hipGetLastError() == hipSuccess ? CSA_OK : CSA_ERR_LAUNCH;
  }
  if (use_prefill_index(FMT, T, HI)) {  // many query rows: the tiled contraction
    if (fuse) return CSA_ERR_UNSUPPORTED;
    dim3 grid(ceil_div(T, kPRows), B);
    hipLaunchKernelGGL((index_prefill_bf16_kernel<4>), grid, dim3(kWaves * 64), 0, stream, (const uint8_t*)q, w,
                       (const uint8_t*)k, T, n_max, pos0, m, so, bound);
    return hipGetLastError() == hipSuccess ? CSA_OK : CSA_ERR_LAUNCH;
  }
  const dim3 grid((unsigned)index_slots(n_max), (unsigned)(B * T));
  dim3 block(kWaves * 64);
#define CSA_IDX_LAUNCH(NT)                                                                                       \
  if (fuse)                                                                                                     \
    hipLaunchKernelGGL((index_mfma_kernel<FMT, NT, true, false>), grid, block, 0, stream, (const uint8_t*)q, q_scale, \
                       w, (const uint8_t*)k, k_scale, T, n_max, pos0, m, so, bound, *fuse, PageMap{});       \
  else                                                                                                          \
    hipLaunchKernelGGL((index_mfma_kernel<FMT, NT, false, false>), grid, block, 0, stream, (const uint8_t*)q,     \
                       q_scale, w, (const uint8_t*)k, k_scale, T, n_max, pos0, m, so, bound, NoFuse{}, PageMap{})
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

int64_t index_bound_keys(int64_t n_max) { return bound_keys_per_row(n_max); }

// the tiled prefill kernel serves bf16 queries of many rows with 64 heads
bool use_prefill_index(int fmt, int T, int HI) { return fmt == CSA_BF16 && T >= kPRows && HI == 64; }



static csa_status launch_index_impl(const void* q, const void* q_scale, const float* w, const void* k,
                                    const void* k_scale, int B, int T, int HI, int cI, int64_t n_max,
                                    const int64_t* pos0, int m, int qk_t, void* scores, int score_t,
                                    uint32_t* bound, const IndexFuse* fuse, const PageMap* pages,
                                    hipStream_t stream);

csa_status launch_index(const void* q, const void* q_scale, const float* w, const void* k, const void* k_scale,
                        int B, int T, int HI, int cI, int64_t n_max, const int64_t* pos0, int m, int qk_t,
                        void* scores, int score_t, uint32_t* bound, hipStream_t stream) {
  return launch_index_impl(q, q_scale, w, k, k_scale, B, T, HI, cI, n_max, pos0, m, qk_t, scores, score_t, bound,
                           nullptr, nullptr, stream);
}

csa_status launch_index_paged(const void* q, const void* q_scale, const float* w, const void* k_pool,
                              const void* k_scale_pool, const csa_pages* pages, int B, int HI, int cI, int64_t n_max,
                              const int64_t* pos0, int m, int qk_t, void* scores, int score_t, uint32_t* bound,
                              hipStream_t stream) {
  int plog2 = 0;
  while ((1 << plog2) < pages->page_tokens / m) ++plog2;
  const PageMap pm{pages->block_table, pages->max_pages, plog2};
  return launch_index_impl(q, q_scale, w, k_pool, k_scale_pool, B, 1, HI, cI, n_max, pos0, m, qk_t, scores, score_t,
                           bound, nullptr, &pm, stream);
}

csa_status launch_compress_index(const CompressJob* jobs, int rows, int m, int64_t row0_pos, int64_t first_entry,
                                 int in_t, const void* q, const void* q_scale, const float* w, const void* k,
                                 const void* k_scale, int B, int HI, int cI, int64_t n_max, const int64_t* pos0,
                                 int qk_t, void* scores, int score_t, uint32_t* bound, hipStream_t stream) {
  IndexFuse fz;
  csa_compress_body::fill_jobs(jobs, 2, fz.jobs);
  fz.rows = rows;
  fz.m = m;
  fz.in_t = in_t;
  fz.row0_pos = row0_pos;
  fz.first_entry = first_entry;
  return launch_index_impl(q, q_scale, w, k, k_scale, B, 1, HI, cI, n_max, pos0, m, qk_t, scores, score_t, bound,
                           &fz, nullptr, stream);
}

static csa_status launch_index_impl(const void* q, const void* q_scale, const float* w, const void* k,
                                    const void* k_scale, int B, int T, int HI, int cI, int64_t n_max,
                                    const int64_t* pos0, int m, int qk_t, void* scores, int score_t,
                                    uint32_t* bound, const IndexFuse* fuse, const PageMap* pages,
                                    hipStream_t stream) {
  const ScoreOut so{scores, score_t == CSA_BF16 ? 1 : 0};
  switch (qk_t) {
    case CSA_F32: {
      if (bound || fuse || pages) return CSA_ERR_UNSUPPORTED;
      dim3 grid(ceil_div(n_max, kF32Threads), B * T);
      size_t lds = (size_t)HI * cI * sizeof(float);
      hipLaunchKernelGGL(index_f32_kernel, grid, dim3(kF32Threads), lds, stream, (const float*)q, w,
                         (const float*)k, T, HI, cI, n_max, pos0, m, so);
      return hipGetLastError() == hipSuccess ? CSA_OK : CSA_ERR_LAUNCH;
    }
    case CSA_BF16:
      return launch_fmt<CSA_BF16>(q, q_scale, w, k, k_scale, B, T, HI, n_max, pos0, m, so, bound, fuse, pages, stream);
    case CSA_FP8_E4M3_ROWSCALE:
      return launch_fmt<CSA_FP8_E4M3_ROWSCALE>(q, q_scale, w, k, k_scale, B, T, HI, n_max, pos0, m, so, bound, fuse, pages, stream);
    case CSA_MXFP4_E8M0_B32:
      return launch_fmt<CSA_MXFP4_E8M0_B32>(q, q_scale, w, k, k_scale, B, T, HI, n_max, pos0, m, so, bound, fuse, pages, stream);
    default:
      return CSA_ERR_UNSUPPORTED;
  }
}

csa_status launch_append_index_paged(const csa_append_job* jobs, const csa_window_job* win, int in_t, const void* q,
                                     const void* q_scale, const float* w, const void* k_pool,
                                     const void* k_scale_pool, const csa_pages* pages, int B, int HI, int cI,
                                     int64_t n_max, const int64_t* pos0, int m, int qk_t, void* scores, int score_t,
                                     uint32_t* bound, hipStream_t stream) {
  csa_compress_body::AppendFuse af;
  csa_compress_body::fill_append(jobs, win, pages, in_t, af);
  int plog2 = 0;
  while ((1 << plog2) < pages->page_tokens / m) ++plog2;
  const PageMap pm{pages->block_table, pages->max_pages, plog2};
  const ScoreOut so{scores, score_t == CSA_BF16 ? 1 : 0};
  switch (qk_t) {
    case CSA_BF16:
      return launch_fmt<CSA_BF16>(q, q_scale, w, k_pool, k_scale_pool, B, 1, HI, n_max, pos0, m, so, bound, nullptr,
                                  &pm, stream, &af);
    case CSA_FP8_E4M3_ROWSCALE:
      return launch_fmt<CSA_FP8_E4M3_ROWSCALE>(q, q_scale, w, k_pool, k_scale_pool, B, 1, HI, n_max, pos0, m, so,
                                               bound, nullptr, &pm, stream, &af);
    case CSA_MXFP4_E8M0_B32:
      return launch_fmt<CSA_MXFP4_E8M0_B32>(q, q_scale, w, k_pool, k_scale_pool, B, 1, HI, n_max, pos0, m, so,
                                            bound, nullptr, &pm, stream, &af);
    default:
      return CSA_ERR_UNSUPPORTED;
  }
}
