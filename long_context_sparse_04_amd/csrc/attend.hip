// csa_attend / hca_attend kernels: shared-KV multi-query attention over the
// selected (CSA) or all visible (HCA) compressed entries plus the sliding window.
//
// "【论文解读】DeepSeek-V4" (wkq9411.github.io), section 一(三)1(3) (shared key-value
// MQA: every entry is both key and value, all query heads share it), 一(三)2(2)
// (HCA: dense over all compressed entries), and 一(三)3 (RMSNorm of query heads and
// KV entries; RoPE on the last dims of queries, entries and outputs, the output
// rotated at -t; the uncompressed sliding window; a per-head sink logit added to
// the softmax denominator).
//
// BF16 path (MFMA).  A workgroup of 4 waves serves one query row, one part of
// its entry list and 16 heads; wave w owns a quarter of the c dims.  The rows of
// up to 128 slots are fetched at once by direct global-to-LDS loads into one
// entry-major LDS tile (the A operand of S^T = E Q^T; the B operand of O = P E
// comes from the same tile through the gfx950 transpose read), so a part costs
// one gather latency.  Each wave forms a partial S^T over its dims; the four
// partials are summed through LDS in a fixed order, so every wave holds the same
// logits.  RMSNorm is factored as a per-entry scalar r_e and a
// per-query scalar r_q applied to the float32 logits, so the non-RoPE dims of q
// and e enter the MFMA as their exact bf16 input bits; only the rotated RoPE dims
// (and gains, if given) are rounded to bf16.  With S^T in the MFMA output layout
// each lane holds one head's logits for 8 entries, so the online softmax needs
// only in-lane work plus two cross-group shuffles, and the probabilities
// (times r_e) are already in the A-operand layout of the PV MFMA.
//
// Decode (T = 1) splits each query's slot list into at most 16 parts at fixed
// boundaries (a length that depends only on the list length) and merges the
// parts in a fixed order in a second kernel; prefill (T > 1) runs one part per
// query and finishes in place.
//
// F32 path (VALU): one workgroup per (query row, head group), waves take entries
// round-robin with their own online softmax and are merged in a fixed order.
#include <utility>

#include "csa_common.h"
#include "csa_internal.h"

namespace {

constexpr int kTile = 32;            // entry slots per staged tile
constexpr int kSplitSlots = 128;     // decode split length (slots)
constexpr float kLog2e = 1.4426950408889634f;
// the running maximum moves (and the accumulators are rescaled) only once a tile's logit exceeds it by
// this much (base-2 units), so later tiles rarely rescale; probabilities stay below 2^8
constexpr float kLazyMax = 8.0f;

struct AttnArgs {
  const uint16_t* q;
  const uint16_t* comp;
  const int32_t* idx;
  const uint16_t* win;
  const float* sink;
  const float* gamma_q;
  const float* gamma_kv;
  const int64_t* pos0;
  void* out;
  uint16_t* ws_o;  // [rows][nsplit][H][C] fp16: each part's output divided by its denominator
  float* ws_ml;    // [rows][nsplit][H][2]
  int T, H, R, k, n_win, m, out_t, mode, nsplit;
  int prepared;           // 0 raw rows; 1 compressed entries stored prepared; 2 window rows prepared too
  const float* comp_scale;  // comp_mixed: the compressed rows' fp8 scales [B][n_max]
  int comp_mixed;           // compressed rows in CSA_FP8_BF16_ROPE (c + R bytes), widened to bf16 in LDS
  const int32_t* table;     // paged: entry s of sequence b is pool row table[b * tstride + (s >> plog2)]
  int tstride, plog2;       //   << plog2 | (s & (2^plog2 - 1)); the window rows are a ring [B][n_win][c]
  int ns_c, s_c, s_w;     // split layout: ns_c compressed parts of s_c slots, then window parts of s_w
  int64_t n_max;
  float scale, eps;
};

struct Slot {
  int64_t row;   // row index into comp (or window) array, -1 = empty
  bool is_win;
  double pos;
};

// The CSA index-list value of a slot of query (b, r), or 0 where no list value is read (HCA, window
// slots, slots past the part's end).  Loaded apart from the slot's resolution so that it can be fetched
// a stage ahead.
CSA_DEV int32_t slot_idx(const AttnArgs& a, int b, int r, int64_t slot, int64_t slot_hi) {
  return (a.mode == 0 && slot < slot_hi && slot < a.k) ? a.idx[((int64_t)b * a.T + r) * a.k + slot] : 0;
}

// slot j of query (b, r) at position t: CSA = idx slots then window; HCA = dense range then window.
// e_idx is the slot's index-list value (slot_idx) for CSA.
CSA_DEV Slot resolve_slot(const AttnArgs& a, int r, int64_t t, int64_t vis, int64_t slot, int32_t e_idx) {
  Slot s;
  s.is_win = false;
  s.row = -1;
  s.pos = 0.0;
  const int64_t ncomp = (a.mode == 0) ? a.k : a.n_max;
  if (slot < ncomp) {
    int64_t e;
    if (a.mode == 0) {
      e = e_idx;
      if (e < 0 || e >= a.n_max) return s;
    } else {
      e = slot;
      if (e >= vis) return s;
    }
    s.row = e;
    s.pos = (double)a.m * (double)e;
    return s;
  }
  const int64_t w = slot - ncomp;
  if (w >= a.n_win) return s;
  const int64_t p = t - a.n_win + 1 + w;
  if (p < 0) return s;
  s.is_win = true;
  s.row = r + w;
  s.pos = (double)p;
  return s;
}

CSA_DEV float bf(uint32_t word, int hi) { return __uint_as_float(hi ? (word & 0xFFFF0000u) : (word << 16)); }

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));

// LDS transpose read (gfx950): inside each 16-lane group, lane 4r+c supplies the
// address of 4 consecutive bf16 of "row" r; lane i receives column i of the 4x16
// block, i.e. element (i & 3) of lane 4r + (i >> 2)'s chunk, for r = 0..3.
CSA_DEV i16x4 lds_read_tr16(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p));
}

// LDS byte address of a pointer into dynamic shared memory
CSA_DEV uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// The batched LDS reads below are written as asm blocks that wait for their own reads before they end,
// so no read is in flight outside the block; the outputs are early-clobber, so that no output register
// can share an address register that a later read of the block still uses.  They are kept out of the
// compiler's sight on purpose: for the builtin transpose read the compiler first waits for every
// outstanding global-to-LDS fetch, which would stall on the next stage's prefetch.
//
// Sixteen transpose reads: rows lo / hi of eight base addresses (dims tiles 8J .. 8J + 7).
template <int OFF_LO, int OFF_HI>
CSA_DEV void lds_read_tr16_x16(i16x4 (&o)[16], const uint32_t (&a)[8]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %16 offset:%24\n\t"
      "ds_read_b64_tr_b16 %1, %16 offset:%25\n\t"
      "ds_read_b64_tr_b16 %2, %17 offset:%24\n\t"
      "ds_read_b64_tr_b16 %3, %17 offset:%25\n\t"
      "ds_read_b64_tr_b16 %4, %18 offset:%24\n\t"
      "ds_read_b64_tr_b16 %5, %18 offset:%25\n\t"
      "ds_read_b64_tr_b16 %6, %19 offset:%24\n\t"
      "ds_read_b64_tr_b16 %7, %19 offset:%25\n\t"
      "ds_read_b64_tr_b16 %8, %20 offset:%24\n\t"
      "ds_read_b64_tr_b16 %9, %20 offset:%25\n\t"
      "ds_read_b64_tr_b16 %10, %21 offset:%24\n\t"
      "ds_read_b64_tr_b16 %11, %21 offset:%25\n\t"
      "ds_read_b64_tr_b16 %12, %22 offset:%24\n\t"
      "ds_read_b64_tr_b16 %13, %22 offset:%25\n\t"
      "ds_read_b64_tr_b16 %14, %23 offset:%24\n\t"
      "ds_read_b64_tr_b16 %15, %23 offset:%25\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3]), "=&v"(o[4]), "=&v"(o[5]), "=&v"(o[6]), "=&v"(o[7]),
        "=&v"(o[8]), "=&v"(o[9]), "=&v"(o[10]), "=&v"(o[11]), "=&v"(o[12]), "=&v"(o[13]), "=&v"(o[14]), "=&v"(o[15])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7]), "i"(OFF_LO),
        "i"(OFF_HI)
      : "memory");
}

// Eight 16-byte reads, o[4j + v] at a[v] + OFF_j, in one block that waits for them.
template <int OFF0, int OFF1>
CSA_DEV void lds_read_b128_x8(u32x4 (&o)[8], const uint32_t (&a)[4]) {
  asm volatile(
      "ds_read_b128 %0, %8 offset:%12\n\t"
      "ds_read_b128 %1, %9 offset:%12\n\t"
      "ds_read_b128 %2, %10 offset:%12\n\t"
      "ds_read_b128 %3, %11 offset:%12\n\t"
      "ds_read_b128 %4, %8 offset:%13\n\t"
      "ds_read_b128 %5, %9 offset:%13\n\t"
      "ds_read_b128 %6, %10 offset:%13\n\t"
      "ds_read_b128 %7, %11 offset:%13\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3]), "=&v"(o[4]), "=&v"(o[5]), "=&v"(o[6]), "=&v"(o[7])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "i"(OFF0), "i"(OFF1)
      : "memory");
}

// Sixteen 16-byte reads, o[8n + 4j + v] at a[4n + v] + OFF_j (two sets of four bases), in one block that
// waits for them.
template <int OFF0, int OFF1>
CSA_DEV void lds_read_b128_x16(u32x4 (&o)[16], const uint32_t (&a)[8]) {
  asm volatile(
      "ds_read_b128 %0, %16 offset:%24\n\t"
      "ds_read_b128 %1, %17 offset:%24\n\t"
      "ds_read_b128 %2, %18 offset:%24\n\t"
      "ds_read_b128 %3, %19 offset:%24\n\t"
      "ds_read_b128 %4, %16 offset:%25\n\t"
      "ds_read_b128 %5, %17 offset:%25\n\t"
      "ds_read_b128 %6, %18 offset:%25\n\t"
      "ds_read_b128 %7, %19 offset:%25\n\t"
      "ds_read_b128 %8, %20 offset:%24\n\t"
      "ds_read_b128 %9, %21 offset:%24\n\t"
      "ds_read_b128 %10, %22 offset:%24\n\t"
      "ds_read_b128 %11, %23 offset:%24\n\t"
      "ds_read_b128 %12, %20 offset:%25\n\t"
      "ds_read_b128 %13, %21 offset:%25\n\t"
      "ds_read_b128 %14, %22 offset:%25\n\t"
      "ds_read_b128 %15, %23 offset:%25\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3]), "=&v"(o[4]), "=&v"(o[5]), "=&v"(o[6]), "=&v"(o[7]),
        "=&v"(o[8]), "=&v"(o[9]), "=&v"(o[10]), "=&v"(o[11]), "=&v"(o[12]), "=&v"(o[13]), "=&v"(o[14]), "=&v"(o[15])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7]), "i"(OFF0), "i"(OFF1)
      : "memory");
}

// Four 16-byte reads, o[v] at a[v] + OFF0.
template <int OFF0>
CSA_DEV void lds_read_b128_x4(u32x4 (&o)[4], const uint32_t (&a)[4]) {
  asm volatile(
      "ds_read_b128 %0, %4 offset:%8\n\t"
      "ds_read_b128 %1, %5 offset:%8\n\t"
      "ds_read_b128 %2, %6 offset:%8\n\t"
      "ds_read_b128 %3, %7 offset:%8\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "i"(OFF0)
      : "memory");
}

// Reductions over the lane pairs (l, l ^ 16) and (l, l ^ 32) with the gfx950 lane-swap instructions (VALU,
// no LDS round trip); both lanes of a pair get the same value
CSA_DEV float pair16_max(float v) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
CSA_DEV float pair32_max(float v) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
CSA_DEV float pair16_sum(float v) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
CSA_DEV float pair32_sum(float v) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

template <typename F, int... I>
CSA_DEV void static_for_impl(F& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
// f(integral_constant<int, i>) for i = 0 .. N-1, unrolled at compile time
template <int N, typename F>
CSA_DEV void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Entry-major LDS rows of C bf16 without padding; 16-byte chunk c of row e is stored at
// chunk position c ^ swz_key(e & 15), which spreads the rows an MFMA operand read touches
// over the LDS banks.
CSA_DEV constexpr int swz_key(int e) { return e & 15; }
template <int C>
CSA_DEV int swz(int e, int c) { return c ^ swz_key(e & 15); }

constexpr int kStage = 64;  // slots fetched into LDS at once (2 compute tiles)

// Bytes of the attention kernel's per-slot control arrays in LDS (in 2-byte units, rounded up to 16 bytes).
template <bool WIDE>
constexpr int lds_ctrl_halfs() {
  constexpr int ne = WIDE ? 2 : 1, nr = WIDE ? 3 : 2;
  constexpr int bytes = 64 * 8 + nr * kStage * (8 + 8 + 8) + (kStage + 64) * 4 + nr * kStage * 4 + 3 * kStage * 4 +
                        ne * kStage * 4 + 2 * nr * 4 + 64 * 8;
  return ((bytes + 15) / 16) * 8;
}

// One workgroup = one query row x one part of its slot list x 16 heads; wave w owns dims
// [w*C/4, (w+1)*C/4).  Per stage: (1) resolve 64 slots (row address, position, validity),
// (2) DMA every row straight into LDS (global_load_lds, 16 B per lane, no registers),
// (3) per-entry RMS scalar and RoPE in place, (4) two 32-slot tiles of MFMA work from LDS.
template <int C, bool WIDE, bool RAW, bool MIX, bool PAGED>
__global__ __launch_bounds__(256) void attend_bf16_kernel(AttnArgs a, RopeTable rt, int nx) {
  // RAW: rows may need RMSNorm / RoPE here (raw compressed entries or raw window rows); without it every
  // row is stored prepared and the kernel has no normalisation or rotation of entries at all
  // narrow: 16 heads per workgroup, wave w owns dims [w C/4, (w+1) C/4) of all 16 (logits summed across
  // waves through LDS); wide: 64 heads per workgroup, wave w owns heads 16w .. 16w+15 over all dims
  constexpr int DW = WIDE ? C : C / 4;  // dims per wave
  constexpr int KSW = DW / 32;  // k-steps of the wave's partial S^T = E Q^T
  constexpr int DTW = DW / 16;  // 16-dim output tiles of the wave
  constexpr int NCR = C / 8;    // 16-byte chunks per row
  constexpr int RPI = 64 / NCR; // rows per DMA instruction
  static_assert(!(WIDE && RAW), "the wide variant reads prepared rows only");
  // the wide variant runs one workgroup per CU (its registers), so it can hold two stages in LDS and
  // fetch stage s + 1 while it computes stage s; slot resolution then runs two stages ahead (3 buffers)
  constexpr int NE = WIDE ? 2 : 1;  // LDS stage buffers
  constexpr int NR = WIDE ? 3 : 2;  // slot-resolution buffers
  // LDS: the per-slot control arrays first (their addresses stay below 64 KB, where LDS instructions take
  // them as immediate offsets), then the narrow variant's logit exchange, then the stage buffers
  extern __shared__ __align__(16) uint16_t s_mem[];
  double* s_theta = reinterpret_cast<double*>(s_mem);                      // [64]
  double* s_pos2 = s_theta + 64;                                           // [NR][kStage]
  const uint16_t** s_src2 = reinterpret_cast<const uint16_t**>(s_pos2 + NR * kStage);  // [NR][kStage]
  const float** s_scp2 = reinterpret_cast<const float**>(s_src2 + NR * kStage);       // [NR][kStage]
  float* s_re = reinterpret_cast<float*>(s_scp2 + NR * kStage);            // [kStage]
  float* s_rq = s_re + kStage;                                             // [4][16]
  int* s_flag2 = reinterpret_cast<int*>(s_rq + 64);                        // [NR][kStage] 1 valid | 2 raw | 4 mixed
  int* s_idx3 = s_flag2 + NR * kStage;  // [3][kStage] (wide, CSA) index-list values, fetched two stages ahead
  float* s_scale = reinterpret_cast<float*>(s_idx3 + 3 * kStage);          // [NE][kStage] mixed rows' fp8 scales
  int* s_raw2 = reinterpret_cast<int*>(s_scale + NE * kStage);             // [NR] stage holds a raw row
  int* s_mix2 = s_raw2 + NR;                                               // [NR] stage holds mixed rows
  float2* s_qcs = reinterpret_cast<float2*>(s_mix2 + NR);                  // [64] the query's RoPE cos, sin
  f32x4* s_part = reinterpret_cast<f32x4*>(s_mem + lds_ctrl_halfs<WIDE>());  // [4 waves][2][64 lanes] (narrow)
  uint16_t* E0 = reinterpret_cast<uint16_t*>(s_part + (WIDE ? 0 : 4 * 2 * 64));  // [NE][kStage][C]

  if ((int)blockIdx.x >= nx) return;  // grid.x is padded to a multiple of 8 (XCD-aligned head groups)
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g = lane >> 4;
  const int sp = blockIdx.x % a.nsplit;
  const int row = blockIdx.x / a.nsplit;
  const int b = row / a.T;
  const int r = row - b * a.T;
  const int h0 = blockIdx.y * (WIDE ? 64 : 16) + (WIDE ? 16 * wave : 0);  // first head of this wave
  const int head = h0 + (lane & 15);
  const int rope_lo = C - a.R;
  const int64_t nslots = ((a.mode == 0) ? a.k : a.n_max) + a.n_win;
  const int64_t ncomp = (a.mode == 0) ? a.k : a.n_max;
  int64_t slot_lo, slot_hi;
  if (sp < a.ns_c) {  // a part of the compressed slots (or, with one part per query, of all slots)
    slot_lo = (int64_t)sp * a.s_c;
    slot_hi = min(slot_lo + a.s_c, a.nsplit > a.ns_c ? ncomp : nslots);
  } else {            // a part of the window slots
    slot_lo = ncomp + (int64_t)(sp - a.ns_c) * a.s_w;
    slot_hi = min(slot_lo + a.s_w, nslots);
  }
  const int dbase = WIDE ? 0 : wave * DW;
  const uint16_t* dummy = a.win + (int64_t)b * (a.T + a.n_win - 1) * C;  // a finite row for empty slots
  // this wave's raw query fragments and the first stage's index-list values go out first: they depend on
  // nothing (the position's load and wait come after them)
  // The position is read by a vector load issued before them (its offset, zero, is hidden from the
  // compiler, which would otherwise make it a scalar load and wait for it before issuing the others).
  int zoff = 0;
  asm volatile("" : "+v"(zoff));
  // RoPE frequency of this thread (lane l of each wave: theta_l), loaded with them
  const double th_l = rt.theta[lane];
  const int64_t p0v = a.pos0[b + zoff];
  const uint16_t* qrow = a.q + ((int64_t)row * a.H + head) * C + dbase;
  u32x4 qraw[KSW];
#pragma unroll
  for (int ks = 0; ks < KSW; ++ks) qraw[ks] = *reinterpret_cast<const u32x4*>(qrow + 32 * ks + 8 * g);
  // (every lane loads, from an in-bounds address also where the value is unused, so that no branch makes
  // the compiler wait for the load where the paths join)
  const int64_t slot0 = slot_lo + (threadIdx.x & (kStage - 1));
  const int32_t idx_raw = *(a.mode == 0 ? a.idx + ((int64_t)b * a.T + r) * a.k + min(slot0, (int64_t)a.k - 1)
                                        : reinterpret_cast<const int32_t*>(a.pos0));
  const int64_t t = (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(p0v >> 32)) << 32) |
                              (uint32_t)__builtin_amdgcn_readfirstlane((int)p0v)) + r;
  const int64_t vis = visible_entries(t, a.m, a.n_max);
  const double tpos = (double)t;
  if (threadIdx.x < 64) s_theta[threadIdx.x] = th_l;
  // the query's rotation at t, once per RoPE pair for every head (wave 1, idle while wave 0 resolves slots)
  if (threadIdx.x >= 64 && threadIdx.x < 64 + a.R / 2) {
    float cs, sn;
    rope_cs(tpos, th_l, cs, sn);
    s_qcs[threadIdx.x - 64] = float2{cs, sn};
  }
  // slot resolution of a stage into buffer h of the resolve arrays, from the slots' index-list values
  // (threads < kStage, i.e. all of wave 0)
  auto commit_stage = [&](int64_t st0, int h, int32_t e_idx) {
    {
      const int64_t slot = st0 + threadIdx.x;
      Slot sl;
      sl.row = -1;
      if (slot < slot_hi) sl = resolve_slot(a, r, t, vis, slot, e_idx);
      const bool valid = sl.row >= 0;
      // compressed rows in the mixed format: c + R bytes each, and their scale
      const bool mixed = MIX && valid && !sl.is_win;
      int64_t crow = (int64_t)b * a.n_max + sl.row;
      if constexpr (PAGED) {  // pool row of the entry (its page looked up in the block table)
        crow = 0;
        if (valid && !sl.is_win)
          crow = ((int64_t)a.table[(int64_t)b * a.tstride + (sl.row >> a.plog2)] << a.plog2) |
                 (sl.row & (((int64_t)1 << a.plog2) - 1));
      }
      // window row: position p of the query's window; paged calls keep the window in a ring (p % n_win)
      const int64_t wrow = PAGED ? (int64_t)b * a.n_win + (int64_t)sl.pos % a.n_win
                                 : (int64_t)b * (a.T + a.n_win - 1) + sl.row;
      const uint16_t* cptr = mixed ? reinterpret_cast<const uint16_t*>(reinterpret_cast<const uint8_t*>(a.comp) +
                                                                       crow * (C + a.R))
                                   : a.comp + crow * C;
      // (a mixed row's address carries a 1 in bit 0: its rows start on 16-byte boundaries)
      s_src2[h * kStage + threadIdx.x] =
          valid ? (sl.is_win ? a.win + wrow * C
                             : reinterpret_cast<const uint16_t*>(reinterpret_cast<uintptr_t>(cptr) | (mixed ? 1u : 0u)))
                : dummy;
      if (MIX) s_scp2[h * kStage + threadIdx.x] = mixed ? a.comp_scale + crow : a.sink;  // (readable when unused)
      s_pos2[h * kStage + threadIdx.x] = sl.pos;
      // raw rows (window tokens, or compressed entries not stored prepared) get RMSNorm and RoPE here
      const bool raw = RAW && valid && (sl.is_win ? a.prepared < 2 : a.prepared == 0);
      s_flag2[h * kStage + threadIdx.x] = valid ? ((raw ? 3 : 1) | (mixed ? 4 : 0)) : 0;
      const uint64_t rm = __ballot(raw);  // threads < kStage are exactly wave 0
      const uint64_t mm = MIX ? __ballot(mixed) : 0;
      if (threadIdx.x == 0) {
        s_raw2[h] = rm != 0;
        if (MIX) s_mix2[h] = mm != 0;
      }
    }
  };
  auto resolve_stage = [&](int64_t st0, int h) {
    if (threadIdx.x < kStage) commit_stage(st0, h, slot_idx(a, b, r, st0 + threadIdx.x, slot_hi));
  };
  if (threadIdx.x < kStage) commit_stage(slot_lo, 0, (a.mode == 0 && slot0 < slot_hi && slot0 < a.k) ? idx_raw : 0);
  // DMA of a stage's rows into E: instruction j of wave w fills rows RPI*(w + 4j) .. +RPI-1; lane l
  // writes LDS chunk position (l % NCR) of row e = RPI*(w + 4j) + l / NCR, so it loads the logical
  // chunk stored there
  // The wave's 16 row addresses are read from LDS at once (lane l % 16 holds that of row
  // RPI (wave + 4 (l / RPI)) + l % RPI) and handed to each instruction's lanes by a lane read.
  // A mixed row (CSA_FP8_BF16_ROPE, bit 0 of its address set) arrives as: its bf16 RoPE chunks at their
  // own positions, and each 16-code chunk of its fp8 part at the positions of both bf16 chunks it widens
  // into (the widening pass reads the first and overwrites both).  Its scale travels by one more
  // 4-byte-per-lane load of wave 0 (lane i -> slot i).
  auto issue_dma = [&](int h, int eb) {
    const uint16_t* const* src_rows = s_src2 + h * kStage;
    uint16_t* E = E0 + eb * kStage * C;
    const bool mix = MIX && s_mix2[h] != 0;  // (uniform)
    const int l16 = lane & 15;
    const int myrow = RPI * (wave + 4 * (l16 / RPI)) + l16 % RPI;
    const uint64_t mine = reinterpret_cast<uint64_t>(src_rows[myrow]);
    const int mlo = (int)(uint32_t)mine, mhi = (int)(uint32_t)(mine >> 32);
    const int nfpc = (C - a.R) >> 3;  // bf16 chunks of the fp8 part
    // (LDS reads come before this call's first load to LDS, so none of them waits for those loads)
    if (mix && wave == 0)
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)s_scp2[h * kStage + lane],
                                       (__attribute__((address_space(3))) void*)(s_scale + eb * kStage), 4, 0, 0);
#pragma unroll
    for (int j = 0; j < kStage / RPI / 4; ++j) {
      const int e0 = RPI * (wave + 4 * j);
      const int e = e0 + lane / NCR;
      const int cpos = lane % NCR;
      uint32_t rlo, rhi;
      if constexpr (RPI == 1) {  // one row per instruction: a wave-uniform address
        rlo = (uint32_t)__builtin_amdgcn_readlane(mlo, j);
        rhi = (uint32_t)__builtin_amdgcn_readlane(mhi, j);
      } else {
        const int srcl = j * RPI + lane / NCR;  // the lane that holds row e's address
        rlo = (uint32_t)__shfl(mlo, srcl, 64);
        rhi = (uint32_t)__shfl(mhi, srcl, 64);
      }
      const int L = swz<C>(e, cpos);  // logical bf16 chunk held at this position
      int off = 16 * L;
      if (MIX && (rlo & 1u))
        off = L >= nfpc ? (C - a.R) + 16 * (L - nfpc)  // a RoPE chunk
                        : 8 * (L & ~1);                // the 16 codes of chunks L & ~1 and (L & ~1) + 1
      const uint8_t* rowb = reinterpret_cast<const uint8_t*>(((uint64_t)rhi << 32) | (rlo & ~1u));
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(rowb + off),
                                       (__attribute__((address_space(3))) void*)(E + e0 * C), 16, 0, 0);
    }
  };
  // Widening of a stage's mixed rows in place: each 16-code chunk becomes two bf16 chunks (code times the
  // row's scale, rounded to nearest even), read from the position of the first and written to both.  Lane
  // l serves row l, wave w its code chunks w + 4i; all of a lane's loads go out before its first
  // conversion.  No LDS load is in flight meanwhile.
  auto widen_stage = [&](int h, int eb) {
    constexpr int MAXI = C / 64;             // code chunks per wave when R = 0
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    const int ncc = (C - a.R) >> 4;          // code chunks per row
    const int e = lane;
    if (!(s_flag2[h * kStage + e] & 4)) return;
    const float sc = s_scale[eb * kStage + e];
    uint16_t* rowp = E0 + (eb * kStage + e) * C;
    u32x4 w[MAXI];
#pragma unroll
    for (int i = 0; i < MAXI; ++i)
      if (wv + 4 * i < ncc) w[i] = *reinterpret_cast<const u32x4*>(rowp + 8 * swz<C>(e, 2 * (wv + 4 * i)));
#pragma unroll
    for (int i = 0; i < MAXI; ++i) {
      const int j = wv + 4 * i;
      if (j >= ncc) break;
      uint32_t o[8];
#pragma unroll
      for (int q = 0; q < 4; ++q) {  // codes 4q .. 4q + 3: exact float32 (OCP e4m3), times the scale
        const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(w[i][q], false);
        const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(w[i][q], true);
        o[2 * q] = pack_bf16x2(lo[0] * sc, lo[1] * sc);
        o[2 * q + 1] = pack_bf16x2(hi[0] * sc, hi[1] * sc);
      }
      *reinterpret_cast<u32x4*>(rowp + 8 * swz<C>(e, 2 * j)) = u32x4{o[0], o[1], o[2], o[3]};
      *reinterpret_cast<u32x4*>(rowp + 8 * swz<C>(e, 2 * j + 1)) = u32x4{o[4], o[5], o[6], o[7]};
    }
  };
  __syncthreads();  // s_theta and the first stage's slots visible
  issue_dma(0, 0);  // the first stage's rows land while the query is prepared
  // wide, CSA: the index-list values of a later stage travel like the rows, straight into LDS (wave 0,
  // lane i -> slot st0 + i, clamped into the list), so that no register load is pending across the
  // stage's compute
  auto fetch_idx = [&](int64_t st0, int buf) {
    if (a.mode == 0 && wave == 0 && st0 < a.k) {
      const int64_t slot = min(st0 + lane, (int64_t)a.k - 1);
      __builtin_amdgcn_global_load_lds(
          (const __attribute__((address_space(1))) void*)(a.idx + ((int64_t)b * a.T + r) * a.k + slot),
          (__attribute__((address_space(3))) void*)(s_idx3 + buf * kStage), 4, 0, 0);
    }
  };
  if (WIDE && slot_lo + kStage < slot_hi) fetch_idx(slot_lo + kStage, 1);

  // ---- query fragment: head lane&15, the wave's dims [dbase + 32ks + 8g, +8)
  bf16x8 qf[KSW];
  float qss;
  {
    u32x4* raw = qraw;
    float ss = 0.0f;
#pragma unroll
    for (int ks = 0; ks < KSW; ++ks) {
#pragma unroll
      for (int j = 0; j < 4; ++j) ss = sumsq_bf16x2(raw[ks][j], ss);
    }
    ss += __shfl_xor(ss, 16, 64);
    ss += __shfl_xor(ss, 32, 64);
    if (!WIDE && g == 0) s_rq[wave * 16 + (lane & 15)] = ss;  // a wide wave holds the whole sum
    qss = ss;
#pragma unroll
    for (int ks = 0; ks < KSW; ++ks) {
      const int d0 = dbase + 32 * ks + 8 * g;
      if (d0 >= rope_lo || a.gamma_q || (a.gamma_kv && !a.prepared)) {
        float x[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) { x[2 * j] = bf(raw[ks][j], 0); x[2 * j + 1] = bf(raw[ks][j], 1); }
        if (a.gamma_q) {
#pragma unroll
          for (int j = 0; j < 8; ++j) x[j] *= a.gamma_q[d0 + j];
        }
        if (d0 >= rope_lo) {
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            const float2 qcs = s_qcs[(d0 - rope_lo) / 2 + p];
            const float cs = qcs.x, sn = qcs.y;
            const float x0 = x[2 * p], x1 = x[2 * p + 1];
            x[2 * p] = x0 * cs - x1 * sn;
            x[2 * p + 1] = x0 * sn + x1 * cs;
          }
        } else if (a.gamma_kv && !a.prepared) {  // raw entries' gain on the non-RoPE dims, moved to q
#pragma unroll
          for (int j = 0; j < 8; ++j) x[j] *= a.gamma_kv[d0 + j];
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) raw[ks][j] = pack_bf16x2(x[2 * j], x[2 * j + 1]);
      }
      qf[ks] = __builtin_bit_cast(bf16x8, raw[ks]);
    }
  }

  f32x4 O[DTW];
#pragma unroll
  for (int d = 0; d < DTW; ++d) O[d] = f32x4{0.f, 0.f, 0.f, 0.f};
  float M = -INFINITY, L = 0.0f;  // running max / denominator of head lane&15 (base-2 units)
  // logits are kept in base-2 units (times log2 e) so that exponentials are single v_exp_f32; the narrow
  // variant sets the factor once the four waves' partial query norms are in s_rq
  float zmul = WIDE ? kLog2e * a.scale / sqrtf(qss / (float)C + a.eps) : 0.0f;

  // Wide variant: LDS offsets of this lane's operand reads, so that every read in a tile is one of a few
  // per-lane bases plus an immediate (the swizzle key of an entry depends on its index mod 16 only, and
  // eb + 16 nt is a multiple of 16).  QK (A operand): entry eb + 16nt + l (l = lane & 15), 16-byte chunk
  // 4ks + g, whose swizzled position splits as 16 (ks >> 2) + ((4 (ks & 3) + g) ^ key(l)).  PV (transpose
  // reads): entry eb + 4g + tr_r (+16), dims 16dt + 4tr_c .. +3, i.e. chunk 2dt + (tr_c >> 1) at swizzled
  // position 16 (dt >> 3) + ((2 (dt & 7) + (tr_c >> 1)) ^ key(4g + tr_r)).
  int qoff[4];        // elements, v = ks & 3
  uint32_t toff[8];   // bytes, u = dt & 7
  if constexpr (WIDE) {
    const int l = lane & 15, tr_r = l >> 2, tr_c = lane & 3, x = 4 * g + tr_r;
#pragma unroll
    for (int v = 0; v < 4; ++v) qoff[v] = l * C + 8 * ((4 * v + g) ^ swz_key(l));
#pragma unroll
    for (int u = 0; u < 8; ++u)
      toff[u] = 2u * (uint32_t)(x * C + 8 * ((2 * u + (tr_c >> 1)) ^ swz_key(x)) + 4 * (tr_c & 1));
  }

  // ---- (4) the compute tiles of 32 slots of a stage held in E (slot flags in s_flag)
  auto compute_stage = [&](const uint16_t* E, int64_t s0, const int* s_flag) {
    const int ntile = (int)min((int64_t)kStage / kTile, (slot_hi - s0 + kTile - 1) / kTile);
#pragma unroll 1
    for (int tl = 0; tl < ntile; ++tl) {
      const int eb = kTile * tl;
      // wide: byte addresses of this tile's operand reads (entries eb + 16 nt + (lane & 15) for QK)
      uint32_t qb[2][4];
      uint32_t ebase = 0;
      if constexpr (WIDE) {
        ebase = lds_addr(E) + (uint32_t)(eb * C * 2);
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
          for (int v = 0; v < 4; ++v) qb[nt][v] = ebase + (uint32_t)(nt * 32 * C + 2 * qoff[v]);
      }
      // S^T over the wave's dims: lane holds entries eb + 16nt + 4g + i, head lane&15
      f32x4 accs[2];
      // narrow, c = 512: the tile's 8 operand chunks of this lane (entries eb + (lane & 15) and + 16, k-steps
      // 0..3; both entries share a swizzle key) in one batched read, then two independent MFMA chains
      constexpr bool kBatchQK = !WIDE && KSW == 4;
      u32x4 qkrd[kBatchQK ? 8 : 1];
      if constexpr (kBatchQK) {
        const int e = eb + (lane & 15);
        uint32_t qa[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) qa[v] = lds_addr(E + e * C + 8 * swz<C>(e, (dbase + 32 * v + 8 * g) >> 3));
        lds_read_b128_x8<0, 32 * C>(qkrd, qa);
      }
      if constexpr (WIDE && KSW >= 8) {
        // both 16-entry halves of the tile at once: batches of 8 k-steps, ks = 8 BI + 4 j + v at qb[nt][v] +
        // 256 (2 BI + j) bytes, 16 reads per batch, and the halves' two MFMA chains interleaved (each MFMA
        // waits for its predecessor in the chain, so one chain alone leaves the matrix core idle in between)
        f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
        const uint32_t qb01[8] = {qb[0][0], qb[0][1], qb[0][2], qb[0][3], qb[1][0], qb[1][1], qb[1][2], qb[1][3]};
        static_for<KSW / 8>([&](auto bc) {
          constexpr int BI = decltype(bc)::value;
          u32x4 rd[16];
          lds_read_b128_x16<512 * BI, 512 * BI + 256>(rd, qb01);
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, rd[q]), qf[8 * BI + q], acc0,
                                                           0, 0, 0);
            acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, rd[8 + q]), qf[8 * BI + q], acc1,
                                                           0, 0, 0);
          }
        });
        accs[0] = acc0;
        accs[1] = acc1;
      }
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        if constexpr (WIDE && KSW >= 8) {
          // (both halves computed above)
        } else if constexpr (WIDE) {  // c = 128: the 4 k-steps in one batch of reads
          u32x4 rd[4];
          lds_read_b128_x4<0>(rd, qb[nt]);
#pragma unroll
          for (int q = 0; q < 4; ++q)
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, rd[q]), qf[q], acc, 0, 0, 0);
          accs[nt] = acc;
        } else if constexpr (kBatchQK) {
#pragma unroll
          for (int ks = 0; ks < KSW; ++ks)
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, qkrd[4 * nt + ks]), qf[ks], acc,
                                                          0, 0, 0);
          s_part[(wave * 2 + nt) * 64 + lane] = acc;
        } else {
          const int e = eb + 16 * nt + (lane & 15);
          const uint16_t* er = E + e * C;
#pragma unroll
          for (int ks = 0; ks < KSW; ++ks) {
            const int c = (dbase + 32 * ks + 8 * g) >> 3;
            const bf16x8 ef = *reinterpret_cast<const bf16x8*>(er + 8 * swz<C>(e, c));
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ef, qf[ks], acc, 0, 0, 0);
          }
          s_part[(wave * 2 + nt) * 64 + lane] = acc;
        }
      }
      if (!WIDE) __syncthreads();
      float z[8], re[8];
      float tmax = -INFINITY;
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        f32x4 sum;
        if (WIDE) {
          sum = accs[nt];
        } else {  // the four waves' partial logits, summed in a fixed order
          sum = s_part[(0 * 2 + nt) * 64 + lane];
#pragma unroll
          for (int w = 1; w < 4; ++w) {
            const f32x4 pw = s_part[(w * 2 + nt) * 64 + lane];
            sum[0] += pw[0]; sum[1] += pw[1]; sum[2] += pw[2]; sum[3] += pw[3];
          }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float rv = WIDE ? (s_flag[eb + 16 * nt + 4 * g + i] ? 1.0f : 0.0f) : s_re[eb + 16 * nt + 4 * g + i];
          re[4 * nt + i] = rv;
          const float zz = rv > 0.0f ? sum[i] * zmul * rv : -INFINITY;
          z[4 * nt + i] = zz;
          tmax = fmaxf(tmax, zz);
        }
      }
      tmax = pair32_max(pair16_max(tmax));
      // lazy running maximum: moved (with O and L rescaled) only when some head of the wave has a logit
      // more than kLazyMax above its current one; a first finite logit always moves it
      if (__any(tmax > M + kLazyMax)) {
        const float Mn = fmaxf(M, tmax);
        const float alpha = Mn == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(M - Mn);
        L *= alpha;
        M = Mn;
        float al[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) al[i] = __shfl(alpha, 4 * g + i, 64);
#pragma unroll
        for (int dt = 0; dt < DTW; ++dt) {
          O[dt][0] *= al[0]; O[dt][1] *= al[1]; O[dt][2] *= al[2]; O[dt][3] *= al[3];
        }
      }
      const bool live = M != -INFINITY;
      float psum = 0.0f;
      uint32_t pw[4];
#pragma unroll
      for (int j = 0; j < 8; j += 2) {
        const float p0 = live ? __builtin_amdgcn_exp2f(z[j] - M) : 0.0f;
        const float p1 = live ? __builtin_amdgcn_exp2f(z[j + 1] - M) : 0.0f;
        psum += p0 + p1;
        pw[j / 2] = pack_bf16x2(p0 * re[j], p1 * re[j + 1]);
      }
      psum = pair32_sum(pair16_sum(psum));
      L += psum;
      const bf16x8 pf = __builtin_bit_cast(bf16x8, u32x4{pw[0], pw[1], pw[2], pw[3]});
      // O += P E over the wave's dims; B operand by transpose reads of the entry-major rows
      if constexpr (WIDE) {
        uint32_t tb[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) tb[u] = ebase + toff[u];
        // batches of 8 output tiles: dt = 8J + u, u = 0..7
        static_for<DTW / 8>([&](auto bc) {
          constexpr int J = decltype(bc)::value;
          i16x4 rd[16];
          lds_read_tr16_x16<256 * J, 256 * J + 32 * C>(rd, tb);
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const i16x4 lo = rd[2 * u], hi = rd[2 * u + 1];
            const bf16x8 ef =
                __builtin_bit_cast(bf16x8, (i16x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
            O[8 * J + u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pf, ef, O[8 * J + u], 0, 0, 0);
          }
        });
      } else if constexpr (DTW == 8) {  // c = 512: the 16 transpose reads of the tile in one batch
        const int tr_r = (lane & 15) >> 2, tr_c = lane & 3;
        const int e_lo = eb + 4 * g + tr_r;  // rows e_lo and e_lo + 16 share a swizzle key
        uint32_t ta[8];
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
          const int hw = dbase + 16 * dt + 4 * tr_c;
          ta[dt] = lds_addr(E + e_lo * C + 8 * swz<C>(e_lo, hw >> 3) + (hw & 7));
        }
        i16x4 rd[16];
        lds_read_tr16_x16<0, 32 * C>(rd, ta);
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
          const i16x4 lo = rd[2 * dt], hi = rd[2 * dt + 1];
          const bf16x8 ef =
              __builtin_bit_cast(bf16x8, (i16x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
          O[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pf, ef, O[dt], 0, 0, 0);
        }
        __syncthreads();  // s_part is rewritten by the next tile; E and the resolve buffer by the next stage
      } else {
        const int tr_r = (lane & 15) >> 2, tr_c = lane & 3;
        const int e_lo = eb + 4 * g + tr_r, e_hi = e_lo + 16;
#pragma unroll
        for (int dt = 0; dt < DTW; ++dt) {
          const int hw = dbase + 16 * dt + 4 * tr_c;  // first of the 4 halfwords this lane addresses
          const i16x4 lo = lds_read_tr16(E + e_lo * C + 8 * swz<C>(e_lo, hw >> 3) + (hw & 7));
          const i16x4 hi = lds_read_tr16(E + e_hi * C + 8 * swz<C>(e_hi, hw >> 3) + (hw & 7));
          const bf16x8 ef =
              __builtin_bit_cast(bf16x8, (i16x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
          O[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pf, ef, O[dt], 0, 0, 0);
        }
        __syncthreads();  // s_part is rewritten by the next tile; E and the resolve buffer by the next stage
      }
    }
  };

  if constexpr (WIDE) {
    // stage st: its rows are in E[st & 1], its slots in resolve buffer st % 3.  One barrier per stage:
    // after it, stage st + 1 is fetched into the other buffer (whose last reader, stage st - 1, is done)
    // and the index-list values of stage st + 2 into s_idx3, while stage st is computed.
    int st = 0;
    for (int64_t s0 = slot_lo; s0 < slot_hi; s0 += kStage, ++st) {
      const bool more = s0 + kStage < slot_hi;
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this stage's rows and the next one's index values
      if (more && threadIdx.x < kStage)
        commit_stage(s0 + kStage, (st + 1) % 3, s_idx3[((st + 1) % 3) * kStage + threadIdx.x]);
      __syncthreads();
      if (MIX && s_mix2[st % 3]) {  // (uniform) before the next stage's loads go out
        widen_stage(st % 3, st & 1);
        __syncthreads();
      }
      if (more) {
        issue_dma((st + 1) % 3, (st + 1) & 1);
        if (s0 + 2 * kStage < slot_hi) fetch_idx(s0 + 2 * kStage, (st + 2) % 3);
      }
      compute_stage(E0 + (st & 1) * kStage * C, s0, s_flag2 + (st % 3) * kStage);
    }
  } else {
    int half = 0;
    for (int64_t s0 = slot_lo; s0 < slot_hi; s0 += kStage, half ^= 1) {
      const double* s_pos = s_pos2 + half * kStage;
      const int* s_flag = s_flag2 + half * kStage;
      // ---- (2) DMA of this stage's rows (the first stage's went out before the query was prepared)
      if (s0 != slot_lo) issue_dma(half, 0);
      // the next stage's slot resolution (index-list loads) overlaps this stage's fetch and compute
      if (s0 + kStage < slot_hi) resolve_stage(s0 + kStage, half ^ 1);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      if (MIX && s_mix2[half]) {
        widen_stage(half, 0);
        __syncthreads();
      }
      if (!WIDE && s0 == slot_lo) {
        zmul = kLog2e * a.scale / sqrtf((s_rq[lane & 15] + s_rq[16 + (lane & 15)] + s_rq[32 + (lane & 15)] +
                                         s_rq[48 + (lane & 15)]) / (float)C + a.eps);
      }
      if (RAW && s_raw2[half]) {
        // ---- (3a) per-entry RMS scalar of the raw rows: 8 lanes per entry, two accumulators
        // (prepared entries are already normalised: scalar 1)
#pragma unroll 1
        for (int rd = 0; rd < kStage / 32; ++rd) {
          const int e = 32 * rd + (threadIdx.x >> 3);
          const int sub = threadIdx.x & 7;
          const int fl = s_flag[e];
          const uint16_t* er = E0 + e * C;
          float ss0 = 0.0f, ss1 = 0.0f;
          if (fl & 2) {
#pragma unroll
            for (int j = 0; j < NCR / 8; ++j) {
              const u32x4 w4 = *reinterpret_cast<const u32x4*>(er + 8 * swz<C>(e, sub + 8 * j));
              ss0 = sumsq_bf16x2(w4[0], ss0);
              ss1 = sumsq_bf16x2(w4[1], ss1);
              ss0 = sumsq_bf16x2(w4[2], ss0);
              ss1 = sumsq_bf16x2(w4[3], ss1);
            }
          }
          float ss = ss0 + ss1;
          ss += __shfl_xor(ss, 1, 64);
          ss += __shfl_xor(ss, 2, 64);
          ss += __shfl_xor(ss, 4, 64);
          if (sub == 0) s_re[e] = (fl & 2) ? 1.0f / sqrtf(ss / (float)C + a.eps) : (fl ? 1.0f : 0.0f);
        }
        // ---- (3b) RoPE (and gain) of the raw rows, in place: items (entry, 4-pair chunk), four
        // independent rotations per item so that their dependent sin/cos chains overlap.  With prepared
        // compressed entries the raw (window) rows also take the gain on their non-RoPE dims here.
        {
          const bool all_dims = a.prepared && a.gamma_kv;
          const int c_lo = all_dims ? 0 : (rope_lo >> 3);
          const int nrc = NCR - c_lo;  // chunks per entry
#pragma unroll 1
          for (int it = threadIdx.x; it < kStage * nrc; it += 256) {
            const int e = it / nrc;
            if (!(s_flag[e] & 2)) continue;
            const int c = c_lo + (it - e * nrc);
            const int d0 = 8 * c;
            u32x4* cp = reinterpret_cast<u32x4*>(E0 + e * C + 8 * swz<C>(e, c));
            u32x4 w4 = *cp;
            const double pos = s_pos[e];
            float x[8];
#pragma unroll
            for (int q = 0; q < 4; ++q) { x[2 * q] = bf(w4[q], 0); x[2 * q + 1] = bf(w4[q], 1); }
            if (a.gamma_kv) {
#pragma unroll
              for (int q = 0; q < 8; ++q) x[q] *= a.gamma_kv[d0 + q];
            }
            if (d0 >= rope_lo) {
#pragma unroll
              for (int p = 0; p < 4; ++p) {
                float cs, sn;
                rope_cs(pos, s_theta[(d0 - rope_lo) / 2 + p], cs, sn);
                const float x0 = x[2 * p], x1 = x[2 * p + 1];
                x[2 * p] = x0 * cs - x1 * sn;
                x[2 * p + 1] = x0 * sn + x1 * cs;
              }
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) w4[q] = pack_bf16x2(x[2 * q], x[2 * q + 1]);
            *cp = w4;
          }
        }
      } else if (threadIdx.x < kStage) {
        s_re[threadIdx.x] = s_flag[threadIdx.x] ? 1.0f : 0.0f;
      }
      __syncthreads();
      compute_stage(E0, s0, s_flag);
    }
  }

  if (a.nsplit > 1) {
    // partial state of (row, part, head): O / L over the wave's dims in fp16, plus M and L.  O / L is a
    // convex combination of entry values, so it is bounded by the largest entry magnitude (at most sqrt(c)
    // times the largest gain for normalised entries), far inside fp16's range, and fp16 keeps it to 2^-11
    // relative: half the bytes of float32 partials for the combine to read back.
    const int64_t base = ((int64_t)row * a.nsplit + sp) * a.H;
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float il = __shfl(inv, 4 * g + i, 64);  // the denominator of head 4g + i (lane-row index)
      uint16_t* dst = a.ws_o + (base + h0 + 4 * g + i) * C + dbase + (lane & 15);
      // streaming stores: read once by the combine, so they are not left dirty in L2 for the end of
      // the kernel to write back
#pragma unroll
      for (int dt = 0; dt < DTW; ++dt)
        __builtin_nontemporal_store(__builtin_bit_cast(uint16_t, (_Float16)(O[dt][i] * il)), &dst[16 * dt]);
    }
    if ((WIDE || wave == 0) && g == 0) {
      a.ws_ml[(base + head) * 2 + 0] = M;
      a.ws_ml[(base + head) * 2 + 1] = L;
    }
    return;
  }
  // ---- single part: add the sink, normalise, gains, rotate back by -t, write
  const float zs = kLog2e * a.sink[head];
  const float Mf = fmaxf(M, zs);
  const float Lf = L * __builtin_amdgcn_exp2f(M - Mf) + __builtin_amdgcn_exp2f(zs - Mf);
  const float f = (M == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(M - Mf) / Lf;
  float fi[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) fi[i] = __shfl(f, 4 * g + i, 64);
  const int dcol = lane & 15;
#pragma unroll
  for (int dt = 0; dt < DTW; ++dt) {
    const int d = dbase + 16 * dt + dcol;
    float v[4], other[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = O[dt][i] * fi[i];
#pragma unroll
    for (int i = 0; i < 4; ++i) other[i] = __shfl_xor(v[i], 1, 64);  // pair partner: adjacent dim, adjacent lane
    if (d < rope_lo) {
      if (a.gamma_kv && !a.prepared) {  // raw entries' gain on the non-RoPE dims, applied to the output
        const float gk = a.gamma_kv[d];
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] *= gk;
      }
    } else {
      float cs, sn;
      rope_cs(-tpos, s_theta[(d - rope_lo) / 2], cs, sn);
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = (dcol & 1) ? (other[i] * sn + v[i] * cs) : (v[i] * cs - other[i] * sn);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t o = ((int64_t)row * a.H + h0 + 4 * g + i) * C + d;
      if (a.out_t == CSA_F32)
        static_cast<float*>(a.out)[o] = v[i];
      else
        static_cast<uint16_t*>(a.out)[o] = f32_to_bf16(v[i]);
    }
  }
}

constexpr int kMaxSplits = 16;

// merge the decode parts of one (row, head): fixed order, sink, gains, -t rotation
// One workgroup per (query row, head); thread t owns dims [4t, 4t + 4) (C <= 512).  Every load (the
// parts' maxima / denominators and their partial outputs) is issued before any use.
__global__ __launch_bounds__(128) void attend_combine_kernel(AttnArgs a, int C, RopeTable rt) {
  const int row = blockIdx.x;
  const int h = blockIdx.y;
  const int b = row / a.T;
  const int r = row - b * a.T;
  const int64_t base = ((int64_t)row * a.nsplit) * a.H + h;
  const int ns = a.nsplit;
  const int d0 = 4 * threadIdx.x;
  const bool active = d0 < C;
  const int dl = active ? d0 : 0;  // loads stay in the head's row
  const int rope_lo = C - a.R;
  // this thread's RoPE frequencies (RoPE dims) or output gains (raw entries' non-RoPE dims), loaded with
  // the partials
  float th[2] = {0.0f, 0.0f};
  f32x4 gk = {1.0f, 1.0f, 1.0f, 1.0f};
  if (active && d0 >= rope_lo) {
    th[0] = rt.theta[(d0 - rope_lo) / 2];
    th[1] = rt.theta[(d0 - rope_lo) / 2 + 1];
  } else if (active && a.gamma_kv && !a.prepared) {
#pragma unroll
    for (int i = 0; i < 4; ++i) gk[i] = a.gamma_kv[d0 + i];
  }
  uint2 os[kMaxSplits];  // 4 fp16 values: the part's output over its denominator
  float ms[kMaxSplits], ls[kMaxSplits];
#pragma unroll
  for (int s = 0; s < kMaxSplits; ++s)
    if (s < ns) os[s] = *reinterpret_cast<const uint2*>(a.ws_o + (base + (int64_t)s * a.H) * C + dl);
  // lane s of each wave loads part s's (M, L), lane 62 the sink and lane 63 the position, then every lane
  // takes them by lane exchange: one vector load round for all of them (as uniform scalar loads they
  // would each wait for the previous one)
  const int ln = threadIdx.x & 63;
  f32x2 ml = {-INFINITY, 0.0f};
  int64_t p0 = 0;
  if (ln < ns) ml = *reinterpret_cast<const f32x2*>(a.ws_ml + (base + (int64_t)ln * a.H) * 2);
  // (the offsets are zero, hidden from the compiler so that these stay one lane's vector loads and do
  // not become scalar loads the wave would wait for on their own)
  int z0 = 0;
  asm volatile("" : "+v"(z0));
  if (ln == 62) ml[0] = a.sink[h + z0];
  if (ln == 63) p0 = a.pos0[b + z0];
#pragma unroll
  for (int s = 0; s < kMaxSplits; ++s) {
    ms[s] = __shfl(ml[0], s, 64);
    ls[s] = __shfl(ml[1], s, 64);
  }
  const double tpos = (double)(__shfl(p0, 63, 64) + r);
  const float zs = kLog2e * __shfl(ml[0], 62, 64);  // the parts' maxima are in base-2 units
  float Mx = zs;
#pragma unroll
  for (int s = 0; s < kMaxSplits; ++s)
    if (s < ns) Mx = fmaxf(Mx, ms[s]);
  float Lt = __builtin_amdgcn_exp2f(zs - Mx);
  float v[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < kMaxSplits; ++s) {
    if (s < ns && ms[s] != -INFINITY) {  // fixed order over the parts
      const float wl = ls[s] * __builtin_amdgcn_exp2f(ms[s] - Mx);
      Lt += wl;
      const uint32_t hw[2] = {os[s].x, os[s].y};
#pragma unroll
      for (int i = 0; i < 4; ++i)
        v[i] = fmaf((float)__builtin_bit_cast(_Float16, (uint16_t)(hw[i >> 1] >> (16 * (i & 1)))), wl, v[i]);
    }
  }
  if (!active) return;
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = v[i] / Lt;
  if (d0 < rope_lo) {
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] *= gk[i];
  } else {
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      float cs, sn;
      rope_cs(-tpos, th[p], cs, sn);
      const float x0 = v[2 * p], x1 = v[2 * p + 1];
      v[2 * p] = x0 * cs - x1 * sn;
      v[2 * p + 1] = x0 * sn + x1 * cs;
    }
  }
  const int64_t o = ((int64_t)row * a.H + h) * C + d0;
  if (a.out_t == CSA_F32) {
    *reinterpret_cast<f32x4*>(static_cast<float*>(a.out) + o) = f32x4{v[0], v[1], v[2], v[3]};
  } else {
    uint2 pk;
    pk.x = pack_bf16x2(v[0], v[1]);
    pk.y = pack_bf16x2(v[2], v[3]);
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + o) = pk;
  }
}

// ------------------------------------------------------------------ float32 path
struct AttnArgsF32 {
  const float* q;
  const float* comp;
  const int32_t* idx;
  const float* win;
  const float* sink;
  const float* gamma_q;
  const float* gamma_kv;
  const int64_t* pos0;
  void* out;
  int T, H, C, R, k, n_win, m, out_t, mode, hg, prepared;
  int64_t n_max;
  float scale, eps;
};

constexpr int kF32MaxDPL = 8;  // dims per lane (c <= 512)

// rotate the lane's dims [d0, d0+dpl) if they are RoPE dims (pairs are lane-local)
CSA_DEV void rope_lane(float* x, int dpl, int d0, int rope_lo, double pos, const RopeTable& rt) {
  for (int j = 0; j < dpl; j += 2) {
    const int d = d0 + j;
    if (d < rope_lo) continue;
    float cs, sn;
    rope_cs(pos, rt.theta[(d - rope_lo) / 2], cs, sn);
    const float x0 = x[j], x1 = x[j + 1];
    x[j] = x0 * cs - x1 * sn;
    x[j + 1] = x0 * sn + x1 * cs;
  }
}

__global__ __launch_bounds__(256) void attend_f32_kernel(AttnArgsF32 a, RopeTable rt) {
  extern __shared__ float s_f[];  // q^ [hg][C]  |  merge buffer [hg][C + 2]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int row = blockIdx.y;
  const int b = row / a.T, r = row - b * a.T;
  const int64_t t = a.pos0[b] + r;
  const int64_t vis = visible_entries(t, a.m, a.n_max);
  const int h0 = blockIdx.x * a.hg;
  const int nh = min(a.hg, a.H - h0);
  const int C = a.C, dpl = C / 64, d0 = lane * dpl, rope_lo = C - a.R;
  float* sq = s_f;
  float* sm = s_f + a.hg * C;

  // q^ = RoPE_t(RMSNorm(q)) for the group's heads
  for (int hh = wave; hh < nh; hh += 4) {
    const float* qr = a.q + ((int64_t)row * a.H + h0 + hh) * C;
    float x[kF32MaxDPL];
    float ss = 0.f;
    for (int j = 0; j < dpl; ++j) { x[j] = qr[d0 + j]; ss = fmaf(x[j], x[j], ss); }
    ss = wave_sum(ss);
    const float rn = 1.0f / sqrtf(ss / (float)C + a.eps);
    for (int j = 0; j < dpl; ++j) x[j] = x[j] * rn * (a.gamma_q ? a.gamma_q[d0 + j] : 1.0f);
    rope_lane(x, dpl, d0, rope_lo, (double)t, rt);
    for (int j = 0; j < dpl; ++j) sq[hh * C + d0 + j] = x[j];
  }
  __syncthreads();

  float acc[32][kF32MaxDPL];
  float Mh[32], Lh[32];
  for (int hh = 0; hh < 32; ++hh) {
    Mh[hh] = -INFINITY;
    Lh[hh] = 0.f;
    for (int j = 0; j < kF32MaxDPL; ++j) acc[hh][j] = 0.f;
  }
  const int64_t nslots = ((a.mode == 0) ? a.k : a.n_max) + a.n_win;
  for (int64_t slot = wave; slot < nslots; slot += 4) {
    // resolve the slot (same rule as the bf16 path)
    int64_t erow = -1;
    bool is_win = false;
    double pos = 0.0;
    const int64_t ncomp = (a.mode == 0) ? a.k : a.n_max;
    if (slot < ncomp) {
      int64_t e = (a.mode == 0) ? (int64_t)a.idx[((int64_t)b * a.T + r) * a.k + slot] : slot;
      bool ok = (a.mode == 0) ? (e >= 0 && e < a.n_max) : (e < vis);
      if (ok) { erow = e; pos = (double)a.m * (double)e; }
    } else {
      const int64_t w = slot - ncomp;
      const int64_t p = t - a.n_win + 1 + w;
      if (p >= 0) { erow = r + w; is_win = true; pos = (double)p; }
    }
    if (erow < 0) continue;  // uniform across the wave
    const float* src = is_win ? a.win + ((int64_t)b * (a.T + a.n_win - 1) + erow) * C
                              : a.comp + ((int64_t)b * a.n_max + erow) * C;
    float x[kF32MaxDPL];
    if (is_win ? a.prepared == 2 : a.prepared != 0) {  // stored prepared: used as it is
      for (int j = 0; j < dpl; ++j) x[j] = src[d0 + j];
    } else {
      float ss = 0.f;
      for (int j = 0; j < dpl; ++j) { x[j] = src[d0 + j]; ss = fmaf(x[j], x[j], ss); }
      ss = wave_sum(ss);
      const float rn = 1.0f / sqrtf(ss / (float)C + a.eps);
      for (int j = 0; j < dpl; ++j) x[j] = x[j] * rn * (a.gamma_kv ? a.gamma_kv[d0 + j] : 1.0f);
      rope_lane(x, dpl, d0, rope_lo, pos, rt);
    }
    for (int hh = 0; hh < nh; ++hh) {
      float d = 0.f;
      for (int j = 0; j < dpl; ++j) d = fmaf(sq[hh * C + d0 + j], x[j], d);
      const float z = wave_sum(d) * a.scale;
      const float Mn = fmaxf(Mh[hh], z);
      const float al = expf(Mh[hh] - Mn);
      const float p = expf(z - Mn);
      Lh[hh] = Lh[hh] * al + p;
      for (int j = 0; j < dpl; ++j) acc[hh][j] = fmaf(p, x[j], acc[hh][j] * al);
      Mh[hh] = Mn;
    }
  }
  // merge waves 1..3 into wave 0 in a fixed order
  for (int src_w = 1; src_w < 4; ++src_w) {
    if (wave == src_w) {
      for (int hh = 0; hh < nh; ++hh) {
        for (int j = 0; j < dpl; ++j) sm[hh * (C + 2) + d0 + j] = acc[hh][j];
        if (lane == 0) { sm[hh * (C + 2) + C] = Mh[hh]; sm[hh * (C + 2) + C + 1] = Lh[hh]; }
      }
    }
    __syncthreads();
    if (wave == 0) {
      for (int hh = 0; hh < nh; ++hh) {
        const float Mo = sm[hh * (C + 2) + C], Lo = sm[hh * (C + 2) + C + 1];
        const float Mn = fmaxf(Mh[hh], Mo);
        if (Mn == -INFINITY) continue;
        const float fa = expf(Mh[hh] - Mn), fb = expf(Mo - Mn);
        Lh[hh] = Lh[hh] * fa + Lo * fb;
        for (int j = 0; j < dpl; ++j) acc[hh][j] = acc[hh][j] * fa + sm[hh * (C + 2) + d0 + j] * fb;
        Mh[hh] = Mn;
      }
    }
    __syncthreads();
  }
  if (wave != 0) return;
  for (int hh = 0; hh < nh; ++hh) {
    const int h = h0 + hh;
    const float zs = a.sink[h];
    const float Mf = fmaxf(Mh[hh], zs);
    const float Lf = Lh[hh] * expf(Mh[hh] - Mf) + expf(zs - Mf);
    const float f = (Mh[hh] == -INFINITY) ? 0.0f : expf(Mh[hh] - Mf) / Lf;
    float x[kF32MaxDPL];
    for (int j = 0; j < dpl; ++j) x[j] = acc[hh][j] * f;
    rope_lane(x, dpl, d0, rope_lo, -(double)t, rt);
    const int64_t o = ((int64_t)row * a.H + h) * C + d0;
    for (int j = 0; j < dpl; ++j) {
      if (a.out_t == CSA_F32)
        static_cast<float*>(a.out)[o + j] = x[j];
      else
        static_cast<uint16_t*>(a.out)[o + j] = f32_to_bf16(x[j]);
    }
  }
}

// Decode (T = 1) splits each query's slot list into parts whose boundaries depend only on the list
// lengths: the compressed slots into at most kMaxSplits - 4 parts of at least 128 slots, the window
// slots into at most 4 parts (2 for the wide variant) of at least 64 (multiples of the 32-slot tile).
// Raw window rows are normalised and rotated in the kernel, so keeping them apart keeps the parts of
// similar cost when the compressed entries are stored prepared.  Prefill queries are served by one
// part each.
struct SplitLayout {
  int nsplit, ns_c, s_c, s_w;
};
// The wide variant (64 heads per workgroup) serves prefill and HCA's long dense lists when every row is
// stored prepared (it holds all c dims of 16 heads per wave and has no room for the in-kernel RMSNorm /
// RoPE of raw rows); CSA decode keeps the narrow one, whose 16-head workgroups give a few short rows
// enough parallel work.
bool use_wide(int mode, int T, int H, int prepared) {
  return (H % 64) == 0 && prepared == 2 && (T > 1 || mode == 1);
}
SplitLayout split_layout(int mode, int T, int H, int prepared, int64_t ncomp, int64_t n_win) {
  if (T != 1) return SplitLayout{1, 1, (int)(ncomp + n_win), 0};
  auto len = [](int64_t n, int parts, int minimum) -> int64_t {
    int64_t l = (n + parts - 1) / parts;
    l = ((l + kTile - 1) / kTile) * kTile;
    return l < minimum ? minimum : l;
  };
  const int max_w = use_wide(mode, T, H, prepared) ? 2 : 4;  // window parts (the rest: compressed parts)
  const int64_t sw = len(n_win, max_w, 64);
  const int nsw = ceil_div(n_win, sw);
  const int64_t sc = len(ncomp, kMaxSplits - max_w, kSplitSlots);
  const int nsc = ncomp > 0 ? ceil_div(ncomp, sc) : 0;
  return SplitLayout{nsc + nsw, nsc, (int)sc, (int)sw};
}

// the kernel's LDS carve-up: stage buffers, (narrow) logit exchange, per-slot scalars, RoPE table and
// the slot-resolution buffers
template <int C, bool WIDE>
size_t bf16_lds_bytes() {
  const size_t ne = WIDE ? 2 : 1;
  return (size_t)lds_ctrl_halfs<WIDE>() * 2 + (WIDE ? 0 : 4 * 2 * 64 * 16) + ne * kStage * C * 2;
}

template <int C, bool WIDE, bool RAW, bool MIX, bool PAGED>
csa_status launch_bf16(const AttnArgs& a, const RopeTable& rt, int rows, hipStream_t stream) {
  const size_t lds = bf16_lds_bytes<C, WIDE>();
  static bool attr_set = false;
  if (!attr_set) {
    if (hipFuncSetAttribute((const void*)attend_bf16_kernel<C, WIDE, RAW, MIX, PAGED>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
      return CSA_ERR_LAUNCH;
    attr_set = true;
  }
  // grid.x = (part, row) padded to a multiple of 8 so that workgroups differing only in their
  // head group have equal linear ids modulo 8 and land on the same XCD (shared L2 for the staged KV)
  const int nx = a.nsplit * rows;
  const int nx_pad = (nx + 7) & ~7;
  dim3 grid(nx_pad, a.H / (WIDE ? 64 : 16));
  hipLaunchKernelGGL((attend_bf16_kernel<C, WIDE, RAW, MIX, PAGED>), grid, dim3(256), lds, stream, a, rt, nx);
  if (a.nsplit > 1) hipLaunchKernelGGL(attend_combine_kernel, dim3(rows, a.H), dim3(128), 0, stream, a, C, rt);
  return hipGetLastError() == hipSuccess ? CSA_OK : CSA_ERR_LAUNCH;
}

// MIX: compressed rows in CSA_FP8_BF16_ROPE (a variant of its own, so that the bf16 kernels carry none of
// its code)
template <int C, bool MIX, bool PAGED>
csa_status launch_bf16_fmt(const AttnArgs& a, const RopeTable& rt, int rows, bool wide, hipStream_t stream) {
  if (wide) return launch_bf16<C, true, false, MIX, PAGED>(a, rt, rows, stream);
  return a.prepared == 2 ? launch_bf16<C, false, false, MIX, PAGED>(a, rt, rows, stream)
                         : launch_bf16<C, false, true, MIX, PAGED>(a, rt, rows, stream);
}
template <int C>
csa_status launch_bf16_any(const AttnArgs& a, const RopeTable& rt, int rows, bool wide, hipStream_t stream) {
  if (a.table)
    return a.comp_mixed ? launch_bf16_fmt<C, true, true>(a, rt, rows, wide, stream)
                        : launch_bf16_fmt<C, false, true>(a, rt, rows, wide, stream);
  return a.comp_mixed ? launch_bf16_fmt<C, true, false>(a, rt, rows, wide, stream)
                      : launch_bf16_fmt<C, false, false>(a, rt, rows, wide, stream);
}

}  // namespace

size_t attend_workspace_bytes(int mode, int B, int T, int H, int c, int64_t ncomp, int n_win) {
  (void)mode;
  // the larger of the two layouts, so one workspace size serves every kv_prepared mode
  const int ns = max(split_layout(mode, T, H, 0, ncomp, n_win).nsplit, split_layout(mode, T, H, 2, ncomp, n_win).nsplit);
  if (ns <= 1) return 0;
  const size_t rows = (size_t)B * T;
  const size_t o = rows * ns * H * (size_t)c * 2;  // fp16 partial outputs
  return ((o + 255) & ~(size_t)255) + rows * ns * H * 2 * 4;
}

csa_status launch_attend(int mode, const void* q, const void* comp_kv, const float* comp_scale, bool comp_mixed,
                         const csa_pages* pages, const int32_t* idx, const void* win_kv,
                         const float* sink, const float* gamma_q, const float* gamma_kv, int B, int T, int H,
                         int c, int rope_dims, int k, int n_win, int64_t n_max, const int64_t* pos0, int m,
                         float scale, float eps, float rope_base, int kv_t, int kv_prepared, void* out, int out_t,
                         void* ws, hipStream_t stream) {
  if (pages && (kv_t != CSA_BF16 || T != 1)) return CSA_ERR_UNSUPPORTED;
  const RopeTable rt = make_rope_table(rope_dims, rope_base);
  const int rows = B * T;
  if (kv_t == CSA_F32) {
    AttnArgsF32 a;
    a.q = (const float*)q; a.comp = (const float*)comp_kv; a.idx = idx; a.win = (const float*)win_kv;
    a.sink = sink; a.gamma_q = gamma_q; a.gamma_kv = gamma_kv; a.pos0 = pos0; a.out = out;
    a.T = T; a.H = H; a.C = c; a.R = rope_dims; a.k = k; a.n_win = n_win; a.m = m; a.out_t = out_t;
    a.mode = mode; a.n_max = n_max; a.scale = scale; a.eps = eps; a.prepared = kv_prepared;
    a.hg = 4096 / c;  // heads per workgroup: hg * (c / 64) <= 64 accumulators per lane
    if (a.hg > 32) a.hg = 32;
    size_t lds = (size_t)a.hg * c * 4 + (size_t)a.hg * (c + 2) * 4;
    dim3 grid(ceil_div(H, a.hg), rows);
    hipLaunchKernelGGL(attend_f32_kernel, grid, dim3(256), lds, stream, a, rt);
    return hipGetLastError() == hipSuccess ? CSA_OK : CSA_ERR_LAUNCH;
  }
  AttnArgs a;
  a.q = (const uint16_t*)q; a.comp = (const uint16_t*)comp_kv; a.idx = idx; a.win = (const uint16_t*)win_kv;
  a.sink = sink; a.gamma_q = gamma_q; a.gamma_kv = gamma_kv; a.pos0 = pos0; a.out = out;
  a.T = T; a.H = H; a.R = rope_dims; a.k = k; a.n_win = n_win; a.m = m; a.out_t = out_t; a.mode = mode;
  a.n_max = n_max; a.scale = scale; a.eps = eps; a.prepared = kv_prepared;
  a.comp_scale = comp_scale;
  a.comp_mixed = comp_mixed ? 1 : 0;
  a.table = nullptr;
  a.tstride = a.plog2 = 0;
  if (pages) {
    a.table = pages->block_table;
    a.tstride = pages->max_pages;
    while ((1 << a.plog2) < pages->page_tokens / m) ++a.plog2;
  }
  const SplitLayout lay = split_layout(mode, T, H, kv_prepared, mode == 0 ? (int64_t)k : n_max, n_win);
  a.nsplit = lay.nsplit;
  a.ns_c = lay.ns_c;
  a.s_c = lay.s_c;
  a.s_w = lay.s_w;
  if (a.nsplit > 1) {
    const size_t o = (size_t)rows * a.nsplit * H * (size_t)c * 2;
    a.ws_o = static_cast<uint16_t*>(ws);
    a.ws_ml = reinterpret_cast<float*>(static_cast<char*>(ws) + ((o + 255) & ~(size_t)255));
  } else {
    a.ws_o = nullptr;
    a.ws_ml = nullptr;
  }
  const bool wide = use_wide(mode, T, H, kv_prepared);
  switch (c) {
    case 128: return launch_bf16_any<128>(a, rt, rows, wide, stream);
    case 256: return launch_bf16_any<256>(a, rt, rows, wide, stream);
    case 512: return launch_bf16_any<512>(a, rt, rows, wide, stream);
    default: return CSA_ERR_UNSUPPORTED;
  }
}
