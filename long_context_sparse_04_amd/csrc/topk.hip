// csa_topk kernels: exact top-k with a lower-index tie-break, ascending output.
//
// "【论文解读】DeepSeek-V4" (wkq9411.github.io), section 一(三)1(2): the selector
// keeps the compressed entries whose index scores are in Top-k(I_{t,:}); section
// 二(四) notes the selector's cost (BF16 scores made it 2x faster).
//
// Scores become order-preserving uint32 keys (+0 == -0).  A radix select in 11-bit
// digits finds the k-th key K*; the result is every key > K* plus the lowest-index
// keys == K*, emitted by an ordered (index-order) block compaction, so no sort is
// needed.
//
//  * Row path (many rows, e.g. prefill): one 512-thread workgroup per row; keys
//    cached in LDS when the row fits (<= 32768 entries).
//  * Split path (few long rows, decode): chunks of 4096 scores per workgroup, 16
//    consecutive scores per thread.  Candidates (keys at or above a threshold that
//    cannot exceed K*) are compacted per chunk, in index order, into the chunk's
//    own segment of the workspace; one workgroup per row then gathers them (chunk
//    order == index order), resolves the open bits of K* and writes the output.
//    - With the indexer's bound keys (two per bound set, each the key of a
//      distinct visible entry), the threshold is the K-th largest bound key with
//      at least 16 bits resolved; every chunk workgroup derives it alone and
//      compacts its candidates, then a second launch finishes each row from
//      candidates held in registers.
//  * Row path with bound keys (many rows): one workgroup per row derives the same
//    threshold, keeps the candidates of one streaming pass in LDS and finishes.
//    - Without them: kernel 1 builds the top-digit histogram (LDS, then integer
//      atomics into a per-row global histogram), kernel 2 the second-digit
//      histogram of the keys in the selected bin, kernel 3 compacts the keys at or
//      above the 22-bit prefix, kernel 4 finishes (and clears the histogram).
//    Integer atomics make every result independent of scheduling; the workspace
//    is left zero-filled where it has to start at zero.
#include "compress_body.h"
#include "csa_common.h"
#include "csa_internal.h"

namespace {

constexpr int kBins = 2048;
constexpr int kChunk = 4096;          // scores per workgroup on the split path
constexpr int kSplitThreads = 256;
constexpr int kRowThreads = 512;
constexpr int kRowKeyCap = 32768;     // keys cached in LDS on the row path
constexpr int kSegCap = 6144;         // candidates cached in LDS by the finishing kernel (no bound keys)
constexpr int kMaxChunks = 2048;
// The bound-key path serves rows of at most kBoundMaxChunks chunks (one chunk count per finishing thread).
constexpr int kBoundMaxChunks = 256;

// The decode step's new KV entry (one per sequence), computed by one extra workgroup per row of the
// bound-key launch, beside the selection (it is read by the attention after the selection).
struct TopkFuse {
  csa_compress_body::Jobs jobs;  // j[0]
  int on, rows, m, in_t;
  int64_t row0_pos, first_entry;
};

// ------------------------------------------------------------------ wave / block primitives
// Inclusive prefix sum over the 64 lanes of a wave, in lane order: shifts by 1, 2, 4 and 8 inside
// 16-lane rows (lanes shifted in from outside the row read 0), then the last lane of rows 0 and 2
// added into rows 1 and 3, and the last lane of row 1 into rows 2 and 3.
CSA_DEV uint32_t wave_incl_sum(uint32_t x) {
  x += dpp_u32<0x111>(x);  // row_shr:1
  x += dpp_u32<0x112>(x);  // row_shr:2
  x += dpp_u32<0x114>(x);  // row_shr:4
  x += dpp_u32<0x118>(x);  // row_shr:8
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xA, 0xF, false);  // row_bcast:15 -> rows 1, 3
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xC, 0xF, false);  // row_bcast:31 -> rows 2, 3
  return x;
}

// Smallest / largest over the 64 lanes of a wave; every lane receives it (quad and row exchanges
// inside 16-lane rows, then the row-pair and half-wave swaps).
CSA_DEV uint32_t wave_min_u32(uint32_t v) {
  v = min(v, dpp_u32<0xB1>(v));   // quad_perm [1,0,3,2]
  v = min(v, dpp_u32<0x4E>(v));   // quad_perm [2,3,0,1]
  v = min(v, dpp_u32<0x124>(v));  // row_ror:4
  v = min(v, dpp_u32<0x128>(v));  // row_ror:8
  const auto a = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = min(a[0], a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return min(b[0], b[1]);
}
CSA_DEV uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_u32<0xB1>(v));
  v = max(v, dpp_u32<0x4E>(v));
  v = max(v, dpp_u32<0x124>(v));
  v = max(v, dpp_u32<0x128>(v));
  const auto a = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = max(a[0], a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return max(b[0], b[1]);
}

// Exclusive prefixes of two counts over the block in thread order, and their totals.  s_w holds
// 2 * NT / 64 words.
template <int NT>
CSA_DEV void block_excl_sum2(uint32_t a, uint32_t b, uint32_t* s_w, uint32_t& pa, uint32_t& pb, uint32_t& ta,
                             uint32_t& tb) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t ia = wave_incl_sum(a), ib = wave_incl_sum(b);
  if (lane == 63) {
    s_w[2 * wave] = ia;
    s_w[2 * wave + 1] = ib;
  }
  __syncthreads();
  uint32_t qa = 0, qb = 0, sa = 0, sb = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    const uint32_t xa = s_w[2 * w], xb = s_w[2 * w + 1];
    qa += (w < wave) ? xa : 0u;
    qb += (w < wave) ? xb : 0u;
    sa += xa;
    sb += xb;
  }
  __syncthreads();
  pa = qa + ia - a;
  pb = qb + ib - b;
  ta = sa;
  tb = sb;
}

// Exclusive prefix of a 0/1 flag over the block (in thread order) and its total.
template <int NT>
CSA_DEV int block_flag_scan(bool flag, uint32_t* s_w, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint64_t bal = __ballot(flag);
  const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0));
  if (lane == 0) s_w[wave] = (uint32_t)__popcll(bal);
  __syncthreads();
  int pre = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    const int v = (int)s_w[w];
    pre += (w < wave) ? v : 0;
    tot += v;
  }
  __syncthreads();
  total = tot;
  return pre + below;
}

// Given hist[NB] (counts per digit) and 1 <= need <= the total count, find the digit d with
// count(> d) < need <= count(>= d); writes d and count(> d) to out[0..1].  Thread t holds bins
// [t * NB/NT, (t + 1) * NB/NT) in registers; counts above a thread's bins are a suffix sum (the wave
// total minus the inclusive prefix, plus the totals of later waves).
template <int NT, int NB>
CSA_DEV void select_digit(const uint32_t* hist, int need, uint32_t* s_w, int* out) {
  constexpr int BPT = NB / NT;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t hv[BPT];
  uint32_t local = 0;
#pragma unroll
  for (int j = 0; j < BPT; ++j) {
    hv[j] = hist[tid * BPT + j];
    local += hv[j];
  }
  const uint32_t incl = wave_incl_sum(local);
  if (lane == 63) s_w[wave] = incl;
  __syncthreads();
  uint32_t above = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63) - incl;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) above += (w > wave) ? s_w[w] : 0u;
  const uint32_t nd = (uint32_t)need;
  if (above < nd && above + local >= nd) {
#pragma unroll
    for (int j = BPT - 1; j >= 0; --j) {
      if (above + hv[j] >= nd) {
        out[0] = tid * BPT + j;
        out[1] = (int)above;
        break;
      }
      above += hv[j];
    }
  }
  __syncthreads();
}

// A candidate of the split path: its key and its index in the row.
struct Cand {
  uint32_t key;
  int32_t idx;
};

// One row of scores, float32 or bf16 (a bf16 score's key is that of its exact float32 value, so both
// kinds share the key space and every selection step below).
struct ScoreRow {
  const void* p;
  int bf16;
  CSA_DEV uint32_t key(int64_t i) const {
    return bf16 ? score_key(__uint_as_float((uint32_t)static_cast<const uint16_t*>(p)[i] << 16))
                : score_key(static_cast<const float*>(p)[i]);
  }
};
CSA_DEV ScoreRow score_row(const void* scores, int bf16, int64_t row, int64_t n_max) {
  return ScoreRow{static_cast<const char*>(scores) + row * n_max * (bf16 ? 2 : 4), bf16};
}

// Smallest and largest of the per-thread (lo, hi) over the block; every thread gets both.
template <int NT>
CSA_DEV void block_minmax(uint32_t& lo, uint32_t& hi, uint32_t* s_mm) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  lo = wave_min_u32(lo);
  hi = wave_max_u32(hi);
  if (lane == 0) {
    s_mm[2 * wave] = lo;
    s_mm[2 * wave + 1] = hi;
  }
  __syncthreads();
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    lo = min(lo, s_mm[2 * w]);
    hi = max(hi, s_mm[2 * w + 1]);
  }
  __syncthreads();
}

// Radix step over the keys that agree with pv on their top `known` bits (0 <= known < 32): histogram
// of the 11 bits ending at `shift` (bits already known among them take one value), and the digit of
// the need-th largest.  Updates pv (those 11 bits), need (minus the keys above the digit) and known.
// each(f) calls f(key) for every key the calling thread contributes.
template <int NT, typename Each>
CSA_DEV void radix_step(Each each, uint32_t& pv, int& known, int& need, uint32_t* hist, uint32_t* s_w,
                        int* s_sel) {
  const int shift = max(0, 32 - known - 11);
  for (int j = threadIdx.x; j < kBins; j += NT) hist[j] = 0;
  __syncthreads();
  const uint32_t hmask = known == 0 ? 0u : ~0u << (32 - known);
  const uint32_t hp = pv & hmask;
  each([&](uint32_t kk) {
    if ((kk & hmask) == hp) atomicAdd(&hist[(kk >> shift) & 0x7FFu], 1u);
  });
  __syncthreads();
  select_digit<NT, kBins>(hist, need, s_w, s_sel);
  pv = (pv & ~(0x7FFu << shift)) | ((uint32_t)s_sel[0] << shift);
  need -= s_sel[1];
  known = 32 - shift;
}

// Bits shared by every key in [lo, hi] (lo <= hi).
CSA_DEV int common_bits(uint32_t lo, uint32_t hi) { return lo == hi ? 32 : __clz(lo ^ hi); }

// A row with V <= k: every visible entry, in order.
CSA_DEV void trivial_row(const ScoreRow& srow, int V, int k, int nt, int32_t* orow, float* vrow) {
  for (int j = threadIdx.x; j < k; j += nt) {
    orow[j] = j < V ? j : -1;
    if (vrow) vrow[j] = j < V ? key_to_score(srow.key(j)) : -INFINITY;
  }
}

// ------------------------------------------------------------------ row path
// Exact selection of one row by one workgroup of NT threads over all V visible keys: three digit passes
// (11, 11 and 10 bits) find the K-th key K*, then an ordered compaction emits every key > K* and the
// lowest-index keys == K*.  keys (LDS, nullable): the row's keys are cached there by the first pass.
template <int NT>
CSA_DEV void row_select(const ScoreRow& srow, int V, int K, int k, int32_t* __restrict__ orow,
                        float* __restrict__ vrow, uint32_t* hist, uint32_t* keys, uint32_t* s_w, int* s_sel) {
  const int tid = threadIdx.x;
  auto key_at = [&](int i) -> uint32_t { return keys ? keys[i] : srow.key(i); };

  // digit 0: bits 31..21
  for (int j = tid; j < kBins; j += NT) hist[j] = 0;
  __syncthreads();
  for (int i = tid; i < V; i += NT) {
    uint32_t kk = srow.key(i);
    if (keys) keys[i] = kk;
    atomicAdd(&hist[kk >> 21], 1u);
  }
  __syncthreads();
  select_digit<NT, kBins>(hist, K, s_w, s_sel);
  const uint32_t d0 = s_sel[0];
  int need = K - s_sel[1];
  __syncthreads();

  // digit 1: bits 20..10 among keys with digit 0 == d0
  for (int j = tid; j < kBins; j += NT) hist[j] = 0;
  __syncthreads();
  for (int i = tid; i < V; i += NT) {
    uint32_t kk = key_at(i);
    if ((kk >> 21) == d0) atomicAdd(&hist[(kk >> 10) & 0x7FFu], 1u);
  }
  __syncthreads();
  select_digit<NT, kBins>(hist, need, s_w, s_sel);
  const uint32_t p1 = (d0 << 11) | (uint32_t)s_sel[0];  // top 22 bits
  need -= s_sel[1];
  __syncthreads();

  // digit 2: bits 9..0 among keys with top 22 bits == p1
  for (int j = tid; j < kBins; j += NT) hist[j] = 0;
  __syncthreads();
  for (int i = tid; i < V; i += NT) {
    uint32_t kk = key_at(i);
    if ((kk >> 10) == p1) atomicAdd(&hist[kk & 0x3FFu], 1u);
  }
  __syncthreads();
  select_digit<NT, 1024>(hist, need, s_w, s_sel);
  const uint32_t kstar = (p1 << 10) | (uint32_t)s_sel[0];
  const int ties = need - s_sel[1];  // keys == K* to take, lowest indices first
  __syncthreads();

  // ordered compaction
  int out_base = 0, tie_base = 0;
  for (int c0 = 0; c0 < V && out_base < K; c0 += NT) {
    const int i = c0 + tid;
    uint32_t kk = i < V ? key_at(i) : 0u;
    const bool eq = (i < V) && kk == kstar;
    int eq_tot;
    int eq_rank = tie_base + block_flag_scan<NT>(eq, s_w, eq_tot);
    const bool sel = (i < V) && (kk > kstar || (eq && eq_rank < ties));
    int sel_tot;
    int pos = out_base + block_flag_scan<NT>(sel, s_w, sel_tot);
    if (sel) {
      orow[pos] = i;
      if (vrow) vrow[pos] = key_to_score(kk);
    }
    out_base += sel_tot;
    tie_base += eq_tot;
  }
  for (int j = K + tid; j < k; j += NT) {
    orow[j] = -1;
    if (vrow) vrow[j] = -INFINITY;
  }
}

__global__ __launch_bounds__(kRowThreads) void topk_row_kernel(const void* __restrict__ scores, int sbf16, int T,
                                                               int64_t n_max, const int64_t* __restrict__ pos0,
                                                               int m, int k, int32_t* __restrict__ idx,
                                                               float* __restrict__ vals, int cache_keys) {
  extern __shared__ uint32_t s_dyn[];
  uint32_t* hist = s_dyn;           // kBins
  uint32_t* keys = s_dyn + kBins;   // cache (when enabled)
  __shared__ uint32_t s_w[2 * kRowThreads / 64];
  __shared__ int s_sel[2];

  const int row = blockIdx.x;
  const int b = row / T;
  const int r = row - b * T;
  const int64_t t = pos0[b] + r;
  const int V = (int)visible_entries(t, m, n_max);
  const int K = k < V ? k : V;
  const ScoreRow srow = score_row(scores, sbf16, row, n_max);
  int32_t* orow = idx + (int64_t)row * k;
  float* vrow = vals ? vals + (int64_t)row * k : nullptr;

  if (K == V) {  // everything visible is selected (also covers V == 0)
    trivial_row(srow, V, k, kRowThreads, orow, vrow);
    return;
  }
  row_select<kRowThreads>(srow, V, K, k, orow, vrow, hist, cache_keys ? keys : nullptr, s_w, s_sel);
}

// ------------------------------------------------------------------ split path
struct SplitWs {
  uint32_t* hist;     // [rows][kBins]   digit-0 histogram (zero at rest)
  uint32_t* hist1;    // [rows][kBins]   digit-1 histogram (cleared by kernel 1 of every call)
  uint32_t* info;     // [rows][4]
  uint32_t* cnt;      // [rows][nch]     per chunk: candidates | (candidates above the threshold's prefix) << 16
  Cand* seg;          // [rows][n_max]
  Cand* blk;          // [rows][nch][kBlk] bound-key path: each chunk's first kBlk candidates, in index order
};

// The bound-key path keeps each chunk's first kBlk candidates in a compact block (the rest in the chunk's
// segment), so that the row's finishing workgroup reads them in one coalesced round.
constexpr int kBlk = 64;

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// The split path serves fewer than kSplitMaxRows rows.  Its zero-at-rest region (the digit-0 histograms)
// takes fixed slots for that many rows at the start of the workspace, so that no call of another shape
// ever places it over memory that a previous call left dirty.
constexpr int kSplitMaxRows = 128;
constexpr size_t kHistSlot = (size_t)kSplitMaxRows * kBins * 4;

static SplitWs carve(void* ws, int rows, int64_t n_max, int nch) {
  char* p = static_cast<char*>(ws);
  SplitWs s;
  s.hist = reinterpret_cast<uint32_t*>(p);
  p += kHistSlot;
  s.hist1 = reinterpret_cast<uint32_t*>(p);
  p += align256((size_t)rows * kBins * 4);
  s.info = reinterpret_cast<uint32_t*>(p);
  p += align256((size_t)rows * 16);
  s.cnt = reinterpret_cast<uint32_t*>(p);
  p += align256((size_t)rows * nch * 4);
  s.seg = reinterpret_cast<Cand*>(p);
  p += align256((size_t)rows * n_max * sizeof(Cand));
  s.blk = reinterpret_cast<Cand*>(p);
  return s;
}

static size_t split_bytes(int rows, int64_t n_max, int nch) {
  return kHistSlot + align256((size_t)rows * kBins * 4) + align256((size_t)rows * 16) +
         align256((size_t)rows * nch * 4) + align256((size_t)rows * n_max * sizeof(Cand)) +
         align256((size_t)rows * nch * kBlk * sizeof(Cand));
}

// Thread t of a split-path workgroup owns the 16 consecutive scores [lo + 16 t, lo + 16 t + 16) of
// its chunk, so that one block scan orders a chunk's candidates by index.  All loads are issued before
// any use; addresses are clamped into the row (no branch between loads) and validity is applied
// afterwards from the unclamped positions.
constexpr int kPerThread = kChunk / kSplitThreads;  // 16

struct ChunkKeys {
  uint32_t key[kPerThread];
  bool valid[kPerThread];
};

CSA_DEV ChunkKeys load_chunk(const ScoreRow& srow, int lo, int hi, int64_t n_max) {
  ChunkKeys c;
  const int64_t i0 = lo + kPerThread * (int)threadIdx.x;
  if (srow.bf16 && (n_max & 7) == 0) {
    u32x4 x[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t p = min(i0 + 8 * j, n_max - 8);
      x[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(srow.p) + p));
    }
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        c.key[8 * j + 2 * h] = score_key(__uint_as_float(x[j][h] << 16));
        c.key[8 * j + 2 * h + 1] = score_key(__uint_as_float(x[j][h] & 0xFFFF0000u));
      }
  } else if (!srow.bf16 && (n_max & 3) == 0) {
    f32x4 x[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t p = min(i0 + 4 * j, n_max - 4);
      x[j] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(static_cast<const float*>(srow.p) + p));
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) c.key[4 * j + q] = score_key(x[j][q]);
  } else if (srow.bf16) {  // (one branch around all the loads, so that they go out together)
    uint16_t x[kPerThread];
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) x[e] = static_cast<const uint16_t*>(srow.p)[min(i0 + e, n_max - 1)];
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) c.key[e] = score_key(__uint_as_float((uint32_t)x[e] << 16));
  } else {
    float x[kPerThread];
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) x[e] = static_cast<const float*>(srow.p)[min(i0 + e, n_max - 1)];
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) c.key[e] = score_key(x[e]);
  }
#pragma unroll
  for (int e = 0; e < kPerThread; ++e) c.valid[e] = i0 + e < hi;
  return c;
}

// Write the chunk's keys >= thr in index order: into its segment, or (blk non-NULL) the first kBlk into the
// chunk's compact block and the rest into its segment; returns the chunk totals (candidates, and those whose
// top bits under pmask exceed thr's) to every thread.
CSA_DEV void compact_chunk(const ChunkKeys& ck, int lo, uint32_t thr, uint32_t pmask, Cand* seg, Cand* blk,
                           uint32_t* s_w, uint32_t& c_tot, uint32_t& g_tot) {
  uint32_t c_t = 0, g_t = 0;
#pragma unroll
  for (int e = 0; e < kPerThread; ++e) {
    const bool cand = ck.valid[e] && ck.key[e] >= thr;
    c_t += cand;
    g_t += cand && (ck.key[e] & pmask) > thr;
  }
  uint32_t c_pre, g_pre;
  block_excl_sum2<kSplitThreads>(c_t, g_t, s_w, c_pre, g_pre, c_tot, g_tot);
  const int i0 = lo + kPerThread * (int)threadIdx.x;
  int p = (int)c_pre;  // position inside the chunk
#pragma unroll
  for (int e = 0; e < kPerThread; ++e)
    if (ck.valid[e] && ck.key[e] >= thr) {
      const Cand cd{ck.key[e], i0 + e};
      if (blk && p < kBlk)
        blk[p] = cd;
      else
        seg[lo + p] = cd;
      ++p;
    }
}

// Kernel 1: per-chunk histogram of the top key digit (bits 31..21), added into the row histogram;
// also clears the digit-1 histogram that kernel 2 fills.
__global__ __launch_bounds__(kSplitThreads) void topk_split_hist_kernel(const void* __restrict__ scores, int sbf16,
                                                                        int T, int64_t n_max,
                                                                        const int64_t* __restrict__ pos0, int m,
                                                                        int k, SplitWs ws) {
  __shared__ uint32_t hist[kBins];
  const int tid = threadIdx.x;
  const int row = blockIdx.y;
  const int b = row / T;
  const int r = row - b * T;
  const int V = (int)visible_entries(pos0[b] + r, m, n_max);
  const int K = k < V ? k : V;
  const int lo = blockIdx.x * kChunk;
  const int hi = min(lo + kChunk, V);
  if (blockIdx.x == 0) {
#pragma unroll
    for (int u = 0; u < kBins / kSplitThreads; ++u) ws.hist1[(int64_t)row * kBins + tid + u * kSplitThreads] = 0;
  }
  if (K == V || lo >= hi) return;  // trivial row or empty chunk (uniform per workgroup)
  const ScoreRow srow = score_row(scores, sbf16, row, n_max);
  uint32_t* ghist = ws.hist + (int64_t)row * kBins;
  const ChunkKeys ck = load_chunk(srow, lo, hi, n_max);
  for (int j = tid; j < kBins; j += kSplitThreads) hist[j] = 0;
  __syncthreads();
#pragma unroll
  for (int e = 0; e < kPerThread; ++e)
    if (ck.valid[e]) atomicAdd(&hist[ck.key[e] >> 21], 1u);
  __syncthreads();
  for (int j = tid; j < kBins; j += kSplitThreads)
    if (hist[j]) atomicAdd(&ghist[j], hist[j]);
}

// Load a row histogram (kBins counters) into LDS, all loads issued first.
CSA_DEV void load_hist(const uint32_t* g, uint32_t* hist) {
  const int tid = threadIdx.x;
  uint32_t hv[kBins / kSplitThreads];
#pragma unroll
  for (int u = 0; u < kBins / kSplitThreads; ++u) hv[u] = g[tid + u * kSplitThreads];
#pragma unroll
  for (int u = 0; u < kBins / kSplitThreads; ++u) hist[tid + u * kSplitThreads] = hv[u];
}

// Kernel 2: every workgroup derives digit d0 from the complete digit-0 histogram, then adds the
// histogram of digit 1 (bits 20..10) of its keys whose digit 0 equals d0.
__global__ __launch_bounds__(kSplitThreads) void topk_split_hist1_kernel(const void* __restrict__ scores, int sbf16,
                                                                         int T, int64_t n_max,
                                                                         const int64_t* __restrict__ pos0, int m,
                                                                         int k, SplitWs ws) {
  __shared__ uint32_t hist[kBins];
  __shared__ uint32_t s_w[2 * kSplitThreads / 64];
  __shared__ int s_sel[2];
  const int tid = threadIdx.x;
  const int row = blockIdx.y;
  const int b = row / T;
  const int r = row - b * T;
  const int V = (int)visible_entries(pos0[b] + r, m, n_max);
  const int K = k < V ? k : V;
  if (K == V) return;
  const ScoreRow srow = score_row(scores, sbf16, row, n_max);
  const int lo = blockIdx.x * kChunk;
  const int hi = min(lo + kChunk, V);
  ChunkKeys ck;
  if (lo < hi) ck = load_chunk(srow, lo, hi, n_max);
  load_hist(ws.hist + (int64_t)row * kBins, hist);
  __syncthreads();
  select_digit<kSplitThreads, kBins>(hist, K, s_w, s_sel);
  const uint32_t d0 = (uint32_t)s_sel[0];
  if (blockIdx.x == 0 && tid == 0) {
    ws.info[row * 4 + 0] = d0;
    ws.info[row * 4 + 1] = (uint32_t)s_sel[1];
  }
  if (lo >= hi) return;
  for (int j = tid; j < kBins; j += kSplitThreads) hist[j] = 0;
  __syncthreads();
#pragma unroll
  for (int e = 0; e < kPerThread; ++e)
    if (ck.valid[e] && (ck.key[e] >> 21) == d0) atomicAdd(&hist[(ck.key[e] >> 10) & 0x7FFu], 1u);
  __syncthreads();
  uint32_t* g1 = ws.hist1 + (int64_t)row * kBins;
  for (int j = tid; j < kBins; j += kSplitThreads)
    if (hist[j]) atomicAdd(&g1[j], hist[j]);
}

// Kernel 3: every workgroup derives the 22-bit prefix p1 = (d0, d1) from the digit-1 histogram and
// compacts its chunk's keys with top 22 bits >= p1 into the chunk's own segment, in index order.
__global__ __launch_bounds__(kSplitThreads) void topk_split_collect_kernel(const void* __restrict__ scores, int sbf16,
                                                                           int T, int64_t n_max,
                                                                           const int64_t* __restrict__ pos0, int m,
                                                                           int k, SplitWs ws) {
  __shared__ uint32_t hist[kBins];
  __shared__ uint32_t s_w[2 * kSplitThreads / 64];
  __shared__ int s_sel[2];
  const int tid = threadIdx.x;
  const int row = blockIdx.y;
  const int nch = gridDim.x;
  const int b = row / T;
  const int r = row - b * T;
  const int V = (int)visible_entries(pos0[b] + r, m, n_max);
  const int K = k < V ? k : V;
  if (K == V) return;
  const ScoreRow srow = score_row(scores, sbf16, row, n_max);
  const int lo = blockIdx.x * kChunk;
  const int hi = min(lo + kChunk, V);
  ChunkKeys ck;
  if (lo < hi) ck = load_chunk(srow, lo, hi, n_max);
  const uint32_t d0 = ws.info[row * 4 + 0];
  const int need = K - (int)ws.info[row * 4 + 1];
  load_hist(ws.hist1 + (int64_t)row * kBins, hist);
  __syncthreads();
  select_digit<kSplitThreads, kBins>(hist, need, s_w, s_sel);
  const uint32_t p1 = (d0 << 11) | (uint32_t)s_sel[0];
  if (blockIdx.x == 0 && tid == 0) {
    ws.info[row * 4 + 2] = p1;
    ws.info[row * 4 + 3] = (uint32_t)(need - s_sel[1]);  // keys with prefix p1 still to take
  }
  uint32_t c_tot = 0, g_tot = 0;
  if (lo < hi) compact_chunk(ck, lo, p1 << 10, 0xFFFFFC00u, ws.seg + (int64_t)row * n_max, nullptr, s_w, c_tot, g_tot);
  if (tid == 0) ws.cnt[(int64_t)row * nch + blockIdx.x] = c_tot;
}

// LDS of the finishing pass.
struct FinishLds {
  Cand* s_c;        // [kSegCap]
  uint32_t* hist;   // [kBins]
  int* s_pre;       // [kMaxChunks + 1]
  uint32_t* s_w;    // [2 * kSplitThreads / 64]
  int* s_sel;       // [2]
  uint32_t* s_mm;   // [2 * kSplitThreads / 64]
};

// Finishing pass of one row, by one workgroup, once every chunk's candidates are in the workspace:
// gathers them (chunk order == index order), resolves the open bits of the K-th key and writes the
// ascending index list.  The K-th key is known to start with the top `known` bits of pv and to rank
// need-th among the candidates that do.  With bound keys (bounded), pv is the threshold and need is
// reduced by the candidates whose prefix is above it (when they are fewer than K; otherwise the range
// of the candidates decides), and too few candidates (keys that were no lower bound) send the row to
// a pass over all its visible keys.
template <int SEGCAP, int MAXCH>
CSA_DEV void finish_row(const ScoreRow& srow, int V, int K, int k, int nact, const uint32_t* __restrict__ cnt,
                        const Cand* __restrict__ seg, int64_t n_max, uint32_t pv, int known, int need, bool bounded,
                        int32_t* __restrict__ orow, float* __restrict__ vrow, const FinishLds& L) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  constexpr int kW = kSplitThreads / 64;
  constexpr int kBatch = 16;  // chunks per wave per gather round
  // segment and count loads; counts are clamped to a chunk's size
  auto ldc = [&](int64_t i) -> Cand { return seg[i]; };
  auto ldn = [&](int c) -> uint32_t {
    const uint32_t v = cnt[c];
    return min(v & 0xFFFFu, (uint32_t)kChunk) | (min(v >> 16, (uint32_t)kChunk) << 16);
  };
  // first gather round: 64 candidates of each of the wave's chunks, loaded before the counts are known
  // (a chunk rarely holds more); clamped into the row's segment
  Cand sv[kBatch];
#pragma unroll
  for (int u = 0; u < kBatch; ++u) {
    const int c = wave + kW * u;
    sv[u] = ldc(min((int64_t)(c < nact ? c : 0) * kChunk + lane, n_max - 1));
  }
  // per-chunk counts: prefix (chunk order == index order) and totals
  {
    constexpr int kCpt = MAXCH / kSplitThreads;
    const int cpt = (nact + kSplitThreads - 1) / kSplitThreads;
    const int c0 = tid * cpt;
    uint32_t cv[kCpt];
#pragma unroll
    for (int u = 0; u < kCpt; ++u) cv[u] = ldn(min(c0 + u, nact - 1));
#pragma unroll
    for (int u = 0; u < kCpt; ++u) cv[u] = (u < cpt && c0 + u < nact) ? cv[u] : 0u;
    uint32_t nloc = 0, gloc = 0;
#pragma unroll
    for (int u = 0; u < kCpt; ++u) {
      nloc += cv[u] & 0xFFFFu;
      gloc += cv[u] >> 16;
    }
    uint32_t pre, gpre, ctot, gtot;
    block_excl_sum2<kSplitThreads>(nloc, gloc, L.s_w, pre, gpre, ctot, gtot);
#pragma unroll
    for (int u = 0; u < kCpt; ++u)
      if (u < cpt && c0 + u < nact) {
        L.s_pre[c0 + u] = (int)pre;
        pre += cv[u] & 0xFFFFu;
      }
    if (tid == 0) {
      L.s_pre[nact] = (int)ctot;
      L.s_sel[0] = (int)gtot;
    }
  }
  __syncthreads();
  const int* s_pre = L.s_pre;
  const int G = L.s_sel[0];
  const bool rescan = bounded && s_pre[nact] < K;  // (uniform) candidates from the whole visible row
  const int C = rescan ? V : s_pre[nact];
  const bool in_lds = !rescan && C <= SEGCAP;
  if (in_lds) {
    int nmax = 0;  // (wave-uniform)
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int c = wave + kW * u;
      const int n = c < nact ? s_pre[c + 1] - s_pre[c] : 0;
      nmax = max(nmax, n);
      if (lane < n) L.s_c[s_pre[c] + lane] = sv[u];
    }
    if (nmax > 64) {
#pragma unroll 1
      for (int u = 0; u < kBatch; ++u) {
        const int c = wave + kW * u;
        const int n = c < nact ? s_pre[c + 1] - s_pre[c] : 0;
        for (int i = 64 + lane; i < n; i += 64) L.s_c[s_pre[c] + i] = ldc((int64_t)c * kChunk + i);
      }
    }
    // rows of more than kW * kBatch chunks: later rounds, loads first
    for (int cb = wave + kW * kBatch; cb < nact; cb += kW * kBatch) {
      int dst[kBatch];
      int nm = 0;
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int c = cb + kW * u;
        const int n = c < nact ? s_pre[c + 1] - s_pre[c] : 0;
        nm = max(nm, n);
        dst[u] = lane < n ? s_pre[c] + lane : -1;
        sv[u] = ldc((int64_t)(c < nact ? c : 0) * kChunk + (lane < n ? lane : 0));
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u)
        if (dst[u] >= 0) L.s_c[dst[u]] = sv[u];
      if (nm > 64) {
#pragma unroll 1
        for (int u = 0; u < kBatch; ++u) {
          const int c = cb + kW * u;
          const int n = c < nact ? s_pre[c + 1] - s_pre[c] : 0;
          for (int i = 64 + lane; i < n; i += 64) L.s_c[s_pre[c] + i] = ldc((int64_t)c * kChunk + i);
        }
      }
    }
  }
  __syncthreads();
  auto chunk_of = [&](int j) -> int {  // c with s_pre[c] <= j < s_pre[c+1]
    int lo = 0, hi = nact;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (s_pre[mid] <= j) lo = mid; else hi = mid;
    }
    return lo;
  };
  auto cand = [&](int j) -> Cand {
    if (in_lds) return L.s_c[j];
    if (rescan) return Cand{srow.key(j), j};
    const int c = chunk_of(j);
    return ldc((int64_t)c * kChunk + (j - s_pre[c]));
  };
  // thread t takes the contiguous candidates [j0, j1), held in registers when they are few
  const int per = (C + kSplitThreads - 1) / kSplitThreads;
  const int j0 = min(tid * per, C), j1 = min(j0 + per, C);
  constexpr int kReg = 8;
  const bool regs = in_lds && per <= kReg;  // (uniform)
  uint32_t rk[kReg];
  int32_t ri[kReg];
  if (regs) {
#pragma unroll
    for (int i = 0; i < kReg; ++i) {
      const Cand cd = L.s_c[min(j0 + i, SEGCAP - 1)];
      rk[i] = cd.key;
      ri[i] = cd.idx;
    }
  }
  auto each = [&](auto f) {
    if (regs) {
#pragma unroll
      for (int i = 0; i < kReg; ++i)
        if (j0 + i < j1) f(rk[i]);
    } else {
      for (int j = j0; j < j1; ++j) f(cand(j).key);
    }
  };

  uint32_t kstar = pv;
  if (bounded) {
    if (!rescan && G < K) {
      need = K - G;  // the K-th key shares the threshold's prefix
    } else {
      known = -1;
    }
  }
  if (known < 0) {  // the candidates' range decides the first open bit
    uint32_t lo = 0xFFFFFFFFu, hi = 0u;
    each([&](uint32_t kk) {
      lo = min(lo, kk);
      hi = max(hi, kk);
    });
    block_minmax<kSplitThreads>(lo, hi, L.s_mm);
    kstar = hi;
    known = common_bits(lo, hi);
    need = K;
  }
  while (known < 32) radix_step<kSplitThreads>(each, kstar, known, need, L.hist, L.s_w, L.s_sel);
  const int ties = need;  // keys equal to K* still to take, lowest index first

  // ordered output: thread t's first selected candidate lands after the larger keys of earlier threads
  // and the equal keys they take
  uint32_t n_gt = 0, n_eq = 0;
  each([&](uint32_t kk) {
    n_gt += kk > kstar;
    n_eq += kk == kstar;
  });
  uint32_t gt_base, eq_base, gt_tot, eq_tot;
  block_excl_sum2<kSplitThreads>(n_gt, n_eq, L.s_w, gt_base, eq_base, gt_tot, eq_tot);
  int pos = (int)gt_base + min((int)eq_base, ties);
  int eq_rank = (int)eq_base;
  auto emit = [&](uint32_t kk, int32_t ix) {
    bool sel = kk > kstar;
    if (kk == kstar) sel = eq_rank++ < ties;
    if (sel && pos < K) {
      orow[pos] = ix;
      if (vrow) vrow[pos] = key_to_score(kk);
    }
    pos += sel ? 1 : 0;
  };
  if (regs) {
#pragma unroll
    for (int i = 0; i < kReg; ++i)
      if (j0 + i < j1) emit(rk[i], ri[i]);
  } else {
    for (int j = j0; j < j1; ++j) {
      const Cand cd = cand(j);
      emit(cd.key, cd.idx);
    }
  }
  for (int j = K + tid; j < k; j += kSplitThreads) {
    orow[j] = -1;
    if (vrow) vrow[j] = -INFINITY;
  }
}

#define CSA_FINISH_LDS(SEGCAP, MAXCH)                  \
  __shared__ __align__(16) Cand s_c[SEGCAP];          \
  __shared__ uint32_t s_hist[kBins];                   \
  __shared__ int s_pre[MAXCH + 1];                     \
  __shared__ uint32_t s_w[2 * kSplitThreads / 64];     \
  __shared__ int s_sel[2];                             \
  __shared__ uint32_t s_mm[2 * kSplitThreads / 64];    \
  const FinishLds L{s_c, s_hist, s_pre, s_w, s_sel, s_mm};

// Kernel 4 (no bound keys): one workgroup per row finishes from the 22-bit prefix of kernels 1 to 3
// and clears the row's digit-0 histogram.
__global__ __launch_bounds__(kSplitThreads) void topk_split_finish_kernel(
    const void* __restrict__ scores, int sbf16, int T, int64_t n_max, const int64_t* __restrict__ pos0, int m, int k,
    int nch, int32_t* __restrict__ idx, float* __restrict__ vals, SplitWs ws) {
  CSA_FINISH_LDS(kSegCap, kMaxChunks)
  const int tid = threadIdx.x;
  const int row = blockIdx.x;
  const int b = row / T;
  const int r = row - b * T;
  const int V = (int)visible_entries(pos0[b] + r, m, n_max);
  const int K = k < V ? k : V;
  const ScoreRow srow = score_row(scores, sbf16, row, n_max);
  int32_t* orow = idx + (int64_t)row * k;
  float* vrow = vals ? vals + (int64_t)row * k : nullptr;
  if (K == V) {
    trivial_row(srow, V, k, kSplitThreads, orow, vrow);
    return;
  }
  uint32_t* ghist = ws.hist + (int64_t)row * kBins;
#pragma unroll
  for (int u = 0; u < kBins / kSplitThreads; ++u) ghist[tid + u * kSplitThreads] = 0;
  const int nact = (V + kChunk - 1) / kChunk;
  finish_row<kSegCap, kMaxChunks>(srow, V, K, k, nact, ws.cnt + (int64_t)row * nch, ws.seg + (int64_t)row * n_max, n_max,
             ws.info[row * 4 + 2] << 10, 22, (int)ws.info[row * 4 + 3], false, orow, vrow, L);
}

// ------------------------------------------------------------------ split path with bound keys
// With bound keys from the indexer (two per bound set, each the key of a distinct visible entry) the
// selection takes two launches and no histogram pass:
//  * collect: every chunk workgroup derives tau, the K-th largest bound key with the bits below its radix
//    passes cleared (each pass takes the next 11 bits, starting right under the bits all bound keys share;
//    one pass, or two while fewer than 16 bits are resolved); tau never exceeds the row's K-th largest key,
//    so every selected key is a candidate (typically about 1.1k keys are).  It compacts its chunk's keys
//    >= tau in index order (the first kBlk into the chunk's compact block, the rest into its segment) and
//    writes its counts.
//  * finish: one workgroup per row reads the counts and the compact blocks in one round (a thread holds
//    16 or 32 block slots in registers), stages the candidates in LDS in index order, resolves the K-th key
//    (radix passes while more than 64 candidates share the resolved prefix, then one wave bit by bit) and
//    writes the ascending list.
// The launch boundary orders the two; no workgroup waits for another.
template <int KBK>
__global__ __launch_bounds__(kSplitThreads) void topk_bound_collect_kernel(
    const void* __restrict__ scores, int sbf16, int T, int64_t n_max, const int64_t* __restrict__ pos0, int m, int k,
    const uint32_t* __restrict__ bound, int nb, SplitWs ws, TopkFuse fz) {
  __shared__ __align__(16) f32x4 s_cz[3 * 256];  // the KV-entry workgroup's slice merge
  __shared__ uint32_t s_hist[kBins];
  __shared__ uint32_t s_w[2 * kSplitThreads / 64];
  __shared__ uint32_t s_mm[2 * kSplitThreads / 64];
  __shared__ int s_sel[2];
  __shared__ uint32_t s_nz;
  const int tid = threadIdx.x;
  const int row = blockIdx.y;
  const int nch = (int)((n_max + kChunk - 1) / kChunk);
  if (fz.on && (int)blockIdx.x == nch) {  // the extra workgroup of a row: its sequence's new KV entry
    static_assert(kSplitThreads == 256, "the compression body runs on 256 threads here");
    if (fz.in_t == CSA_F32)
      csa_compress_body::compress_one<float, 256>(fz.jobs.j[0], fz.jobs.theta[0], 0, row, fz.rows, fz.m,
                                                  fz.row0_pos, fz.first_entry, s_cz, s_cz + 256, s_cz + 512,
                                                  reinterpret_cast<float*>(s_mm));
    else
      csa_compress_body::compress_one<uint16_t, 256>(fz.jobs.j[0], fz.jobs.theta[0], 0, row, fz.rows, fz.m,
                                                     fz.row0_pos, fz.first_entry, s_cz, s_cz + 256, s_cz + 512,
                                                     reinterpret_cast<float*>(s_mm));
    return;
  }
  const int b = row / T;
  const int r = row - b * T;
  // The chunk's scores, the row's bound keys and the position go out in one round of loads: the first two
  // do not depend on the position (the chunk is read whole and its entries past the visible range are
  // dropped once the position is known), and the position is a vector load whose zero offset is hidden
  // from the compiler (as a scalar load it would be waited for before the others are issued).
  int zoff = 0;
  asm volatile("" : "+v"(zoff));
  const int64_t p0v = pos0[b + zoff];
  // tau from the bound keys (held in registers when they fit)
  const uint32_t* brow = bound + (int64_t)row * nb;
  // up to KBK * 256 keys stay in registers (8: caches up to 2^18 entries with one bound set per 256 entries;
  // 16: up to 2^19), the register count chosen by the launch so that the common case keeps its occupancy
  constexpr int kBk = KBK;
  const bool breg = nb <= kBk * kSplitThreads;  // (uniform)
  uint32_t bk[kBk];
  if (breg) {
#pragma unroll
    for (int i = 0; i < kBk; ++i) bk[i] = brow[min(tid + i * kSplitThreads, nb - 1)];
  }
  // (issued after the bound keys: converting the chunk's scores waits for its loads)
  const ScoreRow srow = score_row(scores, sbf16, row, n_max);
  const int lo = blockIdx.x * kChunk;
  ChunkKeys ck = load_chunk(srow, lo, lo + kChunk, n_max);
  const int64_t t = (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(p0v >> 32)) << 32) |
                              (uint32_t)__builtin_amdgcn_readfirstlane((int)p0v)) + r;
  const int V = (int)visible_entries(t, m, n_max);
  const int K = k < V ? k : V;
  if (K == V) return;                          // the finishing launch writes the trivial row
  const int nact = (V + kChunk - 1) / kChunk;  // chunks holding visible entries
  if ((int)blockIdx.x >= nact) return;
  const int hi = min(lo + kChunk, V);
#pragma unroll
  for (int e = 0; e < kPerThread; ++e) ck.valid[e] = lo + kPerThread * tid + e < hi;

  // A zero key stands for "no entry" (sets with fewer than two visible entries, e.g. the tail of a cache
  // with room to grow): the key range, and so the radix pass's resolution, spans the real keys only, and
  // the bound is used only when at least K of them exist (else every visible entry is a candidate).
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u, nz = 0u;
  if (breg) {
#pragma unroll
    for (int i = 0; i < kBk; ++i)
      if (tid + i * kSplitThreads < nb && bk[i] != 0u) {
        kmin = min(kmin, bk[i]);
        kmax = max(kmax, bk[i]);
        ++nz;
      }
  } else {
    for (int j = tid; j < nb; j += kSplitThreads) {
      const uint32_t kk = brow[j];
      if (kk != 0u) {
        kmin = min(kmin, kk);
        kmax = max(kmax, kk);
        ++nz;
      }
    }
  }
  if (tid == 0) s_nz = 0u;
  __syncthreads();
  nz = wave_incl_sum(nz);
  if ((tid & 63) == 63) atomicAdd(&s_nz, nz);
  block_minmax<kSplitThreads>(kmin, kmax, s_mm);  // (its barriers also order the count)
  const bool usable = s_nz >= (uint32_t)K;       // (uniform)
  int known = usable ? common_bits(kmin, kmax) : 32, need = K;
  uint32_t tau = usable ? kmax : 0u;
  auto each_bound = [&](auto f) {
    if (breg) {
#pragma unroll
      for (int i = 0; i < kBk; ++i)
        if (tid + i * kSplitThreads < nb) f(bk[i]);
    } else {
      for (int j = tid; j < nb; j += kSplitThreads) f(brow[j]);
    }
  };
  // at least one radix pass, and a second while tau carries fewer than 16 resolved bits (a low outlier key,
  // a run of all-zero scores say, can leave only the sign or exponent in common): 16 bits keep the keys
  // between tau and the row's K-th key to a few per cent of K for smooth score distributions
  for (bool first = true; known < 32 && (first || known < 16); first = false)
    radix_step<kSplitThreads>(each_bound, tau, known, need, s_hist, s_w, s_sel);
  const uint32_t pmask = known >= 32 ? 0xFFFFFFFFu : ~((1u << (32 - known)) - 1u);
  tau &= pmask;

  uint32_t c_tot, g_tot;
  compact_chunk(ck, lo, tau, pmask, ws.seg + (int64_t)row * n_max,
                ws.blk + ((int64_t)row * nch + blockIdx.x) * kBlk, s_w, c_tot, g_tot);
  if (tid == 0) {
    ws.cnt[(int64_t)row * nch + blockIdx.x] = (g_tot << 16) | c_tot;
    if (blockIdx.x == 0) {  // (every chunk derives the same tau)
      ws.info[row * 4 + 0] = tau;
      ws.info[row * 4 + 1] = (uint32_t)known;
    }
  }
}

constexpr int kFinishCap = 4096;  // candidates the finishing workgroup holds in LDS
constexpr int kWaveSel = 64;      // K* is resolved by one wave once its bucket holds at most this many keys
constexpr int kSlotsMin = 16;     // compact-block slots per finishing thread for rows of up to 64 chunks

// The need-th largest among the keys of [lo, hi) in LDS that agree with pv on its top `known` bits (at most
// kWaveSel of them), one bit at a time by one wave: count the keys that extend the resolved prefix with a 1;
// if at least `need` do, the bit is 1, else those keys all rank above and the bit is 0.  On return pv is
// that key and need the number of keys equal to it still to take.  Called by every lane of one wave.
CSA_DEV void wave_select(const uint32_t* keys, int n, uint32_t& pv, int known, int& need) {
  const int lane = threadIdx.x & 63;
  const uint32_t kk = lane < n ? keys[lane] : 0u;
  const bool valid = lane < n;
  pv &= known == 0 ? 0u : ~0u << (32 - known);
  for (int bit = 31 - known; bit >= 0; --bit) {
    const uint32_t want = (pv >> bit) | 1u;
    const int c = (int)__popcll(__ballot(valid && (kk >> bit) == want));
    if (c >= need)
      pv |= 1u << bit;
    else
      need -= c;
  }
}

template <int SLOTS>
__global__ __launch_bounds__(kSplitThreads) void topk_bound_finish_kernel(
    const void* __restrict__ scores, int sbf16, int T, int64_t n_max, const int64_t* __restrict__ pos0, int m, int k,
    int32_t* __restrict__ idx, float* __restrict__ vals, SplitWs ws) {
  // The work per workgroup is small and its code runs once per launch, so the code is kept short: the
  // candidates are staged once in LDS and every later phase is a rolled loop over them.
  __shared__ uint32_t s_key[kFinishCap];
  __shared__ int32_t s_idx[kFinishCap];
  __shared__ __align__(16) uint32_t s_hist[kBins];
  __shared__ int s_pre[kBoundMaxChunks + 1];
  __shared__ int s_n[kBoundMaxChunks];
  __shared__ uint32_t s_w[2 * kSplitThreads / 64];
  __shared__ uint32_t s_k[kWaveSel];
  __shared__ int s_sel[2];
  __shared__ int s_m;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int row = blockIdx.x;
  const int nch = (int)((n_max + kChunk - 1) / kChunk);
  const int b = row / T;
  const int r = row - b * T;
  const uint32_t* cnt = ws.cnt + (int64_t)row * nch;
  const Cand* blk = ws.blk + (int64_t)row * nch * kBlk;
  const Cand* seg = ws.seg + (int64_t)row * n_max;
  // One round of loads, with the position (a vector load whose zero offset is hidden from the compiler, so
  // that it is not a scalar load waited for before the others are issued): this thread's chunk count, the
  // row's tau, and (rows of at most 256 / kParts chunks) slots [SLOTS t, SLOTS t + SLOTS) of the compact
  // blocks, i.e. part t % kParts of chunk t / kParts's block (SLOTS = 16: 64 chunks, the caches up to 2^18
  // entries; 32: 128 chunks).  Every chunk of the cache is read; those past the visible range are dropped
  // once the position is known.  Counts are clamped to a chunk's size.
  constexpr int kSlots = SLOTS;
  constexpr int kParts = kBlk / kSlots;  // threads per chunk block
  int zoff = 0;
  asm volatile("" : "+v"(zoff));
  const int64_t p0v = pos0[b + zoff];
  const bool spec = nch * kParts <= kSplitThreads;  // (uniform) every chunk's block slots fit the threads
  const uint32_t cv_all = tid < nch ? cnt[tid] : 0u;
  const uint32_t tau = ws.info[row * 4 + 0];
  int known = (int)ws.info[row * 4 + 1];
  const int ch = tid / kParts;
  u32x4 mine[kSlots / 2];
  if (spec && ch < nch) {
#pragma unroll
    for (int j = 0; j < kSlots / 2; ++j) mine[j] = reinterpret_cast<const u32x4*>(blk + (int64_t)tid * kSlots)[j];
  }
  const int64_t t = (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(p0v >> 32)) << 32) |
                              (uint32_t)__builtin_amdgcn_readfirstlane((int)p0v)) + r;
  const int V = (int)visible_entries(t, m, n_max);
  const int K = k < V ? k : V;
  const ScoreRow srow = score_row(scores, sbf16, row, n_max);
  int32_t* orow = idx + (int64_t)row * k;
  float* vrow = vals ? vals + (int64_t)row * k : nullptr;
  if (K == V) {
    trivial_row(srow, V, k, kSplitThreads, orow, vrow);
    return;
  }
  const int nact = (V + kChunk - 1) / kChunk;  // <= kBoundMaxChunks = the thread count
  const bool regs = nact * kParts <= kSplitThreads;  // (uniform)
  const uint32_t cv = tid < nact ? cv_all : 0u;
  if (regs && !spec && ch < nact) {   // (a cache with room for more chunks than the slots hold: a second round)
#pragma unroll
    for (int j = 0; j < kSlots / 2; ++j) mine[j] = reinterpret_cast<const u32x4*>(blk + (int64_t)tid * kSlots)[j];
  }
  const uint32_t n_c = min(cv & 0xFFFFu, (uint32_t)kChunk), g_c = min(cv >> 16, (uint32_t)kChunk);
  uint32_t pre, gpre, C, G;
  block_excl_sum2<kSplitThreads>(n_c, g_c, s_w, pre, gpre, C, G);
  if (tid < nact) {
    s_pre[tid] = (int)pre;
    s_n[tid] = (int)n_c;
  }
  if (tid == 0) s_m = 0;
  __syncthreads();
  if ((int)C < K || (int)C > kFinishCap) {  // (uniform) the bound did not prune: the full selection
    row_select<kSplitThreads>(srow, V, K, k, orow, vrow, s_hist, nullptr, s_w, s_sel);
    return;
  }
  // ---- the candidates into LDS in index order (chunk order is index order): the register-held block
  // slots, then whatever the blocks did not hold (the segments' overflow; every block when not loaded)
  if (regs && ch < nact) {
    const int n = s_n[ch], base = s_pre[ch], i0 = (tid % kParts) * kSlots;
#pragma unroll
    for (int j = 0; j < kSlots / 2; ++j) {
      if (i0 + 2 * j < n) {
        s_key[base + i0 + 2 * j] = mine[j][0];
        s_idx[base + i0 + 2 * j] = (int32_t)mine[j][1];
      }
      if (i0 + 2 * j + 1 < n) {
        s_key[base + i0 + 2 * j + 1] = mine[j][2];
        s_idx[base + i0 + 2 * j + 1] = (int32_t)mine[j][3];
      }
    }
  }
  if (__syncthreads_or(!regs || n_c > (uint32_t)kBlk)) {  // (uniform)
    const int from = regs ? kBlk : 0;
    for (int c = wave; c < nact; c += kSplitThreads / 64) {
      const int n = s_n[c], base = s_pre[c];  // (wave-uniform)
      for (int i = from + lane; i < n; i += 64) {
        const Cand cd = i < kBlk ? blk[(int64_t)c * kBlk + i] : seg[(int64_t)c * kChunk + i];
        s_key[base + i] = cd.key;
        s_idx[base + i] = cd.idx;
      }
    }
    __syncthreads();
  }
  const int nc = (int)C;
  auto each = [&](auto f) {
    for (int i = tid; i < nc; i += kSplitThreads) f(s_key[i]);
  };

  // ---- the K-th key among the C candidates: block radix passes while more than kWaveSel candidates share
  // the resolved prefix, then one wave resolves the remaining bits among those
  uint32_t kstar = tau;
  int need = K, inbucket;
  if ((int)G < K) {
    need = K - (int)G;  // the K-th key shares tau's prefix, as do C - G candidates
    inbucket = nc - (int)G;
  } else {  // the candidates' range decides the first open bit
    uint32_t lo = 0xFFFFFFFFu, hi = 0u;
    each([&](uint32_t kk) {
      lo = min(lo, kk);
      hi = max(hi, kk);
    });
    block_minmax<kSplitThreads>(lo, hi, s_w);
    kstar = hi;
    known = common_bits(lo, hi);
    inbucket = nc;
  }
  while (known < 32 && inbucket > kWaveSel) {
    radix_step<kSplitThreads>(each, kstar, known, need, s_hist, s_w, s_sel);
    inbucket = (int)s_hist[(kstar >> (32 - known)) & 0x7FFu];  // the chosen digit's count
    __syncthreads();                                           // (read before the next pass clears it)
  }
  if (known < 32) {  // (uniform) gather the bucket and finish in wave 0
    const uint32_t hmask = known == 0 ? 0u : ~0u << (32 - known);
    const uint32_t hp = kstar & hmask;
    each([&](uint32_t kk) {
      if ((kk & hmask) == hp) {
        const int slot = atomicAdd(&s_m, 1);
        if (slot < kWaveSel) s_k[slot] = kk;  // (the bucket holds at most kWaveSel keys)
      }
    });
    __syncthreads();
    if (wave == 0) {
      wave_select(s_k, min(s_m, kWaveSel), kstar, known, need);
      if (lane == 0) {
        s_sel[0] = (int)kstar;
        s_sel[1] = need;
      }
    }
    __syncthreads();
    kstar = (uint32_t)s_sel[0];
    need = s_sel[1];
  }
  const int ties = need;  // keys equal to K* still to take, lowest index first

  // ---- ordered output: thread t takes a contiguous range of the candidates; its first selected one lands
  // after the larger keys of earlier threads and the equal keys they take
  const int per = (nc + kSplitThreads - 1) / kSplitThreads;
  const int j0 = min(tid * per, nc), j1 = min(j0 + per, nc);
  uint32_t n_gt = 0, n_eq = 0;
  for (int j = j0; j < j1; ++j) {
    const uint32_t kk = s_key[j];
    n_gt += kk > kstar;
    n_eq += kk == kstar;
  }
  uint32_t gt_base, eq_base, gt_tot, eq_tot;
  block_excl_sum2<kSplitThreads>(n_gt, n_eq, s_w, gt_base, eq_base, gt_tot, eq_tot);
  int pos = (int)gt_base + min((int)eq_base, ties);
  int eq_rank = (int)eq_base;
  for (int j = j0; j < j1; ++j) {
    const uint32_t kk = s_key[j];
    bool sel = kk > kstar;
    if (kk == kstar) sel = eq_rank++ < ties;
    if (sel && pos < K) {
      orow[pos] = s_idx[j];
      if (vrow) vrow[pos] = key_to_score(kk);
    }
    pos += sel ? 1 : 0;
  }
  for (int j = K + tid; j < k; j += kSplitThreads) {
    orow[j] = -1;
    if (vrow) vrow[j] = -INFINITY;
  }
}

// ------------------------------------------------------------------ row path with bound keys
// Many rows (prefill) with the indexer's bound keys: one workgroup per row, no cross-workgroup work.
// tau (the K-th largest bound key with 22 bits resolved, derived as on the split path) never exceeds the
// row's K-th largest key, so one streaming pass over the row keeps every key that can be selected: each
// thread takes kRBPer consecutive keys of a chunk and one block scan writes the chunk's candidates into
// LDS in index order.  The K-th key is then resolved among the candidates alone and the ascending list
// written from them.  A row whose bound is unusable (fewer than K real keys) or whose candidates overflow
// the LDS buffer takes the full three-pass selection over all its keys, so the result is exact for any bound.
constexpr int kRBThreads = 256;                     // small workgroups: six rows in flight per CU
constexpr int kRBPer = 16;                          // consecutive keys per thread and chunk
constexpr int kRBChunk = kRBThreads * kRBPer;       // 4096 keys per chunk
constexpr int kRBCap = 2048;                        // candidates held in LDS
constexpr int kRBKeys = 16;                         // bound keys per thread (registers): up to 4096 per row

__global__ __launch_bounds__(kRBThreads) void topk_rowbound_kernel(
    const void* __restrict__ scores, int sbf16, int T, int64_t n_max, const int64_t* __restrict__ pos0, int m,
    int k, const uint32_t* __restrict__ bound, int nb, int32_t* __restrict__ idx, float* __restrict__ vals) {
  __shared__ __align__(16) Cand s_c[kRBCap];
  __shared__ uint32_t s_hist[kBins];
  __shared__ uint32_t s_w[2 * kRBThreads / 64];
  __shared__ uint32_t s_mm[2 * kRBThreads / 64];
  __shared__ int s_sel[2];
  __shared__ uint32_t s_nz;
  constexpr int NT = kRBThreads;
  const int tid = threadIdx.x;
  const int row = blockIdx.x;
  const int b = row / T;
  const int r = row - b * T;
  const int V = (int)visible_entries(pos0[b] + r, m, n_max);
  const int K = k < V ? k : V;
  const ScoreRow srow = score_row(scores, sbf16, row, n_max);
  int32_t* orow = idx + (int64_t)row * k;
  float* vrow = vals ? vals + (int64_t)row * k : nullptr;
  if (K == V) {
    trivial_row(srow, V, k, NT, orow, vrow);
    return;
  }

  // ---- tau from the row's bound keys (zero keys stand for "no entry")
  const uint32_t* brow = bound + (int64_t)row * nb;
  uint32_t bk[kRBKeys];
#pragma unroll
  for (int i = 0; i < kRBKeys; ++i) bk[i] = brow[min(tid + i * NT, nb - 1)];
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u, nz = 0u;
#pragma unroll
  for (int i = 0; i < kRBKeys; ++i)
    if (tid + i * NT < nb && bk[i] != 0u) {
      kmin = min(kmin, bk[i]);
      kmax = max(kmax, bk[i]);
      ++nz;
    }
  if (tid == 0) s_nz = 0u;
  __syncthreads();
  nz = wave_incl_sum(nz);
  if ((tid & 63) == 63) atomicAdd(&s_nz, nz);
  block_minmax<NT>(kmin, kmax, s_mm);  // (its barriers also order the count)
  const bool usable = s_nz >= (uint32_t)K;
  int known = usable ? common_bits(kmin, kmax) : 32, need = K;
  uint32_t tau = usable ? kmax : 0u;
  auto each_bound = [&](auto f) {
#pragma unroll
    for (int i = 0; i < kRBKeys; ++i)
      if (tid + i * NT < nb) f(bk[i]);
  };
  while (known < 22) radix_step<NT>(each_bound, tau, known, need, s_hist, s_w, s_sel);
  const uint32_t pmask = known >= 32 ? 0xFFFFFFFFu : ~((1u << (32 - known)) - 1u);
  tau &= pmask;

  // ---- one pass over the row: candidates (keys >= tau) into LDS in index order
  int C = 0, G = 0;  // candidates so far, and those whose prefix lies above tau's (uniform)
  for (int lo = 0; lo < V; lo += kRBChunk) {
    const int i0 = lo + kRBPer * tid;
    uint32_t key[kRBPer];
    if (!sbf16 && (n_max & 3) == 0) {
      f32x4 x[kRBPer / 4];
#pragma unroll
      for (int j = 0; j < kRBPer / 4; ++j) {
        const int64_t p = min((int64_t)i0 + 4 * j, n_max - 4);
        x[j] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(static_cast<const float*>(srow.p) + p));
      }
#pragma unroll
      for (int j = 0; j < kRBPer / 4; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) key[4 * j + q] = score_key(x[j][q]);
    } else {
#pragma unroll
      for (int e = 0; e < kRBPer; ++e) key[e] = srow.key(min((int64_t)i0 + e, n_max - 1));
    }
    uint32_t c_t = 0, g_t = 0;
#pragma unroll
    for (int e = 0; e < kRBPer; ++e) {
      const bool cand = i0 + e < V && key[e] >= tau;
      c_t += cand;
      g_t += cand && (key[e] & pmask) > tau;
    }
    uint32_t c_pre, g_pre, c_tot, g_tot;
    block_excl_sum2<NT>(c_t, g_t, s_w, c_pre, g_pre, c_tot, g_tot);
    int p = C + (int)c_pre;
#pragma unroll
    for (int e = 0; e < kRBPer; ++e)
      if (i0 + e < V && key[e] >= tau) {
        if (p < kRBCap) s_c[p] = Cand{key[e], i0 + e};
        ++p;
      }
    C += (int)c_tot;
    G += (int)g_tot;
  }
  __syncthreads();
  if (C > kRBCap || C < K) {  // (uniform) the bound did not prune enough: the full selection
    row_select<NT>(srow, V, K, k, orow, vrow, s_hist, nullptr, s_w, s_sel);
    return;
  }

  // ---- the K-th key among the candidates: thread t holds candidates [j0, j1) in registers
  constexpr int kReg = kRBCap / NT;  // 8
  const int per = (C + NT - 1) / NT;
  const int j0 = min(tid * per, C), j1 = min(j0 + per, C);
  uint32_t rk[kReg];
  int32_t ri[kReg];
#pragma unroll
  for (int i = 0; i < kReg; ++i) {
    const Cand cd = s_c[min(j0 + i, kRBCap - 1)];
    rk[i] = cd.key;
    ri[i] = cd.idx;
  }
  auto each = [&](auto f) {
#pragma unroll
    for (int i = 0; i < kReg; ++i)
      if (j0 + i < j1) f(rk[i]);
  };
  uint32_t kstar = tau;
  if (G < K) {
    need = K - G;  // the K-th key shares tau's prefix
  } else {         // the candidates' range decides the first open bit
    uint32_t lo = 0xFFFFFFFFu, hi = 0u;
    each([&](uint32_t kk) {
      lo = min(lo, kk);
      hi = max(hi, kk);
    });
    block_minmax<NT>(lo, hi, s_mm);
    kstar = hi;
    known = common_bits(lo, hi);
    need = K;
  }
  while (known < 32) radix_step<NT>(each, kstar, known, need, s_hist, s_w, s_sel);
  const int ties = need;  // keys equal to K* still to take, lowest index first

  // ---- ordered output: a thread's first selected candidate lands after the larger keys of earlier threads
  // and the equal keys they take
  uint32_t n_gt = 0, n_eq = 0;
  each([&](uint32_t kk) {
    n_gt += kk > kstar;
    n_eq += kk == kstar;
  });
  uint32_t gt_base, eq_base, gt_tot, eq_tot;
  block_excl_sum2<NT>(n_gt, n_eq, s_w, gt_base, eq_base, gt_tot, eq_tot);
  int pos = (int)gt_base + min((int)eq_base, ties);
  int eq_rank = (int)eq_base;
#pragma unroll
  for (int i = 0; i < kReg; ++i) {
    if (j0 + i >= j1) break;
    const uint32_t kk = rk[i];
    bool sel = kk > kstar;
    if (kk == kstar) sel = eq_rank++ < ties;
    if (sel && pos < K) {
      orow[pos] = ri[i];
      if (vrow) vrow[pos] = key_to_score(kk);
    }
    pos += sel ? 1 : 0;
  }
  for (int j = K + tid; j < k; j += NT) {
    orow[j] = -1;
    if (vrow) vrow[j] = -INFINITY;
  }
}

bool use_split(int rows, int64_t n_max) {
  const int64_t nch = (n_max + kChunk - 1) / kChunk;
  return rows < kSplitMaxRows && n_max > 16384 && nch <= kMaxChunks;
}

}  // namespace

size_t topk_workspace_bytes(int B, int T, int64_t n_max, int k) {
  (void)k;
  const int rows = B * T;
  if (!use_split(rows, n_max)) return 0;
  return split_bytes(rows, n_max, ceil_div(n_max, kChunk));
}

csa_status launch_topk(const void* scores, int score_t, int B, int T, int64_t n_max, const int64_t* pos0, int m, int k,
                       const uint32_t* bound, int32_t* idx, float* vals, void* ws, hipStream_t stream,
                       const CompressJob* kv, int kv_rows, int kv_m, int64_t kv_row0, int64_t kv_first, int kv_in_t) {
  if (kv && !(use_split(B * T, n_max) && bound && index_bound_keys(n_max) >= 2 * (int64_t)k &&
              ceil_div(n_max, kChunk) <= kBoundMaxChunks)) {
    // no bound-key launch to carry it: the entry is compressed by a launch of its own first
    const csa_status st = launch_compress_jobs(kv, 1, B, kv_rows, kv_m, kv_row0, kv_first, 1, kv_in_t, stream);
    if (st != CSA_OK) return st;
    kv = nullptr;
  }
  const int rows = B * T;
  const int sbf16 = score_t == CSA_BF16 ? 1 : 0;
  if (use_split(rows, n_max)) {
    const int nch = ceil_div(n_max, kChunk);
    SplitWs s = carve(ws, rows, n_max, nch);
    dim3 grid(nch, rows);
    // bound keys help only when there are enough of them (a K-th largest well inside their range)
    const bool bounded = bound && index_bound_keys(n_max) >= 2 * (int64_t)k && nch <= kBoundMaxChunks;
    if (bounded) {
      const int nb = (int)index_bound_keys(n_max);
      TopkFuse fz{};
      if (kv) {  // one more workgroup per row computes the row's new KV entry
        csa_compress_body::fill_jobs(kv, 1, fz.jobs);
        fz.on = 1;
        fz.rows = kv_rows;
        fz.m = kv_m;
        fz.in_t = kv_in_t;
        fz.row0_pos = kv_row0;
        fz.first_entry = kv_first;
        grid.x += 1;
      }
      if (nb <= 8 * kSplitThreads)
        hipLaunchKernelGGL((topk_bound_collect_kernel<8>), grid, dim3(kSplitThreads), 0, stream, scores, sbf16, T,
                           n_max, pos0, m, k, bound, nb, s, fz);
      else
        hipLaunchKernelGGL((topk_bound_collect_kernel<16>), grid, dim3(kSplitThreads), 0, stream, scores, sbf16, T,
                           n_max, pos0, m, k, bound, nb, s, fz);
      if (nch <= kSplitThreads * kSlotsMin / kBlk)
        hipLaunchKernelGGL((topk_bound_finish_kernel<kSlotsMin>), dim3(rows), dim3(kSplitThreads), 0, stream, scores,
                           sbf16, T, n_max, pos0, m, k, idx, vals, s);
      else
        hipLaunchKernelGGL((topk_bound_finish_kernel<2 * kSlotsMin>), dim3(rows), dim3(kSplitThreads), 0, stream,
                           scores, sbf16, T, n_max, pos0, m, k, idx, vals, s);
      return hipGetLastError() == hipSuccess ? CSA_OK : CSA_ERR_LAUNCH;
    } else {
      hipLaunchKernelGGL(topk_split_hist_kernel, grid, dim3(kSplitThreads), 0, stream, scores, sbf16, T, n_max, pos0,
                         m, k, s);
      hipLaunchKernelGGL(topk_split_hist1_kernel, grid, dim3(kSplitThreads), 0, stream, scores, sbf16, T, n_max, pos0,
                         m, k, s);
      hipLaunchKernelGGL(topk_split_collect_kernel, grid, dim3(kSplitThreads), 0, stream, scores, sbf16, T, n_max,
                         pos0, m, k, s);
      hipLaunchKernelGGL(topk_split_finish_kernel, dim3(rows), dim3(kSplitThreads), 0, stream, scores, sbf16, T,
                         n_max, pos0, m, k, nch, idx, vals, s);
    }
  } else if (bound && index_bound_keys(n_max) >= 2 * (int64_t)k && index_bound_keys(n_max) <= kRBKeys * kRBThreads) {
    // many rows with the indexer's bound keys: one pruning pass per row
    hipLaunchKernelGGL(topk_rowbound_kernel, dim3(rows), dim3(kRBThreads), 0, stream, scores, sbf16, T, n_max, pos0,
                       m, k, bound, (int)index_bound_keys(n_max), idx, vals);
  } else {
    const int cache = n_max <= kRowKeyCap ? 1 : 0;
    size_t lds = (size_t)kBins * 4 + (cache ? (size_t)n_max * 4 : 0);
    static bool attr_set = false;
    if (!attr_set) {
      if (hipFuncSetAttribute((const void*)topk_row_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)((size_t)kBins * 4 + (size_t)kRowKeyCap * 4)) != hipSuccess)
        return CSA_ERR_LAUNCH;
      attr_set = true;
    }
    hipLaunchKernelGGL(topk_row_kernel, dim3(rows), dim3(kRowThreads), lds, stream, scores, sbf16, T, n_max, pos0, m, k,
                       idx, vals, cache);
  }
  return hipGetLastError() == hipSuccess ? CSA_OK : CSA_ERR_LAUNCH;
}
