// csa_topk kernels: exact top-k with a lower-index tie-break, ascending output.
//
// "【论文解读】DeepSeek-V4" (wkq9411.github.io), section 一(三)1(2): the selector
// keeps the compressed entries whose index scores are in Top-k(I_{t,:}); section
// 二(四) notes the selector's cost (BF16 scores made it 2x faster).
//
// Scores become order-preserving uint32 keys (+0 == -0).  A three-digit radix
// select (11 + 11 + 10 bits) finds the k-th key K*; the result is every key > K*
// plus the lowest-index keys == K*, emitted by an ordered (index-order) block
// compaction, so no sort is needed.
//
//  * Row path (many rows, e.g. prefill): one 512-thread workgroup per row; keys
//    cached in LDS when the row fits (<= 32768 entries).
//  * Split path (few long rows, decode): chunks of 4096 scores per workgroup.
//    Kernel 1 builds the top-digit histogram (LDS, then integer atomics into a
//    per-row global histogram).  Kernel 2: each workgroup derives the threshold
//    digit d0 from it and builds the second-digit histogram of the keys in that
//    bin.  Kernel 3: each workgroup derives the 22-bit threshold prefix and
//    compacts its chunk's keys at or above it into its own segment, in index
//    order (about k candidates in total).  Kernel 4 (one workgroup per row) loads
//    all segments (chunk order = index order) into LDS, resolves the last digit,
//    writes the ordered output and clears the first histogram.  Kernel boundaries carry
//    the cross-workgroup hand-offs, so no workgroup waits on another or issues a
//    device-wide fence; integer atomics make the result independent of
//    scheduling, and the workspace is left zero-filled.
#include "csa_common.h"
#include "csa_internal.h"

namespace {

constexpr int kBins = 2048;
constexpr int kChunk = 4096;          // scores per workgroup on the split path
constexpr int kSplitThreads = 256;
constexpr int kRowThreads = 512;
constexpr int kRowKeyCap = 32768;     // keys cached in LDS on the row path
constexpr int kSegCap = 6144;         // candidates cached in LDS by the finishing workgroup
constexpr int kMaxChunks = 2048;

// ------------------------------------------------------------------ block scans
// Exclusive prefix of a 0/1 flag over the block (in thread order) and its total.
template <int NT>
CSA_DEV int block_flag_scan(bool flag, int* s_w, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint64_t bal = __ballot(flag);
  const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0));
  if (lane == 0) s_w[wave] = __popcll(bal);
  __syncthreads();
  int pre = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    int v = s_w[w];
    pre += (w < wave) ? v : 0;
    tot += v;
  }
  __syncthreads();
  total = tot;
  return pre + below;
}

// Exclusive prefix of an int over the block in thread order.
template <int NT>
CSA_DEV int block_int_scan(int v, int* s_w, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) s_w[wave] = x;
  __syncthreads();
  int pre = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    int s = s_w[w];
    pre += (w < wave) ? s : 0;
    tot += s;
  }
  __syncthreads();
  total = tot;
  return pre + x - v;
}

// Given hist[nb] (counts per digit) and need >= 1, find the digit d with
// count(> d) < need <= count(>= d).  Writes d and count(> d) to out[0..1].
template <int NT>
CSA_DEV void select_digit(const uint32_t* hist, int nb, int need, int* s_w, int* out) {
  const int bpt = nb / NT;  // nb is a multiple of NT
  const int tid = threadIdx.x;
  const int u = NT - 1 - tid;  // thread u owns the bins of thread tid counted from the top
  int local = 0;
  for (int j = 0; j < bpt; ++j) local += hist[tid * bpt + j];
  // suffix sums: scan in reversed thread order
  int total;
  // exchange local through LDS to scan in reversed order
  __shared__ int s_rev[kRowThreads];
  s_rev[u] = local;
  __syncthreads();
  int mine = s_rev[tid];  // thread tid now holds the count of original thread NT-1-tid
  int excl = block_int_scan<NT>(mine, s_w, total);
  // original thread o = NT-1-tid has count(bins above its range) = excl
  s_rev[NT - 1 - tid] = excl;
  __syncthreads();
  int above = s_rev[tid];
  if (above < need && above + local >= need) {
    for (int j = bpt - 1; j >= 0; --j) {
      int h = hist[tid * bpt + j];
      if (above + h >= need) {
        out[0] = tid * bpt + j;
        out[1] = above;
        break;
      }
      above += h;
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
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    lo = min(lo, (uint32_t)__shfl_xor((int)lo, o, 64));
    hi = max(hi, (uint32_t)__shfl_xor((int)hi, o, 64));
  }
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

// Radix step over the keys between lo and hi (inclusive) that agree with pv on their top `known` bits:
// histogram of the 11 bits ending at `shift` (bits already known among them take one value), and the
// digit of the need-th largest.  Updates pv (those 11 bits), need (minus the keys above the digit) and
// known.  get(j) returns the j-th key, j < n.
template <typename Get>
CSA_DEV void radix_step(Get get, int n, uint32_t& pv, int& known, int& need, uint32_t* hist, int* s_w, int* s_sel) {
  const int shift = max(0, 32 - known - 11);
  for (int j = threadIdx.x; j < kBins; j += kSplitThreads) hist[j] = 0;
  __syncthreads();
  for (int j = threadIdx.x; j < n; j += kSplitThreads) {
    const uint32_t kk = get(j);
    if (known == 0 || (kk >> (32 - known)) == (pv >> (32 - known))) atomicAdd(&hist[(kk >> shift) & 0x7FFu], 1u);
  }
  __syncthreads();
  select_digit<kSplitThreads>(hist, kBins, need, s_w, s_sel);
  pv = (pv & ~(0x7FFu << shift)) | ((uint32_t)s_sel[0] << shift);
  need -= s_sel[1];
  known = 32 - shift;
}

// Bits shared by every key in [lo, hi] (lo <= hi), and those bits as a prefix value.
CSA_DEV int common_bits(uint32_t lo, uint32_t hi) { return lo == hi ? 32 : __clz(lo ^ hi); }

// ------------------------------------------------------------------ row path
__global__ __launch_bounds__(kRowThreads) void topk_row_kernel(const void* __restrict__ scores, int sbf16, int T,
                                                               int64_t n_max, const int64_t* __restrict__ pos0,
                                                               int m, int k, int32_t* __restrict__ idx,
                                                               float* __restrict__ vals, int cache_keys) {
  extern __shared__ uint32_t s_dyn[];
  uint32_t* hist = s_dyn;           // kBins
  uint32_t* keys = s_dyn + kBins;   // cache (when enabled)
  __shared__ int s_w[kRowThreads / 64];
  __shared__ int s_sel[2];

  const int tid = threadIdx.x;
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
    for (int j = tid; j < k; j += kRowThreads) {
      orow[j] = j < V ? j : -1;
      if (vrow) vrow[j] = j < V ? key_to_score(srow.key(j)) : -INFINITY;
    }
    return;
  }

  auto key_at = [&](int i) -> uint32_t { return cache_keys ? keys[i] : srow.key(i); };

  // digit 0: bits 31..21
  for (int j = tid; j < kBins; j += kRowThreads) hist[j] = 0;
  __syncthreads();
  for (int i = tid; i < V; i += kRowThreads) {
    uint32_t kk = srow.key(i);
    if (cache_keys) keys[i] = kk;
    atomicAdd(&hist[kk >> 21], 1u);
  }
  __syncthreads();
  select_digit<kRowThreads>(hist, kBins, K, s_w, s_sel);
  const uint32_t d0 = s_sel[0];
  int need = K - s_sel[1];
  __syncthreads();

  // digit 1: bits 20..10 among keys with digit 0 == d0
  for (int j = tid; j < kBins; j += kRowThreads) hist[j] = 0;
  __syncthreads();
  for (int i = tid; i < V; i += kRowThreads) {
    uint32_t kk = key_at(i);
    if ((kk >> 21) == d0) atomicAdd(&hist[(kk >> 10) & 0x7FFu], 1u);
  }
  __syncthreads();
  select_digit<kRowThreads>(hist, kBins, need, s_w, s_sel);
  const uint32_t p1 = (d0 << 11) | (uint32_t)s_sel[0];  // top 22 bits
  need -= s_sel[1];
  __syncthreads();

  // digit 2: bits 9..0 among keys with top 22 bits == p1
  for (int j = tid; j < kBins; j += kRowThreads) hist[j] = 0;
  __syncthreads();
  for (int i = tid; i < V; i += kRowThreads) {
    uint32_t kk = key_at(i);
    if ((kk >> 10) == p1) atomicAdd(&hist[kk & 0x3FFu], 1u);
  }
  __syncthreads();
  select_digit<kRowThreads>(hist, 1024, need, s_w, s_sel);
  const uint32_t kstar = (p1 << 10) | (uint32_t)s_sel[0];
  const int ties = need - s_sel[1];  // keys == K* to take, lowest indices first
  __syncthreads();

  // ordered compaction
  int out_base = 0, tie_base = 0;
  for (int c0 = 0; c0 < V && out_base < K; c0 += kRowThreads) {
    const int i = c0 + tid;
    uint32_t kk = i < V ? key_at(i) : 0u;
    const bool eq = (i < V) && kk == kstar;
    int eq_tot;
    int eq_rank = tie_base + block_flag_scan<kRowThreads>(eq, s_w, eq_tot);
    const bool sel = (i < V) && (kk > kstar || (eq && eq_rank < ties));
    int sel_tot;
    int pos = out_base + block_flag_scan<kRowThreads>(sel, s_w, sel_tot);
    if (sel) {
      orow[pos] = i;
      if (vrow) vrow[pos] = key_to_score(kk);
    }
    out_base += sel_tot;
    tie_base += eq_tot;
  }
  for (int j = K + tid; j < k; j += kRowThreads) {
    orow[j] = -1;
    if (vrow) vrow[j] = -INFINITY;
  }
}

// ------------------------------------------------------------------ split path
struct SplitWs {
  uint32_t* hist;     // [rows][kBins]   digit-0 histogram (zero at rest)
  uint32_t* hist1;    // [rows][kBins]   digit-1 histogram (cleared by kernel 1 of every call)
  uint32_t* info;     // [rows][4]
  uint32_t* cnt;      // [rows][nch]
  Cand* seg;          // [rows][n_max]
};

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// The split path serves fewer than kSplitMaxRows rows.  Its digit-0 histograms, the one region that
// must be zero at rest, take a fixed slot for that many rows at the start of the workspace, so that
// no call of another shape ever places them over memory that a previous call left dirty.
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
  return s;
}

static size_t split_bytes(int rows, int64_t n_max, int nch) {
  return kHistSlot + align256((size_t)rows * kBins * 4) + align256((size_t)rows * 16) +
         align256((size_t)rows * nch * 4) + align256((size_t)rows * n_max * sizeof(Cand));
}

// Each thread of a split-path workgroup owns 16 scores of its 4096-score chunk:
// round j (0..3) covers chunk positions [1024 j, 1024 j + 1024), thread t the 4
// consecutive positions 1024 j + 4 t + q.  All 16 loads are issued before any use.
constexpr int kPerThread = kChunk / kSplitThreads;  // 16
constexpr int kRounds = kPerThread / 4;             // 4

struct ChunkKeys {
  uint32_t key[kPerThread];
  bool valid[kPerThread];
};

CSA_DEV ChunkKeys load_chunk(const ScoreRow& srow, int lo, int hi, int64_t n_max) {
  // Addresses are clamped into the row so that every load is issued unconditionally (no branch
  // between loads); validity is applied afterwards from the unclamped positions.
  ChunkKeys c;
  const int t = threadIdx.x;
  if ((n_max & 3) == 0) {
    if (srow.bf16) {
      u32x2 x[kRounds];
#pragma unroll
      for (int j = 0; j < kRounds; ++j) {
        const int64_t i0 = min((int64_t)(lo + 1024 * j + 4 * t), n_max - 4);
        x[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(static_cast<const uint16_t*>(srow.p) + i0));
      }
#pragma unroll
      for (int j = 0; j < kRounds; ++j) {
        c.key[4 * j + 0] = score_key(__uint_as_float(x[j].x << 16));
        c.key[4 * j + 1] = score_key(__uint_as_float(x[j].x & 0xFFFF0000u));
        c.key[4 * j + 2] = score_key(__uint_as_float(x[j].y << 16));
        c.key[4 * j + 3] = score_key(__uint_as_float(x[j].y & 0xFFFF0000u));
      }
    } else {
      f32x4 x[kRounds];
#pragma unroll
      for (int j = 0; j < kRounds; ++j) {
        const int64_t i0 = min((int64_t)(lo + 1024 * j + 4 * t), n_max - 4);
        x[j] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(static_cast<const float*>(srow.p) + i0));
      }
#pragma unroll
      for (int j = 0; j < kRounds; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) c.key[4 * j + q] = score_key(x[j][q]);
    }
  } else {
#pragma unroll
    for (int e = 0; e < kPerThread; ++e)
      c.key[e] = srow.key(min((int64_t)(lo + 1024 * (e / 4) + 4 * t + (e % 4)), n_max - 1));
  }
#pragma unroll
  for (int j = 0; j < kRounds; ++j)
#pragma unroll
    for (int q = 0; q < 4; ++q) c.valid[4 * j + q] = lo + 1024 * j + 4 * t + q < hi;
  return c;
}

// Kernel 1: per-chunk histogram of the top key digit (bits 31..21), added into the row histogram;
// also clears the digit-1 histogram that kernel 2 fills.
__global__ __launch_bounds__(kSplitThreads) void topk_split_hist_kernel(const void* __restrict__ scores, int sbf16, int T,
                                                                        int64_t n_max,
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
__global__ __launch_bounds__(kSplitThreads) void topk_split_hist1_kernel(const void* __restrict__ scores, int sbf16, int T,
                                                                         int64_t n_max,
                                                                         const int64_t* __restrict__ pos0, int m,
                                                                         int k, SplitWs ws) {
  __shared__ uint32_t hist[kBins];
  __shared__ int s_w[kSplitThreads / 64];
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
  select_digit<kSplitThreads>(hist, kBins, K, s_w, s_sel);
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
__global__ __launch_bounds__(kSplitThreads) void topk_split_collect_kernel(const void* __restrict__ scores, int sbf16, int T,
                                                                           int64_t n_max,
                                                                           const int64_t* __restrict__ pos0, int m,
                                                                           int k, SplitWs ws) {
  __shared__ uint32_t hist[kBins];
  __shared__ int s_w[kSplitThreads / 64];
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
  select_digit<kSplitThreads>(hist, kBins, need, s_w, s_sel);
  const uint32_t p1 = (d0 << 11) | (uint32_t)s_sel[0];
  if (blockIdx.x == 0 && tid == 0) {
    ws.info[row * 4 + 2] = p1;
    ws.info[row * 4 + 3] = (uint32_t)(need - s_sel[1]);  // keys with prefix p1 still to take
  }
  int base = 0;
  if (lo < hi) {
    Cand* seg = ws.seg + (int64_t)row * n_max;
#pragma unroll
    for (int j = 0; j < kRounds; ++j) {
      int mine = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) mine += (ck.valid[4 * j + q] && (ck.key[4 * j + q] >> 10) >= p1) ? 1 : 0;
      int tot;
      int pos = base + block_int_scan<kSplitThreads>(mine, s_w, tot);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int e = 4 * j + q;
        if (ck.valid[e] && (ck.key[e] >> 10) >= p1) seg[lo + pos++] = Cand{ck.key[e], lo + 1024 * j + 4 * tid + q};
      }
      base += tot;
    }
  }
  if (tid == 0) ws.cnt[(int64_t)row * nch + blockIdx.x] = base;
}

// With bound keys from the indexer (two per 256-entry wave, each the key of a distinct visible
// entry), kernels 1 to 3 become one: every workgroup derives tau, the 22-bit floor of the K-th largest
// bound key (two digit passes over the row's bound keys), and compacts its chunk's keys >= tau into
// its segment, in index order.  tau never exceeds the row's K-th largest key, so every selected key is
// a candidate; typically about 1.1 k keys are.
__global__ __launch_bounds__(kSplitThreads) void topk_bound_collect_kernel(const void* __restrict__ scores, int sbf16, int T,
                                                                           int64_t n_max,
                                                                           const int64_t* __restrict__ pos0, int m,
                                                                           int k, const uint32_t* __restrict__ bound,
                                                                           int nb, SplitWs ws) {
  __shared__ uint32_t hist[kBins];
  __shared__ int s_w[kSplitThreads / 64];
  __shared__ int s_sel[2];
  __shared__ uint32_t s_mm[2 * kSplitThreads / 64];
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
  const uint32_t* brow = bound + (int64_t)row * nb;
  // tau: the K-th largest bound key with the bits below one 11-bit digit cleared, the digit taken right
  // under the bits that all bound keys share (so one pass resolves it closely)
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
  for (int j = tid; j < nb; j += kSplitThreads) {
    const uint32_t kk = brow[j];
    kmin = min(kmin, kk);
    kmax = max(kmax, kk);
  }
  block_minmax<kSplitThreads>(kmin, kmax, s_mm);
  int known = common_bits(kmin, kmax), need = K;
  uint32_t tau = kmax;
  if (known < 32) radix_step([&](int j) { return brow[j]; }, nb, tau, known, need, hist, s_w, s_sel);
  tau &= known >= 32 ? 0xFFFFFFFFu : ~((1u << (32 - known)) - 1u);
  int base = 0;
  if (lo < hi) {
    Cand* seg = ws.seg + (int64_t)row * n_max;
#pragma unroll
    for (int j = 0; j < kRounds; ++j) {
      int mine = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) mine += (ck.valid[4 * j + q] && ck.key[4 * j + q] >= tau) ? 1 : 0;
      int tot;
      int pos = base + block_int_scan<kSplitThreads>(mine, s_w, tot);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int e = 4 * j + q;
        if (ck.valid[e] && ck.key[e] >= tau) seg[lo + pos++] = Cand{ck.key[e], lo + 1024 * j + 4 * tid + q};
      }
      base += tot;
    }
  }
  if (tid == 0) ws.cnt[(int64_t)row * nch + blockIdx.x] = base;
}

// Kernel 4: one workgroup per row gathers the segments (chunk order == index order), resolves the
// remaining digits of the K-th key among them (the last digit after kernels 1 to 3, all three after
// the bound collect), and writes the ascending index list.  After kernels 1 to 3 it also clears the
// digit-0 histogram of the row.  If the candidates are fewer than K (bound keys that were not the
// indexer's), it selects from the whole visible row instead.
__global__ __launch_bounds__(kSplitThreads) void topk_split_finish_kernel(
    const void* __restrict__ scores, int sbf16, int T, int64_t n_max, const int64_t* __restrict__ pos0, int m, int k,
    int nch, int32_t* __restrict__ idx, float* __restrict__ vals, SplitWs ws, int bounded) {
  __shared__ Cand s_c[kSegCap];
  __shared__ uint32_t hist[kBins];
  __shared__ int s_w[kSplitThreads / 64];
  __shared__ int s_sel[2];
  __shared__ int s_pre[kMaxChunks + 1];
  __shared__ uint32_t s_mm[2 * kSplitThreads / 64];

  const int tid = threadIdx.x;
  const int row = blockIdx.x;
  const int b = row / T;
  const int r = row - b * T;
  const int V = (int)visible_entries(pos0[b] + r, m, n_max);
  const int K = k < V ? k : V;
  const ScoreRow srow = score_row(scores, sbf16, row, n_max);
  const Cand* seg = ws.seg + (int64_t)row * n_max;
  const uint32_t* cnt = ws.cnt + (int64_t)row * nch;
  int32_t* orow = idx + (int64_t)row * k;
  float* vrow = vals ? vals + (int64_t)row * k : nullptr;

  if (K == V) {
    for (int j = tid; j < k; j += kSplitThreads) {
      orow[j] = j < V ? j : -1;
      if (vrow) vrow[j] = j < V ? key_to_score(srow.key(j)) : -INFINITY;
    }
    return;
  }
  if (!bounded) {  // the digit-0 histogram is no longer needed: leave the workspace zero-filled
    uint32_t* ghist = ws.hist + (int64_t)row * kBins;
#pragma unroll
    for (int u = 0; u < kBins / kSplitThreads; ++u) ghist[tid + u * kSplitThreads] = 0;
  }

  // prefix over chunk counts (chunk order == index order); every load is issued before use
  {
    constexpr int kCpt = kMaxChunks / kSplitThreads;  // chunk counts per thread (8)
    const int cpt = (nch + kSplitThreads - 1) / kSplitThreads;
    const int c0 = tid * cpt;
    int cv[kCpt];
#pragma unroll
    for (int u = 0; u < kCpt; ++u) cv[u] = (u < cpt && c0 + u < nch) ? (int)cnt[c0 + u] : 0;
    int local = 0;
#pragma unroll
    for (int u = 0; u < kCpt; ++u) local += cv[u];
    int tot;
    int pre = block_int_scan<kSplitThreads>(local, s_w, tot);
#pragma unroll
    for (int u = 0; u < kCpt; ++u)
      if (u < cpt && c0 + u < nch) {
        s_pre[c0 + u] = pre;
        pre += cv[u];
      }
    if (tid == 0) s_pre[nch] = tot;
  }
  __syncthreads();
  const bool rescan = bounded && s_pre[nch] < K;  // (uniform) candidates from the whole visible row
  const int C = rescan ? V : s_pre[nch];
  const bool in_lds = !rescan && C <= kSegCap;
  auto chunk_of = [&](int j) -> int {  // c with s_pre[c] <= j < s_pre[c+1]
    int lo = 0, hi = nch;
    while (hi - lo > 1) {
      int mid = (lo + hi) >> 1;
      if (s_pre[mid] <= j) lo = mid; else hi = mid;
    }
    return lo;
  };
  auto cand_global = [&](int j) -> Cand {
    const int c = chunk_of(j);
    return seg[(int64_t)c * kChunk + (j - s_pre[c])];
  };
  if (in_lds) {
    // wave w copies the segments of chunks w, w + 4, ...: lane i takes element i (and i + 64, ... of
    // the rare chunk with more than 64 candidates); a batch of kBatch chunks is loaded before storing
    constexpr int kBatch = 16;
    const int lane = tid & 63, wave = tid >> 6;
    for (int c0 = wave; c0 < nch; c0 += 4 * kBatch) {
      Cand cv[kBatch];
      int dst[kBatch];
      int nmax = 0;
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int c = c0 + 4 * u;
        const int n = c < nch ? s_pre[c + 1] - s_pre[c] : 0;
        nmax = max(nmax, n);
        dst[u] = lane < n ? s_pre[c] + lane : -1;
        cv[u] = seg[(int64_t)(c < nch ? c : 0) * kChunk + (lane < n ? lane : 0)];
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u)
        if (dst[u] >= 0) s_c[dst[u]] = cv[u];
      if (nmax > 64) {  // (wave-uniform) a chunk of this batch holds more than 64 candidates
#pragma unroll 1
        for (int u = 0; u < kBatch; ++u) {
          const int c = c0 + 4 * u;
          const int n = c < nch ? s_pre[c + 1] - s_pre[c] : 0;
          for (int i = 64 + lane; i < n; i += 64) s_c[s_pre[c] + i] = seg[(int64_t)c * kChunk + i];
        }
      }
    }
  }
  __syncthreads();
  auto cand = [&](int j) -> Cand {
    if (in_lds) return s_c[j];
    if (rescan) return Cand{srow.key(j), j};
    return cand_global(j);
  };

  // the remaining bits of the K-th key among the candidates: after kernels 1 to 3 the top 22 are known;
  // after the bound collect, those the candidates share, then 11-bit digits below them
  uint32_t kstar;
  int need, known;
  if (bounded) {
    uint32_t lo = 0xFFFFFFFFu, hi = 0u;
    for (int j = tid; j < C; j += kSplitThreads) {
      const uint32_t kk = cand(j).key;
      lo = min(lo, kk);
      hi = max(hi, kk);
    }
    block_minmax<kSplitThreads>(lo, hi, s_mm);
    kstar = hi;
    known = common_bits(lo, hi);
    need = K;
  } else {
    kstar = ws.info[row * 4 + 2] << 10;
    known = 22;
    need = (int)ws.info[row * 4 + 3];
  }
  while (known < 32) radix_step([&](int j) { return cand(j).key; }, C, kstar, known, need, hist, s_w, s_sel);
  const int ties = need;
  __syncthreads();

  // ordered output: thread t owns the contiguous candidates [t*per, (t+1)*per)
  const int per = (C + kSplitThreads - 1) / kSplitThreads;
  const int j0 = min(tid * per, C), j1 = min(j0 + per, C);
  int n_gt = 0, n_eq = 0;
  for (int j = j0; j < j1; ++j) {
    const uint32_t kk = cand(j).key;
    n_gt += kk > kstar;
    n_eq += kk == kstar;
  }
  int tot;
  const int eq_base = block_int_scan<kSplitThreads>(n_eq, s_w, tot);
  const int take_eq = max(0, min(n_eq, ties - eq_base));
  int pos = block_int_scan<kSplitThreads>(n_gt + take_eq, s_w, tot);
  int eq_rank = eq_base;
  for (int j = j0; j < j1; ++j) {
    const Cand cd = cand(j);
    bool sel = cd.key > kstar;
    if (cd.key == kstar) sel = (eq_rank++ < ties);
    if (sel) {
      orow[pos] = cd.idx;
      if (vrow) vrow[pos] = key_to_score(cd.key);
      ++pos;
    }
  }
  for (int j = K + tid; j < k; j += kSplitThreads) {
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
                       const uint32_t* bound, int32_t* idx, float* vals, void* ws, hipStream_t stream) {
  const int rows = B * T;
  const int sbf16 = score_t == CSA_BF16 ? 1 : 0;
  if (use_split(rows, n_max)) {
    const int nch = ceil_div(n_max, kChunk);
    SplitWs s = carve(ws, rows, n_max, nch);
    dim3 grid(nch, rows);
    // bound keys help only when there are enough of them (a K-th largest well inside their range)
    const bool bounded = bound && index_bound_keys(n_max) >= 2 * (int64_t)k;
    if (bounded) {
      hipLaunchKernelGGL(topk_bound_collect_kernel, grid, dim3(kSplitThreads), 0, stream, scores, sbf16, T, n_max, pos0, m,
                         k, bound, (int)index_bound_keys(n_max), s);
    } else {
      hipLaunchKernelGGL(topk_split_hist_kernel, grid, dim3(kSplitThreads), 0, stream, scores, sbf16, T, n_max, pos0, m, k,
                         s);
      hipLaunchKernelGGL(topk_split_hist1_kernel, grid, dim3(kSplitThreads), 0, stream, scores, sbf16, T, n_max, pos0, m,
                         k, s);
      hipLaunchKernelGGL(topk_split_collect_kernel, grid, dim3(kSplitThreads), 0, stream, scores, sbf16, T, n_max, pos0,
                         m, k, s);
    }
    hipLaunchKernelGGL(topk_split_finish_kernel, dim3(rows), dim3(kSplitThreads), 0, stream, scores, sbf16, T, n_max, pos0,
                       m, k, nch, idx, vals, s, bounded ? 1 : 0);
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
