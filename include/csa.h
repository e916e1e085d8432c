/*
 * csa.h -- C ABI of the CSA / HCA layer step for AMD Instinct MI355X (gfx950).
 *
 * The method is DeepSeek-V4's hybrid attention as restated in
 * "【论文解读】DeepSeek-V4" (wkq9411.github.io), section 一(三) "混合注意力架构：CSA + HCA":
 *   (1) compressed KV entries, (2) lightning indexer + top-k selector,
 *   (3) shared key-value MQA, and the "其他技术细节" part (RMSNorm on queries and
 *   KV entries, partial RoPE with the output rotated back by -t, sliding window,
 *   attention sink).  Cited below as [CSA], [HCA] and [details].
 *
 * Conventions shared by every call
 *   - All array arguments are DEVICE pointers owned by the caller (hipMalloc /
 *     torch); the library allocates nothing and keeps no state between calls.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Every call is asynchronous on that stream and never synchronises.
 *   - Shapes are row-major, innermost index last.  B = sequences, T = query rows
 *     per sequence (1 for decode).  Query row r of sequence b sits at absolute
 *     position t = pos0[b] + r, where pos0 is a DEVICE int64 array [B].
 *   - Compressed entry s covers tokens m*s .. m*s+m-1 and is placed at position
 *     m*s for RoPE.  Query t sees compressed entries s < floor(t/m) ([CSA] (2),
 *     the visibility condition of the index score), capped at the cache size.
 *   - Errors: every call validates its arguments on the host in O(1) before any
 *     launch and returns a csa_status; no exception or abort crosses the ABI.
 *     CSA_ERR_LAUNCH reports a failed launch (hipGetLastError); faults during
 *     execution surface at the caller's next synchronisation.
 *   - Calls are reentrant; calls on different streams that share a workspace race.
 */
#ifndef CSA_H
#define CSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  CSA_F32 = 0,               /* IEEE binary32                                                    */
  CSA_BF16 = 1,              /* bfloat16, stored as uint16                                        */
  CSA_FP8_E4M3_ROWSCALE = 2, /* OCP fp8 E4M3 bytes + one float32 scale per row (value = code*scale) */
  CSA_MXFP4_E8M0_B32 = 3,    /* OCP MXFP4: e2m1 pairs (element 2i in the low nibble) + one E8M0    */
                             /* scale byte per 32 elements (value = e2m1 * 2^(scale-127))          */
  CSA_FP8_BF16_ROPE = 4      /* prepared KV row of c values with R RoPE dims: the first c-R values */
                             /* as OCP fp8 E4M3 bytes with one float32 scale per row (value =      */
                             /* code*scale, scale = amax/448 of those values), then the R RoPE     */
                             /* values as bf16; c + R bytes per row, the scales in their own array */
                             /* (the mixed KV storage of the same page, section 一(三)4, item 1)   */
} csa_dtype;

typedef enum {
  CSA_OK = 0,
  CSA_ERR_NULL = 1,        /* a required pointer is NULL                      */
  CSA_ERR_SHAPE = 2,       /* sizes inconsistent or out of range              */
  CSA_ERR_UNSUPPORTED = 3, /* valid request this build does not implement     */
  CSA_ERR_WORKSPACE = 4,   /* workspace missing or smaller than required      */
  CSA_ERR_LAUNCH = 5       /* the kernel launch failed                        */
} csa_status;

/*
 * Preparation of a KV row for core attention ([details] (1) and (2)):
 *   x -> RoPE_pos( x / sqrt(mean(x^2) + eps) * gamma ), RoPE on the pairs
 *   (c-R+2i, c-R+2i+1), R = rope_dims, angle pos * rope_base^(-2i/R).
 * A compressed entry or a token row keeps its position for good, so its prepared
 * form can be stored once (csa_compress with a csa_kv_prep, csa_prepare_kv) and
 * reused by every later query (csa_attend / hca_attend with kv_prepared >= 1).
 */
typedef struct {
  const float* gamma; /* device float32 [c] RMSNorm gain, NULL = 1 */
  float eps;          /* RMSNorm epsilon */
  int rope_dims;      /* R: even, a multiple of 8, <= min(c, 128); 0 = no rotation */
  float rope_base;    /* RoPE base */
} csa_kv_prep;

/* Static, NUL-terminated description of a status code. */
const char* csa_status_string(int status);
/* ABI revision of this header (bumped on any signature change). */
int csa_abi_version(void);

/*
 * csa_compress -- learned per-channel softmax pooling of per-token KV rows.
 * [CSA] (1): entry i, channel j: softmax over the 2m logits
 *   Z^a[mi+r][j] + B^a[r][j] and Z^b[m(i-1)+r][j] + B^b[r][j]   (r = 0..m-1)
 * and C^Comp_i[j] = sum S^a C^a + sum S^b C^b; for i = 0 the b-side is padded
 * with -inf logits / zero values.  [HCA] (1): pass cb = zb = bias_b = NULL to pool
 * m (= m') rows of a single stream with no overlap.
 *
 *   ca, cb, za, zb : [B][rows][c] in in_t (CSA_F32 or CSA_BF16); row k holds the
 *                    token at absolute position row0_pos + k.
 *   bias_a, bias_b : [m][c] float32.
 *   entries        : i = first_entry .. first_entry + num_entries - 1; every row
 *                    they read must lie inside [row0_pos, row0_pos + rows).
 *   out            : entry e of sequence b is row (b * out_batch_stride + e) of
 *                    [..][c] values in out_t (0 for out_batch_stride means
 *                    num_entries).  To append into a cache [B][Nmax][c] pass
 *                    out = cache row first_entry and out_batch_stride = Nmax.
 *                    CSA_F32 / CSA_BF16 (round to nearest even);
 *                    CSA_FP8_E4M3_ROWSCALE: bytes, and out_scale (float32, same
 *                    row indexing) = amax/448, codes = RNE(x/scale) saturated;
 *                    CSA_MXFP4_E8M0_B32: c/2 bytes per row, and out_scale (uint8,
 *                    c/32 per row) = floor(log2 amax) - 2 + 127, codes RNE,
 *                    saturated at 6.  CSA_FP8_BF16_ROPE (prepared entries only,
 *                    R = prep->rope_dims, c - R a multiple of 16): c + R bytes per
 *                    row, out_scale float32 per row.  out_scale is ignored for
 *                    F32 / BF16.
 *   prep           : NULL, or the entries are stored prepared for attention
 *                    (see csa_kv_prep) at position m * i; CSA_F32 / CSA_BF16 /
 *                    CSA_FP8_BF16_ROPE outputs only.
 * Limits: 1 <= m <= 1024, c a multiple of 4 and <= 1024 (of 32 for MXFP4).
 */
csa_status csa_compress(const void* ca, const void* cb, const void* za, const void* zb,
                        const float* bias_a, const float* bias_b,
                        int B, int rows, int c, int m,
                        int64_t row0_pos, int64_t first_entry, int num_entries,
                        int in_t,
                        void* out, void* out_scale, int out_t, int64_t out_batch_stride,
                        const csa_kv_prep* prep, void* stream);

/*
 * csa_compress_pair -- two csa_compress problems in one launch: the same batch,
 * token rows, ratio and entries, each with its own streams, biases, width,
 * output format and output rows.  Meant for a block's KV entry and its
 * indexer-key entry, which [CSA] (2) forms by the same compression from their
 * own streams.  Arguments of problem 0 then problem 1 as in csa_compress
 * (ca .. bias_b, c, out, out_scale, out_t, out_batch_stride, prep), then the
 * shared B, rows, m, row0_pos, first_entry, num_entries, in_t.  Same limits and
 * errors as two csa_compress calls; nothing is launched if either is rejected.
 */
csa_status csa_compress_pair(const void* ca0, const void* cb0, const void* za0, const void* zb0,
                             const float* bias_a0, const float* bias_b0, int c0,
                             void* out0, void* out_scale0, int out_t0, int64_t out_batch_stride0,
                             const csa_kv_prep* prep0,
                             const void* ca1, const void* cb1, const void* za1, const void* zb1,
                             const float* bias_a1, const float* bias_b1, int c1,
                             void* out1, void* out_scale1, int out_t1, int64_t out_batch_stride1,
                             const csa_kv_prep* prep1,
                             int B, int rows, int m, int64_t row0_pos, int64_t first_entry,
                             int num_entries, int in_t, void* stream);

/*
 * csa_prepare_kv -- prepares KV rows for attention (see csa_kv_prep).
 *   in  : [B] blocks of `rows` rows of c values in in_t (CSA_F32 / CSA_BF16);
 *         row j of sequence b at in + (b * in_batch_stride + j) * c.
 *   out : the same layout with out_batch_stride, in out_t (CSA_F32, CSA_BF16, or
 *         CSA_FP8_BF16_ROPE with c + R bytes per row and out_scale float32 per
 *         row, R = prep->rope_dims, c - R a multiple of 16); may alias `in` for
 *         the same type and layout.
 *   position of row j of sequence b: (pos_base ? pos_base[b] : 0) + pos_first
 *   + j * pos_stride (pos_base a device int64 [B] array), e.g. pos_stride = m
 *   for a compressed cache, 1 for token rows.  prep must not be NULL.
 * Limits: c a multiple of 4 and <= 1024; R as in csa_kv_prep.
 */
csa_status csa_prepare_kv(const void* in, int64_t in_batch_stride, void* out, void* out_scale,
                          int64_t out_batch_stride, int B, int rows, int c, int in_t, int out_t,
                          const int64_t* pos_base, int64_t pos_first, int64_t pos_stride,
                          const csa_kv_prep* prep, void* stream);

/*
 * csa_index -- lightning-indexer scores ([CSA] (2), the I_{t,s} equation):
 *   I[b][r][s] = sum_h w[b][r][h] * ReLU( q^I[b][r][h] . K^IComp[b][s] )
 * for s < min(floor(t/m), n_max) with t = pos0[b] + r; every other s in
 * [0, n_max) is written as -inf.  No scale, norm or RoPE is applied.
 *
 *   q       : [B][T][HI][cI] in qk_t (MXFP4: [B][T][HI][cI/2] bytes)
 *   q_scale : CSA_FP8_E4M3_ROWSCALE: float32 [B][T][HI]; CSA_MXFP4_E8M0_B32:
 *             uint8 [B][T][HI][cI/32]; NULL otherwise.
 *   w       : float32 [B][T][HI]
 *   k       : [B][n_max][cI] in qk_t (MXFP4: cI/2 bytes per row)
 *   k_scale : as q_scale with rows [B][n_max].
 *   scores  : [B][T][n_max] in score_t: CSA_F32, or CSA_BF16 (rounded to nearest
 *             even; the selector reads half the bytes)
 *   bound   : NULL, or uint32 [B][T][csa_index_bound_keys(n_max)], 8-byte aligned:
 *             for csa_topk, keys of the two largest visible scores (as stored, in
 *             score_t) of each bound set (order-preserving keys, 0 where a set has
 *             fewer), two per set.  A set is 256 entries when n_max > 65536, 32
 *             entries otherwise (which entries form a set, and where its keys sit,
 *             differ between the decode and the tiled prefill kernels; only the
 *             keys' values matter).  Their K-th largest never exceeds a row's K-th
 *             largest score, so csa_topk can skip its threshold search.  With
 *             CSA_F32 a non-NULL bound is CSA_ERR_UNSUPPORTED.
 * All pointers 16-byte aligned (the MXFP4 q_scale at least 4-byte aligned).
 * Products run on MFMA with float32 accumulation for BF16 / FP8 / MXFP4 (row
 * scales are applied to the float32 dot products; MXFP4 block scales inside
 * the MFMA), and on float32 FMA for CSA_F32.
 * Limits: F32: cI a multiple of 4, cI <= 512, HI <= 128.  BF16 / FP8 / MXFP4:
 * cI = 128 and HI in {16, 32, 64, 128}.
 */
int64_t csa_index_bound_keys(int64_t n_max);
csa_status csa_index(const void* q, const void* q_scale, const float* w,
                     const void* k, const void* k_scale,
                     int B, int T, int HI, int cI, int64_t n_max,
                     const int64_t* pos0, int m, int qk_t,
                     void* scores, int score_t, uint32_t* bound, void* stream);

/*
 * csa_compress_index -- one launch for a decode step's compression and index
 * (T = 1): the same results as csa_compress_pair (job 0: the KV entry, job 1:
 * the indexer key, one entry first_entry per sequence) followed by csa_index,
 * where job 1's output is the key cache itself: entry first_entry of k (and
 * k_scale), stored in qk_t (fp8 with its row scale, MXFP4 with its block
 * scales, or bf16), read by the index scores of the same launch.
 *   job 0 : (out0 NULL: none, the indexer key alone -- e.g. when csa_topk_compress computes the KV
 *           entry) ca0 .. bias_b0, c0, out0 (CSA_F32 / CSA_BF16 rows [B][..][c0], or
 *           CSA_FP8_BF16_ROPE rows with prep0 and their scales in out_scale0,
 *           with batch stride out_batch_stride0, 0 = 1), prep0 as in
 *           csa_compress.
 *   job 1 : ca1 .. bias_b1 with c = cI.
 *   shared: B, rows, m (< 64), row0_pos, first_entry (< n_max), in_t, as in
 *           csa_compress_pair with num_entries = 1.
 *   index : q .. bound as in csa_index with T = 1 (qk_t CSA_BF16, FP8 or MXFP4;
 *           scores in score_t).
 * Each argument group is validated as by the corresponding entry point.
 */
csa_status csa_compress_index(const void* ca0, const void* cb0, const void* za0, const void* zb0,
                              const float* bias_a0, const float* bias_b0, int c0, void* out0, void* out_scale0,
                              int out_t0,
                              int64_t out_batch_stride0, const csa_kv_prep* prep0,
                              const void* ca1, const void* cb1, const void* za1, const void* zb1,
                              const float* bias_a1, const float* bias_b1,
                              int B, int rows, int m, int64_t row0_pos, int64_t first_entry, int in_t,
                              const void* q, const void* q_scale, const float* w, void* k, void* k_scale,
                              int HI, int cI, int64_t n_max, const int64_t* pos0, int qk_t,
                              void* scores, int score_t, uint32_t* bound, void* stream);

/*
 * csa_topk -- top-k selector ([CSA] (2), the C^SprsComp_t equation).
 * Row (b, r) keeps the min(k, V) largest of scores[b][r][0 .. V) with
 * V = min(floor((pos0[b] + r)/m), n_max).  Larger score first; equal scores
 * (+0 and -0 are equal) go to the lower index.  idx[b][r][0..k) receives the kept
 * indices in ascending order followed by -1 padding; vals (nullable) receives
 * their scores (NaN-free inputs assumed; padding slots get -inf).  scores are
 * float32 or bf16 (score_t CSA_F32 / CSA_BF16), as csa_index wrote them; a bf16
 * score is compared by its exact float32 value.
 *
 *   bound     : NULL, or the bound keys csa_index wrote for these scores.  With
 *               them, long rows (the decode case) take two kernels instead of
 *               four; the result is the same.  Keys that are not a lower bound
 *               (larger than the scores they stand for) still give the exact
 *               result, through a slow whole-row pass.
 *   workspace : device memory of csa_topk_workspace_bytes(B, T, n_max, k) bytes
 *               (0 means none is needed).  It must be zero-filled before its
 *               first use.  Every call leaves the part that has to start at zero
 *               zero-filled again, at the same place for every shape, so one
 *               buffer (of the largest size needed) serves later calls of any
 *               shape on the same stream.
 * Limits: 1 <= k <= 2048, n_max < 2^31.
 */
size_t csa_topk_workspace_bytes(int B, int T, int64_t n_max, int k);
csa_status csa_topk(const void* scores, int score_t, int B, int T, int64_t n_max,
                    const int64_t* pos0, int m, int k, const uint32_t* bound,
                    int32_t* idx, float* vals,
                    void* workspace, size_t ws_bytes, void* stream);

/*
 * csa_topk_compress -- csa_topk for decode rows (T = 1) and a csa_compress of one entry per sequence
 * (first_entry; rows, layouts, out_t and prep as in csa_compress with num_entries = 1) in one launch:
 * with the indexer's bound keys the selection's launch carries one more workgroup per sequence that
 * computes the entry (the decode step's new KV entry, read by the attention after the selection);
 * without them the entry is computed by a launch of its own first.  Results equal the two calls.
 * Limits: those of both calls, m < 64.
 */
csa_status csa_topk_compress(const void* scores, int score_t, int B, int64_t n_max, const int64_t* pos0, int m,
                             int k, const uint32_t* bound, int32_t* idx, float* vals, void* workspace,
                             size_t ws_bytes, const void* ca, const void* cb, const void* za, const void* zb,
                             const float* bias_a, const float* bias_b, int c, int rows, int64_t row0_pos,
                             int64_t first_entry, int in_t, void* out, void* out_scale, int out_t,
                             int64_t out_batch_stride, const csa_kv_prep* prep, void* stream);

/*
 * csa_attend -- CSA core attention ([CSA] (3) shared key-value MQA and [details]).
 * For query row (b, r) at t = pos0[b] + r and head h:
 *   entries  E = { comp_kv[b][s] : s = idx[b][r][j] >= 0 }  (position m*s)
 *              u { window token p : max(0, t-n_win+1) <= p <= t }  (position p)
 *   e^ = RoPE_pos(RMSNorm_gamma_kv(e)),  q^ = RoPE_t(RMSNorm_gamma_q(q[b][r][h]))
 *   z_j = scale * q^ . e^_j,   p_j = exp(z_j) / (sum_i exp(z_i) + exp(sink[h]))
 *   out[b][r][h] = RoPE_{-t}( sum_j p_j e^_j )
 * RMSNorm: x / sqrt(mean(x^2) + eps) * gamma over all c dims (gamma NULL = 1).
 * RoPE: pairs (c-R+2i, c-R+2i+1), R = rope_dims, angle pos * rope_base^(-2i/R).
 *
 *   q       : [B][T][H][c] in kv_t        comp_kv : [B][n_max][c] in comp_t
 *   comp_t  : kv_t, or CSA_FP8_BF16_ROPE (kv_t CSA_BF16, kv_prepared >= 1,
 *             c - rope_dims a multiple of 16): rows of c + rope_dims bytes with
 *             their scales in comp_scale (float32 [B][n_max]); otherwise
 *             comp_scale is ignored.  Rows are widened to bf16 in LDS
 *             (code * scale, rounded to nearest even) before use.
 *   idx     : int32 [B][T][k]; entries < 0 or >= n_max are skipped
 *   win_kv  : [B][T + n_win - 1][c] in kv_t; row j holds position pos0[b]-n_win+1+j
 *   sink    : float32 [H]     gamma_q, gamma_kv : float32 [c] or NULL
 *   kv_prepared : 0 = comp_kv holds pooled entries e; 1 = comp_kv holds the
 *               prepared e^ (csa_compress with a csa_kv_prep of the same gamma_kv,
 *               eps, rope_dims and rope_base, or csa_prepare_kv with
 *               pos_stride = m), which are then used as they are, window rows
 *               raw token rows; 2 = as 1, and the window rows are prepared too
 *               (csa_prepare_kv of the token rows at their positions: pos_base =
 *               pos0, pos_first = -(n_win - 1), pos_stride = 1).  Any other value
 *               is CSA_ERR_UNSUPPORTED.  With 2 and H a multiple of 64, prefill
 *               (T > 1) runs a kernel variant with 64 heads per workgroup.
 *   out     : [B][T][H][c] in out_t (CSA_F32 or CSA_BF16)
 *   workspace : csa_attend_workspace_bytes(B, T, H, c, k, n_win) bytes of device
 *               memory (no initial contents needed); may be NULL if that is 0.
 * kv_t is CSA_F32 (float32 FMA path) or CSA_BF16 (MFMA path, float32 softmax
 * and accumulation).  Decode (T = 1) splits each query's entry list (compressed
 * part and window part separately) at fixed boundaries that depend only on the
 * list lengths and merges the parts in a fixed order, so results do not depend
 * on B or on the other rows.  A part's output reaches the merge through the
 * workspace in fp16, divided by its softmax denominator (a convex combination of
 * entry values, so bounded by the largest entry magnitude; 2^-11 relative): on
 * the CSA_BF16 decode path entry values must stay below 65504 in magnitude,
 * which normalised entries (at most sqrt(c) times the largest gain) do.
 * Limits: c in {128, 256, 512}; rope_dims even, a multiple of 8 and <= min(c, 128);
 * H a multiple of 16 for CSA_BF16 (any H >= 1 for CSA_F32); 1 <= k <= 2048;
 * 1 <= n_win <= 4096.
 */
size_t csa_attend_workspace_bytes(int B, int T, int H, int c, int k, int n_win);
csa_status csa_attend(const void* q, const void* comp_kv, const float* comp_scale, const int32_t* idx,
                      const void* win_kv, const float* sink, const float* gamma_q, const float* gamma_kv,
                      int B, int T, int H, int c, int rope_dims, int k, int n_win, int64_t n_max,
                      const int64_t* pos0, int m, float scale, float eps, float rope_base,
                      int kv_t, int comp_t, int kv_prepared, void* out, int out_t,
                      void* workspace, size_t ws_bytes, void* stream);

/*
 * hca_attend -- HCA core attention ([HCA] (2)): as csa_attend, with the
 * compressed part dense: every visible entry s < min(floor(t/m_hca), n_max) of
 * comp_kv, each at position m_hca * s.  Same layouts, limits, comp_t and
 * kv_prepared rules (prepared entries at pos_stride = m_hca; with 2 and H a
 * multiple of 64, decode also runs the 64-head variant) and workspace rule
 * (hca_attend_workspace_bytes).
 */
size_t hca_attend_workspace_bytes(int B, int T, int H, int c, int64_t n_max, int n_win);
csa_status hca_attend(const void* q, const void* comp_kv, const float* comp_scale, const void* win_kv,
                      const float* sink, const float* gamma_q, const float* gamma_kv,
                      int B, int T, int H, int c, int rope_dims, int n_win, int64_t n_max,
                      const int64_t* pos0, int m_hca, float scale, float eps, float rope_base,
                      int kv_t, int comp_t, int kv_prepared, void* out, int out_t,
                      void* workspace, size_t ws_bytes, void* stream);

/*
 * csa_attend_noalloc -- csa_attend for callers that cannot allocate device memory: code being captured
 * into a HIP graph, tight serving loops, harnesses that forbid allocation.  Same arguments, results and
 * errors as csa_attend, without the workspace: the decode split partials live in a device array of the
 * library (64 MiB, which each GPU the library runs on holds until the process ends).  A call whose
 * workspace (csa_attend_workspace_bytes) exceeds 64 MiB returns CSA_ERR_WORKSPACE and launches nothing.
 * The call itself allocates nothing; its first call on a device looks up that device's array address.
 * Every call on one GPU shares that GPU's array (it needs no initial contents), so calls that overlap on
 * one GPU (different streams, or host threads) race and must be ordered by the caller.
 */
csa_status csa_attend_noalloc(const void* q, const void* comp_kv, const float* comp_scale, const int32_t* idx,
                              const void* win_kv, const float* sink, const float* gamma_q, const float* gamma_kv,
                              int B, int T, int H, int c, int rope_dims, int k, int n_win, int64_t n_max,
                              const int64_t* pos0, int m, float scale, float eps, float rope_base, int kv_t,
                              int comp_t, int kv_prepared, void* out, int out_t, void* stream);

/*
 * ---- Decode across steps: the state cache and the paged compressed caches ----
 *
 * "【论文解读】DeepSeek-V4", section 二(六) 推理框架, and "DeepseekV4论文解析", its KV-cache part: the
 * sliding window and the tail tokens that do not yet fill a compression block live in a fixed-size
 * state cache per request; completed CSA / HCA entries live in a paged cache whose blocks cover a
 * multiple of lcm(m, m') raw tokens (128 at m = 4, m' = 128: 32 CSA entries and 1 HCA entry).
 *
 * csa_pages: logical page j of sequence b covers raw tokens [j * page_tokens, (j + 1) * page_tokens)
 * and is physical page block_table[b * max_pages + j] of every paged pool.  A pool of entries at
 * ratio r (m for CSA KV and indexer keys, m_hca for HCA) holds E = page_tokens / r entries per page:
 * entry s of sequence b is pool row block_table[b * max_pages + s / E] * E + s % E (scales: the same
 * row of their own array).  page_tokens is a power of two and a multiple of 128 and of every ratio
 * used with it; block_table is device int32 [B][max_pages] with the pages of entries < n_max
 * mapped (the caller allocates and maps pages; the library never does).
 *
 * The state cache is plain device arrays: a ring of `ring` rows per sequence ([B][ring][c]) holds
 * the row of position p at row p % ring.
 */
typedef struct {
  const int32_t* block_table; /* device int32 [B][max_pages] */
  int max_pages;              /* row length of block_table */
  int page_tokens;            /* raw tokens per page: a power of two, a multiple of 128 */
} csa_pages;

/* One compression problem of csa_decode_append ([CSA] (1); [HCA] (1) when cb = zb = NULL). */
typedef struct {
  const void* ca;             /* the new token's rows, [B][c] each in in_t */
  const void* cb;             /* NULL for HCA (and then zb, bias_b, ring_cb, ring_zb NULL) */
  const void* za;
  const void* zb;
  const float* bias_a;        /* [m][c] */
  const float* bias_b;        /* [m][c] or NULL */
  int c;                      /* width, a multiple of 4, <= 1024 (of 32 for MXFP4 output) */
  int m;                      /* compression ratio: the entry pools 2m rows (m rows for HCA) */
  void* ring_ca;              /* state rings [B][ring][c] in in_t, ring = 2m (m for HCA): the */
  void* ring_cb;              /* streams of tokens [t - ring, t) on entry, of (t - ring, t] on exit */
  void* ring_za;
  void* ring_zb;
  void* out;                  /* paged pool of completed entries, rows as csa_compress's out_t */
  void* out_scale;            /* their scales (fp8: float32 per row; MXFP4: c/32 bytes per row) */
  int out_t;
  const csa_kv_prep* prep;    /* as in csa_compress (entry i prepared at position m * i) */
} csa_append_job;

/* One sliding-window ring of csa_decode_append ([details] (3)). */
typedef struct {
  const void* row;            /* the new token's KV row, [B][c] in in_t */
  void* ring;                 /* [B][n_win][c] in in_t: position p at row p % n_win */
  int c;
  int n_win;
  const csa_kv_prep* prep;    /* NULL: stored as it is; else stored prepared at position t */
} csa_window_job;

/*
 * csa_decode_append -- one decode token per sequence enters the state cache.  For sequence b with
 * t = pos[b] (device int64 [B]):
 *   - every job whose block just completed (t >= m and t % m == 0) computes entry i = t/m - 1 from
 *     its rings (the a-rows of tokens [t - m, t), the b-rows of [t - 2m, t - m); block 0 has no
 *     b-rows) exactly as csa_compress would from the same rows, and writes it to row i of its paged
 *     pool; then every job stores the token's rows at ring row t % ring;
 *   - every window job stores its row at ring row t % n_win.
 * Entry i is visible to queries t' >= m (i + 1), so a decode step appends its token first and then
 * runs csa_index_paged / csa_topk / csa_attend_paged for the same t.  A sequence with pos[b] < 0 is
 * left alone; an entry whose logical page is >= max_pages is not stored (its pages must be mapped
 * before the step; positions live on the device, so the host cannot check them).
 * Limits: 1 <= njobs <= 2, 0 <= nwins <= 2, in_t CSA_F32 or CSA_BF16, B < 65536; the jobs of one
 * call all have m < 64 (256-thread workgroups) or all m >= 64 (1024-thread workgroups), the thread
 * counts csa_compress uses for them, so that an entry's value does not depend on the call (e.g. the
 * KV entry and indexer key in one call, the HCA entry in another).  Errors: CSA_ERR_NULL for a
 * missing pointer, CSA_ERR_SHAPE / CSA_ERR_UNSUPPORTED as csa_compress for the jobs' shapes and
 * formats, and for pages whose page_tokens is not a power of two, a multiple of 128 and of m.
 */
csa_status csa_decode_append(const csa_append_job* jobs, int njobs, const csa_window_job* wins, int nwins, int B,
                             const int64_t* pos, const csa_pages* pages, int in_t, void* stream);

/*
 * csa_index_paged -- csa_index for decode rows (T = 1) over a paged key pool: k_pool / k_scale_pool
 * hold the keys in qk_t (rows as csa_index's k and k_scale), entry s of sequence b at the pool row
 * given by `pages` (ratio m).  Scores [B][1][n_max] and bound keys exactly as csa_index; n_max is
 * the logical cache size and must fit the mapped pages.  The MFMA formats only (bf16, fp8, MXFP4).
 */
csa_status csa_index_paged(const void* q, const void* q_scale, const float* w, const void* k_pool,
                           const void* k_scale_pool, const csa_pages* pages, int B, int HI, int cI, int64_t n_max,
                           const int64_t* pos0, int m, int qk_t, void* scores, int score_t, uint32_t* bound,
                           void* stream);

/*
 * csa_append_index_paged -- csa_decode_append (jobs[0]: the KV entry, jobs[1]: the indexer key, whose
 * out / out_scale / out_t must be k_pool / k_scale_pool / qk_t; win: NULL or the window ring) and
 * csa_index_paged for the same tokens, in one launch: the workgroup whose entries hold the new key
 * compresses it before it reads any key, workgroup 0 of each sequence does the rest of the append.
 * Results equal the two calls made in turn.  Limits: those of both calls, m < 64, widths <= 1024.
 */
csa_status csa_append_index_paged(const csa_append_job* jobs, const csa_window_job* win, int in_t, const void* q,
                                  const void* q_scale, const float* w, const void* k_pool, const void* k_scale_pool,
                                  const csa_pages* pages, int B, int HI, int cI, int64_t n_max, const int64_t* pos0,
                                  int m, int qk_t, void* scores, int score_t, uint32_t* bound, void* stream);

/*
 * csa_attend_paged / hca_attend_paged -- csa_attend / hca_attend for decode rows (T = 1) whose
 * compressed entries sit in a paged pool (comp_pool, comp_scale_pool; ratio m, resp. m_hca) and
 * whose window rows sit in a state ring win_ring [B][n_win][c] (position p at row p % n_win: the
 * ring of csa_decode_append, holding positions t - n_win + 1 .. t).  Everything else, including
 * kv_t = CSA_BF16 and the comp_t / kv_prepared rules (kv_prepared >= 1), is as in the contiguous
 * calls; the workspaces are csa_attend_workspace_bytes(B, 1, ...) and hca_attend_workspace_bytes(B, 1, ...).
 */
csa_status csa_attend_paged(const void* q, const void* comp_pool, const float* comp_scale_pool,
                            const csa_pages* pages, const int32_t* idx, const void* win_ring, const float* sink,
                            const float* gamma_q, const float* gamma_kv, int B, int H, int c, int rope_dims, int k,
                            int n_win, int64_t n_max, const int64_t* pos0, int m, float scale, float eps,
                            float rope_base, int kv_t, int comp_t, int kv_prepared, void* out, int out_t,
                            void* workspace, size_t ws_bytes, void* stream);
csa_status hca_attend_paged(const void* q, const void* comp_pool, const float* comp_scale_pool,
                            const csa_pages* pages, const void* win_ring, const float* sink, const float* gamma_q,
                            const float* gamma_kv, int B, int H, int c, int rope_dims, int n_win, int64_t n_max,
                            const int64_t* pos0, int m_hca, float scale, float eps, float rope_base, int kv_t,
                            int comp_t, int kv_prepared, void* out, int out_t, void* workspace, size_t ws_bytes,
                            void* stream);

/*
 * ---- Dense projections on either side of the step (decode and prefill rows) ----
 *
 * Up to 32 rows a call streams the weights (every weight byte read once, HBM-bound); more rows (chunked
 * prefill) take an LDS-tiled MFMA product of 256-row x 128-column tiles (MFMA-bound).  Both accumulate in
 * float32 over the whole K.
 *
 * Weights are passed PACKED (csa_pack_proj_weights): the [Z][N][K] output-major matrices (row n holds
 * output n's K weights) rearranged once, at load time, into 1 KB MFMA tiles so that the projections
 * stream them in contiguous 1 KB loads.  Packed element (n, k) of batch z sits at
 *   z * N * K + ((n / 16) * (K / 32) + k / 32) * 512 + (((k % 32) / 8) * 16 + n % 16) * 8 + k % 8.
 *
 * csa_pack_proj_weights -- w bf16 [z][n][k] -> packed bf16 (the same size, not aliasing w).  n a multiple
 * of 16, k a multiple of 32.
 */
csa_status csa_pack_proj_weights(const void* w, void* packed, int z, int n, int k, void* stream);

/*
 * csa_q_up_proj -- the queries from the shared low-rank latent ([CSA] (2), the q^I equation, and (3), the
 * q equation): q = c^Q W^UQ and q^I = c^Q W^IUQ in one launch that reads c^Q once.
 *   cq     : bf16 [rows][d_c]
 *   w_uq   : bf16 [n_h * c][d_c]    packed (csa_pack_proj_weights with z = 1)
 *   w_iuq  : bf16 [n_hI * cI][d_c]  packed
 *   q      : bf16 [rows][n_h * c]   (the [B][T][H][c] layout of csa_attend's q)
 *   qi     : in qi_t, the [B][T][HI][cI] layout of csa_index's q: bf16; or CSA_FP8_E4M3_ROWSCALE
 *            (e4m3 codes, qi_scale float32 [rows][n_hI] = amax/448 of the head's values); or
 *            CSA_MXFP4_E8M0_B32 (cI/2 bytes per head, qi_scale [rows][n_hI][cI/32] E8M0 bytes)
 * Accumulation in float32 over d_c; bf16 results rounded to nearest even; quantized q^I is coded from
 * the float32 sums.  Limits: rows >= 0 (0: nothing is done); d_c a multiple of 32; n_h * c and n_hI * cI
 * multiples of 128; cI = 128 for the quantized forms.  CSA_ERR_NULL for a missing pointer;
 * CSA_ERR_UNSUPPORTED unless cq and the weights are 16-byte aligned, q 8-byte aligned and qi 8- (bf16),
 * 4- (fp8) or 2-byte (MXFP4) aligned.
 */
csa_status csa_q_up_proj(const void* cq, const void* w_uq, const void* w_iuq, int rows, int d_c, int n_h, int c,
                         int n_hI, int cI, void* q, void* qi, void* qi_scale, int qi_t, void* stream);

/*
 * csa_grouped_out_proj -- the grouped output projection ([CSA] (4); [HCA] (2) uses the same): the n_h
 * head outputs of a row split into g groups of n_h / g consecutive heads; group i's (n_h / g) * c values
 * are projected to d_g values, and the g * d_g intermediates to d.
 *   o    : bf16 [rows][n_h * c]            (csa_attend's out layout)
 *   w_g  : bf16 [g][d_g][(n_h / g) * c]    packed with z = g (group i's projection)
 *   w_o  : bf16 [d][g * d_g]               packed with z = 1
 *   mid  : bf16 [rows][g * d_g]            (the intermediates, caller-owned, rounded to bf16)
 *   out  : bf16 [rows][d]
 * Two launches (the groups, then the final projection), float32 accumulation.  Limits: rows >= 0 (0:
 * nothing is done); (n_h / g) * c and g * d_g multiples of 32; d_g and d multiples of 16; g divides n_h;
 * o, the weights and mid 16-byte aligned, out 8-byte aligned (else CSA_ERR_UNSUPPORTED).
 */
csa_status csa_grouped_out_proj(const void* o, const void* w_g, const void* w_o, int rows, int n_h, int c, int g,
                                int d_g, int d, void* mid, void* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* CSA_H */
