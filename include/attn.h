/*
 * attn.h -- C ABI of the fused multi-reduction attention library for AMD
 * MI355X (gfx950).  Library file: reduction_attention_amd/libattn.so.
 *
 * The operation is scaled dot-product attention with its multiple
 * reductions fused into one pass: S = scale * Q K^T, the row max, the row
 * sum of exp(S - max), and P V, computed tile by tile with an online
 * softmax so that the score matrix is never stored.  Sources (web pages):
 *   [CA] tip.co.jp article on the Cleave ML compiler (2026-10-10), sections
 *        "Split演算子によるSplit-Kの対応" (Split operator with a split count s
 *        over a reduction dimension) and "複数リダクションのスケジューリング"
 *        (iterative tiling of the reduction dimension; horizontal fusion of
 *        reductions that share a producer; dynamic batch and sequence
 *        dimensions kept as runtime loop bounds).
 *   [AB] arXiv abstract "Cleave: Scaling Tensor Program Optimization via
 *        Decoupled Algebraic Search and Operator Scheduling" (FlashAttention
 *        and FlashDecoding as the hand-written kernels the method targets;
 *        the Split operator; iterative tiling and horizontal fusion).
 *   [ST] gist.science explainer of "Accelerating Sparse Transformer
 *        Inference on GPU" (STOF), 技術概要, "1. 統合 MHA モジュール":
 *        two-level BSR + bitmap mask storage (full / part outer tiles kept
 *        through pointer arrays, one uint64 bitmap per 8x8 inner tile) and
 *        the block-wise kernel that stages Q/K/V sub-blocks on chip.
 *
 * Conventions shared by every entry point:
 *   - Tensors are caller-owned device buffers, densely packed, 16-byte
 *     aligned.  No call allocates or frees device memory; the library keeps
 *     no pointer after returning, and never synchronises the stream except
 *     in the attn_debug_* exports.  Its only device memory of its own is the
 *     fixed scratch array of attn_decode_splitkv_noalloc (loaded with the
 *     library, one per GPU).
 *   - All device work is enqueued, in order, on `hip_stream` (a
 *     hipStream_t; NULL = the default stream).  Calls return before the
 *     work finishes.
 *   - Every argument is validated on the host before any HIP call; on an
 *     error status nothing has been enqueued and no output is written.  A
 *     launch failure returns ATTN_EHIP; attn_last_error() gives details.
 *   - GQA: query head h reads KV head floor(h / G), G = Hq / Hkv.
 *   - LSE outputs are natural-log log-sum-exp of the scaled scores; a query
 *     with no valid key gets O = 0 and LSE = -inf.
 *   - Offsets are computed in 64-bit arithmetic.
 *   - The host cannot read device-resident indptr arrays without a
 *     synchronisation, so it trusts them: they must be non-decreasing, start
 *     at 0 and agree with the length hints passed alongside them.
 */
#ifndef REDUCTION_ATTENTION_AMD_ATTN_H
#define REDUCTION_ATTENTION_AMD_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int attn_status_t;
enum {
  ATTN_OK = 0,
  ATTN_EINVAL = 1,        /* null pointer, bad size, inconsistent arguments */
  ATTN_EUNSUPPORTED = 2,  /* valid request outside what is built (dtype, D, G) */
  ATTN_EWORKSPACE = 3,    /* workspace missing or too small */
  ATTN_EHIP = 4           /* the HIP runtime reported an error */
};

/* Element types of Q/K/V/O. */
enum { ATTN_F32 = 0, ATTN_BF16 = 1, ATTN_F16 = 2 };

/* Human-readable name of a status code (static storage). */
const char* attn_status_string(attn_status_t status);

/* Detail of the last failure on the calling thread ("" if none). */
const char* attn_last_error(void);

/* Number of compute units of the current device (cached on first use);
 * returns 256 when no device can be queried. */
int attn_device_cu_count(void);

/* ---- split-KV grouped-query decode ------------------------------------- */

/* Workspace bytes attn_decode_splitkv needs for `num_splits` splits:
 * num_splits * B * Hq * (D + 2) * 4 (fp32 partial outputs, maxima, sums),
 * rounded up to 256 bytes.  Returns 0 for invalid arguments. */
size_t attn_decode_workspace_bytes(int B, int Hq, int D, int num_splits);

/* The split count s the library picks when num_splits = 0, as
 * s = ceil(max_kv_len / c) clamped to [1, 256], with c the largest power of
 * two >= 256 keys such that:
 *  - equal or nearly equal request lengths (16 * total_kv >= 15 * B *
 *    max_kv_len: the mean length at least 15/16 of the longest), where
 *    attn_decode_splitkv's workgroup takes up to four KV heads:
 *    ceil(Hkv / hpw) * B * ceil(max_kv_len / c)
 *    workgroups (hpw = 4, 2 or 1, at most Hkv) reach one per compute unit;
 *  - otherwise, one KV head per workgroup: Hkv * (total_kv / c + B / 2)
 *    workgroups reach four per compute unit.
 * [CA] leaves the concrete s to the scheduler; this is that scheduler's
 * rule, fitted to measured sweeps on MI355X. */
int attn_decode_choose_splits(int B, int Hq, int Hkv, int D, long long total_kv,
                              int max_kv_len);

/*
 * Split-KV decode: one query token per request attends to the request's
 * packed keys, with the key (reduction) dimension cut by the Split operator
 * into s chunks [CA "Split演算子によるSplit-Kの対応"; AB], each reduced by one
 * workgroup with an online softmax over key tiles [CA "複数リダクションの
 * スケジューリング"], then merged by log-sum-exp weights (attn_merge_lse).
 *
 * q         [B, Hq, D]            element type `dtype`
 * k, v      [total_kv, Hkv, D]    request b owns rows kv_indptr[b] .. kv_indptr[b+1]-1
 * kv_indptr [B + 1] int32, device
 * o         [B, Hq, D]            element type `dtype`
 * lse       [B, Hq] fp32, or NULL
 * max_kv_len  the largest n_b = kv_indptr[b+1] - kv_indptr[b] (>= 1);
 * total_kv    kv_indptr[B].
 * num_splits  s in [1, 256], or 0 to use attn_decode_choose_splits.
 *   Chunk length c = ceil(max_kv_len / s); request b uses ceil(n_b / c)
 *   chunks, chunk i covering keys [i*c, min((i+1)*c, n_b)) of the request.
 *   A request with n_b = 0 yields O = 0, LSE = -inf.
 * workspace   device memory of at least attn_decode_workspace_bytes(B, Hq, D, s)
 *   bytes; its contents on entry do not matter.  Layout: o_part [s, B*Hq, D],
 *   then m_part [s, B*Hq], then l_part [s, B*Hq], all fp32.  Calls that share
 *   one workspace must not overlap in time.
 * Two kernels are enqueued: the Split partials (a request held by a single
 * chunk is written to o / lse directly), then the merge of the requests
 * that span several chunks.
 * Supported: dtype ATTN_F32 (VALU path) or ATTN_BF16 / ATTN_F16 (MFMA
 * path); D in {64, 128}; 1 <= G <= 16.
 */
attn_status_t attn_decode_splitkv(const void* q, const void* k, const void* v,
                                  const int32_t* kv_indptr, void* o, float* lse, int B,
                                  int Hq, int Hkv, int D, int max_kv_len, long long total_kv,
                                  float scale, int num_splits, int dtype, void* workspace,
                                  size_t workspace_bytes, void* hip_stream);

/*
 * attn_decode_splitkv for callers that cannot allocate device memory (code
 * under HIP graph capture, serving loops and harnesses that forbid
 * hipMalloc): the same operation, arguments, kernels and results, without
 * the workspace arguments.  The split partials go to a device array the
 * library holds, ATTN_NOALLOC_SCRATCH_BYTES bytes on each GPU it runs on,
 * kept until the process ends; no call allocates or frees memory.
 * A split count whose partials (attn_decode_workspace_bytes(B, Hq, D, s))
 * exceed that size is rejected with ATTN_EWORKSPACE before any device work.
 * Every call on one GPU shares that GPU's array: calls whose work overlaps
 * in time on one GPU (other streams, other host threads) race and must be
 * serialised by the caller.  The array's contents on entry do not matter
 * (each call writes every partial it reads).
 */
#define ATTN_NOALLOC_SCRATCH_BYTES (64u << 20)
attn_status_t attn_decode_splitkv_noalloc(const void* q, const void* k, const void* v,
                                          const int32_t* kv_indptr, void* o, float* lse, int B,
                                          int Hq, int Hkv, int D, int max_kv_len,
                                          long long total_kv, float scale, int num_splits,
                                          int dtype, void* hip_stream);

/*
 * The Split partials alone [CA "Split演算子によるSplit-Kの対応"]: the first
 * kernel of attn_decode_splitkv, writing every split's partial instead of
 * finishing single-split requests.  For a request b and split i < ceil(n_b /
 * c) it writes o_part[i, b*Hq + h, :] (normalised by its own sum), m_part
 * (max scaled score, natural-log units) and l_part (sum of exp(score - m));
 * splits a request does not use get m = -inf, l = 0.  attn_merge_lse turns
 * the partials into the output, so partials computed over different key
 * ranges (other calls, other devices) can be merged together.
 * Arguments as attn_decode_splitkv, with num_splits >= 1 required;
 * o_part [num_splits, B*Hq, D], m_part, l_part [num_splits, B*Hq] fp32.
 */
attn_status_t attn_decode_partials(const void* q, const void* k, const void* v,
                                   const int32_t* kv_indptr, int B, int Hq, int Hkv, int D,
                                   int max_kv_len, long long total_kv, float scale, int num_splits,
                                   int dtype, float* o_part, float* m_part, float* l_part,
                                   void* hip_stream);

/* ---- split-KV decode over the packed key array (flat plan) -------------- */

/* Piece count P the library picks for attn_decode_splitkv_flat when
 * num_pieces = 0: enough pieces for four waves per compute unit, with
 * workgroups of up to four KV heads (P = ceil(4 * CUs / (ceil(Hkv / hpw) *
 * hpw)), hpw = 4, 2 or 1, at most Hkv), capped so that no piece is shorter
 * than 256 keys, within [1, 65535].  Fitted to a sweep on MI355X. */
int attn_decode_flat_pieces(int B, int Hq, int Hkv, int D, long long total_kv);

/* Most splits one request can have under the flat plan with P pieces of
 * c = ceil(total_kv / P) rows: ceil((max_kv_len - 1) / c) + 1, at most P
 * (1 when total_kv or max_kv_len is 0; 0 for invalid arguments). */
int attn_decode_flat_max_splits(int max_kv_len, long long total_kv, int num_pieces);

/* Workspace bytes of attn_decode_splitkv_flat: s * B * Hq * (D + 2) * 4 with
 * s = attn_decode_flat_max_splits(...), rounded up to 256 (0 if invalid). */
size_t attn_decode_flat_workspace_bytes(int B, int Hq, int D, int max_kv_len, long long total_kv,
                                        int num_pieces);

/*
 * Split-KV decode with the Split operator applied to the packed key array
 * of the whole batch as one reduction dimension [CA "Split演算子による
 * Split-Kの対応": the split is a symbol the scheduler fixes later; AB]: the
 * rows [0, total_kv) of k / v are cut into P pieces of c = ceil(total_kv /
 * P) rows, and split i of request b is the request's intersection with the
 * i-th piece it overlaps.  Every piece holds the same number of keys
 * whatever the length mix, so a ragged batch keeps all compute units busy
 * to the end; one workgroup reduces one piece for up to four KV heads (the
 * request segments inside it one after another, online softmax over key
 * tiles [CA "複数リダクションのスケジューリング"]).  The merge
 * (log-sum-exp weights, as attn_merge_lse) then combines the pieces of each
 * request and writes O = 0, LSE = -inf for empty requests.
 *
 * Arguments as attn_decode_splitkv, except:
 * num_pieces  P in [1, 65535], or 0 for attn_decode_flat_pieces.
 * total_kv    the row count of k and v (<= 2^31 - 1); every kv_indptr entry
 *   must lie in [0, total_kv].  Rows outside every request are not read.
 * workspace   at least attn_decode_flat_workspace_bytes(B, Hq, D, max_kv_len,
 *   total_kv, P) bytes; layout o_part [s, B*Hq, D], m_part [s, B*Hq],
 *   l_part [s, B*Hq] fp32, s = attn_decode_flat_max_splits(...), split i of
 *   request b in slot i.  Calls that share one workspace must not overlap.
 * Supported: dtype ATTN_BF16 or ATTN_F16; D in {64, 128}; 1 <= G <= 16.
 */
attn_status_t attn_decode_splitkv_flat(const void* q, const void* k, const void* v,
                                       const int32_t* kv_indptr, void* o, float* lse, int B,
                                       int Hq, int Hkv, int D, int max_kv_len, long long total_kv,
                                       float scale, int num_pieces, int dtype, void* workspace,
                                       size_t workspace_bytes, void* hip_stream);

/* ---- multi-head latent attention (MLA) decode, absorbed form ----------- */

/* Workspace bytes of attn_mla_decode with s splits: s * B * H * (512 * 2 +
 * 6 * 4) (partial outputs of the 512-wide latent part in fp16, each 128-dim
 * quarter divided by a power-of-two scale kept in fp32, then fp32 maxima and
 * sums), rounded up to 256; 0 for invalid arguments. */
size_t attn_mla_decode_workspace_bytes(int B, int H, int num_splits);

/* The split count attn_mla_decode picks when num_splits = 0.  hg = H / 64
 * workgroups per chunk when H is a multiple of 64 (the many-head kernel),
 * else ceil(H / 16).
 *  - equal lengths: s = ceil(max_kv_len / c), c the largest power of two
 *    >= 256 keys such that hg * B * ceil(max_kv_len / c) reaches one
 *    workgroup per compute unit;
 *  - ragged, 16-head workgroups: the same with chunks counted as total_kv /
 *    c + B / 2, two workgroups per compute unit, and s made odd (so that
 *    the requests' first splits do not all land on the same XCDs);
 *  - ragged, many-head kernel (which launches only the chunks a request
 *    has): with slots = 0.95 * CUs / hg and k the fewest rounds such that
 *    k * slots - B / 2 >= slots / 2, c = max(256, ceil(total_kv / (k *
 *    slots - B / 2))) and s = floor(max_kv_len / c), raised to
 *    min(floor(CUs / (hg B)), floor(max_kv_len / 256)) when that is larger
 *    (B * s units fit one per compute unit whatever the lengths).
 * Within [1, 256].  Fitted to sweeps on MI355X. */
int attn_mla_decode_choose_splits(int B, int H, long long total_kv, int max_kv_len);

/*
 * Multi-head latent attention decode in its absorbed form ([AB] lists MLA
 * among the attention subgraphs; the shapes are not on the pages, so the
 * widths below are those of the published DeepSeek-V2/V3 models): every
 * query head attends to one cache row per token shared by all heads, a
 * latent vector of Dc = 512 elements followed by a rotary key part of
 * Dr = 64.  The score of head h and token j is scale * q_h . kv_j over all
 * 576 elements; the output is the softmax-weighted sum of the latent parts
 * kv_j[0 .. 511].  The Split operator cuts each request's keys into chunks
 * of c = ceil(max_kv_len / s) keys [CA "Split演算子によるSplit-Kの対応"],
 * exactly as attn_decode_splitkv; each chunk is reduced with an online
 * softmax over LDS-staged key tiles [CA "複数リダクションのスケジューリング"]
 * and the chunks are merged with log-sum-exp weights.
 *
 * q         [B, H, 576]           element type `dtype` (latent part first)
 * kv        [total_kv, 576]       request b owns rows kv_indptr[b] .. kv_indptr[b+1]-1
 * kv_indptr [B + 1] int32, device
 * o         [B, H, 512]           element type `dtype`
 * lse       [B, H] fp32 (natural log), or NULL
 * Dc, Dr      512 and 64 (other widths: ATTN_EUNSUPPORTED)
 * max_kv_len  the longest request (keys past max_kv_len of a request are not
 *   attended: s chunks of ceil(max_kv_len / s) keys cover it)
 * total_kv    kv_indptr[B] - kv_indptr[0]; for ragged lengths the
 *   many-head kernel launches min(s * B, ceil(total_kv / c) + B) workgroups
 *   per 64 heads, one per (request, chunk) the request has, so a smaller
 *   total_kv leaves requests unwritten.
 * num_splits  s in [1, 256], or 0 for attn_mla_decode_choose_splits; s = 1
 *   needs no workspace (may be NULL).
 * workspace   at least attn_mla_decode_workspace_bytes(B, H, s) bytes when
 *   s > 1; layout o_part [s, B*H, 512] fp16, then fp32 x_part [s, B*H, 4]
 *   (o_part's 128-dim quarters hold o / x), m_part [s, B*H], l_part [s, B*H].
 *   Calls that share one workspace must not overlap in time.
 * A request with no key yields O = 0, LSE = -inf.  A workgroup serves 64
 * heads when H is a multiple of 64, else 16; any H >= 1 is accepted.  The
 * 64-head kernel weighs a chunk's keys against the row max of its first
 * 32 keys and, should a later key's weight exceed 2^64 (2^15 for
 * ATTN_F16), reduces the chunk a second time against its true row max, so
 * results do not depend on the path.  Supported: ATTN_BF16, ATTN_F16.
 */
attn_status_t attn_mla_decode(const void* q, const void* kv, const int32_t* kv_indptr, void* o,
                              float* lse, int B, int H, int Dc, int Dr, int max_kv_len,
                              long long total_kv, float scale, int num_splits, int dtype,
                              void* workspace, size_t workspace_bytes, void* hip_stream);

/* Piece count attn_mla_decode_flat picks when num_pieces = 0: one 64-head
 * workgroup per compute unit, P = CUs / (H / 64), capped so that no piece
 * is shorter than 256 keys, within [1, 65535]; 1 for invalid arguments. */
int attn_mla_decode_flat_pieces(int B, int H, long long total_kv);

/* Workspace bytes of attn_mla_decode_flat: s * B * H * (512 * 2 + 6 * 4) with
 * s = attn_decode_flat_max_splits(max_kv_len, total_kv, num_pieces), rounded
 * up to 256 (0 for invalid arguments). */
size_t attn_mla_decode_flat_workspace_bytes(int B, int H, int max_kv_len, long long total_kv,
                                            int num_pieces);

/*
 * MLA decode (the operation of attn_mla_decode) with the Split operator
 * applied to the packed cache of the whole batch as one reduction dimension
 * [CA "Split演算子によるSplit-Kの対応": the split is a symbol the scheduler
 * fixes later; AB]: the rows [0, total_kv) of kv are cut into P pieces of
 * c = ceil(total_kv / P) rows, and split i of request b is the request's
 * intersection with the i-th piece it overlaps.  One 64-head workgroup
 * reduces one piece for its heads (the request segments inside it one after
 * another), so every workgroup streams the same number of cache rows
 * whatever the length mix; the merge (log-sum-exp weights) then combines
 * the pieces of each request and writes O = 0, LSE = -inf for empty
 * requests.
 * Arguments as attn_mla_decode, except:
 * H           a multiple of 64 (the many-head kernel); others ATTN_EUNSUPPORTED.
 * num_pieces  P in [1, 65535], or 0 for attn_mla_decode_flat_pieces.
 * total_kv    the row count of kv (<= 2^31 - 1); every kv_indptr entry must
 *   lie in [0, total_kv].  Rows outside every request are not read.
 * workspace   at least attn_mla_decode_flat_workspace_bytes(B, H, max_kv_len,
 *   total_kv, P) bytes (always needed); layout as attn_mla_decode's
 *   (o_part fp16, x_part, m_part, l_part), split i of request b in slot i.  Calls
 *   that share one workspace must not overlap in time.
 */
attn_status_t attn_mla_decode_flat(const void* q, const void* kv, const int32_t* kv_indptr,
                                   void* o, float* lse, int B, int H, int Dc, int Dr,
                                   int max_kv_len, long long total_kv, float scale, int num_pieces,
                                   int dtype, void* workspace, size_t workspace_bytes,
                                   void* hip_stream);

/*
 * Merge of Split partials [CA "Split演算子によるSplit-Kの対応"]: for each row r,
 *   M = max_i m_i over partials with l_i > 0;  w_i = l_i exp(m_i - M);
 *   O = sum_i w_i o_i / sum_i w_i;  LSE = M + ln sum_i w_i.
 * Partials with l_i <= 0 are skipped without reading o_i (an unused split
 * carries m = -inf, l = 0).  A row with no usable partial gets O = 0 and
 * LSE = -inf.
 * o_part [num_splits, rows, D] fp32 (each o_i already normalised by its l_i);
 * m_part, l_part [num_splits, rows] fp32, natural-log units;
 * o [rows, D] of type o_dtype (ATTN_F32, ATTN_BF16 or ATTN_F16);
 * lse [rows] fp32 or NULL.  1 <= num_splits <= 256; D in {64, 128}.
 */
attn_status_t attn_merge_lse(const float* o_part, const float* m_part, const float* l_part,
                             int num_splits, int rows, int D, void* o, int o_dtype, float* lse,
                             void* hip_stream);

/* ---- prefill ----------------------------------------------------------- */

/*
 * Fused prefill attention over a ragged batch, MFMA path: query tiles stay
 * on chip while key/value tiles stream through LDS (iterative tiling of the
 * key dimension), and the row max and row sum are updated in the same loop
 * over the same score tile (horizontal fusion) [CA "複数リダクションの
 * スケジューリング"; AB].
 *
 * q, o  [total_q, Hq, D];  k, v  [total_kv, Hkv, D]  (element type dtype)
 * qo_indptr, kv_indptr [B + 1] int32, device: request b owns query rows
 *   qo_indptr[b] .. qo_indptr[b+1]-1 and key rows kv_indptr[b] .. kv_indptr[b+1]-1.
 * lse [total_q, Hq] fp32, or NULL.
 * max_q_len, max_kv_len: the largest per-request lengths (bounds of the grid).
 * causal: 0 = every key of the request; 1 = key j is valid for query i iff
 *   j <= i + n_kv - n_q (bottom-right aligned; plain j <= i when n_q = n_kv).
 * scale must be positive (as is 1/sqrt(D)).
 * Supported: dtype ATTN_BF16 or ATTN_F16; D in {64, 128}; any G >= 1.
 */
attn_status_t attn_prefill(const void* q, const void* k, const void* v,
                           const int32_t* qo_indptr, const int32_t* kv_indptr, void* o,
                           float* lse, int B, int Hq, int Hkv, int D, int max_q_len,
                           int max_kv_len, float scale, int causal, int dtype,
                           void* hip_stream);

/* Workspace bytes attn_prefill_splitkv needs for `num_splits` splits:
 * num_splits * total_q * Hq * (2 D + 12) (fp16 partial outputs, then fp32
 * maxima, sums and row scales), rounded up to 256 bytes; 0 for invalid
 * arguments. */
size_t attn_prefill_workspace_bytes(long long total_q, int Hq, int D, int num_splits);

/* The split count attn_prefill_splitkv picks when num_splits = 0: 1 when the
 * B * Hq * ceil(max_q_len / 128) query-tile workgroups already give two per
 * compute unit; otherwise enough splits to reach two per compute unit,
 * with chunks of at least 1024 keys, clamped to [1, 256].  [CA] leaves the
 * concrete s to the scheduler; this is that scheduler's rule. */
int attn_prefill_choose_splits(int B, int Hq, int Hkv, int D, int max_q_len, int max_kv_len);

/*
 * Prefill / append with the key dimension cut by the Split operator [CA
 * "Split演算子によるSplit-Kの対応"]: the operation and the arguments of
 * attn_prefill, for batches whose query tiles alone cannot fill the chip
 * (a few new tokens against a long key/value history).  Split i covers key
 * offsets [i*c, min((i+1)*c, n_kv)) of each request, c = ceil(max_kv_len /
 * s); it computes, for every query row, the softmax-weighted output over
 * its valid keys in that range (causal masking as in attn_prefill), and a
 * merge combines the splits by log-sum-exp weights (as attn_merge_lse).
 * total_q   qo_indptr[B] (sizes the workspace).
 * num_splits  s in [1, 256], or 0 to use attn_prefill_choose_splits;
 *   s = 1 is attn_prefill itself (no workspace needed).
 * workspace  device memory of at least attn_prefill_workspace_bytes(total_q,
 *   Hq, D, s) bytes, 16-byte aligned; contents on entry do not matter.
 *   Layout: o_part [s, total_q*Hq, D] fp16, then m_part, l_part and x_part
 *   [s, total_q*Hq] fp32 (row = query row * Hq + head): split i's
 *   normalised output row is o_part[i, row, :] * x_part[i, row], a power
 *   of two that brings the row's largest magnitude into [1/2, 1); a split
 *   without valid keys for a row leaves (m, l) = (-inf, 0) there.  Calls sharing one
 *   workspace must not overlap in time.
 * Two kernels are enqueued on hip_stream: the split partials, then the merge.
 * Supported: as attn_prefill, with ceil(max_q_len / 128) * s <= 65535 and
 * total_q * Hq <= 2^30 when s > 1.
 */
attn_status_t attn_prefill_splitkv(const void* q, const void* k, const void* v,
                                   const int32_t* qo_indptr, const int32_t* kv_indptr, void* o,
                                   float* lse, int B, int Hq, int Hkv, int D, int max_q_len,
                                   int max_kv_len, long long total_q, float scale, int causal,
                                   int num_splits, int dtype, void* workspace,
                                   size_t workspace_bytes, void* hip_stream);

/* ---- block-sparse prefill (BSR outer tiles + 8x8 bitmaps) -------------- */

/*
 * Two-level sparse mask of [ST "2 段階ストレージ形式"]: the L x L mask is cut
 * into 64 x 64 outer tiles (OTs).  An OT whose elements are all valid is a
 * "full" OT; one with valid and invalid elements is a "part" OT; an OT with
 * no valid element is not stored and never read.  Per query block row
 * (64 queries), the stored OTs are listed by key block in CSR form, full and
 * part separately, each list ascending.  A part OT carries 64 uint64 inner
 * tile bitmaps: word ir*8 + ic covers queries 8*ir .. 8*ir+7 and keys
 * 8*ic .. 8*ic+7 of the OT; bit r*8 + c (LSB first) is 1 iff query 8*ir+r
 * may attend key 8*ic+c.
 * The struct lives in host memory; its array pointers are device memory
 * (for attn_prefill_bsr and attn_debug_bsr_decode).
 */
typedef struct {
  int seq_len;                  /* L, a multiple of 64 */
  int num_blocks;               /* L / 64 */
  int nnz_full, nnz_part;       /* stored OT counts */
  const int32_t* full_indptr;   /* [num_blocks + 1] */
  const int32_t* full_kblock;   /* [nnz_full] key-block index of each full OT */
  const int32_t* part_indptr;   /* [num_blocks + 1] */
  const int32_t* part_kblock;   /* [nnz_part] */
  const uint64_t* part_bits;    /* [nnz_part * 64] inner-tile bitmaps */
} attn_bsr_mask;

/*
 * Encode a dense 0/1 mask (host memory, uint8 [L, L], row = query, nonzero =
 * attend) into the canonical two-level form above, on the host.  Call once
 * with all output pointers NULL to get nnz_full / nnz_part, then again with
 * arrays of those sizes (host memory) to fill them.
 */
attn_status_t attn_bsr_encode_host(const uint8_t* dense, int L, int32_t* full_indptr,
                                   int32_t* full_kblock, int32_t* part_indptr,
                                   int32_t* part_kblock, uint64_t* part_bits, int* nnz_full,
                                   int* nnz_part);

/*
 * Block-sparse prefill: the block-wise kernel of [ST "デュアルカーネル戦略"].
 * Per (query block, head, batch) a workgroup walks only the stored OTs of
 * its block row; full OTs take no per-element test, part OTs apply their
 * bitmaps as a predicate before the row max; unstored OTs are never read.
 * q, o [B, L, Hq, D]; k, v [B, L, Hkv, D]; lse [B, L, Hq] fp32 or NULL.
 * One mask serves every batch entry and head.  scale must be positive.
 * Supported: dtype ATTN_F16 or ATTN_BF16; D in {64, 128}; L % 64 == 0.
 */
attn_status_t attn_prefill_bsr(const void* q, const void* k, const void* v,
                               const attn_bsr_mask* mask, void* o, float* lse, int B, int L,
                               int Hq, int Hkv, int D, float scale, int dtype,
                               void* hip_stream);

/*
 * Several masks stacked in one attn_bsr_mask, for per-head (or per head
 * group) sparsity [ST "2 段階ストレージ形式"]: num_masks masks of the same
 * L, mask m's indptr arrays at full_indptr + m*(num_blocks + 1) and
 * part_indptr + m*(num_blocks + 1), with values indexing the concatenated
 * kblock / bits arrays; nnz_full / nnz_part are totals.  Encoder: dense is
 * uint8 [num_masks, L, L]; same two-pass protocol as attn_bsr_encode_host
 * (which is this call with num_masks = 1); indptr outputs need
 * num_masks * (L/64 + 1) entries.
 */
attn_status_t attn_bsr_encode_host_stacked(const uint8_t* dense, int num_masks, int L,
                                           int32_t* full_indptr, int32_t* full_kblock,
                                           int32_t* part_indptr, int32_t* part_kblock,
                                           uint64_t* part_bits, int* nnz_full, int* nnz_part);

/*
 * attn_prefill_bsr with num_masks stacked masks (layout above): query head h
 * uses mask h / (Hq / num_masks); num_masks must divide Hq (1: one mask for
 * every head, Hq: one mask per head).  attn_prefill_bsr is this call with
 * num_masks = 1.
 */
attn_status_t attn_prefill_bsr_heads(const void* q, const void* k, const void* v,
                                     const attn_bsr_mask* mask, int num_masks, void* o,
                                     float* lse, int B, int L, int Hq, int Hkv, int D, float scale,
                                     int dtype, void* hip_stream);

/*
 * Block-sparse prefill, row-wise kernel [ST "デュアルカーネル戦略"]: the same
 * operation, arguments, layouts and errors as attn_prefill_bsr_heads.  Each
 * wave takes 16 query rows of one head on its own (no workgroup barrier) and
 * visits only the 16-key blocks of its outer-tile row in which those rows
 * hold a valid element, so masks whose part tiles are sparse inside cost less
 * than with the block-wise kernel, which computes every stored 64x64 tile.
 */
attn_status_t attn_prefill_bsr_rows(const void* q, const void* k, const void* v,
                                    const attn_bsr_mask* mask, int num_masks, void* o,
                                    float* lse, int B, int L, int Hq, int Hkv, int D, float scale,
                                    int dtype, void* hip_stream);

/*
 * Kernel choice [ST "デュアルカーネル戦略", カーネル選択]: an analytical model
 * over the mask's sparsity and the sequence length picks the row-wise or the
 * block-wise kernel.  Inputs are the host arrays of the encoder (num_masks
 * stacked masks of length L; part_bits may be null when no part tile is
 * stored) and the call's shape (Hq query heads, B batch entries, head dim D
 * 64 or 128).  The model counts the stored outer tiles (block-wise work) and
 * the (16-row slab, 16-key block) pairs holding a valid element (row-wise
 * work), and prices each kernel as a launch floor plus a per-unit time over
 * all heads and batch entries, fitted on MI355X; plan->kernel is the
 * cheaper.  Host only; fails with ATTN_EINVAL on null pointers, L not a
 * positive multiple of 64, num_masks not dividing Hq, or indptr not
 * monotone, and ATTN_EUNSUPPORTED on another D.
 */
enum { ATTN_BSR_BLOCKWISE = 0, ATTN_BSR_ROWWISE = 1 };
typedef struct {
  long long stored_ots; /* full + part outer tiles over all masks */
  long long row_blocks; /* (16-row slab, 16-key block) pairs with a valid element */
  double block_cost;    /* modelled time of the block-wise kernel, us */
  double row_cost;      /* modelled time of the row-wise kernel, us */
  int kernel;           /* ATTN_BSR_BLOCKWISE or ATTN_BSR_ROWWISE */
} attn_bsr_plan;
attn_status_t attn_bsr_plan_host(const int32_t* full_indptr, const int32_t* part_indptr,
                                 const uint64_t* part_bits, int num_masks, int L, int Hq, int B,
                                 int D, attn_bsr_plan* plan);

/* ---- test exports ------------------------------------------------------ */

/* Write, with the device code the decode kernels use, every split's key range
 * into ranges [B, num_splits, 2] int32 (device): [begin, end) as offsets
 * within the request, or -1, -1 for a split the request does not use.
 * Synchronises the stream before returning. */
attn_status_t attn_debug_split_ranges(const int32_t* kv_indptr, int B, int max_kv_len,
                                      int num_splits, int32_t* ranges, void* hip_stream);

/* Write, with the device code attn_decode_splitkv_flat uses, the flat
 * plan's split ranges: ranges [B, s, 2] int32 on the device (s =
 * attn_decode_flat_max_splits(max_kv_len, total_kv, num_pieces)), slot i of
 * request b = [begin, end) as key offsets within the request, -1, -1 for
 * slots the request does not use.  Synchronises the stream. */
attn_status_t attn_debug_flat_ranges(const int32_t* kv_indptr, int B, int max_kv_len,
                                     long long total_kv, int num_pieces, int32_t* ranges,
                                     void* hip_stream);

/* Expand a two-level mask to dense uint8 [L, L] (device) with the predicate
 * the block-sparse kernel applies.  Synchronises the stream. */
attn_status_t attn_debug_bsr_decode(const attn_bsr_mask* mask, uint8_t* dense,
                                    void* hip_stream);

#ifdef __cplusplus
}
#endif
#endif
