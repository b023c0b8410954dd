/*
 * csa.h -- C ABI of the MI355X (gfx950) hybrid compressed attention forward.
 *
 * The method (DeepSeek-V4 hybrid attention) as the pages state it:
 *  - CSA compresses the KV cache every m = 4 tokens into one entry by a
 *    weighted average with overlap between adjacent blocks, scores the
 *    entries with a low-rank FP4 "Lightning Indexer", lets each query token
 *    attend only to its top-k entries, and uses shared-KV multi-query
 *    attention (one entry row is both key and value)
 *        ("DeepSeek-V4: Towards Highly Efficient Million-Token Context
 *          Intelligence" wiki summary, Proposed method, item 1;
 *          "deepseek V4 技术论文", part 1.1, CSA bullets);
 *  - HCA compresses every m' = 128 tokens and attends densely (same places);
 *  - both add a sliding-window branch of n_win = 128 raw tokens, a learnable
 *    per-head attention sink, and partial RoPE on the last 64 dims with the
 *    inverse rotation applied to the attention output (wiki summary, item 1);
 *  - the inference cache keeps the RoPE dims in BF16 and the other dims in
 *    FP8 (wiki summary, Training infrastructure item 5); the indexer QK path
 *    is MXFP4 (wiki summary, Post-training item 3).
 *
 * Conventions shared by every call
 *  - Pointers: every tensor argument is a DEVICE pointer owned by the caller.
 *    The library never allocates, frees or synchronises; it launches only on
 *    the given stream (a hipStream_t passed as void*, NULL = default stream),
 *    so every call is asynchronous and stream-ordered.
 *  - Layout: row-major, contiguous, batch-major [B, ...]; base pointers
 *    16-byte aligned.  bf16 = uint16 bit patterns.  MXFP4 = packed e2m1
 *    nibbles (element 2j in the low nibble of byte j) plus one e8m0 byte
 *    (2^(byte-127)) per 32 consecutive elements.  FP8 = OCP e4m3fn bytes.
 *  - Sizes: D (head dim) = 128, rope_dims = 64 or 0, d_idx = 64.
 *  - Positions are absolute int64.  Query row q of every batch row sits at
 *    t = q_pos0 + q.  Compressed entry s sits at p_s = (s+1)*m - 1 (its last
 *    token) and is visible to t iff p_s <= t.
 *  - RoPE: pairs (D-R+2f, D-R+2f+1) rotated by pos * rope_base^(-2f/R).
 *    q and raw window rows come in pre-RoPE and are rotated on load at t and
 *    j; entries are stored post-RoPE (rotated at p_s by csa_compress).
 *  - Errors: each call returns an int status (CSA_OK = 0 or a negative
 *    code).  Arguments are validated on the host before anything is
 *    launched; on error nothing is launched and csa_last_error() returns a
 *    thread-local message naming the argument.  No exception crosses the ABI.
 *  - Determinism: every result is bitwise reproducible run to run, and a
 *    query row's result depends only on its own inputs (its query, position
 *    and key set), not on the batch size, the number of rows in the call or
 *    which other rows are in it (batch invariance).  csa_index_topk writes
 *    each row's indices in one canonical order, so the attention that
 *    consumes them sees the same key order whatever path selected them.
 */
#ifndef CSA_MI355X_H
#define CSA_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define CSA_OK 0
#define CSA_INVALID_ARG (-1)
#define CSA_UNSUPPORTED (-2)
#define CSA_WORKSPACE_TOO_SMALL (-3)
#define CSA_HIP_ERROR (-4)

/* formats */
#define CSA_FMT_BF16 0          /* entries [.., 128] bf16 / indexer [.., 64] bf16 */
#define CSA_FMT_MXFP4 1         /* indexer: codes [.., 32] u8 + scales [.., 2] u8 */
#define CSA_FMT_FP8_ROPE_BF16 2 /* entries: e4m3 [.., 64] + bf16 [.., 64] + f32 scale [..] */
#define CSA_FMT_NVFP4 3         /* entries: records [.., 72] u8 (64 B e2m1 codes of the 128
                                   post-RoPE dims + 8 e4m3 scales of 16-dim blocks) + f32 scale [..] */
#define CSA_FMT_FP8 4           /* window cache: e4m3 [.., 128] of post-RoPE rows + f32 scale [..]
                                   (amax / 448 over the 128 dims) */
#define CSA_FMT_BF16_ROPED 5    /* window: bf16 [.., 128] rows already rotated at their positions
                                   (csa_rope_rows) */

/*
 * csa_compress -- token-level compressor (CSA: m = 4 with overlap; HCA:
 * m = 128 without).  Wiki summary, Proposed method item 1 ("compress every
 * m tokens into one entry by a weighted average, overlapping adjacent
 * blocks"); "deepseek V4 技术论文" 1.1 (C^b overlaps C^a).
 *
 * Entry i pools the m tokens of block i (role "a") and, when overlap = 1,
 * also the m tokens of block i-1 (role "b").  Slot r of the L = 2m (or m)
 * slots has logit beta[r] + z[j][role] (z = NULL means 0; column 0 = role a,
 * column 1 = role b); slots before token 0 are absent.  The weights are the
 * softmax of the logits computed in fp64 and rounded to fp32; the pooled
 * row is an fp32 fma chain over the slots in ascending order; the KV entry
 * is then rotated at p_i = (i+1)m - 1 (rotation in fp64) and stored.  The
 * indexer-key stream ik is pooled with the same weights, not rotated, and
 * stored as bf16 or MXFP4.
 *
 *  kv        [B, T, 128] bf16, tokens at positions pos0 .. pos0+T-1
 *  ik        [B, T, 64] bf16 or NULL (no indexer stream, e.g. HCA)
 *  z         [B, T, 2] fp32 or NULL
 *  beta      [L] fp32, L = 2m if overlap else m
 *  prev_kv   [B, m, 128] bf16: the m tokens just before pos0; required when
 *            overlap = 1 and pos0 > 0, ignored otherwise (may be NULL)
 *  prev_ik   [B, m, 64] bf16: same for ik (required iff ik and prev_kv are)
 *  prev_z    [B, m, 2] fp32 or NULL
 *  pos0      multiple of m; one entry is written per block of m tokens that
 *            ends inside [pos0, pos0+T): N_new = T / m entries, the first with
 *            entry index pos0/m.  Trailing tokens of an incomplete block form
 *            no entry (the caller passes them again with the next chunk).
 *  entries_out       entry_fmt BF16: [B, N_new, 128] bf16.
 *                    entry_fmt FP8_ROPE_BF16: [B, N_new, 64] e4m3 codes of
 *                    x / scale, scale = amax(dims 0..63) / 448 (fp32).
 *                    entry_fmt NVFP4 (the V4.1 variant of the Russian
 *                    summary: the cache held in NVFP4, quantised after RoPE):
 *                    [B, N_new, 72] u8 records.  Per entry s = amax / 2688
 *                    (= amax / (6 * 448)); block j (dims 16j .. 16j+15) has
 *                    the e4m3 scale b_j = e4m3(amax_j / (6 s)); dim d is the
 *                    e2m1 code of x_d / (b_j s), 0 when b_j s = 0 (every step
 *                    one fp32 operation, round to nearest even; e4m3 and
 *                    e2m1 saturate).  Bytes 0..63: codes, dim 2i in the low
 *                    nibble of byte i; bytes 64..71: b_0 .. b_7.
 *  entries_rope_out  FP8_ROPE_BF16 only: [B, N_new, 64] bf16 (dims 64..127)
 *  entry_scale_out   FP8_ROPE_BF16 and NVFP4: [B, N_new] fp32
 *  kidx_out          [B, N_new, 64] bf16, or [B, N_new, 32] MXFP4 codes
 *  kidx_scale_out    MXFP4 only: [B, N_new, 2] e8m0
 * Returns CSA_INVALID_ARG for a bad shape, format or missing prev rows.
 */
int csa_compress(const void* kv, const void* ik, const float* z, const float* beta,
                 const void* prev_kv, const void* prev_ik, const float* prev_z,
                 int B, int T, int64_t pos0, int D, int d_idx, int m, int overlap,
                 int rope_dims, float rope_base,
                 void* entries_out, void* entries_rope_out, float* entry_scale_out,
                 int entry_fmt, void* kidx_out, uint8_t* kidx_scale_out, int kidx_fmt,
                 void* stream);

/*
 * csa_cache_append -- decode cache write path: one new token per sequence.
 * Wiki summary, Training infrastructure item 5 (inference keeps a state cache
 * of recent raw tokens and a compressed cache: RoPE dims BF16, other dims
 * FP8) and Proposed method item 1 (an entry every m tokens).  The new row of
 * position t is stored in the state rings; if t completes block i (t + 1 =
 * (i+1)m), entry i is pooled exactly as csa_compress pools it (same
 * weights, order, RoPE at p_i = t and storage codes, so the caches are
 * byte-identical to a whole-sequence csa_compress) and written to row i.
 *
 *  kv_new    [B, 128] bf16 raw (pre-RoPE) row of position t
 *  ik_new    [B, 64] bf16 indexer-stream row, or NULL (no indexer, e.g. HCA)
 *  z_new     [B, 2] fp32 slot-logit offsets of the row, or NULL (z = 0)
 *  t         position of the new rows (the same for every sequence)
 *  kv_ring   [B, 2W, 128] bf16 state ring: row j sits at slots j % W and
 *            j % W + W, so the window rows max(0, t-W+1) .. t are contiguous
 *            from slot s0 = max(0, t-W+1) % W.  csa_attend / hca_attend can
 *            read it directly as win_kv with win_len = 2W and win_pos0 =
 *            max(0, t-W+1) - s0.
 *  ik_ring   [B, W, 64] bf16 (slot j % W), with ik_new, else NULL
 *  z_ring    [B, W, 2] fp32 (slot j % W), with z_new, else NULL
 *  win8_ring [B, 2W, 128] e4m3, or NULL: the FP8 sliding-window cache of
 *            the V4.1 variant (the Russian summary: SWA cache in FP8).  Row
 *            t, rotated at t (fp64, as the entries), rounded to fp32 and
 *            coded over all 128 dims with scale amax / 448, goes to slots
 *            t % W and t % W + W like kv_ring, so csa_attend can read it as
 *            an FP8 window (win_fmt = CSA_FMT_FP8) in the same way
 *  win8_scale [B, 2W] fp32, with win8_ring
 *  W         ring length in rows, >= L (2m with overlap, else m); 128 holds
 *            the sliding window
 *  beta, m, overlap, rope_dims, rope_base: as csa_compress
 *  entries, entries_rope, entry_scale, entry_fmt, kidx, kidx_scale,
 *  kidx_fmt: the caches, as csa_compress's outputs but with N_cap rows per
 *            sequence (entry i of sequence b at row b * N_cap + i)
 * The rings must hold the rows of the L - 1 positions before t (earlier
 * calls, or a prefill that filled them the same way).  Cache arguments may be
 * NULL on calls that complete no block.  Calls for one sequence must be
 * ordered on one stream.  Returns CSA_INVALID_ARG for a bad shape, W < L, or
 * an entry index >= N_cap.
 */
int csa_cache_append(const void* kv_new, const void* ik_new, const float* z_new, int B, int64_t t,
                     void* kv_ring, void* ik_ring, float* z_ring, void* win8_ring, float* win8_scale,
                     int W, const float* beta, int m,
                     int overlap, int rope_dims, float rope_base, void* entries, void* entries_rope,
                     float* entry_scale, int entry_fmt, void* kidx, uint8_t* kidx_scale, int kidx_fmt,
                     int N_cap, void* stream);

/*
 * csa_index_topk -- Lightning Indexer scores and per-query top-k selection.
 * Wiki summary item 1 (indexer scores in FP4), "deepseek V4 技术论文" 1.1
 * (low-rank + FP4 indexer selects the top-k entries per query token),
 * aifrontier EP95 "Lightning Indexer and top-k" segment (top-k must see every
 * entry).  The pages give no formula; this library computes the DSA form
 *     I[t,s] = sum_h w[t,h] * relu(<qI[t,h], kI[s]>)
 * for every visible entry s (p_s <= t, s < N): each dot product in fp32
 * (exact for MXFP4 operands), the head sum as an fp32 fma chain in
 * ascending h starting from +0.  It keeps the min(k, n_vis) largest scores,
 * ties going to the lower entry index, and writes their indices followed by
 * -1 padding up to k.  The indices of a row are written in a canonical order
 * that depends on the selected set only: grouped by (index / 32) % 8, the
 * groups in ascending order, ascending within each group.
 *
 *  qidx        fmt BF16: [B, n, H_I, 64] bf16.  fmt MXFP4 with
 *              qidx_scale == NULL: [B, n, H_I, 64] bf16, quantised in-kernel
 *              to MXFP4 (OCP MX rule: E = floor(log2 amax) - 2, RNE,
 *              saturating).  fmt MXFP4 with qidx_scale: [B, n, H_I, 32] codes.
 *  qidx_scale  [B, n, H_I, 2] e8m0 or NULL
 *  widx        [B, n, H_I] fp32 head weights
 *  kidx        fmt BF16: [B, N, 64] bf16; fmt MXFP4: [B, N, 32] codes
 *  kidx_scale  fmt MXFP4: [B, N, 2] e8m0
 *  H_I         1..8; d_idx = 64; 1 <= k <= 2048
 *  idx_out     [B, n, k] int32
 *  ws, ws_bytes  device scratch of at least csa_index_topk_workspace_bytes()
 *              bytes, 16-byte aligned (may be NULL when that is 0).  It is
 *              non-zero for few query rows over long entry lists (n <= 4
 *              and at least 65536 visible entries), where each row's entry
 *              list is split over many work-groups: 32784 bytes per query
 *              row.  Its contents need no initialisation and are undefined
 *              after the call; calls that share a workspace must be ordered
 *              on one stream.
 *  fallback_count  NULL, or a caller-owned device uint32 (4-byte aligned):
 *              the kernels add the number of work-groups that took the exact
 *              streaming path (the sampled threshold, or on the split path
 *              the partitions' own cuts, left fewer than k or more
 *              candidates than a buffer holds, e.g. under massive score
 *              ties).  A diagnostic of slow calls; results are exact either
 *              way.  The caller clears it; it is updated in stream order.
 */
int csa_index_topk(const void* qidx, const uint8_t* qidx_scale, const float* widx,
                   const void* kidx, const uint8_t* kidx_scale, int fmt,
                   int B, int n, int64_t q_pos0, int H_I, int d_idx, int N, int m, int k,
                   int32_t* idx_out, void* ws, size_t ws_bytes, uint32_t* fallback_count,
                   void* stream);

size_t csa_index_topk_workspace_bytes(int B, int n, int64_t q_pos0, int N, int m, int k);

/*
 * csa_index_topk_noalloc -- csa_index_topk for callers that cannot allocate
 * device memory (code under HIP graph capture, serving loops, harnesses that
 * forbid hipMalloc): the same arguments without ws / ws_bytes, the same
 * kernels and results.  The split path's workspace is a static device array
 * of 8 MiB that every GPU the library runs on holds until the process ends
 * (256 query rows of the split path: B * n <= 256 when n <= 4 and a row sees
 * at least 65536 entries).  A call that would need more returns
 * CSA_WORKSPACE_TOO_SMALL and launches nothing.  The first call on a device
 * looks up the array's address there (no allocation); nothing is allocated,
 * freed or synchronised.  Every call on one GPU shares that GPU's array:
 * calls that overlap on one GPU (different streams, or host threads) race
 * and must be ordered by the caller.
 */
int csa_index_topk_noalloc(const void* qidx, const uint8_t* qidx_scale, const float* widx,
                           const void* kidx, const uint8_t* kidx_scale, int fmt,
                           int B, int n, int64_t q_pos0, int H_I, int d_idx, int N, int m, int k,
                           int32_t* idx_out, uint32_t* fallback_count, void* stream);

/*
 * csa_attend -- CSA core attention: sparse entries + sliding window + sink.
 * "deepseek V4 技术论文" 1.1 (each query attends to its top-k entries; the
 * entries are both key and value, shared by all heads: MQA), wiki summary
 * item 1 (n_win = 128 sliding-window branch, attention sink, partial RoPE
 * with inverse RoPE on the output).  For each (t, h) one softmax over
 *     {sink[h]} U {entries idx[t][i] >= 0} U {window rows j, max(0,t-n_win+1) <= j <= t}
 * with logits <rot(q[t,h], t), key> / sqrt(D) and the sink logit sink[h]
 * (zero value).  Value = key row (all 128 dims).  Output dims 64..127 get
 * the inverse rotation by t.  bf16 MFMA products, fp32 softmax and
 * accumulation, bf16 output.
 *
 *  q            [B, n, H, 128] bf16 pre-RoPE; 1 <= H <= 64
 *  entries      BF16: [B, N, 128] bf16 post-RoPE.  FP8_ROPE_BF16:
 *               [B, N, 64] e4m3 codes (value = code * entry_scale).
 *               NVFP4: [B, N, 72] records as csa_compress writes them
 *  entries_rope FP8_ROPE_BF16: [B, N, 64] bf16 (dims 64..127); else NULL
 *  entry_scale  FP8_ROPE_BF16 and NVFP4: [B, N] fp32; else NULL
 *  idx          [B, n, k] int32 entry indices, 16-byte aligned, k <= 2048;
 *               -1 marks an unused slot, and any index outside [0, N) is
 *               likewise no key
 *  win_kv       win_fmt BF16: [B, win_len, 128] bf16 pre-RoPE raw rows at
 *               positions win_pos0 .. win_pos0+win_len-1; must cover
 *               [max(0, q_pos0-n_win+1), q_pos0+n-1] when n_win > 0.
 *               win_fmt FP8 (the V4.1 variant's FP8 sliding-window cache,
 *               FP8 or NVFP4 entries only): [B, win_len, 128] e4m3 codes of
 *               the rows rotated at their positions, value = code *
 *               win_scale (csa_cache_append writes such a ring)
 *  n_win        0 (no window) .. 128; larger values are rejected
 *  win_fmt      CSA_FMT_BF16 (raw rows), CSA_FMT_BF16_ROPED (rows rotated at
 *               their positions by csa_rope_rows; needs rope_dims = 64) or
 *               CSA_FMT_FP8
 *  win_scale    FP8 window: [B, win_len] fp32; else NULL
 *  sink         [H] fp32 or NULL (no sink)
 *  out          [B, n, H, 128] bf16
 *  ws, ws_bytes device scratch of at least csa_attend_workspace_bytes()
 *               bytes, 16-byte aligned (may be NULL when that is 0).  It is
 *               non-zero for FP8 and NVFP4 entries with at least 16 chunks of
 *               32 keys (k + n_win >= 512): each token's keys are then split
 *               over several work-groups (parts of 8 chunks) whose partial
 *               softmax sums are merged in ascending part order.  The split
 *               depends on k and n_win only, never on B or n; the tokens run
 *               in blocks of at most 512, so the workspace is 33280 bytes
 *               per (query row, part) for min(B*n, 512) rows.  Contents are
 *               undefined after the call; calls that share a workspace must
 *               be ordered on one stream.
 */
int csa_attend(const void* q, int B, int n, int64_t q_pos0, int H, int D,
               const void* entries, const void* entries_rope, const float* entry_scale,
               int entry_fmt, int N, int m, const int32_t* idx, int k,
               const void* win_kv, int64_t win_pos0, int win_len, int n_win, int win_fmt,
               const float* win_scale, const float* sink, int rope_dims, float rope_base,
               void* out, void* ws, size_t ws_bytes, void* stream);

/*
 * csa_index_attend -- csa_index_topk followed by csa_attend for one layer's
 * query rows, pipelined over chunks of query tokens on two streams.  The
 * top-k set and the attention of a query token depend on that token's row
 * and the shared caches only ("deepseek V4 技术论文" 1.1: each query token
 * selects and attends to its own top-k entries), so the rows can be taken in
 * any grouping; the results are the bytes the two calls write.  The indexer
 * is bound by vector-ALU work and attention by the matrix cores, so the
 * indexer of chunk c + 1 (on aux_stream) runs beside the attention of chunk
 * c (on stream) and the two share the compute units.
 *
 *  arguments    as in csa_index_topk (qidx .. fallback_count, kidx_fmt =
 *               its fmt) and csa_attend (q .. out); B, n, q_pos0, N and m
 *               are common to both.  The indices are written to idx_out and
 *               read back by the attention.  No workspace: a call that
 *               would need one in either function (few query rows over
 *               long entry lists, FP8 or NVFP4 entries with k + n_win >=
 *               512) returns CSA_WORKSPACE_TOO_SMALL; use the two calls.
 *  n_chunks     requested chunk count.  With B = 1 the call uses
 *               min(n_chunks, n / 512) chunks (at least one) of n / chunks
 *               consecutive tokens; with B > 1 one chunk.
 *  stream       the caller's stream.  Everything already enqueued on it is
 *               complete before any chunk starts, and every chunk's work is
 *               complete before later work on stream starts: to the caller
 *               the call is ordered on stream like the two calls.
 *  aux_stream   a second stream of the same device (not stream, default
 *               priority), used when the call takes more than one chunk;
 *               nothing else enqueued on it is ordered with this call.
 *  events       three distinct hipEvent_t of the device (any creation
 *               flags), owned by the caller, recorded and waited on by the
 *               call; needed when the call takes more than one chunk.  Calls
 *               that share events or aux_stream must be issued from one host
 *               thread.
 *  Errors: every argument is checked before anything is enqueued; a HIP
 *  error during the enqueue returns CSA_HIP_ERROR with the chunks before it
 *  enqueued (the call then still tries to order the aux stream's work
 *  before later work on stream).  Nothing is allocated or synchronised.
 */
int csa_index_attend(const void* qidx, const uint8_t* qidx_scale, const float* widx, const void* kidx,
                     const uint8_t* kidx_scale, int kidx_fmt, int H_I, int d_idx, int k, int32_t* idx_out,
                     uint32_t* fallback_count, const void* q, int H, int D, const void* entries,
                     const void* entries_rope, const float* entry_scale, int entry_fmt, const void* win_kv,
                     int64_t win_pos0, int win_len, int n_win, int win_fmt, const float* win_scale,
                     const float* sink, int rope_dims, float rope_base, void* out, int B, int n, int64_t q_pos0,
                     int N, int m, int n_chunks, void* stream, void* aux_stream, void* const* events);

size_t csa_attend_workspace_bytes(int B, int n, int k, int n_win, int entry_fmt);

/*
 * hca_attend -- HCA dense attention over every visible entry + window + sink
 * (wiki summary item 1: HCA keeps dense attention over the m' = 128
 * compressed entries; "deepseek V4 技术论文" 1.1).  As csa_attend with the
 * entry set {s < N : (s+1)m - 1 <= t}; entries are BF16 [B, N, 128].
 */
int hca_attend(const void* q, int B, int n, int64_t q_pos0, int H, int D,
               const void* entries, int N, int m,
               const void* win_kv, int64_t win_pos0, int win_len, int n_win, int win_fmt,
               const float* sink, int rope_dims, float rope_base, void* out, void* stream);

/*
 * csa_rope_rows -- the window rows rotated once (wiki summary item 1:
 * partial RoPE on the last 64 dims).  out[b, i] = kv[b, i] with each pair
 * (64 + 2f, 65 + 2f) rotated by (pos0 + i) * rope_base^(-2f/64) in fp64,
 * rounded to fp32 and then to bf16 (the same rotation as the entries).
 * Attention that reads such rows as its window (win_fmt =
 * CSA_FMT_BF16_ROPED) does not rotate them per query token.
 *  kv, out  [B, T, 128] bf16, 4-byte aligned device pointers; out may be kv
 *  rope_dims  must be 64
 * Asynchronous on `stream`; nothing is launched on error.
 */
int csa_rope_rows(const void* kv, int B, int T, int64_t pos0, int rope_dims, float rope_base, void* out,
                  void* stream);

/*
 * Projections around the attention path (the step either side of it).
 * Wiki summary, Proposed method item 1: CSA pairs a shared-KV multi-query
 * attention with a grouped output projection, and its Lightning Indexer is
 * made cheap by a low-rank factorisation and FP4 ("deepseek V4 技术论文" 1.1);
 * Post-training item 3: the indexer's QK path is MXFP4.  The pages give no
 * formula; the readings taken are
 *   - every projection is linear, no bias, weights in the [out, in] layout,
 *     bf16 operands, fp32 accumulation;
 *   - the indexer query is q_I = lat . W_up^T with lat the bf16 indexer
 *     latent: an fp32 fma chain over the rank in ascending order, then
 *     MXFP4 per 32 outputs (OCP MX v1.0 rule: scale 2^(floor(log2 amax) - 2),
 *     e2m1 nearest-even, saturating);
 *   - the compression logits z (the per-token slot-logit offsets that
 *     csa_compress takes) are one more linear map of the hidden state;
 *   - the grouped output projection splits the H heads into G groups of
 *     consecutive heads and maps group j's (H/G)*D values onto output
 *     columns [j*d/G, (j+1)*d/G) with its own block of weights (nothing
 *     mixes the groups).
 *
 * csa_project_in -- x [M, d] bf16 (the hidden state of M tokens) times the
 * stacked weights w_in [n_q + n_kv + n_ik + n_lat + n_w + n_z, d] bf16 (W_q,
 * W_kv, W_ik, W_lat, W_w, W_z in that order) in one GEMM:
 *   q_out   [M, n_q]  bf16   (the query rows, pre-RoPE: [B, n, H, 128])
 *   kv_out  [M, n_kv] bf16   (the shared KV rows, pre-RoPE)
 *   ik_out  [M, n_ik] bf16   (the indexer key stream)
 *   lat_out [M, n_lat] bf16  (the indexer latent)
 *   w_out   [M, n_w]  fp32   (the indexer head weights)
 *   z_out   [M, n_z]  fp32   (the compression logits, n_z = 2 for
 *                             csa_compress's z)
 * and, when n_qidx > 0, the indexer query from lat_out and w_up
 * [n_qidx, n_lat] bf16: qidx_out [M, n_qidx/2] MXFP4 codes and
 * qidx_scale_out [M, n_qidx/32] e8m0 scales (the layout csa_index_topk
 * takes).  A width of 0 drops that output (its pointer may be NULL).
 * Outputs are written with row stride equal to their width.
 * Requirements: d a multiple of 32; n_lat in {16, 32, 64} when n_qidx > 0;
 * n_qidx a positive multiple of 32 (at most 2^20); x and w_in below
 * 2 GiB; x, w_in, w_up, lat_out and qidx_out 16-byte aligned.  Device
 * pointers, caller-owned; asynchronous on `stream`; nothing is launched on
 * error.
 *
 * csa_project_qidx -- the indexer-query step alone: lat [M, r] bf16,
 * w_up [n_qidx, r] bf16 -> qidx_out, qidx_scale_out as above, and, when
 * q_f32_out is non-NULL, the fp32 values that were encoded [M, n_qidx].
 *
 * csa_project_out -- grouped output projection: o [M, H*D] bf16 (attention
 * output rows, head-major), w_o [d, (H/G)*D] bf16 with group j's block in
 * rows [j*d/G, (j+1)*d/G) -> y_out [M, d] bf16.  (H/G)*D a multiple of 32,
 * d a multiple of G, o below 4 GiB, o and w_o 16-byte aligned.
 */
int csa_project_in(const void* x, int M, int d, const void* w_in, int n_q, int n_kv, int n_ik,
                   int n_lat, int n_w, int n_z, const void* w_up, int n_qidx, void* q_out,
                   void* kv_out, void* ik_out, void* lat_out, float* w_out, float* z_out,
                   uint8_t* qidx_out, uint8_t* qidx_scale_out, void* stream);

int csa_project_qidx(const void* lat, int M, int r, const void* w_up, int n_qidx,
                     uint8_t* qidx_out, uint8_t* qidx_scale_out, float* q_f32_out, void* stream);

int csa_project_out(const void* o, int M, int H, int D, int G, const void* w_o, int d,
                    void* y_out, void* stream);

/* Thread-local description of the last error (empty string if none). */
const char* csa_last_error(void);
/* Library version: major*10000 + minor*100 + patch. */
int csa_version(void);

#ifdef __cplusplus
}
#endif
#endif
