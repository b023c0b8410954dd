/*
 * csa_oracle.h -- plain, slow CPU oracle for the hybrid compressed attention
 * forward (CSA + HCA, sliding window, sink, partial RoPE).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may load this library.  It shares no code,
 * header, table or constant with the HIP library in
 * long_context_attention_21_amd/csrc, and must never be called by it.
 *
 * Sources (page titles as printed at the top of each page):
 *   [V4-wiki]  "DeepSeek-V4: Towards Highly Efficient Million-Token Context
 *              Intelligence" (wiki summary), section "Proposed method",
 *              item 1 "Hybrid attention (CSA + HCA)", and section
 *              "Training infrastructure" item 5 "Inference framework".
 *   [V4-zh]    "deepseek V4 技术论文", part 1.1 "Hybrid attention: CSA + HCA".
 *   [EP95]     aifrontier.kr podcast EP95, segment "Lightning Indexer and
 *              top-k selection over the KV cache".
 *
 * Every buffer is a plain host pointer; bf16 values are passed as uint16_t
 * bit patterns.  All functions are single-threaded per call unless stated;
 * the row-level drivers use OpenMP over independent rows.
 */
#ifndef CSA_ORACLE_H
#define CSA_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- number formats ------------------------------------------------------ */
uint16_t orc_bf16_from_f32(float x);             /* round to nearest even */
float    orc_bf16_to_f32(uint16_t b);
uint8_t  orc_e4m3_from_f32(float x);             /* OCP e4m3fn, RNE, saturating */
float    orc_e4m3_to_f32(uint8_t c);
float    orc_e2m1_to_f32(uint8_t code);          /* low 4 bits used */
/* MXFP4: n must be a multiple of 32. codes: n/2 bytes, element 2j in the low
 * nibble of byte j; scales: n/32 e8m0 bytes (value 2^(byte-127)). */
void orc_mxfp4_encode(const float* x, int n, uint8_t* codes, uint8_t* scales);
void orc_mxfp4_decode(const uint8_t* codes, const uint8_t* scales, int n, float* out);

/* ---- compression (one batch row) ----------------------------------------- */
/* Emits one entry per block of m tokens completed inside [pos0, pos0+T).
 * kv [T,D] bf16; ik [T,d_idx] bf16 or NULL; z [T,2] fp32 or NULL (slot-role
 * logits: column 0 = current block, column 1 = previous block);
 * beta [L] fp32 with L = 2m (overlap) or m; prev_* hold the m rows just
 * before pos0 (NULL when pos0 == 0).  Outputs (fp32, before storage
 * rounding): entries_out [T/m, D] post-RoPE; kidx_out [T/m, d_idx] (may be
 * NULL).  Returns the number of entries written, or -1 on a bad argument. */
int orc_compress(const uint16_t* kv, const uint16_t* ik, const float* z, const float* beta,
                 const uint16_t* prev_kv, const uint16_t* prev_ik, const float* prev_z,
                 int T, int64_t pos0, int D, int d_idx, int m, int overlap,
                 int rope_dims, double rope_base,
                 float* entries_out, float* kidx_out);

/* Storage of a post-RoPE entry row: bf16, or dims [0, D-R) as e4m3 codes
 * with one fp32 scale (amax/448) and dims [D-R, D) as bf16. */
void orc_store_entry_fp8(const float* row, int D, int rope_dims,
                         uint8_t* codes_out, uint16_t* rope_out, float* scale_out);

/* ---- RoPE ---------------------------------------------------------------- */
/* In-place rotation of dims [D-R, D) of a fp64 row by position pos. */
void orc_rope(double* v, int D, int rope_dims, double rope_base, double pos);

/* ---- Lightning-indexer scores and top-k (one query row) ------------------- */
/* q [H_I, d] and keys [n_vis, d] are already-decoded values (bf16 values, or
 * MXFP4 code x 2^E).  Score I[s] = sum_h w[h] * relu(<q_h, k_s>) with the dot
 * product rounded once to fp32 and the head sum a fp32 fma chain in ascending
 * h.  relu = 0 disables the clamp. */
void orc_index_scores(const float* q, const float* w, const float* keys,
                      int n_vis, int H_I, int d, int relu, float* scores_out);
/* The min(k, n) largest scores (ties: lower index first), written in
 * ascending index order, padded with -1 up to k. */
void orc_topk(const float* scores, int n, int k, int32_t* idx_out);

/* Driver over many query rows (OpenMP): for each listed row q, t = q_pos0+q,
 * n_vis = min(N, (t+1)/m); scores over the visible keys, then top-k.
 * qI [n, H_I, d] decoded, w [n, H_I], kI [N, d] decoded, idx_out [nrows, k]. */
void orc_index_topk_rows(const float* qI, const float* w, const float* kI,
                         int H_I, int d, int N, int m, int64_t q_pos0,
                         const int32_t* rows, int nrows, int k, int relu,
                         int32_t* idx_out);

/* ---- attention (one query row, all heads) -------------------------------- */
/* q [H, D] bf16 pre-RoPE at position t.  Key rows (post-RoPE, fp64) are the
 * union of the chosen compressed entries and the window rows; value = key.
 * sink [H] fp32 logits (NULL = no sink).  out [H, D] fp64, with the inverse
 * rotation by t applied to dims [D-R, D). */
void orc_attend_row(const uint16_t* q, int64_t t, int H, int D,
                    const double* keys, int nk, const float* sink,
                    int rope_dims, double rope_base, double* out);

/* Driver (OpenMP over rows).  Entries are given decoded as fp64 [N, D]
 * (post-RoPE).  mode 0 = CSA: keys = {entries[idx[r][i]] : idx >= 0};
 * mode 1 = HCA: keys = {entries[s] : (s+1)m-1 <= t}.  Window rows
 * j in [max(0, t-n_win+1), t] come from win [win_len, D] bf16 pre-RoPE
 * starting at position win_pos0 and are rotated at j.  q [n, H, D].
 * out [nrows, H, D] fp64.  Returns 0, or -1 if a needed window row is
 * missing from win. */
int orc_attend_rows(const uint16_t* q, int H, int D, int64_t q_pos0,
                    const double* entries, int N, int m,
                    const int32_t* idx, int k, int mode,
                    const uint16_t* win, const double* win_post, int64_t win_pos0, int win_len, int n_win,
                    const float* sink, int rope_dims, double rope_base,
                    const int32_t* rows, int nrows, double* out);


/* ---- array helpers (used by the Python wrapper) --------------------------- */
int orc_set_threads(int n);
void orc_bf16_from_f32_n(const float* x, int64_t n, uint16_t* out);
void orc_bf16_to_f64_n(const uint16_t* b, int64_t n, double* out);
void orc_e4m3_from_f32_n(const float* x, int64_t n, uint8_t* out);
void orc_e4m3_to_f32_n(const uint8_t* c, int64_t n, float* out);
void orc_store_entries_fp8_n(const float* rows, int64_t n, int D, int rope_dims,
                             uint8_t* codes, uint16_t* rope, float* scale);
void orc_load_entries_fp8_n(const uint8_t* codes, const uint16_t* rope, const float* scale,
                            int64_t n, int D, int rope_dims, double* out);
void orc_mxfp4_encode_rows(const float* x, int64_t rows, int n_per_row,
                           uint8_t* codes, uint8_t* scales);
void orc_mxfp4_decode_rows(const uint8_t* codes, const uint8_t* scales, int64_t rows,
                           int n_per_row, float* out);
void orc_store_entry_nvfp4(const float* row, uint8_t* rec_out, float* scale_out);
void orc_store_window_fp8_n(const uint16_t* win, int64_t n, int64_t pos0, int rope_dims,
                            double rope_base, uint8_t* codes, float* scale);
void orc_store_entries_nvfp4_n(const float* rows, int64_t n, uint8_t* recs, float* scale);
void orc_load_entries_nvfp4_n(const uint8_t* recs, const float* scale, int64_t n, double* out);

#ifdef __cplusplus
}
#endif
#endif
