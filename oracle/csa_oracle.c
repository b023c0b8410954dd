/*
 * csa_oracle.c -- plain, slow CPU oracle for the hybrid compressed attention
 * forward.  TEST INFRASTRUCTURE ONLY: it is loaded by the tests, the smoke
 * check and the CPU-baseline leg of the benchmark, never by the library.
 * It shares no code with the HIP path.
 *
 * What it computes follows the pages (titles in csa_oracle.h):
 *  - compression of every m tokens of the KV stream into one entry by a
 *    weighted average, with adjacent blocks overlapping for CSA (m = 4) and
 *    no overlap for HCA (m' = 128)        [V4-wiki, Proposed method, item 1;
 *                                          V4-zh 1.1, CSA bullets]
 *  - a Lightning-Indexer score per (query, entry) in FP4, then top-k per
 *    query token                           [V4-wiki item 1; V4-zh 1.1;
 *                                          EP95, Lightning Indexer segment]
 *  - shared-KV multi-query attention: one compressed entry row is both key
 *    and value                             [V4-zh 1.1, shared-KV MQA bullet]
 *  - a 128-token sliding-window branch, a learnable per-head sink and
 *    partial RoPE on the last 64 dims with inverse RoPE on the attention
 *    output                                [V4-wiki item 1, last three bullets;
 *                                          V4-zh 1.1, auxiliary design]
 *  - KV entries stored with the RoPE dims in BF16 and the rest in FP8
 *                                          [V4-wiki, Training infra, item 5]
 *  - MXFP4 for the indexer QK path         [V4-wiki, Post-training, item 3]
 *
 * The pages print no equations for these steps.  The readings taken where
 * they are silent (overlap geometry, weight form, entry position, indexer
 * formula, one softmax over sink + entries + window, rounding rules) are
 * stated next to each function.
 *
 * Precision: attention is computed in fp64.  Where a float decides an
 * integer (a storage code, a top-k membership) the oracle takes the decision
 * in the precision the GPU kernel uses and in a fixed operation order:
 * pooling weights in fp64 rounded to fp32, pooled values as an fp32 fma
 * chain, indexer dot products rounded once to fp32 and the head sum as an
 * fp32 fma chain in ascending head order.
 */
#include "csa_oracle.h"

#include <fenv.h>
#include <math.h>
#include <omp.h>
#include <stdlib.h>
#include <string.h>

/* ========================================================================== */
/* Number formats                                                             */
/* ========================================================================== */

static uint32_t f32_bits(float x) { uint32_t u; memcpy(&u, &x, 4); return u; }
static float bits_f32(uint32_t u) { float x; memcpy(&x, &u, 4); return x; }

/* bf16 = upper 16 bits of fp32, rounded to nearest, ties to even. */
uint16_t orc_bf16_from_f32(float x)
{
    uint32_t u = f32_bits(x);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu))
        return (uint16_t)((u >> 16) | 0x0040u);           /* quiet NaN */
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7fffu + lsb;
    return (uint16_t)(u >> 16);
}

float orc_bf16_to_f32(uint16_t b) { return bits_f32((uint32_t)b << 16); }

/* OCP FP8 e4m3fn: 1 sign, 4 exponent (bias 7), 3 mantissa bits, no
 * infinities, 0x7f / 0xff are NaN, largest finite 448.  Encoding is round to
 * nearest even on the value grid, saturating at 448; a value that rounds to
 * zero is encoded as +0. */
uint8_t orc_e4m3_from_f32(float x)
{
    if (isnan(x)) return 0x7f;
    double a = fabs((double)x);
    if (a == 0.0) return 0;
    int k;                                   /* binade: a in [2^k, 2^(k+1)) */
    (void)frexp(a, &k);
    k -= 1;
    double step = (k < -6) ? ldexp(1.0, -9) : ldexp(1.0, k - 3);
    double r = nearbyint(a / step);          /* ties to even (default mode) */
    double v = r * step;
    if (v > 448.0) v = 448.0;
    if (v == 0.0) return 0;
    uint8_t code;
    if (v < ldexp(1.0, -6)) {
        code = (uint8_t)(v / ldexp(1.0, -9));             /* subnormal */
    } else {
        int e;
        (void)frexp(v, &e);
        e -= 1;                                          /* v in [2^e, 2^(e+1)) */
        int man = (int)(v / ldexp(1.0, e - 3)) - 8;
        code = (uint8_t)(((e + 7) << 3) | man);
    }
    if (x < 0) code |= 0x80;
    return code;
}

float orc_e4m3_to_f32(uint8_t c)
{
    int s = c >> 7, e = (c >> 3) & 15, man = c & 7;
    if (e == 15 && man == 7) return NAN;
    double v = (e == 0) ? man * ldexp(1.0, -9) : (1.0 + man / 8.0) * ldexp(1.0, e - 7);
    return (float)(s ? -v : v);
}

/* FP4 e2m1: 1 sign, 2 exponent (bias 1), 1 mantissa; magnitudes
 * {0, 0.5, 1, 1.5, 2, 3, 4, 6} for codes 0..7. */
float orc_e2m1_to_f32(uint8_t code)
{
    static const float mag[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};
    float v = mag[code & 7];
    return (code & 8) ? -v : v;
}

/* Round a non-negative value (already divided by the block scale) to the
 * e2m1 magnitude index, nearest with ties to the even index, saturating at 6. */
static int e2m1_round_index(double a)
{
    if (a >= 6.0) return 7;
    if (a < 2.0) return (int)nearbyint(a / 0.5);          /* 0..4 (4 = 2.0) */
    if (a < 4.0) return (int)nearbyint(a) + 2;            /* 4..6 */
    return (int)nearbyint(a / 2.0) + 4;                   /* 6..7 */
}

/* MXFP4 block encoding (OCP Microscaling v1.0 rule for the shared scale):
 * per 32-element block, E = floor(log2(amax)) - emax(e2m1) with emax = 2,
 * scale byte = E + 127 (e8m0), elements RNE(x / 2^E) on the e2m1 grid with
 * saturation at +-6.  An all-zero block gets scale byte 0 and zero codes. */
void orc_mxfp4_encode(const float* x, int n, uint8_t* codes, uint8_t* scales)
{
    memset(codes, 0, (size_t)n / 2);
    for (int b = 0; b < n / 32; ++b) {
        const float* xb = x + 32 * b;
        float amax = 0.0f;
        for (int i = 0; i < 32; ++i) {
            float a = fabsf(xb[i]);
            if (a > amax) amax = a;
        }
        if (amax == 0.0f) { scales[b] = 0; continue; }
        int ex;
        (void)frexpf(amax, &ex);            /* amax = f * 2^ex, f in [0.5, 1) */
        int E = (ex - 1) - 2;
        if (E < -127) E = -127;
        if (E > 127) E = 127;
        scales[b] = (uint8_t)(E + 127);
        for (int i = 0; i < 32; ++i) {
            double v = ldexp((double)xb[i], -E);
            int idx = e2m1_round_index(fabs(v));
            uint8_t c = (uint8_t)idx;
            if (v < 0 && idx != 0) c |= 8;
            int e = 32 * b + i;
            codes[e >> 1] |= (uint8_t)((e & 1) ? (c << 4) : c);
        }
    }
}

void orc_mxfp4_decode(const uint8_t* codes, const uint8_t* scales, int n, float* out)
{
    for (int e = 0; e < n; ++e) {
        uint8_t c = (e & 1) ? (codes[e >> 1] >> 4) : (codes[e >> 1] & 15);
        out[e] = (float)ldexp((double)orc_e2m1_to_f32(c), (int)scales[e / 32] - 127);
    }
}

/* ========================================================================== */
/* RoPE (partial: the last rope_dims dims, adjacent pairs)                    */
/* ========================================================================== */

/* Rotation of pair f = (D-R+2f, D-R+2f+1) by angle pos * base^(-2f/R),
 * angle and products in fp64.  The pages fix only "the last 64 dims"
 * [V4-wiki item 1]; the pairing and base are the usual RoPE convention. */
void orc_rope(double* v, int D, int rope_dims, double rope_base, double pos)
{
    int off = D - rope_dims;
    for (int f = 0; f < rope_dims / 2; ++f) {
        double theta = pow(rope_base, -2.0 * f / rope_dims);
        double phi = pos * theta;
        double c = cos(phi), s = sin(phi);
        double a = v[off + 2 * f], b = v[off + 2 * f + 1];
        v[off + 2 * f] = a * c - b * s;
        v[off + 2 * f + 1] = a * s + b * c;
    }
}

/* ========================================================================== */
/* Compression                                                                */
/* ========================================================================== */

/*
 * Entry i pools the tokens of its own block (role "a": tokens im..im+m-1)
 * and, with overlap, those of the previous block (role "b": tokens
 * (i-1)m..im-1), so adjacent entries share a block [V4-zh 1.1: C^b overlaps
 * C^a; EP95: "two sets are made and combined"].  The weights are a softmax
 * over slot logits beta_r + z_j[role]: a weighted average [V4-wiki item 1].
 * Slots before token 0 are absent (logit -inf).  The entry sits at the
 * position of its last token, p_i = (i+1)m - 1, where RoPE is applied; the
 * indexer-key stream is pooled with the same weights and not rotated.
 * Weights: fp64 softmax (max-subtracted, sum in ascending slot order),
 * each weight rounded to fp32.  Pooling: fp32 fma chain in ascending slot
 * order.  Rotation: fp64, result rounded to fp32.
 */
int orc_compress(const uint16_t* kv, const uint16_t* ik, const float* z, const float* beta,
                 const uint16_t* prev_kv, const uint16_t* prev_ik, const float* prev_z,
                 int T, int64_t pos0, int D, int d_idx, int m, int overlap,
                 int rope_dims, double rope_base,
                 float* entries_out, float* kidx_out)
{
    if (m <= 0 || T < 0 || D <= 0 || pos0 < 0 || pos0 % m != 0) return -1;
    if (rope_dims < 0 || rope_dims > D || (rope_dims & 1)) return -1;
    if (overlap && pos0 > 0 && (prev_kv == NULL || (ik && !prev_ik))) return -1;
    const int L = overlap ? 2 * m : m;
    const int n_new = T / m;
    const int64_t i0 = pos0 / m;
    double* lg = (double*)malloc(sizeof(double) * L);
    float* w = (float*)malloc(sizeof(float) * L);
    double* rot = (double*)malloc(sizeof(double) * D);
    for (int e = 0; e < n_new; ++e) {
        const int64_t i = i0 + e;
        /* slot logits */
        double mx = -INFINITY;
        for (int r = 0; r < L; ++r) {
            int64_t j;
            int role;
            if (overlap) {
                role = (r < m) ? 1 : 0;
                j = (r < m) ? (i - 1) * m + r : i * m + (r - m);
            } else {
                role = 0;
                j = i * m + r;
            }
            if (j < 0) { lg[r] = -INFINITY; continue; }
            double zz = 0.0;
            if (j >= pos0) {
                if (z) zz = z[(j - pos0) * 2 + role];
            } else {
                if (prev_z) zz = prev_z[(j - (pos0 - m)) * 2 + role];
            }
            lg[r] = (double)beta[r] + zz;
            if (lg[r] > mx) mx = lg[r];
        }
        double sum = 0.0;
        for (int r = 0; r < L; ++r) sum += (lg[r] == -INFINITY) ? 0.0 : exp(lg[r] - mx);
        for (int r = 0; r < L; ++r)
            w[r] = (lg[r] == -INFINITY) ? 0.0f : (float)(exp(lg[r] - mx) / sum);
        /* pooling */
        float* c = entries_out + (size_t)e * D;
        float* u = kidx_out ? kidx_out + (size_t)e * d_idx : NULL;
        for (int d = 0; d < D; ++d) c[d] = 0.0f;
        if (u) for (int d = 0; d < d_idx; ++d) u[d] = 0.0f;
        for (int r = 0; r < L; ++r) {
            if (lg[r] == -INFINITY) continue;
            int64_t j = overlap ? ((r < m) ? (i - 1) * m + r : i * m + (r - m)) : i * m + r;
            const uint16_t* x;
            const uint16_t* xi = NULL;
            if (j >= pos0) {
                x = kv + (size_t)(j - pos0) * D;
                if (ik) xi = ik + (size_t)(j - pos0) * d_idx;
            } else {
                x = prev_kv + (size_t)(j - (pos0 - m)) * D;
                if (ik) xi = prev_ik + (size_t)(j - (pos0 - m)) * d_idx;
            }
            for (int d = 0; d < D; ++d) c[d] = fmaf(w[r], orc_bf16_to_f32(x[d]), c[d]);
            if (u && xi)
                for (int d = 0; d < d_idx; ++d) u[d] = fmaf(w[r], orc_bf16_to_f32(xi[d]), u[d]);
        }
        /* RoPE at the entry position */
        if (rope_dims > 0) {
            for (int d = 0; d < D; ++d) rot[d] = c[d];
            orc_rope(rot, D, rope_dims, rope_base, (double)((i + 1) * m - 1));
            for (int d = D - rope_dims; d < D; ++d) c[d] = (float)rot[d];
        }
    }
    free(lg); free(w); free(rot);
    return n_new;
}

/* Mixed-precision entry storage [V4-wiki, Training infra item 5]: the RoPE
 * dims stay BF16, the other dims are FP8 (e4m3fn) with one fp32 scale per
 * row, scale = amax/448 computed in fp32, code = e4m3(x / scale) with an
 * IEEE fp32 division.  An all-zero row stores scale 0 and zero codes. */
void orc_store_entry_fp8(const float* row, int D, int rope_dims,
                         uint8_t* codes_out, uint16_t* rope_out, float* scale_out)
{
    int nq = D - rope_dims;
    float amax = 0.0f;
    for (int d = 0; d < nq; ++d) { float a = fabsf(row[d]); if (a > amax) amax = a; }
    float scale = amax / 448.0f;
    *scale_out = scale;
    for (int d = 0; d < nq; ++d) {
        if (scale == 0.0f) { codes_out[d] = 0; continue; }
        volatile float v = row[d] / scale;
        codes_out[d] = orc_e4m3_from_f32(v);
    }
    for (int d = nq; d < D; ++d) rope_out[d - nq] = orc_bf16_from_f32(row[d]);
}

/* NVFP4 entry storage, the V4.1 cache variant: the pages (the Russian
 * summary of V4.1-Flash) store the compressed KV cache in NVFP4, quantised
 * after RoPE, with the SWA window in FP8.  NVFP4 itself is NVIDIA's format:
 * e2m1 elements in blocks of 16 with an e4m3 block scale, and an fp32
 * second-level scale.  The reading taken for a cache written entry by entry:
 * the second-level scale is per entry, s = amax(entry) / (6 * 448), so the
 * block holding amax gets block scale 448; block j's scale is
 * b_j = e4m3(amax_j / (6 s)) (RNE, saturating); an element is
 * e2m1(x / (e4m3_value(b_j) * s)) (RNE on the e2m1 grid, saturating at 6),
 * 0 where the block scale is 0.  Every step is one fp32 operation, rounded
 * to nearest even, in that order.  Record: 64 bytes of codes (dim 2i in the
 * low nibble of byte i, dim 2i+1 in the high nibble), then the 8 block
 * scales; the fp32 scale is stored apart. */
void orc_store_entry_nvfp4(const float* row, uint8_t* rec_out, float* scale_out)
{
    float amax = 0.0f;
    for (int d = 0; d < 128; ++d) { float a = fabsf(row[d]); if (a > amax) amax = a; }
    volatile float s = amax / 2688.0f;
    *scale_out = s;
    memset(rec_out, 0, 72);
    if (s == 0.0f) return;
    volatile float d6 = 6.0f * s;
    for (int j = 0; j < 8; ++j) {
        float bamax = 0.0f;
        for (int i = 0; i < 16; ++i) { float a = fabsf(row[16 * j + i]); if (a > bamax) bamax = a; }
        volatile float t = bamax / d6;
        uint8_t b = orc_e4m3_from_f32(t);
        rec_out[64 + j] = b;
        volatile float sb = orc_e4m3_to_f32(b) * s;
        if (sb == 0.0f) continue;
        for (int i = 0; i < 16; ++i) {
            int d = 16 * j + i;
            volatile float q = row[d] / sb;
            int idx = e2m1_round_index(fabs((double)q));
            uint8_t c = (uint8_t)idx;
            if (q < 0 && idx != 0) c |= 8;
            rec_out[d >> 1] |= (uint8_t)((d & 1) ? (c << 4) : c);
        }
    }
}

void orc_store_entries_nvfp4_n(const float* rows, int64_t n, uint8_t* recs, float* scale)
{
    for (int64_t i = 0; i < n; ++i) orc_store_entry_nvfp4(rows + i * 128, recs + i * 72, scale + i);
}

/* NVFP4 records -> fp64 rows: e2m1 x e4m3 x s, exact in fp64. */
void orc_load_entries_nvfp4_n(const uint8_t* recs, const float* scale, int64_t n, double* out)
{
    for (int64_t i = 0; i < n; ++i) {
        const uint8_t* r = recs + i * 72;
        for (int d = 0; d < 128; ++d) {
            uint8_t c = (d & 1) ? (r[d >> 1] >> 4) : (r[d >> 1] & 15);
            out[i * 128 + d] = (double)orc_e2m1_to_f32(c) * (double)orc_e4m3_to_f32(r[64 + d / 16]) *
                               (double)scale[i];
        }
    }
}

/* The FP8 sliding-window cache of the V4.1 variant (the Russian summary:
 * the SWA KV cache is held in FP8): each raw window row of position j is
 * rotated at j (fp64, as the entries are), rounded to fp32, and stored as
 * e4m3 codes of all 128 dims with the scale amax / 448 (the FP8 entry rule
 * without bf16 RoPE dims). */
void orc_store_window_fp8_n(const uint16_t* win, int64_t n, int64_t pos0, int rope_dims,
                            double rope_base, uint8_t* codes, float* scale)
{
    double v[128];
    float r[128];
    for (int64_t i = 0; i < n; ++i) {
        for (int d = 0; d < 128; ++d) v[d] = orc_bf16_to_f32(win[i * 128 + d]);
        if (rope_dims > 0) orc_rope(v, 128, rope_dims, rope_base, (double)(pos0 + i));
        for (int d = 0; d < 128; ++d) r[d] = (float)v[d];
        orc_store_entry_fp8(r, 128, 0, codes + i * 128, NULL, scale + i);
    }
}

/* ========================================================================== */
/* Lightning indexer and top-k                                                */
/* ========================================================================== */

/*
 * The pages say the indexer scores compressed entries cheaply with a
 * low-rank factorisation and FP4 arithmetic and is "almost the same" as the
 * DSA indexer [V4-zh 1.1; V4-wiki item 1; EP95].  The reading taken is the
 * DSA form I[t,s] = sum_h w[t,h] * relu(<q[t,h], k[s]>) with one indexer key
 * per entry.  Each dot product is rounded once to fp32 (for FP4 inputs the
 * products and their sum are exact); the head sum is an fp32 fma chain in
 * ascending h starting from +0.  The result is canonicalised so that -0
 * becomes +0.
 */
void orc_index_scores(const float* q, const float* w, const float* keys,
                      int n_vis, int H_I, int d, int relu, float* scores_out)
{
    for (int s = 0; s < n_vis; ++s) {
        const float* k = keys + (size_t)s * d;
        float I = 0.0f;
        for (int h = 0; h < H_I; ++h) {
            double acc = 0.0;
            for (int e = 0; e < d; ++e) acc += (double)q[h * d + e] * (double)k[e];
            float dot = (float)acc;
            float a = relu ? (dot > 0.0f ? dot : 0.0f) : dot;
            I = fmaf(w[h], a, I);
        }
        scores_out[s] = I + 0.0f;
    }
}

typedef struct { float v; int32_t s; } orc_scored;

static int cmp_scored(const void* a, const void* b)
{
    const orc_scored* x = (const orc_scored*)a;
    const orc_scored* y = (const orc_scored*)b;
    if (x->v > y->v) return -1;
    if (x->v < y->v) return 1;
    return (x->s < y->s) ? -1 : (x->s > y->s);
}

static int cmp_i32(const void* a, const void* b)
{
    int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
    return (x > y) - (x < y);
}

/* Each query token attends only to the top-k entries [V4-zh 1.1]; finding
 * them needs every score [EP95].  Reading: a full sort by (score desc,
 * index asc), the first min(k, n) kept, written in ascending index order and
 * padded with -1. */
void orc_topk(const float* scores, int n, int k, int32_t* idx_out)
{
    orc_scored* a = (orc_scored*)malloc(sizeof(orc_scored) * (n > 0 ? n : 1));
    for (int s = 0; s < n; ++s) { a[s].v = scores[s]; a[s].s = s; }
    qsort(a, (size_t)n, sizeof(orc_scored), cmp_scored);
    int kk = n < k ? n : k;
    for (int i = 0; i < kk; ++i) idx_out[i] = a[i].s;
    qsort(idx_out, (size_t)kk, sizeof(int32_t), cmp_i32);
    for (int i = kk; i < k; ++i) idx_out[i] = -1;
    free(a);
}

void orc_index_topk_rows(const float* qI, const float* w, const float* kI,
                         int H_I, int d, int N, int m, int64_t q_pos0,
                         const int32_t* rows, int nrows, int k, int relu,
                         int32_t* idx_out)
{
#pragma omp parallel
    {
        float* sc = (float*)malloc(sizeof(float) * (N > 0 ? N : 1));
#pragma omp for schedule(dynamic, 1)
        for (int r = 0; r < nrows; ++r) {
            int64_t t = q_pos0 + rows[r];
            int64_t nv = (t + 1) / m;
            if (nv > N) nv = N;
            orc_index_scores(qI + (size_t)rows[r] * H_I * d, w + (size_t)rows[r] * H_I,
                             kI, (int)nv, H_I, d, relu, sc);
            orc_topk(sc, (int)nv, k, idx_out + (size_t)r * k);
        }
        free(sc);
    }
}

/* ========================================================================== */
/* Attention                                                                  */
/* ========================================================================== */

/*
 * One softmax per (token, head) over {sink} u {keys}: the sink is a learnable
 * logit with a zero value that lets a head's total attention on real keys be
 * below 1 [V4-wiki item 1; V4-zh 1.1, attention sink].  Keys are
 * shared by every head and the value is the key row itself [V4-zh 1.1,
 * shared-KV MQA].  q is rotated at t, logits are scaled by 1/sqrt(D), and
 * the output's RoPE dims get the inverse rotation by t [V4-wiki item 1].
 */
void orc_attend_row(const uint16_t* q, int64_t t, int H, int D,
                    const double* keys, int nk, const float* sink,
                    int rope_dims, double rope_base, double* out)
{
    double* qq = (double*)malloc(sizeof(double) * D);
    double* lam = (double*)malloc(sizeof(double) * (nk > 0 ? nk : 1));
    const double inv_sqrt_d = 1.0 / sqrt((double)D);
    for (int h = 0; h < H; ++h) {
        for (int d = 0; d < D; ++d) qq[d] = orc_bf16_to_f32(q[(size_t)h * D + d]);
        if (rope_dims > 0) orc_rope(qq, D, rope_dims, rope_base, (double)t);
        double mu = sink ? (double)sink[h] : -INFINITY;
        for (int j = 0; j < nk; ++j) {
            double acc = 0.0;
            const double* kr = keys + (size_t)j * D;
            for (int d = 0; d < D; ++d) acc += qq[d] * kr[d];
            lam[j] = acc * inv_sqrt_d;
            if (lam[j] > mu) mu = lam[j];
        }
        double Z = sink ? exp((double)sink[h] - mu) : 0.0;
        for (int j = 0; j < nk; ++j) Z += exp(lam[j] - mu);
        double* o = out + (size_t)h * D;
        for (int d = 0; d < D; ++d) o[d] = 0.0;
        if (Z > 0.0) {
            for (int j = 0; j < nk; ++j) {
                double p = exp(lam[j] - mu) / Z;
                const double* kr = keys + (size_t)j * D;
                for (int d = 0; d < D; ++d) o[d] += p * kr[d];
            }
        }
        if (rope_dims > 0) orc_rope(o, D, rope_dims, rope_base, -(double)t);
    }
    free(qq); free(lam);
}

/* The sliding-window branch adds the raw tokens t-n_win+1 .. t (rotated at
 * their own positions) to the key set [V4-wiki item 1; V4-zh 1.1].  Reading:
 * one softmax over the concatenation sink + compressed + window, with no
 * de-duplication. */
int orc_attend_rows(const uint16_t* q, int H, int D, int64_t q_pos0,
                    const double* entries, int N, int m,
                    const int32_t* idx, int k, int mode,
                    const uint16_t* win, const double* win_post, int64_t win_pos0, int win_len, int n_win,
                    const float* sink, int rope_dims, double rope_base,
                    const int32_t* rows, int nrows, double* out)
{
    int bad = 0;
    int max_keys = (mode == 0 ? k : N) + (n_win > 0 ? n_win : 0);
#pragma omp parallel reduction(| : bad)
    {
        double* keys = (double*)malloc(sizeof(double) * (size_t)(max_keys > 0 ? max_keys : 1) * D);
#pragma omp for schedule(dynamic, 1)
        for (int r = 0; r < nrows; ++r) {
            int64_t t = q_pos0 + rows[r];
            int nk = 0;
            if (mode == 0) {
                for (int i = 0; i < k; ++i) {
                    int32_t s = idx[(size_t)r * k + i];
                    if (s < 0) continue;
                    memcpy(keys + (size_t)nk * D, entries + (size_t)s * D, sizeof(double) * D);
                    ++nk;
                }
            } else {
                for (int s = 0; s < N; ++s) {
                    if ((int64_t)(s + 1) * m - 1 > t) break;
                    memcpy(keys + (size_t)nk * D, entries + (size_t)s * D, sizeof(double) * D);
                    ++nk;
                }
            }
            if (n_win > 0) {
                int64_t lo = t - n_win + 1;
                if (lo < 0) lo = 0;
                for (int64_t j = lo; j <= t; ++j) {
                    int64_t row = j - win_pos0;
                    if (row < 0 || row >= win_len) { bad = 1; continue; }
                    double* kr = keys + (size_t)nk * D;
                    if (win_post) {  /* stored after RoPE (decoded FP8 window cache) */
                        memcpy(kr, win_post + (size_t)row * D, sizeof(double) * D);
                    } else {
                        for (int d = 0; d < D; ++d) kr[d] = orc_bf16_to_f32(win[(size_t)row * D + d]);
                        if (rope_dims > 0) orc_rope(kr, D, rope_dims, rope_base, (double)j);
                    }
                    ++nk;
                }
            }
            orc_attend_row(q + (size_t)rows[r] * H * D, t, H, D, keys, nk, sink,
                           rope_dims, rope_base, out + (size_t)r * H * D);
        }
        free(keys);
    }
    return bad ? -1 : 0;
}

/* ========================================================================== */
/* Array helpers for the Python wrapper                                       */
/* ========================================================================== */

/* Thread count of the row-parallel loops (top-k rows, attention rows), for
 * timing only: every row is computed by one thread on its own, so results do
 * not depend on it.  Returns the previous count. */
int orc_set_threads(int n)
{
    int prev = omp_get_max_threads();
    if (n > 0) omp_set_num_threads(n);
    return prev;
}

void orc_bf16_from_f32_n(const float* x, int64_t n, uint16_t* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = orc_bf16_from_f32(x[i]);
}

void orc_bf16_to_f64_n(const uint16_t* b, int64_t n, double* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = orc_bf16_to_f32(b[i]);
}

void orc_e4m3_from_f32_n(const float* x, int64_t n, uint8_t* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = orc_e4m3_from_f32(x[i]);
}

void orc_e4m3_to_f32_n(const uint8_t* c, int64_t n, float* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = orc_e4m3_to_f32(c[i]);
}

/* Rows of fp32 entries -> mixed storage (codes [n, D-R], rope bf16 [n, R],
 * scale [n]). */
void orc_store_entries_fp8_n(const float* rows, int64_t n, int D, int rope_dims,
                             uint8_t* codes, uint16_t* rope, float* scale)
{
    for (int64_t i = 0; i < n; ++i)
        orc_store_entry_fp8(rows + i * D, D, rope_dims, codes + i * (D - rope_dims),
                            rope + i * rope_dims, scale + i);
}

/* Mixed storage -> fp64 rows (code x scale for the FP8 dims, exact). */
void orc_load_entries_fp8_n(const uint8_t* codes, const uint16_t* rope, const float* scale,
                            int64_t n, int D, int rope_dims, double* out)
{
    int nq = D - rope_dims;
    for (int64_t i = 0; i < n; ++i) {
        for (int d = 0; d < nq; ++d)
            out[i * D + d] = (double)orc_e4m3_to_f32(codes[i * nq + d]) * (double)scale[i];
        for (int d = 0; d < rope_dims; ++d)
            out[i * D + nq + d] = orc_bf16_to_f32(rope[i * rope_dims + d]);
    }
}

/* MXFP4 over rows of length n_per_row (a multiple of 32). */
void orc_mxfp4_encode_rows(const float* x, int64_t rows, int n_per_row,
                           uint8_t* codes, uint8_t* scales)
{
    for (int64_t r = 0; r < rows; ++r)
        orc_mxfp4_encode(x + r * n_per_row, n_per_row, codes + r * (n_per_row / 2),
                         scales + r * (n_per_row / 32));
}

void orc_mxfp4_decode_rows(const uint8_t* codes, const uint8_t* scales, int64_t rows,
                           int n_per_row, float* out)
{
    for (int64_t r = 0; r < rows; ++r)
        orc_mxfp4_decode(codes + r * (n_per_row / 2), scales + r * (n_per_row / 32),
                         n_per_row, out + r * n_per_row);
}
