// abi.cpp -- the C ABI (include/csa.h): host-side argument validation,
// launch-parameter setup and error reporting.  Nothing is launched unless
// every argument checks out; errors are reported as status codes plus a
// thread-local message.  No allocation, no synchronisation.
#include "../../include/csa.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "kernels.h"

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int ok() {
  g_err.clear();
  return CSA_OK;
}

bool aligned16(const void* p) { return p == nullptr || ((uintptr_t)p & 15u) == 0; }

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(CSA_HIP_ERROR, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

constexpr double kPi = 3.14159265358979323846;

}  // namespace

#define REQUIRE(cond, ...) \
  do {                     \
    if (!(cond)) return fail(CSA_INVALID_ARG, __VA_ARGS__); \
  } while (0)

extern "C" {

const char* csa_last_error(void) { return g_err.c_str(); }

int csa_version(void) { return 100; }

int csa_compress(const void* kv, const void* ik, const float* z, const float* beta,
                 const void* prev_kv, const void* prev_ik, const float* prev_z, int B, int T,
                 int64_t pos0, int D, int d_idx, int m, int overlap, int rope_dims,
                 float rope_base, void* entries_out, void* entries_rope_out,
                 float* entry_scale_out, int entry_fmt, void* kidx_out, uint8_t* kidx_scale_out,
                 int kidx_fmt, void* stream) {
  REQUIRE(B >= 0 && T >= 0, "csa_compress: B=%d and T=%d must be >= 0", B, T);
  REQUIRE(D == 128, "csa_compress: D=%d unsupported (head dim must be 128)", D);
  REQUIRE(m >= 1 && m <= 128, "csa_compress: m=%d must be in [1, 128]", m);
  REQUIRE(overlap == 0 || overlap == 1, "csa_compress: overlap=%d must be 0 or 1", overlap);
  REQUIRE(rope_dims == 0 || rope_dims == 64, "csa_compress: rope_dims=%d must be 0 or 64", rope_dims);
  REQUIRE(rope_dims == 0 || (std::isfinite(rope_base) && rope_base > 1.0f),
          "csa_compress: rope_base must be finite and > 1");
  REQUIRE(pos0 >= 0 && pos0 % m == 0, "csa_compress: pos0=%lld must be a non-negative multiple of m",
          (long long)pos0);
  REQUIRE(beta != nullptr, "csa_compress: beta is NULL");
  const int n_new = T / m;
  if ((int64_t)B * n_new == 0) return ok();
  REQUIRE(kv != nullptr, "csa_compress: kv is NULL");
  REQUIRE(entries_out != nullptr, "csa_compress: entries_out is NULL");
  REQUIRE(entry_fmt == CSA_FMT_BF16 || entry_fmt == CSA_FMT_FP8_ROPE_BF16 || entry_fmt == CSA_FMT_NVFP4,
          "csa_compress: entry_fmt=%d unsupported", entry_fmt);
  if (entry_fmt == CSA_FMT_FP8_ROPE_BF16)
    REQUIRE(entries_rope_out && entry_scale_out,
            "csa_compress: FP8 entries need entries_rope_out and entry_scale_out");
  if (entry_fmt == CSA_FMT_NVFP4)
    REQUIRE(entry_scale_out, "csa_compress: NVFP4 entries need entry_scale_out");
  if (ik) {
    REQUIRE(d_idx == 64, "csa_compress: d_idx=%d unsupported (must be 64)", d_idx);
    if (kidx_out) {
      REQUIRE(kidx_fmt == CSA_FMT_BF16 || kidx_fmt == CSA_FMT_MXFP4,
              "csa_compress: kidx_fmt=%d unsupported", kidx_fmt);
      if (kidx_fmt == CSA_FMT_MXFP4)
        REQUIRE(kidx_scale_out != nullptr, "csa_compress: MXFP4 kidx needs kidx_scale_out");
    }
  }
  const bool need_prev = overlap && pos0 > 0;
  if (need_prev) {
    REQUIRE(prev_kv != nullptr, "csa_compress: prev_kv is required when overlap=1 and pos0>0");
    if (ik) REQUIRE(prev_ik != nullptr, "csa_compress: prev_ik is required when ik is given and pos0>0");
  }
  REQUIRE(((uintptr_t)kv & 3u) == 0 && ((uintptr_t)ik & 3u) == 0 && ((uintptr_t)entries_out & 3u) == 0 &&
              ((uintptr_t)prev_kv & 3u) == 0 && ((uintptr_t)prev_ik & 3u) == 0 &&
              ((uintptr_t)kidx_out & 3u) == 0 && ((uintptr_t)entries_rope_out & 3u) == 0,
          "csa_compress: tensor pointers must be 4-byte aligned");

  csa::CompressParams p{};
  p.kv = (const uint32_t*)kv;
  p.ik = (const uint32_t*)ik;
  p.z = z;
  p.beta = beta;
  p.prev_kv = need_prev ? (const uint32_t*)prev_kv : nullptr;
  p.prev_ik = need_prev ? (const uint32_t*)prev_ik : nullptr;
  p.prev_z = need_prev ? prev_z : nullptr;
  p.B = B;
  p.T = T;
  p.n_new = n_new;
  p.m = m;
  p.L = overlap ? 2 * m : m;
  p.overlap = overlap;
  p.rope_dims = rope_dims;
  p.pos0 = pos0;
  p.entries_out = entries_out;
  p.entries_rope_out = entries_rope_out;
  p.entry_scale_out = entry_scale_out;
  p.entry_fmt = entry_fmt;
  p.kidx_out = ik ? kidx_out : nullptr;
  p.kidx_scale_out = kidx_scale_out;
  p.kidx_fmt = kidx_fmt;
  for (int f = 0; f < 32; ++f) p.theta[f] = std::pow((double)rope_base, -2.0 * f / 64.0);
  return hip_status(csa::launch_compress(p, (hipStream_t)stream), "csa_compress launch");
}

int csa_cache_append(const void* kv_new, const void* ik_new, const float* z_new, int B, int64_t t,
                     void* kv_ring, void* ik_ring, float* z_ring, void* win8_ring, float* win8_scale,
                     int W, const float* beta, int m,
                     int overlap, int rope_dims, float rope_base, void* entries, void* entries_rope,
                     float* entry_scale, int entry_fmt, void* kidx, uint8_t* kidx_scale, int kidx_fmt,
                     int N_cap, void* stream) {
  REQUIRE(B >= 0, "csa_cache_append: B=%d must be >= 0", B);
  REQUIRE(t >= 0, "csa_cache_append: t must be >= 0");
  REQUIRE(m >= 1 && m <= 128, "csa_cache_append: m=%d must be in [1, 128]", m);
  REQUIRE(overlap == 0 || overlap == 1, "csa_cache_append: overlap=%d must be 0 or 1", overlap);
  const int L = overlap ? 2 * m : m;
  REQUIRE(W >= L && W <= 4096, "csa_cache_append: W=%d must be in [%d, 4096] (the pooled rows must be in the ring)",
          W, L);
  REQUIRE(rope_dims == 0 || rope_dims == 64, "csa_cache_append: rope_dims=%d must be 0 or 64", rope_dims);
  REQUIRE(rope_dims == 0 || (std::isfinite(rope_base) && rope_base > 1.0f),
          "csa_cache_append: rope_base must be finite and > 1");
  REQUIRE(N_cap >= 0, "csa_cache_append: N_cap=%d must be >= 0", N_cap);
  if (B == 0) return ok();
  REQUIRE(kv_new && kv_ring && beta, "csa_cache_append: kv_new, kv_ring and beta must be non-NULL");
  REQUIRE((ik_new == nullptr) == (ik_ring == nullptr), "csa_cache_append: ik_new and ik_ring go together");
  REQUIRE((z_new == nullptr) == (z_ring == nullptr), "csa_cache_append: z_new and z_ring go together");
  REQUIRE((win8_ring == nullptr) == (win8_scale == nullptr), "csa_cache_append: win8_ring and win8_scale go together");
  const bool complete = (t + 1) % m == 0;
  if (complete) {
    const int64_t i = (t + 1) / m - 1;
    REQUIRE(i < N_cap, "csa_cache_append: entry %lld does not fit the caches (N_cap=%d)", (long long)i, N_cap);
    REQUIRE(entries != nullptr, "csa_cache_append: entries is NULL");
    REQUIRE(entry_fmt == CSA_FMT_BF16 || entry_fmt == CSA_FMT_FP8_ROPE_BF16 || entry_fmt == CSA_FMT_NVFP4,
            "csa_cache_append: entry_fmt=%d unsupported", entry_fmt);
    if (entry_fmt == CSA_FMT_FP8_ROPE_BF16)
      REQUIRE(entries_rope && entry_scale, "csa_cache_append: FP8 entries need entries_rope and entry_scale");
    if (entry_fmt == CSA_FMT_NVFP4)
      REQUIRE(entry_scale, "csa_cache_append: NVFP4 entries need entry_scale");
    if (ik_new) {
      REQUIRE(kidx != nullptr, "csa_cache_append: kidx is NULL");
      REQUIRE(kidx_fmt == CSA_FMT_BF16 || kidx_fmt == CSA_FMT_MXFP4, "csa_cache_append: kidx_fmt=%d unsupported",
              kidx_fmt);
      if (kidx_fmt == CSA_FMT_MXFP4) REQUIRE(kidx_scale != nullptr, "csa_cache_append: MXFP4 kidx needs kidx_scale");
    }
  }
  REQUIRE(((uintptr_t)kv_new & 3u) == 0 && ((uintptr_t)ik_new & 3u) == 0 && ((uintptr_t)kv_ring & 3u) == 0 &&
              ((uintptr_t)ik_ring & 3u) == 0 && ((uintptr_t)entries & 3u) == 0 &&
              ((uintptr_t)entries_rope & 3u) == 0 && ((uintptr_t)kidx & 3u) == 0 &&
              ((uintptr_t)win8_ring & 3u) == 0,
          "csa_cache_append: tensor pointers must be 4-byte aligned");

  csa::CompressParams p{};
  p.append = 1;
  p.kv_new = (const uint32_t*)kv_new;
  p.ik_new = (const uint32_t*)ik_new;
  p.z_new = z_new;
  p.kv_ring = (uint32_t*)kv_ring;
  p.ik_ring = (uint32_t*)ik_ring;
  p.z_ring = z_ring;
  p.win8_ring = (uint8_t*)win8_ring;
  p.win8_scale = win8_scale;
  p.W = W;
  p.N_cap = N_cap;
  p.t = t;
  p.beta = beta;
  p.B = B;
  p.m = m;
  p.L = L;
  p.overlap = overlap;
  p.rope_dims = rope_dims;
  p.entries_out = entries;
  p.entries_rope_out = entries_rope;
  p.entry_scale_out = entry_scale;
  p.entry_fmt = entry_fmt;
  p.kidx_out = ik_new ? kidx : nullptr;
  p.kidx_scale_out = kidx_scale;
  p.kidx_fmt = kidx_fmt;
  for (int f = 0; f < 32; ++f) p.theta[f] = std::pow((double)rope_base, -2.0 * f / 64.0);
  return hip_status(csa::launch_compress(p, (hipStream_t)stream), "csa_cache_append launch");
}

size_t csa_index_topk_workspace_bytes(int B, int n, int64_t q_pos0, int N, int m, int k) {
  return csa::index_topk_workspace(B, n, q_pos0, N, m, k);
}

static int index_common(const void* qidx, const uint8_t* qidx_scale, const float* widx, const void* kidx,
                        const uint8_t* kidx_scale, int fmt, int B, int n, int64_t q_pos0, int H_I, int d_idx, int N,
                        int m, int k, int32_t* idx_out, void* ws, size_t ws_bytes, bool static_ws,
                        uint32_t* fallback_count, void* stream, const char* name, bool launch = true) {
  REQUIRE(B >= 0 && n >= 0 && N >= 0, "%s: B=%d n=%d N=%d must be >= 0", name, B, n, N);
  REQUIRE(fmt == CSA_FMT_BF16 || fmt == CSA_FMT_MXFP4, "%s: fmt=%d unsupported", name, fmt);
  REQUIRE(d_idx == 64, "%s: d_idx=%d unsupported (must be 64)", name, d_idx);
  REQUIRE(H_I >= 1 && H_I <= 8, "%s: H_I=%d must be in [1, 8]", name, H_I);
  REQUIRE(k >= 1 && k <= 2048, "%s: k=%d must be in [1, 2048]", name, k);
  REQUIRE(m >= 1, "%s: m=%d must be >= 1", name, m);
  REQUIRE(q_pos0 >= 0, "%s: q_pos0 must be >= 0", name);
  if ((int64_t)B * n == 0) return ok();
  REQUIRE(qidx && widx && idx_out, "%s: qidx, widx and idx_out must be non-NULL", name);
  REQUIRE(N == 0 || kidx != nullptr, "%s: kidx is NULL", name);
  if (fmt == CSA_FMT_MXFP4) REQUIRE(N == 0 || kidx_scale != nullptr, "%s: MXFP4 needs kidx_scale", name);
  REQUIRE(aligned16(qidx) && aligned16(kidx), "%s: qidx and kidx must be 16-byte aligned", name);
  REQUIRE(((uintptr_t)fallback_count & 3u) == 0, "%s: fallback_count must be 4-byte aligned", name);
  const size_t need = csa::index_topk_workspace(B, n, q_pos0, N, m, k);
  if (static_ws) {
    if (need > csa::kStaticScratchBytes)
      return fail(CSA_WORKSPACE_TOO_SMALL,
                  "%s: the call needs %zu bytes of scratch; the static scratch holds %zu (%zu rows of the split "
                  "path); use csa_index_topk with a workspace",
                  name, need, csa::kStaticScratchBytes, csa::kStaticScratchBytes / csa::kSplitRowBytes);
    ws_bytes = csa::kStaticScratchBytes;
    ws = nullptr;
    if (need > 0) {
      const int st = hip_status(csa::static_scratch(&ws), "csa_index_topk_noalloc (scratch address)");
      if (st != CSA_OK) return st;
    }
  } else {
    if (ws_bytes < need)
      return fail(CSA_WORKSPACE_TOO_SMALL, "%s: workspace of %zu bytes < %zu needed", name, ws_bytes, need);
    REQUIRE(need == 0 || (ws != nullptr && aligned16(ws)), "%s: ws must be non-NULL and 16-byte aligned", name);
  }
  if (!launch) return ok();
  csa::IndexParams p{};
  p.q = qidx;
  p.q_scale = (fmt == CSA_FMT_MXFP4) ? qidx_scale : nullptr;
  p.w = widx;
  p.kidx = kidx;
  p.kidx_scale = kidx_scale;
  p.fmt = fmt;
  p.B = B;
  p.n = n;
  p.H_I = H_I;
  p.N = N;
  p.m = m;
  p.k = k;
  p.q_pos0 = q_pos0;
  p.idx_out = idx_out;
  p.ws = ws;
  p.ws_bytes = ws_bytes;
  p.fallback_count = fallback_count;
  return hip_status(csa::launch_index_topk(p, (hipStream_t)stream), name);
}

int csa_index_topk(const void* qidx, const uint8_t* qidx_scale, const float* widx,
                   const void* kidx, const uint8_t* kidx_scale, int fmt, int B, int n,
                   int64_t q_pos0, int H_I, int d_idx, int N, int m, int k, int32_t* idx_out,
                   void* ws, size_t ws_bytes, uint32_t* fallback_count, void* stream) {
  return index_common(qidx, qidx_scale, widx, kidx, kidx_scale, fmt, B, n, q_pos0, H_I, d_idx, N, m, k, idx_out, ws,
                      ws_bytes, false, fallback_count, stream, "csa_index_topk");
}

int csa_index_topk_noalloc(const void* qidx, const uint8_t* qidx_scale, const float* widx,
                           const void* kidx, const uint8_t* kidx_scale, int fmt, int B, int n,
                           int64_t q_pos0, int H_I, int d_idx, int N, int m, int k, int32_t* idx_out,
                           uint32_t* fallback_count, void* stream) {
  return index_common(qidx, qidx_scale, widx, kidx, kidx_scale, fmt, B, n, q_pos0, H_I, d_idx, N, m, k, idx_out,
                      nullptr, 0, true, fallback_count, stream, "csa_index_topk_noalloc");
}

static int attend_common(int mode, const void* q, int B, int n, int64_t q_pos0, int H, int D,
                         const void* entries, const void* entries_rope, const float* entry_scale,
                         int N, int m, const int32_t* idx, int k, const void* win_kv,
                         int64_t win_pos0, int win_len, int n_win, int win_fmt, const float* win_scale,
                         const float* sink,
                         int rope_dims, float rope_base, void* out, void* ws, size_t ws_bytes,
                         void* stream, const char* name, bool launch = true) {
  REQUIRE(B >= 0 && n >= 0 && N >= 0 && k >= 0, "%s: B, n, N and k must be >= 0", name);
  REQUIRE(D == 128, "%s: D=%d unsupported (head dim must be 128)", name, D);
  REQUIRE(H >= 1 && H <= 64, "%s: H=%d must be in [1, 64]", name, H);
  REQUIRE(m >= 1, "%s: m=%d must be >= 1", name, m);
  REQUIRE(q_pos0 >= 0, "%s: q_pos0 must be >= 0", name);
  REQUIRE(rope_dims == 0 || rope_dims == 64, "%s: rope_dims=%d must be 0 or 64", name, rope_dims);
  REQUIRE(rope_dims == 0 || (std::isfinite(rope_base) && rope_base > 1.0f),
          "%s: rope_base must be finite and > 1", name);
  REQUIRE(n_win >= 0 && n_win <= 128, "%s: n_win=%d must be in [0, 128]", name, n_win);
  REQUIRE(win_fmt == CSA_FMT_BF16 || win_fmt == CSA_FMT_FP8 || win_fmt == CSA_FMT_BF16_ROPED,
          "%s: win_fmt=%d unsupported", name, win_fmt);
  REQUIRE(win_fmt != CSA_FMT_BF16_ROPED || rope_dims == 64,
          "%s: a pre-rotated window (CSA_FMT_BF16_ROPED) needs rope_dims = 64", name);
  REQUIRE(win_fmt != CSA_FMT_FP8 || mode == 1 || mode == 3,
          "%s: an FP8 window needs FP8 or NVFP4 entries (the decode cache layout)", name);
  // row sources are addressed with 32-bit byte offsets inside the kernel
  REQUIRE((int64_t)N * 256 < 0x7fff0000LL && (int64_t)win_len * 256 < 0x7fff0000LL,
          "%s: N=%d or win_len=%d too large (at most 8388351 rows)", name, N, win_len);
  if ((int64_t)B * n == 0) return ok();
  REQUIRE(q != nullptr && out != nullptr, "%s: q and out must be non-NULL", name);
  REQUIRE(N == 0 || entries != nullptr, "%s: entries is NULL", name);
  if (mode == 0 || mode == 1 || mode == 3) {
    REQUIRE(k <= 2048, "%s: k=%d must be <= 2048", name, k);
    REQUIRE(k == 0 || idx != nullptr, "%s: idx is NULL", name);
    REQUIRE(aligned16(idx), "%s: idx must be 16-byte aligned", name);
  }
  if (mode == 1) REQUIRE(N == 0 || (entries_rope && entry_scale), "%s: FP8 entries need entries_rope and entry_scale", name);
  if (mode == 3) REQUIRE(N == 0 || entry_scale, "%s: NVFP4 entries need entry_scale", name);
  if (n_win > 0) {
    REQUIRE(win_kv != nullptr, "%s: win_kv is NULL but n_win > 0", name);
    REQUIRE(win_fmt != CSA_FMT_FP8 || win_scale != nullptr, "%s: an FP8 window needs win_scale", name);
    int64_t lo = q_pos0 - n_win + 1;
    if (lo < 0) lo = 0;
    const int64_t hi = q_pos0 + n - 1;
    REQUIRE(win_len >= 0 && win_pos0 <= lo && win_pos0 + win_len - 1 >= hi,
            "%s: window source [%lld, %lld) does not cover positions [%lld, %lld]", name,
            (long long)win_pos0, (long long)(win_pos0 + win_len), (long long)lo, (long long)hi);
  }
  REQUIRE(aligned16(q) && aligned16(entries) && aligned16(entries_rope) && aligned16(win_kv) &&
              aligned16(out),
          "%s: q, entries, entries_rope, win_kv and out must be 16-byte aligned", name);
  const size_t need = csa::attend_workspace(mode, B, n, k, n_win);
  if (ws_bytes < need)
    return fail(CSA_WORKSPACE_TOO_SMALL, "%s: workspace of %zu bytes < %zu needed", name, ws_bytes, need);
  REQUIRE(need == 0 || (ws != nullptr && aligned16(ws)), "%s: ws must be non-NULL and 16-byte aligned", name);
  if (!launch) return ok();
  csa::AttendParams p{};
  p.q = (const uint16_t*)q;
  p.B = B;
  p.n = n;
  p.H = H;
  p.q_pos0 = q_pos0;
  p.entries = (const uint16_t*)entries;
  p.entries_rope = (const uint16_t*)entries_rope;
  p.entry_scale = entry_scale;
  p.N = N;
  p.m = m;
  p.idx = idx;
  p.k = (mode == 2) ? 0 : k;
  p.win = (const uint16_t*)win_kv;
  p.win_fp8 = win_fmt == CSA_FMT_FP8 ? 1 : 0;
  p.win_roped = win_fmt == CSA_FMT_BF16_ROPED ? 1 : 0;
  p.win_scale = win_scale;
  p.win_pos0 = win_pos0;
  p.win_len = win_len;
  p.n_win = n_win;
  p.sink = sink;
  p.rope = rope_dims == 64 ? 1 : 0;
  p.qscale = (float)(1.4426950408889634 / std::sqrt(128.0));
  p.out = (uint16_t*)out;
  p.ws = need > 0 ? (float*)ws : nullptr;
  for (int f = 0; f < 32; ++f) p.rev[f] = std::pow((double)rope_base, -2.0 * f / 64.0) / (2.0 * kPi);
  return hip_status(csa::launch_attend(p, mode == 2 ? 2 : mode, (hipStream_t)stream), name);
}

int csa_attend(const void* q, int B, int n, int64_t q_pos0, int H, int D, const void* entries,
               const void* entries_rope, const float* entry_scale, int entry_fmt, int N, int m,
               const int32_t* idx, int k, const void* win_kv, int64_t win_pos0, int win_len,
               int n_win, int win_fmt, const float* win_scale, const float* sink, int rope_dims,
               float rope_base, void* out, void* ws, size_t ws_bytes, void* stream) {
  REQUIRE(entry_fmt == CSA_FMT_BF16 || entry_fmt == CSA_FMT_FP8_ROPE_BF16 || entry_fmt == CSA_FMT_NVFP4,
          "csa_attend: entry_fmt=%d unsupported", entry_fmt);
  const int mode = entry_fmt == CSA_FMT_BF16 ? 0 : entry_fmt == CSA_FMT_FP8_ROPE_BF16 ? 1 : 3;
  return attend_common(mode, q, B, n, q_pos0, H, D, entries,
                       entries_rope, entry_scale, N, m, idx, k, win_kv, win_pos0, win_len, n_win,
                       win_fmt, win_scale, sink, rope_dims, rope_base, out, ws, ws_bytes, stream, "csa_attend");
}

size_t csa_attend_workspace_bytes(int B, int n, int k, int n_win, int entry_fmt) {
  if (B < 0 || n < 0 || k < 0 || n_win < 0) return 0;
  return csa::attend_workspace(entry_fmt == CSA_FMT_FP8_ROPE_BF16 ? 1 : entry_fmt == CSA_FMT_NVFP4 ? 3 : 0, B, n,
                               k, n_win);
}

int csa_index_attend(const void* qidx, const uint8_t* qidx_scale, const float* widx, const void* kidx,
                     const uint8_t* kidx_scale, int kidx_fmt, int H_I, int d_idx, int k, int32_t* idx_out,
                     uint32_t* fallback_count, const void* q, int H, int D, const void* entries,
                     const void* entries_rope, const float* entry_scale, int entry_fmt, const void* win_kv,
                     int64_t win_pos0, int win_len, int n_win, int win_fmt, const float* win_scale,
                     const float* sink, int rope_dims, float rope_base, void* out, int B, int n, int64_t q_pos0,
                     int N, int m, int n_chunks, void* stream, void* aux_stream, void* const* events) {
  static const char* name = "csa_index_attend";
  REQUIRE(entry_fmt == CSA_FMT_BF16 || entry_fmt == CSA_FMT_FP8_ROPE_BF16 || entry_fmt == CSA_FMT_NVFP4,
          "%s: entry_fmt=%d unsupported", name, entry_fmt);
  REQUIRE(n_chunks >= 1, "%s: n_chunks=%d must be >= 1", name, n_chunks);
  const int mode = entry_fmt == CSA_FMT_BF16 ? 0 : entry_fmt == CSA_FMT_FP8_ROPE_BF16 ? 1 : 3;
  // chunks of at least kMinChunk tokens of the one batch row
  constexpr int kMinChunk = 512;
  int C = n_chunks;
  if (B != 1 || (int64_t)C * kMinChunk > n) C = B == 1 ? (n / kMinChunk > 1 ? n / kMinChunk : 1) : 1;
  if (C > 1) {
    REQUIRE(aux_stream != nullptr && aux_stream != stream, "%s: n_chunks > 1 needs an aux_stream other than stream",
            name);
    REQUIRE(events && events[0] && events[1] && events[2], "%s: n_chunks > 1 needs three events", name);
    REQUIRE(events[0] != events[1] && events[0] != events[2] && events[1] != events[2],
            "%s: the three events must be distinct", name);
  }
  // the whole call is checked before anything is enqueued (no workspace:
  // the formats and sizes that need one are refused here)
  int st = index_common(qidx, qidx_scale, widx, kidx, kidx_scale, kidx_fmt, B, n, q_pos0, H_I, d_idx, N, m, k,
                        idx_out, nullptr, 0, false, fallback_count, stream, name, false);
  if (st != CSA_OK) return st;
  st = attend_common(mode, q, B, n, q_pos0, H, D, entries, entries_rope, entry_scale, N, m, idx_out, k, win_kv,
                     win_pos0, win_len, n_win, win_fmt, win_scale, sink, rope_dims, rope_base, out, nullptr, 0,
                     stream, name, false);
  if (st != CSA_OK) return st;
  if ((int64_t)B * n == 0) return ok();
  // per-token byte strides of the token-major arrays (B = 1 when chunked)
  const bool qcodes = kidx_fmt == CSA_FMT_MXFP4 && qidx_scale != nullptr;
  const int64_t s_qidx = (int64_t)H_I * (qcodes ? 32 : 128), s_qsc = (int64_t)H_I * 2;
  const int64_t s_w = H_I, s_idx = k, s_q = (int64_t)H * 256;
  auto index_chunk = [&](int64_t a, int nc, void* strm) {
    return index_common((const uint8_t*)qidx + a * s_qidx, qidx_scale ? qidx_scale + a * s_qsc : nullptr,
                        widx + a * s_w, kidx, kidx_scale, kidx_fmt, B, nc, q_pos0 + a, H_I, d_idx, N, m, k,
                        idx_out + a * s_idx, nullptr, 0, false, fallback_count, strm, name);
  };
  auto attend_chunk = [&](int64_t a, int nc) {
    return attend_common(mode, (const uint8_t*)q + a * s_q, B, nc, q_pos0 + a, H, D, entries, entries_rope,
                         entry_scale, N, m, idx_out + a * s_idx, k, win_kv, win_pos0, win_len, n_win, win_fmt,
                         win_scale, sink, rope_dims, rope_base, (uint8_t*)out + a * s_q, nullptr, 0, stream, name);
  };
  if (C == 1) {
    st = index_chunk(0, n, stream);
    return st != CSA_OK ? st : attend_chunk(0, n);
  }
  hipStream_t sm = (hipStream_t)stream, sx = (hipStream_t)aux_stream;
  hipEvent_t ev0 = (hipEvent_t)events[0], ring[2] = {(hipEvent_t)events[1], (hipEvent_t)events[2]};
  // the aux stream starts after everything already enqueued on stream
  st = hip_status(hipEventRecord(ev0, sm), "csa_index_attend: event record");
  if (st == CSA_OK) st = hip_status(hipStreamWaitEvent(sx, ev0, 0), "csa_index_attend: stream wait");
  auto lo = [&](int c) { return (int64_t)n * c / C; };
  bool aux_used = false;
  for (int c = 0; c <= C && st == CSA_OK; ++c) {
    if (c < C) {  // top-k of chunk c on the aux stream
      aux_used = true;
      st = index_chunk(lo(c), (int)(lo(c + 1) - lo(c)), sx);
      if (st == CSA_OK) st = hip_status(hipEventRecord(ring[c & 1], sx), "csa_index_attend: event record");
    }
    if (c >= 1 && st == CSA_OK) {  // attention of chunk c - 1 once its top-k is written
      // (ring[(c-1) & 1] was last recorded for chunk c - 1: a wait takes the
      // event's latest record at the time of the call)
      st = hip_status(hipStreamWaitEvent(sm, ring[(c - 1) & 1], 0), "csa_index_attend: stream wait");
      if (st == CSA_OK) st = attend_chunk(lo(c - 1), (int)(lo(c) - lo(c - 1)));
    }
  }
  if (st != CSA_OK && aux_used) {
    // best effort: order what the aux stream already holds before later work
    // on the caller's stream (the error message is the first failure's)
    if (hipEventRecord(ev0, sx) == hipSuccess) (void)hipStreamWaitEvent(sm, ev0, 0);
  }
  return st;
}

int hca_attend(const void* q, int B, int n, int64_t q_pos0, int H, int D, const void* entries,
               int N, int m, const void* win_kv, int64_t win_pos0, int win_len, int n_win, int win_fmt,
               const float* sink, int rope_dims, float rope_base, void* out, void* stream) {
  REQUIRE(win_fmt == CSA_FMT_BF16 || win_fmt == CSA_FMT_BF16_ROPED, "hca_attend: win_fmt=%d unsupported",
          win_fmt);
  return attend_common(2, q, B, n, q_pos0, H, D, entries, nullptr, nullptr, N, m, nullptr, 0,
                       win_kv, win_pos0, win_len, n_win, win_fmt, nullptr, sink, rope_dims, rope_base,
                       out, nullptr, 0, stream, "hca_attend");
}

int csa_rope_rows(const void* kv, int B, int T, int64_t pos0, int rope_dims, float rope_base, void* out,
                  void* stream) {
  REQUIRE(B >= 0 && T >= 0, "csa_rope_rows: B=%d and T=%d must be >= 0", B, T);
  REQUIRE(rope_dims == 64, "csa_rope_rows: rope_dims=%d must be 64", rope_dims);
  REQUIRE(std::isfinite(rope_base) && rope_base > 1.0f, "csa_rope_rows: rope_base must be finite and > 1");
  REQUIRE(pos0 >= 0, "csa_rope_rows: pos0 must be >= 0");
  if ((int64_t)B * T == 0) return ok();
  REQUIRE(kv && out, "csa_rope_rows: kv and out must be non-NULL");
  REQUIRE(((uintptr_t)kv & 3u) == 0 && ((uintptr_t)out & 3u) == 0, "csa_rope_rows: kv and out must be 4-byte aligned");
  csa::RopeRowsParams p{};
  p.kv = (const uint32_t*)kv;
  p.out = (uint32_t*)out;
  p.rows = (int64_t)B * T;
  p.T = T;
  p.pos0 = pos0;
  for (int f = 0; f < 32; ++f) p.theta[f] = std::pow((double)rope_base, -2.0 * f / 64.0);
  return hip_status(csa::launch_rope_rows(p, (hipStream_t)stream), "csa_rope_rows");
}

// ---------------------------------------------------------------- projections

namespace {

int qidx_check(const void* lat, int ld_lat, int r, const void* w_up, int n_qidx, const uint8_t* codes,
               const uint8_t* scales, const float* q_f32, const char* who) {
  REQUIRE(r == 16 || r == 32 || r == 64, "%s: rank r=%d must be 16, 32 or 64", who, r);
  REQUIRE(n_qidx > 0 && n_qidx % 32 == 0 && n_qidx <= (1 << 20),
          "%s: n_qidx=%d must be a positive multiple of 32, at most 2^20", who, n_qidx);
  REQUIRE(w_up && codes && scales, "%s: w_up, codes and scales must be non-NULL", who);
  REQUIRE(aligned16(w_up) && aligned16(codes) && aligned16(q_f32),
          "%s: w_up, codes and q_f32 must be 16-byte aligned", who);
  REQUIRE(lat != nullptr && aligned16(lat) && ld_lat % 8 == 0,
          "%s: the latent must be non-NULL with 16-byte aligned rows", who);
  return CSA_OK;
}

int qidx_launch(const void* lat, int ld_lat, int M, int r, const void* w_up, int n_qidx, uint8_t* codes,
                uint8_t* scales, float* q_f32, void* stream, const char* who) {
  csa::QidxParams q{};
  q.lat = (const uint16_t*)lat;
  q.w_up = (const uint16_t*)w_up;
  q.M = M;
  q.r = r;
  q.nq = n_qidx;
  q.ld_lat = ld_lat;
  q.codes = codes;
  q.scales = scales;
  q.q_f32 = q_f32;
  return hip_status(csa::launch_qidx_mxfp4(q, (hipStream_t)stream), who);
}

}  // namespace

int csa_project_qidx(const void* lat, int M, int r, const void* w_up, int n_qidx, uint8_t* qidx_out,
                     uint8_t* qidx_scale_out, float* q_f32_out, void* stream) {
  REQUIRE(M >= 0, "csa_project_qidx: M=%d must be >= 0", M);
  if (qidx_check(lat, r, r, w_up, n_qidx, qidx_out, qidx_scale_out, q_f32_out, "csa_project_qidx") != CSA_OK)
    return CSA_INVALID_ARG;
  if (M == 0) return ok();
  return qidx_launch(lat, r, M, r, w_up, n_qidx, qidx_out, qidx_scale_out, q_f32_out, stream, "csa_project_qidx");
}

int csa_project_in(const void* x, int M, int d, const void* w_in, int n_q, int n_kv, int n_ik, int n_lat,
                   int n_w, int n_z, const void* w_up, int n_qidx, void* q_out, void* kv_out, void* ik_out,
                   void* lat_out, float* w_out, float* z_out, uint8_t* qidx_out, uint8_t* qidx_scale_out,
                   void* stream) {
  REQUIRE(M >= 0, "csa_project_in: M=%d must be >= 0", M);
  REQUIRE(d > 0 && d % 32 == 0, "csa_project_in: d=%d must be a positive multiple of 32", d);
  REQUIRE(n_q >= 0 && n_kv >= 0 && n_ik >= 0 && n_lat >= 0 && n_w >= 0 && n_z >= 0,
          "csa_project_in: output widths must be >= 0");
  const int64_t N64 = (int64_t)n_q + n_kv + n_ik + n_lat + n_w + n_z;
  REQUIRE(N64 < (1 << 24), "csa_project_in: total output width %lld too large", (long long)N64);
  const int N = (int)N64;
  REQUIRE(N > 0, "csa_project_in: no output");
  REQUIRE(n_qidx >= 0, "csa_project_in: n_qidx=%d must be >= 0", n_qidx);
  REQUIRE(x && w_in, "csa_project_in: x and w_in must be non-NULL");
  REQUIRE(aligned16(x) && aligned16(w_in), "csa_project_in: x and w_in must be 16-byte aligned");
  REQUIRE((int64_t)M * d * 2 < (1ll << 31) && (int64_t)N * d * 2 < (1ll << 31),
          "csa_project_in: x and w_in must each be below 2 GiB");
  const int widths[6] = {n_q, n_kv, n_ik, n_lat, n_w, n_z};
  void* ptrs[6] = {q_out, kv_out, ik_out, lat_out, w_out, z_out};
  const char* names[6] = {"q_out", "kv_out", "ik_out", "lat_out", "w_out", "z_out"};
  static_assert(csa::kGemmOuts >= 6, "one GEMM output per projection");
  csa::GemmParams g{};
  int c0 = 0;
  for (int i = 0; i < 6; ++i) {
    if (widths[i] == 0) continue;
    REQUIRE(ptrs[i] != nullptr, "csa_project_in: %s is NULL but its width is %d", names[i], widths[i]);
    csa::GemmOut& o = g.out[g.nout++];
    o.ptr = ptrs[i];
    o.n0 = c0;
    o.n1 = c0 + widths[i];
    o.ld = widths[i];
    o.f32 = i >= 4;
    c0 += widths[i];
  }
  if (n_qidx > 0) {
    REQUIRE(n_lat > 0, "csa_project_in: the indexer query needs the latent (n_lat > 0)");
    if (qidx_check(lat_out, n_lat, n_lat, w_up, n_qidx, qidx_out, qidx_scale_out, nullptr,
                   "csa_project_in (indexer query)") != CSA_OK)
      return CSA_INVALID_ARG;
  }
  if (M == 0) return ok();
  g.A = (const uint16_t*)x;
  g.B = (const uint16_t*)w_in;
  g.M = M;
  g.N = N;
  g.K = d;
  g.lda = d;
  g.ldb = d;
  g.a_bytes = (uint32_t)((int64_t)M * d * 2);
  g.b_bytes = (uint32_t)((int64_t)N * d * 2);
  int st = hip_status(csa::launch_gemm_tn(g, 1, (hipStream_t)stream), "csa_project_in (GEMM)");
  if (st != CSA_OK || n_qidx == 0) return st;
  return qidx_launch(lat_out, n_lat, M, n_lat, w_up, n_qidx, qidx_out, qidx_scale_out, nullptr, stream,
                     "csa_project_in (indexer query)");
}

int csa_project_out(const void* o, int M, int H, int D, int G, const void* w_o, int d, void* y_out,
                    void* stream) {
  REQUIRE(M >= 0, "csa_project_out: M=%d must be >= 0", M);
  REQUIRE(H > 0 && D > 0 && G > 0 && H % G == 0, "csa_project_out: H=%d must be a positive multiple of G=%d", H, G);
  const int KG = H / G * D;
  REQUIRE(KG % 32 == 0, "csa_project_out: (H/G)*D=%d must be a multiple of 32", KG);
  REQUIRE(d > 0 && d % G == 0, "csa_project_out: d=%d must be a positive multiple of G=%d", d, G);
  REQUIRE(o && w_o && y_out, "csa_project_out: o, w_o and y_out must be non-NULL");
  REQUIRE(aligned16(o) && aligned16(w_o), "csa_project_out: o and w_o must be 16-byte aligned");
  REQUIRE((int64_t)M * H * D * 2 < (1ll << 32) - 4096, "csa_project_out: o must be below 4 GiB");
  if (M == 0) return ok();
  const int dg = d / G;
  csa::GemmParams g{};
  g.A = (const uint16_t*)o;
  g.B = (const uint16_t*)w_o;
  g.M = M;
  g.N = dg;
  g.K = KG;
  g.lda = H * D;
  g.ldb = KG;
  g.a_zoff = KG;
  g.b_zoff = (int64_t)dg * KG;
  g.a_bytes = (uint32_t)((int64_t)M * H * D * 2);
  g.a_zbytes = (uint32_t)KG * 2u;
  g.b_bytes = (uint32_t)((int64_t)dg * KG * 2);
  g.c_zcol = dg;
  g.nout = 1;
  g.out[0] = csa::GemmOut{y_out, 0, d, d, 0};
  return hip_status(csa::launch_gemm_tn(g, G, (hipStream_t)stream), "csa_project_out");
}

}  // extern "C"
