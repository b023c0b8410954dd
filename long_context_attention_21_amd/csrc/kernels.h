// kernels.h -- parameter blocks and launchers shared between the C ABI layer
// (abi.cpp) and the HIP kernels.  All pointers are device pointers.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csa {

struct CompressParams {
  const uint32_t* kv;       // [B, T, 128] bf16 (read as bf16 pairs)
  const uint32_t* ik;       // [B, T, 64] bf16 or null
  const float* z;           // [B, T, 2] or null
  const float* beta;        // [L]
  const uint32_t* prev_kv;  // [B, m, 128] or null
  const uint32_t* prev_ik;  // [B, m, 64] or null
  const float* prev_z;      // [B, m, 2] or null
  int B, T, n_new, m, L, overlap, rope_dims;
  int64_t pos0;
  void* entries_out;
  void* entries_rope_out;
  float* entry_scale_out;
  int entry_fmt;  // 0 bf16, 2 fp8 + bf16 rope
  void* kidx_out;
  uint8_t* kidx_scale_out;
  int kidx_fmt;  // 0 bf16, 1 mxfp4
  double theta[32];  // rope_base^(-2f/64), fp64
  // Cache append (decode): one new row per sequence at position t.  Rows
  // j < t come from the rings (slot j % W; the KV ring keeps each row at
  // slots j % W and j % W + W), row t from the *_new arrays, which are also
  // written to the rings.  When t completes a block, its entry is stored at
  // row (t + 1) / m - 1 of caches with N_cap rows per sequence.
  int append;
  const uint32_t* kv_new;  // [B, 128] bf16
  const uint32_t* ik_new;  // [B, 64] bf16 or null
  const float* z_new;      // [B, 2] or null
  uint32_t* kv_ring;       // [B, 2W, 128] bf16
  uint32_t* ik_ring;       // [B, W, 64] bf16 or null
  float* z_ring;           // [B, W, 2] or null
  uint8_t* win8_ring;      // [B, 2W, 128] e4m3 post-RoPE window cache or null (slots as kv_ring)
  float* win8_scale;       // [B, 2W] with win8_ring
  int W, N_cap;
  int64_t t;
  __device__ uint8_t* kidx_out_u8() const { return (uint8_t*)kidx_out; }
};

hipError_t launch_compress(const CompressParams& p, hipStream_t stream);

struct AttendParams {
  const uint16_t* q;  // [B, n, H, 128]
  int B, n, H;
  int64_t q_pos0;
  const uint16_t* entries;       // bf16 [B, N, 128] or e4m3 [B, N, 64]
  const uint16_t* entries_rope;  // fp8 format: bf16 [B, N, 64]
  const float* entry_scale;      // fp8 format: [B, N]
  int N, m;
  const int32_t* idx;  // CSA: [B, n, k]
  int k;
  const uint16_t* win;  // [B, win_len, 128] bf16 pre-RoPE, or e4m3 post-RoPE when win_fp8
  const float* win_scale;  // win_fp8: [B, win_len]
  int win_fp8;
  int win_roped;  // bf16 window rows already rotated at their positions
  int64_t win_pos0;
  int win_len, n_win;
  const float* sink;  // [H] or null
  int rope;           // 1: rotate dims 64..127
  float qscale;       // log2(e) / sqrt(128), folded into q
  uint16_t* out;      // [B, n, H, 128]
  double rev[32];     // theta_f / (2 pi): revolutions per position
  // split decode (FP8 entries, few query rows): `parts` work-groups per token
  // take `cpp` chunks each and leave partial results in ws
  float* ws;
  int parts, cpp;
  int64_t tok0;  // split path: first token of the launch's block
};

// Workspace of the split decode path: per (token, part) the unnormalised
// O[64][128], then the softmax reference and the row sum of each head.
constexpr int kAttendPartFloats = 64 * 128 + 2 * 64;
constexpr int kAttendChunksPerPart = 8;
constexpr int kAttendSplitTokens = 512;  // tokens per split launch (bounds the workspace)
size_t attend_workspace(int mode, int B, int n, int k, int n_win);

// mode: 0 = CSA with bf16 entries, 1 = CSA with fp8+bf16 entries, 2 = HCA,
// 3 = CSA with NVFP4 entries
hipError_t launch_attend(const AttendParams& p, int mode, hipStream_t stream);

// Window rows rotated once: out[row] = kv[row] with dims 64..127 rotated at
// position pos0 + (row % T) in fp64, rounded to fp32, then to bf16.
struct RopeRowsParams {
  const uint32_t* kv;  // [rows, 64] bf16 pairs
  uint32_t* out;
  int64_t rows;
  int T;
  int64_t pos0;
  double theta[32];
};
hipError_t launch_rope_rows(const RopeRowsParams& p, hipStream_t stream);

struct IndexParams {
  const void* q;             // bf16 [B, n, H_I, 64] or mxfp4 codes [B, n, H_I, 32]
  const uint8_t* q_scale;    // [B, n, H_I, 2] or null (quantise bf16 q in-kernel)
  const float* w;            // [B, n, H_I]
  const void* kidx;          // bf16 [B, N, 64] or mxfp4 codes [B, N, 32]
  const uint8_t* kidx_scale; // [B, N, 2]
  int fmt;                   // 0 bf16, 1 mxfp4
  int B, n, H_I, N, m, k;
  int64_t q_pos0;
  int32_t* idx_out;          // [B, n, k]
  void* ws;
  size_t ws_bytes;
  uint32_t* fallback_count;  // caller-owned device counter or null
};

hipError_t launch_index_topk(const IndexParams& p, hipStream_t stream);
size_t index_topk_workspace(int B, int n, int64_t q_pos0, int N, int m, int k);

// Workspace row of the indexer's split path, and the device scratch of the
// allocation-free variant: 256 such rows.  static_scratch() gives the
// scratch's address on the current device.
constexpr size_t kSplitRowBytes = 32784;
constexpr size_t kStaticScratchBytes = 256 * kSplitRowBytes;
hipError_t static_scratch(void** ptr);

// bf16 GEMM C = A . B^T (A [M, K] rows lda apart, B [N, K] rows ldb apart,
// fp32 accumulation; K a multiple of 32).  Output column c (plus z * c_zcol
// for group z) goes to the destination whose range [n0, n1) holds it.
constexpr int kGemmOuts = 6;
struct GemmOut {
  void* ptr;
  int n0, n1, ld, f32;  // column range, leading dimension (elements), fp32 (1) or bf16 (0)
};
struct GemmParams {
  const uint16_t* A;
  const uint16_t* B;
  int M, N, K, lda, ldb;
  int64_t a_zoff, b_zoff;  // elements added to A and B per group z
  uint32_t a_bytes, b_bytes, a_zbytes;  // extents from the (group-0) bases; a_zoff * 2
  int c_zcol;
  int nout;
  GemmOut out[kGemmOuts];
};
hipError_t launch_gemm_tn(const GemmParams& p, int groups, hipStream_t stream);

// Low-rank indexer query: q = lat . W_up^T (fp32 fma chain over the rank r,
// ascending), MXFP4-encoded per 32 outputs.
struct QidxParams {
  const uint16_t* lat;   // [M, r] bf16, rows ld_lat apart
  const uint16_t* w_up;  // [nq, r] bf16
  int M, r, nq, ld_lat;
  uint8_t* codes;        // [M, nq / 2]
  uint8_t* scales;       // [M, nq / 32]
  float* q_f32;          // [M, nq] or null
};
hipError_t launch_qidx_mxfp4(const QidxParams& p, hipStream_t stream);

}  // namespace csa
