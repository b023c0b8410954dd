// proj.hip -- the projections around the attention path: the layer's input
// projections (hidden state -> query rows, the shared KV row, the indexer
// key stream, the indexer latent and head weights), the low-rank indexer
// query with its MXFP4 encoding, and the grouped output projection.
//
// Method: "DeepSeek-V4: Towards Highly Efficient Million-Token Context
// Intelligence" wiki summary, Proposed method item 1 (shared-KV MQA with a
// grouped output projection; the Lightning Indexer made cheap by a low-rank
// factorisation and FP4, "deepseek V4 技术论文" 1.1) and Post-training item 3
// (MXFP4 for the indexer's QK path).
//
// Design: one bf16 GEMM kernel, C = A . B^T with both operands K-contiguous
// (weights in the [out, in] layout), fp32 accumulation in
// v_mfma_f32_32x32x16_bf16.  A work-group of 4 waves computes a 128 x 128
// tile, each wave 64 x 64 (2 x 2 MFMA tiles); K advances 32 at a time
// through a 3-slot LDS ring filled by direct-to-LDS buffer loads issued two
// steps ahead.  A row of a slot holds 32 bf16 (64 bytes, four 16-byte
// pieces); piece c of row r is stored at position c ^ ((r >> 2) & 3), which
// keeps each 16-lane group of an operand read on distinct banks.  The
// epilogue routes output columns to up to 6 destinations (bf16 or fp32), so
// the input projections are one launch.  blockIdx.z selects a group: A, B
// and the output columns move by fixed strides, which is the grouped output
// projection.
#include "device.h"
#include "kernels.h"

namespace csa {

constexpr int kGemmRing = 3;

template <int S>
struct GSlot {
  static constexpr int value = S;
};

__global__ __launch_bounds__(256) void gemm_tn_kernel(GemmParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t As[kGemmRing][128 * 64];
  __shared__ __attribute__((aligned(16))) uint8_t Bs[kGemmRing][128 * 64];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = blockIdx.y * 128, n0 = blockIdx.x * 128, z = blockIdx.z;

  auto uniform_ptr = [](const void* ptr) {
    const uint64_t v = (uint64_t)ptr;
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
    return (void*)(((uint64_t)hi << 32) | lo);
  };
  // descriptors of this group's operands: rows past M (N) lie past the
  // extent and read as zeros
  const u32x4 rA = dma_rsrc(uniform_ptr(p.A + (int64_t)z * p.a_zoff), p.a_bytes - (uint32_t)z * p.a_zbytes);
  const u32x4 rB = dma_rsrc(uniform_ptr(p.B + (int64_t)z * p.b_zoff), p.b_bytes);
  const uint32_t lda2 = (uint32_t)p.lda * 2u, ldb2 = (uint32_t)p.ldb * 2u;
  const int nk = p.K >> 5;

  // This wave's loads of a K step: A rows and B rows 32*wave .. +31 (two
  // loads of 16 rows each).  Lane l of a load fills LDS piece l % 4 of row
  // l / 4 with global piece (l % 4) ^ swz(row).  Steps past the end load
  // nothing useful into a free slot (offset past every extent).
  const int lrow = lane >> 2;
  uint32_t offA[2], offB[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int r = 32 * wave + 16 * q + lrow;
    const uint32_t piece = (uint32_t)(((lane & 3) ^ ((r >> 2) & 3)) << 4);
    offA[q] = (uint32_t)(m0 + r) * lda2 + piece;
    offB[q] = (uint32_t)(n0 + r) * ldb2 + piece;
  }
  const uint32_t lds_a = (uint32_t)__builtin_amdgcn_readfirstlane(
      (int)((uint32_t)(uintptr_t)LDS_PTR(uint8_t, &As[0][0]) + (uint32_t)(wave * 2048)));
  const uint32_t lds_b = (uint32_t)__builtin_amdgcn_readfirstlane(
      (int)((uint32_t)(uintptr_t)LDS_PTR(uint8_t, &Bs[0][0]) + (uint32_t)(wave * 2048)));
  auto issue = [&](int ks, int slot) {
    const uint32_t kb = (uint32_t)ks * 64u;  // bytes into a row
    const bool live = ks < nk;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      dma_b128(rA, lds_a + (uint32_t)(slot * 8192 + q * 1024), live ? offA[q] + kb : 0xfffffff0u);
      dma_b128(rB, lds_b + (uint32_t)(slot * 8192 + q * 1024), live ? offB[q] + kb : 0xfffffff0u);
    }
  };

  // operand reads: row (tile base + lane % 32), K piece kk*2 + lane / 32
  const int orow = lane & 31, ohalf = lane >> 5;
  uint32_t aoff[2][2], boff[2][2];  // [tile][kk] byte offsets inside a slot
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int ra = wm * 64 + t * 32 + orow, rb = wn * 64 + t * 32 + orow;
      const int c = kk * 2 + ohalf;
      aoff[t][kk] = (uint32_t)(ra * 64 + ((c ^ ((ra >> 2) & 3)) << 4));
      boff[t][kk] = (uint32_t)(rb * 64 + ((c ^ ((rb >> 2) & 3)) << 4));
    }

  f32x16 C[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) C[i][j][e] = 0.0f;

  auto step = [&](int ks, auto tag) {
    constexpr int slot = decltype(tag)::value;
    // this wave's loads of step ks have landed (only step ks+1's may still
    // be in flight); the barrier makes every wave's loads visible and ends
    // all reads of step ks-1, whose slot is refilled next
    asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
    __syncthreads();
    issue(ks + 2, (slot + 2) % kGemmRing);
    const uint8_t* a = &As[slot][0];
    const uint8_t* b = &Bs[slot][0];
    bf16x8 fa[2][2], fb[2][2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        fa[t][kk] = *(const bf16x8*)(a + aoff[t][kk]);
        fb[t][kk] = *(const bf16x8*)(b + boff[t][kk]);
      }
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) C[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i][kk], fb[j][kk], C[i][j], 0, 0, 0);
  };
  static_assert(kGemmRing == 3, "the K loop is unrolled over 3 ring slots");
  issue(0, 0);
  issue(1, 1);
  for (int ks = 0; ks < nk; ks += 3) {
    step(ks, GSlot<0>{});
    if (ks + 1 < nk) step(ks + 1, GSlot<1>{});
    if (ks + 2 < nk) step(ks + 2, GSlot<2>{});
  }
  // every load into the ring has landed before the work-group ends
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // ---- epilogue: lane l holds column l % 32 of each tile, rows
  // 8*(e/4) + 4*(l/32) + e%4
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int n = n0 + wn * 64 + j * 32 + orow;
    if (n >= p.N) continue;
    const int ng = z * p.c_zcol + n;  // output column
    int s = 0;
#pragma unroll
    for (int k = 1; k < kGemmOuts; ++k)
      if (k < p.nout && ng >= p.out[k].n0) s = k;
    const GemmOut o = p.out[s];
    const int col = ng - o.n0;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int m = m0 + wm * 64 + i * 32 + 8 * (e >> 2) + 4 * ohalf + (e & 3);
        if (m >= p.M) continue;
        const float v = C[i][j][e];
        if (o.f32) {
          ((float*)o.ptr)[(int64_t)m * o.ld + col] = v;
        } else {
          ((uint16_t*)o.ptr)[(int64_t)m * o.ld + col] = (uint16_t)f32_to_bf16(v);
        }
      }
    }
  }
}

hipError_t launch_gemm_tn(const GemmParams& p, int groups, hipStream_t stream) {
  if (p.M == 0 || p.N == 0 || groups == 0) return hipSuccess;
  dim3 grid((unsigned)((p.N + 127) / 128), (unsigned)((p.M + 127) / 128), (unsigned)groups);
  hipLaunchKernelGGL(gemm_tn_kernel, grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

// ---- low-rank indexer query and its MXFP4 encoding: lane = (row, block of
// 32 outputs); q = lat . W_up^T in fp32 (fma chain over the rank in
// ascending order), then the O4 rule: E = floor(log2(amax)) - 2, codes are
// the e2m1 values of q / 2^E (nearest, ties to even, saturating at 6).
// W_up is staged in LDS by each work-group.
constexpr int kQidxMaxW = 512 * 64;  // bf16 elements of W_up (H_I*64 x r <= 32768)

template <int R>  // rank (8 .. 64, a multiple of 8)
__global__ __launch_bounds__(256) void qidx_mxfp4_kernel(QidxParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t Ws[kQidxMaxW];
  const int nw = p.nq * R;  // W_up elements
  for (int i = threadIdx.x * 8; i < nw; i += 256 * 8) *(u32x4*)&Ws[i] = *(const u32x4*)&p.w_up[i];
  __syncthreads();
  const int nblk = p.nq >> 5;
  const int64_t task = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (task >= (int64_t)p.M * nblk) return;
  const int64_t row = task / nblk;
  const int blk = (int)(task % nblk);
  float lat[R];
#pragma unroll
  for (int k8 = 0; k8 < R / 8; ++k8) {
    const u32x4 v = *(const u32x4*)&p.lat[row * p.ld_lat + k8 * 8];
#pragma unroll
    for (int e = 0; e < 4; ++e) { lat[k8 * 8 + 2 * e] = bf16lo(v[e]); lat[k8 * 8 + 2 * e + 1] = bf16hi(v[e]); }
  }
  float q[32];
  float amax = 0.0f;
#pragma unroll
  for (int c = 0; c < 32; ++c) {
    const uint16_t* w = &Ws[(blk * 32 + c) * R];
    float s = 0.0f;
#pragma unroll
    for (int k = 0; k < R; k += 2) {
      const uint32_t wp = *(const uint32_t*)&w[k];
      s = __builtin_fmaf(lat[k], bf16lo(wp), s);
      s = __builtin_fmaf(lat[k + 1], bf16hi(wp), s);
    }
    q[c] = s;
    amax = fmaxf(amax, fabsf(s));
  }
  uint32_t codes[4] = {0u, 0u, 0u, 0u};
  uint32_t sbyte = 0u;
  if (amax > 0.0f) {
    const int E = mxfp4_exponent(amax);
    sbyte = (uint32_t)(E + 127);
#pragma unroll
    for (int c = 0; c < 32; ++c) codes[c >> 3] |= f32_to_e2m1(__builtin_ldexpf(q[c], -E)) << (4 * (c & 7));
  }
  *(u32x4*)&p.codes[row * (p.nq >> 1) + blk * 16] = u32x4{codes[0], codes[1], codes[2], codes[3]};
  p.scales[row * nblk + blk] = (uint8_t)sbyte;
  if (p.q_f32) {
#pragma unroll
    for (int c = 0; c < 32; ++c) p.q_f32[row * p.nq + blk * 32 + c] = q[c];
  }
}

hipError_t launch_qidx_mxfp4(const QidxParams& p, hipStream_t stream) {
  const int64_t tasks = (int64_t)p.M * (p.nq >> 5);
  if (tasks == 0) return hipSuccess;
  const dim3 grid((unsigned)((tasks + 255) / 256));
  switch (p.r) {
    case 16: hipLaunchKernelGGL(qidx_mxfp4_kernel<16>, grid, dim3(256), 0, stream, p); break;
    case 32: hipLaunchKernelGGL(qidx_mxfp4_kernel<32>, grid, dim3(256), 0, stream, p); break;
    case 64: hipLaunchKernelGGL(qidx_mxfp4_kernel<64>, grid, dim3(256), 0, stream, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace csa
