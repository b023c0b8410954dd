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
// v_mfma_f32_32x32x16_bf16.  A work-group computes a 256 x 256 tile with 8
// waves of 128 x 64 (128 x 128 with 4 waves of 64 x 64 for small problems);
// K advances 32 at a time through a 3-slot LDS ring filled by direct-to-LDS
// buffer loads issued two steps ahead.  A row of a slot holds 32 bf16 (64 bytes, four 16-byte
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

// Tile BM x BN, NWM x NWN waves, each wave (BM/NWM) x (BN/NWN) in 32 x 32
// MFMA tiles.  The grid is one-dimensional: work-group ids are first spread
// so that each of the 8 XCDs (which take ids round robin) runs a contiguous
// range of tiles, and tiles are ordered in stripes of 4 row panels, column
// by column, so the tiles running together on an XCD share a few A and B
// panels in its L2.
template <int BM, int BN, int NWM, int NWN>
__global__ __launch_bounds__(64 * NWM * NWN) void gemm_tn_kernel(GemmParams p, int tm, int tn, int tiles) {
  constexpr int NW = NWM * NWN;
  constexpr int TM = BM / NWM / 32, TN = BN / NWN / 32;  // MFMA tiles per wave
  constexpr int QA = BM / 16 / NW, QB = BN / 16 / NW;    // 16-row loads per wave and step
  constexpr int SA = BM * 64, SB = BN * 64;              // slot bytes
  static_assert(QA >= 1 && QB >= 1 && BM % (16 * NW) == 0 && BN % (16 * NW) == 0, "load split");
  __shared__ __attribute__((aligned(16))) uint8_t As[kGemmRing][SA];
  __shared__ __attribute__((aligned(16))) uint8_t Bs[kGemmRing][SB];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / NWN, wn = wave % NWN;

  // work-group id -> tile
  int t = blockIdx.x;
  const int per = tiles >> 3;
  if (t < per * 8) t = (t & 7) * per + (t >> 3);
  const int per_group = tm * tn;
  const int z = t / per_group;
  t -= z * per_group;
  const int stripe = t / (4 * tn), u = t - stripe * 4 * tn;
  const int h = min(4, tm - 4 * stripe);
  const int my = 4 * stripe + u % h, nx = u / h;
  const int m0 = my * BM, n0 = nx * BN;

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
  // 32-bit byte offsets: below the extent for every row inside M (N); rows
  // of a ragged last tile may wrap, which only loads values that are
  // never stored
  const uint32_t lda2 = (uint32_t)p.lda * 2u, ldb2 = (uint32_t)p.ldb * 2u;
  const int nk = p.K >> 5;

  // This wave's loads of a K step: A rows (BM/NW)*wave + 16 q + lane/4 (and
  // likewise B).  Lane l of a load fills LDS piece l % 4 of its row with
  // global piece (l % 4) ^ swz(row), swz(row) = (row >> 2) & 3.  Steps past
  // the end load nothing useful into a free slot (offset past every extent).
  const int lrow = lane >> 2;
  uint32_t offA[QA], offB[QB];
#pragma unroll
  for (int q = 0; q < QA; ++q) {
    const int r = (BM / NW) * wave + 16 * q + lrow;
    offA[q] = (uint32_t)(m0 + r) * lda2 + (uint32_t)(((lane & 3) ^ ((r >> 2) & 3)) << 4);
  }
#pragma unroll
  for (int q = 0; q < QB; ++q) {
    const int r = (BN / NW) * wave + 16 * q + lrow;
    offB[q] = (uint32_t)(n0 + r) * ldb2 + (uint32_t)(((lane & 3) ^ ((r >> 2) & 3)) << 4);
  }
  const uint32_t lds_a = (uint32_t)__builtin_amdgcn_readfirstlane(
      (int)((uint32_t)(uintptr_t)LDS_PTR(uint8_t, &As[0][0]) + (uint32_t)(wave * (BM / NW) * 64)));
  const uint32_t lds_b = (uint32_t)__builtin_amdgcn_readfirstlane(
      (int)((uint32_t)(uintptr_t)LDS_PTR(uint8_t, &Bs[0][0]) + (uint32_t)(wave * (BN / NW) * 64)));
  auto issue = [&](int ks, int slot) {
    const uint32_t kb = (uint32_t)ks * 64u;  // bytes into a row
    const bool live = ks < nk;
#pragma unroll
    for (int q = 0; q < QA; ++q)
      dma_b128(rA, lds_a + (uint32_t)(slot * SA + q * 1024), live ? offA[q] + kb : 0xfffffff0u);
#pragma unroll
    for (int q = 0; q < QB; ++q)
      dma_b128(rB, lds_b + (uint32_t)(slot * SB + q * 1024), live ? offB[q] + kb : 0xfffffff0u);
  };

  // operand reads: row (tile base + lane % 32), K piece kk*2 + lane / 32
  const int orow = lane & 31, ohalf = lane >> 5;
  uint32_t aoff[TM][2], boff[TN][2];  // byte offsets inside a slot
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    const int c = kk * 2 + ohalf;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int ra = wm * (BM / NWM) + i * 32 + orow;
      aoff[i][kk] = (uint32_t)(ra * 64 + ((c ^ ((ra >> 2) & 3)) << 4));
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int rb = wn * (BN / NWN) + j * 32 + orow;
      boff[j][kk] = (uint32_t)(rb * 64 + ((c ^ ((rb >> 2) & 3)) << 4));
    }
  }

  f32x16 C[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) C[i][j][e] = 0.0f;

  constexpr int kWait = QA + QB;  // loads per wave and step
  auto step = [&](int ks, auto tag) {
    constexpr int slot = decltype(tag)::value;
    // this wave's loads of step ks have landed (only step ks+1's may still
    // be in flight); the barrier makes every wave's loads visible and ends
    // all reads of step ks-1, whose slot is refilled next
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kWait) : "memory");
    __syncthreads();
    const uint8_t* a = &As[slot][0];
    const uint8_t* b = &Bs[slot][0];
    // every operand read of the step is issued first (one LDS round trip),
    // then the next loads, then the MFMAs
    bf16x8 fa[2][TM], fb[2][TN];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
      for (int i = 0; i < TM; ++i) fa[kk][i] = *(const bf16x8*)(a + aoff[i][kk]);
#pragma unroll
      for (int j = 0; j < TN; ++j) fb[kk][j] = *(const bf16x8*)(b + boff[j][kk]);
    }
    issue(ks + 2, (slot + 2) % kGemmRing);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          C[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[kk][i], fb[kk][j], C[i][j], 0, 0, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * (TM + TN), 0);  // LDS reads
    __builtin_amdgcn_sched_group_barrier(0x008, 2 * TM * TN, 0);    // MFMAs
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
  for (int j = 0; j < TN; ++j) {
    const int n = n0 + wn * (BN / NWN) + j * 32 + orow;
    if (n >= p.N) continue;
    const int ng = z * p.c_zcol + n;  // output column
    int s = 0;
#pragma unroll
    for (int k = 1; k < kGemmOuts; ++k)
      if (k < p.nout && ng >= p.out[k].n0) s = k;
    const GemmOut o = p.out[s];
    const int col = ng - o.n0;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int m = m0 + wm * (BM / NWM) + i * 32 + 8 * (e >> 2) + 4 * ohalf + (e & 3);
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

template <int BM, int BN, int NWM, int NWN>
hipError_t launch_tiles(const GemmParams& p, int groups, hipStream_t stream) {
  const int tm = (p.M + BM - 1) / BM, tn = (p.N + BN - 1) / BN;
  const int tiles = tm * tn * groups;
  hipLaunchKernelGGL((gemm_tn_kernel<BM, BN, NWM, NWN>), dim3((unsigned)tiles), dim3(64 * NWM * NWN), 0, stream,
                     p, tm, tn, tiles);
  return hipGetLastError();
}

hipError_t launch_gemm_tn(const GemmParams& p, int groups, hipStream_t stream) {
  if (p.M == 0 || p.N == 0 || groups == 0) return hipSuccess;
  // large problems: 256 x 256 tiles (128 flops per loaded byte, half the
  // per-CU load rate at the MFMA peak); small ones: 128 x 128 tiles
  if (p.M >= 1024 && p.N >= 256) return launch_tiles<256, 256, 2, 4>(p, groups, stream);
  return launch_tiles<128, 128, 2, 2>(p, groups, stream);
}

// ---- low-rank indexer query and its MXFP4 encoding: a work-group takes
// one block of 32 outputs for 256 rows (one row per lane); q = lat . W_up^T
// in fp32 (fma chain over the rank in ascending order), then the O4 rule:
// E = floor(log2(amax)) - 2, codes are the e2m1 values of q / 2^E (nearest,
// ties to even, saturating at 6).  The block's 32 rows of W_up are staged in
// LDS and read as broadcasts.
template <int R>  // rank (16, 32 or 64)
__global__ __launch_bounds__(256) void qidx_mxfp4_kernel(QidxParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t Ws[32 * R];
  const int nblk = p.nq >> 5;
  const int blk = blockIdx.x % nblk;
  const int64_t row = (int64_t)(blockIdx.x / nblk) * 256 + threadIdx.x;
  if (threadIdx.x * 8 < 32 * R)
    *(u32x4*)&Ws[threadIdx.x * 8] = *(const u32x4*)&p.w_up[(int64_t)blk * 32 * R + threadIdx.x * 8];
  __syncthreads();
  if (row >= p.M) return;
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
    const uint16_t* w = &Ws[c * R];
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
    float* dst = &p.q_f32[row * p.nq + blk * 32];
#pragma unroll
    for (int c = 0; c < 32; c += 4) *(f32x4*)&dst[c] = f32x4{q[c], q[c + 1], q[c + 2], q[c + 3]};
  }
}

hipError_t launch_qidx_mxfp4(const QidxParams& p, hipStream_t stream) {
  if (p.M == 0) return hipSuccess;
  const dim3 grid((unsigned)(((int64_t)p.M + 255) / 256 * (p.nq >> 5)));
  switch (p.r) {
    case 16: hipLaunchKernelGGL(qidx_mxfp4_kernel<16>, grid, dim3(256), 0, stream, p); break;
    case 32: hipLaunchKernelGGL(qidx_mxfp4_kernel<32>, grid, dim3(256), 0, stream, p); break;
    case 64: hipLaunchKernelGGL(qidx_mxfp4_kernel<64>, grid, dim3(256), 0, stream, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace csa
