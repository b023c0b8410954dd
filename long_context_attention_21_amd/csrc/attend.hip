// attend.hip -- CSA sparse attention and HCA dense attention, each with the
// sliding-window branch, the per-head sink and partial RoPE.
//
// Method: "deepseek V4 技术论文" 1.1 (each query token attends only to its
// top-k compressed entries; the entries serve as both key and value and are
// shared by all heads: MQA; HCA attends densely to all heavily compressed
// entries; an independent 128-token sliding-window branch; a learnable sink
// that lets a head put attention "into the void"), "DeepSeek-V4: Towards
// Highly Efficient Million-Token Context Intelligence" wiki summary,
// Proposed method item 1 (n_win = 128, sink, partial RoPE on the last 64
// dims with inverse RoPE on the core-attention output).  One softmax per
// (token, head) over sink + entries + window.
//
// Design for CDNA4: because all heads share one KV row (MQA), one wave takes
// one query token and ALL its heads as the N dimension of the MFMA:
//     S^T[key, head] = K[key, :] . Q^T[:, head]      (v_mfma_f32_16x16x32_bf16)
//     O^T[dim, head] += V^T[dim, key] . P^T[key, head]
// Keys arrive in chunks of 32 rows: gathered entry rows (CSA: idx list;
// HCA: every visible entry), then the window rows.  Each lane gathers its
// rows straight into the K-operand register layout (16-byte pieces), so K
// never goes through LDS; the same registers are stored to a double-buffered
// LDS tile from which the V^T operand is read with ds_read_b64_tr_b16.  The
// transposed product leaves P^T in registers in exactly the B-operand layout
// of the PV product.  The loop is software-pipelined: the rows of chunk c+1
// are in flight while chunk c is computed (entry indices three chunks ahead),
// and the head tiles' MFMA and softmax work interleave.  Row sums come
// from one MFMA against a tile of ones.  The softmax scale and log2(e) are
// folded into q; weights are taken against a fixed per-head reference (the
// sink logit or the first chunk's maximum), so the accumulators never need
// rescaling inside the loop.
#include "device.h"
#include "kernels.h"

namespace csa {

constexpr int KP = 136;           // LDS row pitch in bf16 (272 bytes: 16-byte skew per row)
constexpr float kSlack = 64.0f;  // allowed excess of a score over the reference (log2 units)
constexpr int kMaxK = 2048;       // largest top-k whose index row is staged in LDS

struct ChunkRegs {
  u32x4 r[2][4];  // key tile kt (rows kt*16 + l%16), dims ks*32 + 8*(l/16) .. +7
  float sc[2];    // fp8 entry scale per key tile
  bool v[2];      // key validity
};

// SPLIT: work-group (token, part) takes chunks [part * cpp, (part+1) * cpp)
// and leaves its unnormalised O, reference and row sums in the workspace for
// attend_combine_kernel.
template <int NHT, int MODE, bool SPLIT = false>  // MODE 0: CSA bf16, 1: CSA fp8+bf16, 3: CSA NVFP4 entries; 2: HCA
__global__ __launch_bounds__(64) void attend_kernel(AttendParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t Vs[2][32 * KP];
  __shared__ __attribute__((aligned(16))) int32_t Is[MODE == 2 ? 4 : kMaxK];  // the token's idx row
  const int lane = threadIdx.x;
  const int g = lane >> 4, l16 = lane & 15;
  // b * n + q; the split path runs the tokens in blocks (tok0: the block's first)
  const int64_t tok = SPLIT ? p.tok0 + blockIdx.x / p.parts : blockIdx.x;
  const int part = SPLIT ? (int)(blockIdx.x % p.parts) : 0;
  const int b = (int)(tok / p.n);
  const int qi = (int)(tok % p.n);
  const int64_t t = p.q_pos0 + qi;
  const float LOG2E = 1.4426950408889634f;
  const float NEG_INF = -__builtin_inff();

  // ---- Q^T operand: lane l holds head ht*16+l16, dims ks*32 + 8g .. +7.
  // Every load is issued before the first is used (one memory round trip):
  // lanes past the last head read head H-1 and use zeros.
  bf16x8 Q[NHT][4];
  float skv[NHT];  // the heads' sink logits (0 past the last head)
  {
    u32x4 qraw[NHT][4];
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) {
      const int hc = min(ht * 16 + l16, p.H - 1);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) qraw[ht][ks] = *(const u32x4*)(p.q + ((tok * p.H + hc) * 128 + ks * 32 + 8 * g));
      skv[ht] = p.sink ? p.sink[hc] : 0.0f;
      if (ht * 16 + l16 >= p.H) skv[ht] = 0.0f;
    }
    float qc[8], qs[8];
    if (p.rope) {
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int pp = 0; pp < 4; ++pp)
          rope_cs((double)t, p.rev[kk * 16 + 4 * g + pp], qc[kk * 4 + pp], qs[kk * 4 + pp]);
    }
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) {
      const int h = ht * 16 + l16;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        float x[8];
        if (h < p.H) {
          const u32x4 v = qraw[ht][ks];
#pragma unroll
          for (int e = 0; e < 4; ++e) { x[2 * e] = bf16lo(v[e]); x[2 * e + 1] = bf16hi(v[e]); }
          if (p.rope && ks >= 2) {
#pragma unroll
            for (int pp = 0; pp < 4; ++pp) {
              const float c = qc[(ks - 2) * 4 + pp], s = qs[(ks - 2) * 4 + pp];
              const float a0 = x[2 * pp], a1 = x[2 * pp + 1];
              x[2 * pp] = a0 * c - a1 * s;
              x[2 * pp + 1] = a0 * s + a1 * c;
            }
          }
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] = 0.0f;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) Q[ht][ks][e] = (__bf16)(x[e] * p.qscale);
      }
    }
  }

  // ---- softmax state.  Weights are exp2(s - mref) against a fixed reference
  // mref per head (the sink logit, or the first chunk's maximum), so O and
  // the row sums L are only ever touched by MFMAs inside the loop.  If a later
  // chunk exceeds mref by more than 2^kSlack the token restarts with the
  // larger reference (never seen in practice; it keeps the result exact).
  float mref[NHT];
  f32x4 O[8][NHT], Lacc[NHT];
#pragma unroll
  for (int ht = 0; ht < NHT; ++ht) mref[ht] = p.sink ? skv[ht] * LOG2E : -1e30f;
  bf16x8 ones;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones[e] = (__bf16)1.0f;

  // ---- key sequence: entry chunks, then window chunks
  int n_ent;
  if (MODE == 2) {
    const int64_t nv = (t + 1) / p.m;
    n_ent = (int)(nv < p.N ? nv : p.N);
  } else {
    n_ent = p.k;
  }
  const int n_ent_chunks = (n_ent + 31) >> 5;
  int64_t j0 = 0;
  int n_wk = 0;
  if (p.n_win > 0) {
    j0 = t - p.n_win + 1;
    if (j0 < 0) j0 = 0;
    n_wk = (int)(t - j0 + 1);
  }
  const int n_chunks = n_ent_chunks + ((n_wk + 31) >> 5);
  const int c_lo = SPLIT ? part * p.cpp : 0;  // this work-group's chunks [c_lo, c_hi)
  const int c_hi = SPLIT ? (c_lo + p.cpp < n_chunks ? c_lo + p.cpp : n_chunks) : n_chunks;

  // CSA: stage the token's index row in LDS once (coalesced 16-byte loads),
  // so the loop reads indices from LDS and never waits on them in HBM
  if (MODE != 2) {
    const int32_t* irow = p.idx + tok * p.k;
    if ((p.k & 3) == 0) {
      for (int i = 4 * lane; i < p.k; i += 256) *(u32x4*)&Is[i] = *(const u32x4*)&irow[i];
    } else {
      for (int i = lane; i < p.k; i += 64) Is[i] = irow[i];
    }
    __builtin_amdgcn_wave_barrier();
  }

  // entry index of this lane's key kt in chunk c (-1: none)
  auto fetch_idx = [&](int c, int out[2]) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const int kk = c * 32 + kt * 16 + l16;
      int s = -1;
      if (c < n_ent_chunks) {
        if (MODE == 2) s = kk < n_ent ? kk : -1;
        else if (kk < p.k) s = Is[kk];
      }
      if ((uint32_t)s >= (uint32_t)p.N) s = -1;  // -1 padding, or an index past the entries: no key
      out[kt] = s;
    }
  };
  // Row sources as buffer descriptors of this batch row.  The hardware
  // range check returns zeros for offsets past the end, so a missing key
  // (index -1, past the window, past the last chunk) is an unconditional load
  // at an out-of-range offset: no branch, and the compiler can track exactly
  // which loads each use waits for.
  auto uniform_ptr = [](const void* ptr) {
    const uint64_t v = (uint64_t)ptr;
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
    return (void*)(((uint64_t)hi << 32) | lo);
  };
  constexpr int kOOB = 0x7fff0000;  // past every row source (the host bounds them below this)
  const int bu = __builtin_amdgcn_readfirstlane(b);
  const int wrow = p.win_fp8 ? 128 : 256;  // bytes per window row
  __amdgpu_buffer_rsrc_t rW = __builtin_amdgcn_make_buffer_rsrc(
      uniform_ptr(p.win ? (const uint8_t*)p.win + (int64_t)bu * p.win_len * wrow : (const uint8_t*)p.q), (short)0,
      p.win ? __builtin_amdgcn_readfirstlane(p.win_len * wrow) : 0, 0x00020000);
  __amdgpu_buffer_rsrc_t rWS = rW;
  if (p.win_fp8)
    rWS = __builtin_amdgcn_make_buffer_rsrc(uniform_ptr(p.win_scale + (int64_t)bu * p.win_len), (short)0,
                                            __builtin_amdgcn_readfirstlane(p.win_len * 4), 0x00020000);
  __amdgpu_buffer_rsrc_t rE, rR = rW, rS = rW;
  if (MODE == 3) {
    rE = __builtin_amdgcn_make_buffer_rsrc(uniform_ptr((const uint8_t*)p.entries + (int64_t)bu * p.N * 72),
                                           (short)0, __builtin_amdgcn_readfirstlane(p.N * 72), 0x00020000);
    rS = __builtin_amdgcn_make_buffer_rsrc(uniform_ptr(p.entry_scale + (int64_t)bu * p.N), (short)0,
                                           __builtin_amdgcn_readfirstlane(p.N * 4), 0x00020000);
  } else if (MODE == 1) {
    rE = __builtin_amdgcn_make_buffer_rsrc(uniform_ptr((const uint8_t*)p.entries + (int64_t)bu * p.N * 64),
                                           (short)0, __builtin_amdgcn_readfirstlane(p.N * 64), 0x00020000);
    rR = __builtin_amdgcn_make_buffer_rsrc(uniform_ptr(p.entries_rope + (int64_t)bu * p.N * 64), (short)0,
                                           __builtin_amdgcn_readfirstlane(p.N * 128), 0x00020000);
    rS = __builtin_amdgcn_make_buffer_rsrc(uniform_ptr(p.entry_scale + (int64_t)bu * p.N), (short)0,
                                           __builtin_amdgcn_readfirstlane(p.N * 4), 0x00020000);
  } else {
    rE = __builtin_amdgcn_make_buffer_rsrc(uniform_ptr(p.entries + (int64_t)bu * p.N * 128), (short)0,
                                           __builtin_amdgcn_readfirstlane(p.N * 256), 0x00020000);
  }
  const int win_row0 = (int)(j0 - p.win_pos0);  // window source row of key j0

  // issue the loads of chunk c (entry indices ids for entry chunks)
  auto issue = [&](int c, const int ids[2], ChunkRegs& R) {
    const bool ent = c < n_ent_chunks;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      int row;
      if (ent) {
        row = ids[kt];
      } else {
        const int wj = (c - n_ent_chunks) * 32 + kt * 16 + l16;
        row = wj < n_wk ? win_row0 + wj : -1;
      }
      if (c >= c_hi) row = -1;
      R.v[kt] = row >= 0;
      R.sc[kt] = 1.0f;
      if (MODE == 3 && ent) {
        // the lane's dims ks*32 + 8g .. +7: 4 code bytes at 16 ks + 4 g; the
        // 8 block scales ride in words 1 and 2 of the first slot until the
        // chunk is dequantised
        const int o = row >= 0 ? row * 72 : kOOB;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          R.r[kt][ks] = u32x4{__builtin_amdgcn_raw_buffer_load_b32(rE, o + 16 * ks + 4 * g, 0, 0), 0u, 0u, 0u};
        const auto bs = __builtin_amdgcn_raw_buffer_load_b64(rE, o + 64, 0, 0);
        R.r[kt][0][1] = bs[0];
        R.r[kt][0][2] = bs[1];
        R.sc[kt] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rS, row >= 0 ? row * 4 : kOOB, 0, 0));
      } else if (MODE == 1 && ent) {
        const int oc = row >= 0 ? row * 64 + 8 * g : kOOB;
        const int orr = row >= 0 ? row * 128 + 16 * g : kOOB;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const auto cw = __builtin_amdgcn_raw_buffer_load_b64(rE, oc + ks * 32, 0, 0);
          R.r[kt][ks] = u32x4{cw[0], cw[1], 0u, 0u};
        }
#pragma unroll
        for (int ks = 2; ks < 4; ++ks) R.r[kt][ks] = __builtin_amdgcn_raw_buffer_load_b128(rR, orr + (ks - 2) * 64, 0, 0);
        R.sc[kt] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rS, row >= 0 ? row * 4 : kOOB, 0, 0));
      } else if (!ent && p.win_fp8) {
        // FP8 window row (post-RoPE): 8 code bytes of the lane's dims per slice
        const int off = row >= 0 ? row * 128 + 8 * g : kOOB;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const auto cw = __builtin_amdgcn_raw_buffer_load_b64(rW, off + ks * 32, 0, 0);
          R.r[kt][ks] = u32x4{cw[0], cw[1], 0u, 0u};
        }
        R.sc[kt] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rWS, row >= 0 ? row * 4 : kOOB, 0, 0));
      } else {
        const int off = row >= 0 ? row * 256 + 16 * g : kOOB;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          R.r[kt][ks] = __builtin_amdgcn_raw_buffer_load_b128(ent ? rE : rW, off + ks * 64, 0, 0);
      }
    }
  };
  // post-process a loaded chunk: fp8 dequantisation, window-row rotation
  auto finish = [&](int c, ChunkRegs& R) {
    if (c >= c_hi) return;
    if (MODE == 3 && c < n_ent_chunks) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const uint32_t blo = R.r[kt][0][1], bhi = R.r[kt][0][2];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const int blk = 2 * ks + (g >> 1);  // 16-dim block of dims ks*32 + 8g .. +7
          const uint32_t bcode = ((blk < 4 ? blo : bhi) >> (8 * (blk & 3))) & 255u;
          const float sb = e4m3_to_f32(bcode) * R.sc[kt];
          // the hardware conversion with scale 1 gives the two e2m1 values of
          // byte e exactly (low nibble first); the block and entry scale
          // follow in fp32
          const uint32_t w = R.r[kt][ks][0];
          const f32x2 v0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
          const f32x2 v1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
          const f32x2 v2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
          const f32x2 v3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
          R.r[kt][ks][0] = pack_bf16(v0[0] * sb, v0[1] * sb);
          R.r[kt][ks][1] = pack_bf16(v1[0] * sb, v1[1] * sb);
          R.r[kt][ks][2] = pack_bf16(v2[0] * sb, v2[1] * sb);
          R.r[kt][ks][3] = pack_bf16(v3[0] * sb, v3[1] * sb);
        }
      }
    }
    if (MODE == 1 && c < n_ent_chunks) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          // the hardware conversion with scale 1 gives two e4m3 values exactly
          // (bytes 0-1, or 2-3 with the word select); the entry scale follows
          const uint32_t w0 = R.r[kt][ks][0], w1 = R.r[kt][ks][1];
          const float sc = R.sc[kt];
          const f32x2 v0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w0, 1.0f, false);
          const f32x2 v1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w0, 1.0f, true);
          const f32x2 v2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w1, 1.0f, false);
          const f32x2 v3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w1, 1.0f, true);
          R.r[kt][ks][0] = pack_bf16(v0[0] * sc, v0[1] * sc);
          R.r[kt][ks][1] = pack_bf16(v1[0] * sc, v1[1] * sc);
          R.r[kt][ks][2] = pack_bf16(v2[0] * sc, v2[1] * sc);
          R.r[kt][ks][3] = pack_bf16(v3[0] * sc, v3[1] * sc);
        }
    }
    if (c >= n_ent_chunks && p.win_fp8) {
      // FP8 window rows: all four slices, already rotated
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const uint32_t w0 = R.r[kt][ks][0], w1 = R.r[kt][ks][1];
          const float sc = R.sc[kt];
          const f32x2 v0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w0, 1.0f, false);
          const f32x2 v1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w0, 1.0f, true);
          const f32x2 v2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w1, 1.0f, false);
          const f32x2 v3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w1, 1.0f, true);
          R.r[kt][ks][0] = pack_bf16(v0[0] * sc, v0[1] * sc);
          R.r[kt][ks][1] = pack_bf16(v1[0] * sc, v1[1] * sc);
          R.r[kt][ks][2] = pack_bf16(v2[0] * sc, v2[1] * sc);
          R.r[kt][ks][3] = pack_bf16(v3[0] * sc, v3[1] * sc);
        }
    } else if (c >= n_ent_chunks && p.rope && !p.win_roped) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        if (!R.v[kt]) continue;
        const double j = (double)(j0 + (c - n_ent_chunks) * 32 + kt * 16 + l16);
#pragma unroll
        for (int ks = 2; ks < 4; ++ks)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float cs, sn;
            rope_cs(j, p.rev[(ks - 2) * 16 + 4 * g + e], cs, sn);
            const float a0 = bf16lo(R.r[kt][ks][e]), a1 = bf16hi(R.r[kt][ks][e]);
            R.r[kt][ks][e] = pack_bf16(a0 * cs - a1 * sn, a0 * sn + a1 * cs);
          }
      }
    }
  };
  // S^T of a chunk from its registers (K operand) and store V rows to LDS
  auto scores = [&](const ChunkRegs& R, f32x4 S[2][NHT], uint32_t vmask[2], int buf) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      vmask[kt] = (uint32_t)(__builtin_amdgcn_ballot_w64(R.v[kt]) & 0xffffull);
#pragma unroll
      for (int ht = 0; ht < NHT; ++ht) S[kt][ht] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8 a = __builtin_bit_cast(bf16x8, R.r[kt][ks]);
#pragma unroll
        for (int ht = 0; ht < NHT; ++ht)
          S[kt][ht] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, Q[ht][ks], S[kt][ht], 0, 0, 0);
      }
    }
    uint16_t* vb = &Vs[buf][0];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        *(u32x4*)(vb + (kt * 16 + l16) * KP + ks * 32 + 8 * g) = R.r[kt][ks];
  };

  // ---- pipeline: rows of chunk c+1 load while chunk c is computed; entry
  // indices are fetched three chunks ahead of their rows
  for (;;) {
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) {
      // the sink weight belongs to one part only
      const float l0 = (p.sink && part == 0) ? __builtin_amdgcn_exp2f(skv[ht] * LOG2E - mref[ht]) : 0.0f;
      Lacc[ht] = f32x4{l0, l0, l0, l0};
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) O[dt][ht] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
    ChunkRegs R;
    {
      int i0[2];
      fetch_idx(c_lo, i0);
      issue(c_lo, i0, R);
    }
    bool again = false;
    for (int c = c_lo; c < c_hi; ++c) {
      f32x4 S[2][NHT];
      uint32_t msk[2];
      int inext[2];
      fetch_idx(c + 1, inext);
      finish(c, R);
      scores(R, S, msk, c & 1);
      issue(c + 1, inext, R);

      // ---- softmax weights of chunk c (log2 units); masked keys -> -inf
      if ((msk[0] & msk[1]) != 0xffffu) {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (!((msk[kt] >> (4 * g + i)) & 1u)) {
#pragma unroll
              for (int ht = 0; ht < NHT; ++ht) S[kt][ht][i] = NEG_INF;
            }
      }
      float lm[NHT];
      bool over = false;
#pragma unroll
      for (int ht = 0; ht < NHT; ++ht) {
        lm[ht] = fmaxf(fmaxf(fmaxf(S[0][ht][0], S[0][ht][1]), fmaxf(S[0][ht][2], S[0][ht][3])),
                       fmaxf(fmaxf(S[1][ht][0], S[1][ht][1]), fmaxf(S[1][ht][2], S[1][ht][3])));
        over |= lm[ht] > mref[ht] + kSlack;
      }
      if (__builtin_amdgcn_ballot_w64(over)) {
#pragma unroll
        for (int ht = 0; ht < NHT; ++ht) mref[ht] = fmaxf(mref[ht], max_over_groups(lm[ht]));
        again = true;
        break;
      }
      bf16x8 P[NHT];
#pragma unroll
      for (int ht = 0; ht < NHT; ++ht)
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            P[ht][kt * 4 + i] = (__bf16)__builtin_amdgcn_exp2f(S[kt][ht][i] - mref[ht]);

      // ---- O^T += V^T P^T (V^T by LDS transpose reads); L += 1^T P^T
      const uint16_t* vb = &Vs[c & 1][0];
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const int col = dt * 16 + 4 * (l16 & 3);
        const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            LDS_PTR(bf16x4, vb + (4 * g + (l16 >> 2)) * KP + col));
        const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            LDS_PTR(bf16x4, vb + (16 + 4 * g + (l16 >> 2)) * KP + col));
        const bf16x8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
        for (int ht = 0; ht < NHT; ++ht)
          O[dt][ht] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, P[ht], O[dt][ht], 0, 0, 0);
      }
#pragma unroll
      for (int ht = 0; ht < NHT; ++ht)
        Lacc[ht] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, P[ht], Lacc[ht], 0, 0, 0);

    }
    if (!again) break;
  }

  if constexpr (SPLIT) {
    // ---- partial results: O[h][d] unnormalised, then mref[h], L[h]
    float* w = p.ws + ((int64_t)(tok - p.tok0) * p.parts + part) * kAttendPartFloats;
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) {
      const int h = ht * 16 + l16;
      if (h >= p.H) continue;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) *(f32x4*)(w + h * 128 + dt * 16 + 4 * g) = O[dt][ht];
      if (g == 0) {
        w[64 * 128 + h] = mref[ht];
        w[64 * 128 + 64 + h] = Lacc[ht][0];
      }
    }
    return;
  }

  // ---- normalise, inverse RoPE on dims 64..127, store bf16
  float oc[8], os[8];
  if (p.rope) {
#pragma unroll
    for (int dd = 0; dd < 4; ++dd)
#pragma unroll
      for (int pp = 0; pp < 2; ++pp)
        rope_cs((double)t, p.rev[8 * dd + 2 * g + pp], oc[dd * 2 + pp], os[dd * 2 + pp]);
  }
#pragma unroll
  for (int ht = 0; ht < NHT; ++ht) {
    const int h = ht * 16 + l16;
    const float L = Lacc[ht][0];
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
    if (h >= p.H) continue;
    uint16_t* orow = p.out + (tok * p.H + h) * 128;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      float o0 = O[dt][ht][0] * inv, o1 = O[dt][ht][1] * inv;
      float o2 = O[dt][ht][2] * inv, o3 = O[dt][ht][3] * inv;
      if (p.rope && dt >= 4) {
        const int dd = dt - 4;
        const float c0 = oc[dd * 2], s0 = os[dd * 2], c1 = oc[dd * 2 + 1], s1 = os[dd * 2 + 1];
        const float r0 = o0 * c0 + o1 * s0, r1 = o1 * c0 - o0 * s0;
        const float r2 = o2 * c1 + o3 * s1, r3 = o3 * c1 - o2 * s1;
        o0 = r0; o1 = r1; o2 = r2; o3 = r3;
      }
      uint2 w;
      w.x = pack_bf16(o0, o1);
      w.y = pack_bf16(o2, o3);
      *(uint2*)(orow + dt * 16 + 4 * g) = w;
    }
  }
}

// ----------------------------------------------------------------------------
// bf16 entries (CSA) and HCA.  A work-group of NW waves serves one token; wave
// w takes head tiles w*NHT .. w*NHT + NHT - 1 (16 heads each), which keeps a
// wave under 256 registers so that two waves share each SIMD and one wave's
// MFMAs overlap the other's softmax.  The key rows stream through a ring of
// LDS chunk buffers filled by direct-to-LDS buffer loads (no registers in
// flight) kRing - 1 chunks ahead of the one being computed; the waves split
// each chunk's loads and meet at one barrier per chunk.  K (for S^T) and V^T
// both come from the ring.  A key row occupies 256 bytes; its 16-byte pieces
// are XOR-swizzled by the row's low 4 bits so that the K reads (16 rows, one
// piece each) and the transposing V reads avoid bank conflicts.  One load
// instruction fills 4 rows: lane l writes row 4q + l/16, piece l%16, and row
// 4q + h holds key 8h + q of the chunk, so a lane fetches the indices of 8
// consecutive keys.
constexpr int kRing = 3;

template <bool B>
struct PassTag {
  static constexpr bool value = B;
};

__device__ __forceinline__ int ring_key(int r) { return 8 * (r & 3) + (r >> 2); }  // key of ring row r

template <int S>
struct SlotTag {
  static constexpr int value = S;
};

// TOK query tokens per work-group (HCA only: they see the same entries and
// nearly the same window, so one ring serves them all); NW / TOK waves per
// token.
template <int NHT, int NW, int MODE, int TOK = 1>  // MODE 0: CSA bf16 entries, 2: HCA
__global__ __launch_bounds__(64 * NW) void attend_ring_kernel(AttendParams p) {
  static_assert(MODE == 2 || TOK == 1, "CSA tokens have their own key sets");
  constexpr int WPT = NW / TOK;  // waves per token
  __shared__ __attribute__((aligned(16))) uint8_t Ks[kRing][32 * 256];
  // CSA: the token's idx row, padded with -1 up to a multiple of 32 (an
  // index outside [0, N) is stored as -1: no key)
  __shared__ __attribute__((aligned(16))) int32_t Is[MODE == 2 ? 4 : kMaxK];
  __shared__ float2 Rt[TOK][32];  // (cos, sin) of each token's angle t * theta_f, f = 0..31
  __shared__ float Rv[32];        // theta_f / 2pi (revolutions per position)
  __shared__ int flag[2][NW];
  __shared__ int first_bad[NW];  // per wave: first idx position holding a missing key
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, l16 = lane & 15;
  const int nq = (p.n + TOK - 1) / TOK;  // work-groups per batch row
  const int b = (int)(blockIdx.x / nq);
  const int q_first = (int)(blockIdx.x % nq) * TOK;
  const int q_last = min(q_first + TOK, p.n) - 1;
  const int tw = wave / WPT;  // this wave's token slot
  const bool active = q_first + tw < p.n;
  const int qi = min(q_first + tw, p.n - 1);
  const int64_t tok = (int64_t)b * p.n + qi;
  const int64_t t = p.q_pos0 + qi;
  const int64_t t0 = p.q_pos0 + q_first, t_last = p.q_pos0 + q_last;
  const float LOG2E = 1.4426950408889634f;
  const int h0 = (wave % WPT) * NHT * 16;  // first head of this wave

  // ---- the tokens' rotations (angle formed in fp64) and the index row (CSA).
  // The ring needs no clearing: every chunk's loads rewrite all 32 rows (a
  // missing key's row reads as zeros).
  if (tid < 32 * TOK && p.rope) {
    const int ts = tid >> 5, f = tid & 31;
    float cs, sn;
    rope_cs((double)(p.q_pos0 + min(q_first + ts, p.n - 1)), p.rev[f], cs, sn);
    Rt[ts][f] = make_float2(cs, sn);
    if (ts == 0) Rv[f] = (float)p.rev[f];
  }
  const int kpad = (p.k + 31) & ~31;  // <= kMaxK (a multiple of 32)
  if (MODE == 0) {
    // every load is issued before the first is used (addresses clamped into
    // the row; positions past k become -1)
    const int32_t* irow = p.idx + tok * p.k;
    constexpr int kIt = kMaxK / (256 * NW);
    u32x4 v[kIt];
    if (p.k > 0 && (p.k & 3) == 0) {
#pragma unroll
      for (int it = 0; it < kIt; ++it) {
        const int i = 4 * tid + it * 256 * NW;
        const u32x4 x = *(const u32x4*)&irow[min(i, p.k - 4)];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[it][e] = (i + e < p.k && x[e] < (uint32_t)p.N) ? x[e] : 0xffffffffu;
      }
    } else if (p.k > 0) {
#pragma unroll
      for (int it = 0; it < kIt; ++it) {
        const int i = 4 * tid + it * 256 * NW;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t x = (uint32_t)irow[min(i + e, p.k - 1)];
          v[it][e] = (i + e < p.k && x < (uint32_t)p.N) ? x : 0xffffffffu;
        }
      }
    }
    int fb = kpad;
#pragma unroll
    for (int it = 0; it < kIt; ++it) {
      const int i = 4 * tid + it * 256 * NW;
      if (i < kpad) {
        *(u32x4*)&Is[i] = v[it];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if ((int)v[it][e] < 0 && i + e < fb) fb = i + e;
      }
    }
    for (int off = 32; off >= 1; off >>= 1) fb = min(fb, __shfl_xor(fb, off));
    if (lane == 0) first_bad[wave] = fb;
  }
  __syncthreads();

  // ---- Q^T operand: lane l holds head h0 + ht*16 + l16, dims ks*32 + 8g .. +7.
  // Every load is issued before the first is used (one memory round trip):
  // lanes past the last head read head H-1 and use zeros.
  bf16x8 Q[NHT][4];
  u32x4 qraw[NHT][4];
  float skv[NHT];  // the heads' sink logits (0 past the last head)
#pragma unroll
  for (int ht = 0; ht < NHT; ++ht) {
    const int hc = min(h0 + ht * 16 + l16, p.H - 1);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qraw[ht][ks] = *(const u32x4*)(p.q + ((tok * p.H + hc) * 128 + ks * 32 + 8 * g));
    skv[ht] = p.sink ? p.sink[hc] : 0.0f;
  }
#pragma unroll
  for (int ht = 0; ht < NHT; ++ht) {
    const int h = h0 + ht * 16 + l16;
    if (h >= p.H) skv[ht] = 0.0f;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      float x[8];
      if (h < p.H) {
        const u32x4 v = qraw[ht][ks];
#pragma unroll
        for (int e = 0; e < 4; ++e) { x[2 * e] = bf16lo(v[e]); x[2 * e + 1] = bf16hi(v[e]); }
        if (p.rope && ks >= 2) {
#pragma unroll
          for (int pp = 0; pp < 4; ++pp) {
            const float2 r = Rt[tw][(ks - 2) * 16 + 4 * g + pp];
            const float a0 = x[2 * pp], a1 = x[2 * pp + 1];
            x[2 * pp] = a0 * r.x - a1 * r.y;
            x[2 * pp + 1] = a0 * r.y + a1 * r.x;
          }
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = 0.0f;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) Q[ht][ks][e] = (__bf16)(x[e] * p.qscale);
    }
  }

  // ---- key sequence of the work-group: entry chunks, then window chunks
  // (with several tokens: the entries of the last one, then each token's own
  // window in WC chunks per token slot; each wave masks what its own token
  // does not see, so every token's keys sit in the same chunks as in a
  // one-token work-group)
  int n_ent, n_ent_tok;
  if (MODE == 2) {
    const int64_t nv = (t_last + 1) / p.m, nt = (t + 1) / p.m;
    n_ent = (int)(nv < p.N ? nv : p.N);
    n_ent_tok = (int)(nt < p.N ? nt : p.N);
  } else {
    n_ent = n_ent_tok = p.k;
  }
  n_ent = __builtin_amdgcn_readfirstlane(n_ent);  // uniform: keep the loop control scalar
  n_ent_tok = __builtin_amdgcn_readfirstlane(n_ent_tok);
  const int n_ent_chunks = (n_ent + 31) >> 5;
  // chunks before n_full hold 32 keys present for this wave's token (no mask to form)
  int n_full;
  if (MODE == 2) {
    n_full = n_ent_tok >> 5;
  } else {
    int fb = first_bad[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) fb = min(fb, first_bad[w]);
    n_full = __builtin_amdgcn_readfirstlane(fb) >> 5;
  }
  // token slot s: window keys j = j0s[s] + wj, wj in [0, nwks[s]) (the
  // positions max(0, t_s - n_win + 1) .. t_s); slots past the last token hold none
  int64_t j0s[TOK];
  int nwks[TOK];
  int WC = 0;  // window chunks per token slot
#pragma unroll
  for (int s = 0; s < TOK; ++s) {
    const int64_t ts = t0 + s;
    int64_t js = ts - p.n_win + 1;
    if (js < 0) js = 0;
    j0s[s] = js;
    nwks[s] = (p.n_win > 0 && q_first + s <= q_last) ? (int)(ts - js + 1) : 0;
    nwks[s] = __builtin_amdgcn_readfirstlane(nwks[s]);
    WC = max(WC, (nwks[s] + 31) >> 5);
  }
  const int n_chunks = n_ent_chunks + TOK * WC;

  auto uniform_ptr = [](const void* ptr) {
    const uint64_t v = (uint64_t)ptr;
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
    return (void*)(((uint64_t)hi << 32) | lo);
  };
  const int bu = __builtin_amdgcn_readfirstlane(b);
  const u32x4 rW = dma_rsrc(uniform_ptr(p.win ? p.win + (int64_t)bu * p.win_len * 128 : p.q),
                            p.win ? __builtin_amdgcn_readfirstlane(p.win_len * 256) : 0);
  const u32x4 rE = dma_rsrc(uniform_ptr(p.entries + (int64_t)bu * p.N * 128), __builtin_amdgcn_readfirstlane(p.N * 256));
  // window chunk c: its token slot and the window offset of its key 0
  auto win_chunk = [&](int c, int& s, int& wb) {
    const int cw = c - n_ent_chunks;
    s = (TOK == 1 || cw < WC) ? 0 : 1;
    wb = (cw - s * WC) * 32;
  };

  // This wave's share of the loads of chunk c into ring slot `slot`: load
  // instructions q = wave*QPW .. +QPW-1, each 4 rows.  Always issued: a
  // missing key has row -1, whose offset (0xffffff00 + piece) lies past every
  // row source and reads as zeros; so do chunks past the end.
  constexpr int QPW = 8 / NW;
  const int hq = lane >> 4;
  uint32_t colq[QPW];  // this lane's piece offset in load q (XOR swizzle of ring row 4q + hq)
#pragma unroll
  for (int e = 0; e < QPW; ++e) colq[e] = (uint32_t)(((lane & 15) ^ ((4 * (wave * QPW + e) + hq) & 15)) << 4);
  const uint32_t ks_lds = (uint32_t)__builtin_amdgcn_readfirstlane(
      (int)((uint32_t)(uintptr_t)LDS_PTR(uint8_t, &Ks[0][0]) + (uint32_t)(wave * QPW * 1024)));
  auto chunk_rows = [&](int c, int (&rows)[QPW]) {
    const int kb0 = c * 32 + 8 * hq + wave * QPW;  // key of this lane's first row
    if (c < n_ent_chunks) {
      if constexpr (MODE == 0) {
        // kb0 + QPW <= 32 * n_ent_chunks = kpad: inside the padded row
#pragma unroll
        for (int e0 = 0; e0 < QPW; e0 += 4) {
          const u32x4 v = *(const u32x4*)&Is[kb0 + e0];
#pragma unroll
          for (int e = 0; e < 4; ++e) rows[e0 + e] = (int)v[e];
        }
      } else {
#pragma unroll
        for (int e = 0; e < QPW; ++e) rows[e] = kb0 + e < n_ent ? kb0 + e : -1;
      }
    } else {
      int s, wb;
      win_chunk(c, s, wb);
      const int wrow0 = __builtin_amdgcn_readfirstlane((int)(j0s[s] - p.win_pos0));  // window source row of wj = 0
#pragma unroll
      for (int e = 0; e < QPW; ++e) {
        const int wj = wb + 8 * hq + wave * QPW + e;
        rows[e] = (c < n_chunks && wj < nwks[s]) ? wrow0 + wj : -1;
      }
    }
  };
  auto issue_rows = [&](int c, int slot, const int (&rows)[QPW]) {
    const u32x4 rs = c < n_ent_chunks ? rE : rW;
#pragma unroll
    for (int e = 0; e < QPW; ++e)
      dma_b128(rs, ks_lds + (uint32_t)(slot * 8192 + e * 1024), (int)(((uint32_t)rows[e] << 8) | colq[e]));
  };
  auto issue = [&](int c, int slot) {
    int rows[QPW];
    chunk_rows(c, rows);
    issue_rows(c, slot, rows);
  };
  // validity of ring rows r = 0..31 of chunk c (bit r)
  auto chunk_mask = [&](int c) -> uint32_t {
    if (c < n_full) return 0xffffffffu;
    const int r = lane & 31;
    const int kk = ring_key(r);
    bool v = false;
    if (c < n_ent_chunks) {
      const int e = c * 32 + kk;
      if (MODE == 2) v = e < n_ent_tok;
      else v = Is[e] >= 0;  // e < kpad; the padding is -1
    } else if (c < n_chunks) {
      int s, wb;
      win_chunk(c, s, wb);
      v = s == tw && wb + kk < nwks[s];
    }
    return (uint32_t)__builtin_amdgcn_ballot_w64(v && lane < 32);
  };
  // true on every wave if `mine` is true on some wave (flags double-buffered by `par`)
  int par = 0;
  auto any_wave = [&](bool mine) -> bool {
    if (lane == 0) flag[par][wave] = mine ? 1 : 0;
    __syncthreads();
    bool a = false;
#pragma unroll
    for (int w = 0; w < NW; ++w) a |= flag[par][w] != 0;
    par ^= 1;
    return a;
  };
  // wait for chunk c's rows (this wave's loads: only chunk c+1's may still be
  // outstanding); with several waves the barrier makes every wave's loads
  // visible and ends all reads of chunk c-1, whose slot is refilled right
  // after.  A single wave orders its own LDS accesses.
  auto arrive = [&]() {
    static_assert(QPW == 8 || QPW == 4 || QPW == 2, "loads per wave and chunk");
    if constexpr (QPW == 2) asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
    else if constexpr (QPW == 4) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
    if constexpr (NW > 1) __syncthreads();
  };
  // Window chunk c: rotate its rows in place in the ring (dims 64..127 of
  // each key at its position j = t_s - d, t_s the token of the chunk's
  // slot).  R(j) = R(t_s) R(-d) with d in [0, 127] taken in fp32 on the
  // hardware sin/cos.  The 32 rows x 8 pieces
  // of 16 bytes are shared out over the work-group; the caller synchronises.
  auto rotate_window = [&](int c, int slot) {
    for (int pi = tid; pi < 256; pi += 64 * NW) {
      const int r = pi >> 3, rp = pi & 7;
      uint8_t* ptr = &Ks[slot][0] + r * 256 + (((8 + rp) ^ (r & 15)) << 4);
      u32x4 w = *(const u32x4*)ptr;
      int s, wb;
      win_chunk(c, s, wb);
      // d = t_s - j: the slot's own token, as in a one-token work-group
      const float d = (float)((int)(t0 + s - j0s[s]) - (wb + ring_key(r)));
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int f = rp * 4 + e;
        float rv = d * Rv[f];
        rv = rv - __builtin_floorf(rv);
        const float sd = __builtin_amdgcn_sinf(rv), cd = __builtin_amdgcn_cosf(rv);
        const float2 rt = Rt[s][f];
        const float cs = rt.x * cd + rt.y * sd, sn = rt.y * cd - rt.x * sd;  // angle t_s - d = j
        const float a0 = bf16lo(w[e]), a1 = bf16hi(w[e]);
        w[e] = pack_bf16(a0 * cs - a1 * sn, a0 * sn + a1 * cs);
      }
      *(u32x4*)ptr = w;
    }
  };
  // K operand of a chunk: rows kt*16 + l16, dims ks*32 + 8g .. +7
  auto load_k = [&](const uint8_t* kb, bf16x8 (&K)[2][4]) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        K[kt][ks] = *(const bf16x8*)(kb + (kt * 16 + l16) * 256 + (((ks * 4 + g) ^ l16) << 4));
  };

  // ---- softmax reference per head (log2 units): the sink logit, or 0
  // without a sink.  The pass seeds the S accumulators with -mref (MFMA C
  // operand) and takes weights exp2(S) with no per-chunk test.  If on some
  // head the row sum left [2^-100, 2^100) (a weight overflowed, or all
  // underflowed), a max-only pass sets that head's mref to the exact maximum
  // of its sink and scores, after which its weights are <= 1, and the pass
  // reruns.  The other heads keep their reference and recompute the same
  // bits, so a head's result never depends on the other heads or tokens.
  float mref[NHT];
  bool badh[NHT];  // this lane's heads whose row sum left the range
#pragma unroll
  for (int ht = 0; ht < NHT; ++ht) mref[ht] = p.sink ? skv[ht] * LOG2E : 0.0f;
  bf16x8 ones;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones[e] = (__bf16)1.0f;
  f32x4 O[8][NHT], Lacc[NHT];

  // one pass over every chunk; returns true (on every wave) if some head's
  // row sum left [2^-100, 2^100)
  auto run = [&]() -> bool {
    f32x4 Cneg[NHT];
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) {
      const float l0 = p.sink ? __builtin_amdgcn_exp2f(skv[ht] * LOG2E - mref[ht]) : 0.0f;
      Lacc[ht] = f32x4{l0, l0, l0, l0};
      Cneg[ht] = f32x4{-mref[ht], -mref[ht], -mref[ht], -mref[ht]};
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) O[dt][ht] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
    // chunk c in ring slot c % kRing; the loop is unrolled kRing times so that
    // every slot address is a constant
    // The rows of chunk c+2's loads were read from the index row one chunk
    // earlier, so the loads issue without waiting on LDS; the K reads of the
    // chunk go out first.
    int rows_next[QPW];
    auto body = [&](int c, auto tag) {
      constexpr int slot = decltype(tag)::value;
      arrive();
      const uint8_t* kb = &Ks[slot][0];
      if (c >= n_ent_chunks && p.rope && !p.win_roped) {
        rotate_window(c, slot);
        __syncthreads();  // rotated rows visible to every wave
      }
      bf16x8 K[2][4];
      load_k(kb, K);
      issue_rows(c + 2, (slot + 2) % kRing, rows_next);
      chunk_rows(c + 3, rows_next);
      const uint32_t msk = chunk_mask(c);
      // no key of this chunk is this wave's (another token's window, entries
      // past the token's count, index padding): it would add exact zeros
      if (msk == 0u) return;

      // ---- S^T = K Q^T - mref; weights exp2
      f32x4 S[2][NHT];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
        for (int ht = 0; ht < NHT; ++ht)
          S[kt][ht] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(K[kt][0], Q[ht][0], Cneg[ht], 0, 0, 0);
#pragma unroll
        for (int ks = 1; ks < 4; ++ks)
#pragma unroll
          for (int ht = 0; ht < NHT; ++ht)
            S[kt][ht] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(K[kt][ks], Q[ht][ks], S[kt][ht], 0, 0, 0);
      }
      // V^T by transposing LDS reads, four 16-dim tiles ahead of their
      // MFMAs: the first four are read before the exponentials, each later
      // one right after the MFMAs of the tile whose registers it takes
      auto vread = [&](int dt) {
        const int vrow = 4 * g + (l16 >> 2);
        const int piece = ((dt * 2 + ((l16 & 3) >> 1)) ^ vrow) & 15;  // (vrow + 16) & 15 == vrow & 15
        const int boff = (piece << 4) + ((l16 & 1) << 3);
        const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(LDS_PTR(bf16x4, kb + vrow * 256 + boff));
        const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(LDS_PTR(bf16x4, kb + (vrow + 16) * 256 + boff));
        return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      };
      bf16x8 Vt[4];
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) Vt[dt] = vread(dt);
      bf16x8 P[NHT];
#pragma unroll
      for (int ht = 0; ht < NHT; ++ht)
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int i = 0; i < 4; ++i) P[ht][kt * 4 + i] = (__bf16)__builtin_amdgcn_exp2f(S[kt][ht][i]);
      // ---- O^T += V^T P^T; L += 1^T P^T
      auto pv = [&](const bf16x8 (&Pw)[NHT]) {
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
#pragma unroll
          for (int ht = 0; ht < NHT; ++ht)
            O[dt][ht] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Vt[dt % 4], Pw[ht], O[dt][ht], 0, 0, 0);
          if (dt + 4 < 8) Vt[dt % 4] = vread(dt + 4);
        }
#pragma unroll
        for (int ht = 0; ht < NHT; ++ht)
          Lacc[ht] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, Pw[ht], Lacc[ht], 0, 0, 0);
      };
      if (msk != 0xffffffffu) {
        u32x4 keepw;
#pragma unroll
        for (int w2 = 0; w2 < 4; ++w2) {
          const int e = 2 * w2;
          const int r0 = (e >> 2) * 16 + 4 * g + (e & 3);
          keepw[w2] = (((msk >> r0) & 1u) ? 0x0000ffffu : 0u) | (((msk >> (r0 + 1)) & 1u) ? 0xffff0000u : 0u);
        }
        // in place (tied asm operands): the weights stay in the registers the
        // unmasked path uses, so the common path copies nothing
#pragma unroll
        for (int ht = 0; ht < NHT; ++ht) {
          u32x4 pu = __builtin_bit_cast(u32x4, P[ht]);
#pragma unroll
          for (int w2 = 0; w2 < 4; ++w2) asm volatile("v_and_b32 %0, %0, %1" : "+v"(pu[w2]) : "v"(keepw[w2]));
          P[ht] = __builtin_bit_cast(bf16x8, pu);
        }
      }
      pv(P);
    };
    static_assert(kRing == 3, "the chunk loop is unrolled over 3 ring slots");
    issue(0, 0);
    issue(1, 1);
    chunk_rows(2, rows_next);
    for (int c = 0; c < n_chunks; c += 3) {
      body(c, SlotTag<0>{});
      if (c + 1 < n_chunks) body(c + 1, SlotTag<1>{});
      if (c + 2 < n_chunks) body(c + 2, SlotTag<2>{});
    }
    // every load into the ring has landed before the ring is reused or released
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    bool bad = false;
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) {
      badh[ht] = !(Lacc[ht][0] < 0x1p100f && Lacc[ht][0] >= 0x1p-100f);
      bad |= badh[ht];
    }
    return any_wave(__builtin_amdgcn_ballot_w64(bad) != 0);
  };
  // max-only pass: mref = max(sink logit, every valid score) per head
  auto run_max = [&]() {
    float m[NHT];
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) m[ht] = p.sink ? skv[ht] * LOG2E : -__builtin_inff();
    __syncthreads();  // every wave is done with the ring
    issue(0, 0);
    issue(1, 1);
    int slot = 0, slot_next = 2;
    for (int c = 0; c < n_chunks; ++c) {
      arrive();
      issue(c + 2, slot_next);
      const uint32_t msk = chunk_mask(c);
      if (c >= n_ent_chunks && p.rope && !p.win_roped) {
        rotate_window(c, slot);
        __syncthreads();  // rotated rows visible to every wave
      }
      bf16x8 K[2][4];
      load_k(&Ks[slot][0], K);
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        f32x4 S2[NHT];
#pragma unroll
        for (int ht = 0; ht < NHT; ++ht)
          S2[ht] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(K[kt][0], Q[ht][0], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
        for (int ks = 1; ks < 4; ++ks)
#pragma unroll
          for (int ht = 0; ht < NHT; ++ht)
            S2[ht] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(K[kt][ks], Q[ht][ks], S2[ht], 0, 0, 0);
#pragma unroll
        for (int ht = 0; ht < NHT; ++ht)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if ((msk >> (kt * 16 + 4 * g + i)) & 1u) m[ht] = fmaxf(m[ht], S2[ht][i]);
      }
      slot = slot == kRing - 1 ? 0 : slot + 1;
      slot_next = slot_next == kRing - 1 ? 0 : slot_next + 1;
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();  // every wave is done with the ring before the rerun refills it
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) {
      const float mx = fmaxf(max_over_groups(m[ht]), -1e30f);
      if (badh[ht]) mref[ht] = mx;
    }
  };
  if (run()) {
    run_max();
    run();
  }

  // ---- normalise, inverse RoPE on dims 64..127 (by -t), store bf16
#pragma unroll
  for (int ht = 0; ht < NHT; ++ht) {
    const int h = h0 + ht * 16 + l16;
    const float L = Lacc[ht][0];
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
    if (h >= p.H || !active) continue;
    uint16_t* orow = p.out + (tok * p.H + h) * 128;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      float o0 = O[dt][ht][0] * inv, o1 = O[dt][ht][1] * inv;
      float o2 = O[dt][ht][2] * inv, o3 = O[dt][ht][3] * inv;
      if (p.rope && dt >= 4) {
        const float2 r0c = Rt[tw][8 * (dt - 4) + 2 * g], r1c = Rt[tw][8 * (dt - 4) + 2 * g + 1];
        const float r0 = o0 * r0c.x + o1 * r0c.y, r1 = o1 * r0c.x - o0 * r0c.y;
        const float r2 = o2 * r1c.x + o3 * r1c.y, r3 = o3 * r1c.x - o2 * r1c.y;
        o0 = r0; o1 = r1; o2 = r2; o3 = r3;
      }
      uint2 w;
      w.x = pack_bf16(o0, o1);
      w.y = pack_bf16(o2, o3);
      *(uint2*)(orow + dt * 16 + 4 * g) = w;
    }
  }
}

template <int MODE>
static hipError_t launch_ring(const AttendParams& p, hipStream_t stream) {
  const int nht = (p.H + 15) / 16;
  const int64_t bn = (int64_t)p.B * p.n;
  // HCA: two tokens per work-group share the ring when every token sees at
  // least 512 entries (the pair's one extra window chunk is then a small
  // price for halving the row loads) and enough work-groups remain to fill
  // the chip
  int64_t ent0 = p.m > 0 ? (p.q_pos0 + 1) / p.m : 0;
  if (ent0 > p.N) ent0 = p.N;
  const bool pair = MODE == 2 && nht > 2 && bn >= 4096 && ent0 >= 512;
  dim3 grid((unsigned)(pair ? (int64_t)p.B * ((p.n + 1) / 2) : bn));
  // up to 32 heads: one wave; more: two waves of up to 32 heads each
  switch (nht) {
    case 1: hipLaunchKernelGGL((attend_ring_kernel<1, 1, MODE>), grid, dim3(64), 0, stream, p); break;
    case 2: hipLaunchKernelGGL((attend_ring_kernel<2, 1, MODE>), grid, dim3(64), 0, stream, p); break;
    case 3:
    case 4:
      if constexpr (MODE == 2) {
        if (pair) {
          hipLaunchKernelGGL((attend_ring_kernel<2, 4, MODE, 2>), grid, dim3(256), 0, stream, p);
          break;
        }
      }
      hipLaunchKernelGGL((attend_ring_kernel<2, 2, MODE>), grid, dim3(128), 0, stream, p);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Split decode, second kernel: work-group (token, 8 heads), thread (head h,
// 4 dims) merges the parts in ascending order: O = sum_p O_p 2^(m_p - M), L
// likewise, with M the largest part reference; then normalise, inverse
// RoPE, store bf16.  The parts are read kCombineBatch at a time, every load
// of a batch issued before the first use.
constexpr int kCombineBatch = 16;
__global__ __launch_bounds__(256) void attend_combine_kernel(AttendParams p) {
  const int64_t tok = p.tok0 + (blockIdx.x >> 3);
  const int h = (int)(blockIdx.x & 7) * 8 + (threadIdx.x >> 5), d0 = (threadIdx.x & 31) * 4;
  if (h >= p.H) return;
  const float* w0 = p.ws + (tok - p.tok0) * p.parts * kAttendPartFloats;
  float M = -__builtin_inff();
  for (int q0 = 0; q0 < p.parts; q0 += kCombineBatch) {
    float mq[kCombineBatch];
#pragma unroll
    for (int u = 0; u < kCombineBatch; ++u)
      mq[u] = q0 + u < p.parts ? w0[(q0 + u) * kAttendPartFloats + 64 * 128 + h] : -__builtin_inff();
#pragma unroll
    for (int u = 0; u < kCombineBatch; ++u) M = fmaxf(M, mq[u]);
  }
  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  float L = 0.0f;
  for (int q0 = 0; q0 < p.parts; q0 += kCombineBatch) {
    float mq[kCombineBatch], lq[kCombineBatch];
    f32x4 vq[kCombineBatch];
#pragma unroll
    for (int u = 0; u < kCombineBatch; ++u) {
      lq[u] = 0.0f;
      if (q0 + u < p.parts) {
        const float* w = w0 + (q0 + u) * kAttendPartFloats;
        mq[u] = w[64 * 128 + h];
        lq[u] = w[64 * 128 + 64 + h];
        vq[u] = *(const f32x4*)(w + h * 128 + d0);
      }
    }
#pragma unroll
    for (int u = 0; u < kCombineBatch; ++u) {
      if (!(lq[u] > 0.0f)) continue;  // no keys and no sink in this part (or past the last)
      const float sc = __builtin_amdgcn_exp2f(mq[u] - M);
      L = __builtin_fmaf(lq[u], sc, L);
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = __builtin_fmaf(vq[u][i], sc, acc[i]);
    }
  }
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;
  const int64_t t = p.q_pos0 + (int)(tok % p.n);
  uint32_t o[2];
#pragma unroll
  for (int e = 0; e < 4; e += 2) {
    float o0 = acc[e] * inv, o1 = acc[e + 1] * inv;
    if (p.rope && d0 >= 64) {
      float c, s;
      rope_cs((double)t, p.rev[(d0 + e - 64) >> 1], c, s);
      const float r0 = o0 * c + o1 * s, r1 = o1 * c - o0 * s;
      o0 = r0;
      o1 = r1;
    }
    o[e >> 1] = pack_bf16(o0, o1);
  }
  *(uint2*)(p.out + (tok * p.H + h) * 128 + d0) = make_uint2(o[0], o[1]);
}

template <int MODE>
static hipError_t launch_mode(const AttendParams& p_in, hipStream_t stream) {
  const int nht = (p_in.H + 15) / 16;
  const bool split = (MODE == 1 || MODE == 3) && p_in.ws != nullptr && p_in.parts > 1;
  const int64_t bn = (int64_t)p_in.B * p_in.n;
  if (split) {
    // blocks of at most kAttendSplitTokens tokens through the workspace, in order
    AttendParams p = p_in;
    for (int64_t tok0 = 0; tok0 < bn; tok0 += kAttendSplitTokens) {
      const int64_t cnt = bn - tok0 < kAttendSplitTokens ? bn - tok0 : kAttendSplitTokens;
      p.tok0 = tok0;
      dim3 grid((unsigned)(cnt * p.parts)), block(64);
      switch (nht) {
        case 1: hipLaunchKernelGGL((attend_kernel<1, MODE, true>), grid, block, 0, stream, p); break;
        case 2: hipLaunchKernelGGL((attend_kernel<2, MODE, true>), grid, block, 0, stream, p); break;
        case 3: hipLaunchKernelGGL((attend_kernel<3, MODE, true>), grid, block, 0, stream, p); break;
        case 4: hipLaunchKernelGGL((attend_kernel<4, MODE, true>), grid, block, 0, stream, p); break;
        default: return hipErrorInvalidValue;
      }
      hipLaunchKernelGGL(attend_combine_kernel, dim3((unsigned)(cnt * 8)), dim3(256), 0, stream, p);
    }
    return hipGetLastError();
  }
  const AttendParams& p = p_in;
  dim3 grid((unsigned)bn), block(64);
  switch (nht) {
    case 1: hipLaunchKernelGGL((attend_kernel<1, MODE>), grid, block, 0, stream, p); break;
    case 2: hipLaunchKernelGGL((attend_kernel<2, MODE>), grid, block, 0, stream, p); break;
    case 3: hipLaunchKernelGGL((attend_kernel<3, MODE>), grid, block, 0, stream, p); break;
    case 4: hipLaunchKernelGGL((attend_kernel<4, MODE>), grid, block, 0, stream, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// FP8 or NVFP4 entries over long key lists: each token's chunks are split
// over several work-groups (decode: one work-group per token would leave
// most CUs idle).  The choice depends on the token's own key count only, so
// a token's result is the same whatever else is in the call.
static int attend_parts(int mode, int k, int n_win) {
  if (mode != 1 && mode != 3) return 1;
  const int chunks = (k + 31) / 32 + (n_win + 31) / 32;
  if (chunks < 2 * kAttendChunksPerPart) return 1;
  return (chunks + kAttendChunksPerPart - 1) / kAttendChunksPerPart;
}

size_t attend_workspace(int mode, int B, int n, int k, int n_win) {
  const int parts = attend_parts(mode, k, n_win);
  if (parts <= 1) return 0;
  int64_t bn = (int64_t)B * n;
  if (bn > kAttendSplitTokens) bn = kAttendSplitTokens;
  return (size_t)bn * parts * kAttendPartFloats * sizeof(float);
}

hipError_t launch_attend(const AttendParams& p_in, int mode, hipStream_t stream) {
  if ((int64_t)p_in.B * p_in.n == 0) return hipSuccess;
  AttendParams p = p_in;
  p.parts = attend_parts(mode, p.k, p.n_win);
  p.tok0 = 0;
  p.cpp = kAttendChunksPerPart;
  switch (mode) {
    case 0: return launch_ring<0>(p, stream);
    case 1: return launch_mode<1>(p, stream);
    case 3: return launch_mode<3>(p, stream);
    case 2: return launch_ring<2>(p, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace csa
