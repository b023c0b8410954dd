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

struct ChunkRegs {
  u32x4 r[2][4];  // key tile kt (rows kt*16 + l%16), dims ks*32 + 8*(l/16) .. +7
  float sc[2];    // fp8 entry scale per key tile
  bool v[2];      // key validity
};

template <int NHT, int MODE>  // MODE 0: CSA bf16 entries, 1: CSA fp8+bf16 entries, 2: HCA
__global__ __launch_bounds__(64) void attend_kernel(AttendParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t Vs[2][32 * KP];
  const int lane = threadIdx.x;
  const int g = lane >> 4, l16 = lane & 15;
  const int64_t tok = blockIdx.x;  // b * n + q
  const int b = (int)(tok / p.n);
  const int qi = (int)(tok % p.n);
  const int64_t t = p.q_pos0 + qi;
  const float LOG2E = 1.4426950408889634f;
  const float NEG_INF = -__builtin_inff();

  // ---- Q^T operand: lane l holds head ht*16+l16, dims ks*32 + 8g .. +7
  bf16x8 Q[NHT][4];
  {
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
          const u32x4 v = *(const u32x4*)(p.q + ((tok * p.H + h) * 128 + ks * 32 + 8 * g));
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
  for (int ht = 0; ht < NHT; ++ht) {
    const int h = ht * 16 + l16;
    mref[ht] = p.sink ? (h < p.H ? p.sink[h] : 0.0f) * LOG2E : -1e30f;
  }
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

  // entry index of this lane's key kt in chunk c (-1: none); CSA reads idx
  auto fetch_idx = [&](int c, int out[2]) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const int kk = c * 32 + kt * 16 + l16;
      int s = -1;
      if (c < n_ent_chunks) {
        if (MODE == 2) s = kk < n_ent ? kk : -1;
        else if (kk < p.k) s = p.idx[tok * p.k + kk];
      }
      out[kt] = s;
    }
  };
  // issue the loads of chunk c (entry indices ids for entry chunks)
  auto issue = [&](int c, const int ids[2], ChunkRegs& R) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      R.v[kt] = false;
      R.sc[kt] = 1.0f;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) R.r[kt][ks] = u32x4{0u, 0u, 0u, 0u};
      if (c >= n_chunks) continue;
      if (c < n_ent_chunks) {
        const int s = ids[kt];
        if (s < 0) continue;
        R.v[kt] = true;
        if (MODE == 1) {
          const int64_t row = (int64_t)b * p.N + s;
          const uint8_t* codes = (const uint8_t*)p.entries + row * 64 + 8 * g;
          const uint16_t* rope = p.entries_rope + row * 64 + 8 * g;
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            const uint2 cw = *(const uint2*)(codes + ks * 32);
            R.r[kt][ks][0] = cw.x;
            R.r[kt][ks][1] = cw.y;
          }
#pragma unroll
          for (int ks = 2; ks < 4; ++ks) R.r[kt][ks] = *(const u32x4*)(rope + (ks - 2) * 32);
          R.sc[kt] = p.entry_scale[row];
        } else {
          const uint16_t* src = p.entries + ((int64_t)b * p.N + s) * 128 + 8 * g;
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) R.r[kt][ks] = *(const u32x4*)(src + ks * 32);
        }
      } else {
        const int wj = (c - n_ent_chunks) * 32 + kt * 16 + l16;
        if (wj >= n_wk) continue;
        R.v[kt] = true;
        const uint16_t* src = p.win + ((int64_t)b * p.win_len + (j0 + wj - p.win_pos0)) * 128 + 8 * g;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) R.r[kt][ks] = *(const u32x4*)(src + ks * 32);
      }
    }
  };
  // post-process a loaded chunk: fp8 dequantisation, window-row rotation
  auto finish = [&](int c, ChunkRegs& R) {
    if (c >= n_chunks) return;
    if (MODE == 1 && c < n_ent_chunks) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const uint32_t w0 = R.r[kt][ks][0], w1 = R.r[kt][ks][1];
          const float sc = R.sc[kt];
          R.r[kt][ks][0] = pack_bf16(e4m3_to_f32(w0 & 255u) * sc, e4m3_to_f32((w0 >> 8) & 255u) * sc);
          R.r[kt][ks][1] = pack_bf16(e4m3_to_f32((w0 >> 16) & 255u) * sc, e4m3_to_f32(w0 >> 24) * sc);
          R.r[kt][ks][2] = pack_bf16(e4m3_to_f32(w1 & 255u) * sc, e4m3_to_f32((w1 >> 8) & 255u) * sc);
          R.r[kt][ks][3] = pack_bf16(e4m3_to_f32((w1 >> 16) & 255u) * sc, e4m3_to_f32(w1 >> 24) * sc);
        }
    }
    if (c >= n_ent_chunks && p.rope) {
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
      vmask[kt] = (uint32_t)(__ballot(R.v[kt]) & 0xffffull);
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
      const int h = ht * 16 + l16;
      const float l0 = p.sink ? __builtin_amdgcn_exp2f((h < p.H ? p.sink[h] : 0.0f) * LOG2E - mref[ht]) : 0.0f;
      Lacc[ht] = f32x4{l0, l0, l0, l0};
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) O[dt][ht] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
    int idx1[2], idx2[2], idx3[2], idx4[2];
    ChunkRegs R;
    {
      int i0[2];
      fetch_idx(0, i0);
      fetch_idx(1, idx1);
      fetch_idx(2, idx2);
      fetch_idx(3, idx3);
      issue(0, i0, R);
    }
    bool again = false;
    for (int c = 0; c < n_chunks; ++c) {
      f32x4 S[2][NHT];
      uint32_t msk[2];
      finish(c, R);
      scores(R, S, msk, c & 1);
      issue(c + 1, idx1, R);
      fetch_idx(c + 4, idx4);

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
      if (__ballot(over)) {
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

      idx1[0] = idx2[0]; idx1[1] = idx2[1];
      idx2[0] = idx3[0]; idx2[1] = idx3[1];
      idx3[0] = idx4[0]; idx3[1] = idx4[1];
    }
    if (!again) break;
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

template <int MODE>
static hipError_t launch_mode(const AttendParams& p, hipStream_t stream) {
  const int nht = (p.H + 15) / 16;
  dim3 grid((unsigned)((int64_t)p.B * p.n)), block(64);
  switch (nht) {
    case 1: hipLaunchKernelGGL((attend_kernel<1, MODE>), grid, block, 0, stream, p); break;
    case 2: hipLaunchKernelGGL((attend_kernel<2, MODE>), grid, block, 0, stream, p); break;
    case 3: hipLaunchKernelGGL((attend_kernel<3, MODE>), grid, block, 0, stream, p); break;
    case 4: hipLaunchKernelGGL((attend_kernel<4, MODE>), grid, block, 0, stream, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_attend(const AttendParams& p, int mode, hipStream_t stream) {
  if ((int64_t)p.B * p.n == 0) return hipSuccess;
  switch (mode) {
    case 0: return launch_mode<0>(p, stream);
    case 1: return launch_mode<1>(p, stream);
    case 2: return launch_mode<2>(p, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace csa
