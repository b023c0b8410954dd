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
// Every key row staged in LDS is therefore read once per 64 heads.  The
// transposed form leaves P^T in registers in exactly the B-operand layout of
// the PV product (keys 4g..4g+3 and 16+4g..16+4g+3 of head l%16 in lane l),
// so P never goes through LDS; the matching V^T operand comes straight from
// the row-major key tile with ds_read_b64_tr_b16.  Keys arrive in chunks of
// 32 rows: gathered entry rows (CSA: idx list; HCA: every visible entry),
// then the window rows, rotated at their own positions while being staged.
// The softmax scale 1/sqrt(D) and log2(e) are folded into q so scores are
// in log2 units; the sink initialises the running max and sum.
#include "device.h"
#include "kernels.h"

namespace csa {

constexpr int KP = 136;  // LDS row pitch in bf16 (272 bytes: 16-byte skew per row)

template <int NHT, int MODE>  // MODE 0: CSA bf16 entries, 1: CSA fp8+bf16 entries, 2: HCA
__global__ __launch_bounds__(64) void attend_kernel(AttendParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t Ks[32 * KP];
  const int lane = threadIdx.x;
  const int g = lane >> 4, l16 = lane & 15;
  const int64_t tok = blockIdx.x;  // b * n + q
  const int b = (int)(tok / p.n);
  const int qi = (int)(tok % p.n);
  const int64_t t = p.q_pos0 + qi;
  const float LOG2E = 1.4426950408889634f;
  const float NEG_INF = -__builtin_inff();

  // ---- Q^T operand: lane l holds head ht*16+l16, dims ks*32 + 8g .. +7
  float qc[8], qs[8];  // rotation of the pairs this lane holds in ks = 2, 3
  if (p.rope) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int pp = 0; pp < 4; ++pp) rope_cs((double)t, p.rev[kk * 16 + 4 * g + pp], qc[kk * 4 + pp], qs[kk * 4 + pp]);
  }
  bf16x8 Q[NHT][4];
#pragma unroll
  for (int ht = 0; ht < NHT; ++ht) {
    const int h = ht * 16 + l16;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      float x[8];
      if (h < p.H) {
        u32x4 v = *(const u32x4*)(p.q + ((tok * p.H + h) * 128 + ks * 32 + 8 * g));
#pragma unroll
        for (int e = 0; e < 4; ++e) { x[2 * e] = bf16lo(v[e]); x[2 * e + 1] = bf16hi(v[e]); }
        if (p.rope && ks >= 2) {
#pragma unroll
          for (int pp = 0; pp < 4; ++pp) {
            float c = qc[(ks - 2) * 4 + pp], s = qs[(ks - 2) * 4 + pp];
            float a0 = x[2 * pp], a1 = x[2 * pp + 1];
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

  // ---- softmax state (per lane: one head per head tile; groups g hold key subsets)
  float mrow[NHT], lsum[NHT];
  f32x4 O[8][NHT];
#pragma unroll
  for (int ht = 0; ht < NHT; ++ht) {
    const int h = ht * 16 + l16;
    if (p.sink) {
      mrow[ht] = (h < p.H ? p.sink[h] : 0.0f) * LOG2E;
      lsum[ht] = (g == 0) ? 1.0f : 0.0f;  // exp2(sink - m) = 1, counted once per head
    } else {
      mrow[ht] = -1e30f;
      lsum[ht] = 0.0f;
    }
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) O[dt][ht] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  }

  // ---- key sequence: entry chunks, then window chunks
  int n_ent;
  if (MODE == 2) {
    int64_t nv = (t + 1) / p.m;
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
  const int key = lane >> 1, h2 = lane & 1;
  uint16_t* krow = Ks + key * KP;

  for (int c = 0; c < n_chunks; ++c) {
    u32x4 v[8];  // dims [h2*32, +32) in v[0..3], [64+h2*32, +32) in v[4..7]
    bool valid;
    if (c < n_ent_chunks) {
      const int kk = c * 32 + key;
      int64_t s;
      if (MODE == 2) {
        s = kk;
        valid = kk < n_ent;
      } else {
        s = (kk < p.k) ? p.idx[tok * p.k + kk] : -1;
        valid = s >= 0;
      }
      if (valid) {
        if (MODE == 1) {
          const uint8_t* codes = (const uint8_t*)p.entries + ((int64_t)b * p.N + s) * 64 + h2 * 32;
          const float sc = p.entry_scale[(int64_t)b * p.N + s];
          u32x4 c0 = *(const u32x4*)codes, c1 = *(const u32x4*)(codes + 16);
          uint32_t cw[8] = {c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3]};
#pragma unroll
          for (int w = 0; w < 8; ++w) {
            uint32_t x = cw[w];
            float f0 = e4m3_to_f32(x & 255u) * sc, f1 = e4m3_to_f32((x >> 8) & 255u) * sc;
            float f2 = e4m3_to_f32((x >> 16) & 255u) * sc, f3 = e4m3_to_f32(x >> 24) * sc;
            v[w >> 1][(w & 1) * 2 + 0] = pack_bf16(f0, f1);
            v[w >> 1][(w & 1) * 2 + 1] = pack_bf16(f2, f3);
          }
          const u32x4* rp = (const u32x4*)(p.entries_rope + ((int64_t)b * p.N + s) * 64 + h2 * 32);
#pragma unroll
          for (int i = 0; i < 4; ++i) v[4 + i] = rp[i];
        } else {
          const u32x4* src = (const u32x4*)(p.entries + ((int64_t)b * p.N + s) * 128);
#pragma unroll
          for (int i = 0; i < 4; ++i) { v[i] = src[h2 * 4 + i]; v[4 + i] = src[8 + h2 * 4 + i]; }
        }
      }
    } else {
      const int wj = (c - n_ent_chunks) * 32 + key;
      valid = wj < n_wk;
      if (valid) {
        const int64_t j = j0 + wj;
        const u32x4* src = (const u32x4*)(p.win + ((int64_t)b * p.win_len + (j - p.win_pos0)) * 128);
#pragma unroll
        for (int i = 0; i < 4; ++i) { v[i] = src[h2 * 4 + i]; v[4 + i] = src[8 + h2 * 4 + i]; }
        if (p.rope) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int f = h2 * 16 + i * 4 + e;  // pair (64+2f, 65+2f)
              float cs, sn;
              rope_cs((double)j, p.rev[f], cs, sn);
              float a0 = bf16lo(v[4 + i][e]), a1 = bf16hi(v[4 + i][e]);
              v[4 + i][e] = pack_bf16(a0 * cs - a1 * sn, a0 * sn + a1 * cs);
            }
        }
      }
    }
    if (!valid) {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = u32x4{0u, 0u, 0u, 0u};
    }
    const uint64_t bal = __ballot(valid);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *(u32x4*)(krow + h2 * 32 + 8 * i) = v[i];
      *(u32x4*)(krow + 64 + h2 * 32 + 8 * i) = v[4 + i];
    }
    __syncthreads();

    // ---- S^T = K Q^T  (2 key tiles x NHT head tiles)
    f32x4 S[2][NHT];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int ht = 0; ht < NHT; ++ht) S[kt][ht] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        bf16x8 a = *(const bf16x8*)(Ks + (kt * 16 + l16) * KP + ks * 32 + 8 * g);
#pragma unroll
        for (int ht = 0; ht < NHT; ++ht)
          S[kt][ht] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, Q[ht][ks], S[kt][ht], 0, 0, 0);
      }
    }
    if (bal != ~0ull) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int kk = kt * 16 + 4 * g + i;
          if (!((bal >> (2 * kk)) & 1ull)) {
#pragma unroll
            for (int ht = 0; ht < NHT; ++ht) S[kt][ht][i] = NEG_INF;
          }
        }
    }

    // ---- online softmax (log2 units)
    bf16x8 P[NHT];
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) {
      float cm = fmaxf(fmaxf(fmaxf(S[0][ht][0], S[0][ht][1]), fmaxf(S[0][ht][2], S[0][ht][3])),
                       fmaxf(fmaxf(S[1][ht][0], S[1][ht][1]), fmaxf(S[1][ht][2], S[1][ht][3])));
      cm = max_over_groups(cm);
      const float mn = fmaxf(mrow[ht], cm);
      if (__ballot(mn > mrow[ht])) {
        const float alpha = __builtin_amdgcn_exp2f(mrow[ht] - mn);
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) O[dt][ht] *= alpha;
        lsum[ht] *= alpha;
        mrow[ht] = mn;
      }
      float ls = 0.0f;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float pv = __builtin_amdgcn_exp2f(S[kt][ht][i] - mrow[ht]);
          ls += pv;
          P[ht][kt * 4 + i] = (__bf16)pv;
        }
      lsum[ht] += ls;
    }

    // ---- O^T += V^T P^T; V^T operand by LDS transpose reads
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const int col = dt * 16 + 4 * (l16 & 3);
      // Whole-vector concatenation: building the operand element by element
      // from the v4i16 form of this builtin was miscompiled (only the low
      // dword survived), so the v4bf16 form is used with a shuffle.
      bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
          LDS_PTR(bf16x4, Ks + (4 * g + (l16 >> 2)) * KP + col));
      bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
          LDS_PTR(bf16x4, Ks + (16 + 4 * g + (l16 >> 2)) * KP + col));
      bf16x8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
      for (int ht = 0; ht < NHT; ++ht)
        O[dt][ht] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, P[ht], O[dt][ht], 0, 0, 0);
    }
    __syncthreads();
  }

  // ---- normalise, inverse RoPE on dims 64..127, store bf16
  float oc[8], os[8];
  if (p.rope) {
#pragma unroll
    for (int dd = 0; dd < 4; ++dd)
#pragma unroll
      for (int pp = 0; pp < 2; ++pp) rope_cs((double)t, p.rev[8 * dd + 2 * g + pp], oc[dd * 2 + pp], os[dd * 2 + pp]);
  }
#pragma unroll
  for (int ht = 0; ht < NHT; ++ht) {
    const int h = ht * 16 + l16;
    const float L = sum_over_groups(lsum[ht]);
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
    if (h >= p.H) continue;
    uint16_t* orow = p.out + (tok * p.H + h) * 128;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      float o0 = O[dt][ht][0] * inv, o1 = O[dt][ht][1] * inv;
      float o2 = O[dt][ht][2] * inv, o3 = O[dt][ht][3] * inv;
      if (p.rope && dt >= 4) {
        const int dd = dt - 4;
        float c0 = oc[dd * 2], s0 = os[dd * 2], c1 = oc[dd * 2 + 1], s1 = os[dd * 2 + 1];
        float r0 = o0 * c0 + o1 * s0, r1 = o1 * c0 - o0 * s0;
        float r2 = o2 * c1 + o3 * s1, r3 = o3 * c1 - o2 * s1;
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
