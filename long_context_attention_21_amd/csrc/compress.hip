// compress.hip -- token-level KV compressor (CSA m = 4 overlapped, HCA m = 128).
//
// Method: "DeepSeek-V4: Towards Highly Efficient Million-Token Context
// Intelligence" wiki summary, Proposed method item 1 (every m tokens become
// one entry by a weighted average; adjacent blocks overlap for CSA);
// "deepseek V4 技术论文" 1.1 (C^b overlaps C^a).  Storage formats: wiki
// summary, Training infrastructure item 5 (RoPE dims BF16, other dims FP8);
// the V4.1 variant of the Russian summary stores post-RoPE entries in NVFP4
// and Post-training item 3 (MXFP4 indexer QK path).
//
// Design: HBM-bound strided pooling.  One wave per output entry; lane l owns
// KV dims 2l, 2l+1 (one 4-byte load per token row, a 256-byte coalesced row
// per wave) and, for lanes 0..31, indexer dims 2l, 2l+1.  The L <= 256 slot
// logits are staged in LDS: the softmax is evaluated in fp64 (exp of
// max-subtracted logits, summed in ascending slot order) and each weight is
// rounded to fp32; pooling is an fp32 fma chain in ascending slot order.  The
// RoPE dims (lanes 32..63) are rotated in fp64 at the entry position.  This
// fixed order makes the pooled fp32 values -- and so every storage code --
// reproducible and independent of the launch shape.
#include "device.h"
#include "kernels.h"

// The fp64 rotation and the pooling chain must not be contracted further.
#pragma clang fp contract(off)

namespace csa {

constexpr int kCompressWaves = 4;

__global__ __launch_bounds__(256) void compress_kernel(CompressParams p) {
  __shared__ double s_logit[kCompressWaves][256];
  __shared__ double s_exp[kCompressWaves][256];
  __shared__ float s_w[kCompressWaves][256];
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int64_t task = (int64_t)blockIdx.x * kCompressWaves + wv;
  const int m = p.m, L = p.L;
  const float NEG_INF = -__builtin_inff();
  bool active;
  int b, e;
  int64_t i;  // absolute entry index
  if (p.append) {
    // one wave per sequence: store the new row in the rings, then pool the
    // block it completes (if any)
    const bool live = task < p.B;
    b = live ? (int)task : 0;
    e = 0;
    if (live) {
      const int s = (int)(p.t % p.W);
      const uint32_t x = p.kv_new[(int64_t)b * 64 + lane];
      p.kv_ring[((int64_t)b * 2 * p.W + s) * 64 + lane] = x;
      p.kv_ring[((int64_t)b * 2 * p.W + s + p.W) * 64 + lane] = x;
      if (p.ik_new && lane < 32) p.ik_ring[((int64_t)b * p.W + s) * 32 + lane] = p.ik_new[(int64_t)b * 32 + lane];
      if (p.z_new && lane < 2) p.z_ring[((int64_t)b * p.W + s) * 2 + lane] = p.z_new[(int64_t)b * 2 + lane];
      if (p.win8_ring) {
        // FP8 window cache: the row rotated at t (fp64, as the entries), then
        // e4m3 over all 128 dims with scale amax / 448
        float v0 = bf16lo(x), v1 = bf16hi(x);
        if (p.rope_dims == 64 && lane >= 32) {
          const double phi = (double)p.t * p.theta[lane - 32];
          const double c = cos(phi), sn = sin(phi);
          const double x0 = v0, x1 = v1;
          v0 = (float)(x0 * c - x1 * sn);
          v1 = (float)(x0 * sn + x1 * c);
        }
        float amax = fmaxf(fabsf(v0), fabsf(v1));
        for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
        const float scale = __fdiv_rn(amax, 448.0f);
        uint32_t c0 = 0, c1 = 0;
        if (scale != 0.0f) {
          c0 = f32_to_e4m3(__fdiv_rn(v0, scale));
          c1 = f32_to_e4m3(__fdiv_rn(v1, scale));
        }
        const uint16_t cc = (uint16_t)(c0 | (c1 << 8));
        uint16_t* w8 = (uint16_t*)p.win8_ring;
        w8[((int64_t)b * 2 * p.W + s) * 64 + lane] = cc;
        w8[((int64_t)b * 2 * p.W + s + p.W) * 64 + lane] = cc;
        if (lane == 0) {
          p.win8_scale[(int64_t)b * 2 * p.W + s] = scale;
          p.win8_scale[(int64_t)b * 2 * p.W + s + p.W] = scale;
        }
      }
    }
    // t is the same for every wave: a call that completes no block ends here
    // on the whole work-group, before any barrier
    if ((p.t + 1) % m != 0) return;
    active = live;
    i = (p.t + 1) / m - 1;
  } else {
    const int64_t total = (int64_t)p.B * p.n_new;
    active = task < total;
    b = active ? (int)(task / p.n_new) : 0;
    e = active ? (int)(task % p.n_new) : 0;
    i = p.pos0 / m + e;
  }

  // ---- slot logits
  for (int r = lane; r < L; r += 64) {
    int64_t j;
    int role;
    if (p.overlap) {
      role = (r < m) ? 1 : 0;
      j = (r < m) ? (i - 1) * m + r : i * m + (r - m);
    } else {
      role = 0;
      j = i * m + r;
    }
    double lg = (double)NEG_INF;
    if (active && j >= 0 && p.append) {
      double zz = 0.0;
      if (p.z_new)
        zz = (double)(j == p.t ? p.z_new[(int64_t)b * 2 + role] : p.z_ring[((int64_t)b * p.W + j % p.W) * 2 + role]);
      lg = (double)p.beta[r] + zz;
    } else if (active && j >= 0) {
      double zz = 0.0;
      if (j >= p.pos0) {
        if (p.z) zz = (double)p.z[((int64_t)b * p.T + (j - p.pos0)) * 2 + role];
      } else if (p.prev_z) {
        zz = (double)p.prev_z[((int64_t)b * m + (j - (p.pos0 - m))) * 2 + role];
      }
      lg = (double)p.beta[r] + zz;
    }
    s_logit[wv][r] = lg;
  }
  __syncthreads();
  double mx = (double)NEG_INF;
  for (int r = 0; r < L; ++r) mx = fmax(mx, s_logit[wv][r]);
  for (int r = lane; r < L; r += 64) {
    double lg = s_logit[wv][r];
    s_exp[wv][r] = (lg == (double)NEG_INF) ? 0.0 : exp(lg - mx);
  }
  __syncthreads();
  double sum = 0.0;
  for (int r = 0; r < L; ++r) sum += s_exp[wv][r];
  for (int r = lane; r < L; r += 64) {
    double lg = s_logit[wv][r];
    s_w[wv][r] = (lg == (double)NEG_INF) ? NEG_INF : (float)(s_exp[wv][r] / sum);
  }
  __syncthreads();
  if (!active) return;

  // ---- pooling: fp32 fma chain in ascending slot order.  The rows of 8
  // slots are loaded before their fmas so the loads overlap.
  float a0 = 0.0f, a1 = 0.0f, k0 = 0.0f, k1 = 0.0f;
  const bool has_ik = p.append ? p.ik_new != nullptr : p.ik != nullptr;
  auto rows_of = [&](int r, const uint32_t*& xr, const uint32_t*& ur) {
    const int64_t j = p.overlap ? ((r < m) ? (i - 1) * m + r : i * m + (r - m)) : i * m + r;
    ur = nullptr;
    if (p.append) {
      if (j == p.t) {
        xr = p.kv_new + (int64_t)b * 64;
        if (has_ik) ur = p.ik_new + (int64_t)b * 32;
      } else {
        xr = p.kv_ring + ((int64_t)b * 2 * p.W + j % p.W) * 64;
        if (has_ik) ur = p.ik_ring + ((int64_t)b * p.W + j % p.W) * 32;
      }
    } else if (j >= p.pos0) {
      const int64_t row = (int64_t)b * p.T + (j - p.pos0);
      xr = p.kv + row * 64;
      if (has_ik) ur = p.ik + row * 32;
    } else {
      const int64_t row = (int64_t)b * m + (j - (p.pos0 - m));
      xr = p.prev_kv + row * 64;
      if (has_ik) ur = p.prev_ik + row * 32;
    }
  };
  for (int r0 = 0; r0 < L; r0 += 8) {
    float ws[8];
    uint32_t xs[8], us[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int r = r0 + u;
      ws[u] = r < L ? s_w[wv][r] : NEG_INF;
      xs[u] = 0u;
      us[u] = 0u;
      if (ws[u] != NEG_INF) {  // absent slots (before token 0, or past L) are skipped
        const uint32_t* xr;
        const uint32_t* ur;
        rows_of(r, xr, ur);
        xs[u] = xr[lane];
        if (has_ik && lane < 32) us[u] = ur[lane];
      }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (ws[u] == NEG_INF) continue;
      a0 = __builtin_fmaf(ws[u], bf16lo(xs[u]), a0);
      a1 = __builtin_fmaf(ws[u], bf16hi(xs[u]), a1);
      if (has_ik && lane < 32) {
        k0 = __builtin_fmaf(ws[u], bf16lo(us[u]), k0);
        k1 = __builtin_fmaf(ws[u], bf16hi(us[u]), k1);
      }
    }
  }

  // ---- RoPE at p_i = (i+1)m - 1, fp64 rotation (lanes 32..63 own dims 64..127)
  if (p.rope_dims == 64 && lane >= 32) {
    const int f = lane - 32;
    double phi = (double)((i + 1) * m - 1) * p.theta[f];
    double c = cos(phi), s = sin(phi);
    double x0 = a0, x1 = a1;
    double r0 = x0 * c - x1 * s;
    double r1 = x0 * s + x1 * c;
    a0 = (float)r0;
    a1 = (float)r1;
  }

  // ---- store the KV entry
  const int64_t orow = p.append ? (int64_t)b * p.N_cap + i : (int64_t)b * p.n_new + e;
  if (p.entry_fmt == 0) {
    ((uint32_t*)p.entries_out)[orow * 64 + lane] = pack_bf16(a0, a1);
  } else if (p.entry_fmt == 3) {
    // NVFP4 (post-RoPE, all 128 dims): s = amax / (6 * 448) per entry; block
    // j = dims 16j .. 16j+15 (lanes 8j .. 8j+7) gets the e4m3 scale of
    // amax_j / (6 s); codes are e2m1(x / (b_j s)); one fp32 operation per
    // step, rounded to nearest even.  Record: 64 code bytes, 8 scale bytes.
    float amax = fmaxf(fabsf(a0), fabsf(a1));
    float bamax = amax;
    for (int off = 4; off >= 1; off >>= 1) bamax = fmaxf(bamax, __shfl_xor(bamax, off));
    amax = bamax;
    for (int off = 32; off >= 8; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
    const float scale = __fdiv_rn(amax, 2688.0f);
    uint32_t code = 0, bcode = 0;
    if (scale != 0.0f) {
      bcode = f32_to_e4m3(__fdiv_rn(bamax, __fmul_rn(6.0f, scale)));
      const float sb = __fmul_rn(e4m3_to_f32(bcode), scale);
      if (sb != 0.0f) code = f32_to_e2m1(__fdiv_rn(a0, sb)) | (f32_to_e2m1(__fdiv_rn(a1, sb)) << 4);
    }
    uint8_t* rec = (uint8_t*)p.entries_out + orow * 72;
    rec[lane] = (uint8_t)code;
    if ((lane & 7) == 0) rec[64 + (lane >> 3)] = (uint8_t)bcode;
    if (lane == 0) p.entry_scale_out[orow] = scale;
  } else {
    // dims 0..63 (lanes 0..31) -> e4m3 with scale amax/448; dims 64..127 -> bf16
    float amax = (lane < 32) ? fmaxf(fabsf(a0), fabsf(a1)) : 0.0f;
    for (int off = 16; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
    float scale = __fdiv_rn(amax, 448.0f);
    if (lane < 32) {
      uint32_t c0 = 0, c1 = 0;
      if (scale != 0.0f) {
        c0 = f32_to_e4m3(__fdiv_rn(a0, scale));
        c1 = f32_to_e4m3(__fdiv_rn(a1, scale));
      }
      ((uint16_t*)p.entries_out)[orow * 32 + lane] = (uint16_t)(c0 | (c1 << 8));
      if (lane == 0) p.entry_scale_out[orow] = scale;
    } else {
      ((uint32_t*)p.entries_rope_out)[orow * 32 + (lane - 32)] = pack_bf16(a0, a1);
    }
  }

  // ---- store the indexer key
  if (has_ik && p.kidx_out) {
    if (p.kidx_fmt == 0) {
      if (lane < 32) ((uint32_t*)p.kidx_out)[orow * 32 + lane] = pack_bf16(k0, k1);
    } else {
      // MXFP4: block 0 = dims 0..31 (lanes 0..15), block 1 = dims 32..63 (lanes 16..31)
      float amax = fmaxf(fabsf(k0), fabsf(k1));
      for (int off = 8; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
      if (lane < 32) {
        uint32_t code = 0, sbyte = 0;
        if (amax > 0.0f) {
          int E = mxfp4_exponent(amax);
          sbyte = (uint32_t)(E + 127);
          uint32_t c0 = f32_to_e2m1(__builtin_ldexpf(k0, -E));
          uint32_t c1 = f32_to_e2m1(__builtin_ldexpf(k1, -E));
          code = c0 | (c1 << 4);
        }
        p.kidx_out_u8()[orow * 32 + lane] = (uint8_t)code;
        if ((lane & 15) == 0) p.kidx_scale_out[orow * 2 + (lane >> 4)] = (uint8_t)sbyte;
      }
    }
  }
}

// One wave per row: lane l holds dims 2l, 2l+1; lanes 32..63 rotate their
// pair at the row's position exactly as the entries are rotated (fp64).
__global__ __launch_bounds__(256) void rope_rows_kernel(RopeRowsParams p) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= p.rows) return;
  const uint32_t x = p.kv[row * 64 + lane];
  uint32_t y = x;
  if (lane >= 32) {
    const double phi = (double)(p.pos0 + row % p.T) * p.theta[lane - 32];
    const double c = cos(phi), s = sin(phi);
    const double x0 = bf16lo(x), x1 = bf16hi(x);
    y = pack_bf16((float)(x0 * c - x1 * s), (float)(x0 * s + x1 * c));
  }
  p.out[row * 64 + lane] = y;
}

hipError_t launch_rope_rows(const RopeRowsParams& p, hipStream_t stream) {
  if (p.rows == 0) return hipSuccess;
  hipLaunchKernelGGL(rope_rows_kernel, dim3((unsigned)((p.rows + 3) / 4)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_compress(const CompressParams& p, hipStream_t stream) {
  int64_t total = p.append ? (int64_t)p.B : (int64_t)p.B * p.n_new;
  if (total == 0) return hipSuccess;
  dim3 grid((unsigned)((total + kCompressWaves - 1) / kCompressWaves));
  hipLaunchKernelGGL(compress_kernel, grid, dim3(64 * kCompressWaves), 0, stream, p);
  return hipGetLastError();
}

}  // namespace csa
