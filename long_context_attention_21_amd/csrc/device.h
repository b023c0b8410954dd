// device.h -- gfx950 device helpers shared by the kernels of this library:
// vector types for the MFMA builtins, bf16 / e4m3 / e2m1 conversions, RoPE
// angle evaluation and wave-level reductions.
//
// Lane layouts verified on gfx950 hardware (in-bounds probe):
//  * v_mfma_f32_16x16x32_bf16: A lane l holds A[l%16][8*(l/16) + e], e = 0..7;
//    B lane l holds B[8*(l/16) + e][l%16]; C lane l holds C[4*(l/16) + i][l%16].
//  * v_mfma_scale_f32_32x32x64_f8f6f4 (fp4): A lane l holds 32 e2m1 values of
//    row l%32, k = 32*(l/32) + e at bits [4e, 4e+4) of the 128-bit operand,
//    and supplies the e8m0 scale of that (row, k-block); B likewise per
//    column; C lane l holds C[8*(i/4) + 4*(l/32) + i%4][l%32], i = 0..15.
//  * ds_read_b64_tr_b16: in each 16-lane group, lane L receives element L%4
//    of the 8-byte rows read by lanes L/4 + 4i, i = 0..3.
//  * v_permlane16_swap / v_permlane32_swap(x, x) leave the pair
//    (x[lo], x[hi]) of lanes (l, l^16) / (l, l^32) in both lanes.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))

__device__ __forceinline__ float bf16_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16 bits, round to nearest even (the gfx950 conversion).
__device__ __forceinline__ uint32_t f32_to_bf16(float x) {
  __bf16 b = (__bf16)x;
  return (uint32_t)__builtin_bit_cast(uint16_t, b);
}
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  return f32_to_bf16(lo) | (f32_to_bf16(hi) << 16);
}

// OCP e4m3fn encode of a finite fp32 value: round to nearest even on the
// e4m3 grid, saturate to +-448, zero results encoded as +0.  Works on the
// fp32 bit pattern: the e4m3 grid step in binade 2^k (k >= -6) is 2^(k-3),
// below 2^-6 it is 2^-9.
__device__ __forceinline__ uint32_t f32_to_e4m3(float x) {
  uint32_t u = __float_as_uint(x);
  uint32_t sign = (u >> 24) & 0x80u;
  float a = fabsf(x);
  if (!(a == a)) return 0x7fu;
  if (a >= 464.0f) return sign | 0x7eu;  // RNE would leave the finite range
  uint32_t code;
  if (a < 0.015625f) {  // below 2^-6: multiples of 2^-9 (exact scaling)
    float r = __builtin_rintf(a * 512.0f);  // ties to even
    code = (uint32_t)r;                     // 0..8 (8 = 2^-6, exponent field 1)
  } else {
    uint32_t ua = __float_as_uint(a);
    uint32_t e = (ua >> 23) - 127 + 7;   // e4m3 exponent field (1..15)
    uint32_t man = ua & 0x7fffffu;
    uint32_t keep = man >> 20;           // 3 mantissa bits
    uint32_t rest = man & 0xfffffu;
    uint32_t half = 0x80000u;
    if (rest > half || (rest == half && (keep & 1u))) keep += 1;
    code = (e << 3) + keep;              // carry into the exponent is correct
    if (code > 0x7eu) code = 0x7eu;
  }
  if (code == 0) return 0;
  return sign | code;
}

__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  uint32_t e = (c >> 3) & 15u, man = c & 7u;
  float v = (e == 0) ? (float)man * 0.001953125f
                     : __uint_as_float(((e + 120u) << 23) | (man << 20));
  return (c & 0x80u) ? -v : v;
}

// e2m1 code of v (v already divided by the block scale): nearest with ties
// to the even code, saturating at 6.  Grid 0, .5, 1, 1.5, 2, 3, 4, 6.
__device__ __forceinline__ uint32_t f32_to_e2m1(float v) {
  float a = fabsf(v);
  uint32_t c = (a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) +
               (a > 2.5f) + (a >= 3.5f) + (a > 5.0f);
  return (c != 0 && v < 0.0f) ? (c | 8u) : c;
}

// Shared MXFP4 exponent of a block with maximum magnitude amax > 0:
// E = floor(log2(amax)) - 2, clamped to [-127, 127].
__device__ __forceinline__ int mxfp4_exponent(float amax) {
  int fl;
  uint32_t ua = __float_as_uint(amax);
  uint32_t ef = ua >> 23;
  if (ef != 0) {
    fl = (int)ef - 127;
  } else {  // subnormal: position of the leading mantissa bit
    fl = -127 - (__builtin_clz(ua) - 9);
  }
  int E = fl - 2;
  return E < -127 ? -127 : (E > 127 ? 127 : E);
}

// RoPE angle of position pos for a frequency given in revolutions per
// position (theta_f / 2pi, fp64): the fractional revolution is formed in
// fp64, then the hardware sin/cos (inputs in revolutions) give cos, sin.
__device__ __forceinline__ void rope_cs(double pos, double rev_f, float& c, float& s) {
  double r = pos * rev_f;
  r = r - __builtin_floor(r);
  float rf = (float)r;
  s = __builtin_amdgcn_sinf(rf);
  c = __builtin_amdgcn_cosf(rf);
}

// Wave64 reductions over the four 16-lane groups (lanes l, l^16, l^32, l^48).
__device__ __forceinline__ float max_over_groups(float x) {
  uint32_t u = __float_as_uint(x);
  auto p = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  x = fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
  u = __float_as_uint(x);
  auto q = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__uint_as_float(q[0]), __uint_as_float(q[1]));
}
__device__ __forceinline__ float sum_over_groups(float x) {
  uint32_t u = __float_as_uint(x);
  auto p = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  x = __uint_as_float(p[0]) + __uint_as_float(p[1]);
  u = __float_as_uint(x);
  auto q = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}

// Buffer descriptor words (base, stride 0, byte extent, 32-bit data format):
// reads past the extent return zeros.
__device__ __forceinline__ u32x4 dma_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)base;
  return u32x4{(uint32_t)a, (uint32_t)(a >> 32) & 0xffffu, (uint32_t)bytes, 0x00020000u};
}

// Direct-to-LDS load of 16 bytes per lane: lane l's bytes at `voff` land at
// LDS address lds + 16 l.  Issued from inline asm so that the compiler does
// not track it: otherwise it makes every LDS read wait for all outstanding
// loads (vmcnt(0)), including the prefetch of the chunks ahead, which
// serialises the ring.  The caller waits with s_waitcnt vmcnt and a barrier
// before it reads the slot.  M0 carries the LDS address; the leading
// s_nop 4 covers an M0 or descriptor write just before the load.
__device__ __forceinline__ void dma_b128(const u32x4& r, uint32_t lds, uint32_t voff) {
  u32x4 rs;  // wave-uniform: make that explicit so it is taken from SGPRs
#pragma unroll
  for (int i = 0; i < 4; ++i) rs[i] = (uint32_t)__builtin_amdgcn_readfirstlane((int)r[i]);
  asm volatile(
      "s_nop 4\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen lds"
      :
      : "{m0}"((uint32_t)__builtin_amdgcn_readfirstlane((int)lds)), "v"(voff), "s"(rs)
      : "memory");
}

}  // namespace csa
