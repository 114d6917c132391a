// On-chip rebuild of 4-bit groupwise-affine weights into fp16 MFMA operands
// (gfx950). One group of 64 weights along the input dimension shares one
// bf16 scale s and one bf16 bias b, and a weight is w = s * q + b with the
// unsigned 4-bit code q (Lily-ES "Precarga: mantenga los pesos empaquetados,
// siga enrutando en la GPU": groups of 64 with one scale and one bias).
//
// A 32-bit word holds eight codes, low nibble first. Two codes at a time go
// into the mantissas of an fp16 pair "1024 + v" with one v_and_or_b32 (v = q,
// or 16 q for the odd nibbles, which saves a shift), one v_pk_add_f16 removes
// the offset exactly, and one v_pk_fma_f16 applies (s or s/16, b + 8 s):
//   w = fp16(s * (q - 8) + (b + 8 s)).
// The eight weights come out in the order q0 q4 q1 q5 q2 q6 q3 q7; the other
// MFMA operand uses the same order for each run of eight inputs.
//
// Pages cited (titles as published):
//   Lily-ES  "Perplexity open sources Lily: un motor de inferencia ... para
//            Qwen3.6-35B-A3B en Apple Silicon" (7minutos.es)
#pragma once

#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef _Float16 rb_h2 __attribute__((ext_vector_type(2)));
typedef _Float16 rb_h8 __attribute__((ext_vector_type(8)));

// A VGPR holding a constant, so v_and_or_b32 can take the mask from a VGPR
// and the fp16 magic from an SGPR (VOP3 on gfx9 takes no literal).
__device__ __forceinline__ uint32_t rb_vgpr_const(uint32_t v) {
  uint32_t r;
  asm volatile("v_mov_b32 %0, %1" : "=v"(r) : "i"(v));
  return r;
}

// Per-group constants: (fp16 s, fp16 (b + 8 s)) from bf16 bits.
__device__ __forceinline__ uint32_t rb_pack_scale_bias(uint32_t s_bits, uint32_t b_bits) {
  const float sf = __uint_as_float(s_bits << 16), bf = __uint_as_float(b_bits << 16);
  const uint32_t lo = __half_as_ushort(__float2half_rn(sf));
  const uint32_t hi = __half_as_ushort(__float2half_rn(bf + 8.f * sf));
  return lo | (hi << 16);
}

struct RbConsts {
  uint32_t m_lo, m_hi;  // 0x000F000F, 0x00F000F0 in VGPRs
};

__device__ __forceinline__ RbConsts rb_consts() {
  return RbConsts{rb_vgpr_const(0x000F000Fu), rb_vgpr_const(0x00F000F0u)};
}

// A group's constants as the rebuild applies them: (s, s), (s/16, s/16) and
// (b + 8 s, b + 8 s) from the packed pair. For a bf16 scale (8 significant
// bits) s/16 is exact in fp16 from s = 2^-13 up; below that it is a
// subnormal without room for every bit.
struct RbGroup {
  rb_h2 s1, s16, cc;
};
__device__ __forceinline__ RbGroup rb_group(uint32_t sc_packed) {
  const rb_h2 sc = __builtin_bit_cast(rb_h2, sc_packed);
  RbGroup g;
  g.s1 = rb_h2{sc[0], sc[0]};
  g.s16 = g.s1 * rb_h2{(_Float16)0.0625f, (_Float16)0.0625f};
  g.cc = rb_h2{sc[1], sc[1]};
  return g;
}

// Eight weights of one code word with its group's constants.
__device__ __forceinline__ rb_h8 rb_rebuild_g(uint32_t w, const RbGroup &g, const RbConsts &k) {
  const uint32_t magic = 0x64006400u;  // fp16 pair (1024, 1024)
  const rb_h2 off1 = rb_h2{(_Float16)-1032.f, (_Float16)-1032.f};
  const rb_h2 off16 = rb_h2{(_Float16)-1152.f, (_Float16)-1152.f};
  const uint32_t w8 = w >> 8;
  const rb_h2 t0 = __builtin_bit_cast(rb_h2, (w & k.m_lo) | magic) + off1;    // (q0, q4)
  const rb_h2 t1 = __builtin_bit_cast(rb_h2, (w & k.m_hi) | magic) + off16;   // 16 (q1, q5)
  const rb_h2 t2 = __builtin_bit_cast(rb_h2, (w8 & k.m_lo) | magic) + off1;   // (q2, q6)
  const rb_h2 t3 = __builtin_bit_cast(rb_h2, (w8 & k.m_hi) | magic) + off16;  // 16 (q3, q7)
  const rb_h2 w0 = __builtin_elementwise_fma(t0, g.s1, g.cc);
  const rb_h2 w1 = __builtin_elementwise_fma(t1, g.s16, g.cc);
  const rb_h2 w2 = __builtin_elementwise_fma(t2, g.s1, g.cc);
  const rb_h2 w3 = __builtin_elementwise_fma(t3, g.s16, g.cc);
  return rb_h8{w0[0], w0[1], w1[0], w1[1], w2[0], w2[1], w3[0], w3[1]};
}

// Eight weights of one code word in one rounding each, from the pair
// (fp16 s * 2^20, fp16 b) of its group (valid when |s| < 2^-4, so that
// s * 2^20 is a normal fp16): a code moved to bits 4..7 of an fp16 half with
// a zero exponent is the subnormal q * 2^-20, exact, and one v_pk_fma_f16
// forms fp16(q * 2^-20 * s * 2^20 + b) = fp16(s * q + b). Three shifts and
// four ands place the eight codes, in the same order as rb_rebuild_g.
__device__ __forceinline__ rb_h8 rb_rebuild_sub(uint32_t w, const RbGroup &g) {
  const uint32_t m = 0x00F000F0u;
  const rb_h2 t0 = __builtin_bit_cast(rb_h2, (w << 4) & m);  // (q0, q4)
  const rb_h2 t1 = __builtin_bit_cast(rb_h2, w & m);         // (q1, q5)
  const rb_h2 t2 = __builtin_bit_cast(rb_h2, (w >> 4) & m);  // (q2, q6)
  const rb_h2 t3 = __builtin_bit_cast(rb_h2, (w >> 8) & m);  // (q3, q7)
  const rb_h2 w0 = __builtin_elementwise_fma(t0, g.s1, g.cc);
  const rb_h2 w1 = __builtin_elementwise_fma(t1, g.s1, g.cc);
  const rb_h2 w2 = __builtin_elementwise_fma(t2, g.s1, g.cc);
  const rb_h2 w3 = __builtin_elementwise_fma(t3, g.s1, g.cc);
  return rb_h8{w0[0], w0[1], w1[0], w1[1], w2[0], w2[1], w3[0], w3[1]};
}

// The pair rb_rebuild_sub takes, from bf16 bits (its caller checks the range).
__device__ __forceinline__ uint32_t rb_pack_sub(uint32_t s_bits, uint32_t b_bits) {
  const float sf = __uint_as_float(s_bits << 16) * 1048576.f, bf = __uint_as_float(b_bits << 16);
  return (uint32_t)__half_as_ushort(__float2half_rn(sf)) | ((uint32_t)__half_as_ushort(__float2half_rn(bf)) << 16);
}

// Eight weights of one code word; sc = packed (fp16 s, fp16 (b + 8 s)).
__device__ __forceinline__ rb_h8 rb_rebuild(uint32_t w, uint32_t sc_packed, const RbConsts &k) {
  return rb_rebuild_g(w, rb_group(sc_packed), k);
}

// Eight consecutive activations (natural order) -> fp16 in the rebuild order
// 0,4,1,5,2,6,3,7.
__device__ __forceinline__ rb_h8 rb_perm8(const float (&v)[8]) {
  return rb_h8{(_Float16)v[0], (_Float16)v[4], (_Float16)v[1], (_Float16)v[5],
               (_Float16)v[2], (_Float16)v[6], (_Float16)v[3], (_Float16)v[7]};
}

}  // namespace moe
