// Device helpers for top-k selection over router logits, shared by the
// routing kernels and the decode kernels (gfx950, 64-lane waves).
//
// Every candidate becomes a 64-bit key: order-preserving logit bits, then
// the inverted expert index, so "larger logit, then lower index" is plain
// unsigned order and all keys are distinct (the tie rule of the layer's
// router: equal logits go to the lower expert index under IEEE equality).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// Order-preserving key: larger logit first, equal logits (IEEE ==, so -0.0
// ties +0.0) go to the lower expert index. 0 is below every real key.
__device__ __forceinline__ uint64_t make_key(float v, int e) {
  uint32_t u = (v == 0.f) ? 0u : __float_as_uint(v);
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)u << 32) | (uint32_t)~(uint32_t)e;
}
__device__ __forceinline__ int key_index(uint64_t key) { return (int)~(uint32_t)key; }
__device__ __forceinline__ float key_value(uint64_t key) {
  const uint32_t u = (uint32_t)(key >> 32);
  return __uint_as_float((u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u);
}

template <int CTRL>
__device__ __forceinline__ uint64_t dpp64(uint64_t v) {
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, CTRL, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), CTRL, 0xF, 0xF, false);
  return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}
__device__ __forceinline__ uint64_t max64(uint64_t a, uint64_t b) { return a > b ? a : b; }
__device__ __forceinline__ uint64_t readlane64(uint64_t v, int lane) {
  const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)v, lane);
  const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), lane);
  return ((uint64_t)hi << 32) | lo;
}

// Unsigned 32-bit maximum over the 64 lanes, returned uniformly.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t wave_max32(uint32_t v) {
  v = max(v, dpp32<0xB1>(v));   // quad_perm 1,0,3,2
  v = max(v, dpp32<0x4E>(v));   // quad_perm 2,3,0,1
  v = max(v, dpp32<0x124>(v));  // row_ror 4
  v = max(v, dpp32<0x128>(v));  // row_ror 8: every lane holds its row's maximum
  const uint32_t a = max((uint32_t)__builtin_amdgcn_readlane((int)v, 0), (uint32_t)__builtin_amdgcn_readlane((int)v, 16));
  const uint32_t b = max((uint32_t)__builtin_amdgcn_readlane((int)v, 32), (uint32_t)__builtin_amdgcn_readlane((int)v, 48));
  return max(a, b);
}

// Maximum over the 64 lanes, returned uniformly.
__device__ __forceinline__ uint64_t wave_max64(uint64_t v) {
  v = max64(v, dpp64<0xB1>(v));   // quad_perm 1,0,3,2
  v = max64(v, dpp64<0x4E>(v));   // quad_perm 2,3,0,1
  v = max64(v, dpp64<0x124>(v));  // row_ror 4
  v = max64(v, dpp64<0x128>(v));  // row_ror 8: every lane holds its row's maximum
  return max64(max64(readlane64(v, 0), readlane64(v, 16)),
               max64(readlane64(v, 32), readlane64(v, 48)));
}


}  // namespace moe
