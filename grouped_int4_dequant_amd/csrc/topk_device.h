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


// Top-k of one token by one wave: lane j < k ends with the id and gate of
// slot j (slots in descending logit order; gates = softmax over the k picks).
// Each lane first sorts its own keys, so one round is a wave maximum over the
// lanes' heads, after which the winning lane shifts its list up by one.
template <int VPL>
__device__ __forceinline__ void topk_wave(const float *row, int E, int k, int lane, int &my_id, float &my_gate) {
  // every load is unconditional (clamped index) so all are in flight at once
  float v[VPL];
#pragma unroll
  for (int r = 0; r < VPL; ++r) v[r] = row[min(lane + 64 * r, E - 1)];
  uint64_t key[VPL];
#pragma unroll
  for (int r = 0; r < VPL; ++r) {
    const int e = lane + 64 * r;
    key[r] = e < E ? make_key(v[r], e) : 0ull;
  }
  // descending insertion sort of the lane's keys (VPL <= 16, unrolled)
#pragma unroll
  for (int i = 1; i < VPL; ++i)
#pragma unroll
    for (int j = i; j > 0; --j)
      if (key[j] > key[j - 1]) {
        const uint64_t t = key[j];
        key[j] = key[j - 1];
        key[j - 1] = t;
      }
  float v0 = 0.f, sum = 0.f, my_ex = 0.f;
  my_id = 0;
  for (int j = 0; j < k; ++j) {
    // wave maximum of the heads: first over the logit half of the key, then
    // (only when several lanes hold that logit) over the index half among them
    const uint32_t hi = (uint32_t)(key[0] >> 32);
    const uint32_t mhi = wave_max32(hi);
    const uint64_t holders = __ballot(hi == mhi);
    uint64_t win;
    if (__popcll(holders) == 1) {  // one lane holds the maximum logit: its head wins
      win = readlane64(key[0], __ffsll((long long)holders) - 1);
    } else {
      const uint32_t lo = hi == mhi ? (uint32_t)key[0] : 0u;
      win = ((uint64_t)mhi << 32) | wave_max32(lo);
    }
    if (key[0] == win) {  // keys are distinct: one lane wins and drops its head
#pragma unroll
      for (int r = 0; r + 1 < VPL; ++r) key[r] = key[r + 1];
      key[VPL - 1] = 0ull;
    }
    const float wv = key_value(win);
    if (j == 0) v0 = wv;
    const float ex = expf(wv - v0);
    sum += ex;
    if (lane == j) { my_ex = ex; my_id = key_index(win); }
  }
  my_gate = my_ex / sum;
}

}  // namespace moe
