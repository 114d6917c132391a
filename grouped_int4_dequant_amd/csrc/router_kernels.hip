// Router projection for gfx950: logits = x W_r^T, the step just before the
// top-k (Lily-EN "Three Workload Shapes": a router scores every expert for
// each token and the layer keeps the best k).
//
// x and W_r are bf16; products are exact in fp32 and accumulate in fp32 with
// v_mfma_f32_16x16x32_bf16 in a fixed order (32 inputs per MFMA, ascending),
// so repeated calls give identical logits. A workgroup of four waves covers
// 32 tokens x 64 experts; a wave owns 16 experts and both 16-row blocks, and
// reads its operands straight from memory (each 16-byte fragment is one
// token's or one expert's eight consecutive inputs), requesting the next
// four 32-input steps before computing the current four.
//
// Pages cited (titles as published):
//   Lily-EN  "Perplexity Open Sources Lily: A Rust + Metal Inference Engine
//            for Qwen3.6-35B-A3B on Apple Silicon" (insight.aitobox.com)

#include "moe_internal.h"

namespace moe {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf8 __attribute__((ext_vector_type(8)));

constexpr int kRouterRows = 32;     // tokens per workgroup
constexpr int kRouterExperts = 64;  // experts per workgroup (16 per wave)
constexpr int kGroupSteps = 4;      // 32-input steps requested together

__global__ __launch_bounds__(256) void router_kernel(RouterArgs a) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c16 = lane & 15, kq = lane >> 4;
  const int t0 = blockIdx.x * kRouterRows;
  const int e = blockIdx.y * kRouterExperts + wave * 16 + c16;
  // rows and experts past the end read the last valid one (never stored)
  const int ec = min(e, a.E - 1);
  const int tr0 = min(t0 + c16, a.T - 1), tr1 = min(t0 + 16 + c16, a.T - 1);
  const uint4 *xa = reinterpret_cast<const uint4 *>(a.x + (int64_t)tr0 * a.d) + kq;
  const uint4 *xb = reinterpret_cast<const uint4 *>(a.x + (int64_t)tr1 * a.d) + kq;
  const uint4 *wr = reinterpret_cast<const uint4 *>(a.w + (int64_t)ec * a.d) + kq;
  const int steps = a.d / 32;  // 16-byte chunks: 4 per step; this lane's is chunk kq

  f4 acc0 = f4{0.f, 0.f, 0.f, 0.f}, acc1 = f4{0.f, 0.f, 0.f, 0.f};
  uint4 ca[kGroupSteps], cb[kGroupSteps], cw[kGroupSteps];
  auto load = [&](int s0) {
#pragma unroll
    for (int u = 0; u < kGroupSteps; ++u) {
      const int s = min(s0 + u, steps - 1);
      ca[u] = xa[4 * s];
      cb[u] = xb[4 * s];
      cw[u] = wr[4 * s];
    }
  };
  load(0);
  for (int s0 = 0; s0 < steps; s0 += kGroupSteps) {
    uint4 na[kGroupSteps], nb[kGroupSteps], nw[kGroupSteps];
#pragma unroll
    for (int u = 0; u < kGroupSteps; ++u) {
      na[u] = ca[u];
      nb[u] = cb[u];
      nw[u] = cw[u];
    }
    load(s0 + kGroupSteps);  // next group (clamped at the end: reloads the last step)
#pragma unroll
    for (int u = 0; u < kGroupSteps; ++u) {
      if (s0 + u < steps) {
        const bf8 w = __builtin_bit_cast(bf8, nw[u]);
        acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf8, na[u]), w, acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf8, nb[u]), w, acc1, 0, 0, 0);
      }
    }
  }
  // element i of lane (c16, kq): token row 4 kq + i of the block, expert c16
  if (e < a.E) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r0 = t0 + 4 * kq + i, r1 = t0 + 16 + 4 * kq + i;
      if (r0 < a.T) a.logits[(int64_t)r0 * a.E + e] = acc0[i];
      if (r1 < a.T) a.logits[(int64_t)r1 * a.E + e] = acc1[i];
    }
  }
}

}  // namespace

hipError_t launch_router(const RouterArgs &a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  const dim3 grid((unsigned)ceil_div(a.T, kRouterRows), (unsigned)ceil_div(a.E, kRouterExperts));
  hipLaunchKernelGGL(router_kernel, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
