// Router projection for gfx950: logits = x W_r^T, the step just before the
// top-k (Lily-EN "Three Workload Shapes": a router scores every expert for
// each token and the layer keeps the best k).
//
// x and W_r are bf16; products are exact in fp32 and accumulate in fp32 with
// v_mfma_f32_16x16x32_bf16 in a fixed order (32 inputs per MFMA, ascending),
// so repeated calls give identical logits. A workgroup of four waves covers
// 32 tokens x 64 experts; a wave owns 16 experts and both 16-row blocks.
// Both operands pass through LDS in chunks of 256 inputs (double buffered,
// 16-byte units XOR-swizzled by row so the 16 rows read by one MFMA operand
// fetch hit distinct banks): the 32 token rows, shared by the four waves, and
// the 64 expert rows, so every request is a coalesced 512-byte row segment
// (each wave reading its own experts' rows straight from memory, 16 segments
// of 64 bytes per request, took 11.6 against 10.0 us at T=2048 for the same
// logits bit for bit). The next chunk is requested before the current one is
// computed. The chunk loop body has no per-step branch (columns past d are
// staged as zeros, which add exactly zero to accumulators that start at +0,
// and the chunk count is rounded up to the unroll of two), so the compiler
// keeps the next chunk's loads in flight across iterations. Calls of at most
// 16 tokens take a second form (router_small_kernel below) that spreads W_r
// over four times as many workgroups.

// Pages cited (titles as published):
//   Lily-EN  "Perplexity Open Sources Lily: A Rust + Metal Inference Engine
//            for Qwen3.6-35B-A3B on Apple Silicon" (insight.aitobox.com)

#include "moe_internal.h"

namespace moe {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf8 __attribute__((ext_vector_type(8)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));

constexpr int kRouterRows = 32;     // tokens per workgroup
constexpr int kRouterExperts = 64;  // experts per workgroup (16 per wave)
constexpr int kChunkSteps = 8;      // 32-input steps per LDS chunk (256 inputs)
constexpr int kRowBytes = kChunkSteps * 64;  // one token row of a chunk (bf16)

__global__ __launch_bounds__(256) void router_kernel(RouterArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t s_x[2][kRouterRows * kRowBytes];     // 2 x 16 KiB
  __shared__ __attribute__((aligned(16))) uint8_t s_w[2][kRouterExperts * kRowBytes];  // 2 x 32 KiB
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c16 = lane & 15, kq = lane >> 4;
  const int t0 = blockIdx.x * kRouterRows;
  const int e0 = blockIdx.y * kRouterExperts;
  const int e = e0 + wave * 16 + c16;
  const int steps = a.d / 32;
  // chunks rounded up to an even count: the loop body is straight-line code
  // (no per-step branch), so the compiler keeps the next chunk's loads in
  // flight across the loop; columns past d are staged as zeros in x, which
  // add exactly zero to accumulators that start at +0
  const int nchunks = 2 * ((steps + 2 * kChunkSteps - 1) / (2 * kChunkSteps));
  // staging: unit u = tid + 256 i of a chunk is row u / 32 (a token of the
  // block, or an expert of the block), 16-byte column u % 32; rows past T or
  // E repeat the last one, columns past d are clamped (never used: x is zero
  // there)
  static_assert(kRouterRows * (kRowBytes / 16) == 4 * 256, "four 16-byte x units per thread and chunk");
  static_assert(kRouterExperts * (kRowBytes / 16) == 8 * 256, "eight 16-byte weight units per thread and chunk");
  auto x_src = [&](int c, int i) {
    const int u = tid + 256 * i, r = u >> 5, j = u & 31;
    const int tr = min(t0 + r, a.T - 1);
    const int col = min(c * kChunkSteps * 32 + 8 * j, a.d - 8);
    return reinterpret_cast<const uint4 *>(a.x + (int64_t)tr * a.d + col);
  };
  auto x_dst = [&](int buf, int i) {
    const int u = tid + 256 * i, r = u >> 5, j = u & 31;
    return reinterpret_cast<uint4 *>(&s_x[buf][r * kRowBytes + 16 * (j ^ (r & 15))]);
  };
  auto w_src = [&](int c, int i) {
    const int u = tid + 256 * i, r = u >> 5, j = u & 31;
    const int er = min(e0 + r, a.E - 1);
    const int col = min(c * kChunkSteps * 32 + 8 * j, a.d - 8);
    return reinterpret_cast<const uint4 *>(a.w + (int64_t)er * a.d + col);
  };
  auto w_dst = [&](int buf, int i) {
    const int u = tid + 256 * i, r = u >> 5, j = u & 31;
    return reinterpret_cast<uint4 *>(&s_w[buf][r * kRowBytes + 16 * (j ^ (r & 15))]);
  };
  // this thread's units of the next chunk (compiler vector type: a select
  // of the struct form costs about 40 more registers)
  u4 xr[4], wreg[8];
  auto live = [&](int c, int i) { return c * kChunkSteps * 32 + 8 * ((tid + 256 * i) & 31) < a.d; };
  auto load = [&](int c) {
    u4 v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = *reinterpret_cast<const u4 *>(x_src(c, i));
#pragma unroll
    for (int i = 0; i < 8; ++i) wreg[i] = *reinterpret_cast<const u4 *>(w_src(c, i));
#pragma unroll
    for (int i = 0; i < 4; ++i) xr[i] = live(c, i) ? v[i] : u4{0u, 0u, 0u, 0u};
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<u4 *>(x_dst(buf, i)) = xr[i];
#pragma unroll
    for (int i = 0; i < 8; ++i) *reinterpret_cast<u4 *>(w_dst(buf, i)) = wreg[i];
  };
  f4 acc0 = f4{0.f, 0.f, 0.f, 0.f}, acc1 = f4{0.f, 0.f, 0.f, 0.f};
  const int wrow = 16 * wave + c16;  // this lane's expert row of the weight tile
  // One chunk: the barrier publishes chunk c in LDS and frees the other
  // buffers; chunk c+1's rows and weights are requested (the last chunk
  // requests itself again), chunk c is computed, then c+1 goes to LDS.
  auto body = [&](int c) {
    __syncthreads();
    load(min(c + 1, nchunks - 1));
    const uint8_t *xb = s_x[c & 1];
    const uint8_t *wb = s_w[c & 1] + wrow * kRowBytes;
#pragma unroll
    for (int u = 0; u < kChunkSteps; ++u) {
      const int j = 4 * u + kq;
      const uint4 wv = *reinterpret_cast<const uint4 *>(wb + 16 * (j ^ c16));
      const uint4 xa = *reinterpret_cast<const uint4 *>(xb + c16 * kRowBytes + 16 * (j ^ c16));
      acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf8, xa), __builtin_bit_cast(bf8, wv), acc0, 0, 0, 0);
      const uint4 xc = *reinterpret_cast<const uint4 *>(xb + (16 + c16) * kRowBytes + 16 * (j ^ c16));
      acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf8, xc), __builtin_bit_cast(bf8, wv), acc1, 0, 0, 0);
    }
    store((c + 1) & 1);
  };
  load(0);
  store(0);
  for (int c = 0; c < nchunks; c += 2) {
    body(c);
    body(c + 1);
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

// Few tokens (T <= 16, the decode shape): one 16-row MFMA block holds every
// token, so a workgroup takes 16 experts and splits the inputs over its eight
// waves, each requesting its x and W_r operands eight steps at a time before
// the first MFMA. W_r is then streamed by E / 16 workgroups instead of the
// E / 64 of the block form, whose four-wave workgroups each pull 256 KiB
// through one CU. W_r comes in whole 512-byte row segments through a
// per-wave LDS tile (16 row segments of 64 bytes per request, straight in the
// MFMA layout, took 3.9 against 3.0 us per T = 1 call); the token rows are
// read directly (staging them too was slower at T = 1 and 4). The waves'
// partial sums meet in LDS and are added in wave order, so repeated calls
// give identical logits.
constexpr int kSmallRows = 16;   // tokens of the one row block
constexpr int kSmallWaves = 8;   // input slices per workgroup
constexpr int kSmallBatch = 8;   // 32-input steps requested at once
__global__ __launch_bounds__(64 * kSmallWaves) void router_small_kernel(RouterArgs a) {
  __shared__ f4 s_part[kSmallWaves][64];
  // each wave's W_r batch on its way into the MFMA layout: 16 expert rows x
  // 32 16-byte units (eight 32-input steps), units XOR-swizzled by row
  __shared__ u4 s_ws[kSmallWaves][16][32];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c16 = lane & 15, kq = lane >> 4;
  const int e = blockIdx.x * 16 + c16;
  // token rows past T read the last token, expert rows past E the last
  // expert (neither is stored)
  const int tr = min(c16, a.T - 1);
  const int steps = a.d / 32;
  const int s0 = wave * steps / kSmallWaves, s1 = (wave + 1) * steps / kSmallWaves;
  // lane (c16, kq): A row c16 (a token) and B column c16 (an expert), inputs
  // 32 s + 8 kq .. + 7 of step s
  const uint4 *xr = reinterpret_cast<const uint4 *>(a.x + (int64_t)tr * a.d) + kq;
  // W_r in whole 512-byte row segments: request u of a batch covers expert
  // rows 2 u and 2 u + 1 of the 16 (lane l: row 2 u + l / 32, unit l % 32 =
  // step (l % 32) / 4 of the batch, 16-byte quarter l % 4)
  const int wl = lane >> 5, wu = lane & 31;
  f4 acc = f4{0.f, 0.f, 0.f, 0.f};
  for (int sb = s0; sb < s1; sb += kSmallBatch) {
    uint4 xv[kSmallBatch];
    u4 wraw[kSmallBatch];
    const int stu = min(sb + (wu >> 2), s1 - 1);
#pragma unroll
    for (int u = 0; u < kSmallBatch; ++u) {
      const int st = min(sb + u, s1 - 1);
      xv[u] = xr[4 * st];
      const int er = min((int)blockIdx.x * 16 + 2 * u + wl, a.E - 1);
      wraw[u] = reinterpret_cast<const u4 *>(a.w + (int64_t)er * a.d)[4 * stu + (wu & 3)];
    }
    // the previous batch's reads of s_ws are done before it is overwritten,
    // and these writes before the reads below (one wave's LDS operations
    // run in order; the fences keep the compiler from moving them)
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
#pragma unroll
    for (int u = 0; u < kSmallBatch; ++u) s_ws[wave][2 * u + wl][wu ^ (2 * u + wl)] = wraw[u];
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
#pragma unroll
    for (int u = 0; u < kSmallBatch; ++u)
      if (sb + u < s1) {
        const u4 wv = s_ws[wave][c16][(4 * u + kq) ^ c16];
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf8, xv[u]), __builtin_bit_cast(bf8, wv), acc,
                                                      0, 0, 0);
      }
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  }
  s_part[wave][lane] = acc;
  __syncthreads();
  if (wave != 0) return;
  f4 sum = s_part[0][lane];
#pragma unroll
  for (int w = 1; w < kSmallWaves; ++w) sum += s_part[w][lane];
  // element i of lane (c16, kq): token 4 kq + i, expert c16
  if (e < a.E) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = 4 * kq + i;
      if (t < a.T) a.logits[(int64_t)t * a.E + e] = sum[i];
    }
  }
}

}  // namespace

hipError_t launch_router(const RouterArgs &a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  if (a.T <= kSmallRows) {
    hipLaunchKernelGGL(router_small_kernel, dim3((unsigned)ceil_div(a.E, 16)), dim3(64 * kSmallWaves), 0, s, a);
    return hipGetLastError();
  }
  const dim3 grid((unsigned)ceil_div(a.T, kRouterRows), (unsigned)ceil_div(a.E, kRouterExperts));
  hipLaunchKernelGGL(router_kernel, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
