// GPU-resident routing for the MoE layer on gfx950.
//
// The Lily pages keep the routing histogram, prefix scan, scatter and block
// map inside one GPU command buffer so no CPU synchronisation happens inside
// an MoE layer (Lily-EN "Prefill: Keep Weights Packed, Keep Routing on the
// GPU"; Lily-ES "Precarga: mantenga los pesos empaquetados, siga enrutando en
// la GPU"). Here that is two kernels on one stream whose grids depend only on
// T, never on routed counts:
//
//   topk  one wave per token: the k best logits by (value desc, index asc),
//         softmax gates over them, and a 64-bit LDS bitmask per expert for
//         every 64-token sub-chunk (atomicOr is order independent, so the
//         masks are deterministic). Extra workgroups convert x to fp16 and
//         zero y for the combine.
//   scan  one workgroup per sub-chunk: per-expert totals and the sub-chunk's
//         prefix from popcounts of the masks, the exclusive scan over experts,
//         and the stable scatter pos = offset[e] + prefix[c][e] +
//         popcount(mask[c][e] & lanes below t). Workgroup 0 also writes counts,
//         offsets, the 32-row block map and the GEMM work list.
//
// Pages cited (titles as published):
//   Lily-EN  "Perplexity Open Sources Lily: A Rust + Metal Inference Engine
//            for Qwen3.6-35B-A3B on Apple Silicon" (insight.aitobox.com)
//   Lily-ES  "Perplexity open sources Lily: un motor de inferencia ... para
//            Qwen3.6-35B-A3B en Apple Silicon" (7minutos.es)

#include "moe_internal.h"

#include <hip/hip_fp16.h>

namespace moe {
namespace {

constexpr int kWave = 64;
constexpr int kMaxVpl = MOE_MAX_EXPERTS / kWave;  // logits per lane at E = 1024

// Strict total order of router candidates: larger logit first; equal logits
// (IEEE ==, so -0.0 ties +0.0) go to the lower expert index.
__device__ __forceinline__ bool better(float av, int ai, float bv, int bi) {
  return av > bv || (av == bv && ai < bi);
}

__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t two_bf16) {
  float lo = __uint_as_float(two_bf16 << 16);
  float hi = __uint_as_float(two_bf16 & 0xFFFF0000u);
  __half hl = __float2half_rn(lo), hh = __float2half_rn(hi);
  return (uint32_t)__half_as_ushort(hl) | ((uint32_t)__half_as_ushort(hh) << 16);
}

// x (bf16, natural order) -> x16 (fp16, each 8-run stored as 0,4,1,5,2,6,3,7),
// and y = 0. Grid-stride over the auxiliary workgroups.
__device__ void aux_role(const TopkArgs &a, int aux_id, int n_aux) {
  const int64_t n8 = (int64_t)a.T * a.d / 8;
  const int64_t stride = (int64_t)n_aux * kThreads;
  for (int64_t i = (int64_t)aux_id * kThreads + threadIdx.x; i < n8; i += stride) {
    uint4 v = reinterpret_cast<const uint4 *>(a.x)[i];
    // v.x = (e0,e1) v.y = (e2,e3) v.z = (e4,e5) v.w = (e6,e7)
    uint32_t p0 = bf16x2_to_f16x2(__builtin_amdgcn_perm(v.z, v.x, 0x05040100u));  // (e0,e4)
    uint32_t p1 = bf16x2_to_f16x2(__builtin_amdgcn_perm(v.z, v.x, 0x07060302u));  // (e1,e5)
    uint32_t p2 = bf16x2_to_f16x2(__builtin_amdgcn_perm(v.w, v.y, 0x05040100u));  // (e2,e6)
    uint32_t p3 = bf16x2_to_f16x2(__builtin_amdgcn_perm(v.w, v.y, 0x07060302u));  // (e3,e7)
    reinterpret_cast<uint4 *>(a.x16)[i] = make_uint4(p0, p1, p2, p3);
  }
  const int64_t n4 = (int64_t)a.T * a.d / 4;
  for (int64_t i = (int64_t)aux_id * kThreads + threadIdx.x; i < n4; i += stride)
    reinterpret_cast<float4 *>(a.y)[i] = make_float4(0.f, 0.f, 0.f, 0.f);
}

template <int VPL>
__device__ void route_role(const TopkArgs &a, int c) {
  __shared__ unsigned long long smask[MOE_MAX_EXPERTS];
  const int E = a.E, k = a.k;
  for (int e = threadIdx.x; e < E; e += kThreads) smask[e] = 0ull;
  __syncthreads();

  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  for (int i = 0; i < kSubChunk / (kThreads / kWave); ++i) {
    const int tl = wave * (kSubChunk / (kThreads / kWave)) + i;  // token within sub-chunk
    const int t = c * kSubChunk + tl;
    if (t >= a.T) break;
    float v[VPL];
    const float *row = a.logits + (int64_t)t * E;
#pragma unroll
    for (int r = 0; r < VPL; ++r) {
      const int e = lane + kWave * r;
      v[r] = e < E ? row[e] : -__builtin_inff();
    }
    uint32_t taken = 0;
    float sel_v = 0.f;
    int sel_i = 0;
    for (int j = 0; j < k; ++j) {
      float bv = -__builtin_inff();
      int bi = 0x7FFFFFFF;
#pragma unroll
      for (int r = 0; r < VPL; ++r) {
        const int e = lane + kWave * r;
        if (e < E && !((taken >> r) & 1u) && better(v[r], e, bv, bi)) { bv = v[r]; bi = e; }
      }
#pragma unroll
      for (int off = kWave / 2; off > 0; off >>= 1) {
        const float ov = __shfl_xor(bv, off, kWave);
        const int oi = __shfl_xor(bi, off, kWave);
        if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
      }
      if ((bi % kWave) == lane) taken |= 1u << (bi / kWave);
      if (lane == j) { sel_v = bv; sel_i = bi; }
    }
    // softmax over the k picked logits (slot 0 holds the largest)
    const float v0 = __shfl(sel_v, 0, kWave);
    float ex = lane < k ? expf(sel_v - v0) : 0.f;
    float sum = ex;
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) sum += __shfl_xor(sum, off, kWave);
    if (lane < k) {
      a.topk_ids[(int64_t)t * k + lane] = sel_i;
      a.topk_w[(int64_t)t * k + lane] = ex / sum;
      atomicOr(&smask[sel_i], 1ull << tl);
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kThreads) a.masks[(int64_t)c * E + e] = smask[e];
}

template <int VPL>
__global__ __launch_bounds__(kThreads) void topk_kernel(TopkArgs a) {
  if ((int)blockIdx.x < a.n_route_blocks) {
    route_role<VPL>(a, blockIdx.x);
  } else {
    aux_role(a, blockIdx.x - a.n_route_blocks, gridDim.x - a.n_route_blocks);
  }
}

// Exclusive scan of vals[0..n) (n <= 1024) in LDS by one 256-thread workgroup.
// Returns the total. scratch must hold kThreads / 64 ints.
__device__ int block_exclusive_scan(int *vals, int n, int *scratch) {
  const int per = (n + kThreads - 1) / kThreads;  // <= 4
  const int lo = threadIdx.x * per;
  int local[4];
  int run = 0;
  for (int i = 0; i < per; ++i) {
    local[i] = (lo + i < n) ? vals[lo + i] : 0;
    run += local[i];
  }
  // inclusive wave scan of run
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  int incl = run;
  for (int off = 1; off < kWave; off <<= 1) {
    const int o = __shfl_up(incl, off, kWave);
    if (lane >= off) incl += o;
  }
  if (lane == kWave - 1) scratch[wave] = incl;
  __syncthreads();
  int wave_base = 0, total = 0;
  for (int w = 0; w < kThreads / kWave; ++w) {
    if (w < wave) wave_base += scratch[w];
    total += scratch[w];
  }
  int base = wave_base + incl - run;
  for (int i = 0; i < per; ++i) {
    if (lo + i < n) vals[lo + i] = base;
    base += local[i];
  }
  __syncthreads();
  return total;
}

__global__ __launch_bounds__(kThreads) void scan_kernel(ScanArgs a) {
  __shared__ int s_tot[MOE_MAX_EXPERTS];
  __shared__ int s_pre[MOE_MAX_EXPERTS];
  __shared__ int s_off[MOE_MAX_EXPERTS];
  __shared__ int s_blk[MOE_MAX_EXPERTS];
  __shared__ int s_unit[MOE_MAX_EXPERTS];
  __shared__ int s_scratch[kThreads / kWave];
  const int E = a.E, k = a.k, T = a.T;
  const int c = blockIdx.x;
  const int C = (T + kSubChunk - 1) / kSubChunk;

  for (int e = threadIdx.x; e < E; e += kThreads) {
    int tot = 0, pre = 0;
    for (int cc = 0; cc < C; ++cc) {
      const int pc = __popcll(a.masks[(int64_t)cc * E + e]);
      if (cc < c) pre += pc;
      tot += pc;
    }
    s_tot[e] = tot;
    s_pre[e] = pre;
    s_off[e] = tot;
  }
  __syncthreads();
  const int total = block_exclusive_scan(s_off, E, s_scratch);  // == T*k

  // stable scatter of this sub-chunk's (token, slot) pairs
  for (int idx = threadIdx.x; idx < kSubChunk * k; idx += kThreads) {
    const int tl = idx / k, j = idx % k;
    const int t = c * kSubChunk + tl;
    if (t >= T) continue;
    const int e = a.topk_ids[(int64_t)t * k + j];
    const uint64_t m = a.masks[(int64_t)c * E + e];
    const uint64_t below = tl == 0 ? 0ull : (m & ((1ull << tl) - 1ull));
    const int pos = s_off[e] + s_pre[e] + __popcll(below);
    a.sorted_pair[pos] = t * k + j;
    a.sorted_token[pos] = t;
    a.pair_pos[(int64_t)t * k + j] = pos;
  }
  if (c != 0) return;

  // workgroup 0: counts, offsets, block map and GEMM work list
  for (int e = threadIdx.x; e < E; e += kThreads) {
    a.counts[e] = s_tot[e];
    a.offsets[e] = s_off[e];
    s_blk[e] = (s_tot[e] + MOE_BLOCK_ROWS - 1) / MOE_BLOCK_ROWS;
    s_unit[e] = (s_tot[e] + kUnitRows - 1) / kUnitRows;
  }
  if (threadIdx.x == 0) a.offsets[E] = total;
  __syncthreads();
  const int nblocks = block_exclusive_scan(s_blk, E, s_scratch);
  for (int e = threadIdx.x; e < E; e += kThreads) {
    const int tot = s_tot[e];
    for (int b = 0; b * MOE_BLOCK_ROWS < tot; ++b) {
      int32_t *ent = a.block_map + 3 * (int64_t)(s_blk[e] + b);
      ent[0] = e;
      ent[1] = s_off[e] + b * MOE_BLOCK_ROWS;
      ent[2] = min(MOE_BLOCK_ROWS, tot - b * MOE_BLOCK_ROWS);
    }
  }
  for (int i = nblocks + threadIdx.x; i < a.max_blocks; i += kThreads) {
    a.block_map[3 * (int64_t)i + 0] = -1;
    a.block_map[3 * (int64_t)i + 1] = 0;
    a.block_map[3 * (int64_t)i + 2] = 0;
  }
  if (threadIdx.x == 0) *a.num_blocks = nblocks;
  if (a.units == nullptr) return;
  __syncthreads();
  const int nunits = block_exclusive_scan(s_unit, E, s_scratch);
  for (int e = threadIdx.x; e < E; e += kThreads) {
    const int tot = s_tot[e];
    for (int u = 0; u * kUnitRows < tot; ++u) {
      int32_t *ent = a.units + 3 * (int64_t)(s_unit[e] + u);
      ent[0] = e;
      ent[1] = s_off[e] + u * kUnitRows;
      ent[2] = min(kUnitRows, tot - u * kUnitRows);
    }
  }
  if (threadIdx.x == 0) *a.num_units = nunits;
}

}  // namespace

hipError_t launch_topk(const TopkArgs &a, int n_aux_blocks, hipStream_t s) {
  const int vpl = (a.E + kWave - 1) / kWave;
  const dim3 grid(a.n_route_blocks + n_aux_blocks), block(kThreads);
  if (vpl <= 1)       hipLaunchKernelGGL(topk_kernel<1>, grid, block, 0, s, a);
  else if (vpl <= 2)  hipLaunchKernelGGL(topk_kernel<2>, grid, block, 0, s, a);
  else if (vpl <= 4)  hipLaunchKernelGGL(topk_kernel<4>, grid, block, 0, s, a);
  else if (vpl <= 8)  hipLaunchKernelGGL(topk_kernel<8>, grid, block, 0, s, a);
  else                hipLaunchKernelGGL(topk_kernel<kMaxVpl>, grid, block, 0, s, a);
  return hipGetLastError();
}

hipError_t launch_scan(const ScanArgs &a, hipStream_t s) {
  const int C = (a.T + kSubChunk - 1) / kSubChunk;
  hipLaunchKernelGGL(scan_kernel, dim3(C), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
