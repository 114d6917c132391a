// GPU-resident routing for the MoE layer on gfx950.
//
// The Lily pages keep the routing histogram, prefix scan, scatter and block
// map inside one GPU command buffer so no CPU synchronisation happens inside
// an MoE layer (Lily-EN "Prefill: Keep Weights Packed, Keep Routing on the
// GPU"; Lily-ES "Precarga: mantenga los pesos empaquetados, siga enrutando en
// la GPU"). Here that is two kernels on one stream (three above 32768
// pairs) whose grids depend only on T, never on routed counts:
//
//   topk  one wave per token (the x -> fp16 conversion in workgroups of its
//         own, after the routing ones). Every candidate becomes a 64-bit key
//         (order-preserving logit bits, then the inverted expert index), so
//         "larger logit, then lower index" is plain unsigned order and all
//         keys are distinct. Each lane sorts its own keys; k rounds of a wave
//         max over the lanes' heads (DPP inside each 16-lane row, readlane
//         across rows, the logit half first, then the index half) pick the
//         experts; the gates are the softmax over the k picked logits. The
//         same workgroups then convert x to fp16 for the GEMMs.
//   scatter one workgroup per 64-token sub-chunk c: the expert totals and
//         the counts of the pairs before c (up to 32768 pairs each workgroup
//         counts every pair itself in LDS; above that a count pass of one
//         workgroup per sub-chunk writes cnt[c][e] first and the scatter
//         takes column sums of it), an exclusive scan over experts gives the
//         offsets, and a 64-bit token mask per expert for its own sub-chunk
//         gives the stable scatter:
//           pos = offset[e] + before[e] + popcount(mask[e] & tokens below t).
//         Integer atomics commute, so the result is deterministic.
//         One more workgroup writes counts, offsets and the 32-row block
//         map, and (for the layer) another one the GEMM work list.
//
// Pages cited (titles as published):
//   Lily-EN  "Perplexity Open Sources Lily: A Rust + Metal Inference Engine
//            for Qwen3.6-35B-A3B on Apple Silicon" (insight.aitobox.com)
//   Lily-ES  "Perplexity open sources Lily: un motor de inferencia ... para
//            Qwen3.6-35B-A3B en Apple Silicon" (7minutos.es)

#include "moe_internal.h"
#include "topk_device.h"

#include <hip/hip_fp16.h>

#include <algorithm>

namespace moe {
namespace {

constexpr int kWave = 64;
constexpr int kWaves = kThreads / kWave;
constexpr int kMaxVpl = MOE_MAX_EXPERTS / kWave;  // logits per lane at E = 1024
constexpr int kClasses = kUnitRows / 16;           // GEMM unit size classes (16-row blocks)
// Up to this many (token, slot) pairs every scatter workgroup counts all of
// them itself (each reads T*k ids, from L2); above it a count pass writes
// per-sub-chunk counts first.
constexpr int64_t kInlinePairs = 32768;

template <int VPL>
__device__ void route_token(const TopkArgs &a, int t, int lane) {
  int id;
  float g;
  topk_wave<VPL>(a.logits + (int64_t)t * a.E, a.E, a.k, lane, id, g);
  if (lane < a.k) {
    a.topk_ids[(int64_t)t * a.k + lane] = id;
    a.topk_w[(int64_t)t * a.k + lane] = g;
  }
  if (a.ids8 && lane < a.k) a.ids8[(int64_t)t * a.k + lane] = (uint8_t)id;  // the scatter's count reads these
}

__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t two_bf16) {
  const float lo = __uint_as_float(two_bf16 << 16);
  const float hi = __uint_as_float(two_bf16 & 0xFFFF0000u);
  return (uint32_t)__half_as_ushort(__float2half_rn(lo)) |
         ((uint32_t)__half_as_ushort(__float2half_rn(hi)) << 16);
}

// CHECK: report x values that do not convert to a finite fp16.
template <int VPL, bool CHECK>
__global__ __launch_bounds__(kThreads) void topk_kernel(TopkArgs a) {
  const int lane = threadIdx.x % kWave;
  if ((int)blockIdx.x < a.topk_wgs) {
    // routing workgroups: one token per wave
    const int gwave = blockIdx.x * kWaves + threadIdx.x / kWave;
    const int nwaves = a.topk_wgs * kWaves;
    for (int t = gwave; t < a.T; t += nwaves) route_token<VPL>(a, t, lane);
    return;
  }
  // conversion workgroups (their own, so a routing workgroup ends with its
  // last top-k): x (bf16, natural order) -> x16 (fp16, each 8-run stored as
  // 0,4,1,5,2,6,3,7), kUnroll 16-byte chunks per thread in flight
  constexpr int kUnroll = 4;
  const int cb = blockIdx.x - a.topk_wgs, ncb = gridDim.x - a.topk_wgs;
  const int64_t stride = (int64_t)ncb * kThreads;
  const int64_t n8 = a.x16 ? (int64_t)a.T * a.d / 8 : 0;
  int64_t i0 = (int64_t)cb * kThreads + threadIdx.x;
  uint4 v[kUnroll];
  auto load = [&]() {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t i = i0 + u * stride;
      v[u] = i < n8 ? reinterpret_cast<const uint4 *>(a.x)[i] : make_uint4(0, 0, 0, 0);
    }
  };
  load();
  for (; i0 < n8; i0 += kUnroll * stride) {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t i = i0 + u * stride;
      if (i < n8) {
        // v.x = (e0,e1) v.y = (e2,e3) v.z = (e4,e5) v.w = (e6,e7)
        const uint32_t p0 = bf16x2_to_f16x2(__builtin_amdgcn_perm(v[u].z, v[u].x, 0x05040100u));  // (e0,e4)
        const uint32_t p1 = bf16x2_to_f16x2(__builtin_amdgcn_perm(v[u].z, v[u].x, 0x07060302u));  // (e1,e5)
        const uint32_t p2 = bf16x2_to_f16x2(__builtin_amdgcn_perm(v[u].w, v[u].y, 0x05040100u));  // (e2,e6)
        const uint32_t p3 = bf16x2_to_f16x2(__builtin_amdgcn_perm(v[u].w, v[u].y, 0x07060302u));  // (e3,e7)
        reinterpret_cast<uint4 *>(a.x16)[i] = make_uint4(p0, p1, p2, p3);
        if (CHECK)
          note_overflow(a.overflow, f16x2_nonfinite(p0) || f16x2_nonfinite(p1) || f16x2_nonfinite(p2) ||
                                        f16x2_nonfinite(p3), MOE_OVERFLOW_X);
      }
    }
    if (i0 + kUnroll * stride < n8) {
      i0 += kUnroll * stride;
      load();
      i0 -= kUnroll * stride;
    }
  }
}

__device__ __forceinline__ void add_f16x8(float *acc, uint4 v, float w) {
  const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    acc[2 * i] += w * __half2float(__ushort_as_half((uint16_t)(u[i] & 0xFFFFu)));
    acc[2 * i + 1] += w * __half2float(__ushort_as_half((uint16_t)(u[i] >> 16)));
  }
}

// Weighted combine (the fourth part of the layer): one workgroup per token,
// eight outputs per thread, terms added in slot order then the shared
// expert, so y is reproducible bit for bit.
__global__ __launch_bounds__(kThreads) void combine_kernel(CombineArgs a) {
  const int t = blockIdx.x;
  const int k = a.k;
  __shared__ int s_pos[MOE_MAX_EXPERTS];
  __shared__ float s_w[MOE_MAX_EXPERTS];
  for (int j = threadIdx.x; j < k; j += kThreads) {
    s_pos[j] = a.pair_pos[(int64_t)t * k + j];
    s_w[j] = a.topk_w[(int64_t)t * k + j];
  }
  __syncthreads();
  for (int c = threadIdx.x * 8; c < a.d; c += kThreads * 8) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    // eight rows at a time, all requested before the first is added
    // (clamped: past k the last row again, not added); slot order kept
    for (int j0 = 0; j0 < k; j0 += 8) {
      uint4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        v[u] = *reinterpret_cast<const uint4 *>(a.o + (int64_t)s_pos[min(j0 + u, k - 1)] * a.d + c);
      uint4 vs = make_uint4(0u, 0u, 0u, 0u);
      if (a.o_sh && j0 + 8 >= k) vs = *reinterpret_cast<const uint4 *>(a.o_sh + (int64_t)t * a.d + c);
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (j0 + u < k) add_f16x8(acc, v[u], s_w[j0 + u]);
      if (a.o_sh && j0 + 8 >= k) add_f16x8(acc, vs, 1.f);
    }
    float4 *dst = reinterpret_cast<float4 *>(a.y + (int64_t)t * a.d + c);
    dst[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
    dst[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
  }
}

// Exclusive scan of vals[0..n) (n <= 1024) in LDS by one 256-thread workgroup.
// Returns the total. scratch holds kWaves ints.
__device__ int block_exclusive_scan(int *vals, int n, int *scratch) {
  const int per = (n + kThreads - 1) / kThreads;  // <= 4
  const int lo = threadIdx.x * per;
  int local[4];
  int run = 0;
  for (int i = 0; i < per; ++i) {
    local[i] = (lo + i < n) ? vals[lo + i] : 0;
    run += local[i];
  }
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  int incl = run;
  for (int off = 1; off < kWave; off <<= 1) {
    const int o = __shfl_up(incl, off, kWave);
    if (lane >= off) incl += o;
  }
  if (lane == kWave - 1) scratch[wave] = incl;
  __syncthreads();
  int wave_base = 0, total = 0;
  for (int w = 0; w < kWaves; ++w) {
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

// Per 64-token sub-chunk c: how many of its (token, slot) pairs pick each
// expert, into cnt[c][e].
__global__ __launch_bounds__(kThreads) void count_kernel(ScanArgs a) {
  __shared__ int s_cnt[MOE_MAX_EXPERTS];
  const int E = a.E, k = a.k;
  const int c = blockIdx.x;
  const int64_t tk = (int64_t)a.T * k;
  const int64_t lo = (int64_t)c * kSubChunk * k, hi = min(tk, lo + (int64_t)kSubChunk * k);
  for (int e = threadIdx.x; e < E; e += kThreads) s_cnt[e] = 0;
  __syncthreads();
  // four ids per thread at a time, all requested before the first is used
  // (clamped: past the end the last id again, not counted)
  for (int64_t base = lo + threadIdx.x; base < hi; base += 4 * kThreads) {
    int ids[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) ids[u] = a.topk_ids[min(base + (int64_t)u * kThreads, hi - 1)];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (base + (int64_t)u * kThreads < hi) atomicAdd(&s_cnt[ids[u]], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kThreads) a.chunk_counts[(int64_t)c * E + e] = s_cnt[e];
}

// Histogram of n4 groups of four expert ids (16-byte loads, KB per thread in
// flight): groups below lo4 into pre, the others into post.
template <int KB>
__device__ __forceinline__ void count_ids4(const int32_t *ids, int64_t n4, int64_t lo4, int *pre, int *post) {
  const int4 *ids4 = reinterpret_cast<const int4 *>(ids);
  for (int64_t b0 = threadIdx.x; b0 < n4; b0 += (int64_t)KB * kThreads) {
    int4 v[KB];
#pragma unroll
    for (int u = 0; u < KB; ++u) v[u] = ids4[min(b0 + (int64_t)u * kThreads, n4 - 1)];
#pragma unroll
    for (int u = 0; u < KB; ++u) {
      const int64_t i4 = b0 + (int64_t)u * kThreads;
      if (i4 < n4) {
        int *h = i4 < lo4 ? pre : post;
        atomicAdd(&h[v[u].x], 1);
        atomicAdd(&h[v[u].y], 1);
        atomicAdd(&h[v[u].z], 1);
        atomicAdd(&h[v[u].w], 1);
      }
    }
  }
}

// Histogram of n16 groups of sixteen byte ids (16-byte loads, KB per thread
// in flight): groups below lo16 into pre, the others into post.
template <int KB>
__device__ __forceinline__ void count_ids16(const uint8_t *ids, int n16, int lo16, int *pre, int *post) {
  const uint4 *ids16 = reinterpret_cast<const uint4 *>(ids);
  for (int b0 = threadIdx.x; b0 < n16; b0 += KB * kThreads) {
    uint4 v[KB];
#pragma unroll
    for (int u = 0; u < KB; ++u) v[u] = ids16[min(b0 + u * kThreads, n16 - 1)];
#pragma unroll
    for (int u = 0; u < KB; ++u) {
      const int i16 = b0 + u * kThreads;
      if (i16 < n16) {
        int *h = i16 < lo16 ? pre : post;
        const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int b = 0; b < 4; ++b) atomicAdd(&h[(w[q] >> (8 * b)) & 0xFFu], 1);
      }
    }
  }
}

// GEMM work list (one workgroup): each expert's rows split into
// ceil(rows / unit_rows) units whose sizes differ by at most one, listed by 16-row size class, largest first,
// so the GEMM (which hands units to workgroups in list order) starts the
// longest ones first. Positions come from ballots: each wave counts its
// units per class, and a unit's place within its class is (earlier waves'
// units of the class, earlier rounds of this wave, lanes below it in this
// round). Expert e is thread e % kThreads's round e / kThreads (then one
// round per further unit), so the list is the same on every call. Only
// 32-bit arithmetic: a 64-bit division per unit cost about a microsecond
// on this workgroup, which finishes last.
__device__ void write_units(const ScanArgs &a, const int *s_tot, const int *s_off) {
  const int E = a.E, ur = a.unit_rows;
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  __shared__ int s_wcnt[kWaves][kClasses + 1];
  __shared__ int s_base[kWaves][kClasses + 1];
  // visits every unit of this thread's experts in a wave-uniform order;
  // f(class, or -1 when this lane has no unit in the round; rows; expert; first row)
  auto rounds = [&](auto &&f) {
    for (int e0 = 0; e0 < E; e0 += kThreads) {
      const int e = e0 + threadIdx.x;
      const int tot = e < E ? s_tot[e] : 0, nu = (tot + ur - 1) / ur;
      // q rows per unit, the first rr units one more (32-bit arithmetic only)
      const int q = nu > 0 ? tot / nu : 0, rr = tot - q * nu;
      for (int u = 0; __ballot(u < nu) != 0ull; ++u) {
        int cls = -1, b0 = 0, rows = 0;
        if (u < nu) {
          b0 = u * q + min(u, rr);
          rows = q + (u < rr ? 1 : 0);
          cls = kClasses - (rows + 15) / 16;
        }
        f(cls, rows, e, b0);
      }
    }
  };
  int cnt[kClasses + 1];
#pragma unroll
  for (int c = 0; c <= kClasses; ++c) cnt[c] = 0;
  rounds([&](int cls, int, int, int) {
#pragma unroll
    for (int c = 0; c <= kClasses; ++c) cnt[c] += (int)__popcll(__ballot(cls == c));
  });
  if (lane == 0) {
#pragma unroll
    for (int c = 0; c <= kClasses; ++c) s_wcnt[wave][c] = cnt[c];
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int c = 0; c <= kClasses; ++c)
      for (int w = 0; w < kWaves; ++w) {
        s_base[w][c] = run;
        run += s_wcnt[w][c];
      }
    *a.num_units = run;
  }
  __syncthreads();
#pragma unroll
  for (int c = 0; c <= kClasses; ++c) cnt[c] = s_base[wave][c];
  rounds([&](int cls, int rows, int e, int b0) {
    int slot = 0;
#pragma unroll
    for (int c = 0; c <= kClasses; ++c) {
      const uint64_t m = __ballot(cls == c);
      if (cls == c)
        slot = cnt[c] + __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
      cnt[c] += (int)__popcll(m);
    }
    if (cls >= 0) {
      int32_t *ent = a.units + 3 * (int64_t)slot;
      ent[0] = e;
      ent[1] = s_off[e] + b0;
      ent[2] = rows;
    }
  });
}

// Per sub-chunk c: expert totals and the counts of the sub-chunks before c
// (counted here, or column sums of cnt), offsets by an exclusive scan over experts, and the
// stable scatter of c's pairs:
//   pos = offset[e] + before[e] + popcount(mask[e] & tokens of c below t).
// Workgroup C (with no pairs of its own) writes counts, offsets and the
// 32-row block map meanwhile, and workgroup C + 1 (launched with a work list)
// the GEMM work list.
__global__ __launch_bounds__(kThreads) void scatter_kernel(ScanArgs a) {
  __shared__ int s_tot[MOE_MAX_EXPERTS];
  __shared__ int s_pre[MOE_MAX_EXPERTS];
  __shared__ int s_off[MOE_MAX_EXPERTS];
  __shared__ int s_aux[MOE_MAX_EXPERTS];
  __shared__ unsigned long long s_mask[MOE_MAX_EXPERTS];
  __shared__ int s_scratch[kWaves];
  const int E = a.E, k = a.k, T = a.T;
  const int c = blockIdx.x, C = (int)((T + kSubChunk - 1) / kSubChunk);  // sub-chunks; workgroups C, C + 1 hold none
  // pair indices fit 32 bits (T * k <= MOE_MAX_CALL_TOKENS * 64)
  const int tk = T * k;
  const int lo = c * kSubChunk * k, hi = min(tk, lo + kSubChunk * k);
  // this thread's pairs lo + tid + u * kThreads are (token tl, slot rm) of
  // the sub-chunk, stepped without a division per pair
  const int kq = kThreads / k, kr = kThreads - kq * k;
  const int tl0 = (int)threadIdx.x / k, rm0 = (int)threadIdx.x - tl0 * k;
  auto step = [&](int &tl, int &rm) {
    tl += kq;
    rm += kr;
    if (rm >= k) {
      rm -= k;
      ++tl;
    }
  };

  // The first kIdCache ids of this thread's pairs (lo + tid + u * kThreads)
  // are requested first and kept for both passes below; every load here is
  // unconditional (clamped index), so none waits on another.
  constexpr int kIdCache = 4;
  int idc[kIdCache];
  if (c < C) {
#pragma unroll
    for (int u = 0; u < kIdCache; ++u) idc[u] = a.topk_ids[min(lo + (int)threadIdx.x + u * kThreads, hi - 1)];
  }
  auto pair_id = [&](int u, int idx) -> int {
    int id = 0;
#pragma unroll
    for (int q = 0; q < kIdCache; ++q)
      if (u == q) id = idc[q];
    return u < kIdCache ? id : a.topk_ids[idx];
  };

  if (a.count_inline) {
    // Up to kInlinePairs pairs: the workgroup counts every pair itself, those
    // before its sub-chunk into s_pre and the rest into s_aux (free until the
    // block map), thirty-two id loads per thread in flight at a time.
    for (int e = threadIdx.x; e < E; e += kThreads) {
      s_pre[e] = 0;
      s_aux[e] = 0;
      s_mask[e] = 0ull;
    }
    __syncthreads();
    if (a.ids8) {
      // byte ids (E <= 256): sixteen per 16-byte load, a quarter of the
      // bytes every workgroup reads (lo is a multiple of 64 k, so a group of
      // sixteen falls on one side of it)
      count_ids16<4>(a.ids8, tk >> 4, lo >> 4, s_pre, s_aux);
    } else if (a.ids_vec && tk > 16 * kThreads) {
      // more than 4096 pairs, 16-byte aligned ids, T*k a multiple of 4: four
      // ids per load, sixteen loads per thread in flight (lo is a multiple
      // of 64, so the four ids of a load fall on one side of it); up to 4096
      // pairs the one-id loads below were faster (7.4 against 8.0 us at T=512)
      count_ids4<16>(a.topk_ids, (int64_t)(tk >> 2), (int64_t)(lo >> 2), s_pre, s_aux);
    } else {
      constexpr int kBatch = 32;
      for (int b0 = threadIdx.x; b0 < tk; b0 += kBatch * kThreads) {
        int v[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) v[u] = a.topk_ids[min(b0 + u * kThreads, tk - 1)];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          const int idx = b0 + u * kThreads;
          if (idx < tk) atomicAdd(idx < lo ? &s_pre[v[u]] : &s_aux[v[u]], 1);
        }
      }
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += kThreads) {
      const int tot = s_pre[e] + s_aux[e];
      s_tot[e] = tot;
      s_off[e] = tot;
    }
  } else {
    for (int e = threadIdx.x; e < E; e += kThreads) {
      int tot = 0, pre = 0;
      for (int c0 = 0; c0 < C; c0 += 16) {  // sixteen independent loads in flight
        int v[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) v[u] = a.chunk_counts[(int64_t)min(c0 + u, C - 1) * E + e];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          tot += c0 + u < C ? v[u] : 0;
          pre += c0 + u < c ? v[u] : 0;
        }
      }
      s_tot[e] = tot;
      s_pre[e] = pre;
      s_off[e] = tot;
      s_mask[e] = 0ull;
    }
  }
  __syncthreads();
  {
    int u = 0, tl = tl0, rm = rm0;
    for (int idx = lo + (int)threadIdx.x; idx < hi; idx += kThreads, ++u, step(tl, rm))
      atomicOr(&s_mask[pair_id(u, idx)], 1ull << tl);
  }
  const int total = block_exclusive_scan(s_off, E, s_scratch);  // == T*k (syncs inside)

  // stable scatter of this sub-chunk's (token, slot) pairs
  int u = 0, tl = tl0, rm = rm0;
  for (int idx = lo + (int)threadIdx.x; idx < hi; idx += kThreads, ++u, step(tl, rm)) {
    const int t = c * kSubChunk + tl;
    const int e = pair_id(u, idx);
    const uint64_t m = s_mask[e];
    const uint64_t below = tl == 0 ? 0ull : (m & ((1ull << tl) - 1ull));
    const int pos = s_off[e] + s_pre[e] + __popcll(below);
    a.sorted_pair[pos] = idx;
    a.sorted_token[pos] = t;
    a.pair_pos[idx] = pos;
  }
  if (c < C) return;
  if (c == C + 1) {  // with a work list: a second extra workgroup writes it
    write_units(a, s_tot, s_off);
    return;
  }

  // the first extra workgroup (neither holds pairs): counts, offsets and the
  // block map, beside the scatter of the others
  for (int e = threadIdx.x; e < E; e += kThreads) {
    a.counts[e] = s_tot[e];
    a.offsets[e] = s_off[e];
    s_aux[e] = (s_tot[e] + MOE_BLOCK_ROWS - 1) / MOE_BLOCK_ROWS;
  }
  if (threadIdx.x == 0) a.offsets[E] = total;
  __syncthreads();
  const int nblocks = block_exclusive_scan(s_aux, E, s_scratch);
  for (int e = threadIdx.x; e < E; e += kThreads) {
    const int tot = s_tot[e];
    for (int b = 0; b * MOE_BLOCK_ROWS < tot; ++b) {
      int32_t *ent = a.block_map + 3 * (int64_t)(s_aux[e] + b);
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
}

}  // namespace

hipError_t launch_topk(const TopkArgs &args, hipStream_t s, hipEvent_t start, hipEvent_t stop) {
  TopkArgs a = args;
  const int vpl = (a.E + kWave - 1) / kWave;
  // routing workgroups (one token per wave), then conversion workgroups
  a.topk_wgs = (int)std::min<int64_t>(std::max<int64_t>(ceil_div(a.T, kWaves), 1), 4096);
  const int conv = a.x16 ? (int)std::min<int64_t>(1024, ceil_div((int64_t)a.T * a.d / 8, 4 * kThreads)) : 0;
  const dim3 grid(a.topk_wgs + conv), block(kThreads);
  if (a.overflow) {
    if (vpl <= 1)       hipExtLaunchKernelGGL((topk_kernel<1, true>), grid, block, 0, s, start, stop, 0, a);
    else if (vpl <= 2)  hipExtLaunchKernelGGL((topk_kernel<2, true>), grid, block, 0, s, start, stop, 0, a);
    else if (vpl <= 4)  hipExtLaunchKernelGGL((topk_kernel<4, true>), grid, block, 0, s, start, stop, 0, a);
    else if (vpl <= 8)  hipExtLaunchKernelGGL((topk_kernel<8, true>), grid, block, 0, s, start, stop, 0, a);
    else                hipExtLaunchKernelGGL((topk_kernel<kMaxVpl, true>), grid, block, 0, s, start, stop, 0, a);
  } else {
    if (vpl <= 1)       hipExtLaunchKernelGGL((topk_kernel<1, false>), grid, block, 0, s, start, stop, 0, a);
    else if (vpl <= 2)  hipExtLaunchKernelGGL((topk_kernel<2, false>), grid, block, 0, s, start, stop, 0, a);
    else if (vpl <= 4)  hipExtLaunchKernelGGL((topk_kernel<4, false>), grid, block, 0, s, start, stop, 0, a);
    else if (vpl <= 8)  hipExtLaunchKernelGGL((topk_kernel<8, false>), grid, block, 0, s, start, stop, 0, a);
    else                hipExtLaunchKernelGGL((topk_kernel<kMaxVpl, false>), grid, block, 0, s, start, stop, 0, a);
  }
  return hipGetLastError();
}

hipError_t launch_combine(const CombineArgs &a, hipStream_t s, hipEvent_t stop) {
  hipExtLaunchKernelGGL(combine_kernel, dim3(a.T), dim3(kThreads), 0, s, nullptr, stop, 0, a);
  return hipGetLastError();
}

hipError_t launch_scan(const ScanArgs &args, hipStream_t s, hipEvent_t stop) {
  ScanArgs a = args;
  const int C = (int)ceil_div(a.T, kSubChunk);
  a.count_inline = (int64_t)a.T * a.k <= kInlinePairs;
  a.ids_vec = ((uintptr_t)a.topk_ids % 16) == 0 && ((int64_t)a.T * a.k) % 4 == 0;
  if (!a.count_inline) {
    hipLaunchKernelGGL(count_kernel, dim3(C), dim3(kThreads), 0, s, a);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  // one workgroup per sub-chunk, plus one for the block map and one for the
  // work list
  hipExtLaunchKernelGGL(scatter_kernel, dim3(C + 1 + (a.units ? 1 : 0)), dim3(kThreads), 0, s, nullptr, stop, 0, a);
  return hipGetLastError();
}

}  // namespace moe
