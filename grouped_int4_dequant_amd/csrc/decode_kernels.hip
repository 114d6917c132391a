// Decode-shape MoE layer (a few tokens per call) for gfx950: two kernels.
//
// At batch-1 decode the layer has almost no weight reuse, so the bytes of
// the touched experts set the time (Lily-EN "Decode: Minimize Bytes Moved
// Per Token"; Lily-ES "Decodificar: minimizar los bytes movidos por token").
// The prefill schedule gives each expert two workgroups; here the same
// arithmetic is spread over every CU and the launch count is cut to two:
//
//   gate/up  one workgroup per (distinct routed expert or the shared expert,
//            16 columns of h), one wave per 512 inputs.
//            Every workgroup first repeats the top-k for the call's tokens,
//            one token per wave (a wave max over order-preserving 64-bit
//            keys, as in the routing kernel), and ranks the distinct experts with a bitmap, so no
//            routing kernel runs before it. The waves' partial sums meet in
//            LDS; SwiGLU gives h per (token, slot), stored as fp16.
//   down     one workgroup per (token, 8 output columns), one wave per slot
//            (the k routed experts and the shared expert), 512 inputs each. A
//            wave's 16x16 MFMA tile holds its 8 columns twice, over the first
//            and the second 256 inputs, against tile rows that alternate
//            between h's two halves, so the wave runs 8 MFMAs and needs no
//            zeroing. h arrives as fp16 in the MFMA operand order. The partial
//            projections meet in LDS and are combined in slot order with the
//            gates: y = sum_j g_j (o_j' + o_j'') + o_shared, fp32, no atomics.
//
// Weights are rebuilt from the 4-bit codes exactly as in the prefill GEMM
// (rebuild_device.h) and multiplied with v_mfma_f32_16x16x32_f16; the rows
// beyond the call's tokens are zero.
//
// Pages cited (titles as published):
//   Lily-EN  "Perplexity Open Sources Lily: A Rust + Metal Inference Engine
//            for Qwen3.6-35B-A3B on Apple Silicon" (insight.aitobox.com)
//   Lily-ES  "Perplexity open sources Lily: un motor de inferencia ... para
//            Qwen3.6-35B-A3B en Apple Silicon" (7minutos.es)

#include "moe_internal.h"
#include "rebuild_device.h"
#include "topk_device.h"

namespace moe {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u4v __attribute__((ext_vector_type(4)));

constexpr int kSpan = 512;          // inputs per wave
constexpr int kSteps = kSpan / 128;  // 128-input steps per wave
constexpr int kMaxWaves = 8;         // gate/up waves per workgroup (d <= 4096)
constexpr int kDnResident = 768;      // down workgroups resident at once (3 per CU)
// Calls of up to this many tokens run one gate/up item per (token, slot) pair;
// longer ones one item per distinct expert.
#ifndef MOE_DECODE_PAIR_MAXT
#define MOE_DECODE_PAIR_MAXT 8
#endif
constexpr int kDecodePairMaxT = MOE_DECODE_PAIR_MAXT;

// Position of the r-th set bit of m (r < popcount(m)).
__device__ __forceinline__ int nth_bit(uint32_t m, int r) {
  for (int i = 0; i < r; ++i) m &= m - 1;
  return __ffs(m) - 1;
}

// (fp16 s, fp16 b + 8 s) of group 2 s + half from the packed bf16 scales and
// biases of eight consecutive groups.
__device__ __forceinline__ uint32_t group_consts(const u4v &sw, const u4v &bw, int s, int half) {
  const uint32_t sh = 16u * (uint32_t)half;
  return rb_pack_scale_bias((sw[s] >> sh) & 0xFFFFu, (bw[s] >> sh) & 0xFFFFu);
}

// Eight bf16 activations -> fp16 in the rebuild order (as one MFMA operand).
__device__ __forceinline__ uint4 x_chunk_h8(uint4 v) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  float xf[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    xf[2 * i] = __uint_as_float(w[i] << 16);
    xf[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
  return __builtin_bit_cast(uint4, rb_perm8(xf));
}

// ONE: calls of one token (T == 1) at d <= 2048, whose k picks are the
// distinct experts; their code requests are staged through LDS (below).
// Several tokens with up to 512 experts: five waves per SIMD (every T = 4
// workgroup resident at once); the one-token and 1024-expert forms keep
// their registers.
// PAIR (several tokens): each routed item is one (token, slot) pair, as at
// T = 1, instead of one distinct expert for all the tokens that picked it.
template <int VPL, bool ONE, bool PAIR>
__global__ __launch_bounds__(kMaxWaves * 64, (!ONE && VPL <= 8) ? 5 : 1) void decode_gu_kernel(DecodeArgs a) {
  __shared__ int s_ids[kDecodeMaxPairs];
  __shared__ uint32_t s_bits[MOE_MAX_EXPERTS / 32];
  __shared__ int s_uexp[kDecodeMaxPairs];
  __shared__ uint32_t s_umask[kDecodeMaxPairs];
  __shared__ int8_t s_uslot[kDecodeMaxPairs][kDecodeMaxT];  // slot of token t's pick of distinct expert u
  __shared__ int s_U;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nthreads = blockDim.x;
  const int T = a.T, k = a.k, E = a.E, P = T * k;
  const int nwords = (E + 31) / 32;

  const int chunks = a.fmax / 16;
  const int u = blockIdx.x / chunks, hc = blockIdx.x - u * chunks;
  const bool shared = u == P;
  // pair items: token pt, slot pj (one token: item u is slot u)
  constexpr bool kPairs = ONE || PAIR;
  const int pt = kPairs && !shared ? u / k : 0, pj = kPairs && !shared ? u - pt * k : 0;
  // one token's activations, requested at the start (one token, or a pair)
  const bool x_one = ONE || (PAIR && !shared);

  // ---- the call's activations (bf16 [T][d]) go to LDS. One token: each
  // thread's chunk is requested first, so its latency hides behind the
  // routing. Several tokens: the chunks are copied after the weight requests
  // below, so none is held in registers across the top-k.
  // dynamic LDS: the call's activations, then the waves' partial sums
  extern __shared__ uint4 s_x[];  // [T * d / 8]
  float(*s_red)[2][256] = reinterpret_cast<float(*)[2][256]>(s_x + T * (a.d / 8));  // [waves][2][256]
  // one token (at most four waves): then each wave's codes on their way into
  // the MFMA layout, [waves][gate/up][16 rows][16 units], units XOR-swizzled
  // by row
  uint4(*s_wst)[2][16][16] = reinterpret_cast<uint4(*)[2][16][16]>(s_red + nthreads / 64);
  uint4 xr0 = make_uint4(0u, 0u, 0u, 0u);
  if (x_one) xr0 = reinterpret_cast<const uint4 *>(a.x)[pt * nthreads + tid];  // nthreads = d / 8

  // ---- routing, repeated by every workgroup of a routed expert
  if (!shared && kPairs) {
    // pair (token pt, slot pj): only token pt's top-k, and only its first
    // pj + 1 rounds (the lower slots' weight requests go out sooner, so the
    // last slots' streams meet less traffic); the first workgroup of slot 0
    // runs all k, since it writes the token's ids and gates
    if (wave == 0) {
      int id;
      float g;
      const bool writer = pj == 0 && hc == 0;
      const int rounds = writer ? k : min(pj + 1, k);
      topk_wave<VPL>(a.logits + (int64_t)pt * E, E, rounds, lane, id, g);
      if (lane == pj) s_uexp[0] = id;
      if (writer && lane < k) {
        a.ids[pt * k + lane] = id;
        a.gates[pt * k + lane] = g;
      }
    }
    __syncthreads();
  } else if (!shared) {
  for (int i = tid; i < nwords; i += nthreads) s_bits[i] = 0u;
  if (tid < kDecodeMaxPairs) s_umask[tid] = 0u;
  // one token per wave, so the tokens' top-k run side by side
  const int nw = nthreads / 64;
  for (int t = wave; t < T; t += nw) {
    int id;
    float g;
    topk_wave<VPL>(a.logits + (int64_t)t * E, E, k, lane, id, g);
    if (lane < k) {
      s_ids[t * k + lane] = id;
      if (blockIdx.x == 0) {
        a.ids[t * k + lane] = id;
        a.gates[t * k + lane] = g;
      }
    }
  }
  __syncthreads();
  if (tid < P) atomicOr(&s_bits[s_ids[tid] >> 5], 1u << (s_ids[tid] & 31));
  __syncthreads();
  if (tid < P) {
    // rank of this expert among the distinct ones (ascending expert index)
    const int e = s_ids[tid], wi = e >> 5;
    int rank = __popc(s_bits[wi] & ((1u << (e & 31)) - 1u));
    for (int q = 0; q < wi; ++q) rank += __popc(s_bits[q]);
    s_uexp[rank] = e;
    s_uslot[rank][tid / k] = (int8_t)(tid % k);
    atomicOr(&s_umask[rank], 1u << (tid / k));
  }
  if (tid == 0) {
    int U = 0;
    for (int q = 0; q < nwords; ++q) U += __popc(s_bits[q]);
    s_U = U;
  }
  __syncthreads();
  }

  // ---- this workgroup's item: (distinct expert u or the shared expert, 16 h columns)
  int e = 0, fe;
  uint32_t mask;
  if (shared) {
    if (a.f_sh == 0) return;
    fe = a.f_sh;
    mask = (T >= 32) ? 0xFFFFFFFFu : ((1u << T) - 1u);
  } else if (kPairs) {
    e = s_uexp[0];
    mask = 1u << pt;
    fe = a.f;
  } else {
    if (u >= s_U) return;
    e = s_uexp[u];
    mask = s_umask[u];
    fe = a.f;
  }
  if (16 * hc >= fe) return;
  const int nrows = __popc(mask);

  const int d = a.d, G = d / 64;
  const uint32_t *wq = shared ? a.sh_gu_q : a.gu_q + (int64_t)e * a.gu_qs;
  const uint16_t *wsc = shared ? a.sh_gu_s : a.gu_s + (int64_t)e * a.gu_ss;
  const uint16_t *wbi = shared ? a.sh_gu_b : a.gu_b + (int64_t)e * a.gu_ss;
  const int c16 = lane & 15, kq = lane >> 4;
  const int row[2] = {16 * hc + c16, fe + 16 * hc + c16};  // gate row, up row
  const int kbase = wave * kSpan, nwaves = nthreads / 64;

  // ---- requests: codes, scales/biases, activations (all before any use)
  // One token: each wave's 16 rows x 256 bytes of codes per projection come
  // in four whole 1 KiB requests (lane l: row 4 s + l / 16 of the 16, 16-byte
  // unit l % 16 of the row's 256 bytes) and pass through LDS into the MFMA
  // layout below; requests of 16 row segments of 64 bytes each, straight in
  // that layout, took a third more L1 work. Several tokens keep the direct
  // form (the staging's LDS would cost T = 4 its residency); one token with
  // more than four waves (d > 2048), whose staging would pass 64 KiB of LDS,
  // runs as the pair form.
  u4v code[2][kSteps], sw[2], bw[2];
  const int lr = lane >> 4, lu = lane & 15;
  if constexpr (ONE) {
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int s = 0; s < kSteps; ++s) {
        const int grow = (cb == 0 ? 0 : fe) + 16 * hc + 4 * s + lr;
        code[cb][s] = *reinterpret_cast<const u4v *>(wq + (int64_t)grow * (d / 8) + kbase / 8 + 4 * lu);
      }
  } else {
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      const uint32_t *cr = wq + (int64_t)row[cb] * (d / 8) + (kbase + 32 * kq) / 8;
#pragma unroll
      for (int s = 0; s < kSteps; ++s) code[cb][s] = *reinterpret_cast<const u4v *>(cr + 16 * s);
    }
  }
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    sw[cb] = *reinterpret_cast<const u4v *>(wsc + (int64_t)row[cb] * G + kbase / 64);
    bw[cb] = *reinterpret_cast<const u4v *>(wbi + (int64_t)row[cb] * G + kbase / 64);
  }
  // activations into LDS as fp16 in the rebuild order (their loads were
  // issued first), converted once per workgroup; then row c16's fragments:
  // a token of the mask, else the first one again (a row never read)
  if (x_one) {
    const uint4 xc = x_chunk_h8(xr0);
    s_x[pt * nthreads + tid] = xc;
    if (pj == 0 && hc == 0 && !shared)  // each token's x checked once
      note_overflow(a.overflow, f16x2_nonfinite(xc.x) || f16x2_nonfinite(xc.y) || f16x2_nonfinite(xc.z) ||
                                    f16x2_nonfinite(xc.w), MOE_OVERFLOW_X);
  } else {
    // T chunks per thread, requested behind the weights: waiting for them
    // also waits for the weights, which the MFMAs need next anyway. All
    // requests go out before the first store (a load-store loop would wait
    // for memory once per token); indexes past T repeat the last token.
    const uint4 *xg = reinterpret_cast<const uint4 *>(a.x);
    uint4 xc[kDecodeMaxT];
#pragma unroll
    for (int i = 0; i < kDecodeMaxT; ++i) xc[i] = xg[min(i, T - 1) * nthreads + tid];
#pragma unroll
    for (int i = 0; i < kDecodeMaxT; ++i)
      if (i < T) {
        const uint4 h8 = x_chunk_h8(xc[i]);
        s_x[i * nthreads + tid] = h8;
        if (blockIdx.x == 0)
          note_overflow(a.overflow, f16x2_nonfinite(h8.x) || f16x2_nonfinite(h8.y) || f16x2_nonfinite(h8.z) ||
                                        f16x2_nonfinite(h8.w), MOE_OVERFLOW_X);
      }
  }
  if constexpr (ONE) {
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int s = 0; s < kSteps; ++s) {
        const int r16 = 4 * s + lr;
        s_wst[wave][cb][r16][lu ^ r16] = make_uint4(code[cb][s][0], code[cb][s][1], code[cb][s][2], code[cb][s][3]);
      }
  }
  __syncthreads();
  if constexpr (ONE) {
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int s = 0; s < kSteps; ++s) {
        const uint4 v = s_wst[wave][cb][c16][(4 * s + kq) ^ c16];
        code[cb][s] = u4v{v.x, v.y, v.z, v.w};
      }
  }
  const int tok = nth_bit(mask, c16 < nrows ? c16 : 0);
  const uint4 *xl = s_x + ((int64_t)tok * d + kbase + 32 * kq) / 8;

  // ---- MFMAs over this wave's inputs. One token (288 workgroups, all
  // resident): every activation fragment is read from LDS up front. Several
  // tokens: step by step, since holding all of them took 64 registers and
  // kept the kernel at three waves per SIMD, too few for T = 4's workgroups
  // to be resident at once.
  u4v xall[ONE ? kSteps : 1][4];
  if constexpr (ONE) {
#pragma unroll
    for (int s = 0; s < kSteps; ++s)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint4 v = xl[16 * s + j];
        xall[s][j] = u4v{v.x, v.y, v.z, v.w};
      }
  }
  const RbConsts kc = rb_consts();
  f4 acc[2] = {f4{0.f, 0.f, 0.f, 0.f}, f4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
  for (int s = 0; s < kSteps; ++s) {
    u4v xv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if constexpr (ONE) {
        xv[j] = xall[s][j];
      } else {
        const uint4 v = xl[16 * s + j];
        xv[j] = u4v{v.x, v.y, v.z, v.w};
      }
    }
    uint32_t sc[2];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) sc[cb] = group_consts(sw[cb], bw[cb], s, kq >> 1);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const rb_h8 af = __builtin_bit_cast(rb_h8, xv[j]);
#pragma unroll
      for (int cb = 0; cb < 2; ++cb)
        acc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, rb_rebuild(code[cb][s][j], sc[cb], kc), acc[cb], 0,
                                                         0, 0);
    }
  }

  // ---- partial sums of the waves meet in LDS; SwiGLU; fp32 h per (token, slot)
#pragma unroll
  for (int cb = 0; cb < 2; ++cb)
#pragma unroll
    for (int i = 0; i < 4; ++i) s_red[wave][cb][4 * lane + i] = acc[cb][i];
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 4 * kq + i;  // row of the MFMA tile = r-th token of the mask
      if (r < nrows) {
        float g = 0.f, up = 0.f;
        if (nwaves == 4) {  // d = 2048: every partial requested before the first add
          float gv[4], uv[4];
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            gv[w] = s_red[w][0][4 * lane + i];
            uv[w] = s_red[w][1][4 * lane + i];
          }
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            g += gv[w];
            up += uv[w];
          }
        } else {
          for (int w = 0; w < nwaves; ++w) {
            g += s_red[w][0][4 * lane + i];
            up += s_red[w][1][4 * lane + i];
          }
        }
        const int t = nth_bit(mask, r);
        // pairs: the item's slot
        const int slot = shared ? k : kPairs ? pj : s_uslot[u][t];
        // fp16, each 8 columns in the rebuild order, as the down MFMAs take it
        const int n = 16 * hc + c16;
        const float hv = swiglu(g, up);
        note_overflow(a.overflow, f16_out_of_range(hv), MOE_OVERFLOW_H);
        a.h[((int64_t)t * (k + 1) + slot) * a.fmax + (n & ~7) + 2 * (n & 3) + ((n >> 2) & 1)] =
            __builtin_bit_cast(uint16_t, (_Float16)hv);
      }
    }
  }
}

// NT: tiles of 8 output columns per workgroup (one tile: each slot wave's
// 16x16 MFMA tile as above; NT tiles: the wave repeats it for NT column
// groups, each output column computed exactly as with one tile).
template <int NT>
__global__ __launch_bounds__(64 * kDecodeMaxSlots) void decode_dn_kernel(DecodeArgs a) {
  __shared__ float s_part[kDecodeMaxSlots][16 * NT];
  __shared__ float s_gate[kDecodeMaxSlots];
  const int tid = threadIdx.x, lane = tid & 63, j = tid >> 6;  // wave j: slot j (j == k: shared)
  const int k = a.k, d = a.d, blocks = d / (8 * NT);
  const int t = blockIdx.x / blocks, cc = blockIdx.x - t * blocks;
  const int c16 = lane & 15, kq = lane >> 4;
  const bool shared = j == k;
  const bool live = !shared || a.f_sh > 0;  // a shared wave without a shared expert adds zero

  // Requests, all unconditional so no wait covers more than it needs: the
  // slot's pick and gate, the slot's h, then its weights (which need the
  // pick). A dead shared wave reads routed expert 0 and is zeroed at the end.
  const int jr = shared ? 0 : j;
  const int e_slot = a.ids[t * k + jr];
  const float g_slot = a.gates[t * k + jr];
  // A operand: tile row r holds h's half r & 1 (inputs 256 (r & 1) ...), 8
  // fp16 per lane and MFMA, already in the rebuild order
  const uint4 *hs = reinterpret_cast<const uint4 *>(a.h + ((int64_t)t * (k + 1) + j) * a.fmax +
                                                    (kSpan / 2) * (c16 & 1) + 32 * kq);
  u4v hv[kSteps / 2][4];
#pragma unroll
  for (int s = 0; s < kSteps / 2; ++s)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint4 v = hs[16 * s + q];
      hv[s][q] = u4v{v.x, v.y, v.z, v.w};
    }
  // B operand of tile p: tile column c16 is output column 8 (NT cc + p) +
  // (c16 & 7) over the input half c16 >> 3
  const bool use_sh = shared && live;
  const int e = shared ? 0 : e_slot;
  const uint32_t *wq = use_sh ? a.sh_dn_q : a.dn_q + (int64_t)e * a.dn_qs;
  const uint16_t *wsc = use_sh ? a.sh_dn_s : a.dn_s + (int64_t)e * a.dn_ss;
  const uint16_t *wbi = use_sh ? a.sh_dn_b : a.dn_b + (int64_t)e * a.dn_ss;
  const int kh = c16 >> 3;
  u4v code[NT][kSteps / 2];
  uint2 sw[NT], bw[NT];
  // the wave's 8 NT weight rows x 256 bytes come in 2 NT whole 1 KiB requests
  // (request i, lane l: row 4 i + l / 16, 16-byte unit l % 16 of the row) and
  // pass through a per-wave LDS tile (units XOR-swizzled by row) into the
  // MFMA layout; 16 row segments of 64 bytes per request straight in that
  // layout took T = 4 steps 0.7 us longer. One wave's LDS operations run in
  // order; the fences keep the compiler from moving them.
  __shared__ u4v s_dst[kDecodeMaxSlots][8 * NT][16];
  u4v raw[2 * NT];
#pragma unroll
  for (int i = 0; i < 2 * NT; ++i) {
    const int n = 8 * NT * cc + 4 * i + (lane >> 4);
    raw[i] = *reinterpret_cast<const u4v *>(wq + (int64_t)n * (kSpan / 8) + 4 * (lane & 15));
  }
#pragma unroll
  for (int p = 0; p < NT; ++p) {
    const int n = 8 * (NT * cc + p) + (c16 & 7);
    // the four groups of this half: group 2 s + (kq >> 1) of them feeds step s
    sw[p] = *reinterpret_cast<const uint2 *>(wsc + (int64_t)n * (kSpan / 64) + (kSpan / 128) * kh);
    bw[p] = *reinterpret_cast<const uint2 *>(wbi + (int64_t)n * (kSpan / 64) + (kSpan / 128) * kh);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
#pragma unroll
  for (int i = 0; i < 2 * NT; ++i) {
    const int r = 4 * i + (lane >> 4);
    s_dst[j][r][(lane & 15) ^ (r & 15)] = raw[i];
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
#pragma unroll
  for (int p = 0; p < NT; ++p)
#pragma unroll
    for (int s = 0; s < kSteps / 2; ++s) {
      const int r = 8 * p + (c16 & 7);
      code[p][s] = s_dst[j][r][(8 * kh + kq + 4 * s) ^ (r & 15)];
    }

  const RbConsts kc = rb_consts();
  const uint32_t sh = 16u * (uint32_t)(kq >> 1);
#pragma unroll
  for (int p = 0; p < NT; ++p) {
    f4 acc = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < kSteps / 2; ++s) {
      const uint32_t swd = s == 0 ? sw[p].x : sw[p].y, bwd = s == 0 ? bw[p].x : bw[p].y;
      const uint32_t sc = rb_pack_scale_bias((swd >> sh) & 0xFFFFu, (bwd >> sh) & 0xFFFFu);
#pragma unroll
      for (int q = 0; q < 4; ++q)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(rb_h8, hv[s][q]),
                                                     rb_rebuild(code[p][s][q], sc, kc), acc, 0, 0, 0);
    }
    // row 0 (first half) of columns 0-7 and row 1 (second half) of columns
    // 8-15 sit in lanes 0-15 (kq = 0), elements 0 and 1
    if (kq == 0) s_part[j][16 * p + c16] = live ? (c16 < 8 ? acc[0] : acc[1]) : 0.f;
  }
  if (lane == 0 && !shared) s_gate[j] = g_slot;
  __syncthreads();
  if (tid < 8 * NT) {
    const int p = tid >> 3, c = 16 * p + (tid & 7);
    float y = 0.f;
    if (k == 8) {  // top-8: every partial and gate requested before the first add
      float gv[8], pa[9], pb[9];
#pragma unroll
      for (int jj = 0; jj < 9; ++jj) {
        pa[jj] = s_part[jj][c];
        pb[jj] = s_part[jj][c + 8];
      }
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) gv[jj] = s_gate[jj];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) y += gv[jj] * (pa[jj] + pb[jj]);
      y += pa[8] + pb[8];
    } else {
      for (int jj = 0; jj < k; ++jj) y += s_gate[jj] * (s_part[jj][c] + s_part[jj][c + 8]);
      y += s_part[k][c] + s_part[k][c + 8];
    }
    a.y[(int64_t)t * d + 8 * NT * cc + tid] = y;
  }
}

}  // namespace

bool decode_supported(int T, const moe_layer_t *L) {
  return T >= 1 && T <= kDecodeMaxT && T * L->k <= kDecodeMaxPairs && L->k + 1 <= kDecodeMaxSlots &&
         L->d % kSpan == 0 && L->d / kSpan <= kMaxWaves && L->f == kSpan && (L->f_sh == 0 || L->f_sh == kSpan) &&
         L->E <= MOE_MAX_EXPERTS;
}

template <bool ONE, bool PAIR>
static void launch_decode_gu(const DecodeArgs &a, int vpl, dim3 g, dim3 b, size_t lds, hipStream_t s, hipEvent_t start,
                             hipEvent_t stop) {
  if (vpl <= 1)       hipExtLaunchKernelGGL((decode_gu_kernel<1, ONE, PAIR>), g, b, lds, s, start, stop, 0, a);
  else if (vpl <= 2)  hipExtLaunchKernelGGL((decode_gu_kernel<2, ONE, PAIR>), g, b, lds, s, start, stop, 0, a);
  else if (vpl <= 4)  hipExtLaunchKernelGGL((decode_gu_kernel<4, ONE, PAIR>), g, b, lds, s, start, stop, 0, a);
  else if (vpl <= 8)  hipExtLaunchKernelGGL((decode_gu_kernel<8, ONE, PAIR>), g, b, lds, s, start, stop, 0, a);
  else                hipExtLaunchKernelGGL((decode_gu_kernel<16, ONE, PAIR>), g, b, lds, s, start, stop, 0, a);
}

hipError_t launch_decode(const DecodeArgs &a, hipStream_t s, hipEvent_t gu_start, hipEvent_t gu_stop,
                         hipEvent_t dn_stop) {
  const int vpl = (a.E + 63) / 64;
  const dim3 g1((a.T * a.k + 1) * (a.fmax / 16)), b1(64 * (a.d / kSpan));
  // the call's activations, then each wave's partial sums (2 x 256 floats);
  // the one-token form (at most four waves): then each wave's staged codes
  // (2 x 16 x 256 bytes)
  const bool one = a.T == 1 && a.d / kSpan <= 4;
  const size_t xlds = (size_t)a.T * a.d * 2 + (size_t)(a.d / kSpan) * 2 * 256 * sizeof(float) +
                      (one ? (size_t)(a.d / kSpan) * 2 * 16 * 256 : 0);
  if (one)                          launch_decode_gu<true, false>(a, vpl, g1, b1, xlds, s, gu_start, gu_stop);
  else if (a.T <= kDecodePairMaxT)  launch_decode_gu<false, true>(a, vpl, g1, b1, xlds, s, gu_start, gu_stop);
  else                              launch_decode_gu<false, false>(a, vpl, g1, b1, xlds, s, gu_start, gu_stop);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  // Three down workgroups (k + 1 waves each) fit a CU, 768 on MI355X's 256
  // CUs: calls that would need more take 16 output columns per workgroup, so
  // every workgroup is resident at once
  const dim3 b2(64 * (a.k + 1));
  if ((int64_t)a.T * (a.d / 8) > kDnResident)
    hipExtLaunchKernelGGL(decode_dn_kernel<2>, dim3(a.T * (a.d / 16)), b2, 0, s, nullptr, dn_stop, 0, a);
  else
    hipExtLaunchKernelGGL(decode_dn_kernel<1>, dim3(a.T * (a.d / 8)), b2, 0, s, nullptr, dn_stop, 0, a);
  return hipGetLastError();
}

}  // namespace moe
