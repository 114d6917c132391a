// Grouped GEMM over uneven expert groups with on-chip int4 dequantisation,
// written for gfx950 (MI355X).
//
// The Lily pages rebuild the 4-bit groupwise-affine weights one tile at a time
// inside the grouped GEMM, keep the rebuilt tile on chip and accumulate in
// FP32, so the expanded weights never reach memory (Lily-EN "Prefill: Keep
// Weights Packed, Keep Routing on the GPU"; Lily-ES "Precarga: mantenga los
// pesos empaquetados, siga enrutando en la GPU", which also gives the group
// of 64 weights sharing one bf16 scale and one bf16 bias and the 32-row
// tiles). That design targeted Metal tensor ops on bf16; on gfx950 it becomes:
//
//   * Work unit: up to 96 rows (three 32-row blocks) of one expert x one
//     256-column N-slice of the weights. A workgroup is 4 waves, one per
//     SIMD, and two workgroups share a CU (at most 256 registers per lane,
//     about 65 KiB of LDS each), so one workgroup's barrier waits, prologue
//     and epilogue overlap the other's MFMAs. A wave owns 64 weight rows
//     (output columns) as four 16-column MFMA blocks and every row of the
//     unit, so each rebuilt weight feeds every row of the unit. Units come
//     largest first; the last few (a problem's ntail) run as 128-column
//     items with two blocks per wave, so the final round of workgroups is
//     made of half-length pieces.
//   * Each group's scale and bias are read once per work unit with coalesced
//     loads into an LDS table of fp16 (s, b + 8s) pairs; with a prepared copy
//     of the weights (prep_layout.h: codes in the order the item reads them,
//     the pairs pre-formed) each lane instead loads its pairs beside its
//     codes, and every K step of an item reads one contiguous 16 KiB block.
//   * Weights go HBM -> VGPR with one 128-bit load per lane and column block
//     per K step, one step ahead of use (buffer loads whose per-step offset
//     sits in a scalar register when K is a multiple of the step, so stepping
//     costs no per-lane address arithmetic), and are rebuilt in registers:
//     v_and_or_b32 puts two codes into fp16 "1024+v" slots, v_pk_add_f16
//     removes the offset exactly, v_pk_fma_f16 applies the group scale and
//     bias: w = fp16(s*(q-8) + (b+8s)). Only registers hold the rebuilt tile.
//   * Activations (fp16, each 8-run stored as 0,4,1,5,2,6,3,7 to match the
//     register order of the rebuilt codes) are gathered by row with 128-bit
//     loads one step ahead and written to LDS, double buffered, XOR-swizzled
//     so the 16 rows read by one MFMA operand fetch hit distinct banks.
//   * v_mfma_f32_16x16x32_f16 with fp32 accumulators. 16-row MFMA blocks let
//     a partial 32-row block skip its empty half.
//   * Epilogues: SwiGLU into fp16 h (gate/up projection); fp16 expert
//     outputs (down projection; a separate kernel combines them per token in
//     a fixed order); plain fp32 store (stand-alone grouped GEMM).
//
// K loop: step s covers inputs [128s, 128s+128) (K is padded to a multiple of
// 128 with zero weights); 16-lane quarter kq takes the 32 inputs starting at
// 128s + 32kq, which lie in one 64-group. The four lanes of one column thus
// read 64 contiguous bytes of codes per step, and the other half of that
// 128-byte line on the next step, so each line is fetched from HBM once.
//
// Pages cited (titles as published):
//   Lily-EN  "Perplexity Open Sources Lily: A Rust + Metal Inference Engine
//            for Qwen3.6-35B-A3B on Apple Silicon" (insight.aitobox.com)
//   Lily-ES  "Perplexity open sources Lily: un motor de inferencia ... para
//            Qwen3.6-35B-A3B en Apple Silicon" (7minutos.es)

#include "moe_internal.h"
#include "prep_layout.h"
#include "rebuild_device.h"

#include <hip/hip_fp16.h>

#include <type_traits>

// The main build is launch_gemm (units of up to 96 rows, two workgroups per
// CU); gemm_kernels_small.hip compiles this file again as launch_gemm_small
// (units of up to 32 rows, three workgroups per CU).
#ifndef MOE_GEMM_LAUNCH
#define MOE_GEMM_LAUNCH launch_gemm
#endif

namespace moe {
namespace {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = kGemmThreads / 64;
constexpr int kColsMax = kGemmCols;              // weight rows (output columns) of a full-width item
constexpr int kCBFull = kColsMax / (16 * kWaves); // 16-column MFMA blocks per wave, full-width items

constexpr int kKStep = 128;                       // K per step (4 quarters x 32)
constexpr int kRowBytes = kKStep * 2;             // one row of one step in LDS (fp16)
constexpr int kBufBytes = kUnitRows * kRowBytes;  // one step of a full unit (24 KiB)
constexpr int kSlabRows = 1024 / kRowBytes;       // rows per 1 KiB wave store

constexpr int kTabGroups = MOE_GEMM_TAB_GROUPS;    // scale/bias groups held at a time
constexpr int kTabSteps = kTabGroups * 64 / kKStep; // K steps covered by one table fill
constexpr int kTabStride = kColsMax + 16;          // dwords per group row of the table (padded)
static_assert(kCBFull == 4, "a wave owns four 16-column MFMA blocks of a full-width item");
static_assert((kTabGroups & (kTabGroups - 1)) == 0 && kTabGroups * 64 % kKStep == 0, "table of whole steps");
static_assert(MOE_GEMM_WGS_PER_CU * (2 * kBufBytes + kTabGroups * kTabStride * 4 + kUnitRows * 4) <= 160 * 1024,
              "the resident workgroups' LDS fits one CU");

template <int CB>
struct BStage {
  u4 q[CB];            // 4 code words (32 codes) per column block
  uint32_t t[CB];      // prepared weights: the block's (s, b + 8 s) pair for this step
};


// Weights already expanded to fp16 in device memory (the unfused ablation):
// the lane's 32 weights of each column block as four 8-weight chunks.
template <int CB>
struct XStage {
  u4 q[CB][4];
};

// Raw buffer resource over memory from base on, with no range limit (every
// access made through it is in bounds by construction). Loads through it
// take the per-step K offset as the instruction's scalar offset, so a K step
// costs no per-lane address arithmetic.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_rsrc(const void *base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, -1, 0x00020000);
}

__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  const u4 v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// Workgroup barrier that first drains this wave's LDS operations. The memory
// clobber keeps the compiler from moving LDS accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ uint16_t f32_to_f16_bits(float v) {
  return __half_as_ushort(__float2half_rn(v));
}

// Column position of logical column n in the permuted-run activation layout
// (each run of 8 stored as 0,4,1,5,2,6,3,7).
__device__ __forceinline__ int perm_col(int n) {
  return (n & ~7) | ((n & 3) << 1) | ((n >> 2) & 1);
}

struct Unit {
  int e, r0, nr;
  int slice;
};

// NRB = 16-row MFMA blocks of the unit (1..6), fixed at compile time so a K
// step is one branch-free block the compiler can schedule as a whole.
// CHECK: report fp16 values out of range through P.overflow (epilogues).
// BUF: K is a multiple of the 128-input step (and the activations are fp16):
// the K loop's loads are buffer loads with the step offset in a scalar
// register; otherwise per-lane clamped addresses keep the last step's
// quarters past K on their row.
// PREP (implies BUF): codes and the scale/bias pairs come from the prepared
// copy (prep_layout.h): every K step reads one contiguous 16 KiB block of
// codes per full-width slice, and each lane loads its column blocks' pairs
// for the step beside them, so the LDS table is not used.
template <int MODE, bool AF16, bool WX, bool CHECK, int NRB, int CB, bool BUF, bool PREP>
__device__ __forceinline__ void run_unit(const GemmProblem &P, const Unit &U, uint8_t *lds,
                                         const int *s_arow, uint32_t *tab) {
  constexpr int kMaxRB = NRB;
  constexpr int kCB = CB;                    // 16-column MFMA blocks per wave
  constexpr int kHalf = CB / 2;              // gate blocks (then as many up blocks) in SwiGLU mode
  constexpr int kCols = 16 * CB * kWaves;    // weight rows (output columns) of this item
  constexpr int kRB32 = (NRB + 1) / 2;                                    // 32-row blocks staged
  constexpr int kSlabs = (32 * kRB32 / kSlabRows + kWaves - 1) / kWaves;  // A stores per wave
  // WX: the weights come expanded (fp16, each 8-run in the rebuild order)
  // from P.Wx; no codes, no table, no rebuild.
  typedef typename std::conditional<WX, XStage<CB>, BStage<CB>>::type Stage;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c16 = lane & 15, kq = lane >> 4;
  const int N = P.N, K = P.K, G = K >> 6;
  const int steps = (K + kKStep - 1) / kKStep;
  const int nr = U.nr;

  // columns (weight rows) of this wave
  int ncol[kCB];
  bool active;
  if (MODE == kSwiGLU) {
    const int f = N >> 1, ng = U.slice * (kCols / 2) + wave * 8 * kCB;
    active = ng < f;
#pragma unroll
    for (int cb = 0; cb < kCB; ++cb)
      ncol[cb] = (cb < kHalf ? ng + 16 * cb : f + ng + 16 * (cb - kHalf)) + c16;
  } else {
    const int n0 = U.slice * kCols + wave * 16 * kCB;
    active = n0 < N;
#pragma unroll
    for (int cb = 0; cb < kCB; ++cb) ncol[cb] = n0 + 16 * cb + c16;
  }
  if (!active) {  // idle waves still issue in-bounds loads to keep counts uniform
#pragma unroll
    for (int cb = 0; cb < kCB; ++cb) ncol[cb] = c16;
  }

  // table column of each of this lane's column blocks, and the weight row of
  // a table column (-1 past the end)
  int tcol[kCB];
#pragma unroll
  for (int cb = 0; cb < kCB; ++cb)
    tcol[cb] = (MODE == kSwiGLU ? (cb < kHalf ? 8 * kCB * wave + 16 * cb : kCols / 2 + 8 * kCB * wave + 16 * (cb - kHalf))
                                : 16 * kCB * wave + 16 * cb) + c16;
  // PREP: the item lies in full-width slice pslice (a half-width item is
  // half `phalf` of one); lcol is the prepared table column of each column
  // block (lane column 0)
  const int pslice = kCols == kColsMax ? U.slice : (U.slice >> 1);
  const int phalf = kCols == kColsMax ? 0 : (U.slice & 1);
  int lcol[kCB];
#pragma unroll
  for (int cb = 0; cb < kCB; ++cb) {
    lcol[cb] = MODE == kSwiGLU ? (cb < kHalf ? 0 : kColsMax / 2) + phalf * (kCols / 2) + wave * 8 * kCB + 16 * (cb % kHalf)
                               : phalf * kCols + wave * 16 * kCB + 16 * cb;
  }
  auto tab_row = [&](int c) -> int {
    if (MODE == kSwiGLU) {
      const int f = N >> 1, n = U.slice * (kCols / 2) + (c & (kCols / 2 - 1));
      return n < f ? (c < kCols / 2 ? n : f + n) : -1;
    }
    const int n = U.slice * kCols + c;
    return n < N ? n : -1;
  };

  const uint32_t *wq = P.Wq + (int64_t)U.e * P.wq_estride;
  const uint16_t *wsc = P.Ws + (int64_t)U.e * P.ws_estride;
  const uint16_t *wbi = P.Wb + (int64_t)U.e * P.ws_estride;
  const int kw = K >> 3;
  // code-word offset of each column block's weight row within the expert
  // (the host keeps one expert's N * K / 8 words below 2^31)
  uint32_t b_row[kCB];
#pragma unroll
  for (int cb = 0; cb < kCB; ++cb) b_row[cb] = (uint32_t)ncol[cb] * (uint32_t)kw;

  // first input of this lane's quarter at step s (valid iff < K)
  auto lane_k0 = [&](int s) { return kKStep * s + 32 * kq; };

  // BUF (K a multiple of the step, so no lane ever reads past K): codes by
  // buffer loads at lane offset 4 b_row + 16 kq bytes and step offset 64 s
  // bytes.
  // PREP: the lane's 16 bytes of chunk prep_chunk(lcol) of the slice's block
  // for step s, at step offset 16 KiB s.
  const __amdgpu_buffer_rsrc_t rsrc_b =
      raw_rsrc(PREP ? (const void *)(P.Pq + (int64_t)U.e * P.pq_estride) : (const void *)wq);
  uint32_t b_voff[kCB];
#pragma unroll
  for (int cb = 0; cb < kCB; ++cb)
    b_voff[cb] = PREP ? (uint32_t)pslice * (uint32_t)steps * (uint32_t)kPrepBlock +
                            1024u * (uint32_t)prep_chunk(lcol[cb], MODE == kSwiGLU) + 16u * (uint32_t)lane
                      : 4u * b_row[cb] + 16u * (uint32_t)kq;
  // PREP: each lane loads its column blocks' (s, b + 8 s) pairs for the step
  // straight from the prepared table with the codes, group 2 s + kq / 2 of
  // the slice (step offset 2 KiB s): no LDS table, no fills, no refill
  // barriers
  const __amdgpu_buffer_rsrc_t rsrc_t = raw_rsrc(P.Pt + (int64_t)U.e * P.pt_estride);
  uint32_t t_voff[kCB];
#pragma unroll
  for (int cb = 0; cb < kCB; ++cb)
    t_voff[cb] = 4u * (uint32_t)((pslice * G + (kq >> 1)) * kColsMax + lcol[cb] + c16);
  auto load_b = [&](Stage &st, int s) {
    if constexpr (BUF) {
      const uint32_t so = PREP ? (uint32_t)kPrepBlock * (uint32_t)s : 64u * (uint32_t)s;
#pragma unroll
      for (int cb = 0; cb < kCB; ++cb) st.q[cb] = __builtin_bit_cast(u4, buf_load16(rsrc_b, b_voff[cb], so));
      if constexpr (PREP) {
#pragma unroll
        for (int cb = 0; cb < kCB; ++cb)
          st.t[cb] = __builtin_amdgcn_raw_buffer_load_b32(rsrc_t, t_voff[cb], 2048u * (uint32_t)s, 0);
      }
      return;
    }
    const int k0 = lane_k0(s);
    const int kc = k0 < K ? k0 : 0;
    if constexpr (WX) {
      // weight row of each column block: N * K elements per expert, which
      // the host keeps below 2^31
      const uint16_t *wx = P.Wx + (int64_t)U.e * P.wx_estride;
#pragma unroll
      for (int cb = 0; cb < kCB; ++cb)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          st.q[cb][j] = *reinterpret_cast<const u4 *>(wx + ((uint32_t)ncol[cb] * (uint32_t)K + (uint32_t)(kc + 8 * j)));
    } else {
#pragma unroll
      for (int cb = 0; cb < kCB; ++cb)
        st.q[cb] = *reinterpret_cast<const u4 *>(wq + (uint32_t)(b_row[cb] + (kc >> 3)));
    }
  };

  // Scale/bias table for groups [kTabGroups gc, kTabGroups (gc + 1)):
  // tab[g][c] holds (fp16 s, fp16 (b + 8 s)) of group g of table column c.
  // Filled with coalesced loads once per kTabGroups * 64 inputs instead of
  // per step and lane.
  auto fill_table = [&](int gc) {
    const int g0 = kTabGroups * gc, GC = min(kTabGroups, G - g0);
    if ((G & 7) == 0 && (GC & 7) == 0) {
      // every load is issued before the first conversion, so the fill costs
      // one memory round trip
      constexpr int kIt = kCols * (kTabGroups / 8) / kGemmThreads;
      const int per = GC >> 3;  // 8-group vectors per column
      uint4 sv[kIt], bv[kIt];
#pragma unroll
      for (int it = 0; it < kIt; ++it) {
        const int i = tid + it * kGemmThreads;
        const int c = i / per, q8 = i - c * per;
        const int n = i < kCols * per ? tab_row(c) : -1;
        sv[it] = bv[it] = make_uint4(0, 0, 0, 0);
        if (n >= 0) {
          sv[it] = *reinterpret_cast<const uint4 *>(wsc + (int64_t)n * G + g0 + 8 * q8);
          bv[it] = *reinterpret_cast<const uint4 *>(wbi + (int64_t)n * G + g0 + 8 * q8);
        }
      }
#pragma unroll
      for (int it = 0; it < kIt; ++it) {
        const int i = tid + it * kGemmThreads;
        if (i < kCols * per) {
          const int c = i / per, q8 = i - c * per;
          const bool live = tab_row(c) >= 0;
          const uint32_t sw[4] = {sv[it].x, sv[it].y, sv[it].z, sv[it].w};
          const uint32_t bw[4] = {bv[it].x, bv[it].y, bv[it].z, bv[it].w};
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            tab[(8 * q8 + 2 * u) * kTabStride + c] = live ? rb_pack_scale_bias(sw[u] & 0xFFFFu, bw[u] & 0xFFFFu) : 0u;
            tab[(8 * q8 + 2 * u + 1) * kTabStride + c] = live ? rb_pack_scale_bias(sw[u] >> 16, bw[u] >> 16) : 0u;
          }
        }
      }
    } else {
      for (int i = tid; i < kCols * GC; i += kGemmThreads) {
        const int c = i / GC, gg = i - c * GC;
        const int n = tab_row(c);
        tab[gg * kTabStride + c] =
            n >= 0 ? rb_pack_scale_bias(wsc[(int64_t)n * G + g0 + gg], wbi[(int64_t)n * G + g0 + gg]) : 0u;
      }
    }
  };

  // A tile of step s -> LDS buffer, staged through registers. Slot (row r,
  // 16-byte position p) of a buffer holds logical chunk p ^ (r & 15):
  // quarter (chunk >> 2), 8-run (chunk & 3). One 1 KiB wave store covers 4
  // rows. bf16 activations are converted to fp16 on the way.
  // Per slab of this wave: the activation row and the 16-byte chunk this lane
  // moves, fixed for the whole unit; only the K offset changes per step.
  // element offset of the activation row and this lane's 16-byte chunk: 32
  // bits for fp16 activations (the layer's own buffers, whose size the host
  // bounds), 64 bits for a caller's bf16 matrix
  typedef typename std::conditional<AF16, uint32_t, uint64_t>::type AOff;
  const uint16_t *a_base = reinterpret_cast<const uint16_t *>(P.A);
  AOff a_row_off[kSlabs];
  int a_q32[kSlabs], a_in[kSlabs];
#pragma unroll
  for (int ii = 0; ii < kSlabs; ++ii) {
    const int r = kSlabRows * (wave + kWaves * ii) + (lane >> 4);
    const int ch = (lane & 15) ^ (r & 15);
    a_row_off[ii] = (AOff)s_arow[min(r, nr - 1)] * (AOff)P.lda;
    a_q32[ii] = 32 * (ch >> 2);
    a_in[ii] = 32 * (ch >> 2) + 8 * (ch & 3);
  }
  auto a_src = [&](int s, int ii) {
    const int off = kKStep * s;
    const int kel = off + a_q32[ii] < K ? off + a_in[ii] : 0;
    return a_base + (a_row_off[ii] + (AOff)kel);
  };

  uint4 a_regs[kSlabs];
  // BUF: fp16 activations by buffer loads at lane offset = the byte offset
  // of its row and chunk, step offset 256 s bytes.
  const __amdgpu_buffer_rsrc_t rsrc_a = raw_rsrc(P.A);
  uint32_t a_voff[kSlabs];
#pragma unroll
  for (int ii = 0; ii < kSlabs; ++ii) a_voff[ii] = 2u * (uint32_t)(a_row_off[ii] + (AOff)a_in[ii]);
  auto load_a = [&](int s) {
    if constexpr (BUF) {
#pragma unroll
      for (int ii = 0; ii < kSlabs; ++ii) a_regs[ii] = buf_load16(rsrc_a, a_voff[ii], 256u * (uint32_t)s);
      return;
    }
#pragma unroll
    for (int ii = 0; ii < kSlabs; ++ii)
      a_regs[ii] = *reinterpret_cast<const uint4 *>(a_src(s, ii));
  };
  auto store_a = [&](int buf) {
    uint8_t *dst0 = lds + buf * kBufBytes;
#pragma unroll
    for (int ii = 0; ii < kSlabs; ++ii) {
      const int i = wave + kWaves * ii;
      uint4 o = a_regs[ii];
      if (!AF16) {  // natural-order bf16 run -> permuted fp16 run
        const uint4 v = o;
        auto cvt = [](uint32_t lo_src, uint32_t hi_src, bool upper) {
          const uint32_t l = upper ? (lo_src & 0xFFFF0000u) : (lo_src << 16);
          const uint32_t h = upper ? (hi_src & 0xFFFF0000u) : (hi_src << 16);
          return (uint32_t)f32_to_f16_bits(__uint_as_float(l)) |
                 ((uint32_t)f32_to_f16_bits(__uint_as_float(h)) << 16);
        };
        o.x = cvt(v.x, v.z, false);  // (e0, e4)
        o.y = cvt(v.x, v.z, true);   // (e1, e5)
        o.z = cvt(v.y, v.w, false);  // (e2, e6)
        o.w = cvt(v.y, v.w, true);   // (e3, e7)
      }
      *reinterpret_cast<uint4 *>(dst0 + i * 1024 + 16 * lane) = o;
    }
  };

  f4 acc[kMaxRB][kCB];
#pragma unroll
  for (int rb = 0; rb < kMaxRB; ++rb)
#pragma unroll
    for (int cb = 0; cb < kCB; ++cb) acc[rb][cb] = f4{0.f, 0.f, 0.f, 0.f};

  const RbConsts rbk = rb_consts();

  auto compute = [&](const Stage &st, int s, int buf) {
    const int k0 = lane_k0(s);
    const bool kvalid = k0 < K;
    const int gt = ((k0 >> 6) & (kTabGroups - 1)) * kTabStride;  // group row in the table
    RbGroup grp[kCB];
#pragma unroll
    for (int cb = 0; cb < kCB && !WX; ++cb) {
      uint32_t tv;
      if constexpr (PREP) tv = st.t[cb];
      else tv = kvalid ? tab[gt + tcol[cb]] : 0u;
      grp[cb] = rb_group(tv);
    }
    const uint8_t *abuf = lds + buf * kBufBytes + c16 * kRowBytes;
    // rebuild the 32 codes of quarter-step j for column block cb
    auto rebuild = [&](int j, int cb) -> h8 {
      // expanded weights: inputs past K (the last step's loads were clamped
      // to the row start) contribute zero, as the zero table does below
      if constexpr (WX) return kvalid ? __builtin_bit_cast(h8, st.q[cb][j]) : h8{};
      else if constexpr (PREP) return rb_rebuild_sub(st.q[cb][j], grp[cb]);
      else return rb_rebuild_g(st.q[cb][j], grp[cb], rbk);
    };
    auto read_a = [&](int j, int rb) -> h8 {
      const int aoff = 16 * ((4 * kq + j) ^ c16);
      return *reinterpret_cast<const h8 *>(abuf + rb * 16 * kRowBytes + aoff);
    };
    // Software pipeline over the four quarter-steps, one chunk per column
    // block: the MFMAs of (quarter j, block cb) run while the VALU rebuilds
    // (quarter j, block cb+1) or (j+1, 0); each rebuilt fragment is written
    // into registers its block has just finished with. The activation
    // fragments of quarter j+1 are read from LDS behind the last block's
    // MFMAs of quarter j. Scheduling barriers keep the chunks in this order.
    h8 bq[kCB], af[kMaxRB];
    bq[0] = rebuild(0, 0);
#pragma unroll
    for (int rb = 0; rb < kMaxRB; ++rb) af[rb] = read_a(0, rb);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int cb = 0; cb < kCB; ++cb) {
        if (j == 0 && cb + 1 < kCB) bq[cb + 1] = rebuild(0, cb + 1);
        if (j + 1 < 4 && cb > 0) bq[cb - 1] = rebuild(j + 1, cb - 1);
#pragma unroll
        for (int rb = 0; rb < kMaxRB; ++rb) {
          // down projection: weights as the first operand, so a lane's four
          // accumulators are four adjacent output columns of one row
          if constexpr (MODE == kStoreH)
            acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(bq[cb], af[rb], acc[rb][cb], 0, 0, 0);
          else
            acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[rb], bq[cb], acc[rb][cb], 0, 0, 0);
          if (cb == kCB - 1 && j + 1 < 4) af[rb] = read_a(j + 1, rb);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if (j + 1 < 4) bq[kCB - 1] = rebuild(j + 1, kCB - 1);
    }
  };

  // One K step: the barrier publishes A(s) (written to LDS during the
  // previous step) and frees the other buffer; A(s+1) and B(s+1) are
  // requested, step s is computed, then A(s+1) is written to LDS. Loads are
  // issued unconditionally (clamped to the last step) so every step has the
  // same number in flight and the compiler's wait counts stay exact.
  auto body = [&](int s, const Stage &cur, Stage &nxt) {
    lds_barrier();
    if (!WX && !PREP && s > 0 && s < steps && s % kTabSteps == 0) {  // next table chunk
      fill_table(s / kTabSteps);
      lds_barrier();
    }
    const int sn = min(s + 1, steps - 1);
    load_a(sn);
    load_b(nxt, sn);
    if (active && s < steps) compute(cur, s, s & 1);
    store_a((s + 1) & 1);
  };

  Stage b0, b1;
  if (!WX && !PREP) fill_table(0);
  load_a(0);
  load_b(b0, 0);
  store_a(0);
  for (int s = 0; s < steps; s += 2) {
    body(s, b0, b1);
    body(s + 1, b1, b0);
  }

  // ------------------------------------------------------------- epilogue
  if constexpr (MODE == kSwiGLU) {
    // Gate/up projection: h = silu(gate) * up goes out through LDS in whole
    // 16-byte stores, one 8-run of the permuted-run layout each. The tile
    // (up to 96 rows x kCols/2 h columns, 256-byte rows) sits in the free
    // activation buffers with its 16-byte chunks XOR-swizzled by row (chunk
    // c of row r at c ^ (r & 15)). Accumulator element i of lane (c16, kq)
    // in block (rb, cb) is row 16*rb + 4*kq + i, h column 16*cb + c16 of the
    // wave's gate (cb < kHalf) or up (cb >= kHalf) half. Idle waves take
    // part in the barriers.
    constexpr int kHCols = kCols / 2;
    lds_barrier();
    bool bad = false;
    if (active) {
#pragma unroll
      for (int rb = 0; rb < kMaxRB; ++rb) {
#pragma unroll
        for (int cb = 0; cb < kHalf; ++cb) {
          const int lc = perm_col(wave * 8 * kCB + 16 * cb + c16);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = 16 * rb + 4 * kq + i;
            const float g = acc[rb][cb][i], u = acc[rb][cb + kHalf][i];
            const float h = swiglu(g, u);
            if (CHECK) bad |= r < nr && f16_out_of_range(h);
            *reinterpret_cast<uint16_t *>(lds + r * 256 + 16 * ((lc >> 3) ^ (r & 15)) + 2 * (lc & 7)) =
                f32_to_f16_bits(h);
          }
        }
      }
    }
    if (CHECK) note_overflow(P.overflow, bad, MOE_OVERFLOW_H);
    lds_barrier();
    constexpr int kRowLanes = kHCols / 8;
    constexpr int kRowsPerPass = kGemmThreads / kRowLanes;
    const int j = tid % kRowLanes, n = U.slice * kHCols + 8 * j;
    for (int r = tid / kRowLanes; r < nr; r += kRowsPerPass) {
      if (n < (N >> 1)) {
        const uint4 v = *reinterpret_cast<const uint4 *>(lds + r * 256 + 16 * (j ^ (r & 15)));
        *reinterpret_cast<uint4 *>(P.H + (int64_t)(U.r0 + r) * P.ldh + n) = v;
      }
    }
    return;
  }

  if constexpr (MODE == kStoreH) {
    // Down projection: the tile leaves through LDS so every row goes out as
    // whole 16-byte lane stores (32 lanes per 512-byte row of 256 columns)
    // instead of 2-byte ones. The activation buffers (2 x 24 KiB) are free
    // once every wave has finished its last step: they hold the item's
    // fp16 tile, 96 rows x 512 bytes, in 8-byte units XOR-swizzled by row
    // (unit u of row r at u ^ (r & 15)) so the writes of one instruction
    // spread over all banks. Accumulator element i of lane (c16, kq) in
    // block (rb, cb) is row 16*rb + c16, column 16*cb + 4*kq + i of the
    // wave's tile. Idle waves take part in the barriers.
    constexpr int kUnits = kCols / 4;  // 8-byte units of one tile row
    static_assert(kUnitRows * 512 <= 2 * kBufBytes, "output tile fits the activation buffers");
    lds_barrier();
    bool bad = false;
    if (active) {
#pragma unroll
      for (int rb = 0; rb < kMaxRB; ++rb) {
        const int r = 16 * rb + c16;
#pragma unroll
        for (int cb = 0; cb < kCB; ++cb) {
          const int u = wave * 4 * kCB + 4 * cb + kq;
          if (CHECK && r < nr)
            bad |= f16_out_of_range(acc[rb][cb][0]) || f16_out_of_range(acc[rb][cb][1]) ||
                   f16_out_of_range(acc[rb][cb][2]) || f16_out_of_range(acc[rb][cb][3]);
          const uint32_t lo = f32_to_f16_bits(acc[rb][cb][0]) | ((uint32_t)f32_to_f16_bits(acc[rb][cb][1]) << 16);
          const uint32_t hi = f32_to_f16_bits(acc[rb][cb][2]) | ((uint32_t)f32_to_f16_bits(acc[rb][cb][3]) << 16);
          *reinterpret_cast<uint2 *>(lds + r * 512 + 8 * (u ^ (r & 15))) = make_uint2(lo, hi);
        }
      }
    }
    if (CHECK) note_overflow(P.overflow, bad, MOE_OVERFLOW_O);
    lds_barrier();
    // 16-byte chunk j (units 2j, 2j+1) of row r; kUnits / 2 lanes per row
    constexpr int kRowLanes = kUnits / 2;
    constexpr int kRowsPerPass = kGemmThreads / kRowLanes;
    const int j = tid % kRowLanes, n = U.slice * kCols + 8 * j;
    for (int r = tid / kRowLanes; r < nr; r += kRowsPerPass) {
      if (n < N) {
        const uint8_t *src = lds + r * 512;
        const uint2 a = *reinterpret_cast<const uint2 *>(src + 8 * ((2 * j) ^ (r & 15)));
        const uint2 b = *reinterpret_cast<const uint2 *>(src + 8 * ((2 * j + 1) ^ (r & 15)));
        *reinterpret_cast<uint4 *>(P.H + (int64_t)(U.r0 + r) * P.ldh + n) = make_uint4(a.x, a.y, b.x, b.y);
      }
    }
    return;
  }

  // stand-alone grouped GEMM: fp32 C stored directly (accumulator element i
  // of lane (c16, kq) in block (rb, cb) is row 16*rb + 4*kq + i, column
  // 16*cb + c16 of the wave's tile)
  if (!active) return;
  {
    const int n0 = U.slice * kCols + wave * 16 * kCB;
#pragma unroll
    for (int rb = 0; rb < kMaxRB; ++rb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * rb + 4 * kq + i;
        if (r < nr) {
          float *crow = P.C + (int64_t)(U.r0 + r) * P.ldc + n0 + c16;
#pragma unroll
          for (int cb = 0; cb < kCB; ++cb) crow[16 * cb] = acc[rb][cb][i];
        }
      }
    }
  }
}

// The unit's 16-row block count picks the compiled form.
template <int MODE, bool AF16, bool WX, bool CHECK, int CB, bool BUF, bool PREP>
__device__ __forceinline__ void run_rows(const GemmProblem &P, const Unit &U, uint8_t *lds, const int *s_arow,
                                         uint32_t *tab) {
  if constexpr (kUnitRows <= 32) {  // the small-unit build: one or two row blocks
    if (U.nr <= 16) run_unit<MODE, AF16, WX, CHECK, 1, CB, BUF, PREP>(P, U, lds, s_arow, tab);
    else            run_unit<MODE, AF16, WX, CHECK, 2, CB, BUF, PREP>(P, U, lds, s_arow, tab);
  } else {
    switch ((U.nr + 15) >> 4) {
      case 1: run_unit<MODE, AF16, WX, CHECK, 1, CB, BUF, PREP>(P, U, lds, s_arow, tab); break;
      case 2: run_unit<MODE, AF16, WX, CHECK, 2, CB, BUF, PREP>(P, U, lds, s_arow, tab); break;
      case 3: run_unit<MODE, AF16, WX, CHECK, 3, CB, BUF, PREP>(P, U, lds, s_arow, tab); break;
      case 4: run_unit<MODE, AF16, WX, CHECK, 4, CB, BUF, PREP>(P, U, lds, s_arow, tab); break;
      case 5: run_unit<MODE, AF16, WX, CHECK, 5, CB, BUF, PREP>(P, U, lds, s_arow, tab); break;
      default: run_unit<MODE, AF16, WX, CHECK, 6, CB, BUF, PREP>(P, U, lds, s_arow, tab); break;
    }
  }
}

// One item (at most kUnitRows rows): the row indices to LDS, then the
// compiled form for its width, weight source and row-block count.
template <int MODE, bool AF16, bool WX, bool CHECK, bool kCanBuf, bool kCanPrep>
__device__ __forceinline__ void run_item(const GemmProblem &P, const Unit &U, uint8_t *lds, int *s_arow,
                                         uint32_t *tab, bool buf, bool prep, bool narrow) {
  for (int r = threadIdx.x; r < kUnitRows; r += kGemmThreads) {
    const int p = U.r0 + min(r, U.nr - 1);
    s_arow[r] = P.a_row ? P.a_row[p] : p;
  }
  __syncthreads();
  // half-width items: the same code with half the column blocks per wave
  // (always, for expanded weights: their stages take four times the registers)
  if (WX || narrow) {
    if (prep)     run_rows<MODE, AF16, WX, CHECK, kCBFull / 2, kCanBuf, kCanPrep>(P, U, lds, s_arow, tab);
    else if (buf) run_rows<MODE, AF16, WX, CHECK, kCBFull / 2, kCanBuf, false>(P, U, lds, s_arow, tab);
    else          run_rows<MODE, AF16, WX, CHECK, kCBFull / 2, false, false>(P, U, lds, s_arow, tab);
  } else {
    if (prep)     run_rows<MODE, AF16, WX, CHECK, kCBFull, kCanBuf, kCanPrep>(P, U, lds, s_arow, tab);
    else if (buf) run_rows<MODE, AF16, WX, CHECK, kCBFull, kCanBuf, false>(P, U, lds, s_arow, tab);
    else          run_rows<MODE, AF16, WX, CHECK, kCBFull, false, false>(P, U, lds, s_arow, tab);
  }
}

// The flag of a problem without a prepared copy.
__device__ const uint32_t g_flag_off = 0u;

template <int MODE, bool AF16, bool WX, bool CHECK = false>
__global__ __launch_bounds__(kGemmThreads, MOE_GEMM_WGS_PER_CU) void gemm_kernel(GemmArgs args) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[2 * kBufBytes];
  __shared__ uint32_t tab[kTabGroups * kTabStride];
  __shared__ int s_arow[kUnitRows];

  const int b = blockIdx.x;
  const bool second = args.nprob > 1 && b >= args.prob[1].wg_begin;
  const GemmProblem P = second ? args.prob[1] : args.prob[0];
  // the prepared copy's flag, requested first so its latency overlaps the
  // work list and row-index reads
  constexpr bool kCanBuf = AF16 && !WX;
  constexpr bool kCanPrep = kCanBuf && MODE != kStoreC;  // the layer's projections
  const uint32_t pflag = *(kCanPrep && P.Pq != nullptr ? P.Pflag : &g_flag_off);  // unconditional load
  // Workgroup i runs on XCD i % 8. Consecutive groups of 8 workgroups take 8
  // units (one per XCD); the N-slices of one unit stay on one XCD, so its
  // gathered activation rows are fetched into that XCD's L2 once.
  const int lb = b - P.wg_begin;
  Unit U;
  int unit, nsl = P.nslices;
  bool narrow = false;
  if (P.units) {
    // Listed units (largest first): all but the last ntail or so run as
    // nslices full-width items; the tail runs as 2 * nslices half-width
    // items, so the last round is made of short pieces. nbig is a multiple
    // of 8, so both parts keep a unit's slices on one XCD.
    const int nu = *P.num_units;
    const int nbig = P.ntail > 0 ? max(nu - P.ntail, 0) & ~7 : nu;
    const int big_wgs = ((nbig + 7) & ~7) * nsl;  // whole groups of 8 units
    int j = lb;
    if (j >= big_wgs) {
      j -= big_wgs;
      nsl *= 2;
      narrow = true;
    }
    const int slot = j >> 3;
    unit = (narrow ? nbig : 0) + (slot / nsl) * 8 + (j & 7);
    U.slice = slot % nsl;
    if (unit >= nu) return;
    const int32_t *u = P.units + 3 * (int64_t)unit;
    U.e = u[0];
    U.r0 = u[1];
    U.nr = u[2];
  } else {
    const int slot = lb >> 3;
    unit = (slot / nsl) * 8 + (lb & 7);
    U.slice = slot % nsl;
    const int urows = P.unit_rows > 0 ? P.unit_rows : kUnitRows;
    U.e = 0;
    U.r0 = unit * urows;
    U.nr = min(urows, P.implicit_rows - U.r0);
    if (U.nr <= 0) return;
  }

  // prepared weights (the host sets Pq only when K is a multiple of the
  // step; the projection's flag says whether its scales allowed the
  // prepared form), else buffer loads when K is a multiple of the step
  const bool buf = kCanBuf && (P.K & (kKStep - 1)) == 0;
  const bool prep = buf && pflag != 0u;
  // A unit has at most kUnitRows rows: the layer's lists by construction; a
  // caller's block map for the stand-alone GEMM by contract (blocks of 1..32
  // rows), and of a longer block only its first kUnitRows rows are computed.
  // (A loop over pieces of a long block around the item made the compiler
  // spill the item's registers and move code into called functions.)
  if (U.nr <= 0) return;
  U.nr = min(U.nr, kUnitRows);
  run_item<MODE, AF16, WX, CHECK, kCanBuf, kCanPrep>(P, U, lds, s_arow, tab, buf, prep, narrow);
}

}  // namespace

hipError_t MOE_GEMM_LAUNCH(const GemmArgs &a, int mode, bool a_f16, hipStream_t s, hipEvent_t start,
                           hipEvent_t stop, bool expanded) {
  const dim3 grid(a.total_wg), block(kGemmThreads);
  if (a.total_wg == 0) return hipSuccess;
#ifdef MOE_GEMM_SMALL_BUILD
  // the small-unit build serves the layer's two projections over fp16
  // activations only
  if (expanded || !a_f16 || (mode != kSwiGLU && mode != kStoreH)) return hipErrorInvalidValue;
  const bool check = a.prob[0].overflow != nullptr;
  if (mode == kSwiGLU) {
    if (check) hipExtLaunchKernelGGL((gemm_kernel<kSwiGLU, true, false, true>), grid, block, 0, s, start, stop, 0, a);
    else       hipExtLaunchKernelGGL((gemm_kernel<kSwiGLU, true, false>), grid, block, 0, s, start, stop, 0, a);
  } else {
    if (check) hipExtLaunchKernelGGL((gemm_kernel<kStoreH, true, false, true>), grid, block, 0, s, start, stop, 0, a);
    else       hipExtLaunchKernelGGL((gemm_kernel<kStoreH, true, false>), grid, block, 0, s, start, stop, 0, a);
  }
  return hipGetLastError();
#else
  if (expanded) {  // layer GEMMs over expanded weights (unfused ablation)
    switch (mode) {
      case kSwiGLU: hipExtLaunchKernelGGL((gemm_kernel<kSwiGLU, true, true>), grid, block, 0, s, start, stop, 0, a); break;
      case kStoreH: hipExtLaunchKernelGGL((gemm_kernel<kStoreH, true, true>), grid, block, 0, s, start, stop, 0, a); break;
      default: return hipErrorInvalidValue;
    }
  } else if (a_f16) {
    switch (mode) {
      case kSwiGLU:
        if (a.prob[0].overflow)
          hipExtLaunchKernelGGL((gemm_kernel<kSwiGLU, true, false, true>), grid, block, 0, s, start, stop, 0, a);
        else
          hipExtLaunchKernelGGL((gemm_kernel<kSwiGLU, true, false>), grid, block, 0, s, start, stop, 0, a);
        break;
      case kStoreH:
        if (a.prob[0].overflow)
          hipExtLaunchKernelGGL((gemm_kernel<kStoreH, true, false, true>), grid, block, 0, s, start, stop, 0, a);
        else
          hipExtLaunchKernelGGL((gemm_kernel<kStoreH, true, false>), grid, block, 0, s, start, stop, 0, a);
        break;
      default: hipExtLaunchKernelGGL((gemm_kernel<kStoreC, true, false>), grid, block, 0, s, start, stop, 0, a); break;
    }
  } else if (mode == kSwiGLU) {
    // bf16 activations converted while staged: the shared expert's gate/up
    // beside the routing (concurrent graph form)
    hipExtLaunchKernelGGL((gemm_kernel<kSwiGLU, false, false>), grid, block, 0, s, start, stop, 0, a);
  } else {
    // bf16 activations: stand-alone GEMM over block-map entries (<= 32 rows)
    hipExtLaunchKernelGGL((gemm_kernel<kStoreC, false, false>), grid, block, 0, s, start, stop, 0, a);
  }
  return hipGetLastError();
#endif
}

#ifndef MOE_GEMM_SMALL_BUILD
// Weights of `rows` rows of K inputs (all experts of a projection, stored
// back to back) rebuilt once into fp16 in device memory, each 8-run in the
// rebuild order, with the same arithmetic as the GEMM's on-chip rebuild.
__global__ __launch_bounds__(256) void expand_kernel(const uint32_t *q, const uint16_t *sc, const uint16_t *bi,
                                                     int64_t words, int K, uint16_t *out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= words) return;
  const int kw = K >> 3, G = K >> 6;
  const int64_t row = i / kw;
  const int wi = (int)(i - row * kw);
  const int64_t gi = row * G + (wi >> 3);
  const uint32_t packed = rb_pack_scale_bias(sc[gi], bi[gi]);
  const rb_h8 w = rb_rebuild(q[i], packed, rb_consts());
  reinterpret_cast<rb_h8 *>(out)[i] = w;
}

// Prepared codes (prep_layout.h): one thread per 16-byte chunk, i.e. per
// (expert, slice, step, wave, block, lane).
__global__ __launch_bounds__(256) void prep_codes_kernel(const uint32_t *q, int E, int N, int K, bool swiglu,
                                                         uint4 *pq) {
  const int steps = K / kPrepStep;
  const int64_t per_e = (int64_t)prep_slices(N, swiglu) * steps * (kPrepBlock / 16);
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= per_e * E) return;
  const int e = (int)(i / per_e);
  const int64_t r = i - e * per_e;
  const int blk = (int)(r >> 10), in = (int)(r & 1023);
  const int t = blk / steps, st = blk - t * steps;
  const int chunk = in >> 6, lane = in & 63;
  const int w = chunk >> 2, b = chunk & 3, qq = lane >> 4, c = lane & 15;
  const int lc = (swiglu ? (b < 2 ? 32 * w + 16 * b : 128 + 32 * w + 16 * (b - 2)) : 64 * w + 16 * b) + c;
  const int n = prep_row(t, lc, N, swiglu);
  uint4 v = make_uint4(0u, 0u, 0u, 0u);
  if (n >= 0)
    v = *reinterpret_cast<const uint4 *>(q + (int64_t)e * N * (K / 8) + (int64_t)n * (K / 8) + 16 * st + 4 * qq);
  pq[i] = v;
}

__global__ void prep_flag_init_kernel(uint32_t *flag, uint32_t v) { *flag = v; }

// Clears the flag when any scale is outside the range of the one-rounding
// rebuild (one atomic per wave that holds such a scale).
__global__ __launch_bounds__(256) void prep_check_kernel(const uint16_t *sc, int64_t n, uint32_t *flag) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const bool bad = i < n && !prep_scale_ok(__uint_as_float((uint32_t)sc[i] << 16));
  const uint64_t m = __ballot(bad);
  if (m != 0ull && (threadIdx.x & 63) == (int)(__ffsll((long long)m) - 1)) atomicAnd(flag, 0u);
}

// Prepared table: one thread per (expert, slice, group, table column) dword.
__global__ __launch_bounds__(256) void prep_table_kernel(const uint16_t *sc, const uint16_t *bi, int E, int N, int K,
                                                         bool swiglu, const uint32_t *flag, uint32_t *pt) {
  const int G = K / 64;
  const int64_t per_e = (int64_t)prep_slices(N, swiglu) * G * kPrepCols;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= per_e * E) return;
  const int e = (int)(i / per_e);
  const int64_t r = i - e * per_e;
  const int c = (int)(r % kPrepCols), tg = (int)(r / kPrepCols);
  const int t = tg / G, g = tg - t * G;
  const int n = prep_row(t, c, N, swiglu);
  const int64_t gi = (int64_t)e * N * G + (int64_t)n * G + g;
  pt[i] = n >= 0 && *flag != 0u ? rb_pack_sub(sc[gi], bi[gi]) : 0u;
}

hipError_t launch_prepare(const uint32_t *q, const uint16_t *sc, const uint16_t *bi, int E, int N, int K,
                          bool swiglu, uint8_t *pq, uint32_t *pt, uint32_t *flag, hipStream_t s) {
  const int64_t n16 = (int64_t)E * prep_code_bytes(N, K, swiglu) / 16;
  const int64_t nt = (int64_t)E * prep_table_dwords(N, K, swiglu);
  const int64_t ns = (int64_t)E * N * (K / 64);
  hipLaunchKernelGGL(prep_flag_init_kernel, dim3(1), dim3(1), 0, s, flag, 1u);
  if (ns > 0)
    hipLaunchKernelGGL(prep_check_kernel, dim3((unsigned)ceil_div(ns, 256)), dim3(256), 0, s, sc, ns, flag);
  if (n16 > 0)
    hipLaunchKernelGGL(prep_codes_kernel, dim3((unsigned)ceil_div(n16, 256)), dim3(256), 0, s, q, E, N, K, swiglu,
                       reinterpret_cast<uint4 *>(pq));
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || nt == 0) return err;
  hipLaunchKernelGGL(prep_table_kernel, dim3((unsigned)ceil_div(nt, 256)), dim3(256), 0, s, sc, bi, E, N, K, swiglu,
                     flag, pt);
  return hipGetLastError();
}

hipError_t launch_prep_flag(uint32_t *flag, uint32_t v, hipStream_t s) {
  hipLaunchKernelGGL(prep_flag_init_kernel, dim3(1), dim3(1), 0, s, flag, v);
  return hipGetLastError();
}

hipError_t launch_expand(const uint32_t *q, const uint16_t *sc, const uint16_t *bi, int64_t rows, int K,
                         uint16_t *out, hipStream_t s) {
  const int64_t words = rows * (K / 8);
  if (words == 0) return hipSuccess;
  hipLaunchKernelGGL(expand_kernel, dim3((unsigned)ceil_div(words, 256)), dim3(256), 0, s, q, sc, bi, words, K, out);
  return hipGetLastError();
}

#endif  // MOE_GEMM_SMALL_BUILD

}  // namespace moe
