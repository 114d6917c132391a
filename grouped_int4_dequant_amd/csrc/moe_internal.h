// Internal declarations of the MI355X (gfx950) MoE layer library: kernel
// argument blocks, launch helpers and small device utilities. Not installed;
// the public interface is include/moe_int4.h.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_int4.h"

namespace moe {

constexpr int kGroup = 64;         // weights per scale/bias group
// Max rows of one GEMM work unit: three 32-row blocks, or (the small-unit
// GEMM build, for calls whose experts hold few rows each) one.
#ifndef MOE_UNIT_ROWS
#define MOE_UNIT_ROWS 96
#endif
constexpr int kUnitRows = MOE_UNIT_ROWS;
constexpr int kUnitRowsSmall = 32;
constexpr int kSubChunk = 64;      // tokens per routing bitmask (one wave's lanes)
constexpr int kThreads = 256;      // threads per workgroup of the routing and combine kernels
// Grouped-GEMM workgroup shape (compile-time; the defaults are the measured
// best): waves per workgroup (each owns 64 weight rows, i.e. output
// columns, of a full-width item), scale/bias groups held in the LDS table at
// a time, and workgroups resident per CU. Two 4-wave workgroups per CU (one wave of each per SIMD,
// about 65 KiB of LDS each) keep the matrix pipes busy while the other
// workgroup waits at its barrier or runs its prologue or epilogue.
#ifndef MOE_GEMM_WAVES
#define MOE_GEMM_WAVES 4
#endif
#ifndef MOE_GEMM_TAB_GROUPS
#define MOE_GEMM_TAB_GROUPS 16
#endif
#ifndef MOE_GEMM_WGS_PER_CU
#define MOE_GEMM_WGS_PER_CU 2
#endif
constexpr int kGemmThreads = 64 * MOE_GEMM_WAVES;  // threads per workgroup of the grouped GEMM
constexpr int kGemmCols = 64 * MOE_GEMM_WAVES;     // weight rows of a full-width GEMM item (64 per wave)

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// A value the path stores in fp16 fell outside fp16's finite range (or was
// NaN): OR `bit` into the caller's overflow word, when one was given.
__device__ __forceinline__ bool f16_out_of_range(float v) { return !(fabsf(v) < 65520.f); }
// Either fp16 half of a packed pair is infinite or NaN.
__device__ __forceinline__ bool f16x2_nonfinite(uint32_t p) {
  return (p & 0x7C00u) == 0x7C00u || (p & 0x7C000000u) == 0x7C000000u;
}
__device__ __forceinline__ void note_overflow(uint32_t *flag, bool bad, uint32_t bit) {
  if (flag && bad) atomicOr(flag, bit);
}
inline int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }

// SwiGLU of one (gate, up) pair: silu(g) * u with silu(g) = g / (1 + e^-g).
// The reciprocal is one v_rcp_f32 (about 1 ulp) instead of a correctly
// rounded division (about ten instructions per element, a fifth of the
// gate/up kernel's VALU work at 64 rows per expert); h is stored in fp16,
// whose rounding is 2^13 times coarser.
__device__ __forceinline__ float swiglu(float g, float u) {
  return g * __builtin_amdgcn_rcpf(1.f + __expf(-g)) * u;
}

// ------------------------------------------------------------------ routing
struct TopkArgs {
  const float *logits;
  int T, E, k;
  int32_t *topk_ids;
  float *topk_w;
  // auxiliary work (layer forward only; x16 == nullptr disables it)
  const uint16_t *x;        // bf16 [T][d]
  uint16_t *x16;            // fp16 [T][d], each 8-element run stored as 0,4,1,5,2,6,3,7
  int d;
  uint32_t *overflow;       // nullable: MOE_OVERFLOW_X when an x16 value is not finite
  uint8_t *ids8;            // nullable: topk_ids again, one byte each (E <= 256)
  int topk_wgs;             // set by launch_topk: workgroups [0, topk_wgs) route, the rest convert x
};

// y[t] = sum_j w[t][j] * o[pair_pos[t*k+j]] + o_sh[t], slot order, fp32.
struct CombineArgs {
  int T, d, k;
  const uint16_t *o;        // fp16 [T*k][d] routed expert outputs, expert-sorted rows
  const uint16_t *o_sh;     // fp16 [T][d] shared expert outputs (nullptr: none)
  const int32_t *pair_pos;  // [T*k]
  const float *topk_w;      // [T][k]
  float *y;                 // fp32 [T][d]
};

struct ScanArgs {
  int T, E, k;
  const int32_t *topk_ids;
  int32_t *counts, *offsets, *sorted_pair, *sorted_token, *pair_pos;
  int32_t *block_map, *num_blocks;
  int max_blocks;
  int32_t *units, *num_units;   // optional GEMM work list (nullptr: none)
  int max_units;
  int unit_rows;                // rows per GEMM work unit at most (16..kUnitRows)
  int32_t *chunk_counts;        // scratch [ceil(T/64)][E] (two-pass form only)
  int count_inline;             // set by launch_scan: the scatter workgroups count every pair themselves
  int ids_vec;                  // set by launch_scan: topk_ids 16-byte aligned and T*k a multiple of 4
  const uint8_t *ids8;          // nullable: byte copy of topk_ids (E <= 256, 16-byte aligned, T*k % 16 == 0)
};

// logits[t][e] = sum_k x[t][k] * w[e][k] (bf16 inputs, fp32 accumulation).
struct RouterArgs {
  const uint16_t *x;        // bf16 [T][d]
  const uint16_t *w;        // bf16 [E][d]
  int T, d, E;
  float *logits;            // fp32 [T][E]
};
hipError_t launch_router(const RouterArgs &a, hipStream_t s);


// Optional events (nullable) are attached to a kernel's dispatch: start at
// its first wave, stop at its end, with no extra packet between kernels.
hipError_t launch_topk(const TopkArgs &a, hipStream_t s, hipEvent_t start = nullptr,
                       hipEvent_t stop = nullptr);
hipError_t launch_scan(const ScanArgs &a, hipStream_t s, hipEvent_t stop = nullptr);
hipError_t launch_combine(const CombineArgs &a, hipStream_t s, hipEvent_t stop = nullptr);

// --------------------------------------------------------------- grouped GEMM
// Epilogue modes of the grouped GEMM kernel.
enum GemmMode : int {
  kStoreC = 0,    // C[p][n] = acc (fp32)                     (stand-alone GEMM)
  kSwiGLU = 1,    // H[p][n] = fp16(silu(acc_gate) * acc_up)  (gate/up projection)
  kStoreH = 2,    // H[p][n] = fp16(acc)                      (down projection)
};

// One grouped problem: a list of work units (expert, first row, rows) over a
// row space p, each row p reading activation row arow(p).
struct GemmProblem {
  const void *A;             // activations, row-major [*][lda]
  int lda;
  const int32_t *a_row;      // row p reads A[a_row[p]]; nullptr: A[p]
  const uint32_t *Wq;        // expert 0 packed codes [N][K/8]
  const uint16_t *Ws, *Wb;   // expert 0 scales / biases [N][K/64]
  int64_t wq_estride, ws_estride;  // per-expert element strides
  const uint16_t *Wx;        // expanded fp16 weights [N][K] of expert 0 (unfused ablation only)
  int64_t wx_estride;
  int N, K;
  const int32_t *units;      // [*][3] (expert, first row, rows <= 128); nullptr: implicit
  const int32_t *num_units;  // device count of units
  int implicit_rows;         // implicit units: rows [0, implicit_rows) of expert 0
  int unit_rows;             // implicit units: rows per unit (16..kUnitRows; 0 means kUnitRows)
  int nslices;               // workgroups per unit along N
  int ntail;                 // listed units: about this many trailing units run as 2*nslices half-width items
  int wg_begin;              // first workgroup (in remapped order) of this problem
  // prepared weights (nullptr: read Wq/Ws/Wb): codes in tile order and the
  // (fp16 s, fp16 b + 8 s) table in table order, per expert (K a multiple of
  // 128; layout in prep_layout.h)
  const uint8_t *Pq; int64_t pq_estride;   // bytes
  const uint32_t *Pt; int64_t pt_estride;  // dwords
  const uint32_t *Pflag;                   // the projection's flag: 0 = use Wq/Ws/Wb after all
  // outputs
  float *C; int ldc;          // kStoreC
  uint16_t *H; int ldh;       // kSwiGLU (permuted-run columns), kStoreH (natural columns)
  uint32_t *overflow;         // nullable: MOE_OVERFLOW_H / _O when a stored fp16 value is out of range
};

struct GemmArgs {
  GemmProblem prob[2];
  int nprob;
  int total_wg;              // workgroups in the launch (multiple of 8)
};

// a_f16: the A operand is fp16 in the permuted-run layout (fast path);
// otherwise bf16 in natural order, converted while staging.
// expanded: the weights are read expanded from Wx (unfused ablation; modes
// kSwiGLU and kStoreH).
hipError_t launch_gemm(const GemmArgs &a, int mode, bool a_f16, hipStream_t s, hipEvent_t start = nullptr,
                       hipEvent_t stop = nullptr, bool expanded = false);
// The same GEMM compiled for units of at most kUnitRowsSmall rows (148
// registers, three workgroups per CU): the layer's projections when its
// experts hold about 20 rows or fewer on average.
hipError_t launch_gemm_small(const GemmArgs &a, int mode, bool a_f16, hipStream_t s, hipEvent_t start = nullptr,
                             hipEvent_t stop = nullptr, bool expanded = false);
// Prepared copy of one projection's weights for E experts (prep_layout.h):
// swiglu: rows 0..N/2-1 gate, N/2..N-1 up.
hipError_t launch_prepare(const uint32_t *q, const uint16_t *sc, const uint16_t *bi, int E, int N, int K,
                          bool swiglu, uint8_t *pq, uint32_t *pt, uint32_t *flag, hipStream_t s);
// One flag word of a prepared copy set to v (a kernel, so the call can be captured).
hipError_t launch_prep_flag(uint32_t *flag, uint32_t v, hipStream_t s);
// Unfused ablation: weights of rows x K expanded into fp16 (rebuild order).
hipError_t launch_expand(const uint32_t *q, const uint16_t *sc, const uint16_t *bi, int64_t rows, int K,
                         uint16_t *out, hipStream_t s);

// ------------------------------------------------------------------ decode
// Calls of at most kDecodeMaxT tokens run as two kernels (decode_kernels.hip):
// gate/up with the routing repeated in every workgroup, then down with the
// weighted combine. y is written directly.
constexpr int kDecodeMaxT = 8;
constexpr int kDecodeMaxPairs = 64;   // T * k
constexpr int kDecodeMaxSlots = 12;   // k + 1 (waves of a down workgroup)

struct DecodeArgs {
  const float *logits;        // [T][E]
  const uint16_t *x;          // bf16 [T][d]
  int T, d, f, f_sh, E, k, fmax;
  const uint32_t *gu_q; const uint16_t *gu_s, *gu_b; int64_t gu_qs, gu_ss;  // routed, per-expert strides
  const uint32_t *dn_q; const uint16_t *dn_s, *dn_b; int64_t dn_qs, dn_ss;
  const uint32_t *sh_gu_q; const uint16_t *sh_gu_s, *sh_gu_b;
  const uint32_t *sh_dn_q; const uint16_t *sh_dn_s, *sh_dn_b;
  int32_t *ids; float *gates; // [T][k], written by the gate/up kernel
  uint16_t *h;                // fp16 [T][k+1][fmax] (slot k: shared expert); within each
                              // 8 columns, the rebuild order 0,4,1,5,2,6,3,7
  float *y;                   // fp32 [T][d]
  uint32_t *overflow;         // nullable: MOE_OVERFLOW_X / _H bits
};

bool decode_supported(int T, const moe_layer_t *L);
// gu_start, gu_stop, dn_stop (nullable): dispatch events of the two kernels.
hipError_t launch_decode(const DecodeArgs &a, hipStream_t s, hipEvent_t gu_start, hipEvent_t gu_stop,
                         hipEvent_t dn_stop);

}  // namespace moe
