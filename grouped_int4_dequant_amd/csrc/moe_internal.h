// Internal declarations of the MI355X (gfx950) MoE layer library: kernel
// argument blocks, launch helpers and small device utilities. Not installed;
// the public interface is include/moe_int4.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_int4.h"

namespace moe {

constexpr int kGroup = 64;         // weights per scale/bias group
constexpr int kUnitRows = 96;      // max rows of one GEMM work unit (three 32-row blocks)
constexpr int kSubChunk = 64;      // tokens per routing bitmask (one wave's lanes)
constexpr int kThreads = 256;      // threads per workgroup of the routing and combine kernels
constexpr int kGemmThreads = 512;  // threads per workgroup of the grouped GEMM (8 waves)

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }

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
};

hipError_t launch_topk(const TopkArgs &a, hipStream_t s);
hipError_t launch_scan(const ScanArgs &a, hipStream_t s);
hipError_t launch_combine(const CombineArgs &a, hipStream_t s);

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
  int N, K;
  const int32_t *units;      // [*][3] (expert, first row, rows <= 128); nullptr: implicit
  const int32_t *num_units;  // device count of units
  int implicit_rows;         // implicit units: rows [0, implicit_rows) of expert 0
  int nslices;               // workgroups per unit along N
  int wg_begin;              // first workgroup (in remapped order) of this problem
  // outputs
  float *C; int ldc;          // kStoreC
  uint16_t *H; int ldh;       // kSwiGLU (permuted-run columns), kStoreH (natural columns)
};

struct GemmArgs {
  GemmProblem prob[2];
  int nprob;
  int total_wg;              // workgroups in the launch (multiple of 8)
};

// a_f16: the A operand is fp16 in the permuted-run layout (fast path);
// otherwise bf16 in natural order, converted while staging.
hipError_t launch_gemm(const GemmArgs &a, int mode, bool a_f16, hipStream_t s);

}  // namespace moe
