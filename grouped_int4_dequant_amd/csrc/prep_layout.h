// Prepared weight layout of the prefill grouped GEMM (gfx950): one
// projection's int4 codes rearranged into the order in which a workgroup
// item reads them, and its scale/bias table pre-converted into the order of
// the item's LDS table, so that every K step reads one contiguous 16 KiB
// block of codes and every table fill is a plain copy of contiguous rows.
//
// The content is the pages' format unchanged (4-bit codes, one scale and one
// bias per 64 weights of a row; Lily-ES "Precarga: mantenga los pesos
// empaquetados, siga enrutando en la GPU"); only the order of the bytes and
// the pre-computed fp16 pair (s, b + 8 s) of the rebuild differ.
//
// A projection has N weight rows (output columns) and K inputs, K a multiple
// of 128. Its columns are cut into slices of 256 table columns: for the
// gate/up projection (swiglu, N = 2 f) slice t holds gate rows 128 t + c for
// table columns c < 128 and up rows f + 128 t + c - 128 for c >= 128; for a
// plain projection slice t holds rows 256 t + c. Rows at or past their end
// are zero codes and zero table entries.
//
// Codes, per expert: slice t, then K step s (128 inputs), then a 16 KiB
// block of 16 chunks of 1 KiB; chunk 4 w + b (w = wave 0..3, b = 16-column
// block 0..3 of the wave) holds, for lane l = 16 q + c (q = 32-input quarter,
// c = column within the block), the 16 bytes of codes of that column's row
// for inputs [128 s + 32 q, 128 s + 32 q + 32), in the original packing.
// The column of chunk (w, b), lane column c, in table order: swiglu: gate
// 32 w + 16 b + c for b < 2, up 128 + 32 w + 16 (b - 2) + c for b >= 2;
// plain: 64 w + 16 b + c.
//
// Table, per expert: slice t, then group g (64 inputs, K / 64 groups), then
// 256 dwords, one per table column: fp16 (s * 2^20) in the low half and
// fp16 b in the high half, both exact from the bf16 scale and bias when
// |s| < 2^-4, the pair of the one-rounding rebuild (rb_rebuild_sub). A
// projection with any scale outside that range keeps a zero table and its
// flag (below) at 0, and its GEMM reads the original arrays.
//
// Flags: the prepared copy starts with a 256-byte header whose uint32 words
// 0..3 hold, for the routed gate/up, routed down, shared gate/up and shared
// down projections, 1 when the projection's prepared form is in use.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kPrepCols = 256;     // table columns of a slice
constexpr int kPrepStep = 128;     // inputs per K step
constexpr int kPrepBlock = 16384;  // bytes of codes per slice and step

// slices of a projection with N rows: swiglu (N = 2 f) f / 128, plain N / 256
__host__ __device__ inline int prep_slices(int N, bool swiglu) {
  return swiglu ? (N / 2 + 127) / 128 : (N + kPrepCols - 1) / kPrepCols;
}
__host__ __device__ inline int64_t prep_code_bytes(int N, int K, bool swiglu) {
  return (int64_t)prep_slices(N, swiglu) * (K / kPrepStep) * kPrepBlock;
}
__host__ __device__ inline int64_t prep_table_dwords(int N, int K, bool swiglu) {
  return (int64_t)prep_slices(N, swiglu) * (K / 64) * kPrepCols;
}

constexpr int kPrepHeader = 256;   // bytes of the flags header
enum PrepFlag : int { kFlagGu = 0, kFlagDn = 1, kFlagShGu = 2, kFlagShDn = 3 };

// a scale the one-rounding rebuild takes: 0, or 2^-34 <= |s| < 2^-4 (s * 2^20
// a normal fp16 that holds all 8 bits of a bf16 scale)
__host__ __device__ inline bool prep_scale_ok(float s) {
  const float a = s < 0.f ? -s : s;
  return a == 0.f || (a >= 5.820766091346741e-11f && a < 0.0625f);
}

// weight row of table column c (0..255) of slice t, or -1 past the end
__host__ __device__ inline int prep_row(int t, int c, int N, bool swiglu) {
  if (swiglu) {
    const int f = N / 2, j = 128 * t + (c & 127);
    return j < f ? (c < 128 ? j : f + j) : -1;
  }
  const int n = kPrepCols * t + c;
  return n < N ? n : -1;
}

// chunk (4 w + b) of the 16 KiB block that holds table column lc (a
// multiple of 16)
__host__ __device__ inline int prep_chunk(int lc, bool swiglu) {
  if (swiglu) {
    const int u = lc & 127;
    return 4 * (u >> 5) + ((u >> 4) & 1) + (lc >= 128 ? 2 : 0);
  }
  return 4 * (lc >> 6) + ((lc >> 4) & 3);
}

}  // namespace moe
