/*
 * moe_int4.h - C ABI of the grouped int4-dequant Mixture-of-Experts layer for
 * AMD MI355X (gfx950).
 *
 * The layer is the prefill MoE block the Lily pages describe for
 * Qwen3.6-35B-A3B: a router picks k of E experts per token plus one shared
 * expert that sees every token; routing (histogram, prefix scan, scatter,
 * block map) stays on the GPU with no host synchronisation; a grouped GEMM
 * streams 4-bit groupwise-affine weights and dequantises them on chip, one
 * tile at a time, accumulating in FP32 so the expanded weights never reach
 * device memory; the expert outputs are combined with the router weights.
 *
 * Pages cited (titles as published):
 *   Lily-EN  "Perplexity Open Sources Lily: A Rust + Metal Inference Engine for
 *            Qwen3.6-35B-A3B on Apple Silicon" (insight.aitobox.com), sections
 *            "Three Workload Shapes", "Prefill: Keep Weights Packed, Keep
 *            Routing on the GPU", "Decode: Minimize Bytes Moved Per Token".
 *   Lily-ES  "Perplexity open sources Lily: un motor de inferencia ... para
 *            Qwen3.6-35B-A3B en Apple Silicon" (7minutos.es), sections
 *            "Precarga: mantenga los pesos empaquetados, siga enrutando en la
 *            GPU" and "Decodificar: minimizar los bytes movidos por token".
 *
 * Conventions shared by every entry point
 *   - Pointers are DEVICE pointers owned by the caller, unless stated. The
 *     library never allocates, frees or retains them past the call.
 *   - bf16 and fp16 values are passed as uint16_t bit patterns.
 *   - Every array is contiguous and row-major.
 *   - Calls only enqueue work on the given stream and return; they never
 *     synchronise and never read device memory on the host. A device-side
 *     fault surfaces at the caller's next synchronisation.
 *   - Return value: MOE_OK (0) or a negative MOE_E* code. Argument checks run
 *     before anything is enqueued; on an error nothing is enqueued.
 *   - Calls on different streams with different workspaces are independent.
 *     Calls that share a workspace must be ordered by the caller.
 *
 * Quantised weight format (Lily-ES "Precarga..."; the Lily-HE prefill section
 * says the same): every 64 consecutive weights along the input (K) dimension
 * form a group that shares one bf16 scale s and one bf16 bias b; the weight is
 * w = s * q + b with the 4-bit code q in 0..15. Codes are packed eight to a
 * uint32, low nibble first: q[n][8c+i] = (Wq[n][c] >> 4i) & 15.
 *
 * Numerics of the GPU path: each 64-weight group is rebuilt in registers as
 * fp16 values fp16(s*(q-8) + (b+8s)), which is within one fp16 rounding of
 * s*q + b for scales of at least 2^-14; activations enter the matrix cores as
 * fp16 and products accumulate in fp32. A bf16 x converts to fp16 exactly
 * when x == 0 or 2^-17 <= |x| <= 65280 (the largest bf16 value below fp16's
 * overflow); smaller magnitudes round to fp16's subnormal spacing 2^-24 (below
 * 2^-25 to zero) and |x| >= 65536 becomes infinite. The expert intermediates
 * h and the expert outputs are held as fp16 (they must stay below 65520 in
 * magnitude or they become infinite); y is fp32.
 */
#ifndef MOE_INT4_H
#define MOE_INT4_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define MOE_OK            0
#define MOE_EINVAL       -1  /* null pointer, bad size, k > E, misaligned pointer */
#define MOE_EUNSUPPORTED -2  /* d, f or f_sh not a multiple of 64, E > 1024, T too large */
#define MOE_EWORKSPACE   -3  /* ws_bytes smaller than the size the call needs */
#define MOE_EHIP         -4  /* the HIP runtime reported an error at launch */

/* Limits. */
#define MOE_MAX_EXPERTS   1024
#define MOE_MAX_TOKENS    (1 << 20)  /* per moe_prefill_chunked call */
#define MOE_MAX_CALL_TOKENS 16384    /* per moe_route / moe_layer_forward call and per chunk */
#define MOE_BLOCK_ROWS    32  /* rows per block of the block map (32-row tiles) */

/*
 * One MoE layer (Lily-EN "Three Workload Shapes": a router scores E experts
 * and picks k, plus one shared expert that sees every token). The expert FFN
 * is SwiGLU: a = W_gu x, h = silu(a[0:f]) * a[f:2f], o = W_dn h.
 *
 *   gu_q  [E][2f][d/8]   gu_s, gu_b  [E][2f][d/64]  rows 0..f-1 gate, f..2f-1 up
 *   dn_q  [E][d][f/8]    dn_s, dn_b  [E][d][f/64]
 *   sh_*  the same for the shared expert without the E dimension and with
 *         f_sh in place of f; f_sh == 0 means the layer has no shared expert
 *         and the sh_* pointers are ignored.
 *   prep  NULL, or a prepared copy of the same weights written by
 *         moe_prepare_weights for this layer (256-byte aligned, kept alive
 *         and unchanged by the caller). When set, the prefill grouped GEMMs
 *         read it instead of the arrays above (see moe_prepare_weights for
 *         the arithmetic); the few-token form and the ablation forms still
 *         read the arrays, which must stay valid.
 * All weight pointers must be 16-byte aligned.
 */
typedef struct moe_layer {
  int32_t d, f, E, k, f_sh;
  const uint32_t *gu_q;    const uint16_t *gu_s,    *gu_b;
  const uint32_t *dn_q;    const uint16_t *dn_s,    *dn_b;
  const uint32_t *sh_gu_q; const uint16_t *sh_gu_s, *sh_gu_b;
  const uint32_t *sh_dn_q; const uint16_t *sh_dn_s, *sh_dn_b;
  const void *prep;
} moe_layer_t;

/*
 * Bytes of device memory a prepared copy of L's weights takes (about the
 * size of the weights themselves: the same codes, and one 4-byte pair per
 * group in place of the bf16 scale and bias), or 0 when L is invalid or d,
 * f or f_sh is not a multiple of 128. Host-only: reads L's scalar fields.
 */
size_t moe_prepared_bytes(const moe_layer_t *L);

/*
 * Write the prepared copy of L's weights into dst (device memory of at least
 * moe_prepared_bytes(L) bytes, 256-byte aligned), enqueued on stream; then
 * set L->prep = dst (the caller does) to have the prefill GEMMs use it.
 * The copy holds the same 4-bit codes rearranged so that one workgroup item
 * of the grouped GEMM reads each 128-input step of its 256 output columns as
 * one contiguous 16 KiB block, and each group's scale and bias as the fp16
 * pair (s * 2^20, b) in the order of the item's columns, from which one
 * fused multiply-add per two weights forms fp16(s * q + b) with a single
 * rounding (Lily-EN "Prefill: Keep Weights Packed, Keep Routing on the
 * GPU": the weights stay 4-bit in memory; the layout is this library's).
 * That form needs |s| < 2^-4 (and s = 0 or |s| >= 2^-34); a projection with
 * any other scale keeps its flag at 0 and its GEMM reads the original
 * arrays. dst then holds, each part starting at a multiple of 256 bytes: a
 * header whose uint32 words 0..3 are the flags of the routed gate/up,
 * routed down, shared gate/up and shared down projections (1: prepared form
 * in use), the routed experts' gate/up codes, their table, the routed down
 * codes, their table, and (f_sh > 0) the same four parts of the shared
 * expert. Results equal those of the original arrays bit for bit whenever
 * b + 8 s is exact in fp16 (as for the synthetic workloads' weights, whose
 * |b + 8 s| stays below s); otherwise the prepared form is the one that
 * rounds once. One-time work per layer (a few hundred microseconds per GB).
 * L->prep is ignored. Errors: MOE_EINVAL (invalid layer, null or
 * misaligned dst), MOE_EUNSUPPORTED (d, f or f_sh not a multiple of 128),
 * MOE_EWORKSPACE (dst_bytes too small), MOE_EHIP.
 */
int moe_prepare_weights(const moe_layer_t *L, void *dst, size_t dst_bytes, hipStream_t stream);

/*
 * Routing outputs for T tokens (Lily-EN "Prefill: Keep Weights Packed, Keep
 * Routing on the GPU": histogram, prefix scan, scatter and block map all stay
 * on the GPU). Caller-owned device buffers:
 *   topk_ids     int32 [T][k]  picked experts, by (logit desc, expert asc);
 *                equal logits (IEEE ==, so -0.0 == +0.0) go to the lower index
 *   topk_w       fp32  [T][k]  softmax over the k picked logits
 *   counts       int32 [E]     pairs (t, j) routed to each expert
 *   offsets      int32 [E+1]   exclusive prefix sum of counts; offsets[E] = T*k
 *   sorted_pair  int32 [T*k]   pair index t*k+j of each expert-sorted row;
 *                stable: ascending t*k+j inside each expert's segment
 *   sorted_token int32 [T*k]   token of each sorted row
 *   pair_pos     int32 [T*k]   sorted row of pair t*k+j (inverse permutation)
 *   block_map    int32 [max_blocks][3] with max_blocks = ceil(T*k/32) + E:
 *                (expert, first sorted row, rows in 1..32) for every 32-row
 *                block of every non-empty expert, expert-major; unused
 *                entries hold (-1, 0, 0)  (Lily-ES "Precarga...": 32-row tiles)
 *   num_blocks   int32 [1]     number of used block_map entries
 * Every field must be non-null.
 */
typedef struct moe_routing {
  int32_t *topk_ids; float *topk_w;
  int32_t *counts, *offsets;
  int32_t *sorted_pair, *sorted_token, *pair_pos;
  int32_t *block_map, *num_blocks;
} moe_routing_t;

/* Number of block_map rows for T tokens: ceil(T*k/32) + E. */
int32_t moe_max_blocks(int32_t T, int32_t E, int32_t k);

/*
 * Bytes of device workspace moe_layer_forward needs for T tokens of layer L
 * (routing scratch, the fp16 activation copy, the fp16 expert
 * intermediates, the fp16 expert outputs and room for the router's logits;
 * about 105 MB at T=2048, d=2048, f=512, E=256, k=8). Non-decreasing in T, so a workspace sized for
 * T serves every call of fewer tokens.
 * moe_prefill_chunked needs moe_workspace_bytes(chunk, L). Host-only: reads
 * the scalar fields of L. Returns 0 when the arguments are invalid.
 */
size_t moe_workspace_bytes(int32_t T, const moe_layer_t *L);

/*
 * Where a moe_layer_forward call of T tokens keeps its fp16 intermediates
 * inside the workspace, for tests and debugging (the values are those the
 * layer's numerics rest on: activations entering the matrix cores, the SwiGLU
 * output h and each expert's output o). Byte offsets from the workspace start;
 * -1 where the buffer does not exist. Host-only; MOE_EINVAL for T < 1, a null
 * out or an invalid layer. After a call on the prefill form completes on its
 * stream:
 *   x16   fp16 [T][d]      x rounded to fp16
 *   h     fp16 [T*k][f]    SwiGLU output per expert-sorted row (row p is
 *                          sorted pair p)
 *   h_sh  fp16 [T][f_sh]   the shared expert's SwiGLU output
 *   o     fp16 [T*k][d]    expert output per expert-sorted row
 *   o_sh  fp16 [T][d]      the shared expert's output
 * x16, h and h_sh store each run of 8 columns in the order 0,4,1,5,2,6,3,7;
 * o and o_sh are in natural order. decode_form is 1 when the call takes the
 * few-token form; then only
 *   dec_h fp16 [T][k+1][max(f, f_sh)]  h per (token, slot), slot k the shared
 *                          expert, 8-runs permuted as above
 * holds data (x16, h and o are not written).
 */
typedef struct moe_workspace_layout {
  int32_t decode_form;
  int64_t x16, h, h_sh, o, o_sh, dec_h;
} moe_workspace_layout_t;
int moe_workspace_layout(int32_t T, const moe_layer_t *L, moe_workspace_layout_t *out);

/* Bytes of device workspace moe_route needs for T tokens over E experts (the
 * per-64-token expert counts; 32 KiB at T=2048, E=256). Host-only; 0 on
 * invalid arguments. */
size_t moe_route_workspace_bytes(int32_t T, int32_t E);

/*
 * Router projection, the step before routing (Lily-EN "Three Workload
 * Shapes": a router scores every expert per token): logits[t][e] =
 * sum_k x[t][k] * w_r[e][k]. x bf16 [T][d] and w_r bf16 [E][d] (device, row
 * major, 16-byte aligned, caller-owned); logits fp32 [T][E] (device, written).
 * Products are exact in fp32 and accumulate in fp32 in a fixed order, so a
 * call is deterministic. Calls of up to 16 tokens use a second kernel form
 * (16 experts per workgroup, inputs split over eight waves) whose order
 * differs, so a token's logits may differ in the last bits between a call of
 * at most 16 tokens and a longer one; each is within the fp32 summation
 * bound of the exact value. Errors: MOE_EINVAL (null or unaligned pointer,
 * T < 0, d < 1, E < 1), MOE_EUNSUPPORTED (d not a multiple of 32, E >
 * MOE_MAX_EXPERTS, T > MOE_MAX_CALL_TOKENS). T == 0 enqueues nothing. One
 * kernel; allocates nothing.
 */
int moe_router_logits(const uint16_t *x, int32_t T, int32_t d, const uint16_t *w_r, int32_t E,
                      float *logits, hipStream_t stream);

/*
 * Router projection followed by the top-k (Lily-EN "Three Workload Shapes": a
 * router scores 256 experts and keeps 8): logits[t][e] = sum_k x[t][k] *
 * w_r[e][k] exactly as moe_router_logits computes them (written to logits,
 * fp32 [T][E], device), then topk_ids [T][k] and topk_w [T][k] exactly as
 * moe_route derives them from those logits. Two kernels on the stream. x bf16
 * [T][d], w_r bf16 [E][d] (16-byte aligned, d a multiple of 32).
 * Errors: MOE_EINVAL (null or unaligned pointer, T < 0, d < 1, k < 1, k > E),
 * MOE_EUNSUPPORTED (d % 32, E > MOE_MAX_EXPERTS, k > 64, T >
 * MOE_MAX_CALL_TOKENS). T == 0 enqueues nothing.
 */
int moe_router_topk(const uint16_t *x, int32_t T, int32_t d, const uint16_t *w_r, int32_t E, int32_t k,
                    float *logits, int32_t *topk_ids, float *topk_w, hipStream_t stream);

/*
 * The whole layer from the router weights instead of logits: the router
 * projection (x w_r^T, as moe_router_logits) writes the logits into the
 * workspace and the layer of moe_layer_forward runs on them, so the results
 * equal moe_layer_forward's on moe_router_logits' output bit for bit.
 * w_r bf16 [E][d], 16-byte aligned, d a multiple of 32. ws as
 * moe_workspace_bytes(T, L), which covers this call. Other arguments and
 * errors as moe_layer_forward.
 */
int moe_layer_forward_router(const moe_layer_t *L, const uint16_t *x, const uint16_t *w_r, int32_t T,
                             float *y, const moe_routing_t *routing, void *ws, size_t ws_bytes,
                             hipStream_t stream);

/*
 * Routing only. logits fp32 [T][E] (device). Fills every field of *out (the
 * struct itself is read on the host; its pointers are device pointers).
 * ws: device workspace of at least moe_route_workspace_bytes(T, E) bytes,
 * 256-byte aligned (its contents need not be initialised).
 * Errors: MOE_EINVAL (null, unaligned ws, T < 0, k < 1, k > E),
 * MOE_EUNSUPPORTED (E > 1024, k > 64, T > MOE_MAX_CALL_TOKENS),
 * MOE_EWORKSPACE (ws_bytes too small). T == 0 enqueues nothing. Launches
 * two kernels (top-k; expert counts, offsets, stable scatter and block map),
 * and above 32768 (token, slot) pairs a per-64-token count pass between
 * them.
 */
int moe_route(const float *logits, int32_t T, int32_t E, int32_t k,
              const moe_routing_t *out, void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * Grouped GEMM over uneven expert groups with on-chip int4 dequantisation
 * (Lily-ES "Precarga...": weights are rebuilt one tile at a time inside the
 * grouped GEMM and accumulated in FP32; Lily-EN "Prefill..." names the same
 * fusion). For every block (e, r0, n) of block_map[0 .. *num_blocks) and every
 * row p in [r0, r0+n):
 *     C[p][j] = sum_k A[row(p)][k] * W_e[j][k],   j < N, k < K,
 * with W_e[j][k] = s*q + b from Wq + e*N*(K/8), Ws/Wb + e*N*(K/64), and
 * row(p) = a_row[p] when a_row is non-null, else p.
 *   A         bf16 [*][lda], 16-byte aligned, lda % 8 == 0
 *   Wq        uint32 [G][N][K/8]; Ws, Wb bf16 [G][N][K/64]; 16-byte aligned
 *   block_map int32 [max_blocks][3] as produced by moe_route; num_blocks [1]
 *   C         fp32 [*][ldc]; rows not covered by a block are not written
 * N and K must be multiples of 64 (else MOE_EUNSUPPORTED, as is N * K / 8
 * reaching 2^31). The block map contract gives every block 1..32 rows, and
 * each block is one work unit of the kernel. Of a longer block (a caller's
 * own map) only the first 96 rows are computed; the C rows past them keep
 * their contents, as do those of a block of zero or fewer rows (nothing is
 * checked on the host: the map lives on the device).
 */
int moe_grouped_gemm_int4(const uint16_t *A, int32_t lda, const int32_t *a_row,
                          int32_t N, int32_t K,
                          const uint32_t *Wq, const uint16_t *Ws, const uint16_t *Wb,
                          const int32_t *block_map, const int32_t *num_blocks, int32_t max_blocks,
                          float *C, int32_t ldc, hipStream_t stream);

/*
 * The whole layer for T tokens:
 *     y[t] = sum_j topk_w[t][j] * FFN_(topk_ids[t][j])(x[t]) + FFN_shared(x[t])
 * x bf16 [T][d]; logits fp32 [T][E]; y fp32 [T][d], fully overwritten.
 * routing: optional (may be NULL); when given, it receives the routing
 * tensors of this call. ws: device workspace of at least
 * moe_workspace_bytes(T, L) bytes, 256-byte aligned. Never synchronises.
 * Prefill enqueues five kernels (top-k, counts/scan/scatter, gate-up, down,
 * combine; six above 32768 (token, slot) pairs, with a per-64-token count
 * pass). Calls of at most 8 tokens with d a multiple of
 * 512, f == 512 and f_sh in {0, 512} take the decode form instead: two
 * kernels (gate-up with the top-k repeated in each workgroup; down with
 * the combine), plus the routing kernels only when routing is requested
 * (Lily-EN "Decode: Minimize Bytes Moved Per Token": decode is bound by the
 * bytes of the touched experts). Either way the k weighted expert rows are
 * added in slot order and then the shared expert's row, in fp32, so y is
 * reproducible bit for bit. T == 0 enqueues nothing.
 * Errors: MOE_EINVAL (null or misaligned pointer, T < 0, k > E),
 * MOE_EUNSUPPORTED (E > 1024, k > 64, d/f/f_sh not multiples of 64,
 * T > MOE_MAX_CALL_TOKENS, or a layer so large that T * (k + 1) * max(f, f_sh),
 * T * d reach 2^31 or one expert's 2 * max(f, f_sh) * d / 8 code words 2^30),
 * MOE_EWORKSPACE, MOE_EHIP.
 */
int moe_layer_forward(const moe_layer_t *L, const uint16_t *x, const float *logits, int32_t T,
                      float *y, const moe_routing_t *routing,
                      void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * moe_layer_forward for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc. The same kernels and results as moe_layer_forward (bit for bit),
 * with the workspace taken from a static device array of
 * MOE_NOALLOC_SCRATCH_BYTES that each GPU the library runs on holds until
 * the process ends. The call allocates nothing (no hipMalloc, no hipFree);
 * its first call on a device looks up that device's array once.
 *   - stream must belong to the current device (else MOE_EINVAL); the
 *     current device's array is used.
 *   - T is limited by moe_workspace_bytes(T, L) <= MOE_NOALLOC_SCRATCH_BYTES
 *     (about 1300 tokens at d=2048, f=512, E=256, k=8); a larger call returns
 *     MOE_EWORKSPACE before anything is enqueued. Longer prompts go through
 *     moe_prefill_chunked with a caller workspace.
 *   - Every call on one GPU shares that GPU's array, which keeps the last
 *     call's contents; nothing in it needs to start at zero (each kernel
 *     writes what it reads before reading it). Calls that overlap on one GPU
 *     (streams not ordered against each other) race on the array: the caller
 *     must order them.
 * Other arguments and errors as moe_layer_forward (MOE_EHIP also when the
 * array's address cannot be obtained).
 */
#define MOE_NOALLOC_SCRATCH_BYTES (64u << 20)
int moe_layer_forward_noalloc(const moe_layer_t *L, const uint16_t *x, const float *logits, int32_t T,
                              float *y, const moe_routing_t *routing, hipStream_t stream);

/*
 * moe_layer_forward with a check of the fp16 range. The path keeps x, the
 * SwiGLU output h and each expert's output o in fp16 (the header's numerics
 * note); a value outside fp16's finite range (magnitude 65520 or more, or
 * NaN) becomes infinite or NaN there and reaches y. overflow: device pointer
 * to one uint32 that the caller has set (usually to 0); the call ORs into it
 *   MOE_OVERFLOW_X  an x value did not convert to a finite fp16
 *   MOE_OVERFLOW_H  an h value was out of range
 *   MOE_OVERFLOW_O  an expert output o was out of range (prefill form; the
 *                   few-token form keeps o in fp32 and never sets it)
 * and leaves it unchanged when every stored value is finite. overflow may be
 * NULL (then this is moe_layer_forward). Values of |x| below 2^-17 lose low
 * bits in fp16 (subnormal spacing 2^-24) without setting a bit: their
 * products are far below the other terms' rounding. Other arguments and
 * errors as moe_layer_forward.
 */
#define MOE_OVERFLOW_X 1u
#define MOE_OVERFLOW_H 2u
#define MOE_OVERFLOW_O 4u
int moe_layer_forward_checked(const moe_layer_t *L, const uint16_t *x, const float *logits, int32_t T,
                              float *y, const moe_routing_t *routing, void *ws, size_t ws_bytes,
                              hipStream_t stream, uint32_t *overflow);

/*
 * moe_layer_forward with stage timing, for measurement. The events are
 * attached to the kernel dispatches themselves (no marker packets between
 * kernels, so timing adds no idle time): events[0] at the start of the top-k
 * kernel, events[1] at its end, events[2] at the end of the count/scatter
 * kernels, events[3] at the end of the gate/up kernel and events[4] at the end
 * of the last kernel (down + combine). In the few-token form without routing
 * outputs there are no routing kernels: events[0] and events[1] are recorded
 * as markers and events[2] is the start of the gate/up kernel. events: host
 * array of 5 caller-created hipEvent_t handles; a null entry leaves that
 * point unrecorded (fewer events, less timing overhead). Requires T >= 1;
 * otherwise as moe_layer_forward.
 */
int moe_layer_forward_timed(const moe_layer_t *L, const uint16_t *x, const float *logits,
                            int32_t T, float *y, const moe_routing_t *routing,
                            void *ws, size_t ws_bytes, hipStream_t stream, hipEvent_t *events);

/*
 * The layer with one of the pages' ablations, for measurement only (Lily-EN
 * "Prefill: Keep Weights Packed, Keep Routing on the GPU" and Lily-ES
 * "Precarga...": dequantisation fused into the GEMM, routing kept on the GPU
 * and 32-row rather than 16-row tiles are the changes they measure). Always
 * takes the prefill form (also for T <= 8); otherwise as moe_layer_forward,
 * with the same results (bit for bit: the GEMMs accumulate in the same
 * order and the unfused form expands weights with the same arithmetic).
 * ws_bytes must be at least moe_ablation_workspace_bytes(T, L, variant).
 *   MOE_ABLATION_NONE          the default prefill sequence
 *   MOE_ABLATION_TILE16        GEMM work units of at most 16 rows (instead of
 *                              96), so each rebuilt weight feeds 16 rows
 *   MOE_ABLATION_HOST_ROUTING  after the top-k kernel, the expert ids are
 *                              copied to the host, which builds counts,
 *                              offsets, scatter, block map and work list and
 *                              copies them back: synchronises the stream
 *                              twice and allocates host memory
 *   MOE_ABLATION_UNFUSED       every expert's weights (routed and shared) are
 *                              first expanded to fp16 in the workspace, one
 *                              projection at a time, and the grouped GEMMs
 *                              read the expanded weights (no on-chip rebuild)
 * Errors: as moe_layer_forward; MOE_EINVAL for an unknown variant.
 */
#define MOE_ABLATION_NONE 0
#define MOE_ABLATION_TILE16 1
#define MOE_ABLATION_HOST_ROUTING 2
#define MOE_ABLATION_UNFUSED 3
/* Workspace bytes for moe_layer_forward_ablation: moe_workspace_bytes(T, L)
 * plus, for MOE_ABLATION_UNFUSED, an fp16 buffer for the larger projection's
 * expanded weights (2 x max(E*2f*d + 2 f_sh*d, E*d*f + d*f_sh) bytes). 0 for
 * an invalid layer, T or variant. Host only. */
size_t moe_ablation_workspace_bytes(int32_t T, const moe_layer_t *L, int32_t variant);
int moe_layer_forward_ablation(const moe_layer_t *L, const uint16_t *x, const float *logits, int32_t T,
                               float *y, const moe_routing_t *routing, void *ws, size_t ws_bytes,
                               hipStream_t stream, int32_t variant);

/*
 * Bounded-chunk prefill for long prompts (Lily-ES "Precarga...", Lily-HE
 * prefill section: long prompts run in bounded chunks so temporary
 * activations do not compete with weights for memory). Runs
 * moe_layer_forward on consecutive chunks of at most `chunk` tokens, in order,
 * on one stream, reusing one workspace of moe_workspace_bytes(chunk, L)
 * bytes. Tokens are independent, so y equals the unchunked result; routing
 * tensors are per chunk and not returned.
 */
int moe_prefill_chunked(const moe_layer_t *L, const uint16_t *x, const float *logits, int32_t T,
                        int32_t chunk, float *y, void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * A layer call captured once into a HIP graph and launched many times
 * (Lily-EN "Decode: Minimize Bytes Moved Per Token": a recorded pass whose
 * real dependencies let independent kernels overlap). The graph is bound to
 * the given x, logits, y and workspace: each launch recomputes y from their
 * current contents, with results equal bit for bit to moe_layer_forward's.
 * flags:
 *   MOE_GRAPH_CONCURRENT  prefill form with a shared expert: its gate/up
 *                         (reading bf16 x directly) and down run on a
 *                         branch beside the routing kernels and the routed
 *                         GEMMs, joined before the combine; items of
 *                         shared_unit_rows rows (16..96, multiple of 16; 0
 *                         means 96). Without the flag the capture is the
 *                         one-stream sequence of moe_layer_forward.
 * stream: a non-default stream to capture on (the capture is thread-local);
 * nothing is executed while capturing. The graph holds a side stream and two
 * events (allocated here, released by moe_layer_graph_destroy). Calls that
 * launch the same graph, or share its workspace, must be ordered.
 * Errors: MOE_EINVAL (as moe_layer_forward, T < 1, a null stream or out,
 * unknown flags, bad shared_unit_rows), MOE_EUNSUPPORTED, MOE_EWORKSPACE,
 * MOE_EHIP (stream, event or graph creation failed).
 */
#define MOE_GRAPH_CONCURRENT 1
typedef struct moe_layer_graph moe_layer_graph_t;
int moe_layer_graph_create(const moe_layer_t *L, const uint16_t *x, const float *logits, int32_t T, float *y,
                           void *ws, size_t ws_bytes, int32_t flags, int32_t shared_unit_rows,
                           hipStream_t stream, moe_layer_graph_t **graph);
/* Enqueue one run of the captured layer on stream. */
int moe_layer_graph_launch(moe_layer_graph_t *graph, hipStream_t stream);
/* Release the graph and what it holds (after its launches have completed). */
int moe_layer_graph_destroy(moe_layer_graph_t *graph);

/* Static description of a status code. Never NULL. */
const char *moe_status_string(int status);

#ifdef __cplusplus
}
#endif
#endif /* MOE_INT4_H */
