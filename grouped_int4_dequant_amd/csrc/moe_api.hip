// C ABI of the MoE layer library: argument validation, workspace carving and
// the launch sequence. Every check runs on the host before anything is
// enqueued; nothing here reads device memory or synchronises.
//
// Pages cited (titles as published):
//   Lily-EN  "Perplexity Open Sources Lily: A Rust + Metal Inference Engine
//            for Qwen3.6-35B-A3B on Apple Silicon" (insight.aitobox.com)
//   Lily-ES  "Perplexity open sources Lily: un motor de inferencia ... para
//            Qwen3.6-35B-A3B en Apple Silicon" (7minutos.es)

#include "moe_internal.h"
#include "prep_layout.h"

#include <algorithm>
#include <mutex>
#include <new>
#include <vector>

using namespace moe;

namespace {

constexpr size_t kAlign = 256;
constexpr int kMaxRouteTokens = MOE_MAX_CALL_TOKENS;
constexpr int kMaxTopK = 64;  // one selected expert per lane of the top-k wave
// Trailing units of the routed work lists that run as half-width items, so
// the last round of workgroups is made of short pieces.
#ifndef MOE_GEMM_NARROW_TAIL
#define MOE_GEMM_NARROW_TAIL 32
#endif
constexpr int kNarrowTail = MOE_GEMM_NARROW_TAIL;
// The down projection's items are short (K = f, four steps at f = 512), so
// its routed work list runs without a half-width tail: splitting the last
// round measured 2 % slower there.
#ifndef MOE_GEMM_NARROW_TAIL_DOWN
#define MOE_GEMM_NARROW_TAIL_DOWN 0
#endif
constexpr int kNarrowTailDown = MOE_GEMM_NARROW_TAIL_DOWN;

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// Bump allocator over the caller's workspace; with base == nullptr it only
// measures. `last` is the byte offset of the most recent buffer.
struct Carver {
  char *base;
  size_t off = 0;
  size_t last = 0;
  template <typename T>
  T *take(size_t count) {
    off = (size_t)round_up((int64_t)off, kAlign);
    last = off;
    T *p = base ? reinterpret_cast<T *>(base + off) : nullptr;
    off += count * sizeof(T);
    return p;
  }
};

constexpr int kMinUnitRows = 16;  // smallest work unit (the 16-row tile variant)

int64_t max_units_routed(int T, int k, int E, int unit_rows = kUnitRows) {
  return ceil_div((int64_t)T * k, unit_rows) + E;
}

// Layer forward variants: the default, and the pages' ablations (measurement
// only, through moe_layer_forward_ablation).
struct FwdOptions {
  int unit_rows = kUnitRows;  // rows per GEMM work unit at most
  int ntail = 0;              // routed units run as half-width items at the end
  bool host_routing = false;  // counts, offsets, scatter, block map and work list built on the host
  bool few_token_form = true; // calls of at most 8 tokens take the two-kernel decode form
  bool unfused = false;       // weights expanded to fp16 in the workspace, then read by the GEMMs
  // Concurrent form (graph capture): the shared expert's gate/up (from bf16
  // x) and down run on `side`, forked from the main stream before routing
  // and joined before the combine; `shared_unit_rows` rows per item there.
  hipStream_t side = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
  int shared_unit_rows = kUnitRows;
};

// Unfused ablation: fp16 buffer for one projection's expanded weights (all
// routed experts, then the shared expert), reused by gate/up and down.
size_t expand_bytes(const moe_layer_t *L) {
  const int64_t gu = (int64_t)L->E * 2 * L->f * L->d + (int64_t)2 * L->f_sh * L->d;
  const int64_t dn = (int64_t)L->E * L->d * L->f + (int64_t)L->d * L->f_sh;
  return (size_t)round_up(2 * std::max(gu, dn), kAlign);
}

int check_layer(const moe_layer_t *L) {
  if (!L) return MOE_EINVAL;
  if (L->d <= 0 || L->f <= 0 || L->E <= 0 || L->k <= 0 || L->f_sh < 0) return MOE_EINVAL;
  if (L->k > L->E) return MOE_EINVAL;
  if (L->k > kMaxTopK) return MOE_EUNSUPPORTED;
  if (L->E > MOE_MAX_EXPERTS) return MOE_EUNSUPPORTED;
  if (L->d % 64 || L->f % 64 || L->f_sh % 64) return MOE_EUNSUPPORTED;
  const void *req[] = {L->gu_q, L->gu_s, L->gu_b, L->dn_q, L->dn_s, L->dn_b};
  for (const void *p : req)
    if (!p || !aligned16(p)) return MOE_EINVAL;
  if (L->f_sh > 0) {
    const void *sh[] = {L->sh_gu_q, L->sh_gu_s, L->sh_gu_b, L->sh_dn_q, L->sh_dn_s, L->sh_dn_b};
    for (const void *p : sh)
      if (!p || !aligned16(p)) return MOE_EINVAL;
  }
  if (L->prep && ((uintptr_t)L->prep % kAlign)) return MOE_EINVAL;
  return MOE_OK;
}

// Where each projection's prepared codes and table sit in a prepared copy
// (byte offsets from its start; prep_layout.h gives the order inside).
struct PrepLayout {
  int64_t gu_q, gu_t, dn_q, dn_t, sh_gu_q, sh_gu_t, sh_dn_q, sh_dn_t, total;
};

bool prep_supported(const moe_layer_t *L) { return L->d % 128 == 0 && L->f % 128 == 0 && L->f_sh % 128 == 0; }

PrepLayout prep_layout(const moe_layer_t *L) {
  const int d = L->d, f = L->f, fs = L->f_sh;
  const int64_t E = L->E;
  PrepLayout p{};
  int64_t at = kPrepHeader;  // the flags come first
  auto take = [&](int64_t bytes) {
    const int64_t o = at;
    at += round_up(bytes, kAlign);
    return o;
  };
  p.gu_q = take(E * prep_code_bytes(2 * f, d, true));
  p.gu_t = take(E * prep_table_dwords(2 * f, d, true) * 4);
  p.dn_q = take(E * prep_code_bytes(d, f, false));
  p.dn_t = take(E * prep_table_dwords(d, f, false) * 4);
  p.sh_gu_q = p.sh_gu_t = p.sh_dn_q = p.sh_dn_t = -1;
  if (fs > 0) {
    p.sh_gu_q = take(prep_code_bytes(2 * fs, d, true));
    p.sh_gu_t = take(prep_table_dwords(2 * fs, d, true) * 4);
    p.sh_dn_q = take(prep_code_bytes(d, fs, false));
    p.sh_dn_t = take(prep_table_dwords(d, fs, false) * 4);
  }
  p.total = at;
  return p;
}

// Point a GEMM problem at the prepared copy of one projection (expert
// stride from the layout), when the layer has one.
void use_prep(GemmProblem &p, const moe_layer_t *L, int flag, int64_t q_ofs, int64_t t_ofs, int N, int K,
              bool swiglu, bool per_expert) {
  if (!L->prep || !prep_supported(L)) return;
  const uint8_t *base = static_cast<const uint8_t *>(L->prep);
  p.Pflag = reinterpret_cast<const uint32_t *>(base) + flag;
  p.Pq = base + q_ofs;
  p.Pt = reinterpret_cast<const uint32_t *>(base + t_ofs);
  p.pq_estride = per_expert ? prep_code_bytes(N, K, swiglu) : 0;
  p.pt_estride = per_expert ? prep_table_dwords(N, K, swiglu) : 0;
}

int check_routing(const moe_routing_t *r) {
  if (!r) return MOE_EINVAL;
  const void *req[] = {r->topk_ids, r->topk_w, r->counts, r->offsets, r->sorted_pair,
                       r->sorted_token, r->pair_pos, r->block_map, r->num_blocks};
  for (const void *p : req)
    if (!p) return MOE_EINVAL;
  return MOE_OK;
}

struct Workspace {
  moe_routing_t rt;
  int32_t *units, *num_units;
  int32_t *chunk_counts;
  uint16_t *x16, *h, *h_sh, *o, *o_sh;
  uint16_t *dec_h;  // decode-shape calls only
  float *logits;    // [T][E]: router logits of moe_layer_forward_router when they go through memory
  uint8_t *ids8;    // [T*k]: the top-k ids as bytes, for the scatter's count (E <= 256)
};

// Layout of the layer workspace for T tokens (base == nullptr: size only).
// lay (nullable) receives the byte offsets of the fp16 intermediates.
size_t carve_layer(int T, const moe_layer_t *L, char *base, Workspace *w,
                   moe_workspace_layout_t *lay = nullptr) {
  Carver c{base};
  moe_workspace_layout_t ofs{};
  ofs.decode_form = decode_supported(T, L) ? 1 : 0;
  ofs.x16 = ofs.h = ofs.h_sh = ofs.o = ofs.o_sh = ofs.dec_h = -1;
  const int E = L->E, k = L->k;
  const int64_t tk = (int64_t)T * k;
  Workspace o;
  o.rt.topk_ids = c.take<int32_t>(tk);
  o.rt.topk_w = c.take<float>(tk);
  o.rt.counts = c.take<int32_t>(E);
  o.rt.offsets = c.take<int32_t>(E + 1);
  o.rt.sorted_pair = c.take<int32_t>(tk);
  o.rt.sorted_token = c.take<int32_t>(tk);
  o.rt.pair_pos = c.take<int32_t>(tk);
  o.rt.block_map = c.take<int32_t>(3 * (size_t)moe_max_blocks(T, E, k));
  o.rt.num_blocks = c.take<int32_t>(1);
  o.units = c.take<int32_t>(3 * (size_t)max_units_routed(T, k, E, kMinUnitRows));  // any unit size
  o.num_units = c.take<int32_t>(1);
  o.chunk_counts = c.take<int32_t>((size_t)ceil_div(T, kSubChunk) * E);
  o.logits = c.take<float>((size_t)T * E);
  o.x16 = c.take<uint16_t>((size_t)T * L->d);
  ofs.x16 = (int64_t)c.last;
  // The shared expert's rows follow the routed rows in h and o when their
  // widths match, so one grouped GEMM can cover both.
  const bool joint_h = L->f_sh == L->f;
  o.h = c.take<uint16_t>((size_t)tk * L->f + (joint_h ? (size_t)T * L->f_sh : 0));
  ofs.h = (int64_t)c.last;
  if (joint_h) {
    o.h_sh = base ? o.h + (size_t)tk * L->f : nullptr;
    ofs.h_sh = L->f_sh > 0 ? ofs.h + 2 * tk * L->f : -1;
  } else {
    o.h_sh = c.take<uint16_t>((size_t)T * L->f_sh);
    ofs.h_sh = L->f_sh > 0 ? (int64_t)c.last : -1;
  }
  o.o = c.take<uint16_t>((size_t)(tk + (L->f_sh > 0 ? T : 0)) * L->d);
  ofs.o = (int64_t)c.last;
  o.o_sh = (L->f_sh > 0 && base) ? o.o + (size_t)tk * L->d : nullptr;
  ofs.o_sh = L->f_sh > 0 ? ofs.o + 2 * tk * L->d : -1;
  const int fmax = L->f > L->f_sh ? L->f : L->f_sh;
  if (ofs.decode_form) {
    o.dec_h = c.take<uint16_t>((size_t)T * (L->k + 1) * fmax);
    ofs.dec_h = (int64_t)c.last;
  } else {
    o.dec_h = nullptr;
  }
  o.ids8 = c.take<uint8_t>((size_t)round_up(tk, 16));
  if (w) *w = o;
  if (lay) *lay = ofs;
  return (size_t)round_up((int64_t)c.off, kAlign);
}

// Workspace bytes for T tokens, made non-decreasing in T: the few-token form
// carves a buffer the prefill form does not, so a workspace sized for T also
// covers every smaller call (a chunked call's shorter last chunk included).
size_t layer_ws_bytes(int T, const moe_layer_t *L) {
  return std::max(carve_layer(T, L, nullptr, nullptr), carve_layer(std::min(T, kDecodeMaxT), L, nullptr, nullptr));
}

int hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_EHIP; }

int enqueue_scan(int T, int E, int k, const moe_routing_t &rt, int32_t *chunk_counts, int32_t *units,
                 int32_t *num_units, hipStream_t s, hipEvent_t *ev, int unit_rows, const uint8_t *ids8 = nullptr);

// The byte copy of the ids is used when every id fits a byte and the pairs
// come in whole 16-byte groups.
bool use_ids8(int T, int E, int k, const uint8_t *ids8) {
  return ids8 != nullptr && E <= 256 && ((int64_t)T * k) % 16 == 0;
}

int record(hipEvent_t *ev, int i, hipStream_t s);

int enqueue_route(const float *logits, int T, int E, int k, const moe_routing_t &rt,
                  int32_t *chunk_counts, int32_t *units, int32_t *num_units, const uint16_t *x,
                  uint16_t *x16, int d, hipStream_t s, hipEvent_t *ev = nullptr, int unit_rows = kUnitRows,
                  uint32_t *overflow = nullptr, uint8_t *ids8 = nullptr) {
  hipError_t err;
  TopkArgs ta{};
  ta.overflow = overflow;
  ta.logits = logits;
  ta.T = T;
  ta.E = E;
  ta.k = k;
  ta.topk_ids = rt.topk_ids;
  ta.topk_w = rt.topk_w;
  ta.x = x;
  ta.x16 = x16;
  ta.d = d;
  ta.ids8 = use_ids8(T, E, k, ids8) ? ids8 : nullptr;
  err = launch_topk(ta, s, ev ? ev[0] : nullptr, ev ? ev[1] : nullptr);
  if (err != hipSuccess) return MOE_EHIP;
  return enqueue_scan(T, E, k, rt, chunk_counts, units, num_units, s, ev, unit_rows, ta.ids8);
}

// Histogram, scan, stable scatter, block map and work list from rt.topk_ids.
int enqueue_scan(int T, int E, int k, const moe_routing_t &rt, int32_t *chunk_counts, int32_t *units,
                 int32_t *num_units, hipStream_t s, hipEvent_t *ev, int unit_rows, const uint8_t *ids8) {
  ScanArgs sa{};
  sa.ids8 = use_ids8(T, E, k, ids8) ? ids8 : nullptr;
  sa.T = T;
  sa.E = E;
  sa.k = k;
  sa.topk_ids = rt.topk_ids;
  sa.counts = rt.counts;
  sa.offsets = rt.offsets;
  sa.sorted_pair = rt.sorted_pair;
  sa.sorted_token = rt.sorted_token;
  sa.pair_pos = rt.pair_pos;
  sa.block_map = rt.block_map;
  sa.num_blocks = rt.num_blocks;
  sa.max_blocks = moe_max_blocks(T, E, k);
  sa.units = units;
  sa.chunk_counts = chunk_counts;
  sa.num_units = num_units;
  sa.max_units = units ? (int)max_units_routed(T, k, E, unit_rows) : 0;
  sa.unit_rows = unit_rows;
  return hip_status(launch_scan(sa, s, ev ? ev[2] : nullptr));
}

// Workgroups of one grouped problem: units rounded up to a multiple of 8 (one
// unit per XCD per round) times the N-slices.
int problem_wgs(int64_t max_units, int nslices) { return (int)(round_up(max_units, 8) * nslices); }

int record(hipEvent_t *ev, int i, hipStream_t s) {
  return ev && ev[i] ? hip_status(hipEventRecord(ev[i], s)) : MOE_OK;
}

int enqueue_combine(int T, int d, int k, const uint16_t *o, const uint16_t *o_sh, const moe_routing_t &rt,
                    float *y, hipStream_t s, hipEvent_t *ev) {
  CombineArgs ca{};
  ca.T = T;
  ca.d = d;
  ca.k = k;
  ca.o = o;
  ca.o_sh = o_sh;
  ca.pair_pos = rt.pair_pos;
  ca.topk_w = rt.topk_w;
  ca.y = y;
  return hip_status(launch_combine(ca, s, ev ? ev[4] : nullptr));
}

// The pages' "before" configuration: after the top-k kernel, the selected
// expert ids come back to the host, which builds counts, offsets, the stable
// scatter, the 32-row block map and the GEMM work list (the same results as
// the scan/scatter kernels), and sends them back. Synchronises the stream
// twice. Measurement only.
int host_route(int T, int E, int k, int unit_rows, const moe_routing_t &rt, int32_t *units,
               int32_t *num_units, hipStream_t s) {
  const int64_t tk = (int64_t)T * k;
  std::vector<int32_t> ids(tk);
  if (hipMemcpyAsync(ids.data(), rt.topk_ids, tk * sizeof(int32_t), hipMemcpyDeviceToHost, s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    return MOE_EHIP;
  std::vector<int32_t> cnt(E, 0), off(E + 1, 0), cur(E, 0), sorted_pair(tk), sorted_token(tk), pair_pos(tk);
  for (int64_t i = 0; i < tk; ++i) ++cnt[ids[i]];
  for (int e = 0; e < E; ++e) off[e + 1] = off[e] + cnt[e];
  for (int64_t i = 0; i < tk; ++i) {  // ascending pair index: stable
    const int e = ids[i];
    const int pos = off[e] + cur[e]++;
    sorted_pair[pos] = (int32_t)i;
    sorted_token[pos] = (int32_t)(i / k);
    pair_pos[i] = pos;
  }
  const int max_blocks = moe_max_blocks(T, E, k);
  std::vector<int32_t> bmap(3 * (size_t)max_blocks);
  int nb = 0;
  for (int e = 0; e < E; ++e)
    for (int b = 0; b * MOE_BLOCK_ROWS < cnt[e]; ++b, ++nb) {
      bmap[3 * nb] = e;
      bmap[3 * nb + 1] = off[e] + b * MOE_BLOCK_ROWS;
      bmap[3 * nb + 2] = std::min(MOE_BLOCK_ROWS, cnt[e] - b * MOE_BLOCK_ROWS);
    }
  for (int i = nb; i < max_blocks; ++i) {
    bmap[3 * i] = -1;
    bmap[3 * i + 1] = 0;
    bmap[3 * i + 2] = 0;
  }
  // work list: the same units as the scatter kernel, largest size class first
  std::vector<int32_t> ulist;
  const int classes = kUnitRows / 16;
  for (int c = classes; c >= 1; --c)
    for (int e = 0; e < E; ++e) {
      const int tot = cnt[e], nu = (tot + unit_rows - 1) / unit_rows;
      for (int u = 0; u < nu; ++u) {
        const int b0 = (int)((int64_t)u * tot / nu), b1 = (int)((int64_t)(u + 1) * tot / nu);
        if ((b1 - b0 + 15) / 16 != c) continue;
        ulist.push_back(e);
        ulist.push_back(off[e] + b0);
        ulist.push_back(b1 - b0);
      }
    }
  const int32_t nunits = (int32_t)(ulist.size() / 3);
  struct Copy { void *dst; const void *src; size_t bytes; };
  const Copy copies[] = {
      {rt.counts, cnt.data(), E * sizeof(int32_t)},
      {rt.offsets, off.data(), (E + 1) * sizeof(int32_t)},
      {rt.sorted_pair, sorted_pair.data(), tk * sizeof(int32_t)},
      {rt.sorted_token, sorted_token.data(), tk * sizeof(int32_t)},
      {rt.pair_pos, pair_pos.data(), tk * sizeof(int32_t)},
      {rt.block_map, bmap.data(), bmap.size() * sizeof(int32_t)},
      {rt.num_blocks, &nb, sizeof(int32_t)},
      {units, ulist.data(), ulist.size() * sizeof(int32_t)},
      {num_units, &nunits, sizeof(int32_t)},
  };
  for (const Copy &c : copies)
    if (c.bytes && hipMemcpyAsync(c.dst, c.src, c.bytes, hipMemcpyHostToDevice, s) != hipSuccess) return MOE_EHIP;
  return hip_status(hipStreamSynchronize(s));  // the host vectors must outlive the copies
}

int forward_one(const moe_layer_t *L, const uint16_t *x, const float *logits, int T, float *y,
                const moe_routing_t *routing, void *ws, size_t ws_bytes, hipStream_t s,
                hipEvent_t *ev = nullptr, const FwdOptions &opt_in = FwdOptions{kUnitRows, kNarrowTail, false, true},
                uint32_t *overflow = nullptr, const uint16_t *w_r = nullptr) {
  // Calls whose routed experts hold about 20 rows or fewer on average (short
  // prompts) run the small-unit GEMM build: units of at most 32 rows, three
  // workgroups per CU (T=512 of the Qwen-shaped layer 116 against 121 us;
  // at 64 rows per expert, units that small cost a third more)
  FwdOptions opt = opt_in;
  const bool small_units = opt.unit_rows == kUnitRows && !opt.unfused && !opt.host_routing &&
                           opt.side == nullptr && (int64_t)T * L->k <= 20 * (int64_t)L->E;
  if (small_units) opt.unit_rows = kUnitRowsSmall;
  auto gemm = small_units ? launch_gemm_small : launch_gemm;
  const size_t need = layer_ws_bytes(T, L);
  if (ws_bytes < need + (opt.unfused ? expand_bytes(L) : 0)) return MOE_EWORKSPACE;
  Workspace w;
  carve_layer(T, L, static_cast<char *>(ws), &w);
  uint16_t *wx = opt.unfused ? reinterpret_cast<uint16_t *>(static_cast<char *>(ws) + need) : nullptr;
  const moe_routing_t &rt = routing ? *routing : w.rt;
  const int d = L->d, f = L->f, E = L->E, k = L->k, fs = L->f_sh;
  // The GEMM addresses the layer's fp16 activation buffers and one expert's
  // codes with 32-bit byte offsets.
  const int64_t wmax = std::max<int64_t>(f, fs);
  if ((int64_t)T * (k + 1) * wmax >= (1LL << 31) || (int64_t)T * d >= (1LL << 31) ||
      2 * wmax * d / 8 >= (1LL << 30))
    return MOE_EUNSUPPORTED;

  int st = MOE_OK;
  const bool decode_form = opt.few_token_form && decode_supported(T, L);
  if (w_r) {
    // the router's logits go through the workspace; the layer then runs as usual
    RouterArgs ra{};
    ra.x = x; ra.w = w_r; ra.T = T; ra.d = d; ra.E = E; ra.logits = w.logits;
    st = hip_status(launch_router(ra, s));
    if (st != MOE_OK) return st;
    logits = w.logits;
  }
  if (decode_form) {
    // A few tokens: gate/up (routing repeated inside) and down + combine.
    // Routing tensors are produced by the routing kernels only when asked for.
    if (routing) {
      st = enqueue_route(logits, T, E, k, rt, w.chunk_counts, w.units, w.num_units, nullptr, nullptr, d, s, ev);
    } else {
      for (int i = 0; i < 2 && st == MOE_OK; ++i) st = record(ev, i, s);  // no routing kernels
    }
    if (st != MOE_OK) return st;
    DecodeArgs a{};
    a.logits = logits; a.x = x;
    a.T = T; a.d = d; a.f = f; a.f_sh = fs; a.E = E; a.k = k; a.fmax = f > fs ? f : fs;
    a.gu_q = L->gu_q; a.gu_s = L->gu_s; a.gu_b = L->gu_b;
    a.gu_qs = (int64_t)2 * f * (d / 8); a.gu_ss = (int64_t)2 * f * (d / 64);
    a.dn_q = L->dn_q; a.dn_s = L->dn_s; a.dn_b = L->dn_b;
    a.dn_qs = (int64_t)d * (f / 8); a.dn_ss = (int64_t)d * (f / 64);
    a.sh_gu_q = L->sh_gu_q; a.sh_gu_s = L->sh_gu_s; a.sh_gu_b = L->sh_gu_b;
    a.sh_dn_q = L->sh_dn_q; a.sh_dn_s = L->sh_dn_s; a.sh_dn_b = L->sh_dn_b;
    a.ids = w.rt.topk_ids; a.gates = w.rt.topk_w;  // the workspace's own routing buffers
    a.h = w.dec_h; a.y = y;
    a.overflow = overflow;
    hipEvent_t gu_start = (ev && !routing) ? ev[2] : nullptr;
    return hip_status(launch_decode(a, s, gu_start, ev ? ev[3] : nullptr, ev ? ev[4] : nullptr));
  }

  // concurrent form: the shared expert on the side stream, beside the routing
  const PrepLayout pl = prep_layout(L);
  const bool split = opt.side != nullptr && fs > 0 && !opt.unfused;
  if (split) {
    if (hipEventRecord(opt.fork, s) != hipSuccess || hipStreamWaitEvent(opt.side, opt.fork, 0) != hipSuccess)
      return MOE_EHIP;
    GemmArgs gs{};
    GemmProblem &p = gs.prob[0];
    p.A = x; p.lda = d; p.a_row = nullptr;  // bf16 x, converted to fp16 while staged
    p.Wq = L->sh_gu_q; p.Ws = L->sh_gu_s; p.Wb = L->sh_gu_b;
    p.N = 2 * fs; p.K = d;
    p.units = nullptr; p.num_units = nullptr; p.implicit_rows = T; p.unit_rows = opt.shared_unit_rows;
    p.nslices = (int)ceil_div(fs, kGemmCols / 2);
    p.H = w.h_sh; p.ldh = fs;
    p.overflow = overflow;
    gs.nprob = 1;
    gs.total_wg = problem_wgs(ceil_div(T, opt.shared_unit_rows), p.nslices);
    st = hip_status(launch_gemm(gs, kSwiGLU, false, opt.side));
    if (st != MOE_OK) return st;
    GemmArgs gd{};
    GemmProblem &q = gd.prob[0];
    q.A = w.h_sh; q.lda = fs; q.a_row = nullptr;
    q.Wq = L->sh_dn_q; q.Ws = L->sh_dn_s; q.Wb = L->sh_dn_b;
    use_prep(q, L, kFlagShDn, pl.sh_dn_q, pl.sh_dn_t, d, fs, false, false);
    q.N = d; q.K = fs;
    q.units = nullptr; q.num_units = nullptr; q.implicit_rows = T; q.unit_rows = opt.shared_unit_rows;
    q.nslices = (int)ceil_div(d, kGemmCols);
    q.H = w.o_sh; q.ldh = d;
    q.overflow = overflow;
    gd.nprob = 1;
    gd.total_wg = problem_wgs(ceil_div(T, opt.shared_unit_rows), q.nslices);
    st = hip_status(launch_gemm(gd, kStoreH, true, opt.side));
    if (st != MOE_OK) return st;
    if (hipEventRecord(opt.join, opt.side) != hipSuccess) return MOE_EHIP;
  }

  if (opt.host_routing) {
    TopkArgs ta{};
    ta.logits = logits; ta.T = T; ta.E = E; ta.k = k;
    ta.topk_ids = rt.topk_ids; ta.topk_w = rt.topk_w;
    ta.x = x; ta.x16 = w.x16; ta.d = d;
    ta.overflow = overflow;
    st = hip_status(launch_topk(ta, s));
    if (st == MOE_OK) st = host_route(T, E, k, opt.unit_rows, rt, w.units, w.num_units, s);
  } else {
    st = enqueue_route(logits, T, E, k, rt, w.chunk_counts, w.units, w.num_units, x, w.x16, d, s, ev, opt.unit_rows,
                       overflow, w.ids8);
  }
  if (st != MOE_OK) return st;

  // gate/up projection + SwiGLU: shared expert (implicit units), routed experts
  // (unfused ablation: weights first expanded into the workspace, items of
  // 128 columns of h)
  const int hcols = opt.unfused ? kGemmCols / 4 : kGemmCols / 2;
  if (opt.unfused) {
    st = hip_status(launch_expand(L->gu_q, L->gu_s, L->gu_b, (int64_t)E * 2 * f, d, wx, s));
    if (st == MOE_OK && fs > 0)
      st = hip_status(launch_expand(L->sh_gu_q, L->sh_gu_s, L->sh_gu_b, 2 * fs, d, wx + (int64_t)E * 2 * f * d, s));
    if (st != MOE_OK) return st;
  }
  GemmArgs g1{};
  int nwg = 0, np = 0;
  if (fs > 0 && !split) {
    GemmProblem &p = g1.prob[np++];
    p.A = w.x16; p.lda = d; p.a_row = nullptr;
    p.Wq = L->sh_gu_q; p.Ws = L->sh_gu_s; p.Wb = L->sh_gu_b;
    p.wq_estride = 0; p.ws_estride = 0;
    p.N = 2 * fs; p.K = d;
    p.Wx = wx ? wx + (int64_t)E * 2 * f * d : nullptr; p.wx_estride = 0;
    if (!opt.unfused) use_prep(p, L, kFlagShGu, pl.sh_gu_q, pl.sh_gu_t, 2 * fs, d, true, false);
    p.units = nullptr; p.num_units = nullptr; p.implicit_rows = T; p.unit_rows = opt.unit_rows;
    p.nslices = (int)ceil_div(fs, hcols);
    p.wg_begin = nwg;
    p.H = w.h_sh; p.ldh = fs;
    p.overflow = overflow;
    nwg += problem_wgs(ceil_div(T, opt.unit_rows), p.nslices);
  }
  {
    GemmProblem &p = g1.prob[np++];
    p.A = w.x16; p.lda = d; p.a_row = rt.sorted_token;
    p.Wq = L->gu_q; p.Ws = L->gu_s; p.Wb = L->gu_b;
    p.wq_estride = (int64_t)2 * f * (d / 8); p.ws_estride = (int64_t)2 * f * (d / 64);
    p.N = 2 * f; p.K = d;
    p.Wx = wx; p.wx_estride = (int64_t)2 * f * d;
    if (!opt.unfused) use_prep(p, L, kFlagGu, pl.gu_q, pl.gu_t, 2 * f, d, true, true);
    p.units = w.units; p.num_units = w.num_units; p.implicit_rows = 0;
    p.nslices = (int)ceil_div(f, hcols);
    p.ntail = opt.ntail;
    p.wg_begin = nwg;
    p.H = w.h; p.ldh = f;
    p.overflow = overflow;
    // full-width items, plus up to ntail + 14 units' extra half-width items
    nwg += problem_wgs(max_units_routed(T, k, E, opt.unit_rows) + 2 * (opt.ntail + 16), p.nslices);
  }
  g1.nprob = np;
  g1.total_wg = nwg;
  st = hip_status(gemm(g1, kSwiGLU, true, s, nullptr, ev ? ev[3] : nullptr, opt.unfused));
  if (st != MOE_OK) return st;
  const int ocols = opt.unfused ? kGemmCols / 2 : kGemmCols;
  if (opt.unfused) {
    st = hip_status(launch_expand(L->dn_q, L->dn_s, L->dn_b, (int64_t)E * d, f, wx, s));
    if (st == MOE_OK && fs > 0)
      st = hip_status(launch_expand(L->sh_dn_q, L->sh_dn_s, L->sh_dn_b, d, fs, wx + (int64_t)E * d * f, s));
    if (st != MOE_OK) return st;
  }

  // down projection into fp16 expert outputs, then the weighted combine
  GemmArgs g2{};
  nwg = 0;
  np = 0;
  if (fs > 0 && !split) {
    GemmProblem &p = g2.prob[np++];
    p.A = w.h_sh; p.lda = fs; p.a_row = nullptr;
    p.Wq = L->sh_dn_q; p.Ws = L->sh_dn_s; p.Wb = L->sh_dn_b;
    p.wq_estride = 0; p.ws_estride = 0;
    p.N = d; p.K = fs;
    p.Wx = wx ? wx + (int64_t)E * d * f : nullptr; p.wx_estride = 0;
    if (!opt.unfused) use_prep(p, L, kFlagShDn, pl.sh_dn_q, pl.sh_dn_t, d, fs, false, false);
    p.units = nullptr; p.num_units = nullptr; p.implicit_rows = T; p.unit_rows = opt.unit_rows;
    p.nslices = (int)ceil_div(d, ocols);
    p.wg_begin = nwg;
    p.H = w.o_sh; p.ldh = d;
    p.overflow = overflow;
    nwg += problem_wgs(ceil_div(T, opt.unit_rows), p.nslices);
  }
  {
    GemmProblem &p = g2.prob[np++];
    p.A = w.h; p.lda = f; p.a_row = nullptr;
    p.Wq = L->dn_q; p.Ws = L->dn_s; p.Wb = L->dn_b;
    p.wq_estride = (int64_t)d * (f / 8); p.ws_estride = (int64_t)d * (f / 64);
    p.N = d; p.K = f;
    p.Wx = wx; p.wx_estride = (int64_t)d * f;
    if (!opt.unfused) use_prep(p, L, kFlagDn, pl.dn_q, pl.dn_t, d, f, false, true);
    p.units = w.units; p.num_units = w.num_units; p.implicit_rows = 0;
    p.nslices = (int)ceil_div(d, ocols);
    p.ntail = opt.ntail > 0 ? kNarrowTailDown : 0;  // ablation forms: no tail
    p.wg_begin = nwg;
    p.H = w.o; p.ldh = d;
    p.overflow = overflow;
    // full-width items, plus (with a tail) up to ntail + 14 units' extra half-width items
    nwg += problem_wgs(max_units_routed(T, k, E, opt.unit_rows) + (p.ntail > 0 ? 2 * (p.ntail + 16) : 0), p.nslices);
  }
  g2.nprob = np;
  g2.total_wg = nwg;
  st = hip_status(gemm(g2, kStoreH, true, s, nullptr, nullptr, opt.unfused));
  if (st != MOE_OK) return st;
  if (split && hipStreamWaitEvent(s, opt.join, 0) != hipSuccess) return MOE_EHIP;

  return enqueue_combine(T, d, k, w.o, fs > 0 ? w.o_sh : nullptr, rt, y, s, ev);
}

}  // namespace

extern "C" {

int32_t moe_max_blocks(int32_t T, int32_t E, int32_t k) {
  if (T < 0 || E <= 0 || k <= 0) return 0;
  return (int32_t)(ceil_div((int64_t)T * k, MOE_BLOCK_ROWS) + E);
}

size_t moe_route_workspace_bytes(int32_t T, int32_t E) {
  if (T < 0 || E <= 0 || E > MOE_MAX_EXPERTS || T > kMaxRouteTokens) return 0;
  // per-sub-chunk expert counts
  return (size_t)round_up(std::max<int64_t>(ceil_div(T, kSubChunk), 1) * E * (int64_t)sizeof(int32_t), kAlign);
}

size_t moe_prepared_bytes(const moe_layer_t *L) {
  if (!L || L->d <= 0 || L->f <= 0 || L->E <= 0 || L->f_sh < 0 || L->E > MOE_MAX_EXPERTS) return 0;
  if (!prep_supported(L)) return 0;
  return (size_t)prep_layout(L).total;
}

int moe_prepare_weights(const moe_layer_t *L, void *dst, size_t dst_bytes, hipStream_t stream) {
  int st = check_layer(L);
  if (st != MOE_OK) return st;
  if (!dst || ((uintptr_t)dst % kAlign)) return MOE_EINVAL;
  if (!prep_supported(L)) return MOE_EUNSUPPORTED;
  const PrepLayout pl = prep_layout(L);
  if (dst_bytes < (size_t)pl.total) return MOE_EWORKSPACE;
  uint8_t *b = static_cast<uint8_t *>(dst);
  const int d = L->d, f = L->f, fs = L->f_sh, E = L->E;
  auto tab = [&](int64_t o) { return reinterpret_cast<uint32_t *>(b + o); };
  uint32_t *flags = reinterpret_cast<uint32_t *>(b);
  st = hip_status(launch_prepare(L->gu_q, L->gu_s, L->gu_b, E, 2 * f, d, true, b + pl.gu_q, tab(pl.gu_t),
                                 flags + kFlagGu, stream));
  if (st == MOE_OK)
    st = hip_status(launch_prepare(L->dn_q, L->dn_s, L->dn_b, E, d, f, false, b + pl.dn_q, tab(pl.dn_t),
                                   flags + kFlagDn, stream));
  if (st == MOE_OK && fs > 0)
    st = hip_status(launch_prepare(L->sh_gu_q, L->sh_gu_s, L->sh_gu_b, 1, 2 * fs, d, true, b + pl.sh_gu_q,
                                   tab(pl.sh_gu_t), flags + kFlagShGu, stream));
  if (st == MOE_OK && fs > 0)
    st = hip_status(launch_prepare(L->sh_dn_q, L->sh_dn_s, L->sh_dn_b, 1, d, fs, false, b + pl.sh_dn_q,
                                   tab(pl.sh_dn_t), flags + kFlagShDn, stream));
  if (st == MOE_OK && fs == 0) {  // no shared expert: its flags read 0
    st = hip_status(launch_prep_flag(flags + kFlagShGu, 0u, stream));
    if (st == MOE_OK) st = hip_status(launch_prep_flag(flags + kFlagShDn, 0u, stream));
  }
  return st;
}

size_t moe_workspace_bytes(int32_t T, const moe_layer_t *L) {
  if (!L || T < 0 || T > kMaxRouteTokens) return 0;
  if (L->d <= 0 || L->f <= 0 || L->E <= 0 || L->k <= 0 || L->k > L->E || L->f_sh < 0) return 0;
  if (L->E > MOE_MAX_EXPERTS || L->k > kMaxTopK || L->d % 64 || L->f % 64 || L->f_sh % 64) return 0;
  return layer_ws_bytes(T, L);
}

int moe_workspace_layout(int32_t T, const moe_layer_t *L, moe_workspace_layout_t *out) {
  if (!out || moe_workspace_bytes(T, L) == 0 || T < 1) return MOE_EINVAL;
  carve_layer(T, L, nullptr, nullptr, out);
  return MOE_OK;
}

size_t moe_ablation_workspace_bytes(int32_t T, const moe_layer_t *L, int32_t variant) {
  const size_t base = moe_workspace_bytes(T, L);
  if (base == 0 || variant < MOE_ABLATION_NONE || variant > MOE_ABLATION_UNFUSED) return 0;
  return base + (variant == MOE_ABLATION_UNFUSED ? expand_bytes(L) : 0);
}

int moe_router_logits(const uint16_t *x, int32_t T, int32_t d, const uint16_t *w_r, int32_t E,
                      float *logits, hipStream_t stream) {
  if (T < 0 || d < 1 || E < 1) return MOE_EINVAL;
  if (d % 32 || E > MOE_MAX_EXPERTS || T > kMaxRouteTokens) return MOE_EUNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!x || !w_r || !logits || !aligned16(x) || !aligned16(w_r) || !aligned16(logits)) return MOE_EINVAL;
  RouterArgs a{};
  a.x = x; a.w = w_r; a.T = T; a.d = d; a.E = E; a.logits = logits;
  return hip_status(launch_router(a, stream));
}

int moe_route(const float *logits, int32_t T, int32_t E, int32_t k, const moe_routing_t *out,
              void *ws, size_t ws_bytes, hipStream_t stream) {
  if (T < 0 || E <= 0 || k < 1 || k > E) return MOE_EINVAL;
  if (E > MOE_MAX_EXPERTS || T > kMaxRouteTokens || k > kMaxTopK) return MOE_EUNSUPPORTED;
  if (check_routing(out) != MOE_OK) return MOE_EINVAL;
  if (T == 0) return MOE_OK;
  if (!logits || !ws || ((uintptr_t)ws % kAlign)) return MOE_EINVAL;
  if (ws_bytes < moe_route_workspace_bytes(T, E)) return MOE_EWORKSPACE;
  return enqueue_route(logits, T, E, k, *out, static_cast<int32_t *>(ws), nullptr, nullptr, nullptr, nullptr, 0,
                       stream);
}

int moe_grouped_gemm_int4(const uint16_t *A, int32_t lda, const int32_t *a_row, int32_t N,
                          int32_t K, const uint32_t *Wq, const uint16_t *Ws, const uint16_t *Wb,
                          const int32_t *block_map, const int32_t *num_blocks, int32_t max_blocks,
                          float *C, int32_t ldc, hipStream_t stream) {
  if (!A || !Wq || !Ws || !Wb || !block_map || !num_blocks || !C) return MOE_EINVAL;
  if (N <= 0 || K <= 0 || max_blocks < 0 || lda < K || ldc < N) return MOE_EINVAL;
  if (N % 64 || K % 64) return MOE_EUNSUPPORTED;
  if ((int64_t)N * (K / 8) >= (1LL << 31)) return MOE_EUNSUPPORTED;  // 32-bit code offsets
  if (!aligned16(A) || lda % 8 || !aligned16(Wq) || !aligned16(Ws) || !aligned16(Wb))
    return MOE_EINVAL;
  if (max_blocks == 0) return MOE_OK;
  GemmArgs g{};
  GemmProblem &p = g.prob[0];
  p.A = A; p.lda = lda; p.a_row = a_row;
  p.Wq = Wq; p.Ws = Ws; p.Wb = Wb;
  p.wq_estride = (int64_t)N * (K / 8); p.ws_estride = (int64_t)N * (K / 64);
  p.N = N; p.K = K;
  p.units = block_map; p.num_units = num_blocks; p.implicit_rows = 0;
  p.nslices = (int)ceil_div(N, kGemmCols);
  p.wg_begin = 0;
  p.C = C; p.ldc = ldc;
  g.nprob = 1;
  g.total_wg = problem_wgs(max_blocks, p.nslices);
  return hip_status(launch_gemm(g, kStoreC, false, stream));
}

int moe_layer_forward(const moe_layer_t *L, const uint16_t *x, const float *logits, int32_t T,
                      float *y, const moe_routing_t *routing, void *ws, size_t ws_bytes,
                      hipStream_t stream) {
  int st = check_layer(L);
  if (st != MOE_OK) return st;
  if (T < 0) return MOE_EINVAL;
  if (T > kMaxRouteTokens) return MOE_EUNSUPPORTED;
  if (routing && check_routing(routing) != MOE_OK) return MOE_EINVAL;
  if (T == 0) return MOE_OK;
  if (!x || !logits || !y || !ws) return MOE_EINVAL;
  if (!aligned16(x) || !aligned16(y) || ((uintptr_t)ws % kAlign)) return MOE_EINVAL;
  return forward_one(L, x, logits, T, y, routing, ws, ws_bytes, stream);
}

int moe_router_topk(const uint16_t *x, int32_t T, int32_t d, const uint16_t *w_r, int32_t E, int32_t k,
                    float *logits, int32_t *topk_ids, float *topk_w, hipStream_t stream) {
  if (T < 0 || d < 1 || E < 1 || k < 1 || k > E) return MOE_EINVAL;
  if (d % 32 || E > MOE_MAX_EXPERTS || k > kMaxTopK || T > kMaxRouteTokens) return MOE_EUNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!x || !w_r || !logits || !topk_ids || !topk_w || !aligned16(x) || !aligned16(w_r) || !aligned16(logits))
    return MOE_EINVAL;
  RouterArgs ra{};
  ra.x = x; ra.w = w_r; ra.T = T; ra.d = d; ra.E = E; ra.logits = logits;
  int st = hip_status(launch_router(ra, stream));
  if (st != MOE_OK) return st;
  TopkArgs ta{};
  ta.logits = logits; ta.T = T; ta.E = E; ta.k = k; ta.topk_ids = topk_ids; ta.topk_w = topk_w;
  return hip_status(launch_topk(ta, stream));
}

int moe_layer_forward_router(const moe_layer_t *L, const uint16_t *x, const uint16_t *w_r, int32_t T,
                             float *y, const moe_routing_t *routing, void *ws, size_t ws_bytes,
                             hipStream_t stream) {
  int st = check_layer(L);
  if (st != MOE_OK) return st;
  if (T < 0) return MOE_EINVAL;
  if (T > kMaxRouteTokens || L->d % 32) return MOE_EUNSUPPORTED;
  if (routing && check_routing(routing) != MOE_OK) return MOE_EINVAL;
  if (T == 0) return MOE_OK;
  if (!x || !w_r || !y || !ws) return MOE_EINVAL;
  if (!aligned16(x) || !aligned16(w_r) || !aligned16(y) || ((uintptr_t)ws % kAlign)) return MOE_EINVAL;
  // logits are computed into the workspace where needed; forward_one reads them from there
  Workspace w;
  carve_layer(T, L, static_cast<char *>(ws), &w);
  return forward_one(L, x, w.logits, T, y, routing, ws, ws_bytes, stream, nullptr,
                     FwdOptions{kUnitRows, kNarrowTail, false, true}, nullptr, w_r);
}

int moe_layer_forward_checked(const moe_layer_t *L, const uint16_t *x, const float *logits, int32_t T,
                              float *y, const moe_routing_t *routing, void *ws, size_t ws_bytes,
                              hipStream_t stream, uint32_t *overflow) {
  int st = check_layer(L);
  if (st != MOE_OK) return st;
  if (T < 0) return MOE_EINVAL;
  if (T > kMaxRouteTokens) return MOE_EUNSUPPORTED;
  if (routing && check_routing(routing) != MOE_OK) return MOE_EINVAL;
  if (T == 0) return MOE_OK;
  if (!x || !logits || !y || !ws) return MOE_EINVAL;
  if (!aligned16(x) || !aligned16(y) || ((uintptr_t)ws % kAlign) || ((uintptr_t)overflow % 4)) return MOE_EINVAL;
  return forward_one(L, x, logits, T, y, routing, ws, ws_bytes, stream, nullptr,
                     FwdOptions{kUnitRows, kNarrowTail, false, true}, overflow);
}

int moe_layer_forward_timed(const moe_layer_t *L, const uint16_t *x, const float *logits,
                            int32_t T, float *y, const moe_routing_t *routing, void *ws,
                            size_t ws_bytes, hipStream_t stream, hipEvent_t *events) {
  if (!events) return MOE_EINVAL;
  int st = check_layer(L);
  if (st != MOE_OK) return st;
  if (T < 1) return MOE_EINVAL;
  if (T > kMaxRouteTokens) return MOE_EUNSUPPORTED;
  if (routing && check_routing(routing) != MOE_OK) return MOE_EINVAL;
  if (!x || !logits || !y || !ws) return MOE_EINVAL;
  if (!aligned16(x) || !aligned16(y) || ((uintptr_t)ws % kAlign)) return MOE_EINVAL;
  return forward_one(L, x, logits, T, y, routing, ws, ws_bytes, stream, events);
}

int moe_layer_forward_ablation(const moe_layer_t *L, const uint16_t *x, const float *logits, int32_t T,
                               float *y, const moe_routing_t *routing, void *ws, size_t ws_bytes,
                               hipStream_t stream, int32_t variant) {
  FwdOptions opt{kUnitRows, kNarrowTail, false, false};
  switch (variant) {
    case MOE_ABLATION_NONE: break;
    case MOE_ABLATION_TILE16: opt.unit_rows = 16; opt.ntail = 0; break;
    case MOE_ABLATION_HOST_ROUTING: opt.host_routing = true; break;
    case MOE_ABLATION_UNFUSED: opt.unfused = true; opt.ntail = 0; break;
    default: return MOE_EINVAL;
  }
  int st = check_layer(L);
  if (st != MOE_OK) return st;
  if (T < 0) return MOE_EINVAL;
  if (T > kMaxRouteTokens) return MOE_EUNSUPPORTED;
  if (routing && check_routing(routing) != MOE_OK) return MOE_EINVAL;
  if (T == 0) return MOE_OK;
  if (!x || !logits || !y || !ws) return MOE_EINVAL;
  if (!aligned16(x) || !aligned16(y) || ((uintptr_t)ws % kAlign)) return MOE_EINVAL;
  return forward_one(L, x, logits, T, y, routing, ws, ws_bytes, stream, nullptr, opt);
}

int moe_prefill_chunked(const moe_layer_t *L, const uint16_t *x, const float *logits, int32_t T,
                        int32_t chunk, float *y, void *ws, size_t ws_bytes, hipStream_t stream) {
  int st = check_layer(L);
  if (st != MOE_OK) return st;
  if (T < 0 || chunk < 1) return MOE_EINVAL;
  if (chunk > kMaxRouteTokens || T > MOE_MAX_TOKENS) return MOE_EUNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!x || !logits || !y || !ws) return MOE_EINVAL;
  if (!aligned16(x) || !aligned16(y) || ((uintptr_t)ws % kAlign)) return MOE_EINVAL;
  // every chunk's need is checked before the first is enqueued (the
  // workspace size is non-decreasing in T, so the first chunk's covers the
  // shorter last one)
  const int32_t c0 = std::min(chunk, T), tail = T - (T - 1) / chunk * chunk;
  if (ws_bytes < moe_workspace_bytes(c0, L) || ws_bytes < moe_workspace_bytes(tail, L)) return MOE_EWORKSPACE;
  for (int32_t t0 = 0; t0 < T; t0 += chunk) {
    const int32_t n = std::min(chunk, T - t0);
    st = forward_one(L, x + (int64_t)t0 * L->d, logits + (int64_t)t0 * L->E, n,
                     y + (int64_t)t0 * L->d, nullptr, ws, ws_bytes, stream);
    if (st != MOE_OK) return st;
  }
  return MOE_OK;
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Workspace for callers that cannot allocate: one static device array per GPU
// the library runs on, held until the process ends. In host code `scratch`
// names a host-side stand-in, not device memory; its device address comes
// from hipGetSymbolAddress, once per device with that device current, and
// only that address is handed to kernels.
__device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxDevices] = {};

// Device address of this device's scratch array (nullptr on failure).
void *device_scratch(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void *ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

int moe_layer_forward_noalloc(const moe_layer_t *L, const uint16_t *x, const float *logits, int32_t T,
                              float *y, const moe_routing_t *routing, hipStream_t stream) {
  int st = check_layer(L);
  if (st != MOE_OK) return st;
  if (T < 0) return MOE_EINVAL;
  if (T > kMaxRouteTokens) return MOE_EUNSUPPORTED;
  if (routing && check_routing(routing) != MOE_OK) return MOE_EINVAL;
  if (T == 0) return MOE_OK;
  if (!x || !logits || !y) return MOE_EINVAL;
  if (!aligned16(x) || !aligned16(y)) return MOE_EINVAL;
  if (layer_ws_bytes(T, L) > (size_t)MOE_NOALLOC_SCRATCH_BYTES) return MOE_EWORKSPACE;
  // the stream must belong to the current device, whose scratch array is used
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_EHIP;
  if (stream) {
    hipDevice_t sdev = -1;
    if (hipStreamGetDevice(stream, &sdev) != hipSuccess) return MOE_EHIP;
    if ((int)sdev != dev) return MOE_EINVAL;
  }
  void *ws = device_scratch(dev);
  if (!ws) return MOE_EHIP;
  return forward_one(L, x, logits, T, y, routing, ws, (size_t)MOE_NOALLOC_SCRATCH_BYTES, stream);
}

}  // extern "C"

// A captured layer call: the executable graph and the side stream and events
// its concurrent form was captured with.
struct moe_layer_graph {
  hipGraphExec_t exec = nullptr;
  hipStream_t side = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};

namespace {
void destroy_graph(moe_layer_graph_t *g) {
  if (!g) return;
  if (g->exec) (void)hipGraphExecDestroy(g->exec);
  if (g->fork) (void)hipEventDestroy(g->fork);
  if (g->join) (void)hipEventDestroy(g->join);
  if (g->side) (void)hipStreamDestroy(g->side);
  delete g;
}
}  // namespace

extern "C" {

int moe_layer_graph_create(const moe_layer_t *L, const uint16_t *x, const float *logits, int32_t T, float *y,
                           void *ws, size_t ws_bytes, int32_t flags, int32_t shared_unit_rows, hipStream_t stream,
                           moe_layer_graph_t **out) {
  if (!out) return MOE_EINVAL;
  *out = nullptr;
  int st = check_layer(L);
  if (st != MOE_OK) return st;
  if (T < 1 || !stream || (flags & ~MOE_GRAPH_CONCURRENT)) return MOE_EINVAL;
  if (shared_unit_rows == 0) shared_unit_rows = kUnitRows;
  if (shared_unit_rows < 16 || shared_unit_rows > kUnitRows || shared_unit_rows % 16) return MOE_EINVAL;
  if (T > kMaxRouteTokens) return MOE_EUNSUPPORTED;
  if (!x || !logits || !y || !ws) return MOE_EINVAL;
  if (!aligned16(x) || !aligned16(y) || ((uintptr_t)ws % kAlign)) return MOE_EINVAL;
  if (ws_bytes < layer_ws_bytes(T, L)) return MOE_EWORKSPACE;
  moe_layer_graph_t *g = new (std::nothrow) moe_layer_graph_t();
  if (!g) return MOE_EHIP;
  FwdOptions opt{kUnitRows, kNarrowTail, false, true};
  if (flags & MOE_GRAPH_CONCURRENT) {
    // default-priority side stream; events only order work
    if (hipStreamCreateWithFlags(&g->side, hipStreamNonBlocking) != hipSuccess ||
        hipEventCreateWithFlags(&g->fork, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&g->join, hipEventDisableTiming) != hipSuccess) {
      destroy_graph(g);
      return MOE_EHIP;
    }
    opt.side = g->side;
    opt.fork = g->fork;
    opt.join = g->join;
    opt.shared_unit_rows = shared_unit_rows;
  }
  hipGraph_t graph = nullptr;
  if (hipStreamBeginCapture(stream, hipStreamCaptureModeThreadLocal) != hipSuccess) {
    destroy_graph(g);
    return MOE_EHIP;
  }
  st = forward_one(L, x, logits, T, y, nullptr, ws, ws_bytes, stream, nullptr, opt);
  const hipError_t end = hipStreamEndCapture(stream, &graph);
  if (st == MOE_OK && (end != hipSuccess || !graph)) st = MOE_EHIP;
  if (st == MOE_OK && hipGraphInstantiate(&g->exec, graph, nullptr, nullptr, 0) != hipSuccess) st = MOE_EHIP;
  if (graph) (void)hipGraphDestroy(graph);
  if (st != MOE_OK) {
    destroy_graph(g);
    return st;
  }
  *out = g;
  return MOE_OK;
}

int moe_layer_graph_launch(moe_layer_graph_t *g, hipStream_t stream) {
  if (!g || !g->exec) return MOE_EINVAL;
  return hip_status(hipGraphLaunch(g->exec, stream));
}

int moe_layer_graph_destroy(moe_layer_graph_t *g) {
  if (!g) return MOE_EINVAL;
  destroy_graph(g);
  return MOE_OK;
}

const char *moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_EINVAL: return "invalid argument (null or misaligned pointer, bad size, k > E)";
    case MOE_EUNSUPPORTED: return "unsupported shape (d, f, f_sh not multiples of 64; E > 1024; too many tokens)";
    case MOE_EWORKSPACE: return "workspace too small";
    case MOE_EHIP: return "HIP runtime error at launch";
    default: return "unknown status";
  }
}

}  // extern "C"
