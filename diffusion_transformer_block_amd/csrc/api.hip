// C ABI of the block-stage library: argument validation, packed-weight and
// workspace layouts, the block driver and the graph-captured denoise loop.
// The meaning of every entry point is documented in include/blk.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/blk.h"
#include "common.h"
#include "attn_small.h"
#include "internal.h"
#include "skinny.h"
#include "stage.h"

using namespace blk;

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

#define HIP_TRY(expr)                                                                  \
  do {                                                                                 \
    hipError_t e_ = (expr);                                                            \
    if (e_ != hipSuccess) return fail(BLK_EHIP, "%s: %s", #expr, hipGetErrorString(e_)); \
  } while (0)

constexpr size_t kAlign = 256;
inline size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

constexpr size_t kSkCtrWords = 4096;    // split-K counters per skinny GEMM: one per group block
constexpr size_t kBigCtrWords = kBigMaxSplitTiles;

// ---------------------------------------------------------------- validation
int check_config(const blk_config* c) {
  if (!c) return fail(BLK_EINVAL, "cfg is NULL");
  if (c->hidden <= 0 || c->ffn <= 0 || c->n_q_heads <= 0 || c->n_kv_heads <= 0 ||
      c->head_dim <= 0 || c->max_pos <= 0)
    return fail(BLK_EINVAL, "cfg has a non-positive size");
  if (!std::isfinite(c->rope_base) || c->rope_base <= 0.f)
    return fail(BLK_EINVAL, "rope_base must be finite and > 0");
  if (!std::isfinite(c->rms_eps) || c->rms_eps < 0.f)
    return fail(BLK_EINVAL, "rms_eps must be finite and >= 0");
  const int d = c->head_dim;
  if (d != 64 && d != 128 && d != 256)
    return fail(BLK_EUNSUPPORTED, "head_dim %d not in {64, 128, 256}", d);
  if (c->hidden % 128 != 0 || c->hidden > 16384)
    return fail(BLK_EUNSUPPORTED, "hidden %d must be a multiple of 128 and <= 16384", c->hidden);
  if (c->ffn % 128 != 0 || c->ffn > 65536)
    return fail(BLK_EUNSUPPORTED, "ffn %d must be a multiple of 128 and <= 65536", c->ffn);
  if (c->n_q_heads % c->n_kv_heads != 0)
    return fail(BLK_EUNSUPPORTED, "n_q_heads %d is not a multiple of n_kv_heads %d",
                c->n_q_heads, c->n_kv_heads);
  if ((c->n_q_heads * d) % 128 != 0 || ((c->n_q_heads + 2 * c->n_kv_heads) * d) % 128 != 0)
    return fail(BLK_EUNSUPPORTED, "Hq*d and (Hq+2Hkv)*d must be multiples of 128");
  if (c->max_pos > (1 << 20)) return fail(BLK_EUNSUPPORTED, "max_pos > 2^20");
  if ((size_t)(c->n_q_heads + 2 * c->n_kv_heads) * d / 32 > kSkCtrWords)
    return fail(BLK_EUNSUPPORTED, "(Hq + 2 Hkv) * head_dim above %zu", kSkCtrWords * 32);
  return BLK_OK;
}

// ---------------------------------------------------------------- packed layout
struct Layout {
  size_t rope_cos = 0, rope_sin = 0;
  size_t layer0 = 0, layer_bytes = 0;
  size_t wqkv = 0, wo = 0, wgu = 0, wd = 0;  // offsets inside a layer
  bool has_head = false;
  size_t h_wfused = 0, h_table = 0, h_dt = 0, h_w3 = 0, h_b3 = 0, h_ws = 0, h_bs = 0,
         h_wout = 0, h_bout = 0;
  size_t total = 0;
  int n_layers = 0, n_steps = 0, n_actions = 0, action_dim = 0;
};

Layout make_layout(const blk_config& c, int n_layers, bool head, int n_steps, int N, int A) {
  Layout L;
  const size_t D = c.hidden, F = c.ffn, d = c.head_dim, Hq = c.n_q_heads, Hkv = c.n_kv_heads;
  size_t off = 0;
  L.rope_cos = off;
  off += align_up((size_t)c.max_pos * (d / 2) * 4);
  L.rope_sin = off;
  off += align_up((size_t)c.max_pos * (d / 2) * 4);
  L.layer0 = off;
  size_t lo = 0;
  L.wqkv = lo;
  lo += align_up(D * (Hq + 2 * Hkv) * d * 2);
  L.wo = lo;
  lo += align_up(Hq * d * D * 2);
  L.wgu = lo;
  lo += align_up(D * 2 * F * 2);
  L.wd = lo;
  lo += align_up(F * D * 2);
  L.layer_bytes = lo;
  off += (size_t)n_layers * lo;
  L.n_layers = n_layers;
  if (head) {
    L.has_head = true;
    L.n_steps = n_steps;
    L.n_actions = N;
    L.action_dim = A;
    L.h_wfused = off;
    off += align_up((size_t)A * D * 4);
    L.h_table = off;
    off += align_up((size_t)n_steps * D * 4);
    L.h_dt = off;
    off += align_up((size_t)n_steps * 4);
    L.h_w3 = off;
    off += align_up(D * D * 2);
    L.h_b3 = off;
    off += align_up(D * 4);
    L.h_ws = off;
    off += align_up((size_t)A * D * 4);
    L.h_bs = off;
    off += align_up(D * 4);
    L.h_wout = off;
    off += align_up(D * (size_t)A * 4);
    L.h_bout = off;
    off += align_up((size_t)A * 4);
  }
  L.total = off;
  return L;
}

struct PackRecord {
  blk_config cfg;
  Layout lay;
};

std::mutex g_mu;
std::map<const void*, PackRecord> g_packs;

bool same_cfg(const blk_config& a, const blk_config& b) {
  return a.hidden == b.hidden && a.ffn == b.ffn && a.n_q_heads == b.n_q_heads &&
         a.n_kv_heads == b.n_kv_heads && a.head_dim == b.head_dim && a.max_pos == b.max_pos &&
         a.rope_base == b.rope_base && a.rms_eps == b.rms_eps;
}

int lookup(const void* packed, const blk_config& cfg, PackRecord* out) {
  std::lock_guard<std::mutex> lk(g_mu);
  auto it = g_packs.find(packed);
  if (it == g_packs.end())
    return fail(BLK_ESTATE, "packed buffer %p was not prepared by blk_prepare_weights", packed);
  if (!same_cfg(it->second.cfg, cfg))
    return fail(BLK_ESTATE, "cfg differs from the one the packed buffer was prepared with");
  *out = it->second;
  return BLK_OK;
}

// ---------------------------------------------------------------- workspace layout
// Every workspace starts with the same synchronization region, whatever the
// config and whichever entry point uses it: the skinny GEMMs' split-K arrival
// counters, the large GEMMs' tail-split counters, the persistent kernel's
// phase flags and its epoch / done / abort words.  Counters are zero at rest
// (each call leaves them zero); flags and the epoch only grow.  Activations
// and partials follow the region, so a workspace can be reused across shapes
// and entry points without a counter ever landing on stale activation bytes.
struct SyncRegion {
  size_t ctr_qkv, ctr_o, ctr_gu, ctr_d, big_ctr, flags, sync, total;
};
constexpr SyncRegion make_sync_region() {
  SyncRegion r{};
  size_t off = 0;
  r.ctr_qkv = off;
  off += kSkCtrWords * 4;
  r.ctr_o = off;
  off += kSkCtrWords * 4;
  r.ctr_gu = off;
  off += kSkCtrWords * 4;
  r.ctr_d = off;
  off += kSkCtrWords * 4;
  r.big_ctr = off;
  off += kBigCtrWords * 4;
  r.flags = off;
  off += (size_t)kPhCount * kStageMaxFlags * 4;
  r.sync = off;
  off += 256;
  r.total = off;
  return r;
}
constexpr SyncRegion kSync = make_sync_region();
static_assert(kSync.total % 256 == 0, "the sync region keeps the activations 256-byte aligned");
static_assert(kSync.total == BLK_WS_SYNC_BYTES, "blk.h states the sync region's size");
// the persistent kernel's words in the sync slot: [1] done counter, [2] abort
static_assert(kSync.sync + 2 * sizeof(unsigned) == BLK_WS_ABORT_OFFSET, "blk.h states the abort word's offset");

struct BlockWs {
  size_t q, o, h, a, r1, r2, part;
  size_t ctr_qkv, ctr_o, ctr_gu, ctr_d;
  size_t big_part, big_ctr;     // large-chunk GEMM K splits
  size_t sm_att_o, sm_att_ml;   // small-chunk attention key-slice partials
  size_t xb0, xb1, flags, sync;
  size_t plen;                  // per-stream prefix lengths (blk_forward_chunks)
  size_t total;
};

// Activations and partials of one block stage from offset `base` (at least
// the end of the sync region) on.
BlockWs block_ws_layout(const blk_config& c, int B, int T, int P, size_t base,
                        size_t extra_part = 0) {
  BlockWs w;
  const size_t M = (size_t)B * T;
  const int D = c.hidden, F = c.ffn, d = c.head_dim, Hq = c.n_q_heads, Hkv = c.n_kv_heads;
  const int gq = (Hq + 2 * Hkv) * d / 32, go = D / 32, ggu = F / 16, gd = D / 32;
  w.ctr_qkv = kSync.ctr_qkv;
  w.ctr_o = kSync.ctr_o;
  w.ctr_gu = kSync.ctr_gu;
  w.ctr_d = kSync.ctr_d;
  w.big_ctr = kSync.big_ctr;
  w.flags = kSync.flags;
  w.sync = kSync.sync;
  // activations between operators are in operand order, padded to 16-row
  // tiles; Q is in the attention's operand order (32-row tiles per kv head)
  const bool small = M > 0 && (int)M <= kSkinnyMaxM;
  const size_t Mp = (size_t)16 * mt_of((int)M);
  const size_t q_rows = std::max(Mp * Hq, (size_t)B * Hkv * 32 * (((Hq / Hkv) * (size_t)T + 31) / 32));
  size_t off = std::max(base, kSync.total);
  w.q = off;
  off += align_up(q_rows * d * 2);
  w.o = off;
  off += align_up(Mp * Hq * d * 2);
  w.h = off;
  off += align_up(Mp * D * 2);
  w.a = off;   // also x in operand order ahead of the large-chunk QKV step
  off += align_up(Mp * std::max(F, D) * 2);
  w.r1 = off;
  off += align_up(M * 4);
  w.r2 = off;
  off += align_up(M * 4);
  size_t part = 0;
  part = std::max(part, extra_part);
  if (small) {
    const int m = (int)M;
    for (size_t v : {sk_part_floats(m, D, gq, true), sk_part_floats(m, D, gq, false),
                     sk_part_floats(m, Hq * d, go, false), sk_part_floats(m, D, ggu, false),
                     sk_part_floats(m, F, gd, false)})
      part = std::max(part, v);
  }
  w.part = off;
  off += align_up(part * 4);
  {
    size_t bp = 0;
    if (!small && M > 0) {
      const int m = (int)M;
      for (const BigPlan& pl : {big_plan(m, gq, D), big_plan(m, go, Hq * d), big_plan(m, ggu, D),
                                big_plan(m, gd, F)})
        bp = std::max(bp, big_part_floats(pl));
    }
    w.big_part = off;
    off += align_up(bp * 4);
  }
  w.sm_att_o = off;
  off += align_up(attn_sm_part_o_elems(B, T, P, Hq, Hkv, d) * 2);
  w.sm_att_ml = off;
  off += align_up(attn_sm_part_ml_floats(B, T, P, Hq, Hkv, d) * 4);
  w.xb0 = off;
  off += align_up(Mp * D * 2);
  w.xb1 = off;
  off += align_up(Mp * D * 2);
  w.plen = off;
  off += align_up(kMaxVarStreams * 4);
  w.total = off;
  return w;
}

template <class T>
T* at(void* base, size_t off) {
  return reinterpret_cast<T*>(reinterpret_cast<char*>(base) + off);
}
template <class T>
const T* at(const void* base, size_t off) {
  return reinterpret_cast<const T*>(reinterpret_cast<const char*>(base) + off);
}

// ---------------------------------------------------------------- operator timing
// While on, blk_forward brackets each operator of the stage with HIP events on
// the caller's stream (nothing else changes); blk_operator_times reads them.
constexpr size_t kTimerMaxEvents = 6 * 4096;
struct OpTimer {
  bool on = false;
  std::vector<hipEvent_t> pool;   // created on first use, reused after each read
  size_t used = 0;
  struct Rec {
    int op;
    size_t e0, e1;
  };
  std::vector<Rec> recs;
  double sum_ms[BLK_N_OPS] = {};
  int calls[BLK_N_OPS] = {};
};
OpTimer g_timer;
std::mutex g_timer_mu;
// Set by blk_forward for the duration of one enqueue when timing is on (the
// stream may be the null stream, hence the separate flag).
thread_local bool g_marking = false;
thread_local hipStream_t g_mark_stream = nullptr;
thread_local size_t g_mark_prev = 0;

hipError_t timer_event(hipStream_t st, size_t* idx) {
  if (g_timer.used == g_timer.pool.size()) {
    // no system-scope fence (an L2 write-back per event) between the kernels
    hipEvent_t e;
    const hipError_t r = hipEventCreateWithFlags(&e, hipEventDisableSystemFence);
    if (r != hipSuccess) return r;
    g_timer.pool.push_back(e);
  }
  *idx = g_timer.used++;
  return hipEventRecord(g_timer.pool[*idx], st);
}

// End of operator `op` of the stage being enqueued (no-op unless timing).
void op_done(int op) {
  if (!g_marking) return;
  size_t e;
  if (timer_event(g_mark_stream, &e) != hipSuccess) return;
  g_timer.recs.push_back({op, g_mark_prev, e});
  g_mark_prev = e;
}

// ---------------------------------------------------------------- persistent stage plan
int g_exec_mode = 0;   // 0 auto, 1 per-operator kernels, 2 persistent stage kernel only

// Whether auto mode takes the persistent stage kernel.  It does not yet: on the
// 64-token block the graph of per-operator kernels measures faster.
bool want_persistent() { return g_exec_mode == 2; }

// Fills the shapes, splits, phase maps and attention plan of a stage launch;
// false if the persistent kernel does not cover this shape.
bool stage_plan(const blk_config& c, int B, int T, int P, int flow_N, int nwg, StageArgs& sa) {
  const int D = c.hidden, F = c.ffn, d = c.head_dim, Hq = c.n_q_heads, Hkv = c.n_kv_heads;
  const int M = B * T;
  if (nwg <= 0 || M <= 0 || M > kSkinnyMaxM) return false;
  if (flow_N > 0 && flow_N + 1 != M) return false;
  const int G_q = (Hq + 2 * Hkv) * d / 32, G_o = D / 32, G_gu = F / 16, G_d = D / 32;
  // a block's first layer reads the caller's row-major input, later layers
  // the operand-order buffers; both plan alike
  const SkPlan p_qkv = sk_plan(M, D, G_q, true), p_o = sk_plan(M, Hq * d, G_o, false),
               p_gu = sk_plan(M, D, G_gu, false), p_d = sk_plan(M, F, G_d, false),
               p_w3 = flow_N > 0 ? sk_plan(flow_N, D, G_o, false) : SkPlan{1, 1};
  for (const SkPlan& p : {p_qkv, p_o, p_gu, p_d, p_w3})
    if (p.splits < 1) return false;
  sa.split_qkv = p_qkv.splits;
  sa.split_o = p_o.splits;
  sa.split_gu = p_gu.splits;
  sa.split_d = p_d.splits;
  sa.split_w3 = p_w3.splits;
  sa.gpw_qkv = p_qkv.gpw;
  sa.gpw_o = p_o.gpw;
  sa.gpw_gu = p_gu.gpw;
  sa.gpw_d = p_d.gpw;
  sa.gpw_w3 = p_w3.gpw;
  int splits = 1, kps = 32;
  attn_sm_plan(B, T, P, Hq, Hkv, &splits, &kps, nullptr);
  const int n_rbt = B * Hkv * (((Hq / Hkv) * T + 63) / 64);
  const int n_att = n_rbt * splits;
  const int n_cmb = splits > 1 ? (attn_combine_items(B, T, Hq, Hkv, d) + 255) / 256 : 0;
  const int n_emb = (flow_N + 1 + 3) / 4;
  // tasks of a GEMM phase: (group block, split); one flag per group block
  auto nt = [](int G, const SkPlan& p) { return G / p.gpw * p.splits; };
  for (int n : {nt(G_q, p_qkv), n_att, n_cmb, nt(G_o, p_o), nt(G_gu, p_gu), nt(G_d, p_d), nt(G_o, p_w3),
                n_emb, flow_N})
    if (n > kStageMaxFlags) return false;
  sa.B = B;
  sa.T = T;
  sa.P = P;
  sa.M = M;
  sa.D = D;
  sa.F = F;
  sa.Hq = Hq;
  sa.Hkv = Hkv;
  sa.d = d;
  sa.eps = c.rms_eps;
  sa.att_splits = splits;
  sa.att_kps = kps;
  sa.att_merge_tasks = n_cmb;
  sa.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)d));
  int w0 = 0;
  auto map = [&](int type, int n_tasks, int n_flags) {
    PhaseMap& m = sa.ph[type];
    m.n_tasks = n_tasks;
    m.n_flags = n_flags;
    m.nw = std::max(1, std::min(n_tasks, nwg));
    m.w0 = w0 % nwg;
    w0 = (w0 + n_tasks) % nwg;
  };
  if (flow_N > 0) {
    map(kPhEMB, n_emb, n_emb);
    map(kPhW3, nt(G_o, p_w3), G_o / p_w3.gpw);
  }
  map(kPhQKV, nt(G_q, p_qkv), G_q / p_qkv.gpw);
  map(kPhATT, n_att, n_att);
  if (n_cmb > 0) map(kPhCMB, n_cmb, n_cmb);
  map(kPhO, nt(G_o, p_o), G_o / p_o.gpw);
  map(kPhGU, nt(G_gu, p_gu), G_gu / p_gu.gpw);
  map(kPhD, nt(G_d, p_d), G_d / p_d.gpw);
  if (flow_N > 0) map(kPhVEL, flow_N, flow_N);
  return true;
}

void stage_fill_common(StageArgs& sa, const Layout& lay, const void* packed, void* ws,
                       const BlockWs& w) {
  sa.packed = reinterpret_cast<const uint8_t*>(packed);
  sa.layer0 = lay.layer0;
  sa.layer_bytes = lay.layer_bytes;
  sa.off_qkv = lay.wqkv;
  sa.off_o = lay.wo;
  sa.off_gu = lay.wgu;
  sa.off_d = lay.wd;
  sa.cos_t = at<float>(packed, lay.rope_cos);
  sa.sin_t = at<float>(packed, lay.rope_sin);
  sa.xb[0] = at<bf16_t>(ws, w.xb0);
  sa.xb[1] = at<bf16_t>(ws, w.xb1);
  sa.q = at<bf16_t>(ws, w.q);
  sa.o = at<bf16_t>(ws, w.o);
  sa.h = at<bf16_t>(ws, w.h);
  sa.a = at<bf16_t>(ws, w.a);
  sa.att_part_o = at<bf16_t>(ws, w.sm_att_o);
  sa.att_part_ml = at<float>(ws, w.sm_att_ml);
  sa.part = at<float>(ws, w.part);
  sa.ctr_qkv = at<unsigned>(ws, w.ctr_qkv);
  sa.ctr_o = at<unsigned>(ws, w.ctr_o);
  sa.ctr_gu = at<unsigned>(ws, w.ctr_gu);
  sa.ctr_d = at<unsigned>(ws, w.ctr_d);
  sa.flags = at<unsigned>(ws, w.flags);
  sa.done_ctr = at<unsigned>(ws, w.sync) + 1;
  sa.abort_word = at<unsigned>(ws, w.sync) + 2;
}

// ---------------------------------------------------------------- block driver
struct BlockIO {
  const bf16_t* x;
  const bf16_t* kp;
  const bf16_t* vp;
  int64_t prefix_stride;
  bf16_t* y;
  bf16_t* kn;
  bf16_t* vn;
  int64_t new_stride;
  const int32_t* plen;    // host: stream b's prefix length (NULL: every stream has P)
};

// The per-stream prefix lengths travel to one small kernel by value and from
// there, through the workspace, to the block's kernels.
struct StreamLens {
  int n;
  int len[kMaxVarStreams];
};
__global__ void write_lens_kernel(int* dst, StreamLens v) {
  if ((int)threadIdx.x < v.n) dst[threadIdx.x] = v.len[threadIdx.x];
}
// Enqueues the lengths' copy into the workspace; NULL when every stream has P.
const int* stream_prefix_of(const BlockIO& io, int B, void* ws, const BlockWs& w, hipStream_t st) {
  if (!io.plen) return nullptr;
  StreamLens v{};
  v.n = B;
  for (int b = 0; b < B; ++b) v.len[b] = io.plen[b];
  int* dst = at<int>(ws, w.plen);
  write_lens_kernel<<<1, kMaxVarStreams, 0, st>>>(dst, v);
  return dst;
}

// Whether every skinny GEMM of a small chunk has a valid split.
bool small_plan_ok(const blk_config& c, int M, bool x_rowmajor) {
  const int D = c.hidden, F = c.ffn, d = c.head_dim, Hq = c.n_q_heads, Hkv = c.n_kv_heads;
  return sk_plan(M, D, (Hq + 2 * Hkv) * d / 32, x_rowmajor).splits >= 1 &&
         sk_plan(M, Hq * d, D / 32, false).splits >= 1 && sk_plan(M, D, F / 16, false).splits >= 1 &&
         sk_plan(M, F, D / 32, false).splits >= 1;
}

// Small chunk (B * T <= 64 rows): one launch per operator, activations in
// operand order.  x (block input, also the first residual) and y (block
// output) are row-major caller buffers for a single block, or operand-order
// rows inside the denoise loop (x_frag / y_frag).
void enqueue_block_small(const blk_config& c, const Layout& lay, const void* packed, int layer,
                         int B, int T, int P, const BlockIO& io, bool x_frag, bool y_frag, void* ws,
                         const BlockWs& w, hipStream_t st, bool prefetch = false,
                         const uint8_t* next_qkv = nullptr) {
  const int M = B * T, MT = mt_of(M);
  const int D = c.hidden, F = c.ffn, d = c.head_dim, Hq = c.n_q_heads, Hkv = c.n_kv_heads;
  const uint8_t* lw = at<uint8_t>(packed, lay.layer0 + (size_t)layer * lay.layer_bytes);
  const int* plen = stream_prefix_of(io, B, ws, w, st);
  bf16_t* q = at<bf16_t>(ws, w.q);
  bf16_t* o = at<bf16_t>(ws, w.o);
  bf16_t* h = at<bf16_t>(ws, w.h);
  bf16_t* a = at<bf16_t>(ws, w.a);
  SkArgs base{};
  base.M = M;
  base.eps = c.rms_eps;
  base.part = at<float>(ws, w.part);

  // 1. RMS(x) -> fused QKV GEMM with row scale and RoPE epilogue
  {
    SkArgs ga = base;
    ga.A = io.x;
    ga.lda = D;
    ga.K = D;
    ga.Bp = lw + lay.wqkv;
    ga.n_groups = (Hq + 2 * Hkv) * d / 32;
    const SkPlan p = sk_plan(M, D, ga.n_groups, !x_frag);
    ga.splits = p.splits;
    ga.counters = at<unsigned>(ws, w.ctr_qkv);
    EpiQkvS e{q, io.kn, io.vn, io.new_stride, at<float>(packed, lay.rope_cos),
              at<float>(packed, lay.rope_sin), T, P, Hq, Hkv, d};
    e.plen = plen;
    launch_sk_qkv(ga, p.gpw, !x_frag, e, st);
    op_done(BLK_OP_QKV);
  }
  // 2. attention over [prefix ; own]
  {
    AttnSmArgs aa{};
    aa.q = q;
    aa.kp = io.kp;
    aa.vp = io.vp;
    aa.prefix_stride = io.prefix_stride;
    aa.kn = io.kn;
    aa.vn = io.vn;
    aa.new_stride = io.new_stride;
    aa.o = o;
    aa.B = B;
    aa.T = T;
    aa.P = P;
    aa.Hq = Hq;
    aa.Hkv = Hkv;
    // (128-row blocks exist for d <= 128; at d = 256 the 64-row blocks take
    // their own plan)
    attn_sm_plan(B, T, P, Hq, Hkv, &aa.splits, &aa.kps, d <= 128 ? &aa.long_rows : nullptr);
    aa.plen = plen;
    aa.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)d));
    aa.part_o = at<bf16_t>(ws, w.sm_att_o);
    aa.part_ml = at<float>(ws, w.sm_att_ml);
    // (prefetch: chains of layers -- the denoise loop, the prefix stage --
    // whose weights stream from HBM)
    // Workgroups beside the attention's tasks read the layer's O and gate/up
    // weights, so those launches find them in the memory-side cache rather
    // than in HBM: 128 of them took the 18 x 10 loop 7.33 -> 7.21 ms (96
    // made the attention's tail wait for the prefetch, 176 crowded it;
    // gate/up prefetched from the O launch slowed O by more than gate/up
    // gained).  A single block call may find its weights resident, where the
    // prefetch costs about 1 us (the 64-token stage 39.4 -> 40.45 us; four
    // 16-token chunks replayed on one layer 48.6 -> 50.8 us), against 0.2 us
    // saved when they are cold, so it is left to chains of layers.  Small
    // ranges (the 16-token block's 1.2 MB: 17.20 -> 17.8 us) fit the cache
    // anyway and are never fetched.
    Prefetch pf;
    if (prefetch && lay.wd - lay.wo >= ((size_t)8 << 20)) {
      pf.p = lw + lay.wo;
      pf.bytes = lay.wd - lay.wo;
      pf.wgs = 128;
    }
    launch_attn_sm(aa, d, st, pf);
    op_done(BLK_OP_ATTENTION);
  }
  // 3. h = x + O W_o
  {
    SkArgs ga = base;
    ga.A = o;
    ga.K = Hq * d;
    ga.Bp = lw + lay.wo;
    ga.n_groups = D / 32;
    const SkPlan p = sk_plan(M, ga.K, ga.n_groups, false);
    ga.splits = p.splits;
    ga.counters = at<unsigned>(ws, w.ctr_o);
    EpiResidS e{io.x, x_frag ? 1 : 0, MT, nullptr, h, 1, MT, 0, D};
    launch_sk_resid(ga, p.gpw, e, st);
    op_done(BLK_OP_O_PROJ);
  }
  // 4. RMS(h) -> gate/up GEMM with SiLU(gate) * up epilogue
  {
    SkArgs ga = base;
    ga.A = h;
    ga.K = D;
    ga.Bp = lw + lay.wgu;
    ga.n_groups = F / 16;
    const SkPlan p = sk_plan(M, D, ga.n_groups, false);
    ga.splits = p.splits;
    ga.counters = at<unsigned>(ws, w.ctr_gu);
    launch_sk_gateup(ga, p.gpw, EpiGateUpS{a, MT}, st);
    op_done(BLK_OP_GATE_UP);
  }
  // 5. y = h + a W_d
  {
    SkArgs ga = base;
    ga.A = a;
    ga.K = F;
    ga.Bp = lw + lay.wd;
    ga.n_groups = D / 32;
    const SkPlan p = sk_plan(M, F, ga.n_groups, false);
    ga.splits = p.splits;
    ga.counters = at<unsigned>(ws, w.ctr_d);
    EpiResidS e{h, 1, MT, nullptr, io.y, y_frag ? 1 : 0, MT, 0, D};
    // (next_qkv: the next layer's QKV weights, in the denoise loop) one
    // prefetching workgroup per task reads them on the compute units the
    // split GEMM leaves free: the loop 7.30 -> 7.16 ms (one box)
    Prefetch pf;
    if (prefetch && next_qkv && lay.wo - lay.wqkv >= ((size_t)4 << 20)) {
      pf.p = next_qkv;
      pf.bytes = lay.wo - lay.wqkv;
    }
    launch_sk_resid(ga, p.gpw, e, st, pf);
    op_done(BLK_OP_DOWN);
  }
}

void enqueue_block(const blk_config& c, const Layout& lay, const void* packed, int layer, int B,
                   int T, int P, const BlockIO& io, void* ws, const BlockWs& w, hipStream_t st,
                   bool prefetch = false) {
  const int M = B * T;
  if (M <= kSkinnyMaxM) {
    enqueue_block_small(c, lay, packed, layer, B, T, P, io, false, false, ws, w, st, prefetch);
    return;
  }
  const int D = c.hidden, F = c.ffn, d = c.head_dim, Hq = c.n_q_heads, Hkv = c.n_kv_heads;
  const int MT = mt_of(M);
  const uint8_t* lw = at<uint8_t>(packed, lay.layer0 + (size_t)layer * lay.layer_bytes);
  const int* plen = stream_prefix_of(io, B, ws, w, st);
  bf16_t* q = at<bf16_t>(ws, w.q);
  bf16_t* o = at<bf16_t>(ws, w.o);
  bf16_t* h = at<bf16_t>(ws, w.h);
  bf16_t* a = at<bf16_t>(ws, w.a);
  float* r1 = at<float>(ws, w.r1);
  float* r2 = at<float>(ws, w.r2);

  GemmArgs base{};
  base.M = M;
  base.part = at<float>(ws, w.big_part);
  base.ctr = at<unsigned>(ws, w.big_ctr);

  // 1. RMS(x) -> fused QKV GEMM with row scale and RoPE epilogue (Q in the
  //    attention's operand order)
  {
    GemmArgs ga = base;
    ga.A = a;   // x in operand order (a is free until the gate/up step)
    ga.lda = D;
    ga.K = D;
    ga.Bp = lw + lay.wqkv;
    ga.n_groups = (Hq + 2 * Hkv) * d / 32;
    launch_rms_rows(io.x, M, D, false, c.rms_eps, r1, a, st);
    ga.r = r1;
    EpiQKV e{q, io.kn, io.vn, io.new_stride, at<float>(packed, lay.rope_cos),
             at<float>(packed, lay.rope_sin), T, P, Hq, Hkv, d};
    e.plen = plen;
    launch_gemm_qkv(ga, e, st);
    op_done(BLK_OP_QKV);
  }
  // 2. attention over [prefix ; own]: the chunk attention of the small path,
  //    64 query rows per workgroup over all keys (or key slices and a merge
  //    when there are few row blocks); O in operand order
  {
    AttnSmArgs aa{};
    aa.q = q;
    aa.kp = io.kp;
    aa.vp = io.vp;
    aa.prefix_stride = io.prefix_stride;
    aa.kn = io.kn;
    aa.vn = io.vn;
    aa.new_stride = io.new_stride;
    aa.o = o;
    aa.B = B;
    aa.T = T;
    aa.P = P;
    aa.Hq = Hq;
    aa.Hkv = Hkv;
    // (128-row blocks exist for d <= 128; at d = 256 the 64-row blocks take
    // their own plan)
    attn_sm_plan(B, T, P, Hq, Hkv, &aa.splits, &aa.kps, d <= 128 ? &aa.long_rows : nullptr);
    aa.plen = plen;
    aa.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)d));
    aa.part_o = at<bf16_t>(ws, w.sm_att_o);
    aa.part_ml = at<float>(ws, w.sm_att_ml);
    // (prefetch: the prefix stage's chain of layers) workgroups on the
    // compute units the attention leaves free read the layer's O and gate/up
    // weights ahead of those GEMMs, as in the denoise loop: the 768-token
    // prefix stage 1,783 -> 1,762 us (64 of them beside its 192 tasks)
    Prefetch pf;
    if (prefetch && lay.wd - lay.wo >= ((size_t)8 << 20)) {
      pf.p = lw + lay.wo;
      pf.bytes = lay.wd - lay.wo;
      pf.wgs = 128;
    }
    launch_attn_sm(aa, d, st, pf);
    op_done(BLK_OP_ATTENTION);
  }
  // 3. h = x + O W_o (h in operand order)
  {
    GemmArgs ga = base;
    ga.A = o;
    ga.lda = Hq * d;
    ga.K = Hq * d;
    ga.Bp = lw + lay.wo;
    ga.n_groups = D / 32;
    launch_gemm_residual(ga, EpiResidual{io.x, 0, h, 1, D, MT}, st);
    op_done(BLK_OP_O_PROJ);
  }
  // 4. RMS(h) -> gate/up GEMM with SiLU(gate) * up epilogue
  {
    GemmArgs ga = base;
    ga.A = h;
    ga.lda = D;
    ga.K = D;
    ga.Bp = lw + lay.wgu;
    ga.n_groups = F / 16;
    launch_rms_rows(h, M, D, true, c.rms_eps, r2, nullptr, st);
    ga.r = r2;
    launch_gemm_gateup(ga, EpiGateUp{a, MT}, st);
    op_done(BLK_OP_GATE_UP);
  }
  // 5. y = h + a W_d (y row-major, the caller's)
  {
    GemmArgs ga = base;
    ga.A = a;
    ga.lda = F;
    ga.K = F;
    ga.Bp = lw + lay.wd;
    ga.n_groups = D / 32;
    launch_gemm_residual(ga, EpiResidual{h, 1, io.y, 0, D, MT}, st);
    op_done(BLK_OP_DOWN);
  }
}

// K and V of a chunk only (no attention, O projection or FFN): RMS(x), then the
// fused QKV GEMM over its K and V column groups with the RoPE epilogue.  The
// last layer of a prefix stack runs this way, since only its K/V is read.
void enqueue_kv_only(const blk_config& c, const Layout& lay, const void* packed, int layer, int T,
                     int P, const bf16_t* x, bf16_t* kn, bf16_t* vn, void* ws, const BlockWs& w,
                     hipStream_t st) {
  const int M = T;
  const int D = c.hidden, d = c.head_dim, Hq = c.n_q_heads, Hkv = c.n_kv_heads;
  const uint8_t* lw = at<uint8_t>(packed, lay.layer0 + (size_t)layer * lay.layer_bytes);
  const int g_kv = Hq * d / 32, n_kv = 2 * Hkv * d / 32;
  const uint8_t* bp = lw + lay.wqkv + frag_offset(g_kv, 0, 0, D / 32);
  if (M <= kSkinnyMaxM) {
    SkArgs ga{};
    ga.A = x;
    ga.lda = D;
    ga.M = M;
    ga.K = D;
    ga.Bp = bp;
    ga.n_groups = n_kv;
    ga.eps = c.rms_eps;
    ga.part = at<float>(ws, w.part);
    const SkPlan p = sk_plan(M, D, n_kv, true);
    ga.splits = p.splits;
    ga.counters = at<unsigned>(ws, w.ctr_qkv);
    EpiQkvS e{nullptr, kn, vn, 0, at<float>(packed, lay.rope_cos), at<float>(packed, lay.rope_sin),
              T, P, Hq, Hkv, d, g_kv};
    launch_sk_qkv(ga, p.gpw, true, e, st);
    return;
  }
  bf16_t* a = at<bf16_t>(ws, w.a);
  float* r1 = at<float>(ws, w.r1);
  launch_rms_rows(x, M, D, false, c.rms_eps, r1, a, st);
  GemmArgs ga{};
  ga.A = a;
  ga.lda = D;
  ga.M = M;
  ga.K = D;
  ga.Bp = bp;
  ga.n_groups = n_kv;
  ga.r = r1;
  ga.part = at<float>(ws, w.big_part);
  ga.ctr = at<unsigned>(ws, w.big_ctr);
  EpiQKV e{nullptr, kn, vn, 0, at<float>(packed, lay.rope_cos), at<float>(packed, lay.rope_sin),
           T, P, Hq, Hkv, d, g_kv};
  launch_gemm_qkv(ga, e, st);
}

// ---------------------------------------------------------------- prefix stage
struct PrefillWs {
  BlockWs blk;
  size_t h0, h1, total;
};

PrefillWs prefill_ws_layout(const blk_config& c, int T) {
  PrefillWs f;
  size_t off = kSync.total;
  f.h0 = off;   // hidden states between layers, row-major [T][D]
  off += align_up((size_t)T * c.hidden * 2);
  f.h1 = off;
  off += align_up((size_t)T * c.hidden * 2);
  f.blk = block_ws_layout(c, 1, T, 0, off);
  f.total = f.blk.total;
  return f;
}

// ---------------------------------------------------------------- flow workspace + driver
struct FlowWs {
  BlockWs blk;
  size_t x0, x1, z, kn, vn, total;
};

FlowWs flow_ws_layout(const blk_config& c, int N, int P) {
  FlowWs f;
  const int T = N + 1;
  const size_t D = c.hidden;
  size_t off = kSync.total;
  // X and z rows in operand order, padded to 16-row tiles
  f.x0 = off;
  off += align_up((size_t)16 * mt_of(T) * D * 2);
  f.x1 = off;
  off += align_up((size_t)16 * mt_of(T) * D * 2);
  f.z = off;
  off += align_up((size_t)16 * mt_of(T) * D * 2);   // row tiles of X (>= those of z's N rows)
  f.kn = off;
  off += align_up((size_t)T * c.n_kv_heads * c.head_dim * 2);
  f.vn = off;
  off += align_up((size_t)T * c.n_kv_heads * c.head_dim * 2);
  // the embedding's W3 GEMM (N rows, K = D, D/32 groups) shares the split-K scratch
  f.blk = block_ws_layout(c, 1, T, P, off, sk_part_floats(N, (int)D, (int)D / 32, false));
  f.total = f.blk.total;
  return f;
}

void enqueue_flow(const blk_config& c, const Layout& lay, const void* packed, int n_layers,
                  int n_steps, int P, const uint16_t* const* kp, const uint16_t* const* vp,
                  const float* noise, const float* state, float* actions, void* ws,
                  const FlowWs& fw, hipStream_t st) {
  const int N = lay.n_actions, A = lay.action_dim, D = c.hidden, T = N + 1;
  bf16_t* X[2] = {at<bf16_t>(ws, fw.x0), at<bf16_t>(ws, fw.x1)};
  bf16_t* z = at<bf16_t>(ws, fw.z);
  for (int s = 0; s < n_steps; ++s) {
    const float* a_in = s == 0 ? noise : actions;
    FlowEmbedArgs ea{a_in,
                     state,
                     at<float>(packed, lay.h_wfused),
                     at<float>(packed, lay.h_table) + (size_t)s * D,
                     at<float>(packed, lay.h_ws),
                     at<float>(packed, lay.h_bs),
                     z,
                     X[0],
                     N,
                     A,
                     D};
    launch_flow_embed(ea, st);
    {
      SkArgs ga{};
      ga.A = z;
      ga.M = N;
      ga.K = D;
      ga.Bp = at<uint8_t>(packed, lay.h_w3);
      ga.n_groups = D / 32;
      const SkPlan p = sk_plan(N, D, ga.n_groups, false);
      ga.splits = p.splits;
      ga.part = at<float>(ws, fw.blk.part);
      ga.counters = at<unsigned>(ws, fw.blk.ctr_o);  // W3 has W_o's group count (D / 32)
      EpiResidS e{nullptr, 0, 0, at<float>(packed, lay.h_b3), X[0], 1, mt_of(T), 1, D};
      launch_sk_resid(ga, p.gpw, e, st);
    }
    int cur = 0;
    for (int l = 0; l < n_layers; ++l) {
      BlockIO io{X[cur],  kp[l],  vp[l], 0, X[cur ^ 1], at<bf16_t>(ws, fw.kn),
                 at<bf16_t>(ws, fw.vn), 0};
      const uint8_t* next_qkv =
          l + 1 < n_layers ? at<uint8_t>(packed, lay.layer0 + (size_t)(l + 1) * lay.layer_bytes + lay.wqkv)
                           : nullptr;
      enqueue_block_small(c, lay, packed, l, 1, T, P, io, true, true, ws, fw.blk, st, true, next_qkv);
      cur ^= 1;
    }
    FlowVelArgs va{X[cur],
                   at<float>(packed, lay.h_wout),
                   at<float>(packed, lay.h_bout),
                   a_in,
                   actions,
                   at<float>(packed, lay.h_dt) + s,
                   N,
                   A,
                   D,
                   c.rms_eps};
    launch_flow_velocity(va, st);
  }
}

// ---------------------------------------------------------------- graph cache
struct GraphKey {
  int device;
  const void* packed;
  int n_layers, n_steps, P;
  std::vector<const void*> ptrs;
  blk_config cfg;
  bool operator<(const GraphKey& o) const {
    if (device != o.device) return device < o.device;
    if (packed != o.packed) return packed < o.packed;
    if (n_layers != o.n_layers) return n_layers < o.n_layers;
    if (n_steps != o.n_steps) return n_steps < o.n_steps;
    if (P != o.P) return P < o.P;
    if (ptrs != o.ptrs) return ptrs < o.ptrs;
    return std::memcmp(&cfg, &o.cfg, sizeof cfg) < 0;
  }
};

struct GraphEntry {
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
};

std::mutex g_graph_mu;
std::map<GraphKey, GraphEntry> g_graphs;
constexpr size_t kMaxGraphs = 16;

void destroy_entry(GraphEntry& e) {
  if (e.exec) (void)hipGraphExecDestroy(e.exec);
  if (e.graph) (void)hipGraphDestroy(e.graph);
  e.exec = nullptr;
  e.graph = nullptr;
}

// ---------------------------------------------------------------- block entry helpers
// Shape checks that precede the workspace layout.
int forward_shape_checks(const blk_config* cfg, int batch, int tokens, int prefix) {
  int rc = check_config(cfg);
  if (rc) return rc;
  if (batch < 0 || tokens < 0 || prefix < 0) return fail(BLK_EINVAL, "negative batch/tokens/prefix");
  if ((long)prefix + tokens > cfg->max_pos)
    return fail(BLK_EUNSUPPORTED, "prefix + tokens = %ld exceeds max_pos %d",
                (long)prefix + tokens, cfg->max_pos);
  if ((long)batch * tokens > (1L << 24)) return fail(BLK_EUNSUPPORTED, "batch * tokens too large");
  // the large-chunk kernels address an activation matrix with 32-bit byte offsets
  const long widest = std::max({(long)cfg->hidden, (long)cfg->ffn, (long)cfg->n_q_heads * cfg->head_dim});
  if ((long)batch * tokens * widest > (1L << 30))
    return fail(BLK_EUNSUPPORTED, "batch * tokens * max(hidden, ffn, Hq d) exceeds 2^30");
  return BLK_OK;
}

// The remaining argument checks; *nothing = true for an empty chunk.
int forward_arg_checks(const blk_config* cfg, const void* packed, int layer, int batch, int tokens,
                       int prefix, const uint16_t* x, const uint16_t* k_prefix,
                       const uint16_t* v_prefix, int64_t prefix_stride, uint16_t* y,
                       uint16_t* k_new, uint16_t* v_new, int64_t new_stride, PackRecord* rec,
                       bool* nothing) {
  *nothing = false;
  if (!packed) return fail(BLK_EINVAL, "packed is NULL");
  int rc = lookup(packed, *cfg, rec);
  if (rc) return rc;
  if (layer < 0 || layer >= rec->lay.n_layers)
    return fail(BLK_EINVAL, "layer %d out of range [0, %d)", layer, rec->lay.n_layers);
  if (batch == 0 || tokens == 0) {
    *nothing = true;
    return BLK_OK;
  }
  if (!x || !y || !k_new || !v_new) return fail(BLK_EINVAL, "x, y, k_new and v_new must be non-NULL");
  if (prefix > 0 && (!k_prefix || !v_prefix)) return fail(BLK_EINVAL, "prefix K/V is NULL with prefix > 0");
  for (const void* p : {(const void*)x, (const void*)y, (const void*)k_new, (const void*)v_new,
                        (const void*)k_prefix, (const void*)v_prefix})
    if (reinterpret_cast<uintptr_t>(p) % 16 != 0)
      return fail(BLK_EINVAL, "x, y, k_new, v_new, k_prefix and v_prefix must be 16-byte aligned");
  if (prefix_stride % 8 != 0 || new_stride % 8 != 0)
    return fail(BLK_EINVAL, "prefix_stride and new_stride must be multiples of 8 elements");
  const int64_t kvrow = (int64_t)cfg->n_kv_heads * cfg->head_dim;
  if (batch > 1) {
    // prefix_stride 0: every stream reads one shared prefix (read only)
    if (prefix > 0 && prefix_stride != 0 && prefix_stride < (int64_t)prefix * kvrow)
      return fail(BLK_EINVAL, "prefix_stride is neither 0 (shared) nor at least one stream's prefix");
    if (new_stride < (int64_t)tokens * kvrow)
      return fail(BLK_EINVAL, "new_stride smaller than one stream's tokens");
  }
  if (batch * tokens <= kSkinnyMaxM && !small_plan_ok(*cfg, batch * tokens, true))
    return fail(BLK_EUNSUPPORTED, "hidden %d too wide for a %d-row chunk", cfg->hidden, batch * tokens);
  return BLK_OK;
}

// Enqueues one validated block stage on `st` with workspace ws (layout w).
// `timing`: whether operator timing (when on) may record events.
int forward_enqueue(const blk_config& c, const PackRecord& rec, const void* packed, int layer,
                    int batch, int tokens, int prefix, const uint16_t* x, const uint16_t* k_prefix,
                    const uint16_t* v_prefix, int64_t prefix_stride, uint16_t* y, uint16_t* k_new,
                    uint16_t* v_new, int64_t new_stride, void* ws, const BlockWs& w,
                    hipStream_t st, bool timing, const int32_t* prefix_lens = nullptr) {
  std::unique_lock<std::mutex> tlk(g_timer_mu, std::defer_lock);
  if (timing && g_timer.on) {
    tlk.lock();
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    HIP_TRY(hipStreamIsCapturing(st, &cs));
    if (cs != hipStreamCaptureStatusNone)
      return fail(BLK_ESTATE, "operator timing is on while the stream is being captured");
    if (g_timer.used + BLK_N_OPS + 1 > kTimerMaxEvents)
      return fail(BLK_ESIZE, "operator timing holds %zu events; read them with blk_operator_times",
                  kTimerMaxEvents);
    HIP_TRY(timer_event(st, &g_mark_prev));
    g_mark_stream = st;
    g_marking = true;
  }
  struct MarkReset {
    ~MarkReset() { g_marking = false; }
  } mark_reset;
  (void)hipGetLastError();
  if (prefix_lens && g_exec_mode == 2)
    return fail(BLK_EUNSUPPORTED, "per-stream prefix lengths run on the per-operator kernels only");
  if (!prefix_lens && want_persistent()) {
    StageArgs sa{};
    const int nwg = stage_grid(c.head_dim, batch * tokens);
    if (stage_plan(c, batch, tokens, prefix, 0, nwg, sa)) {
      stage_fill_common(sa, rec.lay, packed, ws, w);
      sa.flow = 0;
      sa.n_layers = 1;
      sa.layer_first = layer;
      sa.n_steps = 1;
      sa.x = x;
      sa.y = y;
      sa.kn = k_new;
      sa.vn = v_new;
      sa.new_stride = new_stride;
      sa.kp[0] = k_prefix;
      sa.vp[0] = v_prefix;
      sa.prefix_stride = prefix_stride;
      HIP_TRY(launch_stage(sa, nwg, st));
      op_done(BLK_OP_STAGE);
      return BLK_OK;
    }
    if (g_exec_mode == 2) return fail(BLK_EUNSUPPORTED, "the persistent stage kernel does not cover this shape");
  }
  BlockIO io{x, k_prefix, v_prefix, prefix_stride, y, k_new, v_new, new_stride, prefix_lens};
  enqueue_block(c, rec.lay, packed, layer, batch, tokens, prefix, io, ws, w, st);
  HIP_TRY(hipGetLastError());
  return BLK_OK;
}

// ---------------------------------------------------------------- static scratch
// For callers that cannot allocate (code under graph capture, tight serving
// loops): blk_forward_noalloc's workspace is this file-scope array, one copy
// per GPU, held until the process ends.  Host code never passes `scratch`
// itself to a kernel (on the host it is a stand-in symbol, not a device
// address): the device address comes from hipGetSymbolAddress, once per device.
constexpr size_t kScratchBytes = size_t(16) << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];
static_assert(kScratchBytes == BLK_NOALLOC_SCRATCH_BYTES, "blk.h states the scratch size");

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

__global__ void zero_words_kernel(uint32_t* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

// Device address of the current device's scratch; its first use on a device
// also enqueues (on st) a fill kernel that zeroes the sync region.
int scratch_for_current_device(hipStream_t st, void** out) {
  int dev = 0;
  HIP_TRY(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return fail(BLK_EUNSUPPORTED, "device %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    HIP_TRY(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)));
    if (!ptr) return fail(BLK_EHIP, "hipGetSymbolAddress returned NULL for the scratch array");
    (void)hipGetLastError();
    zero_words_kernel<<<(unsigned)((kSync.total / 4 + 255) / 256), 256, 0, st>>>(
        reinterpret_cast<uint32_t*>(ptr), kSync.total / 4);
    HIP_TRY(hipGetLastError());
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return BLK_OK;
}

}  // namespace

// ============================================================================ exports
extern "C" {

const char* blk_last_error(void) { return g_err.c_str(); }

int blk_version(void) { return 1; }

int blk_set_execution_mode(int mode) {
  g_err.clear();
  if (mode < 0 || mode > 2) return fail(BLK_EINVAL, "execution mode %d not in {0, 1, 2}", mode);
  g_exec_mode = mode;
  return BLK_OK;
}

int blk_workspace_status(const void* ws, void* stream) {
  g_err.clear();
  if (!ws) return fail(BLK_EINVAL, "ws is NULL");
  HIP_TRY(hipStreamSynchronize((hipStream_t)stream));
  unsigned word = 0;
  HIP_TRY(hipMemcpy(&word, at<unsigned>(ws, BLK_WS_ABORT_OFFSET), sizeof word, hipMemcpyDeviceToHost));
  if (word != 0u)
    return fail(BLK_EABORTED,
                "a persistent launch on this workspace timed out waiting for other workgroups "
                "(its outputs hold NaN); zero-fill the workspace to use it again");
  return BLK_OK;
}

int blk_set_operator_timing(int enable) {
  g_err.clear();
  if (enable != 0 && enable != 1) return fail(BLK_EINVAL, "enable %d not in {0, 1}", enable);
  std::lock_guard<std::mutex> lk(g_timer_mu);
  g_timer.on = enable == 1;
  g_timer.used = 0;
  g_timer.recs.clear();
  for (int i = 0; i < BLK_N_OPS; ++i) {
    g_timer.sum_ms[i] = 0.0;
    g_timer.calls[i] = 0;
  }
  return BLK_OK;
}

int blk_operator_times(double* avg_us, int* calls, int n) {
  g_err.clear();
  if (n < 0 || (n > 0 && (!avg_us || !calls))) return fail(BLK_EINVAL, "avg_us / calls NULL or n < 0");
  std::lock_guard<std::mutex> lk(g_timer_mu);
  if (!g_timer.recs.empty()) HIP_TRY(hipEventSynchronize(g_timer.pool[g_timer.recs.back().e1]));
  for (const auto& r : g_timer.recs) {
    float ms = 0.f;
    HIP_TRY(hipEventElapsedTime(&ms, g_timer.pool[r.e0], g_timer.pool[r.e1]));
    g_timer.sum_ms[r.op] += ms;
    g_timer.calls[r.op] += 1;
  }
  g_timer.recs.clear();
  g_timer.used = 0;
  for (int i = 0; i < n && i < BLK_N_OPS; ++i) {
    calls[i] = g_timer.calls[i];
    avg_us[i] = g_timer.calls[i] ? 1e3 * g_timer.sum_ms[i] / g_timer.calls[i] : 0.0;
  }
  return BLK_OK;
}

void blk_release(void) {
  {
    std::lock_guard<std::mutex> lk(g_graph_mu);
    for (auto& kv : g_graphs) destroy_entry(kv.second);
    g_graphs.clear();
  }
  std::lock_guard<std::mutex> lk(g_mu);
  g_packs.clear();
}

int blk_prepare_weights(const blk_config* cfg, const blk_layer_src* layers, int n_layers,
                        const blk_flow_head_src* head, const double* t_schedule, int n_steps,
                        void* dst, size_t* bytes, void* stream) {
  g_err.clear();
  int rc = check_config(cfg);
  if (rc) return rc;
  if (!bytes) return fail(BLK_EINVAL, "bytes is NULL");
  if (n_layers < 0) return fail(BLK_EINVAL, "n_layers < 0");
  if (n_layers > 0 && !layers) return fail(BLK_EINVAL, "layers is NULL");
  int N = 0, A = 0;
  if (head) {
    N = head->n_actions;
    A = head->action_dim;
    if (N <= 0 || N + 1 > kSkinnyMaxM)
      return fail(BLK_EUNSUPPORTED, "n_actions %d must be in [1, %d]", N, kSkinnyMaxM - 1);
    if (A <= 0 || A > 64) return fail(BLK_EUNSUPPORTED, "action_dim %d must be in [1, 64]", A);
    if (cfg->hidden > 8192) return fail(BLK_EUNSUPPORTED, "flow head needs hidden <= 8192");
    if (n_steps <= 0 || n_steps > kMaxSteps)
      return fail(BLK_EUNSUPPORTED, "n_steps %d must be in [1, %d]", n_steps, kMaxSteps);
    if (!t_schedule) return fail(BLK_EINVAL, "t_schedule is NULL");
    for (int s = 0; s < n_steps; ++s)
      if (!std::isfinite(t_schedule[s])) return fail(BLK_EINVAL, "t_schedule[%d] is not finite", s);
    const void* hp[] = {head->w1, head->b1, head->w2, head->b2, head->w3, head->b3, head->ws,
                        head->bs, head->g_f, head->w_out, head->b_out};
    for (const void* p : hp)
      if (!p) return fail(BLK_EINVAL, "a flow head pointer is NULL");
  }
  const Layout lay = make_layout(*cfg, n_layers, head != nullptr, n_steps, N, A);
  if (!dst) {
    *bytes = lay.total;
    return BLK_OK;
  }
  if (*bytes < lay.total)
    return fail(BLK_ESIZE, "dst has %zu bytes, %zu needed", *bytes, lay.total);
  for (int l = 0; l < n_layers; ++l) {
    const blk_layer_src& s = layers[l];
    const void* lp[] = {s.g_attn, s.w_q, s.w_k, s.w_v, s.w_o, s.g_ffn, s.w_gate, s.w_up, s.w_down};
    for (const void* p : lp)
      if (!p) return fail(BLK_EINVAL, "layer %d has a NULL pointer", l);
  }

  hipStream_t st = (hipStream_t)stream;
  const blk_config& c = *cfg;
  const int D = c.hidden, F = c.ffn, d = c.head_dim, Hq = c.n_q_heads, Hkv = c.n_kv_heads;
  uint8_t* base = reinterpret_cast<uint8_t*>(dst);
  (void)hipGetLastError();
  launch_rope_table(c.max_pos, d / 2, (double)c.rope_base, at<float>(dst, lay.rope_cos),
                    at<float>(dst, lay.rope_sin), st);
  for (int l = 0; l < n_layers; ++l) {
    const blk_layer_src& s = layers[l];
    uint8_t* lw = base + lay.layer0 + (size_t)l * lay.layer_bytes;
    {
      PackSrc ps{{(const bf16_t*)s.w_q, (const bf16_t*)s.w_k, (const bf16_t*)s.w_v},
                 {Hq * d, Hkv * d, Hkv * d},
                 3,
                 s.g_attn};
      ColMapArgs cm{kColRopePairs, d, (Hq + Hkv) * d, 0};
      launch_pack_frag(ps, cm, D, (Hq + 2 * Hkv) * d / 32, lw + lay.wqkv, st);
    }
    {
      PackSrc ps{{(const bf16_t*)s.w_o, nullptr, nullptr}, {D, 0, 0}, 1, nullptr};
      ColMapArgs cm{kColPlain, d, 0, 0};
      launch_pack_frag(ps, cm, Hq * d, D / 32, lw + lay.wo, st);
    }
    {
      PackSrc ps{{(const bf16_t*)s.w_gate, (const bf16_t*)s.w_up, nullptr}, {F, F, 0}, 2, s.g_ffn};
      ColMapArgs cm{kColGateUp, d, 0, F};
      launch_pack_frag(ps, cm, D, F / 16, lw + lay.wgu, st);
    }
    {
      PackSrc ps{{(const bf16_t*)s.w_down, nullptr, nullptr}, {D, 0, 0}, 1, nullptr};
      ColMapArgs cm{kColPlain, d, 0, 0};
      launch_pack_frag(ps, cm, F, D / 32, lw + lay.wd, st);
    }
  }
  if (head) {
    launch_fold_action((const bf16_t*)head->w1, (const bf16_t*)head->w2, A, D,
                       at<float>(dst, lay.h_wfused), st);
    Schedule sched{};
    sched.n = n_steps;
    for (int s = 0; s < n_steps; ++s) sched.t[s] = t_schedule[s];
    launch_fold_time(head->b1, (const bf16_t*)head->w2, head->b2, D, sched,
                     at<float>(dst, lay.h_table), at<float>(dst, lay.h_dt), st);
    PackSrc ps{{(const bf16_t*)head->w3, nullptr, nullptr}, {D, 0, 0}, 1, nullptr};
    ColMapArgs cm{kColPlain, d, 0, 0};
    launch_pack_frag(ps, cm, D, D / 32, base + lay.h_w3, st);
    launch_copy_f32(head->b3, D, at<float>(dst, lay.h_b3), st);
    launch_widen((const bf16_t*)head->ws, nullptr, D, (size_t)A * D, at<float>(dst, lay.h_ws), st);
    launch_copy_f32(head->bs, D, at<float>(dst, lay.h_bs), st);
    launch_widen((const bf16_t*)head->w_out, head->g_f, A, (size_t)D * A,
                 at<float>(dst, lay.h_wout), st);
    launch_copy_f32(head->b_out, A, at<float>(dst, lay.h_bout), st);
  }
  HIP_TRY(hipGetLastError());
  std::lock_guard<std::mutex> lk(g_mu);
  g_packs[dst] = PackRecord{c, lay};
  return BLK_OK;
}

int blk_forward(const blk_config* cfg, const void* packed, int layer, int batch, int tokens,
                int prefix, const uint16_t* x, const uint16_t* k_prefix,
                const uint16_t* v_prefix, int64_t prefix_stride, uint16_t* y, uint16_t* k_new,
                uint16_t* v_new, int64_t new_stride, void* ws, size_t* ws_bytes, void* stream) {
  g_err.clear();
  int rc = forward_shape_checks(cfg, batch, tokens, prefix);
  if (rc) return rc;
  if (!ws_bytes) return fail(BLK_EINVAL, "ws_bytes is NULL");
  const BlockWs w = block_ws_layout(*cfg, batch, tokens, prefix, 0);
  if (!ws) {
    *ws_bytes = w.total;
    return BLK_OK;
  }
  if (*ws_bytes < w.total) return fail(BLK_ESIZE, "ws has %zu bytes, %zu needed", *ws_bytes, w.total);
  PackRecord rec;
  bool nothing = false;
  rc = forward_arg_checks(cfg, packed, layer, batch, tokens, prefix, x, k_prefix, v_prefix,
                          prefix_stride, y, k_new, v_new, new_stride, &rec, &nothing);
  if (rc || nothing) return rc;
  return forward_enqueue(*cfg, rec, packed, layer, batch, tokens, prefix, x, k_prefix, v_prefix,
                         prefix_stride, y, k_new, v_new, new_stride, ws, w, (hipStream_t)stream,
                         true);
}

int blk_forward_chunks(const blk_config* cfg, const void* packed, int layer, int batch,
                       int tokens, int prefix, const int32_t* prefix_lens, const uint16_t* x,
                       const uint16_t* k_prefix, const uint16_t* v_prefix, int64_t prefix_stride,
                       uint16_t* y, uint16_t* k_new, uint16_t* v_new, int64_t new_stride, void* ws,
                       size_t* ws_bytes, void* stream) {
  g_err.clear();
  int rc = forward_shape_checks(cfg, batch, tokens, prefix);
  if (rc) return rc;
  if (!ws_bytes) return fail(BLK_EINVAL, "ws_bytes is NULL");
  if (batch > kMaxVarStreams)
    return fail(BLK_EUNSUPPORTED, "batch %d exceeds %d streams with their own prefix lengths", batch,
                kMaxVarStreams);
  const BlockWs w = block_ws_layout(*cfg, batch, tokens, prefix, 0);
  if (!ws) {
    *ws_bytes = w.total;
    return BLK_OK;
  }
  if (*ws_bytes < w.total) return fail(BLK_ESIZE, "ws has %zu bytes, %zu needed", *ws_bytes, w.total);
  if (batch > 0 && !prefix_lens) return fail(BLK_EINVAL, "prefix_lens is NULL");
  for (int b = 0; b < batch; ++b)
    if (prefix_lens[b] < 0 || prefix_lens[b] > prefix)
      return fail(BLK_EINVAL, "prefix_lens[%d] = %d outside [0, %d]", b, prefix_lens[b], prefix);
  PackRecord rec;
  bool nothing = false;
  rc = forward_arg_checks(cfg, packed, layer, batch, tokens, prefix, x, k_prefix, v_prefix,
                          prefix_stride, y, k_new, v_new, new_stride, &rec, &nothing);
  if (rc || nothing) return rc;
  return forward_enqueue(*cfg, rec, packed, layer, batch, tokens, prefix, x, k_prefix, v_prefix,
                         prefix_stride, y, k_new, v_new, new_stride, ws, w, (hipStream_t)stream,
                         true, prefix_lens);
}

int blk_forward_noalloc(const blk_config* cfg, const void* packed, int layer, int batch,
                        int tokens, int prefix, const uint16_t* x, const uint16_t* k_prefix,
                        const uint16_t* v_prefix, int64_t prefix_stride, uint16_t* y,
                        uint16_t* k_new, uint16_t* v_new, int64_t new_stride, void* stream) {
  g_err.clear();
  int rc = forward_shape_checks(cfg, batch, tokens, prefix);
  if (rc) return rc;
  const BlockWs w = block_ws_layout(*cfg, batch, tokens, prefix, 0);
  if (w.total > kScratchBytes)
    return fail(BLK_ESIZE, "the stage needs %zu bytes of scratch; the library's static scratch holds %zu",
                w.total, kScratchBytes);
  PackRecord rec;
  bool nothing = false;
  rc = forward_arg_checks(cfg, packed, layer, batch, tokens, prefix, x, k_prefix, v_prefix,
                          prefix_stride, y, k_new, v_new, new_stride, &rec, &nothing);
  if (rc || nothing) return rc;
  hipStream_t st = (hipStream_t)stream;
  void* ws = nullptr;
  rc = scratch_for_current_device(st, &ws);
  if (rc) return rc;
  return forward_enqueue(*cfg, rec, packed, layer, batch, tokens, prefix, x, k_prefix, v_prefix,
                         prefix_stride, y, k_new, v_new, new_stride, ws, w, st, false);
}

int prefix_prefill(const blk_config* cfg, const void* packed, int n_layers, int tokens,
                   const uint16_t* x, uint16_t* const* k_cache, uint16_t* const* v_cache, void* ws,
                   size_t* ws_bytes, void* stream) {
  g_err.clear();
  int rc = forward_shape_checks(cfg, 1, tokens, 0);
  if (rc) return rc;
  if (!ws_bytes) return fail(BLK_EINVAL, "ws_bytes is NULL");
  if (n_layers <= 0 || tokens <= 0) return fail(BLK_EINVAL, "n_layers and tokens must be > 0");
  const PrefillWs pw = prefill_ws_layout(*cfg, tokens);
  if (!ws) {
    *ws_bytes = pw.total;
    return BLK_OK;
  }
  if (*ws_bytes < pw.total) return fail(BLK_ESIZE, "ws has %zu bytes, %zu needed", *ws_bytes, pw.total);
  if (!packed) return fail(BLK_EINVAL, "packed is NULL");
  PackRecord rec;
  rc = lookup(packed, *cfg, &rec);
  if (rc) return rc;
  if (n_layers > rec.lay.n_layers)
    return fail(BLK_EINVAL, "n_layers %d exceeds the %d prepared layers", n_layers, rec.lay.n_layers);
  if (!x || !k_cache || !v_cache) return fail(BLK_EINVAL, "x, k_cache and v_cache must be non-NULL");
  if (reinterpret_cast<uintptr_t>(x) % 16) return fail(BLK_EINVAL, "x must be 16-byte aligned");
  for (int l = 0; l < n_layers; ++l) {
    if (!k_cache[l] || !v_cache[l]) return fail(BLK_EINVAL, "cache pointer of layer %d is NULL", l);
    if (reinterpret_cast<uintptr_t>(k_cache[l]) % 16 || reinterpret_cast<uintptr_t>(v_cache[l]) % 16)
      return fail(BLK_EINVAL, "cache buffers must be 16-byte aligned");
  }
  if (tokens <= kSkinnyMaxM && !small_plan_ok(*cfg, tokens, true))
    return fail(BLK_EUNSUPPORTED, "hidden %d too wide for a %d-row chunk", cfg->hidden, tokens);
  hipStream_t st = (hipStream_t)stream;
  (void)hipGetLastError();
  bf16_t* h[2] = {at<bf16_t>(ws, pw.h0), at<bf16_t>(ws, pw.h1)};
  const bf16_t* in = reinterpret_cast<const bf16_t*>(x);
  for (int l = 0; l + 1 < n_layers; ++l) {
    BlockIO io{in, nullptr, nullptr, 0, h[l & 1], k_cache[l], v_cache[l], 0};
    enqueue_block(*cfg, rec.lay, packed, l, 1, tokens, 0, io, ws, pw.blk, st, true);
    in = h[l & 1];
  }
  enqueue_kv_only(*cfg, rec.lay, packed, n_layers - 1, tokens, 0, in, k_cache[n_layers - 1],
                  v_cache[n_layers - 1], ws, pw.blk, st);
  HIP_TRY(hipGetLastError());
  return BLK_OK;
}

int flow_denoise(const blk_config* cfg, const void* packed, int n_layers, int n_steps, int prefix,
                 const uint16_t* const* k_prefix, const uint16_t* const* v_prefix,
                 const float* noise, const float* state, float* actions, void* ws,
                 size_t* ws_bytes, void* stream) {
  g_err.clear();
  int rc = check_config(cfg);
  if (rc) return rc;
  if (!ws_bytes) return fail(BLK_EINVAL, "ws_bytes is NULL");
  if (!packed) return fail(BLK_EINVAL, "packed is NULL");
  if (prefix < 0 || n_layers <= 0 || n_steps <= 0)
    return fail(BLK_EINVAL, "prefix must be >= 0, n_layers and n_steps > 0");
  PackRecord rec;
  rc = lookup(packed, *cfg, &rec);
  if (rc) return rc;
  const Layout& lay = rec.lay;
  if (!lay.has_head) return fail(BLK_ESTATE, "packed buffer has no flow head");
  if (n_steps != lay.n_steps)
    return fail(BLK_ESTATE, "n_steps %d differs from the prepared schedule's %d", n_steps, lay.n_steps);
  if (n_layers > lay.n_layers)
    return fail(BLK_EINVAL, "n_layers %d exceeds the %d prepared layers", n_layers, lay.n_layers);
  const int T = lay.n_actions + 1;
  if ((long)prefix + T > cfg->max_pos)
    return fail(BLK_EUNSUPPORTED, "prefix + %d tokens exceeds max_pos %d", T, cfg->max_pos);
  const FlowWs fw = flow_ws_layout(*cfg, lay.n_actions, prefix);
  if (!ws) {
    *ws_bytes = fw.total;
    return BLK_OK;
  }
  if (*ws_bytes < fw.total) return fail(BLK_ESIZE, "ws has %zu bytes, %zu needed", *ws_bytes, fw.total);
  if (!noise || !state || !actions) return fail(BLK_EINVAL, "noise, state and actions must be non-NULL");
  if (prefix > 0) {
    if (!k_prefix || !v_prefix) return fail(BLK_EINVAL, "k_prefix / v_prefix arrays are NULL");
    for (int l = 0; l < n_layers; ++l)
      if (!k_prefix[l] || !v_prefix[l]) return fail(BLK_EINVAL, "prefix pointer of layer %d is NULL", l);
    for (int l = 0; l < n_layers; ++l)
      if (reinterpret_cast<uintptr_t>(k_prefix[l]) % 16 || reinterpret_cast<uintptr_t>(v_prefix[l]) % 16)
        return fail(BLK_EINVAL, "prefix buffers must be 16-byte aligned");
  }
  if (!small_plan_ok(*cfg, T, false) || sk_plan(lay.n_actions, cfg->hidden, cfg->hidden / 32, false).splits < 1)
    return fail(BLK_EUNSUPPORTED, "hidden %d too wide for the denoise loop", cfg->hidden);
  hipStream_t st = (hipStream_t)stream;
  int dev = 0;
  HIP_TRY(hipGetDevice(&dev));
  GraphKey key;
  key.device = dev;
  key.packed = packed;
  key.n_layers = n_layers;
  key.n_steps = n_steps;
  key.P = prefix;
  key.cfg = *cfg;
  for (int l = 0; l < n_layers; ++l) {
    key.ptrs.push_back(prefix > 0 ? k_prefix[l] : nullptr);
    key.ptrs.push_back(prefix > 0 ? v_prefix[l] : nullptr);
  }
  key.ptrs.push_back(reinterpret_cast<const void*>((uintptr_t)g_exec_mode));
  key.ptrs.push_back(noise);
  key.ptrs.push_back(state);
  key.ptrs.push_back(actions);
  key.ptrs.push_back(ws);

  std::lock_guard<std::mutex> lk(g_graph_mu);
  auto it = g_graphs.find(key);
  if (it == g_graphs.end()) {
    if (g_graphs.size() >= kMaxGraphs) {
      destroy_entry(g_graphs.begin()->second);
      g_graphs.erase(g_graphs.begin());
    }
    std::vector<const uint16_t*> kp(n_layers, nullptr), vp(n_layers, nullptr);
    for (int l = 0; l < n_layers && prefix > 0; ++l) {
      kp[l] = k_prefix[l];
      vp[l] = v_prefix[l];
    }
    hipStream_t cs = nullptr;
    HIP_TRY(hipStreamCreateWithFlags(&cs, hipStreamNonBlocking));
    GraphEntry e;
    (void)hipGetLastError();
    StageArgs sa{};
    const int nwg = want_persistent() ? stage_grid(cfg->head_dim, lay.n_actions + 1) : 0;
    const bool use_stage = nwg > 0 && n_layers <= kStageMaxLayers &&
                           stage_plan(*cfg, 1, lay.n_actions + 1, prefix, lay.n_actions, nwg, sa);
    if (!use_stage && g_exec_mode == 2) {
      (void)hipStreamDestroy(cs);
      return fail(BLK_EUNSUPPORTED, "the persistent stage kernel does not cover this shape");
    }
    if (use_stage) {
      stage_fill_common(sa, lay, packed, ws, fw.blk);
      sa.flow = 1;
      sa.n_layers = n_layers;
      sa.layer_first = 0;
      sa.n_steps = n_steps;
      sa.xb[0] = at<bf16_t>(ws, fw.x0);
      sa.xb[1] = at<bf16_t>(ws, fw.x1);
      sa.kn = at<bf16_t>(ws, fw.kn);
      sa.vn = at<bf16_t>(ws, fw.vn);
      sa.new_stride = 0;
      for (int l = 0; l < n_layers; ++l) {
        sa.kp[l] = kp[l];
        sa.vp[l] = vp[l];
      }
      sa.prefix_stride = 0;
      sa.N = lay.n_actions;
      sa.A = lay.action_dim;
      sa.w_fused = at<float>(packed, lay.h_wfused);
      sa.table = at<float>(packed, lay.h_table);
      sa.dt = at<float>(packed, lay.h_dt);
      sa.w3 = at<uint8_t>(packed, lay.h_w3);
      sa.b3 = at<float>(packed, lay.h_b3);
      sa.ws_f = at<float>(packed, lay.h_ws);
      sa.bs = at<float>(packed, lay.h_bs);
      sa.w_out = at<float>(packed, lay.h_wout);
      sa.b_out = at<float>(packed, lay.h_bout);
      sa.noise = noise;
      sa.state = state;
      sa.actions = actions;
      sa.z = at<bf16_t>(ws, fw.z);
    }
    hipError_t err = hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal);
    if (err == hipSuccess) {
      if (use_stage) {
        (void)launch_stage(sa, nwg, cs);
      } else {
        enqueue_flow(*cfg, lay, packed, n_layers, n_steps, prefix, kp.data(), vp.data(), noise,
                     state, actions, ws, fw, cs);
      }
      hipError_t launch_err = hipGetLastError();
      err = hipStreamEndCapture(cs, &e.graph);
      if (err == hipSuccess) err = launch_err;
    }
    if (err == hipSuccess) err = hipGraphInstantiate(&e.exec, e.graph, nullptr, nullptr, 0);
    (void)hipStreamDestroy(cs);
    if (err != hipSuccess) {
      destroy_entry(e);
      return fail(BLK_EHIP, "graph capture of the denoise loop failed: %s", hipGetErrorString(err));
    }
    it = g_graphs.emplace(key, e).first;
  }
  HIP_TRY(hipGraphLaunch(it->second.exec, st));
  return BLK_OK;
}

}  // extern "C"
