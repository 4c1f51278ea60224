// Standalone kernels of the small-chunk path (M = B * T <= 64 rows): the
// skinny GEMM with its epilogues and the chunk attention, one launch per
// operator, plus the planners that pick their splits.  The device code lives
// in skinny.h and attn_small.h, shared with the persistent stage kernel.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <type_traits>
#include <cmath>

#include "attn_small.h"
#include "common.h"
#include "internal.h"
#include "skinny.h"

namespace blk {

// ============================================================================ planners
int device_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

// Cost model of a skinny GEMM plan (K splits x 32-column groups per
// workgroup), fitted to a sweep of every (split, groups) plan of the 64-row
// O, down, gate/up and QKV shapes on this chip (within ~0.5 us of each):
//  * one compute unit streams about 90 GB/s of operands;
//  * the activation slab, re-read by every workgroup from L2, is served at
//    about 9.4 TB/s in aggregate;
//  * the weights stream from HBM at about 5 TB/s;
//  * K splits add a hand-off (publish, count, reload in split order) of
//    about 1 us plus 0.35 us per split;
//  * workgroups beyond one per compute unit run in further rounds.
constexpr double kCuBytesPerUs = 90e3, kL2BytesPerUs = 9.4e6, kHbmBytesPerUs = 5e6;
constexpr double kSplitUs = 1.0, kSplitPerUs = 0.35;

SkPlan sk_plan(int M, int K, int n_groups, bool a_rowmajor) {
  (void)a_rowmajor;   // both activation layouts stream alike
  const int KT = K / 32, MT = mt_of(M);
  const int n_cu = device_cus();
  SkPlan best{-1, 1};
  double best_t = 1e30;
  for (int gpw = 1; gpw <= kSkPlanMaxGpw; ++gpw) {
    if (n_groups % gpw != 0) continue;
    for (int s = 1; s <= kSkMaxSplits; s *= 2) {
      if (KT % (4 * s) != 0) break;
      const int n_wg = n_groups / gpw * s;
      if (s > 1 && n_wg > n_cu) break;
      const double per_wg = (double)(2 * gpw + MT) * (KT / s) * kFragBytes;
      const double a_all = (double)n_wg * MT * (KT / s) * kFragBytes;
      const double w_all = 2.0 * n_groups * KT * kFragBytes;
      double t = std::max(per_wg / kCuBytesPerUs, std::max(a_all / kL2BytesPerUs, w_all / kHbmBytesPerUs));
      t *= (n_wg + n_cu - 1) / n_cu;
      if (s > 1) t += kSplitUs + kSplitPerUs * s;
      if (t < best_t - 1e-9) {
        best_t = t;
        best = SkPlan{s, gpw};
      }
    }
  }
  return best;
}

size_t sk_part_floats(int M, int K, int n_groups, bool a_rowmajor) {
  const SkPlan p = sk_plan(M, K, n_groups, a_rowmajor);
  if (p.splits <= 1) return 0;
  return (size_t)p.splits * n_groups * (64 * 32 + 64);
}

// k-tiles in flight per wave: a divisor of the wave's k-tiles, at most
// max_nb, whose loads (2 GPW weight + MT activation fragments per k-tile) fit
// in 192 registers.  A wave issues its whole ring before its first MFMA, so
// a shorter ring starts the k loop's matrix work while later loads are still
// arriving: with the RMS statistic's extra MFMAs a ring of 4 measured faster
// than 8 (64-token QKV 8.94 -> 8.73 us, gate/up 8.85 -> 8.45 us), without it
// 8 (the down projection 9.02 against 9.26 us at 4).
int sk_nb(int KW, int gpw, int MT, int max_nb) {
  for (int nb = max_nb; nb > 1; nb >>= 1)
    if (KW % nb == 0 && nb * (2 * gpw + MT) <= 48) return nb;
  return 1;
}

// Key slices per 64-row block: enough workgroups (about 96) that each takes
// few 64-key steps -- one memory round trip for its K/V -- and the merge
// kernel spreads the combine over every row; slices are whole 64-key tiles
// (multiples of 32 keys, a wave's half of a step, for the shortest runs).
void attn_sm_plan(int B, int T, int P, int Hq, int Hkv, int* splits, int* kps, int* long_rows) {
  const int G = Hq / Hkv;
  const int n_rbt = B * Hkv * ((G * T + 63) / 64);
  const int L = P + T;
  // many 128-row blocks (long chunks): 128 rows per K/V tile, and the number
  // of key slices (each at least 4 tiles) that minimises rounds of the chip's
  // workgroup slots (two per compute unit) x 64-key steps per slice, plus the
  // merge: about a hundredth of a step per block and slice (the batched
  // 8 x 880-token attention took ~100 us longer with 2 slices than with one
  // for 27 fewer steps per slot).  long_rows == NULL: the caller runs 64-row
  // blocks.
  const int n_rbt_long = B * Hkv * ((G * T + 127) / 128);
  if (long_rows) *long_rows = 0;
  if (long_rows && n_rbt_long >= 32) {
    const long slots = 2L * device_cus();
    const int tiles = (L + 63) / 64;
    const int s_max = std::max(1, std::min(kAttnMaxSplits, L / 256));
    int best_kt = tiles;
    double best = 1e30;
    for (int s = 1; s <= s_max; ++s) {
      const int kt = (tiles + s - 1) / s;    // tiles per slice
      const int ns = (tiles + kt - 1) / kt;  // slices this makes
      const long wgs = (long)n_rbt_long * ns;
      const double cost = (double)((wgs + slots - 1) / slots) * kt + (ns > 1 ? 0.01 * (double)wgs : 0.0);
      if (cost < best - 1e-9) {
        best = cost;
        best_kt = kt;
      }
    }
    *kps = best_kt * 64;
    *splits = (L + *kps - 1) / *kps;
    *long_rows = 1;
    return;
  }
  // many 64-row blocks (one workgroup per compute unit at d = 256): the same
  // cost model over one slot per compute unit, plus about three steps for
  // the merge kernel when there are slices (the 768-token prefix attention:
  // 96 blocks in 2 slices of 6 tiles, where the 128-row plan's 3 slices made
  // 288 workgroups, a second round for 32 of them)
  if (n_rbt >= 32) {
    const long slots = device_cus();
    const int tiles = (L + 63) / 64;
    const int s_max = std::max(1, std::min(kAttnMaxSplits, L / 256));
    int best_kt = tiles;
    double best = 1e30;
    for (int s = 1; s <= s_max; ++s) {
      const int kt = (tiles + s - 1) / s;
      const int ns = (tiles + kt - 1) / kt;
      const long wgs = (long)n_rbt * ns;
      const double cost = (double)((wgs + slots - 1) / slots) * kt + (ns > 1 ? 3.0 + 0.01 * (double)wgs : 0.0);
      if (cost < best - 1e-9) {
        best = cost;
        best_kt = kt;
      }
    }
    *kps = best_kt * 64;
    *splits = (L + *kps - 1) / *kps;
    return;
  }
  int s = std::max(1, std::min(kAttnMaxSplits, (96 + n_rbt - 1) / n_rbt));
  s = std::min(s, (L + 31) / 32);
  // up to two 64-key tiles: one workgroup runs both (one more step) rather
  // than slices and the merge kernel's launch
  if (L <= 128) s = 1;
  int k = (L + s - 1) / s;
  if (L > 128) {
    // whole 64-key tiles: a slice of 64 + 32 keys costs a second step for a
    // third more keys (measured at 832 keys: 13 slices of 64 beat 9 of 96)
    int k64 = std::max(64, k / 64 * 64);
    if ((L + k64 - 1) / k64 > kAttnMaxSplits) k64 = (k + 63) / 64 * 64;
    k = k64;
  } else {
    k = (k + 31) / 32 * 32;
  }
  *kps = k;
  *splits = (L + k - 1) / k;
}

// partials of the larger of the two plans (with and without 128-row blocks):
// both index them by 64-row block
size_t attn_sm_part_o_elems(int B, int T, int P, int Hq, int Hkv, int d) {
  int s0 = 1, s1 = 1, k = 32, lr = 0;
  attn_sm_plan(B, T, P, Hq, Hkv, &s0, &k, nullptr);
  attn_sm_plan(B, T, P, Hq, Hkv, &s1, &k, &lr);
  const int s = std::max(s0, s1);
  if (s <= 1) return 0;
  const int n_rbt = B * Hkv * ((Hq / Hkv * T + 63) / 64);
  return (size_t)s * n_rbt * 64 * d;
}
size_t attn_sm_part_ml_floats(int B, int T, int P, int Hq, int Hkv, int d) {
  return attn_sm_part_o_elems(B, T, P, Hq, Hkv, d) / d * 2;
}

// ============================================================================ skinny GEMM
template <int MT, int NB, int GPW, bool RMS, bool AROW, class Epi>
__global__ __launch_bounds__(256) void sk_kernel(SkArgs ga, Epi epi) {
  extern __shared__ __attribute__((aligned(16))) char sk_dsm[];
  // with K splits: tasks in split-major order, a contiguous run of them per
  // XCD (the hardware deals workgroups round-robin over the 8 XCDs), so the
  // workgroups of one XCD read the same K slice of the activations and its
  // L2 fetches that slice alone (64-token O and down: 17 and 20 % fewer bytes
  // fetched; their times within the run-to-run spread).  Without splits the
  // hardware's interleaved order stays (in runs per XCD, the 64-token QKV
  // took 9.13 against 8.74 us).
  int gx = (int)blockIdx.x, split = (int)blockIdx.y;
  if (gridDim.y > 1) {
    const int nx = (int)gridDim.x, n = nx * (int)gridDim.y;
    const int id = gx + split * nx;
    const int xcd = id & 7, jx = id >> 3, qx = n >> 3, rx = n & 7;
    const int task = xcd * qx + min(xcd, rx) + jx;
    split = task / nx;
    gx = task - split * nx;
  }
  sk_task<MT, NB, GPW, RMS, AROW>(ga, epi, gx, split, *reinterpret_cast<SkSmem<AROW, GPW>*>(sk_dsm),
                                  NoWait{});
}

// The same tasks plus a second grid layer of workgroups that prefetch (a
// kernel of its own, so launches without a prefetch keep the plain one).
template <int MT, int NB, int GPW, bool RMS, bool AROW, class Epi>
__global__ __launch_bounds__(256) void sk_pf_kernel(SkArgs ga, Epi epi, Prefetch pf) {
  extern __shared__ __attribute__((aligned(16))) char sk_dsm[];
  if (blockIdx.z != 0) {
    prefetch_range(pf, (int)(blockIdx.x + blockIdx.y * gridDim.x));
    return;
  }
  int gx = (int)blockIdx.x, split = (int)blockIdx.y;
  if (gridDim.y > 1) {
    const int nx = (int)gridDim.x, n = nx * (int)gridDim.y;
    const int id = gx + split * nx;
    const int xcd = id & 7, jx = id >> 3, qx = n >> 3, rx = n & 7;
    const int task = xcd * qx + min(xcd, rx) + jx;
    split = task / nx;
    gx = task - split * nx;
  }
  sk_task<MT, NB, GPW, RMS, AROW>(ga, epi, gx, split, *reinterpret_cast<SkSmem<AROW, GPW>*>(sk_dsm),
                                  NoWait{});
}

template <int MT, int NB, int GPW, bool RMS, bool AROW, class Epi>
static void sk_go(const SkArgs& ga, const Epi& e, hipStream_t st, Prefetch pf) {
  auto kern = sk_kernel<MT, NB, GPW, RMS, AROW, Epi>;
  const size_t smem = sizeof(SkSmem<AROW, GPW>);
  static bool attr_set = false;
  if (!attr_set) {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    attr_set = true;
  }
  const int nx = (ga.n_groups + GPW - 1) / GPW;
  // (only the residual launches prefetch: the denoise loop's down projections)
  if constexpr (std::is_same_v<Epi, EpiResidS>) {
    if (pf.p) {
      auto kp = sk_pf_kernel<MT, NB, GPW, RMS, AROW, Epi>;
      static bool pf_attr_set = false;
      if (!pf_attr_set) {
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kp),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
        pf_attr_set = true;
      }
      pf.wgs = nx * ga.splits;
      hipLaunchKernelGGL(kp, dim3(nx, ga.splits, 2), dim3(256), smem, st, ga, e, pf);
      return;
    }
  }
  hipLaunchKernelGGL(kern, dim3(nx, ga.splits), dim3(256), smem, st, ga, e);
}

template <int MT, int GPW, bool RMS, bool AROW, class Epi>
static void sk_go_nb(const SkArgs& ga, const Epi& e, hipStream_t st, const Prefetch& pf) {
  switch (sk_nb(ga.K / 32 / ga.splits / 4, GPW, MT, RMS ? 4 : 8)) {
    case 8: sk_go<MT, 8, GPW, RMS, AROW>(ga, e, st, pf); break;
    case 4: sk_go<MT, 4, GPW, RMS, AROW>(ga, e, st, pf); break;
    case 2: sk_go<MT, 2, GPW, RMS, AROW>(ga, e, st, pf); break;
    default: sk_go<MT, 1, GPW, RMS, AROW>(ga, e, st, pf); break;
  }
}

template <int MT, bool RMS, bool AROW, class Epi>
static void sk_go_gpw(const SkArgs& ga, int gpw, const Epi& e, hipStream_t st, const Prefetch& pf) {
  if constexpr (kSkPlanMaxGpw >= 2) {
    if (gpw == 2) return sk_go_nb<MT, 2, RMS, AROW>(ga, e, st, pf);
  }
  (void)gpw;
  sk_go_nb<MT, 1, RMS, AROW>(ga, e, st, pf);
}

template <bool RMS, bool AROW, class Epi>
static void sk_launch(const SkArgs& ga, int gpw, const Epi& e, hipStream_t st, const Prefetch& pf = {}) {
  switch (mt_of(ga.M)) {
    case 1: sk_go_gpw<1, RMS, AROW>(ga, gpw, e, st, pf); break;
    case 2: sk_go_gpw<2, RMS, AROW>(ga, gpw, e, st, pf); break;
    case 3: sk_go_gpw<3, RMS, AROW>(ga, gpw, e, st, pf); break;
    default: sk_go_gpw<4, RMS, AROW>(ga, gpw, e, st, pf); break;
  }
}

void launch_sk_qkv(const SkArgs& ga, int gpw, bool a_rowmajor, const EpiQkvS& e, hipStream_t st) {
  if (a_rowmajor) sk_launch<true, true>(ga, gpw, e, st);
  else sk_launch<true, false>(ga, gpw, e, st);
}
void launch_sk_resid(const SkArgs& ga, int gpw, const EpiResidS& e, hipStream_t st, const Prefetch& pf) {
  sk_launch<false, false>(ga, gpw, e, st, pf);
}
void launch_sk_gateup(const SkArgs& ga, int gpw, const EpiGateUpS& e, hipStream_t st) {
  sk_launch<true, false>(ga, gpw, e, st);
}

// ============================================================================ attention
// (128-row mode: registers capped for two workgroups per compute unit)
template <int HD, bool LONG, bool DSPLIT = false>
__global__ __launch_bounds__(256, LONG ? 2 : 1) void attn_sm_kernel(AttnSmArgs a, int n_rb) {
  extern __shared__ __attribute__((aligned(16))) char at_dsm[];
  // Tasks in the order (stream x kv head, key slice, row block), row block
  // fastest; the hardware deals workgroups round-robin over the 8 XCDs, so
  // hand each XCD a contiguous run of tasks: the row blocks that read the
  // same K/V tiles then share one L2.
  const int nwg = gridDim.x, id = blockIdx.x;
  const int xcd = id & 7, jx = id >> 3, qx = nwg >> 3, rx = nwg & 7;
  const int task = xcd * qx + min(xcd, rx) + jx;
  const int rb = task % n_rb, rest = task / n_rb;
  const int ks = rest % a.splits, bh = rest / a.splits;
  attn_sm_task<HD, LONG, DSPLIT>(a, bh, rb, ks, *reinterpret_cast<AttnSmSmem<HD>*>(at_dsm), NoWait{});
}

// The same tasks plus pf.wgs workgroups past them that prefetch (a kernel of
// its own: the extra argument and branch cost the plain launch 0.3 us).
template <int HD, bool LONG, bool DSPLIT = false>
__global__ __launch_bounds__(256, LONG ? 2 : 1) void attn_sm_pf_kernel(AttnSmArgs a, int n_rb, Prefetch pf) {
  extern __shared__ __attribute__((aligned(16))) char at_dsm[];
  const int nwg = (int)gridDim.x - pf.wgs, id = blockIdx.x;
  if (id >= nwg) {
    prefetch_range(pf, id - nwg);
    return;
  }
  const int xcd = id & 7, jx = id >> 3, qx = nwg >> 3, rx = nwg & 7;
  const int task = xcd * qx + min(xcd, rx) + jx;
  const int rb = task % n_rb, rest = task / n_rb;
  const int ks = rest % a.splits, bh = rest / a.splits;
  attn_sm_task<HD, LONG, DSPLIT>(a, bh, rb, ks, *reinterpret_cast<AttnSmSmem<HD>*>(at_dsm), NoWait{});
}

// one wave per workgroup: the merge is a single memory round trip per item,
// spread over as many compute units as there are items
template <int HD>
__global__ __launch_bounds__(64) void attn_combine_kernel(AttnSmArgs a) {
  attn_combine_task<HD>(a, blockIdx.x);
}

template <int HD, bool LONG, bool DSPLIT = false>
static void attn_sm_launch(const AttnSmArgs& a, Prefetch pf, hipStream_t st) {
  const size_t smem = sizeof(AttnSmSmem<HD>);
  const int G = a.Hq / a.Hkv;
  const int n_rb = (G * a.T + (LONG ? 127 : 63)) / (LONG ? 128 : 64);
  const int n_task = a.splits * n_rb * a.B * a.Hkv;
  // prefetch workgroups only on compute units the tasks leave free
  pf.wgs = pf.p ? std::max(0, std::min(pf.wgs, device_cus() - n_task)) : 0;
  if (pf.wgs > 0) {
    auto kern = attn_sm_pf_kernel<HD, LONG, DSPLIT>;
    static bool attr_set = false;
    if (!attr_set) {
      (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
      attr_set = true;
    }
    hipLaunchKernelGGL(kern, dim3(n_task + pf.wgs), dim3(256), smem, st, a, n_rb, pf);
    return;
  }
  auto kern = attn_sm_kernel<HD, LONG, DSPLIT>;
  static bool attr_set = false;
  if (!attr_set) {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    attr_set = true;
  }
  hipLaunchKernelGGL(kern, dim3(n_task), dim3(256), smem, st, a, n_rb);
}

template <int HD>
static void attn_sm_go(const AttnSmArgs& a, const Prefetch& pf, hipStream_t st) {
  // (at HD 256 the 128-row variant spills; 64-row blocks over the one slice)
  bool launched = false;
  if constexpr (HD <= 128) {
    if (a.long_rows) {
      attn_sm_launch<HD, true>(a, pf, st);
      launched = true;
    }
  }
  // 64-row blocks: at d = 256 the waves of a row tile split the output dims
  // (each computes every score; no merge of key halves: the 64-token
  // attention 12.07 -> 11.53 us); at d = 64 duplicating the scores costs more
  // than the merge saves (the 16-token block 17.25 -> 17.42 us)
  if (!launched) {
    if constexpr (HD == 256)
      attn_sm_launch<HD, false, true>(a, pf, st);
    else
      attn_sm_launch<HD, false>(a, pf, st);
  }
  if (a.splits > 1) {
    const int items = attn_combine_items(a.B, a.T, a.Hq, a.Hkv, HD);
    hipLaunchKernelGGL(attn_combine_kernel<HD>, dim3((items + 63) / 64), dim3(64), 0, st, a);
  }
}

void launch_attn_sm(const AttnSmArgs& a, int head_dim, hipStream_t st, const Prefetch& pf) {
  switch (head_dim) {
    case 64: attn_sm_go<64>(a, pf, st); break;
    case 128: attn_sm_go<128>(a, pf, st); break;
    default: attn_sm_go<256>(a, pf, st); break;
  }
}

}  // namespace blk
