// Persistent stage kernel for small chunks (M = B * T <= 64 rows).
//
// [TR] TileRT article: at decode-sized work, kernel launches, cross-kernel
// barriers and memory round trips between operators dominate ("execution
// gaps"); the remedy is one resident kernel that runs the whole operator
// sequence as tile tasks.  [RT] reading note on "Running VLAs at Real-time
// Speed" §3 (graph capture) and §6.2 (the action expert is memory bound).
//
// One launch runs a whole program -- one block stage ([PS] a stage is one
// block at one denoise step), several layers, or the full flow-matching loop
// ([RT] §2: 10 steps x 18 layers plus the suffix embedding and the velocity
// head) -- on one workgroup per compute unit.  Each operator is a phase made of
// independent tasks (the device tasks of skinny.h / attn_small.h, the same
// code the per-operator kernels run):
//   QKV  one or two 32-column groups (x K split) of the fused QKV matrix, RMS + RoPE
//   ATT  one 64-row block x key slice of chunk attention
//   CMB  merge of the key slices (256 output chunks per task), if sliced
//   O    one or two 32-column groups (x K split) of W_o, residual epilogue
//   GU   one or two gate/up groups (x K split), RMS + SiLU-gate epilogue
//   D    one or two 32-column groups (x K split) of W_down, residual epilogue
//   EMB, W3, VEL  the flow head (embedding, its linear, velocity + Euler step)
// Task t of a phase runs on workgroup (w0 + t mod nw); the phases' workgroup
// sets are rotated so that consecutive phases start on different units.
//
// Overlap: a GEMM task issues its weight loads -- at these shapes its whole
// weight slice -- before it waits for the producing phase, and a workgroup
// with no task in a phase moves straight on to the next one, so weight
// streaming of later phases runs under the current one.
//
// Hand-off: a task's outputs are written with device-coherent stores; after
// they are acknowledged the workgroup adds one to an arrival counter of its
// phase type, one of kShards counters (each on its own 128-byte line) picked
// by the task's flag index.  A workgroup entering a phase polls (one wave,
// lane i reads counter i) until each counter of the producing phase type has
// reached (instance number) x (arrivals per instance), which orders every
// phase after all earlier ones.  One counter per task polled by every
// workgroup took 4.7 us per all-to-all step on this chip; 32 sharded counters
// 2.5 us.  Counters start each launch at zero: the last workgroup to finish
// clears them.  Every wait is bounded: on time-out the workgroup raises an
// abort word that all other waits also watch, so the grid always drains; a
// workspace with the abort word set makes later launches return at once.
#include <type_traits>

#include "attn_small.h"
#include "common.h"
#include "internal.h"
#include "skinny.h"
#include "stage.h"

namespace blk {

constexpr unsigned kMaxSpins = 1u << 22;   // ~ seconds of polling (each poll is a memory round trip)

__device__ __forceinline__ unsigned ld_u32c(const unsigned* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_u32c(unsigned* p, unsigned v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Arrival counter `sh` of phase type `type` (kShards per type, 128 bytes apart).
__device__ __forceinline__ unsigned* phase_ctr(unsigned* base, int type, int sh) {
  return base + ((size_t)type * kShards + sh) * kShardWords;
}

// Wave 0 polls the kShards counters of one phase type until counter i holds at
// least inst x (the number of flag indices f < n_flags with f % kShards == i);
// returns false on abort.
__device__ bool wait_counts(unsigned* type_ctrs, int n_flags, unsigned inst, unsigned* abort_word) {
  // (the verdict goes through an LDS word of this function's own, not a
  // pointer to one: the compiler mishandles generic pointers to LDS
  // variables captured in the task lambdas)
  __shared__ int ok_sh;
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    const unsigned per = lane < kShards && n_flags > lane ? (unsigned)((n_flags - lane + kShards - 1) / kShards) : 0u;
    const unsigned want = inst * per;
    const unsigned* ctr = type_ctrs + (size_t)(lane < kShards ? lane : 0) * kShardWords;
    unsigned spins = 0;
    int ok = 1;
    for (;;) {
      const bool ready = want == 0u || ld_u32c(ctr) >= want;
      if (__all(ready)) break;
      if (ld_u32c(abort_word) != 0u) {
        ok = 0;
        break;
      }
      if (++spins > kMaxSpins) {
        if (lane == 0) st_u32c(abort_word, 1u);
        ok = 0;
        break;
      }
    }
    if (lane == 0) ok_sh = ok;
  }
  __syncthreads();
  return ok_sh != 0;
}

// All of this workgroup's task outputs are acknowledged, then count the arrival.
__device__ __forceinline__ void signal_count(unsigned* ctr) {
  wait_stores();
  __syncthreads();
  if (threadIdx.x == 0) __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// An aborted launch writes NaN over its outputs (y, K_new and V_new of a block,
// or the actions of the loop), so that no caller reads stale values as a
// result; every workgroup that sees the abort covers all of them.
__device__ void poison_outputs(const StageArgs& sa) {
  const uint32_t nan2 = 0x7FC07FC0u;   // two bf16 quiet NaNs
  if (sa.flow) {
    const int n = sa.N * sa.A;
    for (int i = threadIdx.x; i < n; i += blockDim.x) sa.actions[i] = __uint_as_float(0x7FC00000u);
    return;
  }
  const size_t ny = (size_t)sa.M * sa.D / 2;
  for (size_t i = threadIdx.x; i < ny; i += blockDim.x) reinterpret_cast<uint32_t*>(sa.y)[i] = nan2;
  const size_t nkv = (size_t)sa.T * sa.Hkv * sa.d / 2;
  for (int b = 0; b < sa.B; ++b)
    for (size_t i = threadIdx.x; i < nkv; i += blockDim.x) {
      reinterpret_cast<uint32_t*>(sa.kn + (size_t)b * sa.new_stride)[i] = nan2;
      reinterpret_cast<uint32_t*>(sa.vn + (size_t)b * sa.new_stride)[i] = nan2;
    }
}

// ---------------------------------------------------------------- flow head tasks
struct FlowSmem {
  float xs[8192];
  float red[256];
  float vin[4][64];
  float wsum[4];
};

// Per-step view of the flow head; z ([N][D]) and X ([N + 1][D]) are in the
// skinny GEMMs' operand order.
struct FlowTask {
  const float* a_in;      // actions at this step's start (noise at step 0)
  const float* state;
  const float* w_fused;   // [A][D] W1 W2a
  const float* bias;      // [D] time table row of this step
  const float* ws_f;      // [A][D]
  const float* bs;
  bf16_t* z;
  bf16_t* x0;             // X (the state token goes to row 0)
  const bf16_t* X;        // output of the last layer
  const float* w_out;     // [D][A] (final gain folded)
  const float* b_out;
  float* actions;         // [N][A]
  float dt;
  int N, A, D;
  int MTz;                // row tiles of z's operand order (those of X, so W3 can share MT)
  float eps;
};

// rows [4t, 4t + 4) of [z rows 0..N-1 ; state row N]
__device__ void emb_task(const FlowTask& f, int t, FlowSmem& fs) {
  const int r0 = 4 * t;
  const int nr = min(4, f.N + 1 - r0);
  const int MTz = f.MTz, MTx = mt_of(f.N + 1);
  __syncthreads();
  for (int i = threadIdx.x; i < nr * f.A; i += 256) {
    const int rr = i / f.A, k = i - rr * f.A;
    const int r = r0 + rr;
    fs.vin[rr][k] = r < f.N ? ld_f32c(f.a_in + (size_t)r * f.A + k) : f.state[k];
  }
  __syncthreads();
  for (int n = threadIdx.x; n < f.D; n += 256) {
    for (int rr = 0; rr < nr; ++rr) {
      const int r = r0 + rr;
      if (r < f.N) {
        float acc = f.bias[n];
        for (int k = 0; k < f.A; ++k) acc = fmaf(fs.vin[rr][k], f.w_fused[(size_t)k * f.D + n], acc);
        st_act(f.z + fa_index(r, n, MTz), silu(acc));
      } else {
        float acc = f.bs[n];
        for (int k = 0; k < f.A; ++k) acc = fmaf(fs.vin[rr][k], f.ws_f[(size_t)k * f.D + n], acc);
        st_act(f.x0 + fa_index(0, n, MTx), acc);
      }
    }
  }
}

// action row i: v = RMS(X[i+1]) . W_out' + b_out; actions[i] = a_in[i] + dt v
__device__ void vel_task(const FlowTask& f, int i, FlowSmem& fs) {
  const int tid = threadIdx.x;
  const int MTx = mt_of(f.N + 1);
  __syncthreads();
  float ss = 0.f;
  for (int k = tid; k < f.D; k += 256) {
    const float v = ld_act(f.X + fa_index(i + 1, k, MTx));
    fs.xs[k] = v;
    ss = fmaf(v, v, ss);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) ss += __shfl_xor(ss, o);
  if ((tid & 63) == 0) fs.wsum[tid >> 6] = ss;
  __syncthreads();
  const float r = rsqrtf(((fs.wsum[0] + fs.wsum[1]) + (fs.wsum[2] + fs.wsum[3])) / (float)f.D + f.eps);
  const int nsl = 256 / f.A;
  const int col = tid % f.A, sl = tid / f.A;
  float acc = 0.f;
  if (sl < nsl) {
    const int kper = (f.D + nsl - 1) / nsl;
    const int k0 = sl * kper, k1 = min(f.D, k0 + kper);
    for (int k = k0; k < k1; ++k) acc = fmaf(fs.xs[k], f.w_out[(size_t)k * f.A + col], acc);
  }
  fs.red[tid] = acc;
  __syncthreads();
  if (tid < f.A) {
    float v = 0.f;
    for (int q = 0; q < nsl; ++q) v += fs.red[q * f.A + tid];
    v = v * r + f.b_out[tid];
    const float a = ld_f32c(f.a_in + (size_t)i * f.A + tid);
    __hip_atomic_store(f.actions + (size_t)i * f.A + tid, a + f.dt * v, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  }
}

// ---------------------------------------------------------------- tasks
// Each task runs in its own (non-inlined) function so that its register
// allocation does not inherit the pressure of the others; it receives small
// argument structs by value (the kernel's large argument block never escapes).
// `wait` performs the wait for the producing phase.  Return: true if this
// workgroup completed the task's outputs (false also when it only published a
// split partial; the phase checks separately whether the grid aborted).

template <int MT, int NB, int GPW, bool RMS, bool AROW, class Epi, class W>
__device__ __noinline__ bool sk_run(SkArgs ga, Epi e, int gb, int s, uint8_t* smem, W& wait) {
  return sk_task<MT, NB, GPW, RMS, AROW>(ga, e, gb, s, *reinterpret_cast<SkSmem<AROW, GPW>*>(smem), wait);
}

template <int MT, int GPW, bool RMS, bool AROW, class Epi, class W>
__device__ __forceinline__ bool sk_dispatch_nb(const SkArgs& ga, const Epi& e, int gb, int s, uint8_t* smem,
                                               W& wait) {
  const int KW = ga.K / 32 / ga.splits / 4;
  constexpr int P = 2 * GPW + MT;   // fragments per k-tile; at most 48 in flight per lane
  if (KW % 8 == 0 && 8 * P <= 48) return sk_run<MT, 8, GPW, RMS, AROW>(ga, e, gb, s, smem, wait);
  if (KW % 4 == 0 && 4 * P <= 48) return sk_run<MT, 4, GPW, RMS, AROW>(ga, e, gb, s, smem, wait);
  if (KW % 2 == 0) return sk_run<MT, 2, GPW, RMS, AROW>(ga, e, gb, s, smem, wait);
  return sk_run<MT, 1, GPW, RMS, AROW>(ga, e, gb, s, smem, wait);
}

// task t of a GEMM phase = (group block t / splits, split t % splits)
template <int MT, bool RMS, bool AROW, class Epi, class W>
__device__ __forceinline__ bool sk_dispatch(const SkArgs& ga, int gpw, const Epi& e, int t, uint8_t* smem,
                                            W& wait) {
  const int gb = t / ga.splits, s = t - gb * ga.splits;
  if constexpr (kSkPlanMaxGpw >= 2) {
    if (gpw == 2) return sk_dispatch_nb<MT, 2, RMS, AROW>(ga, e, gb, s, smem, wait);
  }
  (void)gpw;
  return sk_dispatch_nb<MT, 1, RMS, AROW>(ga, e, gb, s, smem, wait);
}

template <int HD, class W>
__device__ __noinline__ void attn_run(AttnSmArgs aa, int bh, int rb, int ks, uint8_t* smem, W& wait) {
  (void)attn_sm_task<HD>(aa, bh, rb, ks, *reinterpret_cast<AttnSmSmem<HD>*>(smem), wait);
}

template <int HD, class W>
__device__ __noinline__ void cmb_run(AttnSmArgs aa, int t, W& wait) {
  if (wait()) attn_combine_task<HD>(aa, t);
}

template <class W>
__device__ __noinline__ void emb_run(FlowTask f, int t, uint8_t* smem, W& wait) {
  if (wait()) emb_task(f, t, *reinterpret_cast<FlowSmem*>(smem));
}

template <class W>
__device__ __noinline__ void vel_run(FlowTask f, int t, uint8_t* smem, W& wait) {
  if (wait()) vel_task(f, t, *reinterpret_cast<FlowSmem*>(smem));
}

// ---------------------------------------------------------------- the kernel
template <int MT, int HD>
__global__ __launch_bounds__(256) void stage_kernel(StageArgs sa) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ int ok_sh;

  if (threadIdx.x == 0) ok_sh = ld_u32c(sa.abort_word) == 0u;
  __syncthreads();
  if (!ok_sh) {   // an earlier launch on this workspace aborted
    poison_outputs(sa);
    return;
  }
  const int nwg = gridDim.x;
  unsigned* const ctrs = sa.flags;
  unsigned* const abort_word = sa.abort_word;

  // Runs this workgroup's tasks of phase `type`, each after every task of
  // instance `winst` (1-based, counted from this launch's start) of phase type
  // `wtype` has arrived (wtype < 0: no wait).  task(t, wait) returns the flag
  // index whose shard counts its arrival (or -1); wait() waits once per phase.
  // Returns false if the grid aborted.
  auto phase = [&](int type, int wtype, unsigned winst, auto&& task) -> bool {
    const PhaseMap pm = sa.ph[type];
    const int my = (int)((blockIdx.x + nwg - pm.w0) % nwg);
    bool waited = wtype < 0, alive = true;
    unsigned* const wctrs = phase_ctr(ctrs, wtype < 0 ? 0 : wtype, 0);
    const int wn = wtype < 0 ? 0 : sa.ph[wtype].n_flags;
    auto wait = [&waited, &alive, wctrs, wn, winst, abort_word]() -> bool {
      if (!waited) {
        waited = true;
        alive = wait_counts(wctrs, wn, winst, abort_word);
      }
      return alive;
    };
    if (my < pm.nw) {
      for (int t = my; t < pm.n_tasks; t += pm.nw) {
        const int fl = task(t, wait);
        if (!alive) return false;
        if (fl >= 0) signal_count(phase_ctr(ctrs, type, fl % kShards));
      }
    }
    return true;
  };

  const int D = sa.D, F = sa.F, d = sa.d, Hq = sa.Hq, Hkv = sa.Hkv, M = sa.M;
  const int MTm = mt_of(M);
  const int n_rb = ((Hq / Hkv) * sa.T + 63) / 64;

  // in_frag: the layer input (and first residual) is in operand order;
  // out_frag: likewise for its output
  // li: the layer instance within this launch (0-based); the QKV step waits
  // for instance qinst of phase type qwait (the producer of `in`)
  auto run_layer = [&](int layer, unsigned li, int qwait, unsigned qinst, const bf16_t* in,
                       bool in_frag, bf16_t* out, bool out_frag, const bf16_t* kp,
                       const bf16_t* vp) -> bool {
    const unsigned inst = li + 1;
    const uint8_t* lw = sa.packed + sa.layer0 + (size_t)layer * sa.layer_bytes;
    SkArgs base{};
    base.M = M;
    base.eps = sa.eps;
    base.part = sa.part;
    if (!phase(kPhQKV, qwait, qinst, [&](int t, auto& wait) {
          SkArgs ga = base;
          ga.A = in;
          ga.lda = D;
          ga.K = D;
          ga.Bp = lw + sa.off_qkv;
          ga.n_groups = (Hq + 2 * Hkv) * d / 32;
          ga.splits = sa.split_qkv;
          ga.counters = sa.ctr_qkv;
          EpiQkvS e{sa.q, sa.kn, sa.vn, sa.new_stride, sa.cos_t, sa.sin_t, sa.T, sa.P, Hq, Hkv, d};
          const bool done = in_frag ? sk_dispatch<MT, true, false>(ga, sa.gpw_qkv, e, t, smem, wait)
                                    : sk_dispatch<MT, true, true>(ga, sa.gpw_qkv, e, t, smem, wait);
          return done ? t / ga.splits : -1;
        }))
      return false;
    AttnSmArgs aa{};
    aa.q = sa.q;
    aa.kp = kp;
    aa.vp = vp;
    aa.prefix_stride = sa.prefix_stride;
    aa.kn = sa.kn;
    aa.vn = sa.vn;
    aa.new_stride = sa.new_stride;
    aa.o = sa.o;
    aa.B = sa.B;
    aa.T = sa.T;
    aa.P = sa.P;
    aa.Hq = Hq;
    aa.Hkv = Hkv;
    aa.splits = sa.att_splits;
    aa.kps = sa.att_kps;
    aa.scale_log2 = sa.scale_log2;
    aa.part_o = sa.att_part_o;
    aa.part_ml = sa.att_part_ml;
    if (!phase(kPhATT, kPhQKV, inst, [&](int t, auto& wait) {
          const int rbt = t / aa.splits, ks = t - rbt * aa.splits;
          const int bh = rbt / n_rb, rb = rbt - bh * n_rb;
          attn_run<HD>(aa, bh, rb, ks, smem, wait);
          return t;
        }))
      return false;
    if (aa.splits > 1 && !phase(kPhCMB, kPhATT, inst, [&](int t, auto& wait) {
          cmb_run<HD>(aa, t, wait);
          return t;
        }))
      return false;
    if (!phase(kPhO, aa.splits > 1 ? kPhCMB : kPhATT, inst, [&](int t, auto& wait) {
          SkArgs ga = base;
          ga.A = sa.o;
          ga.K = Hq * d;
          ga.Bp = lw + sa.off_o;
          ga.n_groups = D / 32;
          ga.splits = sa.split_o;
          ga.counters = sa.ctr_o;
          EpiResidS e{in, in_frag ? 1 : 0, MTm, nullptr, sa.h, 1, MTm, 0, D};
          return sk_dispatch<MT, false, false>(ga, sa.gpw_o, e, t, smem, wait) ? t / ga.splits : -1;
        }))
      return false;
    if (!phase(kPhGU, kPhO, inst, [&](int t, auto& wait) {
          SkArgs ga = base;
          ga.A = sa.h;
          ga.K = D;
          ga.Bp = lw + sa.off_gu;
          ga.n_groups = F / 16;
          ga.splits = sa.split_gu;
          ga.counters = sa.ctr_gu;
          return sk_dispatch<MT, true, false>(ga, sa.gpw_gu, EpiGateUpS{sa.a, MTm}, t, smem, wait) ? t / ga.splits
                                                                                                   : -1;
        }))
      return false;
    return phase(kPhD, kPhGU, inst, [&](int t, auto& wait) {
      SkArgs ga = base;
      ga.A = sa.a;
      ga.K = F;
      ga.Bp = lw + sa.off_d;
      ga.n_groups = D / 32;
      ga.splits = sa.split_d;
      ga.counters = sa.ctr_d;
      EpiResidS e{sa.h, 1, MTm, nullptr, out, out_frag ? 1 : 0, MTm, 0, D};
      return sk_dispatch<MT, false, false>(ga, sa.gpw_d, e, t, smem, wait) ? t / ga.splits : -1;
    });
  };

  bool ok = true;
  if (!sa.flow) {
    for (int li = 0; li < sa.n_layers && ok; ++li) {
      const bool first = li == 0, last = li == sa.n_layers - 1;
      const bf16_t* in = first ? sa.x : sa.xb[(li - 1) & 1];
      bf16_t* out = last ? sa.y : sa.xb[li & 1];
      ok = run_layer(sa.layer_first + li, (unsigned)li, first ? -1 : kPhD, (unsigned)li, in, !first, out,
                     !last, sa.kp[0], sa.vp[0]);
    }
  } else {
    for (int s = 0; s < sa.n_steps && ok; ++s) {
      FlowTask f{};
      f.a_in = s == 0 ? sa.noise : sa.actions;
      f.state = sa.state;
      f.w_fused = sa.w_fused;
      f.bias = sa.table + (size_t)s * D;
      f.ws_f = sa.ws_f;
      f.bs = sa.bs;
      f.z = sa.z;
      f.x0 = sa.xb[0];
      f.X = sa.xb[sa.n_layers & 1];
      f.w_out = sa.w_out;
      f.b_out = sa.b_out;
      f.actions = sa.actions;
      f.dt = sa.dt[s];
      f.N = sa.N;
      f.A = sa.A;
      f.D = D;
      f.MTz = mt_of(sa.N + 1);
      f.eps = sa.eps;
      const unsigned L = (unsigned)sa.n_layers;
      ok = phase(kPhEMB, s == 0 ? -1 : kPhVEL, (unsigned)s, [&](int t, auto& wait) {
        emb_run(f, t, smem, wait);
        return t;
      });
      if (ok)
        ok = phase(kPhW3, kPhEMB, (unsigned)s + 1, [&](int t, auto& wait) {
          SkArgs ga{};
          ga.A = sa.z;
          ga.M = sa.N;
          ga.K = D;
          ga.Bp = sa.w3;
          ga.n_groups = D / 32;
          ga.splits = sa.split_w3;
          ga.part = sa.part;
          ga.counters = sa.ctr_o;
          EpiResidS e{nullptr, 0, 0, sa.b3, sa.xb[0], 1, mt_of(sa.N + 1), 1, D};
          return sk_dispatch<MT, false, false>(ga, sa.gpw_w3, e, t, smem, wait) ? t / ga.splits : -1;
        });
      for (int l = 0; l < sa.n_layers && ok; ++l)
        ok = run_layer(l, (unsigned)s * L + l, l == 0 ? kPhW3 : kPhD, l == 0 ? (unsigned)s + 1 : (unsigned)s * L + l,
                       sa.xb[l & 1], true, sa.xb[(l + 1) & 1], true, sa.kp[l], sa.vp[l]);
      if (ok)
        ok = phase(kPhVEL, kPhD, ((unsigned)s + 1) * L, [&](int t, auto& wait) {
          vel_run(f, t, smem, wait);
          return t;
        });
    }
  }
  if (!ok) {
    poison_outputs(sa);
    return;
  }
  // the last workgroup to finish (every wait of every workgroup is over)
  // clears the arrival counters for the next launch
  __shared__ int last_sh;
  if (threadIdx.x == 0) {
    const unsigned old = __hip_atomic_fetch_add(sa.done_ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    last_sh = old == (unsigned)nwg - 1u;
  }
  __syncthreads();
  if (last_sh) {
    for (int i = threadIdx.x; i < kPhCount * kShards; i += blockDim.x)
      st_u32c(phase_ctr(ctrs, i / kShards, i % kShards), 0u);
    if (threadIdx.x == 0) st_u32c(sa.done_ctr, 0u);
  }
}

// ---------------------------------------------------------------- host side
template <int MT, int HD>
static hipError_t go(const StageArgs& sa, int nwg, size_t smem, hipStream_t st) {
  stage_kernel<MT, HD><<<nwg, 256, smem, st>>>(sa);
  return hipGetLastError();
}

// Raises the kernel's dynamic LDS limit (outside any stream capture) and
// returns how many of its workgroups fit on one compute unit.
template <int MT, int HD>
static int prepare(size_t smem) {
  if (hipFuncSetAttribute(reinterpret_cast<const void*>(&stage_kernel<MT, HD>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem) != hipSuccess)
    return 0;
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, stage_kernel<MT, HD>, 256, smem) != hipSuccess)
    return 0;
  return n;
}

template <int HD>
static int prepare_mt(int mt, size_t smem) {
  switch (mt) {
    case 1: return prepare<1, HD>(smem);
    case 2: return prepare<2, HD>(smem);
    case 3: return prepare<3, HD>(smem);
    default: return prepare<4, HD>(smem);
  }
}

int stage_grid(int head_dim, int rows) {
  const int cus = device_cus();
  const size_t smem = stage_smem_bytes(head_dim);
  const int mt = (rows + 15) / 16;
  const int occ = head_dim == 64 ? prepare_mt<64>(mt, smem)
                  : head_dim == 128 ? prepare_mt<128>(mt, smem)
                                    : prepare_mt<256>(mt, smem);
  return occ >= 1 ? cus : 0;
}

size_t stage_smem_bytes(int head_dim) {
  size_t att = head_dim == 64    ? sizeof(AttnSmSmem<64>)
               : head_dim == 128 ? sizeof(AttnSmSmem<128>)
                                 : sizeof(AttnSmSmem<256>);
  size_t m = sizeof(SkSmem<true, kSkPlanMaxGpw>);
  if (sizeof(SkSmem<false, kSkPlanMaxGpw>) > m) m = sizeof(SkSmem<false, kSkPlanMaxGpw>);
  if (att > m) m = att;
  if (sizeof(FlowSmem) > m) m = sizeof(FlowSmem);
  return (m + 255) / 256 * 256;
}

template <int MT>
static hipError_t go_hd(const StageArgs& sa, int nwg, size_t smem, hipStream_t st) {
  switch (sa.d) {
    case 64: return go<MT, 64>(sa, nwg, smem, st);
    case 128: return go<MT, 128>(sa, nwg, smem, st);
    default: return go<MT, 256>(sa, nwg, smem, st);
  }
}

hipError_t launch_stage(const StageArgs& sa, int nwg, hipStream_t st) {
  const size_t smem = stage_smem_bytes(sa.d);
  const int rows = sa.flow ? sa.N + 1 : sa.M;
  switch ((rows + 15) / 16) {
    case 1: return go_hd<1>(sa, nwg, smem, st);
    case 2: return go_hd<2>(sa, nwg, smem, st);
    case 3: return go_hd<3>(sa, nwg, smem, st);
    default: return go_hd<4>(sa, nwg, smem, st);
  }
}

}  // namespace blk
