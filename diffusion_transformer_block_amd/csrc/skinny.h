// Skinny GEMM (M <= 64 rows) of the small-chunk path, as a device task shared
// by the standalone kernels and the persistent stage kernel.
//
// [RT] = reading note on "Running VLAs at Real-time Speed" (Ma et al.,
// arXiv:2510.26742v1).  §5: bias / residual / activation merged into the GEMM
// tail; the gated FFN's two up-projections share one load of their input; the
// RMS statistic is consumed fused as a row scale; a partial split-K balances
// skinny shapes over the compute units; §6.2: at few tokens a GEMM is bound by
// reading its bf16 weights.
//
// One task = GPW (1 or 2) consecutive 32-column groups of a packed weight
// (a group holds both 16-column tiles, as the fused QKV and gate/up epilogues
// need) over the K-range of split s.  Two groups per workgroup halve the
// number of workgroups that each read the whole activation slab -- those
// re-reads, all served by L2, bound the widest GEMMs otherwise.
//  * Weights: fragments (g, kt, 0..1), 1 KiB each, one 16-byte streaming load
//    per lane.
//  * Activations: in operand order (fa_index in common.h: one contiguous
//    1 KiB load per fragment), or row-major (the block's input, owned by the
//    caller), loaded straight into registers two k-tiles at a time: each load
//    covers 8 rows x one whole 128-byte line (the rows of one parity), and a
//    swap of adjacent lanes between the two loads of a pair gives the two
//    fragments (16 rows x 64 bytes per load instead would touch twice the
//    cache lines per instruction; measured 11.0 -> 9.8 us on the 64-token
//    QKV).  Either way the loads ride the weights' pipeline.
//  * The four waves split the K-range; each keeps a ring of NB k-tiles of
//    loads in flight ahead of its MFMAs (weights of the first NB k-tiles are
//    issued before the task's wait, since they do not depend on earlier work).
//  * The waves' tiles meet in LDS and are summed in a fixed order; K splits
//    publish fp32 tiles and the last split to arrive (device counter, reset by
//    it) sums all of them in split order, so results do not depend on timing.
//  * With RMS the waves also sum x^2 of the rows they load (the statistic
//    costs no extra pass: one MFMA of each activation fragment with itself,
//    whose diagonal is the rows' sums of squares) and the epilogue gets
//    r = (mean x^2 + eps)^-1/2.
//  * The epilogue reads the summed 64 x 32 tile from LDS in the order it
//    stores (row-contiguous 16-byte stores).
#pragma once
#include <type_traits>

#include "common.h"

namespace blk {

constexpr int kSkMaxSplits = 16;
constexpr int kSkMaxGpw = 2;        // 32-column groups per workgroup
// Two groups per workgroup measured slower on every 64-row shape of the AE
// block (the per-unit operand stream, not the L2 re-reads, binds), so plans
// keep one; the two-group variant stays available to the kernels.
constexpr int kSkPlanMaxGpw = 1;

// row stride (floats) of the LDS result tile of GPW groups: 32 GPW + 4 pad
__host__ __device__ constexpr int sk_tile_stride(int gpw) { return 32 * gpw + 4; }

struct SkArgs {
  const bf16_t* A;      // activations, operand order (MT = ceil(M/16)), or row-major (lda)
  int lda;              // row-major only
  int M, K;
  const uint8_t* Bp;    // packed weight fragments
  int n_groups;
  int splits;           // K splits (KT % (4 splits) == 0)
  float eps;            // RMS epsilon
  float* part;          // [splits][n_groups][64 * 32] tiles, then [splits][n_groups][64] x^2 sums
  unsigned* counters;   // [n_groups / GPW], zero on entry and on exit
};

template <bool AROW, int GPW>
struct SkSmem {
  f32x4 red[4][4 * GPW * 2 * 64];              // per-wave accumulators in MFMA C order
  float tile[64 * sk_tile_stride(GPW)];        // summed tile [row][col]
  float ss[4][64];
  float rrow[64];
  int last_flag;
};

struct NoWait {
  __device__ __forceinline__ bool operator()() const { return true; }
};

__device__ __forceinline__ float sumsq8(uint4 v) {
  float x[8];
  unpack8(v, x);
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) s = fmaf(x[i], x[i], s);
  return s;
}

// Runs one task -- groups [GPW gb, GPW gb + GPW) over split s -- and stores
// its outputs through `epi` (see the epilogues below).  `wait()` is called
// after the first weight loads are issued and before anything that depends on
// earlier work; it returns false to abandon the task.  Returns false when
// this workgroup did not run the epilogue (abandoned, or it only published a
// split partial).
template <int MT, int NB, int GPW, bool RMS, bool AROW, class Epi, class Wait>
__device__ bool sk_task(const SkArgs& ga, const Epi& epi, int gb, int s, SkSmem<AROW, GPW>& sm,
                        Wait&& wait) {
  constexpr int TS = sk_tile_stride(GPW);
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index (uniform)
  const int l = tid & 63, lr = l & 15;
  const int KT = ga.K >> 5;
  const int KTS = KT / ga.splits;
  const int KW = KTS >> 2;             // k-tiles per wave, a multiple of NB
  const int kb = s * KTS;              // first k-tile of this split
  const int uw = w * KW;               // first k-tile of this wave, relative to kb
  const int g0 = gb * GPW;
  const int ng = min(GPW, ga.n_groups - g0);

  // ---- weights of the first NB k-tiles (independent of earlier work); the
  //      groups' fragments are contiguous, [group][kt][tile]
  const __amdgpu_buffer_rsrc_t rb =
      make_rsrc(ga.Bp + frag_offset(g0, 0, 0, KT), (size_t)ng * KT * 2 * kFragBytes);
  const int boff = (kb + uw) * 2 * kFragBytes + l * 16;
  uint4 bw[NB][GPW][2];
  auto issue_w = [&](int b, int u) {
#pragma unroll
    for (int j = 0; j < GPW; ++j) {
      const int o = boff + (j * KT + u) * 2 * kFragBytes;
      bw[b][j][0] = buf_ld_stream(rb, o);
      bw[b][j][1] = buf_ld_stream(rb, o + kFragBytes);
    }
  };
#pragma unroll
  for (int b = 0; b < NB; ++b) issue_w(b, b);
  if (!wait()) return false;
  typename Epi::Pre pre[GPW];
#pragma unroll
  for (int j = 0; j < GPW; ++j) pre[j] = epi.prefetch(g0 + min(j, ng - 1), ga.M);
  // ---- activations: an A fragment is 16 bytes per lane.  Operand order:
  //      one contiguous 1 KiB fragment.  Row-major (the caller's input), k-tiles
  //      in pairs: load h of a pair takes the rows of parity h of each 16-row
  //      tile, 8 rows x one whole 128-byte line (both k-tiles), lane l holding
  //      row 2 ((l >> 1) & 7) + h, k-tile l & 1, 16-byte chunk l >> 4; one
  //      swap of adjacent lanes between the two loads (swap_pair) then yields
  //      the pair's two fragments.  Without pairs (a ring of one k-tile) a load
  //      takes 16 rows x 64 bytes.  Rows past M are clamped to M - 1 (their
  //      results are never stored).
  constexpr bool PAIR = AROW && NB % 2 == 0;
  uint4 av[NB][MT];
  __amdgpu_buffer_rsrc_t ra;
  int aoff[2][MT];
  if (AROW) {
    ra = make_rsrc(ga.A, (size_t)ga.M * ga.lda * 2);
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        aoff[h][mt] = PAIR ? (min(16 * mt + 2 * ((l >> 1) & 7) + h, ga.M - 1) * ga.lda +
                              (kb + uw) * 32 + 32 * (l & 1) + 8 * (l >> 4)) * 2
                           : (min(16 * mt + lr, ga.M - 1) * ga.lda + (kb + uw) * 32 + 8 * (l >> 4)) * 2;
  } else {
    ra = make_rsrc(ga.A, (size_t)KT * MT * kFragBytes);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) aoff[0][mt] = ((kb + uw) * MT * 64 + l) * 16 + mt * kFragBytes;
  }
  // ring slot b holds k-tile u (same parity); with pairs, load b & 1 of the
  // pair that starts at k-tile u - (b & 1)
  auto issue_a = [&](int b, int u) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      if (PAIR) av[b][mt] = buf_ld_act(ra, aoff[b & 1][mt] + (u - (b & 1)) * 64);
      else av[b][mt] = buf_ld_act(ra, aoff[0][mt] + u * (AROW ? 64 : MT * kFragBytes));
    }
  };
  const bool odd_lane = (l & 1) != 0;
  auto swap_pair = [&](int b) {   // slots b (even rows), b + 1 (odd rows) -> fragments
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const uint32_t x[4] = {av[b][mt].x, av[b][mt].y, av[b][mt].z, av[b][mt].w};
      const uint32_t y[4] = {av[b + 1][mt].x, av[b + 1][mt].y, av[b + 1][mt].z, av[b + 1][mt].w};
      uint32_t f0[4], f1[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        // quad_perm [1, 0, 3, 2]: each lane reads its neighbour l ^ 1
        const uint32_t xs = (uint32_t)__builtin_amdgcn_mov_dpp((int)x[e], 0xB1, 0xF, 0xF, true);
        const uint32_t ys = (uint32_t)__builtin_amdgcn_mov_dpp((int)y[e], 0xB1, 0xF, 0xF, true);
        f0[e] = odd_lane ? ys : x[e];
        f1[e] = odd_lane ? y[e] : xs;
      }
      av[b][mt] = uint4{f0[0], f0[1], f0[2], f0[3]};
      av[b + 1][mt] = uint4{f1[0], f1[1], f1[2], f1[3]};
    }
  };
  auto get_a = [&](int b, int, int mt) -> uint4 { return av[b][mt]; };

  // With RMS, ss[mt] = A_mt A_mt^T accumulated on the matrix unit: the same
  // fragment as both operands puts each row's sum of squares on the diagonal
  // (one MFMA per fragment instead of 16 vector instructions).
  f32x4 acc[MT][GPW][2];
  f32x4 ss[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int j = 0; j < GPW; ++j) {
      acc[mt][j][0] = f32x4{0.f, 0.f, 0.f, 0.f};
      acc[mt][j][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    ss[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int b = 0; b < NB; ++b) issue_a(b, b);
  for (int u0 = 0; u0 < KW; u0 += NB) {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int u = u0 + b;
      if (PAIR && (b & 1) == 0) swap_pair(b);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const uint4 a = get_a(b, u, mt);
        if (RMS) ss[mt] = mfma16(as_bf16x8(a), as_bf16x8(a), ss[mt]);
#pragma unroll
        for (int j = 0; j < GPW; ++j) {
          acc[mt][j][0] = mfma16(as_bf16x8(a), as_bf16x8(bw[b][j][0]), acc[mt][j][0]);
          acc[mt][j][1] = mfma16(as_bf16x8(a), as_bf16x8(bw[b][j][1]), acc[mt][j][1]);
        }
      }
      if (u + NB < KW) {
        issue_w(b, u + NB);
        issue_a(b, u + NB);
      }
    }
  }

  // ---- the four waves' tiles -> summed tile [row][col] in LDS
  __syncthreads();   // a previous task's readers of sm are done
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int j = 0; j < GPW; ++j)
#pragma unroll
      for (int i = 0; i < 2; ++i) sm.red[w][((mt * GPW + j) * 2 + i) * 64 + l] = acc[mt][j][i];
  if (RMS) {
    // C layout: lane l holds rows 4 (l >> 4) + i of column l & 15, so row r's
    // diagonal entry sits in lane 16 (r >> 2) + r, element r & 3
    const int di = l & 3;
    if (((l & 15) >> 2) == (l >> 4)) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const f32x4 v = ss[mt];
        sm.ss[w][16 * mt + lr] = di == 0 ? v[0] : di == 1 ? v[1] : di == 2 ? v[2] : v[3];
      }
    }
  }
  __syncthreads();
  for (int sl = tid; sl < MT * GPW * 128; sl += 256) {
    const f32x4 v = ((sm.red[0][sl] + sm.red[1][sl]) + sm.red[2][sl]) + sm.red[3][sl];
    const int q = sl >> 6, ll = sl & 63;           // q = (mt * GPW + j) * 2 + i
    const int i = q & 1, j = (q >> 1) % GPW, mt = (q >> 1) / GPW;
    const int row = 16 * mt + 4 * (ll >> 4), col = 32 * j + 16 * i + (ll & 15);
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) sm.tile[(row + jj) * TS + col] = v[jj];
  }
  float ssum = 0.f;
  if (RMS && tid < 16 * MT) ssum = ((sm.ss[0][tid] + sm.ss[1][tid]) + sm.ss[2][tid]) + sm.ss[3][tid];
  __syncthreads();

  // ---- K splits: publish, last arriver sums every split in order
  if (ga.splits > 1) {
    const int r = tid >> 2, c0 = (tid & 3) * 8;
    const size_t tile_floats = 64 * 32;
    const size_t ss_base = (size_t)ga.splits * ga.n_groups * tile_floats;
    const __amdgpu_buffer_rsrc_t rp =
        make_rsrc(ga.part, (ss_base + (size_t)ga.splits * ga.n_groups * 64) * 4);
    const int tstride = (int)((size_t)ga.n_groups * tile_floats * 4);   // bytes between splits
    const int soff = (int)((ss_base + (size_t)g0 * 64 + tid) * 4);
    const int sstride = ga.n_groups * 64 * 4;
#pragma unroll
    for (int j = 0; j < GPW; ++j) {
      const int toff = (int)(((size_t)(g0 + j) * tile_floats + r * 32 + c0) * 4);
      const float* tp = &sm.tile[r * TS + 32 * j + c0];
      if (j < ng) {
        buf_st16(rp, toff + s * tstride, *reinterpret_cast<const uint4*>(tp));
        buf_st16(rp, toff + s * tstride + 16, *reinterpret_cast<const uint4*>(tp + 4));
      }
    }
    if (RMS && tid < 64) buf_st4(rp, soff + s * sstride, ssum);
    if (!arrive_last(&ga.counters[gb], (unsigned)ga.splits, &sm.last_flag)) return false;
#pragma unroll
    for (int j = 0; j < GPW; ++j) {
      if (j >= ng) break;
      const int toff = (int)(((size_t)(g0 + j) * tile_floats + r * 32 + c0) * 4);
      uint4 pv[kSkMaxSplits][2];
#pragma unroll
      for (int sp = 0; sp < kSkMaxSplits; ++sp)
        if (sp < ga.splits) {
          pv[sp][0] = buf_ld_act(rp, toff + sp * tstride);
          pv[sp][1] = buf_ld_act(rp, toff + sp * tstride + 16);
        }
      float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int sp = 0; sp < kSkMaxSplits; ++sp)
        if (sp < ga.splits) {
          const uint32_t u[8] = {pv[sp][0].x, pv[sp][0].y, pv[sp][0].z, pv[sp][0].w,
                                 pv[sp][1].x, pv[sp][1].y, pv[sp][1].z, pv[sp][1].w};
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] += __uint_as_float(u[e]);
        }
#pragma unroll
      for (int e = 0; e < 8; ++e) sm.tile[r * TS + 32 * j + c0 + e] = v[e];
    }
    if (RMS) {
      float ps[kSkMaxSplits];
#pragma unroll
      for (int sp = 0; sp < kSkMaxSplits; ++sp)
        if (sp < ga.splits) ps[sp] = tid < 64 ? buf_ld4_act(rp, soff + sp * sstride) : 0.f;
      ssum = 0.f;
#pragma unroll
      for (int sp = 0; sp < kSkMaxSplits; ++sp)
        if (sp < ga.splits) ssum += ps[sp];
    }
  }
  if (RMS) {
    if (tid < 64) sm.rrow[tid] = rsqrtf(ssum / (float)ga.K + ga.eps);
  }
  if (RMS || ga.splits > 1) __syncthreads();
#pragma unroll
  for (int j = 0; j < GPW; ++j)
    if (j < ng) epi.run(sm.tile + 32 * j, TS, sm.rrow, RMS, g0 + j, ga.M, pre[j]);
  return true;
}

// ============================================================================ epilogues
// Each epilogue is called by all 256 threads with the summed tile of its
// group, tile[row * ts + col] (row < 64, col < 32 = the group's two 16-column
// tiles), and the row scale rrow (used when `rms`).  prefetch() runs right
// after the task's wait, so its loads overlap the activation loads.  All
// stores are device-coherent.

// Attention operand order of Q (written by the QKV epilogue, read by the
// attention): for stream b and kv head hk the rows are ar = t G + gh over the
// G = Hq / Hkv query heads sharing that kv head; row tile ar / 32 and the
// 16-column slice dd / 16 form one 1 KiB fragment, lane ar % 32 + 32 ((dd % 16) / 8)
// holding 8 consecutive dd (the B operand of a 32 x 32 x 16 MFMA).
__host__ __device__ inline size_t qa_index(int bh, int n_rt, int NDS, int ar, int dd) {
  return ((((size_t)bh * n_rt + (ar >> 5)) * NDS + (dd >> 4)) * 64 + (ar & 31) + 32 * ((dd >> 3) & 1)) * 8 +
         (dd & 7);
}

// Fused QKV: row scale, RoPE on the rotated (Q, K) groups (column j with
// j + d/2 in one group), Q into the attention operand order, K_new and V_new
// row-major ([T][Hkv][d] per stream at b * new_stride).
struct EpiQkvS {
  bf16_t* q;
  bf16_t* kn;
  bf16_t* vn;
  int64_t new_stride;
  const float* cos_t;   // [max_pos][d/2]
  const float* sin_t;
  int T, P, Hq, Hkv, d;
  int g_base;           // packed group of the GEMM's group 0 (> 0: a K/V-only run)
  const int* plen;      // device: stream b's prefix length (NULL: all P); token t at P_b + t
  // this thread's cos / sin quadruple, loaded while the GEMM runs
  struct Pre {
    float4 cs, sn;
  };
  __device__ Pre prefetch(int g, int M) const {
    g += g_base;
    const int t = threadIdx.x, r = t >> 2;
    const int gpr = d >> 5;
    Pre p{make_float4(1.f, 1.f, 1.f, 1.f), make_float4(0.f, 0.f, 0.f, 0.f)};
    if (r < M && g < (Hq + Hkv) * gpr) {
      const int b = r / T, tt = r - b * T, head = g / gpr;
      const size_t ti = (size_t)(stream_prefix(plen, P, b) + tt) * (d >> 1) + 16 * (g - head * gpr) + (t & 3) * 4;
      p.cs = *reinterpret_cast<const float4*>(cos_t + ti);
      p.sn = *reinterpret_cast<const float4*>(sin_t + ti);
    }
    return p;
  }
  __device__ void run(const float* tile, int ts, const float* rrow, bool rms, int g, int M, const Pre& pf) const {
    g += g_base;
    const int t = threadIdx.x;
    const int r = t >> 2;
    if (r >= M) return;
    const float rs = rms ? rrow[r] : 1.f;
    const int b = r / T, tt = r - b * T;
    const int gpr = d >> 5, n_rot_groups = (Hq + Hkv) * gpr;
    const float* tr = tile + r * ts;
    if (g < n_rot_groups) {
      const int q4 = (t & 3) * 4;
      const int head = g / gpr;
      const int half = d >> 1;
      const int j0 = 16 * (g - head * gpr) + q4;
      const float c4[4] = {pf.cs.x, pf.cs.y, pf.cs.z, pf.cs.w}, s4[4] = {pf.sn.x, pf.sn.y, pf.sn.z, pf.sn.w};
      float lo[4], hi[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float v0 = tr[q4 + i] * rs, v1 = tr[16 + q4 + i] * rs;
        lo[i] = v0 * c4[i] - v1 * s4[i];
        hi[i] = v0 * s4[i] + v1 * c4[i];
      }
      if (head < Hq) {
        const int G = Hq / Hkv;
        const int hk = head / G, gh = head - hk * G;
        const int n_rt = (G * T + 31) >> 5;
        const int ar = tt * G + gh, bh = b * Hkv + hk;
        st8c(q + qa_index(bh, n_rt, d >> 4, ar, j0), pack2(lo[0], lo[1]), pack2(lo[2], lo[3]));
        st8c(q + qa_index(bh, n_rt, d >> 4, ar, j0 + half), pack2(hi[0], hi[1]), pack2(hi[2], hi[3]));
      } else {
        bf16_t* dst = kn + (size_t)b * new_stride + ((size_t)tt * Hkv + (head - Hq)) * d;
        st8c(dst + j0, pack2(lo[0], lo[1]), pack2(lo[2], lo[3]));
        st8c(dst + j0 + half, pack2(hi[0], hi[1]), pack2(hi[2], hi[3]));
      }
    } else {
      const int c0 = (t & 3) * 8;
      float v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = tr[c0 + i] * rs;
      bf16_t* dst = vn + (size_t)b * new_stride + (size_t)tt * Hkv * d + 32 * (g - n_rot_groups) + c0;
      st16c(dst, pack8(v));
    }
  }
};

// out[row_off + m][n] = acc (+ res[m][n]) (+ bias[n]) for the group's 32
// columns n = 32 g + c: O and down projections (residual), the flow
// embedding's W3 (bias).  res and out are each in operand order (MT of their
// own row count) or row-major with leading dimension N.
struct EpiResidS {
  const bf16_t* res;    // may be NULL
  int res_frag, res_MT;
  const float* bias;    // may be NULL
  bf16_t* out;
  int out_frag, out_MT, row_off;
  int N;
  struct Pre {
    uint4 v;
  };
  __device__ Pre prefetch(int g, int M) const {
    const int t = threadIdx.x, ln = t & 63;
    const int r = 16 * (t >> 6) + (ln & 15), c = 32 * g + 8 * (ln >> 4);
    Pre p{make_uint4(0, 0, 0, 0)};
    if (res && r < M) p.v = ld16c(res + (res_frag ? fa_index(r, c, res_MT) : (size_t)r * N + c));
    return p;
  }
  __device__ void run(const float* tile, int ts, const float*, bool, int g, int M, const Pre& p) const {
    const int t = threadIdx.x, ln = t & 63;
    const int r = 16 * (t >> 6) + (ln & 15), cl = 8 * (ln >> 4), c = 32 * g + cl;
    if (r >= M) return;
    float v[8], rv[8];
    unpack8(p.v, rv);
    const float* tr = tile + r * ts + cl;
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = tr[i] + rv[i];
    if (bias) {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] += bias[c + i];
    }
    const int ro = r + row_off;
    st16c(out + (out_frag ? fa_index(ro, c, out_MT) : (size_t)ro * N + c), pack8(v));
  }
};

// a[m][j] = SiLU(r * gate) * (r * up) for j = 16 g + c: tile 0 holds the gate
// columns, tile 1 the up columns of the same j; a is in operand order.
struct EpiGateUpS {
  bf16_t* out;
  int MT;
  struct Pre {};
  __device__ Pre prefetch(int, int) const { return {}; }
  __device__ void run(const float* tile, int ts, const float* rrow, bool rms, int g, int M, const Pre&) const {
    const int t = threadIdx.x;
    if (t >= 128) return;
    const int q = t & 31;
    const int r = 16 * (t >> 5) + (q & 15), hf = q >> 4;
    if (r >= M) return;
    const float rs = rms ? rrow[r] : 1.f;
    const float* tr = tile + r * ts + 8 * hf;
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = silu(tr[i] * rs) * (tr[16 + i] * rs);
    st16c(out + fa_index(r, 16 * g + 8 * hf, MT), pack8(v));
  }
};

}  // namespace blk
