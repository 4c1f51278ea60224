// MFMA GEMMs of the block with fused epilogues.
//
// [RT] = reading note on "Running VLAs at Real-time Speed" (Ma et al.,
// arXiv:2510.26742v1).  §5: bias / residual / activation are merged into the
// GEMM tail; the gated FFN's two up-projections share one load of their input
// and the activation, elementwise gate and write-back are fused; the per-row
// RMS statistic is computed first and consumed fused (with the gain already
// folded into the weights it is just a row scale of the product); a partial
// split-K balances skinny shapes over the compute units.  §6.2: at few tokens
// a GEMM is bound by reading its bf16 weights.
//
// The large-chunk GEMM (M > 64 rows; chunks of <= 64 rows run the skinny
// GEMM of skinny.h): 256 x 256 (224 x 256 where that pads fewer rows; or
// 128 x 128, 128 x 64 on narrow shapes) output tiles, both operands
// moved into LDS by the load DMA as MFMA fragments, 2 x 2 waves of
// 16 x 16 x 32 MFMAs, XCD-aware tile order (big_gemm_kernel below).
#include "common.h"
#include "internal.h"
#include "skinny.h"

#include <utility>

namespace blk {

__device__ __forceinline__ void EpiQKV::store(int m, int g, int qc, const float* srow, const Pre& p) const {
  g += g_base;
  const int b = m / T, t = m - b * T;
  const int gpr = d >> 5, n_rot_groups = (Hq + Hkv) * gpr;
  float x1[8], x2[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    x1[e] = srow[8 * qc + e];
    x2[e] = srow[16 + 8 * qc + e];
  }
  if (g < n_rot_groups) {
    const float cs[8] = {p.c0.x, p.c0.y, p.c0.z, p.c0.w, p.c1.x, p.c1.y, p.c1.z, p.c1.w};
    const float sn[8] = {p.s0.x, p.s0.y, p.s0.z, p.s0.w, p.s1.x, p.s1.y, p.s1.z, p.s1.w};
    float y1[8], y2[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      y1[e] = x1[e] * cs[e] - x2[e] * sn[e];
      y2[e] = x1[e] * sn[e] + x2[e] * cs[e];
    }
    const int head = g / gpr;
    const int col = 16 * (g - head * gpr) + 8 * qc;   // column j of the pair; j + d/2 holds its partner
    bf16_t *d1, *d2;
    if (head < Hq) {
      const int G = Hq / Hkv, hk = head / G, gh = head - hk * G;
      const int n_rt = (G * T + 31) >> 5, NDS = d >> 4;
      d1 = q + qa_index(b * Hkv + hk, n_rt, NDS, t * G + gh, col);
      d2 = q + qa_index(b * Hkv + hk, n_rt, NDS, t * G + gh, col + (d >> 1));
    } else {
      d1 = kn + (size_t)b * new_stride + ((size_t)t * Hkv + (head - Hq)) * d + col;
      d2 = d1 + (d >> 1);
    }
    *reinterpret_cast<uint4*>(d1) = pack8(y1);
    *reinterpret_cast<uint4*>(d2) = pack8(y2);
  } else {
    bf16_t* d1 = vn + (size_t)b * new_stride + (size_t)t * Hkv * d + 32 * (g - n_rot_groups) + 8 * qc;
    *reinterpret_cast<uint4*>(d1) = pack8(x1);
    *reinterpret_cast<uint4*>(d1 + 16) = pack8(x2);
  }
}

// ============================================================================ large-chunk GEMM

// Instruction order of one K step: the R fragment reads of the next stage
// (LDS) alternate with the F MFMAs of this one, one read ahead of each run of
// F / R MFMAs.  Issued together in front of the MFMAs, the reads of four
// waves fill the LDS command queue at once and hold every wave's MFMAs back
// until they drain.
template <int F, int R, int... I>
__device__ __forceinline__ void sched_reads_between_mfmas(std::integer_sequence<int, I...>) {
  ((__builtin_amdgcn_sched_group_barrier(0x100, 1, 0),
    __builtin_amdgcn_sched_group_barrier(0x008, (I + 1) * F / R - I * F / R, 0)),
   ...);
}

// BM x BN output tile per workgroup (4 waves in a 2 x 2 grid, each BM/2 x
// BN/2 of 16 x 16 x 32 MFMAs), one 32-wide k-tile per LDS stage, four stages
// (three in flight ahead of the one in use; measured 3 % faster on the large
// chunks than two stages of 64).  A stage holds the tile's operands as 1 KiB
// MFMA fragments: B (packed weights) and, for AFRAG, A (an operand-order
// activation, fa_index) one contiguous fragment each; a row-major A is
// gathered as 16 rows x 64 bytes per fragment.  The loop is
// software-pipelined: after the barrier that publishes stage s + 1 a wave
// issues the DMA of stage s + 3 and reads stage s + 1's fragments while
// stage s's MFMAs run.
template <int BM, int BN, bool AFRAG, class Epi>
__global__ __launch_bounds__(256) void big_gemm_kernel(GemmArgs ga, Epi epi, int n_tm, int n_tn,
                                                       int n_full, int splits) {
  extern __shared__ __attribute__((aligned(1024))) uint8_t big_dsm[];
  constexpr int BK = 32;                  // one k-tile per LDS stage
  constexpr int NST = 4;                  // LDS stages (three in flight ahead of the one in use)
  constexpr int MTB = BM / 16;            // 16-row tiles per block
  constexpr int GB = BN / 32;             // 32-column groups per block
  constexpr int MTW = MTB / 2, GW = GB / 2;
  constexpr int AFR = MTB, BFR = GB * 2, NFR = AFR + BFR;
  constexpr int STAGE = NFR * kFragBytes;
  // fragments each wave moves per stage: f = w + 4 i < NFR (waves w < PER_X
  // move one more when NFR is not a multiple of 4, e.g. 224-row tiles)
  constexpr int PER_X = NFR % 4, PER = NFR / 4 + (PER_X ? 1 : 0);
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l = tid & 63;
  const int wm = w >> 1, wn = w & 1;
  const bool full_per = PER_X == 0 || w < PER_X;   // this wave moves PER fragments, else PER - 1
  // vmcnt allowing this wave's DMAs of the last `st` stages to be in flight
  auto wait_stages = [&](auto st) {
    constexpr int S = decltype(st)::value;
    if (full_per) asm volatile("s_waitcnt vmcnt(%0)" :: "n"(S * PER) : "memory");
    else asm volatile("s_waitcnt vmcnt(%0)" :: "n"(S * (PER - 1)) : "memory");
  };
  // Units: the first n_full tiles whole, then each remaining tile as `splits`
  // K slices (adjacent).  The hardware deals workgroups round-robin over the
  // 8 XCDs (XCD x runs ids x, x + 8, ... in order): each XCD gets a
  // contiguous run of whole tiles and then a contiguous run of slices, so the
  // slices -- the last round -- spread over every XCD.  Tiles go in bands of
  // GM row tiles with the column tiles outer, so the tiles an XCD runs at once
  // share row and column blocks in its L2.
  const int nwg = gridDim.x, id = blockIdx.x;
  const int xcd = id & 7, jx = id >> 3;
  auto share = [](int n, int x) { return n / 8 + (x < n % 8 ? 1 : 0); };
  auto start = [](int n, int x) { return x * (n / 8) + min(x, n % 8); };
  const int f_x = share(n_full, xcd);
  int tile, split, nsplit;
  if (jx < f_x) {
    tile = start(n_full, xcd) + jx;
    split = 0;
    nsplit = 1;
  } else {
    const int u = start(nwg, xcd) - start(n_full, xcd) + (jx - f_x);
    tile = n_full + u / splits;
    split = u - (u / splits) * splits;
    nsplit = splits;
  }
  constexpr int GM = 4;
  const int band = tile / (GM * n_tn), tib = tile - band * GM * n_tn;
  const int rows_b = min(GM, n_tm - band * GM);
  const int tm = band * GM + tib % rows_b, tn = tib / rows_b;
  const int m0 = tm * BM, g0 = tn * GB;
  const int KT = ga.K >> 5;
  const int nk = ga.K / BK / nsplit, sk0 = split * nk;   // this unit's K steps
  const int MTa = mt_of(ga.M);

  // this wave's fragments of a stage: f = w + 4 i (A fragments first); rows
  // and groups past the matrix are clamped (their results are not stored)
  const uint8_t* gsrc[PER];
  int gstep[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int f = min(w + 4 * i, NFR - 1);   // past NFR: never issued
    if (f < AFR) {
      const int mt = f;
      if (AFRAG) {
        const int rt = min(m0 / 16 + mt, MTa - 1);
        gsrc[i] = reinterpret_cast<const uint8_t*>(ga.A) + (size_t)rt * kFragBytes + 16 * l;
        gstep[i] = MTa * kFragBytes;
      } else {
        const int row = min(m0 + 16 * mt + (l & 15), ga.M - 1);
        gsrc[i] = reinterpret_cast<const uint8_t*>(ga.A) + ((size_t)row * ga.lda + 8 * (l >> 4)) * 2;
        gstep[i] = BK * 2;
      }
    } else {
      const int fb = f - AFR, gg = fb >> 1, ii = fb & 1;
      gsrc[i] = ga.Bp + frag_offset(min(g0 + gg, ga.n_groups - 1), 0, ii, KT) + 16 * l;
      gstep[i] = 2 * kFragBytes;
    }
  }
  const unsigned lds0 = lds_u32(big_dsm);
  auto issue = [&](int s, int buf) {
#pragma unroll
    for (int i = 0; i < PER; ++i)
      if (i < PER - 1 || full_per)
        dma16(lds0 + buf * STAGE + (w + 4 * i) * kFragBytes, gsrc[i] + (size_t)(sk0 + s) * gstep[i]);
  };
  auto rd = [&](int buf, uint4 (&af)[MTW], uint4 (&bfv)[GW][2]) {
    const uint8_t* base = big_dsm + buf * STAGE;
#pragma unroll
    for (int mt = 0; mt < MTW; ++mt)
      af[mt] = *reinterpret_cast<const uint4*>(base + (wm * MTW + mt) * kFragBytes + 16 * l);
#pragma unroll
    for (int gg = 0; gg < GW; ++gg)
#pragma unroll
      for (int ii = 0; ii < 2; ++ii)
        bfv[gg][ii] = *reinterpret_cast<const uint4*>(
            base + (AFR + (wn * GW + gg) * 2 + ii) * kFragBytes + 16 * l);
  };
  f32x4 acc[MTW][GW][2];
#pragma unroll
  for (int a = 0; a < MTW; ++a)
#pragma unroll
    for (int b = 0; b < GW; ++b) {
      acc[a][b][0] = f32x4{0.f, 0.f, 0.f, 0.f};
      acc[a][b][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  auto mm = [&](const uint4 (&af)[MTW], const uint4 (&bfv)[GW][2]) {
#pragma unroll
    for (int mt = 0; mt < MTW; ++mt)
#pragma unroll
      for (int gg = 0; gg < GW; ++gg)
#pragma unroll
        for (int ii = 0; ii < 2; ++ii)
          acc[mt][gg][ii] = mfma16(as_bf16x8(af[mt]), as_bf16x8(bfv[gg][ii]), acc[mt][gg][ii]);
  };

  // prologue: stages 0..2 in flight, stage 0 landed and its fragments read
  issue(0, 0);
  if (nk > 1) issue(1, 1);
  if (nk > 2) issue(2, 2);
  if (nk > 2) wait_stages(std::integral_constant<int, 2>{});
  else if (nk > 1) wait_stages(std::integral_constant<int, 1>{});
  else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  uint4 a0[MTW], b0[GW][2], a1[MTW], b1[GW][2];
  rd(0, a0, b0);
  // stage s: its fragments are in registers; stage s + 1 lands (stages s + 2
  // and, after the barrier, s + 3 stay in flight) and is read while stage
  // s's MFMAs run
  // (the reads of stage s + 1 run unconditionally, so that they share one
  // basic block with the MFMAs: past the last stage they read a stale buffer
  // whose values are never used)
  auto step = [&](int s, uint4 (&ca)[MTW], uint4 (&cb)[GW][2], uint4 (&na)[MTW], uint4 (&nb)[GW][2]) {
    if (s + 2 < nk) wait_stages(std::integral_constant<int, 1>{});
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();   // stage s + 1 visible; every wave is done with stage s - 1's buffer
    if (s + 3 < nk) issue(s + 3, (s + 3) & (NST - 1));
    rd((s + 1) & (NST - 1), na, nb);
    mm(ca, cb);
    sched_reads_between_mfmas<2 * MTW * GW, MTW + 2 * GW>(std::make_integer_sequence<int, MTW + 2 * GW>{});
  };
  for (int s = 0; s < nk; s += 2) {
    step(s, a0, b0, a1, b1);
    if (s + 1 < nk) step(s + 1, a1, b1, a0, b0);
  }
  __syncthreads();

  // ---- K splits: every split publishes its accumulators in MFMA layout (16
  //      coherent bytes per lane); the last to arrive at the tile's counter
  //      sums all of them in split order and runs the epilogue
  if (nsplit > 1) {
    constexpr int NACC = MTW * GW * 2;                  // f32x4 per lane
    constexpr int SPLIT_BYTES = 4 * NACC * 64 * 16;     // one split of a tile
    const __amdgpu_buffer_rsrc_t rp = make_rsrc(
        ga.part + (size_t)(tile - n_full) * nsplit * (SPLIT_BYTES / 4), (size_t)nsplit * SPLIT_BYTES);
    auto slot = [&](int sp, int q) { return sp * SPLIT_BYTES + ((w * NACC + q) * 64 + l) * 16; };
#pragma unroll
    for (int mt = 0; mt < MTW; ++mt)
#pragma unroll
      for (int gg = 0; gg < GW; ++gg)
#pragma unroll
        for (int ii = 0; ii < 2; ++ii) {
          const f32x4 v = acc[mt][gg][ii];
          buf_st16(rp, slot(split, (mt * GW + gg) * 2 + ii),
                   make_uint4(__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                              __float_as_uint(v[3])));
        }
    if (!arrive_last(&ga.ctr[tile - n_full], (unsigned)nsplit, reinterpret_cast<int*>(big_dsm))) return;
    // every split (this one too) has published: re-read all of them in split
    // order, two 16-row fragments' worth of loads in flight per round trip
#pragma unroll
    for (int mt = 0; mt < MTW; ++mt)
#pragma unroll
      for (int gg = 0; gg < GW; ++gg) {
        acc[mt][gg][0] = f32x4{0.f, 0.f, 0.f, 0.f};
        acc[mt][gg][1] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    for (int sp = 0; sp < nsplit; ++sp) {
#pragma unroll
      for (int mt0 = 0; mt0 < MTW; mt0 += 2) {
        uint4 u[2][GW][2];
#pragma unroll
        for (int dm = 0; dm < 2; ++dm)
#pragma unroll
          for (int gg = 0; gg < GW; ++gg)
#pragma unroll
            for (int ii = 0; ii < 2; ++ii)
              if (mt0 + dm < MTW) u[dm][gg][ii] = buf_ld_act(rp, slot(sp, ((mt0 + dm) * GW + gg) * 2 + ii));
#pragma unroll
        for (int dm = 0; dm < 2; ++dm)
#pragma unroll
          for (int gg = 0; gg < GW; ++gg)
#pragma unroll
            for (int ii = 0; ii < 2; ++ii)
              if (mt0 + dm < MTW) {
                const uint4 v = u[dm][gg][ii];
                acc[mt0 + dm][gg][ii] += f32x4{__uint_as_float(v.x), __uint_as_float(v.y),
                                               __uint_as_float(v.z), __uint_as_float(v.w)};
              }
      }
    }
    __syncthreads();   // the arrival flag's LDS word is reused below
  }

  // ---- epilogue, 32 rows of the wave's tile at a time: math() in the MFMA
  //      layout into this wave's LDS region, then 16-byte row stores.  The
  //      row scales of every pass are loaded at once, and each pass's
  //      store-side operands one pass ahead, so the passes share one memory
  //      round trip instead of paying one each.  The staging region is the
  //      wave's own and LDS runs a wave's accesses in order: no barriers.
  constexpr int LROW = 32 * GW + 4;       // floats per staged row
  constexpr int SC = Epi::SLOT_CHUNKS;
  constexpr int NP = (MTW + 1) / 2;       // passes of 32 rows (16 in the last of an odd MTW)
  constexpr int GS = GW * SC;             // store items per staged row (divides 64)
  constexpr int RPI = 64 / GS;            // staged rows per store round
  constexpr int NIT = 32 / RPI;           // store rounds per pass
  float* stg = reinterpret_cast<float*>(big_dsm) + w * 32 * LROW;
  const int mw = m0 + wm * (BM / 2);      // first row of the wave's tile
  const int gg_s = (l % GS) / SC, qc_s = l % SC;   // this lane's store column: group, chunk
  const int g_s = g0 + wn * GW + gg_s;
  float rr[NP][2][4];
#pragma unroll
  for (int pass = 0; pass < NP; ++pass)
#pragma unroll
    for (int mh = 0; mh < 2; ++mh)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int row = min(mw + 16 * (2 * pass + mh) + 4 * (l >> 4) + j, ga.M - 1);
        rr[pass][mh][j] = ga.r ? ga.r[row] : 1.f;
      }
  typename Epi::Pre pre[2][NIT];
  auto load_pre = [&](int pass, typename Epi::Pre (&pp)[NIT]) {
#pragma unroll
    for (int it = 0; it < NIT; ++it)
      pp[it] = epi.pre(min(mw + 32 * pass + it * RPI + l / GS, ga.M - 1), min(g_s, ga.n_groups - 1), qc_s);
  };
  load_pre(0, pre[0]);
#pragma unroll
  for (int pass = 0; pass < NP; ++pass) {
    const int pass_rows = min(32, 16 * (MTW - 2 * pass));
    if (pass + 1 < NP) load_pre(pass + 1, pre[(pass + 1) & 1]);
#pragma unroll
    for (int mh = 0; mh < 2; ++mh) {
      const int mt = min(2 * pass + mh, MTW - 1);
      if (2 * pass + mh >= MTW) break;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int rl = 16 * mh + 4 * (l >> 4) + j;
#pragma unroll
        for (int gg = 0; gg < GW; ++gg) {
          const float2 o = epi.math(acc[mt][gg][0][j], acc[mt][gg][1][j], rr[pass][mh][j]);
          stg[rl * LROW + 32 * gg + (l & 15)] = o.x;
          stg[rl * LROW + 32 * gg + 16 + (l & 15)] = o.y;
        }
      }
    }
    asm volatile("" ::: "memory");
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int rl = it * RPI + l / GS;
      const int row = mw + 32 * pass + rl;
      if (rl < pass_rows && row < ga.M && g_s < ga.n_groups)
        epi.store(row, g_s, qc_s, &stg[rl * LROW + 32 * gg_s], pre[pass & 1][it]);
    }
    asm volatile("" ::: "memory");
  }
}

template <int BM, int BN, bool AFRAG, class Epi>
static void launch_big(const GemmArgs& ga, const Epi& e, const BigPlan& p, hipStream_t st) {
  constexpr int NFR = (BM / 16) + (BN / 32) * 2;
  const size_t smem = 4 * (size_t)NFR * kFragBytes;
  auto kern = big_gemm_kernel<BM, BN, AFRAG, Epi>;
  static bool attr_set = false;
  if (!attr_set) {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    attr_set = true;
  }
  const int n_tm = (ga.M + BM - 1) / BM, n_tn = (ga.n_groups + BN / 32 - 1) / (BN / 32);
  const int units = p.n_full + (n_tm * n_tn - p.n_full) * p.splits;
  hipLaunchKernelGGL(kern, dim3(units), dim3(256), smem, st, ga, e, n_tm, n_tn, p.n_full, p.splits);
}

// 256 x 256 tiles where they fill the chip (about one workgroup per compute
// unit or more), else 128 x 128 where those do, else 128 x 64.  Costs in
// rounds of whole-tile work per compute unit.  Two K splits of every tile
// (long K only) where rounds of half-length units beat whole ones with a
// fifth in hand (measured: 3 whole rounds of 256 x 256 tiles beat 5 half
// ones; 2 whole rounds of 128 x 64 tiles lose to 3 half ones).  Or whole
// tiles for the full rounds and only the last, partial round's tiles in s K
// slices that fit in one round: its cost counted at 1/s + 0.3.
BigPlan big_plan(int M, int n_groups, int K) {
  const long cus = device_cus();
  auto tiles = [&](int bm, int bn) { return (long)((M + bm - 1) / bm) * ((n_groups + bn / 32 - 1) / (bn / 32)); };
  BigPlan p{128, 64, 1, 0, 0};
  if (tiles(256, 256) >= cus * 15 / 16) {
    p = BigPlan{256, 256, 1, 0, 0};
    // 224-row tiles where they leave less padding per round of the chip
    // (1560 rows: 7 x 224 = 1568 against 7 x 256 = 1792)
    auto round_rows = [&](int bm) { return (tiles(bm, 256) + cus - 1) / cus * bm; };
    if (round_rows(224) < round_rows(256)) p.bm = 224;
  }
  else if (tiles(128, 128) >= cus * 15 / 16) p = BigPlan{128, 128, 1, 0, 0};
  else if (K >= 4096 && (K / 64) % 2 == 0 && 2 * tiles(128, 128) >= cus && tiles(128, 128) <= cus) {
    // a long K over too few 128 x 128 tiles for the chip: those tiles in two
    // K slices (two workgroups fit a compute unit; a 64 x 64 wave tile reads
    // half the LDS bytes per MFMA of 128 x 64's 64 x 32): the video down
    // projection 74.7 -> 69.0 us against 128 x 64 tiles in two slices (with
    // K = 1536 the O projection went 18 -> 28 us, so short K keeps 128 x 64)
    const int t = (int)tiles(128, 128);
    return BigPlan{128, 128, 2, t, 0};
  }
  p.tiles = (int)tiles(p.bm, p.bn);
  p.n_full = p.tiles;
  // too few tiles to give half the compute units one (a 768-row chunk's O and
  // down projections: 96 tiles): every tile in K slices, the most (of 2, 4,
  // 8; at least 8 k-steps each) that keep to one workgroup per compute unit.
  // Filling every unit instead made the 768-token prefix stage faster alone
  // (1.76 against 1.86 ms) but slower beside the denoise loop on a second
  // stream, whose small kernels then wait for free units (14.49 against
  // 14.36 ms for the prefix stage and a 16-step loop).
  if (2 * p.tiles <= cus) {
    auto most_splits = [&](long t) {
      int best = 1;
      for (int s = 2; s <= 8; s *= 2) {
        if ((K / 64) % s != 0 || K / 32 / s < 8 || t * s > cus) break;
        best = s;
      }
      return best;
    };
    int best = most_splits(p.tiles);
    // 128 x 128 tiles in more slices where one unit then moves fewer operand
    // bytes ((rows + columns) x its K length): the 768-row O and down
    // projections as 48 tiles in 4 slices (524 KiB per unit) instead of 96
    // in 2 (768 KiB): the 18-layer prefix stage 1,821 -> 1,795 us on one
    // box; 8 slices, two units per compute unit, took 27.6 against 19.6 us
    const long t2 = tiles(128, 128);
    const int s2 = most_splits(t2);
    if (t2 * s2 >= p.tiles * best && 256L * K / s2 < (long)(p.bm + p.bn) * K / best) {
      p = BigPlan{128, 128, 1, (int)t2, (int)t2};
      best = s2;
    }
    if (best > 1 && p.tiles <= kBigMaxSplitTiles) {
      p.splits = best;
      p.n_full = 0;
    }
    return p;
  }
  const long ks = K / 64;
  const long r1 = (p.tiles + cus - 1) / cus, r2 = (2L * p.tiles + cus - 1) / cus;   // r2 half-length rounds
  double best = (double)r1;
  if (K >= 4096 && ks % 2 == 0 && 10 * r2 <= 16 * r1) {
    best = 0.5 * (double)r2;
    p.n_full = 0;
    p.splits = 2;
  }
  const long full = p.tiles / cus * cus, tail = p.tiles - full;
  if (full > 0 && tail > 0) {
    for (int s = 8; s >= 2; --s) {
      if (ks % s != 0 || tail * s > cus || ks / s < 2) continue;
      const double c = (double)(full / cus) + 1.0 / s + 0.3;
      if (c < best) {
        p.n_full = (int)full;
        p.splits = s;
      }
      break;
    }
  }
  if (p.splits > 1 && p.tiles - p.n_full > kBigMaxSplitTiles) {   // more split tiles than counters
    p.splits = 1;
    p.n_full = p.tiles;
  }
  return p;
}
size_t big_part_floats(const BigPlan& p) {
  return p.splits > 1 ? (size_t)(p.tiles - p.n_full) * p.splits * p.bm * p.bn : 0;
}

template <bool AFRAG, class Epi>
static void launch_tiled(const GemmArgs& ga, const Epi& e, hipStream_t st) {
  const BigPlan p = big_plan(ga.M, ga.n_groups, ga.K);
  if (p.bm == 256) launch_big<256, 256, AFRAG>(ga, e, p, st);
  else if (p.bm == 224) launch_big<224, 256, AFRAG>(ga, e, p, st);
  else if (p.bn == 128) launch_big<128, 128, AFRAG>(ga, e, p, st);
  else launch_big<128, 64, AFRAG>(ga, e, p, st);
}

// ============================================================================ dispatch
void launch_gemm_qkv(const GemmArgs& ga, const EpiQKV& e, hipStream_t st) { launch_tiled<true>(ga, e, st); }
void launch_gemm_residual(const GemmArgs& ga, const EpiResidual& e, hipStream_t st) {
  launch_tiled<true>(ga, e, st);
}
void launch_gemm_gateup(const GemmArgs& ga, const EpiGateUp& e, hipStream_t st) { launch_tiled<true>(ga, e, st); }

// ============================================================================ RMS rows
// r[m] = (sum_k x[m][k]^2 / K + eps)^-1/2.  One workgroup per 16-row tile:
// wave w takes the k-tiles kt = w, w + 4, ...; with frag (x in operand order,
// fa_index over mt_of(M) row tiles) each load is one whole 1 KiB fragment.
// Row-major x is read two k-tiles at a time, each load 8 rows x one whole
// 128-byte line (the rows of one parity; lane l: row 2 ((l >> 1) & 7) + h,
// k-tile l & 1, 16-byte chunk l >> 4), and one swap of adjacent lanes turns
// the pair of loads into the two k-tiles' fragments, which are stored whole
// into the operand-order copy when xf is given (16 rows x 64 bytes per load
// instead touched twice the cache lines).  Lane l holds row l % 16 of each
// fragment; lanes of a row fold by shuffles, the waves meet in LDS.  Rows
// past M (clamped loads) fill the last tile's padding; their r is not written.
__global__ __launch_bounds__(256) void rms_rows_kernel(const bf16_t* __restrict__ x, int M, int K,
                                                       int frag, float eps, float* __restrict__ r,
                                                       bf16_t* __restrict__ xf) {
  __shared__ float part[4][16];
  const int mt = blockIdx.x, MT = mt_of(M);
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int nkt = K >> 5;
  auto slot = [&](int kt) { return ((size_t)(kt * MT + mt) * 64 + l) * 8; };   // lane's slot of fragment (kt, mt)
  float s = 0.f;
  // loads go out in batches (indices past the end clamped: loaded, not used)
  // ahead of their first use
  if (frag) {
    for (int kt0 = w; kt0 < nkt; kt0 += 32) {
      uint4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        v[u] = *reinterpret_cast<const uint4*>(x + slot(min(kt0 + 4 * u, nkt - 1)));
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (kt0 + 4 * u < nkt) s += sumsq8(v[u]);
    }
  } else if ((nkt & 1) == 0) {
    const bool odd = (l & 1) != 0;
    const int npr = nkt >> 1;
    const bf16_t* xr[2];
#pragma unroll
    for (int h = 0; h < 2; ++h)
      xr[h] = x + (size_t)min(16 * mt + 2 * ((l >> 1) & 7) + h, M - 1) * K + 32 * (l & 1) + 8 * (l >> 4);
    for (int kp0 = w; kp0 < npr; kp0 += 16) {
      uint4 ld[4][2];
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int h = 0; h < 2; ++h)   // h = 0: even rows, 1: odd rows
          ld[u][h] = *reinterpret_cast<const uint4*>(xr[h] + 64 * min(kp0 + 4 * u, npr - 1));
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int kp = kp0 + 4 * u;
        if (kp >= npr) break;
        const uint4 a = ld[u][0], b = ld[u][1];
        const uint32_t av[4] = {a.x, a.y, a.z, a.w}, bv[4] = {b.x, b.y, b.z, b.w};
        uint32_t f0[4], f1[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          // quad_perm [1, 0, 3, 2]: each lane reads its neighbour l ^ 1
          const uint32_t as = (uint32_t)__builtin_amdgcn_mov_dpp((int)av[e], 0xB1, 0xF, 0xF, true);
          const uint32_t bs = (uint32_t)__builtin_amdgcn_mov_dpp((int)bv[e], 0xB1, 0xF, 0xF, true);
          f0[e] = odd ? bs : av[e];
          f1[e] = odd ? bv[e] : as;
        }
        const uint4 v0{f0[0], f0[1], f0[2], f0[3]}, v1{f1[0], f1[1], f1[2], f1[3]};
        if (xf) {
          *reinterpret_cast<uint4*>(xf + slot(2 * kp)) = v0;
          *reinterpret_cast<uint4*>(xf + slot(2 * kp + 1)) = v1;
        }
        s += sumsq8(v0) + sumsq8(v1);
      }
    }
  } else {
    const int row = min(16 * mt + (l & 15), M - 1);
#pragma unroll 8
    for (int kt = w; kt < nkt; kt += 4) {
      const uint4 v = *reinterpret_cast<const uint4*>(x + (size_t)row * K + kt * 32 + 8 * (l >> 4));
      if (xf) *reinterpret_cast<uint4*>(xf + slot(kt)) = v;
      s += sumsq8(v);
    }
  }
  s += __shfl_xor(s, 16);
  s += __shfl_xor(s, 32);
  if (l < 16) part[w][l] = s;
  __syncthreads();
  if (threadIdx.x < 16) {
    const int m = 16 * mt + threadIdx.x;
    const float t = ((part[0][threadIdx.x] + part[1][threadIdx.x]) + part[2][threadIdx.x]) +
                    part[3][threadIdx.x];
    if (m < M) r[m] = rsqrtf(t / (float)K + eps);
  }
}

void launch_rms_rows(const bf16_t* x, int M, int K, bool frag, float eps, float* r, bf16_t* xf,
                     hipStream_t st) {
  rms_rows_kernel<<<mt_of(M), 256, 0, st>>>(x, M, K, frag ? 1 : 0, eps, r, xf);
}

}  // namespace blk
