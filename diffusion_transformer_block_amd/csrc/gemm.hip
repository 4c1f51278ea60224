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
// GEMM of skinny.h): 256 x 256 (or 128 x 128) output tiles, both operands
// moved into LDS by the buffer-load DMA as MFMA fragments, 2 x 2 waves of
// 16 x 16 x 32 MFMAs, XCD-aware tile order (big_gemm_kernel below).
#include "common.h"
#include "internal.h"
#include "skinny.h"

namespace blk {

// ============================================================================ large-chunk GEMM
// LDS DMA of one 1 KiB fragment: lane l's 16 bytes at voffset land at lds + 16 l.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, void* lds, int voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff, 0,
                                           0, 0);
}

// BM x BN output tile per workgroup (4 waves in a 2 x 2 grid), K steps of 64.
// Each stage holds the tile's A and B operands in LDS as 1 KiB MFMA
// fragments -- A (row-major activations) gathered by the DMA as 16 rows x
// 64 bytes per fragment, B (packed weights) one contiguous fragment each --
// in two buffers: a wave reads all of its fragments of the current stage
// into registers, then issues the next stage's DMA (after its reads, so they
// do not wait on it), then runs its MFMAs.
template <int BM, int BN, class Epi>
__global__ __launch_bounds__(256) void big_gemm_kernel(GemmArgs ga, Epi epi, int n_tm) {
  extern __shared__ __attribute__((aligned(1024))) uint8_t big_dsm[];
  constexpr int BK = 64;
  constexpr int MTB = BM / 16;            // 16-row tiles per block
  constexpr int GB = BN / 32;             // 32-column groups per block
  constexpr int MTW = MTB / 2, GW = GB / 2;
  constexpr int AFR = MTB * 2, BFR = GB * 4, NFR = AFR + BFR;
  constexpr int STAGE = NFR * kFragBytes;
  constexpr int PER = NFR / 4;            // fragments each wave moves per stage
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l = tid & 63;
  const int wm = w >> 1, wn = w & 1;
  // The hardware deals workgroups round-robin over the 8 XCDs: give each XCD
  // a contiguous run of tiles, taken in bands of GM row tiles with the column
  // tiles outer, so the tiles an XCD runs at once share row and column blocks
  // in its L2.
  const int nwg = gridDim.x, id = blockIdx.x;
  const int xcd = id & 7, jx = id >> 3, qx = nwg >> 3, rx = nwg & 7;
  const int tile = xcd * qx + min(xcd, rx) + jx;
  constexpr int GM = 4;
  const int n_tn = nwg / n_tm;
  const int band = tile / (GM * n_tn), tib = tile - band * GM * n_tn;
  const int rows_b = min(GM, n_tm - band * GM);
  const int tm = band * GM + tib % rows_b, tn = tib / rows_b;
  const int m0 = tm * BM, g0 = tn * GB;
  const int KT = ga.K >> 5, nk = ga.K / BK;

  const __amdgpu_buffer_rsrc_t ra = make_rsrc(ga.A, (size_t)ga.M * ga.lda * 2);
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(ga.Bp, (size_t)ga.n_groups * KT * 2 * kFragBytes);
  // this wave's fragments of a stage: f = w + 4 i (A fragments first); rows
  // and groups past the matrix are clamped (their results are not stored)
  int voff[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int f = w + 4 * i;
    if (f < AFR) {
      const int kt = f / MTB, mt = f - kt * MTB;
      const int row = min(m0 + 16 * mt + (l & 15), ga.M - 1);
      voff[i] = (row * ga.lda + 32 * kt + 8 * (l >> 4)) * 2;
    } else {
      const int fb = f - AFR, gg = fb >> 2, kt = (fb >> 1) & 1, ii = fb & 1;
      voff[i] = (int)frag_offset(min(g0 + gg, ga.n_groups - 1), kt, ii, KT) + 16 * l;
    }
  }
  auto issue = [&](int s, int buf) {
    uint8_t* base = big_dsm + buf * STAGE;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int f = w + 4 * i;
      if (f < AFR) dma16(ra, base + f * kFragBytes, voff[i] + s * BK * 2);
      else dma16(rb, base + f * kFragBytes, voff[i] + s * 2 * 2 * kFragBytes);
    }
  };

  f32x4 acc[MTW][GW][2];
#pragma unroll
  for (int a = 0; a < MTW; ++a)
#pragma unroll
    for (int b = 0; b < GW; ++b) {
      acc[a][b][0] = f32x4{0.f, 0.f, 0.f, 0.f};
      acc[a][b][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

  issue(0, 0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  for (int s = 0; s < nk; ++s) {
    const int cur = s & 1;
    const uint8_t* base = big_dsm + cur * STAGE;
    uint4 af[2][MTW], bfv[2][GW][2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int mt = 0; mt < MTW; ++mt)
        af[kt][mt] =
            *reinterpret_cast<const uint4*>(base + (kt * MTB + wm * MTW + mt) * kFragBytes + 16 * l);
#pragma unroll
      for (int gg = 0; gg < GW; ++gg)
#pragma unroll
        for (int ii = 0; ii < 2; ++ii)
          bfv[kt][gg][ii] = *reinterpret_cast<const uint4*>(
              base + (AFR + (wn * GW + gg) * 4 + kt * 2 + ii) * kFragBytes + 16 * l);
    }
    if (s + 1 < nk) issue(s + 1, cur ^ 1);
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int mt = 0; mt < MTW; ++mt)
#pragma unroll
        for (int gg = 0; gg < GW; ++gg)
#pragma unroll
          for (int ii = 0; ii < 2; ++ii)
            acc[mt][gg][ii] = mfma16(as_bf16x8(af[kt][mt]), as_bf16x8(bfv[kt][gg][ii]), acc[mt][gg][ii]);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the next stage has landed
    __syncthreads();                                    // and every wave is done with this one
  }

  // ---- epilogue, 32 rows of the wave's tile at a time: math() in the MFMA
  //      layout into this wave's LDS region, then 16-byte row stores
  constexpr int LROW = 32 * GW + 4;       // floats per staged row
  constexpr int SC = Epi::SLOT_CHUNKS;
  float* stg = reinterpret_cast<float*>(big_dsm) + w * 32 * LROW;
#pragma unroll
  for (int pass = 0; pass < MTW / 2; ++pass) {
#pragma unroll
    for (int mh = 0; mh < 2; ++mh) {
      const int mt = 2 * pass + mh;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int rl = 16 * mh + 4 * (l >> 4) + j;
        const int row = min(m0 + wm * (BM / 2) + 16 * mt + 4 * (l >> 4) + j, ga.M - 1);
        const float r = ga.r ? ga.r[row] : 1.f;
#pragma unroll
        for (int gg = 0; gg < GW; ++gg) {
          const int g = min(g0 + wn * GW + gg, ga.n_groups - 1);
          const float2 o = epi.math(row, g, l & 15, acc[mt][gg][0][j], acc[mt][gg][1][j], r);
          stg[rl * LROW + 32 * gg + (l & 15)] = o.x;
          stg[rl * LROW + 32 * gg + 16 + (l & 15)] = o.y;
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < 32 * GW * SC / 64; ++it) {
      const int idx = it * 64 + l;
      const int rl = idx / (GW * SC), rem = idx - rl * (GW * SC);
      const int gg = rem / SC, qc = rem - gg * SC;
      const int row = m0 + wm * (BM / 2) + 32 * pass + rl;
      const int g = g0 + wn * GW + gg;
      const float4 lo = *reinterpret_cast<const float4*>(&stg[rl * LROW + 32 * gg + 8 * qc]);
      const float4 hi = *reinterpret_cast<const float4*>(&stg[rl * LROW + 32 * gg + 8 * qc + 4]);
      const float v[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
      if (row < ga.M && g < ga.n_groups) epi.store8(row, g, qc, v);
    }
    __syncthreads();
  }
}

template <int BM, int BN, class Epi>
static void launch_big(const GemmArgs& ga, const Epi& e, hipStream_t st) {
  constexpr int NFR = (BM / 16) * 2 + (BN / 32) * 4;
  const size_t smem = 2 * (size_t)NFR * kFragBytes;
  auto kern = big_gemm_kernel<BM, BN, Epi>;
  static bool attr_set = false;
  if (!attr_set) {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    attr_set = true;
  }
  const int n_tm = (ga.M + BM - 1) / BM, n_tn = (ga.n_groups + BN / 32 - 1) / (BN / 32);
  hipLaunchKernelGGL(kern, dim3(n_tm * n_tn), dim3(256), smem, st, ga, e, n_tm);
}

// 256 x 256 tiles where they fill the chip (about one workgroup per compute
// unit or more), 128 x 128 otherwise.
template <class Epi>
static void launch_tiled(const GemmArgs& ga, const Epi& e, hipStream_t st) {
  const long big_tiles = (long)((ga.M + 255) / 256) * ((ga.n_groups + 7) / 8);
  if (big_tiles >= (long)device_cus() * 15 / 16) launch_big<256, 256>(ga, e, st);
  else launch_big<128, 128>(ga, e, st);
}

// ============================================================================ dispatch
void launch_gemm_qkv(const GemmArgs& ga, const EpiQKV& e, hipStream_t st) { launch_tiled(ga, e, st); }
void launch_gemm_residual(const GemmArgs& ga, const EpiResidual& e, hipStream_t st) {
  launch_tiled(ga, e, st);
}
void launch_gemm_gateup(const GemmArgs& ga, const EpiGateUp& e, hipStream_t st) { launch_tiled(ga, e, st); }

// ============================================================================ RMS rows
// r[m] = (sum_k x[m][k]^2 / K + eps)^-1/2, one wave per row
__global__ __launch_bounds__(256) void rms_rows_kernel(const bf16_t* __restrict__ x, int M, int K,
                                                       float eps, float* __restrict__ r) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int l = threadIdx.x & 63;
  if (row >= M) return;
  const bf16_t* p = x + (size_t)row * K;
  float s = 0.f;
  for (int k = 8 * l; k < K; k += 512) s += sumsq8(*reinterpret_cast<const uint4*>(p + k));
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) s += __shfl_xor(s, o);
  if (l == 0) r[row] = rsqrtf(s / (float)K + eps);
}

void launch_rms_rows(const bf16_t* x, int M, int K, float eps, float* r, hipStream_t st) {
  rms_rows_kernel<<<(M + 3) / 4, 256, 0, st>>>(x, M, K, eps, r);
}

}  // namespace blk
