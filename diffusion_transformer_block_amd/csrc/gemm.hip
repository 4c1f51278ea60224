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
// GEMM of skinny.h):
//  * tiled_gemm: 128 x 128 output tile per workgroup, K step 64,
//    A (activations) staged through double-buffered LDS, B (packed weight
//    fragments) loaded straight into registers one step ahead; 2 x 2 waves of
//    64 x 64 each.
#include "common.h"
#include "internal.h"
#include "skinny.h"

namespace blk {

// ============================================================================ tiled
template <class Epi>
__global__ __launch_bounds__(256) void tiled_gemm_kernel(GemmArgs ga, Epi epi) {
  constexpr int BM = 128, BK = 64, LDS_ROW = BK + 8;
  __shared__ __attribute__((aligned(16))) bf16_t As[2][BM * LDS_ROW];

  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63, lr = l & 15, lg = l >> 4;
  const int wm = w >> 1, wn = w & 1;
  const int nb = blockIdx.x, mb = blockIdx.y;
  const int KT = ga.K >> 5;
  const int nsteps = ga.K / BK;

  const bf16_t* ag[4];
  int lds_off[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int cidx = tid + 256 * q;
    const int row = cidx >> 3, col = (cidx & 7) * 8;
    const int grow = min(mb * BM + row, ga.M - 1);
    ag[q] = ga.A + (size_t)grow * ga.lda + col;
    lds_off[q] = row * LDS_ROW + col;
  }
  const uint4* bg[2];
#pragma unroll
  for (int gi = 0; gi < 2; ++gi) {
    const int gq = min(4 * nb + 2 * wn + gi, ga.n_groups - 1);
    bg[gi] = reinterpret_cast<const uint4*>(ga.Bp + frag_offset(gq, 0, 0, KT)) + l;
  }

  uint4 areg[4], breg[2][2][2];
#pragma unroll
  for (int q = 0; q < 4; ++q) areg[q] = *reinterpret_cast<const uint4*>(ag[q]);
#pragma unroll
  for (int gi = 0; gi < 2; ++gi)
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int i = 0; i < 2; ++i) breg[gi][kk][i] = bg[gi][(kk * 2 + i) * 64];
#pragma unroll
  for (int q = 0; q < 4; ++q) *reinterpret_cast<uint4*>(&As[0][lds_off[q]]) = areg[q];
  __syncthreads();

  f32x4 acc[4][4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int step = 0; step < nsteps; ++step) {
    const int cur = step & 1;
    const bool more = step + 1 < nsteps;
    uint4 bnext[2][2][2];
    if (more) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        areg[q] = *reinterpret_cast<const uint4*>(ag[q] + (size_t)(step + 1) * BK);
#pragma unroll
      for (int gi = 0; gi < 2; ++gi)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
          for (int i = 0; i < 2; ++i)
            bnext[gi][kk][i] = bg[gi][(((step + 1) * 2 + kk) * 2 + i) * 64];
    }
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const uint4 af = *reinterpret_cast<const uint4*>(
            &As[cur][(64 * wm + 16 * mt + lr) * LDS_ROW + 32 * kk + 8 * lg]);
#pragma unroll
        for (int gi = 0; gi < 2; ++gi)
#pragma unroll
          for (int i = 0; i < 2; ++i)
            acc[mt][2 * gi + i] =
                mfma16(as_bf16x8(af), as_bf16x8(breg[gi][kk][i]), acc[mt][2 * gi + i]);
      }
    }
    if (more) {
#pragma unroll
      for (int q = 0; q < 4; ++q) *reinterpret_cast<uint4*>(&As[cur ^ 1][lds_off[q]]) = areg[q];
#pragma unroll
      for (int gi = 0; gi < 2; ++gi)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
          for (int i = 0; i < 2; ++i) breg[gi][kk][i] = bnext[gi][kk][i];
    }
    __syncthreads();
  }

#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int gi = 0; gi < 2; ++gi) {
      const int g = 4 * nb + 2 * wn + gi;
      if (g >= ga.n_groups) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int row = mb * BM + 64 * wm + 16 * mt + 4 * lg + j;
        if (row < ga.M) {
          const float r = ga.r ? ga.r[row] : 1.f;
          epi.store(row, g, lr, acc[mt][2 * gi][j], acc[mt][2 * gi + 1][j], r);
        }
      }
    }
}

template <class Epi>
static void launch_tiled(const GemmArgs& ga, const Epi& e, hipStream_t st) {
  dim3 grid((ga.n_groups + 3) / 4, (ga.M + 127) / 128);
  tiled_gemm_kernel<Epi><<<grid, 256, 0, st>>>(ga, e);
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
