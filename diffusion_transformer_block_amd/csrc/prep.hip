// Weight-prep kernels: gain folds, QKV / gate-up concatenation into MFMA
// fragments, RoPE tables and the flow head's folded embedding tables.
//
// [RT] = reading note on "Running VLAs at Real-time Speed" (Ma et al.,
// arXiv:2510.26742v1).  §4.1: an RMSNorm gain g is absorbed into the next
// linear layer as diag(g) W.  §4.2: the action linear and the linear after
// the [action, time] concatenation have no nonlinearity between them, so
// their weights are pre-multiplied; the time branch at the fixed timesteps is
// tabulated and folded into the bias ahead of SiLU.  §4.3: Q, K and V become
// one matrix; the fixed position-encoding quantities are precomputed.
#include "common.h"
#include "internal.h"

namespace blk {

// Round a float64 value to bf16 once (round to nearest even): round to float32
// with round-to-odd first (exact sticky bit), then to bf16.  Round-to-odd at
// 24 bits followed by RNE at 8 bits equals a single RNE at 8 bits.
__device__ __forceinline__ bf16_t f64_to_bf16(double v) {
  float t = __double2float_rz(v);
  if ((double)t != v) t = __uint_as_float(__float_as_uint(t) | 1u);
  return f2bf(t);
}

// One thread per (fragment, lane): 8 bf16 of W'[k][n] = g[k] * W[k][n], taken
// from up to three source matrices concatenated along columns.
__global__ void pack_frag_kernel(PackSrc src, ColMapArgs cm, int K, int n_groups,
                                 uint8_t* __restrict__ dst) {
  const int KT = K / 32;
  const size_t total = (size_t)n_groups * KT * 2 * 64;
  for (size_t idx = blockIdx.x * (size_t)blockDim.x + threadIdx.x; idx < total;
       idx += (size_t)gridDim.x * blockDim.x) {
    const int lane = (int)(idx & 63);
    const size_t frag = idx >> 6;
    const int i = (int)(frag & 1);
    const int kt = (int)((frag >> 1) % KT);
    const int g = (int)((frag >> 1) / KT);
    int col = col_of_group(cm, g, i) + (lane & 15);
    // locate the source matrix holding logical column `col`
    int m = 0;
    while (m + 1 < src.n_src && col >= src.cols[m]) { col -= src.cols[m]; ++m; }
    const bf16_t* w = src.w[m];
    const int ld = src.cols[m];
    uint32_t out[4];
    for (int e = 0; e < 8; e += 2) {
      bf16_t h[2];
      for (int q = 0; q < 2; ++q) {
        const int k = kt * 32 + 8 * (lane >> 4) + e + q;
        const bf16_t wb = w[(size_t)k * ld + col];
        if (src.gain) {
          h[q] = f64_to_bf16((double)src.gain[k] * (double)bf2f(wb));
        } else {
          h[q] = wb;
        }
      }
      out[e / 2] = (uint32_t)h[0] | ((uint32_t)h[1] << 16);
    }
    *(uint4*)(dst + frag * kFragBytes + lane * 16) = make_uint4(out[0], out[1], out[2], out[3]);
  }
}

// cos / sin of pos * base^(-2j/d) for pos < max_pos, j < d/2 (float64 math).
__global__ void rope_table_kernel(int max_pos, int half, double base, float* cos_t,
                                  float* sin_t) {
  const size_t total = (size_t)max_pos * half;
  for (size_t idx = blockIdx.x * (size_t)blockDim.x + threadIdx.x; idx < total;
       idx += (size_t)gridDim.x * blockDim.x) {
    const int j = (int)(idx % half);
    const double pos = (double)(idx / half);
    const double theta = pow(base, -2.0 * (double)j / (double)(2 * half));
    const double ang = pos * theta;
    cos_t[idx] = (float)cos(ang);
    sin_t[idx] = (float)sin(ang);
  }
}

// W_fused[a][n] = sum_j W1[a][j] W2[j][n] (W2's action rows), float64 sums.
__global__ void fold_action_kernel(const bf16_t* __restrict__ w1, const bf16_t* __restrict__ w2,
                                   int A, int D, float* __restrict__ w_fused) {
  const int n = blockIdx.x * blockDim.x + threadIdx.x;
  const int a = blockIdx.y;
  if (n >= D || a >= A) return;
  double acc = 0.0;
  for (int j = 0; j < D; ++j) acc += (double)bf2f(w1[(size_t)a * D + j]) * (double)bf2f(w2[(size_t)j * D + n]);
  w_fused[(size_t)a * D + n] = (float)acc;
}

// table[s][n] = sum_j b1[j] W2[j][n] + sum_j tau_j(t_s) W2[D + j][n] + b2[n],
// tau = [sin(t w_j), cos(t w_j)], w_j = 10000^(-j / (D/2)); float64 sums.
// dt[s] = t_{s+1} - t_s with t_{n_steps} = 0.
__global__ void fold_time_kernel(const float* __restrict__ b1, const bf16_t* __restrict__ w2,
                                 const float* __restrict__ b2, int D, Schedule sched,
                                 float* __restrict__ table, float* __restrict__ dt) {
  const int n = blockIdx.x * blockDim.x + threadIdx.x;
  const int s = blockIdx.y;
  if (n >= D || s >= sched.n) return;
  const double t = sched.t[s];
  const int half = D / 2;
  double acc = (double)b2[n];
  for (int j = 0; j < D; ++j) acc += (double)b1[j] * (double)bf2f(w2[(size_t)j * D + n]);
  for (int j = 0; j < D; ++j) {
    const int jj = j < half ? j : j - half;
    const double omega = pow(10000.0, -(double)jj / (double)half);
    const double tau = j < half ? sin(t * omega) : cos(t * omega);
    acc += tau * (double)bf2f(w2[(size_t)(D + j) * D + n]);
  }
  table[(size_t)s * D + n] = (float)acc;
  if (n == 0) {
    const double t_next = (s + 1 < sched.n) ? sched.t[s + 1] : 0.0;
    dt[s] = (float)(t_next - t);
  }
}

// out[i] = (float)in_bf16[i] * (gain ? gain[i / cols] : 1)   (exact float32 product)
__global__ void widen_kernel(const bf16_t* __restrict__ in, const float* __restrict__ gain,
                             int cols, size_t n, float* __restrict__ out) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x) {
    float v = bf2f(in[i]);
    if (gain) v *= gain[i / cols];
    out[i] = v;
  }
}

__global__ void copy_f32_kernel(const float* __restrict__ in, size_t n, float* __restrict__ out) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    out[i] = in[i];
}

static int grid_for(size_t n) {
  size_t g = (n + 255) / 256;
  return (int)(g > 8192 ? 8192 : (g == 0 ? 1 : g));
}

void launch_pack_frag(const PackSrc& src, const ColMapArgs& cm, int K, int n_groups, uint8_t* dst,
                      hipStream_t st) {
  const size_t total = (size_t)n_groups * (K / 32) * 2 * 64;
  pack_frag_kernel<<<grid_for(total), 256, 0, st>>>(src, cm, K, n_groups, dst);
}

void launch_rope_table(int max_pos, int half, double base, float* cos_t, float* sin_t,
                       hipStream_t st) {
  rope_table_kernel<<<grid_for((size_t)max_pos * half), 256, 0, st>>>(max_pos, half, base, cos_t,
                                                                      sin_t);
}

void launch_fold_action(const bf16_t* w1, const bf16_t* w2, int A, int D, float* w_fused,
                        hipStream_t st) {
  fold_action_kernel<<<dim3((D + 255) / 256, A), 256, 0, st>>>(w1, w2, A, D, w_fused);
}

void launch_fold_time(const float* b1, const bf16_t* w2, const float* b2, int D,
                      const Schedule& sched, float* table, float* dt, hipStream_t st) {
  fold_time_kernel<<<dim3((D + 255) / 256, sched.n), 256, 0, st>>>(b1, w2, b2, D, sched, table,
                                                                   dt);
}

void launch_widen(const bf16_t* in, const float* gain, int cols, size_t n, float* out,
                  hipStream_t st) {
  widen_kernel<<<grid_for(n), 256, 0, st>>>(in, gain, cols, n, out);
}

void launch_copy_f32(const float* in, size_t n, float* out, hipStream_t st) {
  copy_f32_kernel<<<grid_for(n), 256, 0, st>>>(in, n, out);
}

}  // namespace blk
