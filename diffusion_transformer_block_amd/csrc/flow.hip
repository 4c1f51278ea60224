// Flow-matching head of the action expert: suffix embedding ahead of the
// layer stack and velocity + Euler update behind it.
//
// [RT] reading note on "Running VLAs at Real-time Speed" (Ma et al.,
// arXiv:2510.26742v1): §2 -- 63 action tokens plus the state token, actions
// padded to 32 dims, 10 flow-matching steps; §4.2 -- the action projection
// and the linear after the [action, time] concatenation are pre-multiplied
// (W_fused = W1 W2a) and the time branch at the fixed timesteps is a table
// folded into the bias ahead of SiLU.  The linear after SiLU (W3) runs as a
// skinny MFMA GEMM with a bias epilogue; these two kernels are the small
// float32 pieces around it.
#include "common.h"
#include "internal.h"

namespace blk {

// Block (row, column tile): rows 0..N-1 -> z[row] = SiLU(a[row] W_fused + bias);
// row N -> X row 0 = state Ws + bs (the state token, constant over steps but
// recomputed here so the loop needs no other kernel).  z ([N][D]) and X
// ([N + 1][D]) are in the skinny GEMMs' operand order (fa_index).
__global__ __launch_bounds__(256) void flow_embed_kernel(FlowEmbedArgs a) {
  __shared__ float vin[64];
  const int row = blockIdx.y;
  const int n = blockIdx.x * 256 + threadIdx.x;
  const bool state_row = row == a.N;
  if (threadIdx.x < a.A)
    vin[threadIdx.x] = state_row ? a.state[threadIdx.x] : a.act[(size_t)row * a.A + threadIdx.x];
  __syncthreads();
  if (n >= a.D) return;
  if (state_row) {
    float acc = a.bs[n];
    for (int k = 0; k < a.A; ++k) acc = fmaf(vin[k], a.ws[(size_t)k * a.D + n], acc);
    a.x0[fa_index(0, n, mt_of(a.N + 1))] = f2bf(acc);
  } else {
    float acc = a.bias_row[n];
    for (int k = 0; k < a.A; ++k) acc = fmaf(vin[k], a.w_fused[(size_t)k * a.D + n], acc);
    a.z[fa_index(row, n, mt_of(a.N))] = f2bf(silu(acc));
  }
}

void launch_flow_embed(const FlowEmbedArgs& a, hipStream_t st) {
  flow_embed_kernel<<<dim3((a.D + 255) / 256, a.N + 1), 256, 0, st>>>(a);
}

// One block per action row i: r = RMS(X[i + 1]); v[c] = r sum_k X[i+1][k] W_out'[k][c]
// + b_out[c]; a_out[i][c] = a_in[i][c] + dt v[c].  Thread t takes k = t, t + 256,
// ... and 32 columns at a time, its W_out' rows as 16-byte loads (all of them
// independent: one memory round trip); a wave folds its 64 lanes' 32 column
// sums in 5 exchange rounds (each lane keeps half of what it holds and sends
// the other half), the 4 waves' sums meet in LDS in a fixed order.  X is in
// operand order (fa_index, N + 1 rows).
// NK = k values per thread (a power of two >= D / 256): every load has a
// valid, clamped address and no condition, so a thread's loads are issued
// together rather than one round trip each; k >= D contributes x = 0.
template <int NK>
__global__ __launch_bounds__(256) void flow_velocity_kernel(FlowVelArgs a) {
  constexpr int CW = 32;              // columns per pass
  __shared__ float part[4][64];
  __shared__ float wsum[4];
  const int i = blockIdx.x;
  const int tid = threadIdx.x, l = tid & 63, w = tid >> 6;
  const int MT = mt_of(a.N + 1);
  float xk[NK];
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < NK; ++j) {
    const int k = tid + 256 * j;
    const float v = bf2f(a.X[fa_index(i + 1, min(k, a.D - 1), MT)]);
    xk[j] = k < a.D ? v : 0.f;
    ss = fmaf(xk[j], xk[j], ss);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) ss += __shfl_xor(ss, o);
  if (l == 0) wsum[w] = ss;
  __syncthreads();
  const float r = rsqrtf(((wsum[0] + wsum[1]) + (wsum[2] + wsum[3])) / (float)a.D + a.eps);
  const float dt = *a.dt;
  const bool vec = (a.A & 3) == 0;
  for (int c0 = 0; c0 < a.A; c0 += CW) {
    const int nc = min(CW, a.A - c0);
    float acc[CW];
#pragma unroll
    for (int c = 0; c < CW; ++c) acc[c] = 0.f;
    if (vec && nc == CW) {
      // all of the thread's W_out' rows in flight at once (in batches of up
      // to 4 rows = 128 registers), then the FMAs
      constexpr int JB = NK < 4 ? NK : 4;
#pragma unroll
      for (int j0 = 0; j0 < NK; j0 += JB) {
        float4 wv[JB][CW / 4];
#pragma unroll
        for (int jj = 0; jj < JB; ++jj) {
          const float* wr = a.w_out + (size_t)min(tid + 256 * (j0 + jj), a.D - 1) * a.A + c0;
#pragma unroll
          for (int c4 = 0; c4 < CW / 4; ++c4) wv[jj][c4] = *reinterpret_cast<const float4*>(wr + 4 * c4);
        }
#pragma unroll
        for (int jj = 0; jj < JB; ++jj)
#pragma unroll
          for (int c4 = 0; c4 < CW / 4; ++c4) {
            const float xv = xk[j0 + jj];
            acc[4 * c4] = fmaf(xv, wv[jj][c4].x, acc[4 * c4]);
            acc[4 * c4 + 1] = fmaf(xv, wv[jj][c4].y, acc[4 * c4 + 1]);
            acc[4 * c4 + 2] = fmaf(xv, wv[jj][c4].z, acc[4 * c4 + 2]);
            acc[4 * c4 + 3] = fmaf(xv, wv[jj][c4].w, acc[4 * c4 + 3]);
          }
      }
    } else {
#pragma unroll
      for (int j = 0; j < NK; ++j) {
        const float* wr = a.w_out + (size_t)min(tid + 256 * j, a.D - 1) * a.A + c0;
#pragma unroll
        for (int c = 0; c < CW; ++c) acc[c] = fmaf(xk[j], wr[min(c, nc - 1)], acc[c]);
      }
    }
    // fold the wave: after the round with offset o (16, 8, 4, 2, 1) a lane
    // holds the sums of o columns over 32 / o lanes; lanes with bit o set keep
    // the upper half.  Column of lane l at the end: the bits of l & 31.
#pragma unroll
    for (int o = 16; o >= 1; o >>= 1) {
      const bool up = (l & o) != 0;
#pragma unroll
      for (int c = 0; c < o; ++c) {
        const float send = up ? acc[c] : acc[c + o];
        const float got = __shfl_xor(send, o);
        acc[c] = (up ? acc[c + o] : acc[c]) + got;
      }
    }
    // lane l now holds column col(l) summed over its half-wave; add the other half
    const float v = acc[0] + __shfl_xor(acc[0], 32);
    int col = 0;
#pragma unroll
    for (int o = 16, b = 0; o >= 1; o >>= 1, ++b) col |= (l & o) ? o : 0;
    if (l < 32) part[w][col] = v;
    __syncthreads();
    if (tid < nc) {
      float vs = ((part[0][tid] + part[1][tid]) + part[2][tid]) + part[3][tid];
      vs = vs * r + a.b_out[c0 + tid];
      const size_t o = (size_t)i * a.A + c0 + tid;
      a.a_out[o] = a.a_in[o] + dt * vs;
    }
    __syncthreads();
  }
}

// The same velocity and Euler step for A a multiple of 32 (actions padded to
// 32 dims), with W_out' read coalesced: thread t takes the 4 columns 4 (t % 8)
// of a 32-column block over the rows t / 8 + 32 m, so a wave's load covers 8
// consecutive rows x 128 bytes (8 cache lines) instead of 64 rows x 16 bytes;
// the X row is staged once in LDS; the 32 threads of a column chunk (8 per
// wave) fold by shuffles and the 4 waves meet in LDS in a fixed order.
__global__ __launch_bounds__(256) void flow_velocity32_kernel(FlowVelArgs a) {
  __shared__ float xs[8192];          // D <= 8192 (checked by the caller)
  __shared__ float4 part[4][8];
  __shared__ float wsum[4];
  const int i = blockIdx.x;
  const int tid = threadIdx.x, l = tid & 63, w = tid >> 6;
  const int MT = mt_of(a.N + 1);
  float ss = 0.f;
  for (int k = tid; k < a.D; k += 256) {
    const float v = bf2f(a.X[fa_index(i + 1, k, MT)]);
    xs[k] = v;
    ss = fmaf(v, v, ss);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) ss += __shfl_xor(ss, o);
  if (l == 0) wsum[w] = ss;
  __syncthreads();
  const float r = rsqrtf(((wsum[0] + wsum[1]) + (wsum[2] + wsum[3])) / (float)a.D + a.eps);
  const float dt = *a.dt;
  const int cc = tid & 7, r0 = tid >> 3;
  for (int c0 = 0; c0 < a.A; c0 += 32) {
    const float* wb = a.w_out + c0 + 4 * cc;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 16
    for (int row = r0; row < a.D; row += 32) {
      const float4 wv = *reinterpret_cast<const float4*>(wb + (size_t)row * a.A);
      const float xv = xs[row];
      acc.x = fmaf(xv, wv.x, acc.x);
      acc.y = fmaf(xv, wv.y, acc.y);
      acc.z = fmaf(xv, wv.z, acc.z);
      acc.w = fmaf(xv, wv.w, acc.w);
    }
#pragma unroll
    for (int o = 8; o <= 32; o <<= 1) {
      acc.x += __shfl_xor(acc.x, o);
      acc.y += __shfl_xor(acc.y, o);
      acc.z += __shfl_xor(acc.z, o);
      acc.w += __shfl_xor(acc.w, o);
    }
    if (l < 8) part[w][l] = acc;
    __syncthreads();
    if (tid < 32) {
      const float* p0 = reinterpret_cast<const float*>(&part[0][0]);
      const float* p1 = reinterpret_cast<const float*>(&part[1][0]);
      const float* p2 = reinterpret_cast<const float*>(&part[2][0]);
      const float* p3 = reinterpret_cast<const float*>(&part[3][0]);
      float vs = ((p0[tid] + p1[tid]) + p2[tid]) + p3[tid];
      vs = vs * r + a.b_out[c0 + tid];
      const size_t o = (size_t)i * a.A + c0 + tid;
      a.a_out[o] = a.a_in[o] + dt * vs;
    }
    __syncthreads();
  }
}

void launch_flow_velocity(const FlowVelArgs& a, hipStream_t st) {
  if (a.A % 32 == 0 && a.D <= 8192) {
    flow_velocity32_kernel<<<a.N, 256, 0, st>>>(a);
    return;
  }
  const int need = (a.D + 255) / 256;   // D <= 8192 (checked by the caller)
  if (need <= 1) flow_velocity_kernel<1><<<a.N, 256, 0, st>>>(a);
  else if (need <= 2) flow_velocity_kernel<2><<<a.N, 256, 0, st>>>(a);
  else if (need <= 4) flow_velocity_kernel<4><<<a.N, 256, 0, st>>>(a);
  else if (need <= 8) flow_velocity_kernel<8><<<a.N, 256, 0, st>>>(a);
  else if (need <= 16) flow_velocity_kernel<16><<<a.N, 256, 0, st>>>(a);
  else flow_velocity_kernel<32><<<a.N, 256, 0, st>>>(a);
}

}  // namespace blk
