// Internal launch interfaces of the block-stage kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "common.h"

namespace blk {

// ---------------------------------------------------------------- weight prep
struct PackSrc {
  const bf16_t* w[3];  // source matrices [K][cols[m]], concatenated along columns
  int cols[3];
  int n_src;
  const float* gain;   // optional [K] gain folded into every row
};

constexpr int kMaxSteps = 64;
struct Schedule {
  int n;
  double t[kMaxSteps];
};

void launch_pack_frag(const PackSrc& src, const ColMapArgs& cm, int K, int n_groups, uint8_t* dst,
                      hipStream_t st);
void launch_rope_table(int max_pos, int half, double base, float* cos_t, float* sin_t,
                       hipStream_t st);
void launch_fold_action(const bf16_t* w1, const bf16_t* w2, int A, int D, float* w_fused,
                        hipStream_t st);
void launch_fold_time(const float* b1, const bf16_t* w2, const float* b2, int D,
                      const Schedule& sched, float* table, float* dt, hipStream_t st);
void launch_widen(const bf16_t* in, const float* gain, int cols, size_t n, float* out,
                  hipStream_t st);
void launch_copy_f32(const float* in, size_t n, float* out, hipStream_t st);

// ---------------------------------------------------------------- GEMM epilogues
// Each epilogue receives one output pair: row m, group g, column c < 16 inside
// the group's tiles, the fp32 sums v0 (tile 0) and v1 (tile 1), and the row
// scale r (the RMS statistic, or 1 when the GEMM has no norm ahead of it).
// store1 takes a single tile i of group g (only for plain column groups).
// Loads of activations and all stores are device-coherent, so a consumer
// workgroup of the same persistent kernel can read them.

// Fused QKV: scale by r, rotate (Q, K) pairs, scatter into Q / K_new / V_new.
struct EpiQKV {
  bf16_t* q;            // [M][Hq d]
  bf16_t* kn;           // stream b at b * new_stride, [T][Hkv][d]
  bf16_t* vn;
  int64_t new_stride;
  const float* cos_t;   // [max_pos][d/2]
  const float* sin_t;
  int T, P, Hq, Hkv, d;

  __device__ __forceinline__ void store(int m, int g, int c, float v0, float v1, float r) const {
    const int b = m / T, t = m - b * T;
    const int gpr = d >> 5;
    const int n_rot_groups = (Hq + Hkv) * d / 32;
    v0 *= r;
    v1 *= r;
    if (g < n_rot_groups) {
      const int head = g / gpr;
      const int j = 16 * (g - head * gpr) + c;  // < d/2
      const int half = d >> 1;
      const size_t ti = (size_t)(P + t) * half + j;
      const float cs = cos_t[ti], sn = sin_t[ti];
      const float lo = v0 * cs - v1 * sn;
      const float hi = v0 * sn + v1 * cs;
      bf16_t* dst;
      if (head < Hq) {
        dst = q + (size_t)m * Hq * d + (size_t)head * d;
      } else {
        dst = kn + (size_t)b * new_stride + ((size_t)t * Hkv + (head - Hq)) * d;
      }
      st_act(dst + j, lo);
      st_act(dst + j + half, hi);
    } else {
      const int col0 = 32 * (g - n_rot_groups) + c;
      bf16_t* base = vn + (size_t)b * new_stride + (size_t)t * Hkv * d;
      st_act(base + col0, v0);       // V row layout [Hkv][d] is contiguous in col
      st_act(base + col0 + 16, v1);
    }
  }
};

// out[m][n] = res[m][n] + acc (residual add; O projection and down projection).
struct EpiResidual {
  const bf16_t* res;
  bf16_t* out;
  int ld;
  __device__ __forceinline__ void store(int m, int g, int c, float v0, float v1, float) const {
    const size_t o = (size_t)m * ld + 32 * g + c;
    st_act(out + o, ld_act(res + o) + v0);
    st_act(out + o + 16, ld_act(res + o + 16) + v1);
  }
  __device__ __forceinline__ void store1(int m, int g, int i, int c, float v, float) const {
    const size_t o = (size_t)m * ld + 32 * g + 16 * i + c;
    st_act(out + o, ld_act(res + o) + v);
  }
};

// out[m][j] = SiLU(r * gate) * (r * up), j = 16 g + c (gate/up interleave).
struct EpiGateUp {
  bf16_t* out;
  int ld;
  __device__ __forceinline__ void store(int m, int g, int c, float v0, float v1, float r) const {
    st_act(out + (size_t)m * ld + 16 * g + c, silu(v0 * r) * (v1 * r));
  }
};

// ---------------------------------------------------------------- GEMM launch
struct GemmArgs {
  const bf16_t* A;      // activations [M][K], row-major, leading dimension lda
  int lda;
  int M, K;
  const uint8_t* Bp;    // packed weight fragments
  int n_groups;
  // row scale r (the RMS statistic; may be NULL = 1)
  const float* r;
};

// The large-chunk (M > 64) tiled GEMMs.
void launch_gemm_qkv(const GemmArgs& ga, const EpiQKV& e, hipStream_t st);
void launch_gemm_residual(const GemmArgs& ga, const EpiResidual& e, hipStream_t st);
void launch_gemm_gateup(const GemmArgs& ga, const EpiGateUp& e, hipStream_t st);

// Chunks of at most this many rows (B * T) take the small-chunk path.
constexpr int kSkinnyMaxM = 64;

// ---------------------------------------------------------------- RMS statistics
// r[m] = (sum_k x[m][k]^2 / K + eps)^-1/2
void launch_rms_rows(const bf16_t* x, int M, int K, float eps, float* r, hipStream_t st);

// ---------------------------------------------------------------- attention
struct AttnArgs {
  const bf16_t* q;          // [B*T][Hq d]
  const bf16_t* kp;         // stream b at b * prefix_stride, [P][Hkv][d]
  const bf16_t* vp;
  int64_t prefix_stride;
  const bf16_t* kn;         // stream b at b * new_stride, [T][Hkv][d]
  const bf16_t* vn;
  int64_t new_stride;
  bf16_t* o;                // [B*T][Hq d]
  int B, T, P, Hq, Hkv, d;
  int splits, keys_per_split;
  float scale_log2;         // log2(e) / sqrt(d)
  float* part_o;            // split partials
  float* part_ml;
  unsigned* counters;
};
void attn_plan(int B, int T, int P, int Hq, int Hkv, int d, int* splits, int* keys_per_split);
size_t attn_part_o_floats(int B, int T, int P, int Hq, int Hkv, int d);
size_t attn_part_ml_floats(int B, int T, int P, int Hq, int Hkv, int d);
size_t attn_counters(int B, int T, int P, int Hq, int Hkv, int d);
void launch_attention(const AttnArgs& a, hipStream_t st);

// ---------------------------------------------------------------- small-chunk path
// (M = B * T <= 64): activations in operand order, see skinny.h / attn_small.h
struct SkArgs;
struct EpiQkvS;
struct EpiResidS;
struct EpiGateUpS;
struct AttnSmArgs;
int device_cus();
// Plan of a skinny GEMM: K splits and 32-column groups per workgroup
// (splits = -1: no valid plan, a row-major input too wide to stage)
struct SkPlan {
  int splits, gpw;
};
SkPlan sk_plan(int M, int K, int n_groups, bool a_rowmajor);
size_t sk_part_floats(int M, int K, int n_groups, bool a_rowmajor);
int sk_nb(int KW, int gpw, int MT);
void launch_sk_qkv(const SkArgs& ga, int gpw, bool a_rowmajor, const EpiQkvS& e, hipStream_t st);
void launch_sk_resid(const SkArgs& ga, int gpw, const EpiResidS& e, hipStream_t st);
void launch_sk_gateup(const SkArgs& ga, int gpw, const EpiGateUpS& e, hipStream_t st);
void attn_sm_plan(int B, int T, int P, int Hq, int Hkv, int* splits, int* kps);
size_t attn_sm_part_o_elems(int B, int T, int P, int Hq, int Hkv, int d);
size_t attn_sm_part_ml_floats(int B, int T, int P, int Hq, int Hkv, int d);
void launch_attn_sm(const AttnSmArgs& a, int head_dim, hipStream_t st);

// ---------------------------------------------------------------- flow head
struct FlowEmbedArgs {
  const float* act;        // [N][A] current actions
  const float* state;      // [A]
  const float* w_fused;    // [A][D]
  const float* bias_row;   // [D] table row of this step
  const float* ws;         // [A][D]
  const float* bs;         // [D]
  bf16_t* z;               // [N][D] SiLU(a W_fused + bias)
  bf16_t* x0;              // [D] row 0 of X: state embedding
  int N, A, D;
};
void launch_flow_embed(const FlowEmbedArgs& a, hipStream_t st);

struct FlowVelArgs {
  const bf16_t* X;         // [N + 1][D], row 0 = state token
  const float* w_out;      // [D][A] (final gain folded)
  const float* b_out;      // [A]
  const float* a_in;       // [N][A]
  float* a_out;            // [N][A]
  const float* dt;         // device pointer to this step's dt
  int N, A, D;
  float eps;
};
void launch_flow_velocity(const FlowVelArgs& a, hipStream_t st);

}  // namespace blk
