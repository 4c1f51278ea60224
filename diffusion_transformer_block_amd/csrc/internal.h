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
// The large-chunk GEMM finishes a tile in two phases.  math() sees one output
// pair in the MFMA layout -- the fp32 sums v0 (tile 0) and v1 (tile 1) of
// column c < 16 of a group's two tiles and the row scale r (the RMS
// statistic, or 1) -- and returns the group's staged slots c and 16 + c.  The
// slots go through LDS; store() then gets one row's 32 staged slots of group
// g and writes chunk q < SLOT_CHUNKS of them (16-byte stores), with the
// operands pre() loaded for it one pass of rows ahead.  The stores are plain:
// the next kernel reads them.

// Fused QKV: scale by r; in the store phase, rotate (Q, K) pairs (slot c =
// column j, slot 16 + c = column j + d/2 of the rotated head), with the
// cos / sin of 8 consecutive j loaded as two 16-byte vectors each; Q into the
// chunk attention's operand order (qa_index in skinny.h), K_new / V_new
// row-major.  Chunk q < 2 of a group covers slots 8 q .. 8 q + 7 and
// 16 + 8 q .. 16 + 8 q + 7 (both halves of a rotated pair).
struct EpiQKV {
  static constexpr int SLOT_CHUNKS = 2;
  bf16_t* q;
  bf16_t* kn;           // stream b at b * new_stride, [T][Hkv][d]
  bf16_t* vn;
  int64_t new_stride;
  const float* cos_t;   // [max_pos][d/2]
  const float* sin_t;
  int T, P, Hq, Hkv, d;
  int g_base;           // packed group of the GEMM's group 0 (> 0: a K/V-only run)
  const int* plen;      // device: stream b's prefix length (NULL: all P); token t at P_b + t

  __device__ __forceinline__ float2 math(float v0, float v1, float r) const {
    return make_float2(v0 * r, v1 * r);
  }
  // cos / sin of columns j .. j + 7 at row m's position: the index is valid
  // for every group (V groups ignore it), so the loads carry no condition and
  // a whole pass of them is issued before the first use
  struct Pre {
    float4 c0, c1, s0, s1;
  };
  __device__ __forceinline__ Pre pre(int m, int g, int qc) const {
    g += g_base;
    const int gpr = d >> 5;
    const int b = m / T;
    const size_t ti = (size_t)(stream_prefix(plen, P, b) + m - b * T) * (d >> 1) + 16 * (g % gpr) + 8 * qc;
    const float4* cp = reinterpret_cast<const float4*>(cos_t + ti);
    const float4* sp = reinterpret_cast<const float4*>(sin_t + ti);
    return {cp[0], cp[1], sp[0], sp[1]};
  }
  __device__ __forceinline__ void store(int m, int g, int qc, const float* srow, const Pre& p) const;
};

// out = res + acc (residual add; O projection and down projection).  res and
// out are each row-major [M][ld] or in operand order (fa_index, MT row tiles).
struct EpiResidual {
  static constexpr int SLOT_CHUNKS = 4;
  const bf16_t* res;
  int res_frag;
  bf16_t* out;
  int out_frag;
  int ld, MT;
  __device__ __forceinline__ float2 math(float v0, float v1, float) const {
    return make_float2(v0, v1);
  }
  // the residual chunk, loaded a pass ahead of the stores (out may alias res:
  // a pass's loads and stores cover the same rows, later passes other rows)
  struct Pre {
    uint4 r;
  };
  __device__ __forceinline__ Pre pre(int m, int g, int qc) const {
    const int c = 32 * g + 8 * qc;
    const size_t ro = res_frag ? fa_index(m, c, MT) : (size_t)m * ld + c;
    return {*reinterpret_cast<const uint4*>(res + ro)};
  }
  __device__ __forceinline__ void store(int m, int g, int qc, const float* srow, const Pre& p) const {
    const int c = 32 * g + 8 * qc;
    const size_t oo = out_frag ? fa_index(m, c, MT) : (size_t)m * ld + c;
    float x[8];
    unpack8(p.r, x);
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] += srow[8 * qc + e];
    *reinterpret_cast<uint4*>(out + oo) = pack8(x);
  }
};

// out[m][j] = SiLU(r * gate) * (r * up), j = 16 g + c (gate/up interleave):
// 16 slots per group, stored in operand order (fa_index, MT row tiles).
struct EpiGateUp {
  static constexpr int SLOT_CHUNKS = 2;
  bf16_t* out;
  int MT;
  __device__ __forceinline__ float2 math(float v0, float v1, float r) const {
    return make_float2(silu(v0 * r) * (v1 * r), 0.f);
  }
  struct Pre {};
  __device__ __forceinline__ Pre pre(int, int, int) const { return {}; }
  __device__ __forceinline__ void store(int m, int g, int qc, const float* srow, const Pre&) const {
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = srow[8 * qc + e];
    *reinterpret_cast<uint4*>(out + fa_index(m, 16 * g + 8 * qc, MT)) = pack8(v);
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
  // K splits (big_plan) and their scratch: fp32 partial tiles and one
  // self-resetting arrival counter per output tile (zero on entry)
  float* part;
  unsigned* ctr;
};

// Tile shape and K splits of a large-chunk GEMM, and the scratch they need.
// At most kBigMaxSplitTiles tiles run in K slices (their arrival counters are
// indexed by tile - n_full).
constexpr int kBigMaxSplitTiles = 2048;
struct BigPlan {
  int bm, bn, splits, tiles;
  int n_full;   // tiles run whole (the first n_full); the rest in `splits` K slices each
};
BigPlan big_plan(int M, int n_groups, int K);
size_t big_part_floats(const BigPlan& p);

// The large-chunk (M > 64) GEMMs; A in operand order (fa_index).
void launch_gemm_qkv(const GemmArgs& ga, const EpiQKV& e, hipStream_t st);
void launch_gemm_residual(const GemmArgs& ga, const EpiResidual& e, hipStream_t st);
void launch_gemm_gateup(const GemmArgs& ga, const EpiGateUp& e, hipStream_t st);

// Chunks of at most this many rows (B * T) take the small-chunk path.
constexpr int kSkinnyMaxM = 64;

// ---------------------------------------------------------------- RMS statistics
// r[m] = (sum_k x[m][k]^2 / K + eps)^-1/2
// xf (may be NULL) receives a row-major x in operand order.
void launch_rms_rows(const bf16_t* x, int M, int K, bool frag, float eps, float* r, bf16_t* xf,
                     hipStream_t st);


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
int sk_nb(int KW, int gpw, int MT, int max_nb);
void launch_sk_qkv(const SkArgs& ga, int gpw, bool a_rowmajor, const EpiQkvS& e, hipStream_t st);
void launch_sk_resid(const SkArgs& ga, int gpw, const EpiResidS& e, hipStream_t st,
                     const Prefetch& pf = {});
void launch_sk_gateup(const SkArgs& ga, int gpw, const EpiGateUpS& e, hipStream_t st);
// long_rows: set to 1 for 128-row blocks over one key slice (NULL: 64-row blocks only)
void attn_sm_plan(int B, int T, int P, int Hq, int Hkv, int* splits, int* kps, int* long_rows);
size_t attn_sm_part_o_elems(int B, int T, int P, int Hq, int Hkv, int d);
size_t attn_sm_part_ml_floats(int B, int T, int P, int Hq, int Hkv, int d);
void launch_attn_sm(const AttnSmArgs& a, int head_dim, hipStream_t st, const Prefetch& pf = {});

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
