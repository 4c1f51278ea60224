// Arguments of the persistent stage kernel (stage.hip).
#pragma once
#include <hip/hip_runtime.h>

#include "internal.h"

namespace blk {

enum StagePhase : int { kPhQKV = 0, kPhATT, kPhCMB, kPhO, kPhGU, kPhD, kPhEMB, kPhW3, kPhVEL, kPhCount };
constexpr int kStageMaxLayers = 64;
constexpr int kStageMaxFlags = 1024;   // tasks (flag indices) per phase
// arrival counters: kShards per phase type, kShardWords apart (128 bytes)
constexpr int kShards = 32;
constexpr int kShardWords = 32;
static_assert(kPhCount * kShards * kShardWords <= kPhCount * kStageMaxFlags,
              "the counters fit the workspace's flag region");

// Task t of a phase runs on workgroup (w0 + t mod nw); n_flags tasks publish a flag.
struct PhaseMap {
  int w0, nw, n_tasks, n_flags;
};

struct StageArgs {
  int flow;                 // 0: n_layers blocks on x -> y; 1: the denoise loop
  int n_layers;
  int layer_first;          // block mode: first layer of the packed stack
  int n_steps;              // flow: denoise steps
  int B, T, P, M;
  int D, F, Hq, Hkv, d;
  float eps;
  // packed weights
  const uint8_t* packed;
  size_t layer0, layer_bytes, off_qkv, off_o, off_gu, off_d;
  const float* cos_t;
  const float* sin_t;
  // activations: x / y are the caller's row-major block input / output (block
  // mode); everything else is in the skinny GEMMs' operand order
  const bf16_t* x;
  bf16_t* y;
  bf16_t* xb[2];            // layer inputs / outputs between layers (flow: X)
  bf16_t* q;                // attention operand order
  bf16_t* o;
  bf16_t* h;
  bf16_t* a;
  bf16_t* kn;
  bf16_t* vn;
  int64_t new_stride;
  const bf16_t* kp[kStageMaxLayers];   // block mode: [0] (streams at prefix_stride)
  const bf16_t* vp[kStageMaxLayers];
  int64_t prefix_stride;
  // K splits of the GEMM steps (last arriver reduces) and their scratch
  int split_qkv, split_o, split_gu, split_d, split_w3;
  int gpw_qkv, gpw_o, gpw_gu, gpw_d, gpw_w3;   // 32-column groups per task
  float* part;
  unsigned* ctr_qkv;
  unsigned* ctr_o;
  unsigned* ctr_gu;
  unsigned* ctr_d;
  // attention: key slices and their partials, merge tasks
  int att_splits, att_kps, att_merge_tasks;
  float scale_log2;
  bf16_t* att_part_o;
  float* att_part_ml;
  // flow head
  int N, A;
  const float* w_fused;
  const float* table;
  const float* dt;
  const uint8_t* w3;
  const float* b3;
  const float* ws_f;
  const float* bs;
  const float* w_out;
  const float* b_out;
  const float* noise;
  const float* state;
  float* actions;
  bf16_t* z;
  // synchronisation words (workspace, zero-filled before first use)
  unsigned* flags;          // arrival counters [kPhCount][kShards] (kShardWords apart)
  unsigned* done_ctr;
  unsigned* abort_word;
  PhaseMap ph[kPhCount];
};

size_t stage_smem_bytes(int head_dim);
// Workgroups of the persistent grid (one per compute unit when a workgroup fits),
// 0 if the kernel cannot be resident on every unit.
int stage_grid(int head_dim, int rows);
hipError_t launch_stage(const StageArgs& sa, int nwg, hipStream_t st);

}  // namespace blk
