// Chunk attention over cached K/V: softmax(q K^T / sqrt(d)) V, no mask.
//
// [PS] AREX Feed article on PhysisServe: a chunk's denoise step reads the
// KV cache earlier chunks left at the current step (history / prefix) next to
// its own; history length is one of the drivers of stage latency.
// [RT] reading note on "Running VLAs at Real-time Speed" §2: the action
// expert's 64 query positions attend to the cached vision/language prefix.
//
// Layout of work: for stream b and kv-head hk the query rows are the
// (token, head) pairs of the G = Hq / Hkv query heads that share hk
// (row = t * G + head-in-group), so a multi-query head's 8 heads x 64 tokens
// form one 512-row problem against one K/V.  A workgroup takes 64 rows (16
// per wave) and one slice of the keys; the keys [prefix ; own chunk] are
// streamed in tiles of 32 through double-buffered LDS: the workgroup loads a
// tile once with coalesced 16-byte loads and all four waves use it, the tile
// after next is already in registers while the current one is computed.
//
// Per tile and wave:  S^T = K Q^T with MFMA 16x16x32 (K rows from LDS as the
// A operand, the wave's 16 query rows as the B operand kept in registers), so
// each lane holds 8 scores of ONE query row (lane % 16) -- exactly the B
// operand layout that O^T += V^T P^T needs, and the softmax statistics live
// in the same lane as that query's output columns: no shuffles besides the
// two cross-group max / sum steps.  V is written to LDS transposed, two keys
// per 32-bit store (bank-conflict free with a 72-byte row pitch), so V^T's A
// fragments are two 8-byte reads.  Online softmax in base 2 (scale folded
// into log2(e) / sqrt(d)).
//
// Key slices: when (rows / 64) x streams x kv-heads is far below the number of
// compute units, keys are split across workgroups; each writes its unnormalised
// O, its running max and sum, and the last-arriving workgroup of a row block
// (device-scope counter, reset by that workgroup) combines the slices in order.
#include "attn_dev.h"
#include "common.h"
#include "internal.h"

namespace blk {


template <int HD>
__global__ __launch_bounds__(256) void chunk_attn_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) AttnSmem<HD> sm;
  attn_task<HD>(a, blockIdx.x, blockIdx.y, blockIdx.z, sm);
}

void attn_plan(int B, int T, int P, int Hq, int Hkv, int d, int* splits, int* keys_per_split) {
  (void)d;

  const int G = Hq / Hkv;
  const int n_rb = (G * T + 63) / 64;
  const long wgs = (long)n_rb * B * Hkv;
  const int L = P + T;
  int s = 1;
  if (wgs < 32) {
    s = (int)((32 + wgs - 1) / wgs);
    const int max_s = (L + 2 * kKeyTile - 1) / (2 * kKeyTile);  // at least two key tiles per slice
    if (s > max_s) s = max_s;
    if (s < 1) s = 1;
  }
  int kps = (L + s - 1) / s;
  kps = (kps + kKeyTile - 1) / kKeyTile * kKeyTile;
  if (kps < kKeyTile) kps = kKeyTile;
  s = (L + kps - 1) / kps;
  if (s < 1) s = 1;
  *splits = s;
  *keys_per_split = kps;
}

size_t attn_part_o_floats(int B, int T, int P, int Hq, int Hkv, int d) {
  int s, kps;
  attn_plan(B, T, P, Hq, Hkv, d, &s, &kps);
  if (s == 1) return 0;
  const size_t n_rb = (size_t)((Hq / Hkv) * T + 63) / 64;
  return (size_t)s * B * Hkv * n_rb * 64 * d;
}

size_t attn_part_ml_floats(int B, int T, int P, int Hq, int Hkv, int d) {
  int s, kps;
  attn_plan(B, T, P, Hq, Hkv, d, &s, &kps);
  if (s == 1) return 0;
  const size_t n_rb = (size_t)((Hq / Hkv) * T + 63) / 64;
  return (size_t)s * B * Hkv * n_rb * 64 * 2;
}

size_t attn_counters(int B, int T, int P, int Hq, int Hkv, int d) {
  (void)P;
  (void)d;
  const size_t n_rb = (size_t)((Hq / Hkv) * T + 63) / 64;
  return (size_t)B * Hkv * n_rb;
}

void launch_attention(const AttnArgs& a, hipStream_t st) {
  const int G = a.Hq / a.Hkv;
  const int n_rb = (G * a.T + 63) / 64;
  dim3 grid(n_rb, a.B * a.Hkv, a.splits);
  switch (a.d) {
    case 64: chunk_attn_kernel<64><<<grid, 256, 0, st>>>(a); break;
    case 128: chunk_attn_kernel<128><<<grid, 256, 0, st>>>(a); break;
    default: chunk_attn_kernel<256><<<grid, 256, 0, st>>>(a); break;
  }
}

}  // namespace blk
