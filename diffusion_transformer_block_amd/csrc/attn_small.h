// Attention of a small query chunk over [cached prefix ; the chunk's own keys]
// as a device task shared by the standalone kernel and the persistent stage
// kernel.
//
// [PS] = AREX Feed article on PhysisServe, section on splitting the pipeline
// per denoise step and block: a stage runs one block for a chunk of query
// tokens against the cached KV of earlier chunks plus its own;
// [RT] = reading note on "Running VLAs at Real-time Speed" (Ma et al.,
// arXiv:2510.26742v1) §2: the action
// expert's 64 query tokens attend to the cached prefix and to each other with
// no causal mask inside the chunk.
//
// The rows of one (stream b, kv head hk) are the G = Hq / Hkv query heads of
// each of the T tokens, row ar = t G + gh; they all read that kv head's keys,
// so one K/V tile serves a block of rows.  A task takes a row block and one
// slice of the keys, in steps of 64 keys:
//  * K / V tiles move one step ahead by LDS DMA into double-buffered,
//    unpadded LDS tiles whose 16-byte chunks are XOR-swizzled per row (no
//    bank conflicts for the K fragment reads or the transposed V reads);
//  * 64-row blocks: wave w takes 32 query rows (w % 2) and one 32-key half
//    (w / 2) of every step; 128-row blocks (LONG, long key runs): wave w takes
//    32 rows and both halves, so a tile serves twice the rows and the halves
//    need no merge; 64-row blocks split by output dims (DSPLIT): wave w takes
//    32 rows (w % 2), both key halves for the scores (each pair of waves
//    computes them twice) and half of the head dims (w / 2) for O, so the
//    halves need no merge either; 32 x 32 x 16 MFMAs throughout (twice the
//    operand reuse of 16 x 16 tiles);
//  * S^T = K Q^T: K rows as the A operand (LDS), Q^T as the B operand held in
//    registers (the QKV epilogue stores Q in exactly that operand order,
//    qa_index), so a lane holds 16 keys of one query row;
//  * online softmax per row in base 2 (scores pre-scaled by log2(e)/sqrt(d));
//    the output is rescaled only when a row's max grows by more than 2^8,
//    checked once per 32-key half, or once per tile where a wave takes both
//    halves;
//  * O^T += V^T P^T: P^T is the B operand straight from the score registers
//    (slot e of the u-th 16-key step is S^T value 8 u + e, keys
//    16 u + 4 (l/32) + e or 16 u + 8 + 4 (l/32) + e - 4), V^T the A operand
//    read out of the row-major V tile with ds_read_b64_tr_b16, which hands
//    lane i of each 16-lane group element i % 4 of the 8 bytes at lane
//    4 k + i / 4 (k < 4): pointing lane i at key row 4 k' + i / 4, dims
//    4 (i % 4) .. + 3 yields V[key k][dim i] in that key order;
//  * (64-row blocks over key halves) the two key halves of a row pair merge
//    through an LDS hand-off in register order, each wave finishing half the
//    d tiles; lanes then store whole 16-byte chunks (lane pairs l, l ^ 32
//    swap halves).  One key slice writes the normalised rows straight into
//    the O projection's operand order (every mode); several slices publish bf16 partials
//    normalised by their own sum plus (max, sum), which a separate merge step
//    (attn_combine_task, one thread per 8 output bytes, all slices' loads in
//    flight together) combines in slice order.  Many small slices keep every
//    workgroup to about one memory round trip.
#pragma once
#include "common.h"
#include "skinny.h"

#include <type_traits>
#include <utility>

namespace blk {

struct AttnSmArgs {
  const bf16_t* q;        // qa_index order
  const bf16_t* kp;       // prefix K: stream b at b * prefix_stride, [P][Hkv][d]
  const bf16_t* vp;
  int64_t prefix_stride;
  const bf16_t* kn;       // own K: stream b at b * new_stride, [T][Hkv][d]
  const bf16_t* vn;
  int64_t new_stride;
  bf16_t* o;              // fa_index order of [B*T][Hq*d]
  int B, T, P, Hq, Hkv;
  int splits, kps;        // key slices and keys per slice (multiple of 32)
  float scale_log2;       // log2(e) / sqrt(d)
  bf16_t* part_o;         // [splits][n_rbt][64 * d] (normalised partials, attn_part_slot order)
  float* part_ml;         // [splits][n_rbt][64][2] (max, sum)
  int long_rows;          // 1: 128-row blocks over a single key slice (attn_sm_task LONG)
  const int* plen;        // device: per-stream prefix lengths (<= P; P sizes the key slices) or NULL
};

constexpr int kAttnMaxSplits = 16;

// A slice partial of a 64-row block holds 16-byte chunks (row r < 64, 8-dim
// chunk c) in the O projection's operand order, restricted to the block:
// 16 rows x 4 chunks per group of 64 slots.  The attention's lanes then store
// 512-byte runs, and the merge step reads one slot per thread, coalesced.
__host__ __device__ inline int attn_part_slot(int r, int c) {
  return ((c >> 2) * 4 + (r >> 4)) * 64 + (r & 15) + 16 * (c & 3);
}

template <int HD>
struct AttnSmSmem {
  // K / V tiles of 64 key rows, unpadded: the 16-byte chunks of a row are
  // XOR-swizzled (attn_swz_k / attn_swz_v) so that the fragment reads hit
  // distinct banks.  After the key loop the K tiles carry the key-half
  // hand-off.
  bf16_t k[2][64 * HD];
  bf16_t v[2][64 * HD];
  float2 mlh[2][64];                 // per key half and row: (max, sum)
};

// Physical 16-byte chunk of logical chunk c of tile row r is c ^ swz(r).
// K is read as MFMA A fragments: 16 lanes take 16 consecutive rows at one
// chunk, so the swizzle must spread 16 rows over the 16 four-bank groups.
// V is read with ds_read_b64_tr_b16: 16 lanes take 4 consecutive rows x 4
// consecutive chunks (aligned to 4), so 4 rows must land in distinct groups
// of 4 chunks.  At HD 64 a row is 8 chunks (half the banks), so row parity
// contributes the other half.
template <int HD>
__device__ __forceinline__ int attn_swz_k(int r) {
  return HD >= 128 ? (r & 15) : ((r >> 1) & 7);
}
template <int HD>
__device__ __forceinline__ int attn_swz_v(int r) {
  return HD >= 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1);
}

__device__ __forceinline__ uint2 lds_tr16(const bf16_t* p) {
  typedef short v4s __attribute__((ext_vector_type(4)));
  const v4s v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)(p));
  return __builtin_bit_cast(uint2, v);
}

typedef float f32x16 __attribute__((ext_vector_type(16)));

// max of three floats in one instruction (v_maximum3_f32).  fmaxf would
// first quiet every MFMA result as a possible signalling NaN; the IEEE
// maximum needs no such pass, and as a builtin (not inline assembly) it lets
// the compiler insert the wait states between an MFMA and its reader.
__device__ __forceinline__ float max3_f32(float a, float b, float c) {
  return __builtin_elementwise_maximum(__builtin_elementwise_maximum(a, b), c);
}
// Instruction order of the S^T MFMAs and their K fragment reads (LDS): R
// reads first, then one read after each MFMA, so R reads stay in flight.
template <int R, int... I>
__device__ __forceinline__ void attn_sched_reads_ahead(std::integer_sequence<int, I...>) {
  __builtin_amdgcn_sched_group_barrier(0x100, R, 0);
  ((__builtin_amdgcn_sched_group_barrier(0x008, 1, 0), __builtin_amdgcn_sched_group_barrier(0x100, 1, 0 * I)), ...);
  __builtin_amdgcn_sched_group_barrier(0x008, R, 0);
}
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// One task: stream x kv head bh, row block rb, key slice ks.  Returns true
// if this workgroup wrote the block's final rows (a single key slice).
// Row blocks are 64 rows: wave w takes 32 rows (w % 2) and one 32-key half
// (w / 2) of every tile, and the halves merge at the end.  LONG (long key
// runs) makes them 128 rows: wave w takes 32 rows and both key halves of
// every tile in turn, so a K/V tile serves twice the rows and no merge is
// needed; its slice partials go out per 64-row half, as the merge step reads
// them.  DSPLIT keeps 64-row blocks without the merge: the two waves of a
// row tile both take every key (the same scores and probabilities, computed
// twice) and each accumulates O for half of the head dims.
template <int HD, bool LONG = false, bool DSPLIT = false, class Wait>
__device__ bool attn_sm_task(const AttnSmArgs& a, int bh_in, int rb_in, int ks_in, AttnSmSmem<HD>& sm,
                             Wait&& wait) {
  // task coordinates are workgroup-uniform; saying so keeps every buffer
  // descriptor built from them in scalar registers
  const int bh = __builtin_amdgcn_readfirstlane(bh_in);
  const int rb = __builtin_amdgcn_readfirstlane(rb_in);
  const int ks = __builtin_amdgcn_readfirstlane(ks_in);
  constexpr int NDS = HD / 16;                 // 16-wide d steps of S^T (32x32x16)
  constexpr int NDT = HD / 32;                 // 32-row d tiles of O^T
  constexpr int CPR = HD / 8;                  // 16-byte chunks per key row
  constexpr int NCH = 64 * CPR / 256;          // DMA passes per 64-key tile (K or V)
  constexpr unsigned TILE_BYTES = 64 * HD * 2;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index (uniform)
  const int l = tid & 63;
  const int rp = LONG ? w : (w & 1);          // 32-row tile of the block
  const int kh_w = w >> 1;                     // the wave's 32-key half of a tile (not LONG / DSPLIT)
  static_assert(!(LONG && DSPLIT), "one block mode");
  // (integer division runs on the vector unit; readfirstlane keeps the
  // quotients scalar)
  const int b = __builtin_amdgcn_readfirstlane(bh / a.Hkv), hk = bh - b * a.Hkv;
  const int G = __builtin_amdgcn_readfirstlane(a.Hq / a.Hkv);
  const int rows = G * a.T;
  const int n_rt = (rows + 31) >> 5;           // 32-row tiles of this (stream, kv head)
  // this stream's prefix length (streams of one call may differ; the key
  // slices are sized for the longest) and its keys
  const int Pb = __builtin_amdgcn_readfirstlane(stream_prefix(a.plen, a.P, b));
  const int L = Pb + a.T;
  const int key_begin = ks * a.kps;
  const int key_end = min(L, key_begin + a.kps);
  const int n_tiles = (key_end - key_begin + 63) >> 6;
  const int kvrow = a.Hkv * HD;

  // K / V sources: prefix (caller's cache, read once: streaming) and the
  // chunk's own rows (written by the QKV step, possibly earlier in the same
  // launch: device-coherent loads)
  const bf16_t* kpb = a.kp ? a.kp + (size_t)b * a.prefix_stride + (size_t)hk * HD : nullptr;
  const bf16_t* vpb = a.vp ? a.vp + (size_t)b * a.prefix_stride + (size_t)hk * HD : nullptr;
  const bf16_t* knb = a.kn + (size_t)b * a.new_stride + (size_t)hk * HD;
  const bf16_t* vnb = a.vn + (size_t)b * a.new_stride + (size_t)hk * HD;
  // Tiles move by LDS DMA, 1 KiB per wave and pass: thread tid fills 16-byte
  // slot c0 of tile rows kk0 + j RPJ (j < NCH) with the row's logical chunk
  // c0 ^ swz(row).  Rows past the slice repeat its last key (finite values;
  // their scores are masked and their probabilities are exactly 0).
  constexpr int RPJ = 256 / CPR;               // key rows per pass of the workgroup
  const int kk0 = tid / CPR, c0 = tid - kk0 * CPR;
  const unsigned lds_k = __builtin_amdgcn_readfirstlane(lds_u32(&sm.k[0][0]));
  const unsigned lds_v = __builtin_amdgcn_readfirstlane(lds_u32(&sm.v[0][0]));
  auto load_tile = [&](int tile, int buf) {
    const int row0 = key_begin + 64 * tile;
    const bool prefix_only = row0 + 64 <= Pb;   // uniform
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      const int r = kk0 + j * RPJ;
      const int key = min(row0 + r, key_end - 1);
      const bool pre = key < Pb;
      const size_t ro = (size_t)(pre ? key : key - Pb) * kvrow;
      const bf16_t* kg = (pre ? kpb : knb) + ro + 8 * (c0 ^ attn_swz_k<HD>(r));
      const bf16_t* vg = (pre ? vpb : vnb) + ro + 8 * (c0 ^ attn_swz_v<HD>(r));
      const unsigned off = buf * TILE_BYTES + (j * 256 + w * 64) * 16;
      if (prefix_only) {
        dma16_nt(lds_k + off, kg);
        dma16_nt(lds_v + off, vg);
      } else {
        dma16_sc1(lds_k + off, kg);
        dma16_sc1(lds_v + off, vg);
      }
    }
  };

  __syncthreads();   // a previous task's readers of sm are done (the DMA writes it)
  // the first tile, if wholly in the prefix, does not depend on earlier work
  // and starts before the wait
  const bool pre0 = key_begin + 64 <= Pb;
  if (n_tiles > 0 && pre0) load_tile(0, 0);
  if (!wait()) {
    __builtin_amdgcn_s_waitcnt(0x0F70);   // no DMA may land after the workgroup ends
    return false;
  }
  if (n_tiles <= 0) {
    // a key slice past this stream's keys (a stream with a shorter prefix
    // than the call's longest): its rows' (max, sum) are (-inf, 0), which the
    // merge weights by zero (several slices exist whenever one can be empty)
    constexpr int BR = LONG ? 128 : 64;
    const int n_rb64 = (rows + 63) >> 6;
    const int n_rbt64 = a.B * a.Hkv * n_rb64;
    const int arow = BR * rb + tid;
    if (tid < BR && arow < rows) {
      const __amdgpu_buffer_rsrc_t rpm =
          make_rsrc(a.part_ml + ((size_t)ks * n_rbt64 + bh * n_rb64 + (arow >> 6)) * 128, 512);
      buf_st8(rpm, (arow & 63) * 8, __float_as_uint(-INFINITY), __float_as_uint(0.f));
    }
    return false;
  }
  if (!pre0) load_tile(0, 0);

  // this wave's 32 query rows: Q^T fragments (B operand), one per d step
  const int rt = __builtin_amdgcn_readfirstlane(min((LONG ? 4 : 2) * rb + rp, n_rt - 1));
  const __amdgpu_buffer_rsrc_t rq =
      make_rsrc(a.q + (size_t)(bh * n_rt + rt) * NDS * 512, (size_t)NDS * kFragBytes);
  uint4 qf[NDS];
#pragma unroll
  for (int s = 0; s < NDS; ++s) qf[s] = buf_ld_act(rq, s * kFragBytes + l * 16);
  // Q and tile 0 land here, before tile 1 is issued: the compiler counts
  // only Q among the loads, and a DMA still in flight behind Q would make
  // its waits for Q (at the head of the key loop) wait for that DMA too.
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  if (n_tiles > 1) load_tile(1, 1);

  // O^T d tiles this wave accumulates: all, or (DSPLIT) half, from d tile dbase
  constexpr int NDO = DSPLIT ? NDT / 2 : NDT;
  const int dbase = DSPLIT ? (w >> 1) * NDO : 0;
  // O^T accumulators: the slice's first tile (every slice has one) writes
  // them with zero C operands, so they need no zero fill
  f32x16 o[NDO];
  // running reference max (may trail the true max by up to 2^8, see below) and sum
  float m_run = -INFINITY, l_run = 0.f;
  __syncthreads();

  // lane roles: query row l % 32 of this wave's 32 rows; S^T keys
  // 32 kh + 8 (v/4) + 4 (l/32) + v%4 of the 64-key tile, v < 16
  const int hl = l >> 5;
  const int p16 = l & 15;
  // K fragment (A operand): row 32 kh + l % 32, logical chunk 2 s + hl, i.e.
  // physical chunk 2 s ^ xk: byte (32 s) ^ kx of the row
  const unsigned kx = 16 * (hl ^ attn_swz_k<HD>(l & 31));
  // V^T operand (transposed LDS reads): d = 32 dt + 16 ((l/16) % 2) + 4 (p16 % 4),
  // key rows 32 kh + 16 u + 4 hl + p16 / 4 (+ 8 for the second read): logical
  // chunk 4 dt + cl, physical 4 (dt ^ (swz / 4)) + cl, byte (64 dt) ^ vx + 16 cl
  const int vrow = 4 * hl + (p16 >> 2);
  const unsigned vt_off0 = vrow * HD * 2 + 16 * (2 * ((l >> 4) & 1) + ((p16 & 3) >> 1)) + 8 * (p16 & 1);
  const unsigned vx = 16 * attn_swz_v<HD>(vrow);

  // key halves this wave takes of every tile: both (LONG, DSPLIT) or its own
  constexpr int NH = (LONG || DSPLIT) ? 2 : 1;
  // S^T accumulation chains per half: two (even / odd d steps) for a single
  // half, one per half when two halves already interleave
  constexpr int NC = NH == 1 ? 2 : 1;
  constexpr int VB = NDO < 4 ? NDO : 4;   // transposed V reads issued ahead of their MFMAs
  const float sc = a.scale_log2;
  auto step = [&](int it, auto cur_c, auto first_c) {
    constexpr int cur = decltype(cur_c)::value;          // LDS buffer of tile it
    constexpr bool FIRST = decltype(first_c)::value;     // it == 0
    // ---- S^T (32 keys x 32 rows) of each half: K fragments read from LDS in
    //      batches ahead of their MFMAs
    f32x16 sacc[NH][NC];
#pragma unroll
    for (int h = 0; h < NH; ++h)
#pragma unroll
      for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int v = 0; v < 16; ++v) sacc[h][c][v] = 0.f;
    constexpr int KB = NDS < 8 ? NDS : 8;   // K fragments read ahead of their MFMAs
#pragma unroll
    for (int s0 = 0; s0 < NDS; s0 += KB) {
      uint4 kf[NH][KB];
      // (read in the MFMAs' order)
#pragma unroll
      for (int s = 0; s < KB; ++s)
#pragma unroll
        for (int h = 0; h < NH; ++h) {
          const int kh = NH == 2 ? h : kh_w;
          const uint8_t* kr = reinterpret_cast<const uint8_t*>(&sm.k[cur][(32 * kh + (l & 31)) * HD]);
          kf[h][s] = *reinterpret_cast<const uint4*>(kr + ((32u * (s0 + s)) ^ kx));
        }
#pragma unroll
      for (int s = 0; s < KB; ++s)
#pragma unroll
        for (int h = 0; h < NH; ++h)
          sacc[h][s % NC] = mfma32(as_bf16x8(kf[h][s]), as_bf16x8(qf[s0 + s]), sacc[h][s % NC]);
    }
    // K fragment reads kept four ahead of their MFMAs: left to itself the
    // compiler reads each just before its MFMA and waits on it
    constexpr int KRA = NH * NDS < 4 ? NH * NDS : 4;
    attn_sched_reads_ahead<KRA>(std::make_integer_sequence<int, NH * NDS - KRA>{});
    f32x16 sv[NH];
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      sv[h] = sacc[h][0];
      if constexpr (NC == 2) sv[h] += sacc[h][1];
    }
    // keys past the slice exist only in its last tile: their scores become
    // -inf (a uniform branch), and v_exp_f32 maps them to exactly 0
    if (key_begin + 64 * it + 64 > key_end) {
#pragma unroll
      for (int h = 0; h < NH; ++h) {
        const int base = key_begin + 64 * it + 32 * (NH == 2 ? h : kh_w);
#pragma unroll
        for (int v = 0; v < 16; ++v)
          if (base + 8 * (v >> 2) + 4 * hl + (v & 3) >= key_end) sv[h][v] = -INFINITY;
      }
    }
    if constexpr (NH == 2) {
      // ---- both key halves: one reference max per tile (one rescale
      //      decision), then each half's probabilities and O^T += V^T P^T
      //      (two 16-key steps; P^T slots e <-> S^T values 8 u + e).  Half 1's
      //      probabilities depend on nothing half 0's MFMAs write, so they
      //      can issue among them.
      auto read_v = [&](int h, int u, int d0, uint2 (&vlo)[VB], uint2 (&vhi)[VB]) {
        const uint8_t* vt = reinterpret_cast<const uint8_t*>(&sm.v[cur][0]) + vt_off0 + 32 * h * HD * 2 +
                            16 * u * HD * 2;
#pragma unroll
        for (int dt = 0; dt < VB; ++dt) {
          const unsigned dx = (64u * (dbase + d0 + dt)) ^ vx;
          vlo[dt] = lds_tr16(reinterpret_cast<const bf16_t*>(vt + dx));
          vhi[dt] = lds_tr16(reinterpret_cast<const bf16_t*>(vt + 8 * HD * 2 + dx));
        }
      };
      uint2 vlo0[VB], vhi0[VB];
      read_v(0, 0, 0, vlo0, vhi0);
      // the row max over the tile's keys: raw scores (the scale is positive),
      // then the row's other keys in lane l ^ 32
      float mx = -INFINITY;
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int v = 0; v < 16; v += 2) mx = max3_f32(mx, sv[h][v], sv[h][v + 1]);
      const float ms = mx * sc;
      const auto mw = __builtin_amdgcn_permlane32_swap(__float_as_uint(ms), __float_as_uint(ms), false, false);
      const float mloc = fmaxf(__uint_as_float(mw[0]), __uint_as_float(mw[1]));
      // Rescale only when some row's max grew past the reference by more than
      // 2^8 (2^(s - reference) stays <= 256: exact enough in bf16 and far from
      // fp32 overflow); otherwise keep it.  Rows whose reference is still
      // -inf hold zero sums: nothing to rescale (a slice's first tile writes O
      // with zero C operands and skips the pass entirely).
      const bool grow = mloc > m_run + 8.f;
      if (FIRST) {
        m_run = grow ? mloc : m_run;
      } else if (__builtin_amdgcn_ballot_w64(grow) != 0) {
        const float m_new = grow ? mloc : m_run;
        if (__builtin_amdgcn_ballot_w64(grow && m_run != -INFINITY) != 0) {
          const float alpha = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
          for (int dt = 0; dt < NDO; ++dt) o[dt] = o[dt] * alpha;
          l_run *= alpha;
        }
        m_run = m_new;
      }
      const float nref = m_run == -INFINITY ? 0.f : -m_run;
      uint32_t pw[2][8];
      float psum = 0.f;
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int v = 0; v < 16; v += 2) {
          const float p0 = __builtin_amdgcn_exp2f(fmaf(sv[h][v], sc, nref));
          const float p1 = __builtin_amdgcn_exp2f(fmaf(sv[h][v + 1], sc, nref));
          pw[h][v / 2] = pack2(p0, p1);
          psum += p0 + p1;
        }
      l_run += psum;
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const bf16x8 pb = as_bf16x8(make_uint4(pw[h][4 * u], pw[h][4 * u + 1], pw[h][4 * u + 2], pw[h][4 * u + 3]));
#pragma unroll
          for (int d0 = 0; d0 < NDO; d0 += VB) {
            uint2 vlo[VB], vhi[VB];
            if (h == 0 && u == 0 && d0 == 0) {
#pragma unroll
              for (int dt = 0; dt < VB; ++dt) {
                vlo[dt] = vlo0[dt];
                vhi[dt] = vhi0[dt];
              }
            } else {
              read_v(h, u, d0, vlo, vhi);
            }
#pragma unroll
            for (int dt = 0; dt < VB; ++dt) {
              const bf16x8 va = as_bf16x8(make_uint4(vlo[dt].x, vlo[dt].y, vhi[dt].x, vhi[dt].y));
              if (FIRST && h == 0 && u == 0)
                o[d0 + dt] = mfma32(va, pb, f32x16{});
              else
                o[d0 + dt] = mfma32(va, pb, o[d0 + dt]);
            }
          }
        }
    } else {
      // ---- per half: online softmax in base 2, then O^T += V^T P^T (two
      //      16-key steps; P^T slots e <-> S^T values 8 u + e).  The half's first
      //      transposed V reads are issued ahead of its softmax.
#pragma unroll
      for (int h = 0; h < NH; ++h) {
        const uint8_t* vt0 = reinterpret_cast<const uint8_t*>(&sm.v[cur][0]) + vt_off0 + 32 * (NH == 2 ? h : kh_w) * HD * 2;
        auto read_v = [&](int u, int d0, uint2 (&vlo)[VB], uint2 (&vhi)[VB]) {
          const uint8_t* vt = vt0 + 16 * u * HD * 2;
#pragma unroll
          for (int dt = 0; dt < VB; ++dt) {
            const unsigned dx = (64u * (dbase + d0 + dt)) ^ vx;
            vlo[dt] = lds_tr16(reinterpret_cast<const bf16_t*>(vt + dx));
            vhi[dt] = lds_tr16(reinterpret_cast<const bf16_t*>(vt + 8 * HD * 2 + dx));
          }
        };
        uint2 vlo0[VB], vhi0[VB];
        read_v(0, 0, vlo0, vhi0);
        // the row max over this half's keys: raw scores (the scale is
        // positive), then the row's other 16 keys in lane l ^ 32
        float mx = -INFINITY;
#pragma unroll
        for (int v = 0; v < 16; v += 2) mx = max3_f32(mx, sv[h][v], sv[h][v + 1]);
        const float ms = mx * sc;
        const auto mw = __builtin_amdgcn_permlane32_swap(__float_as_uint(ms), __float_as_uint(ms), false, false);
        const float mloc = fmaxf(__uint_as_float(mw[0]), __uint_as_float(mw[1]));
        // Rescale only when some row's max grew past the reference by more than
        // 2^8 (2^(s - reference) stays <= 256: exact enough in bf16 and far from
        // fp32 overflow); otherwise keep it.  Rows whose reference is still
        // -inf hold zero sums: nothing to rescale (a slice's first half-tile
        // writes O with zero C operands and skips the pass entirely).
        const bool grow = mloc > m_run + 8.f;
        if (FIRST && h == 0) {
          m_run = grow ? mloc : m_run;
        } else if (__builtin_amdgcn_ballot_w64(grow) != 0) {
          const float m_new = grow ? mloc : m_run;
          if (__builtin_amdgcn_ballot_w64(grow && m_run != -INFINITY) != 0) {
            const float alpha = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
            for (int dt = 0; dt < NDO; ++dt) o[dt] = o[dt] * alpha;
            l_run *= alpha;
          }
          m_run = m_new;
        }
        // a row that has seen no key yet (reference -inf, every score -inf)
        // takes reference 0; its probabilities are exactly 0
        const float nref = m_run == -INFINITY ? 0.f : -m_run;
        // p = 2^(s scale - reference) (arguments <= 8 or -inf)
        uint32_t pw[8];
        float psum = 0.f;
#pragma unroll
        for (int v = 0; v < 16; v += 2) {
          const float p0 = __builtin_amdgcn_exp2f(fmaf(sv[h][v], sc, nref));
          const float p1 = __builtin_amdgcn_exp2f(fmaf(sv[h][v + 1], sc, nref));
          pw[v / 2] = pack2(p0, p1);
          psum += p0 + p1;
        }
        l_run += psum;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const bf16x8 pb = as_bf16x8(make_uint4(pw[4 * u], pw[4 * u + 1], pw[4 * u + 2], pw[4 * u + 3]));
#pragma unroll
          for (int d0 = 0; d0 < NDO; d0 += VB) {
            uint2 vlo[VB], vhi[VB];
            if (u == 0 && d0 == 0) {
#pragma unroll
              for (int dt = 0; dt < VB; ++dt) {
                vlo[dt] = vlo0[dt];
                vhi[dt] = vhi0[dt];
              }
            } else {
              read_v(u, d0, vlo, vhi);
            }
#pragma unroll
            for (int dt = 0; dt < VB; ++dt) {
              const bf16x8 va = as_bf16x8(make_uint4(vlo[dt].x, vlo[dt].y, vhi[dt].x, vhi[dt].y));
              if (FIRST && h == 0 && u == 0)
                o[d0 + dt] = mfma32(va, pb, f32x16{});
              else
                o[d0 + dt] = mfma32(va, pb, o[d0 + dt]);
            }
          }
        }
      }
    }
    // ---- tile it + 1 (the only loads in flight) has landed in the other
    //      buffer once every wave has waited for its own DMA; then refill
    //      this buffer, which no wave reads any more, with tile it + 2
    if (it + 1 < n_tiles) __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __syncthreads();
    if (it + 2 < n_tiles) load_tile(it + 2, cur);
  };
  step(0, std::integral_constant<int, 0>{}, std::true_type{});
  for (int it = 1; it < n_tiles; it += 2) {
    step(it, std::integral_constant<int, 1>{}, std::false_type{});
    if (it + 1 < n_tiles) step(it + 1, std::integral_constant<int, 0>{}, std::false_type{});
  }

  // ---- epilogue.  Lane l holds O^T slots v of query row l % 32: dims
  //      32 dt + 8 (v / 4) + 4 (l / 32) + v % 4.  Its four values of an 8-dim
  //      output chunk pair up with the other four in lane l ^ 32 through
  //      v_permlane32_swap, so every lane stores whole 16-byte chunks: the
  //      normalised rows in the O projection's operand order (one key slice),
  //      or this slice's normalised bf16 partial and its (max, sum) per row
  //      (several).  Upper lanes give dims 4..7 of chunk 2 j and take dims
  //      0..3 of chunk 2 j + 1, so lane l ends with dims 16 j + 8 (l / 32) + 0..7.
  const float l_tot = l_run + __shfl_xor(l_run, 32);   // the two lanes of a row share m_run
  auto chunk_of = [&](const float (&v)[8]) {
    const auto s0 = __builtin_amdgcn_permlane32_swap(pack2(v[0], v[1]), pack2(v[4], v[5]), false, false);
    const auto s1 = __builtin_amdgcn_permlane32_swap(pack2(v[2], v[3]), pack2(v[6], v[7]), false, false);
    return make_uint4(s0[0], s1[0], s0[1], s1[1]);
  };
  const int row32 = l & 31;
  const int MTo = mt_of(a.B * a.T);
  const __amdgpu_buffer_rsrc_t ro = make_rsrc(a.o, (size_t)MTo * 16 * a.Hq * HD * 2);
  const size_t slab = (size_t)64 * HD;     // bf16 per (slice, 64-row block)
  const int n_rb64 = (rows + 63) >> 6;
  const int n_rbt64 = a.B * a.Hkv * n_rb64;
  if constexpr (LONG || DSPLIT) {
    // ---- every wave holds its rows' whole result (DSPLIT: for its half of
    //      the dims): normalise and store
    constexpr int BR = LONG ? 128 : 64;
    const int arow = BR * rb + 32 * rp + row32;
    const bool live = arow < rows;
    const float inv = 1.f / l_tot;
    // the 64-row block of this wave's rows (uniform; past the last block
    // only for a wave with no live rows, which stores nothing)
    const int rb_id = __builtin_amdgcn_readfirstlane(bh * n_rb64 + ((BR * rb + 32 * rp) >> 6));
    const __amdgpu_buffer_rsrc_t rpo =
        make_rsrc(a.part_o + ((size_t)ks * n_rbt64 + rb_id) * slab, a.splits > 1 ? slab * 2 : 0);
    const int t = arow / G, hq = hk * G + (arow - t * G);
#pragma unroll
    for (int dt = 0; dt < NDO; ++dt)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = o[dt][8 * j + e] * inv;
        const uint4 chunk = chunk_of(v);
        const int dd = 32 * (dbase + dt) + 16 * j + 8 * hl;
        if (live) {
          if (a.splits == 1)
            buf_st16(ro, (int)(fa_index(b * a.T + t, hq * HD + dd, MTo) * 2), chunk);
          else
            buf_st16(rpo, attn_part_slot(arow & 63, dd >> 3) * 16, chunk);
        }
      }
    // (both waves of a DSPLIT row tile hold the same (max, sum); one stores it)
    if (a.splits > 1 && hl == 0 && live && (!DSPLIT || dbase == 0)) {
      const __amdgpu_buffer_rsrc_t rpm = make_rsrc(a.part_ml + ((size_t)ks * n_rbt64 + rb_id) * 128, 512);
      buf_st8(rpm, (arow & 63) * 8, __float_as_uint(m_run), __float_as_uint(l_tot));
    }
    return a.splits == 1;
  } else {
    // ---- merge the two key halves (64-row blocks).  The waves of a pair hold
    //      the same 32 rows over different keys; each merges half of the d
    //      tiles: it hands the partner's half of its unnormalised O^T registers
    //      to LDS in register order (lane-contiguous 16-byte slots, no bank
    //      conflicts), reads the partner's copy of its own half, and combines
    //      and stores slot by slot as above.
    constexpr int NH2 = NDT / 2;   // d tiles each wave of a pair merges
    static_assert(sizeof(sm.k) >= sizeof(float4) * 4 * NH2 * 4 * 64, "hand-off slots fit in the K tiles");
    float4* hand = reinterpret_cast<float4*>(&sm.k[0][0]);   // [row tile][dest half][NH2 * 4][64 lanes]
    auto give = [&](auto off_c) {
      constexpr int off = decltype(off_c)::value;   // first d tile the partner merges
      float4* dst = hand + (rp * 2 + (kh_w ^ 1)) * (NH2 * 4 * 64) + l;
#pragma unroll
      for (int i = 0; i < NH2; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          dst[(4 * i + q) * 64] = make_float4(o[off + i][4 * q], o[off + i][4 * q + 1],
                                              o[off + i][4 * q + 2], o[off + i][4 * q + 3]);
    };
    if (kh_w == 0)
      give(std::integral_constant<int, NH2>{});
    else
      give(std::integral_constant<int, 0>{});
    if (hl == 0) sm.mlh[kh_w][rp * 32 + row32] = make_float2(m_run, l_tot);
    __syncthreads();

    const float2 pm = sm.mlh[kh_w ^ 1][rp * 32 + row32];
    const float mm = fmaxf(m_run, pm.x);
    const float a_own = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - mm);
    const float a_oth = pm.x == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(pm.x - mm);
    const float lsum = l_tot * a_own + pm.y * a_oth;   // > 0: key half 0 of a slice has a key
    const float s_own = a_own / lsum, s_oth = a_oth / lsum;
    const int row64 = 32 * rp + row32, arow = 64 * rb + row64;
    const bool live = arow < rows;
    const int rb_id = __builtin_amdgcn_readfirstlane(bh * n_rb64 + rb);
    const __amdgpu_buffer_rsrc_t rpo =
        make_rsrc(a.part_o + ((size_t)ks * n_rbt64 + rb_id) * slab, a.splits > 1 ? slab * 2 : 0);
    const int t = arow / G, hq = hk * G + (arow - t * G);
    auto merge_store = [&](auto off_c) {
      constexpr int off = decltype(off_c)::value;   // first d tile this wave merges
      const float4* src = hand + (rp * 2 + kh_w) * (NH2 * 4 * 64) + l;
#pragma unroll
      for (int i = 0; i < NH2; ++i) {
        float p[16];
#pragma unroll
        for (int q = 0; q < 4; ++q) *reinterpret_cast<float4*>(&p[4 * q]) = src[(4 * i + q) * 64];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          float v[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = o[off + i][8 * j + e] * s_own + p[8 * j + e] * s_oth;
          const uint4 chunk = chunk_of(v);
          const int dd = 32 * (off + i) + 16 * j + 8 * hl;
          if (live) {
            if (a.splits == 1)
              buf_st16(ro, (int)(fa_index(b * a.T + t, hq * HD + dd, MTo) * 2), chunk);
            else
              buf_st16(rpo, attn_part_slot(row64, dd >> 3) * 16, chunk);
          }
        }
      }
    };
    if (kh_w == 0)
      merge_store(std::integral_constant<int, 0>{});
    else
      merge_store(std::integral_constant<int, NH2>{});
    if (a.splits > 1 && kh_w == 0 && hl == 0 && live) {
      const __amdgpu_buffer_rsrc_t rpm = make_rsrc(a.part_ml + ((size_t)ks * n_rbt64 + rb_id) * 128, 512);
      buf_st8(rpm, row64 * 8, __float_as_uint(mm), __float_as_uint(lsum));
    }
    return a.splits == 1;
  }
}

// Items of the key-slice merge: one per (row block, row, 8-byte half of a
// 16-byte chunk).  Half chunks halve each thread's serial arithmetic (the
// merge is one memory round trip and then vector work on one wave per
// compute unit) at twice the threads.
__host__ __device__ inline int attn_combine_items(int B, int T, int Hq, int Hkv, int HD) {
  return B * Hkv * ((Hq / Hkv * T + 63) / 64) * 64 * (HD / 4);
}

// Merges the key slices of attn_sm_task for the blockDim.x items of task
// `task`: o = sum_s w_s o_s / sum_s w_s with w_s = l_s 2^(m_s - max m),
// in slice order, stored in the O projection's operand order.
template <int HD>
__device__ void attn_combine_task(const AttnSmArgs& a, int task) {
  constexpr int CPR = HD / 8;
  const int G = a.Hq / a.Hkv;
  const int rows = G * a.T;
  const int n_rb = (rows + 63) >> 6;
  const int n_rbt = a.B * a.Hkv * n_rb;
  const int i = task * (int)blockDim.x + (int)threadIdx.x;
  if (i >= n_rbt * 128 * CPR) return;
  const int rb_id = i / (128 * CPR), rem = i - rb_id * 128 * CPR;
  const int slot = rem >> 1, half = rem & 1;   // 16-byte slot, its 8-byte half
  const int gi = slot & 63, gg = slot >> 6;
  const int row = 16 * (gg & 3) + (gi & 15), c = 4 * (gg >> 2) + (gi >> 4);   // inverse of attn_part_slot
  const int bh = rb_id / n_rb, rb = rb_id - bh * n_rb;
  const int b = bh / a.Hkv, hk = bh - b * a.Hkv;
  const int ar = 64 * rb + row;
  if (ar >= rows) return;
  const size_t slab = (size_t)64 * HD;
  const __amdgpu_buffer_rsrc_t rpo = make_rsrc(a.part_o, (size_t)a.splits * n_rbt * slab * 2);
  const __amdgpu_buffer_rsrc_t rpm = make_rsrc(a.part_ml, (size_t)a.splits * n_rbt * 512);
  float2 ml[kAttnMaxSplits];
  u32x2v pv[kAttnMaxSplits];
#pragma unroll
  for (int sp = 0; sp < kAttnMaxSplits; ++sp)
    if (sp < a.splits) {
      const u32x2v u = __builtin_amdgcn_raw_buffer_load_b64(rpm, ((sp * n_rbt + rb_id) * 64 + row) * 8, 0, 16);
      ml[sp] = make_float2(__uint_as_float(u[0]), __uint_as_float(u[1]));
      pv[sp] = __builtin_amdgcn_raw_buffer_load_b64(
          rpo, (int)((((size_t)sp * n_rbt + rb_id) * slab + 8 * (size_t)slot) * 2) + 8 * half, 0, 16);
    }
  float mx = -INFINITY;
#pragma unroll
  for (int sp = 0; sp < kAttnMaxSplits; ++sp)
    if (sp < a.splits) mx = fmaxf(mx, ml[sp].x);
  float den = 0.f;
  float f[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int sp = 0; sp < kAttnMaxSplits; ++sp)
    if (sp < a.splits) {
      // an empty slice ((max, sum) = (-inf, 0)) wrote no partial rows: skip
      // them rather than multiply whatever they hold by zero
      if (ml[sp].x != -INFINITY) {
        const float wgt = ml[sp].y * __builtin_amdgcn_exp2f(ml[sp].x - mx);   // argument <= 0
        den += wgt;
        const float x[4] = {__uint_as_float(pv[sp][0] << 16), __uint_as_float(pv[sp][0] & 0xffff0000u),
                            __uint_as_float(pv[sp][1] << 16), __uint_as_float(pv[sp][1] & 0xffff0000u)};
#pragma unroll
        for (int e = 0; e < 4; ++e) f[e] = fmaf(wgt, x[e], f[e]);
      }
    }
  const float inv = __builtin_amdgcn_rcpf(den);
  const int t = ar / G, h = hk * G + (ar - t * G);
  const int MTo = mt_of(a.B * a.T);
  const __amdgpu_buffer_rsrc_t ro = make_rsrc(a.o, (size_t)MTo * 16 * a.Hq * HD * 2);
  buf_st8(ro, (int)(fa_index(b * a.T + t, h * HD + 8 * c, MTo) * 2) + 8 * half, pack2(f[0] * inv, f[1] * inv),
          pack2(f[2] * inv, f[3] * inv));
}

}  // namespace blk
