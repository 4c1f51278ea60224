// Attention of a small query chunk over [cached prefix ; the chunk's own keys]
// as a device task shared by the standalone kernel and the persistent stage
// kernel.
//
// [PS] = "PhysisServe" (arXiv:2605.11143): a stage runs one block for a chunk
// of query tokens against the cached KV of earlier chunks plus its own;
// [RT] = "Running VLAs at Real-time Speed" (arXiv:2510.26742v1) §2: the action
// expert's 64 query tokens attend to the cached prefix and to each other with
// no causal mask inside the chunk.
//
// The rows of one (stream b, kv head hk) are the G = Hq / Hkv query heads of
// each of the T tokens, row ar = t G + gh; they all read that kv head's keys,
// so one K/V tile serves a block of rows.  A task takes a row block and one
// slice of the keys, in steps of 64 keys:
//  * K / V tiles are loaded with row-contiguous 16-byte loads one step ahead
//    and staged through double-buffered LDS;
//  * 64-row blocks: wave w takes 32 query rows (w % 2) and one 32-key half
//    (w / 2) of every step; 128-row blocks (LONG, long key runs): wave w takes
//    32 rows and both halves, so a tile serves twice the rows and the halves
//    need no merge; 32 x 32 x 16 MFMAs throughout (twice the operand reuse of
//    16 x 16 tiles);
//  * S^T = K Q^T: K rows as the A operand (LDS), Q^T as the B operand held in
//    registers (the QKV epilogue stores Q in exactly that operand order,
//    qa_index), so a lane holds 16 keys of one query row;
//  * online softmax per row in base 2 (scores pre-scaled by log2(e)/sqrt(d));
//    the output is rescaled only when a row's max grows by more than 2^8;
//  * O^T += V^T P^T: P^T is the B operand straight from the score registers
//    (slot e of the u-th 16-key step is S^T value 8 u + e, keys
//    16 u + 4 (l/32) + e or 16 u + 8 + 4 (l/32) + e - 4), V^T the A operand
//    read out of the row-major V tile with ds_read_b64_tr_b16, which hands
//    lane i of each 16-lane group element i % 4 of the 8 bytes at lane
//    4 k + i / 4 (k < 4): pointing lane i at key row 4 k' + i / 4, dims
//    4 (i % 4) .. + 3 yields V[key k][dim i] in that key order;
//  * (64-row blocks) the two key halves meet in LDS; one key slice then
//    writes the normalised rows straight into the O projection's operand
//    order (both modes); several slices
//    publish bf16 partials normalised by their own sum plus (max, sum), which
//    a separate merge step (attn_combine_task, one thread per 16 output
//    bytes, all slices' loads in flight together) combines in slice order.
//    Many small slices keep every workgroup to about one memory round trip.
#pragma once
#include "common.h"
#include "skinny.h"

#include <type_traits>

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
  bf16_t* part_o;         // [splits][n_rbt][64][d] (normalised partials)
  float* part_ml;         // [splits][n_rbt][64][2] (max, sum)
  int long_rows;          // 1: 128-row blocks over a single key slice (attn_sm_task LONG)
};

constexpr int kAttnMaxSplits = 16;

template <int HD>
struct AttnSmSmem {
  // K / V tiles; after the key loop both arrays hold the two key halves'
  // unnormalised rows [2][64][HD + 4] (fp32, fits in k and v together)
  bf16_t k[2][64 * (HD + 8)];
  bf16_t v[2][64 * (HD + 16)];
  float2 mlh[2][64];                 // per key half and row: (max, sum)
};

__device__ __forceinline__ uint2 lds_tr16(const bf16_t* p) {
  typedef short v4s __attribute__((ext_vector_type(4)));
  const v4s v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)(p));
  return __builtin_bit_cast(uint2, v);
}

typedef float f32x16 __attribute__((ext_vector_type(16)));
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
// them.
template <int HD, bool LONG = false, class Wait>
__device__ bool attn_sm_task(const AttnSmArgs& a, int bh, int rb, int ks, AttnSmSmem<HD>& sm,
                             Wait&& wait) {
  constexpr int KROW = HD + 8, VROW = HD + 16;
  constexpr int NDS = HD / 16;                 // 16-wide d steps of S^T (32x32x16)
  constexpr int NDT = HD / 32;                 // 32-row d tiles of O^T
  constexpr int CPR = HD / 8;                  // 16-byte chunks per key row
  constexpr int NCH = 64 * CPR / 256;          // chunks per thread per 64-key tile (K or V)
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index (uniform)
  const int l = tid & 63;
  const int rp = LONG ? w : (w & 1);          // 32-row tile of the block
  const int kh_w = w >> 1;                     // the wave's 32-key half of a tile (not LONG)
  const int b = bh / a.Hkv, hk = bh - b * a.Hkv;
  const int G = a.Hq / a.Hkv;
  const int rows = G * a.T;
  const int n_rt = (rows + 31) >> 5;           // 32-row tiles of this (stream, kv head)
  const int L = a.P + a.T;
  const int key_begin = ks * a.kps;
  const int key_end = min(L, key_begin + a.kps);
  const int n_tiles = (key_end - key_begin + 63) >> 6;
  const int kvrow = a.Hkv * HD;

  // K / V sources: prefix (caller's cache, read once) and the chunk's own rows
  // (written by the QKV step, possibly earlier in the same launch: coherent)
  const __amdgpu_buffer_rsrc_t rkp =
      make_rsrc(a.kp ? a.kp + (size_t)b * a.prefix_stride + (size_t)hk * HD : a.kn, (size_t)a.P * kvrow * 2);
  const __amdgpu_buffer_rsrc_t rvp =
      make_rsrc(a.vp ? a.vp + (size_t)b * a.prefix_stride + (size_t)hk * HD : a.vn, (size_t)a.P * kvrow * 2);
  const __amdgpu_buffer_rsrc_t rkn = make_rsrc(a.kn + (size_t)b * a.new_stride + (size_t)hk * HD, (size_t)a.T * kvrow * 2);
  const __amdgpu_buffer_rsrc_t rvn = make_rsrc(a.vn + (size_t)b * a.new_stride + (size_t)hk * HD, (size_t)a.T * kvrow * 2);
  uint4 reg[2][NCH];   // one tile in flight: [K, V][chunk]
  // thread tid moves 16-byte chunk c0 of key rows kk0 + j RPJ, j < NCH
  constexpr int RPJ = 256 / CPR;               // key rows per pass of the workgroup
  const int kk0 = tid / CPR, c0 = tid - kk0 * CPR;
  auto load_tile = [&](int tile) {
    const int base = key_begin + 64 * tile + kk0;
    if (base - kk0 + 64 <= a.P) {   // wholly in the prefix (uniform)
      const int off0 = (base * kvrow + 8 * c0) * 2;
#pragma unroll
      for (int j = 0; j < NCH; ++j) {
        reg[0][j] = buf_ld_stream(rkp, off0 + j * RPJ * kvrow * 2);
        reg[1][j] = buf_ld_stream(rvp, off0 + j * RPJ * kvrow * 2);
      }
    } else {
#pragma unroll
      for (int j = 0; j < NCH; ++j) {
        const int key = base + j * RPJ;
        if (key >= key_end) {
          reg[0][j] = make_uint4(0, 0, 0, 0);
          reg[1][j] = make_uint4(0, 0, 0, 0);
        } else if (key < a.P) {
          const int off = (key * kvrow + 8 * c0) * 2;
          reg[0][j] = buf_ld_stream(rkp, off);
          reg[1][j] = buf_ld_stream(rvp, off);
        } else {
          const int off = ((key - a.P) * kvrow + 8 * c0) * 2;
          reg[0][j] = buf_ld_act(rkn, off);
          reg[1][j] = buf_ld_act(rvn, off);
        }
      }
    }
  };
  auto store_tile = [&](int buf) {
    bf16_t* kd = &sm.k[buf][kk0 * KROW + 8 * c0];
    bf16_t* vd = &sm.v[buf][kk0 * VROW + 8 * c0];
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      *reinterpret_cast<uint4*>(kd + j * RPJ * KROW) = reg[0][j];
      *reinterpret_cast<uint4*>(vd + j * RPJ * VROW) = reg[1][j];
    }
  };

  // the first tile, if wholly in the prefix, does not depend on earlier work
  // and starts before the wait
  const bool pre0 = key_begin + 64 <= a.P;
  if (n_tiles > 0 && pre0) load_tile(0);
  if (!wait()) return false;
  if (n_tiles > 0 && !pre0) load_tile(0);

  // this wave's 32 query rows: Q^T fragments (B operand), one per d step
  const int rt = min((LONG ? 4 : 2) * rb + rp, n_rt - 1);
  const __amdgpu_buffer_rsrc_t rq =
      make_rsrc(a.q + (size_t)(bh * n_rt + rt) * NDS * 512, (size_t)NDS * kFragBytes);
  uint4 qf[NDS];
#pragma unroll
  for (int s = 0; s < NDS; ++s) qf[s] = buf_ld_act(rq, s * kFragBytes + l * 16);
  // Let Q land here, once: otherwise the compiler's wait for Q sits at the
  // head of the key loop, where (counters being in order) it waits for each
  // step's K/V prefetch as well.  (vmcnt(0); expcnt, lgkmcnt left free)
  __builtin_amdgcn_s_waitcnt(0x0F70);

  f32x16 o[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int v = 0; v < 16; ++v) o[dt][v] = 0.f;
  // running reference max (may trail the true max by up to 2^8, see below) and sum
  float m_run = -INFINITY, l_run = 0.f;

  __syncthreads();   // a previous task's readers of sm are done
  if (n_tiles > 0) {
    store_tile(0);
    if (n_tiles > 1) load_tile(1);
  }
  __syncthreads();

  // lane roles: query row l % 32 of this wave's 32 rows; S^T keys
  // 32 kh + 8 (v/4) + 4 (l/32) + v%4 of the 64-key tile, v < 16
  const int hl = l >> 5;
  const int p16 = l & 15;
  // V^T operand (transposed LDS reads): d = 32 dt + 16 ((l/16) % 2) + 4 (p16 % 4),
  // key rows 32 kh + 16 u + 4 hl + p16 / 4 (+ 8 for the second read)
  const int vt_off0 = (4 * hl + (p16 >> 2)) * VROW + 16 * ((l >> 4) & 1) + 4 * (p16 & 3);

  // key halves this wave takes of every tile: both (LONG) or its own
  constexpr int NH = LONG ? 2 : 1;
  auto step = [&](int it, auto cur_c) {
    constexpr int cur = decltype(cur_c)::value;   // LDS buffer of tile it
    // ---- S^T (32 keys x 32 rows) of each half: K fragments read from LDS in
    //      batches ahead of their MFMAs; the halves' chains (and at HD < 256
    //      two per half) are independent
    f32x16 sacc[NH], sacc2[NH];
#pragma unroll
    for (int h = 0; h < NH; ++h)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        sacc[h][v] = 0.f;
        sacc2[h][v] = 0.f;
      }
    constexpr int KB = NDS < 8 ? NDS : (HD >= 256 ? 4 : 8);   // registers bound the batch at HD 256
#pragma unroll
    for (int s0 = 0; s0 < NDS; s0 += KB) {
      uint4 kf[NH][KB];
#pragma unroll
      for (int h = 0; h < NH; ++h) {
        const int kh = LONG ? h : kh_w;
        const bf16_t* kr = &sm.k[cur][(32 * kh + (l & 31)) * KROW + 8 * hl];
#pragma unroll
        for (int s = 0; s < KB; ++s) kf[h][s] = *reinterpret_cast<const uint4*>(kr + 16 * (s0 + s));
      }
#pragma unroll
      for (int s = 0; s < KB; s += 2)
#pragma unroll
        for (int h = 0; h < NH; ++h) {
          sacc[h] = mfma32(as_bf16x8(kf[h][s]), as_bf16x8(qf[s0 + s]), sacc[h]);
          if (s + 1 < KB) {
            if constexpr (HD >= 256)
              sacc[h] = mfma32(as_bf16x8(kf[h][s + 1]), as_bf16x8(qf[s0 + s + 1]), sacc[h]);
            else
              sacc2[h] = mfma32(as_bf16x8(kf[h][s + 1]), as_bf16x8(qf[s0 + s + 1]), sacc2[h]);
          }
        }
    }
    // ---- online softmax in base 2, one update for all of the wave's keys
    float x[NH][16];
    float mloc = -INFINITY;
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      sacc[h] += sacc2[h];
      const int base = key_begin + 64 * it + 32 * (LONG ? h : kh_w);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int key = base + 8 * (v >> 2) + 4 * hl + (v & 3);
        x[h][v] = key < key_end ? sacc[h][v] * a.scale_log2 : -INFINITY;
        mloc = fmaxf(mloc, x[h][v]);
      }
    }
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
    // Rescale only when some row's max grew past the reference by more than
    // 2^8 (exp2 of scores against a stale reference stays <= 256: exact
    // enough in bf16 and far from fp32 overflow); otherwise keep it.
    const bool grow = mloc > m_run + 8.f;
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
      const float m_new = grow ? mloc : m_run;
      const float alpha = m_run == -INFINITY ? 0.f : exp2f(m_run - m_new);
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) o[dt] = o[dt] * alpha;
      l_run *= alpha;
      m_run = m_new;
    }
    // masked keys (and rows that have seen no key yet) contribute exactly 0
    float psum = 0.f;
    uint32_t pw[NH][8];
#pragma unroll
    for (int h = 0; h < NH; ++h)
#pragma unroll
      for (int v = 0; v < 16; v += 2) {
        const float p0 = x[h][v] == -INFINITY ? 0.f : exp2f(x[h][v] - m_run);
        const float p1 = x[h][v + 1] == -INFINITY ? 0.f : exp2f(x[h][v + 1] - m_run);
        psum += p0 + p1;
        pw[h][v / 2] = pack2(p0, p1);
      }
    l_run += psum;
    // ---- O^T += V^T P^T, two 16-key steps per half (P^T slots e <-> S^T
    //      values 8 u + e)
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      const int vt_off = vt_off0 + 32 * (LONG ? h : kh_w) * VROW;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const bf16x8 pb =
            as_bf16x8(make_uint4(pw[h][4 * u], pw[h][4 * u + 1], pw[h][4 * u + 2], pw[h][4 * u + 3]));
        const bf16_t* vt = &sm.v[cur][vt_off + 16 * u * VROW];
        constexpr int VB = NDT < 4 ? NDT : 4;   // transposed reads issued ahead of their MFMAs
#pragma unroll
        for (int d0 = 0; d0 < NDT; d0 += VB) {
          uint2 vlo[VB], vhi[VB];
#pragma unroll
          for (int dt = 0; dt < VB; ++dt) {
            vlo[dt] = lds_tr16(vt + 32 * (d0 + dt));
            vhi[dt] = lds_tr16(vt + 8 * VROW + 32 * (d0 + dt));
          }
#pragma unroll
          for (int dt = 0; dt < VB; ++dt)
            o[d0 + dt] =
                mfma32(as_bf16x8(make_uint4(vlo[dt].x, vlo[dt].y, vhi[dt].x, vhi[dt].y)), pb, o[d0 + dt]);
        }
      }
    }
    // ---- stage the next tile into the other buffer (last read one tile ago)
    //      and start the loads of the tile after it
    if (it + 1 < n_tiles) {
      store_tile(cur ^ 1);
      if (it + 2 < n_tiles) load_tile(it + 2);
    }
    __syncthreads();
  };
  for (int it = 0; it < n_tiles; it += 2) {
    step(it, std::integral_constant<int, 0>{});
    if (it + 1 < n_tiles) step(it + 1, std::integral_constant<int, 1>{});
  }

  // ---- merge the two key halves: every wave parks its unnormalised O^T rows
  //      (fp32) and (max, sum) in LDS -- the K / V tiles are no longer read --
  //      then all 256 threads combine 16-byte output chunks and store them
  //      (one key slice: the O projection's operand order; several: this
  //      slice's normalised bf16 partial and its (max, sum))
  const float l_tot = l_run + __shfl_xor(l_run, 32);   // the two lanes of a row share m_run
  constexpr int PROW = HD + 4;
  if constexpr (LONG) {
    // ---- every wave holds its rows' whole result: park them (fp32, with
    //      1 / sum) in LDS and store the 128 rows in the O projection's
    //      operand order, 16 bytes per lane as in the merge below
    float* park = reinterpret_cast<float*>(&sm.k[0][0]);   // [128 rows][PROW]
    float* inv_row = &sm.mlh[0][0].x;                        // [128]
    const int row32 = l & 31;
    {
      float* dst = park + (32 * rp + row32) * PROW + 4 * hl;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          *reinterpret_cast<float4*>(dst + 32 * dt + 8 * q) =
              make_float4(o[dt][4 * q], o[dt][4 * q + 1], o[dt][4 * q + 2], o[dt][4 * q + 3]);
      if (hl == 0) inv_row[32 * rp + row32] = 1.f / l_tot;
      if (a.splits > 1 && hl == 0) {
        // this slice's (max, sum) of the row, by 64-row block
        const int row = 32 * rp + row32, ar = 128 * rb + row;
        const int n_rb64 = (rows + 63) >> 6;
        const int sub = __builtin_amdgcn_readfirstlane((128 * rb + 32 * rp) >> 6);   // wave-uniform
        if (ar < rows) {
          const size_t rb_id = (size_t)bh * n_rb64 + sub;
          const __amdgpu_buffer_rsrc_t rpm = make_rsrc(
              a.part_ml + ((size_t)ks * a.B * a.Hkv * n_rb64 + rb_id) * 128, 512);
          buf_st8(rpm, (ar & 63) * 8, __float_as_uint(m_run), __float_as_uint(l_tot));
        }
      }
    }
    __syncthreads();
    const int MTo = mt_of(a.B * a.T);
    const __amdgpu_buffer_rsrc_t ro = make_rsrc(a.o, (size_t)MTo * 16 * a.Hq * HD * 2);
    constexpr int LPR = HD / 8, RPP = 64 / LPR, PASSES = 128 / (4 * RPP);
    const int c = l % LPR, odd = c & 1;
    uint4 res[PASSES];
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      const int row = (w + 4 * p) * RPP + l / LPR;
      const float inv = inv_row[row];
      const float* p0 = park + row * PROW;
      uint2 half[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const float4 x = *reinterpret_cast<const float4*>(p0 + 4 * (LPR * e + c));
        half[e] = make_uint2(pack2(x.x * inv, x.y * inv), pack2(x.z * inv, x.w * inv));
      }
      const uint2 give = odd ? half[0] : half[1];
      const uint2 got = make_uint2(__shfl_xor(give.x, 1), __shfl_xor(give.y, 1));
      res[p] = odd ? make_uint4(got.x, got.y, half[1].x, half[1].y)
                   : make_uint4(half[0].x, half[0].y, got.x, got.y);
    }
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      const int row = (w + 4 * p) * RPP + l / LPR;
      const int ch = (c >> 1) + (odd ? LPR / 2 : 0);
      const int ar = 128 * rb + row;
      if (ar < rows) {
        if (a.splits == 1) {
          const int t = ar / G, h = hk * G + (ar - t * G);
          buf_st16(ro, (int)(fa_index(b * a.T + t, h * HD + 8 * ch, MTo) * 2), res[p]);
        } else {
          // the slice's normalised partial row, in its 64-row block's slab
          const int n_rb64 = (rows + 63) >> 6;
          // a wave's rows of a pass lie in one 64-row block (wave-uniform)
          const int sub = __builtin_amdgcn_readfirstlane((128 * rb + (w + 4 * p) * RPP) >> 6);
          const size_t rb_id = (size_t)bh * n_rb64 + sub;
          const size_t slab = (size_t)64 * HD;
          const __amdgpu_buffer_rsrc_t rpo = make_rsrc(
              a.part_o + ((size_t)ks * a.B * a.Hkv * n_rb64 + rb_id) * slab, slab * 2);
          buf_st16(rpo, ((ar & 63) * HD + 8 * ch) * 2, res[p]);
        }
      }
    }
    return a.splits == 1;
  }
  const int kh = kh_w;
  float* park = reinterpret_cast<float*>(&sm.k[0][0]);   // [2 key halves][64 rows][PROW]
  const int row32 = l & 31;
  {
    float* dst = park + (kh * 64 + rp * 32 + row32) * PROW + 4 * hl;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<float4*>(dst + 32 * dt + 8 * q) =
            make_float4(o[dt][4 * q], o[dt][4 * q + 1], o[dt][4 * q + 2], o[dt][4 * q + 3]);
    if (hl == 0) sm.mlh[kh][rp * 32 + row32] = make_float2(m_run, l_tot);
  }
  __syncthreads();

  const int n_rb = (rows + 63) >> 6;
  const int rb_id = bh * n_rb + rb;
  const int n_rbt = a.B * a.Hkv * n_rb;
  const size_t slab = (size_t)64 * HD;     // bf16 per (slice, row block)
  const int MTo = mt_of(a.B * a.T);
  const __amdgpu_buffer_rsrc_t ro = make_rsrc(a.o, (size_t)MTo * 16 * a.Hq * HD * 2);
  const __amdgpu_buffer_rsrc_t rpo =
      make_rsrc(a.part_o + ((size_t)ks * n_rbt + rb_id) * slab, a.splits > 1 ? slab * 2 : 0);
  // LPR = HD / 8 lanes share a row: lane c reads float4 c and LPR + c of
  // both halves (adjacent lanes, adjacent 16 bytes: no LDS bank conflicts),
  // combines each into four bf16 and swaps one 8-byte half with its
  // neighbour, so even lane 2j ends with the row's 16-byte output chunk j and
  // odd lane 2j + 1 with chunk LPR / 2 + j.  A wave covers 64 / LPR rows per
  // pass, the workgroup's 4 waves the 64 rows in LPR / 4 passes.
  constexpr int LPR = HD / 8, RPP = 64 / LPR, PASSES = LPR / 4;
  const int c = l % LPR, odd = c & 1;
  uint4 res[PASSES];
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int row = (w + 4 * p) * RPP + l / LPR;
    const float2 h0 = sm.mlh[0][row], h1 = sm.mlh[1][row];
    const float mm = fmaxf(h0.x, h1.x);
    const float a0 = h0.x == -INFINITY ? 0.f : exp2f(h0.x - mm);
    const float a1 = h1.x == -INFINITY ? 0.f : exp2f(h1.x - mm);
    const float inv = 1.f / (h0.y * a0 + h1.y * a1);
    const float s0 = a0 * inv, s1 = a1 * inv;
    const float* p0 = park + row * PROW;
    const float* p1 = p0 + 64 * PROW;
    uint2 half[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int f4 = LPR * e + c;
      const float4 x = *reinterpret_cast<const float4*>(p0 + 4 * f4);
      const float4 y = *reinterpret_cast<const float4*>(p1 + 4 * f4);
      half[e] = make_uint2(pack2(x.x * s0 + y.x * s1, x.y * s0 + y.y * s1),
                           pack2(x.z * s0 + y.z * s1, x.w * s0 + y.w * s1));
    }
    const uint2 give = odd ? half[0] : half[1];
    const uint2 got = make_uint2(__shfl_xor(give.x, 1), __shfl_xor(give.y, 1));
    res[p] = odd ? make_uint4(got.x, got.y, half[1].x, half[1].y)
                 : make_uint4(half[0].x, half[0].y, got.x, got.y);
  }
  // then all the stores (interleaved with the reads they would serialise them)
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int row = (w + 4 * p) * RPP + l / LPR;
    const int ch = (c >> 1) + (odd ? LPR / 2 : 0);   // 16-byte chunk of the row
    if (a.splits == 1) {
      const int ar = 64 * rb + row;
      if (ar < rows) {
        const int t = ar / G, h = hk * G + (ar - t * G);
        buf_st16(ro, (int)(fa_index(b * a.T + t, h * HD + 8 * ch, MTo) * 2), res[p]);
      }
    } else {
      buf_st16(rpo, (row * HD + 8 * ch) * 2, res[p]);
    }
  }
  if (a.splits == 1) return true;
  if (tid < 64) {
    const float2 h0 = sm.mlh[0][tid], h1 = sm.mlh[1][tid];
    const float mm = fmaxf(h0.x, h1.x);
    const float a0 = h0.x == -INFINITY ? 0.f : exp2f(h0.x - mm);
    const float a1 = h1.x == -INFINITY ? 0.f : exp2f(h1.x - mm);
    const __amdgpu_buffer_rsrc_t rpm = make_rsrc(a.part_ml + ((size_t)ks * n_rbt + rb_id) * 128, 512);
    buf_st8(rpm, tid * 8, __float_as_uint(mm), __float_as_uint(h0.y * a0 + h1.y * a1));
  }
  return false;
}

// Items of the key-slice merge: one per (row block, row, 16-byte chunk).
__host__ __device__ inline int attn_combine_items(int B, int T, int Hq, int Hkv, int HD) {
  return B * Hkv * ((Hq / Hkv * T + 63) / 64) * 64 * (HD / 8);
}

// Merges the key slices of attn_sm_task for the 256 items of workgroup-sized
// task `task`: o = sum_s w_s o_s / sum_s w_s with w_s = l_s 2^(m_s - max m),
// in slice order, stored in the O projection's operand order.
template <int HD>
__device__ void attn_combine_task(const AttnSmArgs& a, int task) {
  constexpr int CPR = HD / 8;
  const int G = a.Hq / a.Hkv;
  const int rows = G * a.T;
  const int n_rb = (rows + 63) >> 6;
  const int n_rbt = a.B * a.Hkv * n_rb;
  const int i = task * 256 + (int)threadIdx.x;
  if (i >= n_rbt * 64 * CPR) return;
  const int rb_id = i / (64 * CPR), rem = i - rb_id * 64 * CPR;
  const int row = rem / CPR, c = rem - row * CPR;
  const int bh = rb_id / n_rb, rb = rb_id - bh * n_rb;
  const int b = bh / a.Hkv, hk = bh - b * a.Hkv;
  const int ar = 64 * rb + row;
  if (ar >= rows) return;
  const size_t slab = (size_t)64 * HD;
  const __amdgpu_buffer_rsrc_t rpo = make_rsrc(a.part_o, (size_t)a.splits * n_rbt * slab * 2);
  const __amdgpu_buffer_rsrc_t rpm = make_rsrc(a.part_ml, (size_t)a.splits * n_rbt * 512);
  float2 ml[kAttnMaxSplits];
  uint4 pv[kAttnMaxSplits];
#pragma unroll
  for (int sp = 0; sp < kAttnMaxSplits; ++sp)
    if (sp < a.splits) {
      const u32x2v u = __builtin_amdgcn_raw_buffer_load_b64(rpm, ((sp * n_rbt + rb_id) * 64 + row) * 8, 0, 16);
      ml[sp] = make_float2(__uint_as_float(u[0]), __uint_as_float(u[1]));
      pv[sp] = buf_ld_act(rpo, (int)((((size_t)sp * n_rbt + rb_id) * 64 + row) * HD + 8 * c) * 2);
    }
  float mx = -INFINITY;
#pragma unroll
  for (int sp = 0; sp < kAttnMaxSplits; ++sp)
    if (sp < a.splits) mx = fmaxf(mx, ml[sp].x);
  float den = 0.f;
  float f[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int sp = 0; sp < kAttnMaxSplits; ++sp)
    if (sp < a.splits) {
      const float wgt = ml[sp].x == -INFINITY ? 0.f : ml[sp].y * exp2f(ml[sp].x - mx);
      den += wgt;
      float x[8];
      unpack8(pv[sp], x);
#pragma unroll
      for (int e = 0; e < 8; ++e) f[e] = fmaf(wgt, x[e], f[e]);
    }
  const float inv = 1.f / den;
#pragma unroll
  for (int e = 0; e < 8; ++e) f[e] *= inv;
  const int t = ar / G, h = hk * G + (ar - t * G);
  const int MTo = mt_of(a.B * a.T);
  const __amdgpu_buffer_rsrc_t ro = make_rsrc(a.o, (size_t)MTo * 16 * a.Hq * HD * 2);
  buf_st16(ro, (int)(fa_index(b * a.T + t, h * HD + 8 * c, MTo) * 2), pack8(f));
}

}  // namespace blk
