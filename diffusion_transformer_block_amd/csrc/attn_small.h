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
// so one K/V tile serves 64 rows (16 per wave).  A task takes 64 rows and one
// slice of the keys:
//  * K / V tiles of 32 keys are loaded with row-contiguous 16-byte loads two
//    tiles ahead of use and staged through double-buffered LDS;
//  * S^T = K Q^T on MFMA, K rows as the A operand (LDS), Q^T as the B operand
//    held in registers (the QKV epilogue stores Q in exactly that operand
//    order, qa_index), so a lane ends up with 4 keys of one row;
//  * online softmax per row in base 2 (scores pre-scaled by log2(e)/sqrt(d));
//  * O^T += V^T P^T on MFMA: P^T is the B operand straight from the score
//    registers (slot e of lane group lg is key 4 lg + e, or 16 + 4 lg + e - 4
//    for e >= 4), V^T the A operand read out of the row-major V tile with
//    ds_read_b64_tr_b16, which hands lane i of each 16-lane group element
//    i % 4 of the 8 bytes at lane 4 k + i / 4 (k < 4): pointing lane i at
//    key 4 lg + i / 4, dims 4 (i % 4) .. + 3 yields V[4 lg + k][i] -- the
//    same key order as P^T;
//  * one key slice writes the normalised rows straight into the O
//    projection's operand order; several slices publish bf16 partials
//    normalised by their own sum plus (max, sum), and the last slice to arrive
//    (device counter, reset by it) combines all of them in slice order.
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
  unsigned* counters;     // [n_rbt]
};

constexpr int kAttnMaxSplits = 8;

template <int HD>
struct AttnSmSmem {
  bf16_t k[2][32 * (HD + 8)];
  bf16_t v[2][32 * (HD + 16)];
  int last_flag;
};

__device__ __forceinline__ uint2 lds_tr16(const bf16_t* p) {
  typedef short v4s __attribute__((ext_vector_type(4)));
  const v4s v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)(p));
  return __builtin_bit_cast(uint2, v);
}

// One task: stream x kv head bh, 64-row block rb, key slice ks.  Returns true
// if this workgroup wrote the block's final rows.
template <int HD, class Wait>
__device__ bool attn_sm_task(const AttnSmArgs& a, int bh, int rb, int ks, AttnSmSmem<HD>& sm,
                             Wait&& wait) {
  constexpr int KROW = HD + 8, VROW = HD + 16;
  constexpr int NKS = HD / 32;                 // 32-wide k-steps of S^T
  constexpr int NDT = HD / 16;                 // 16-row tiles of O^T
  constexpr int CPR = HD / 8;                  // 16-byte chunks per key row
  constexpr int NCH = 32 * CPR / 256;          // chunks per thread per tile (K or V)
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index (uniform)
  const int l = tid & 63, lr = l & 15, lg = l >> 4;
  const int b = bh / a.Hkv, hk = bh - b * a.Hkv;
  const int G = a.Hq / a.Hkv;
  const int rows = G * a.T;
  const int n_rt = (rows + 15) >> 4;
  const int L = a.P + a.T;
  const int key_begin = ks * a.kps;
  const int key_end = min(L, key_begin + a.kps);
  const int n_tiles = (key_end - key_begin + 31) >> 5;

  const bf16_t* kpb = a.kp ? a.kp + (size_t)b * a.prefix_stride + (size_t)hk * HD : nullptr;
  const bf16_t* vpb = a.vp ? a.vp + (size_t)b * a.prefix_stride + (size_t)hk * HD : nullptr;
  const bf16_t* knb = a.kn + (size_t)b * a.new_stride + (size_t)hk * HD;
  const bf16_t* vnb = a.vn + (size_t)b * a.new_stride + (size_t)hk * HD;
  const int kvrow = a.Hkv * HD;
  // K (h = 0) / V (h = 1) chunk c of key `key`; zero past the slice
  auto ld_kv = [&](int h, int key, int c) -> uint4 {
    if (key >= key_end) return make_uint4(0, 0, 0, 0);
    if (key < a.P) {
      const bf16_t* p = (h ? vpb : kpb) + (size_t)key * kvrow + 8 * c;
      return *reinterpret_cast<const uint4*>(p);
    }
    return ld16c((h ? vnb : knb) + (size_t)(key - a.P) * kvrow + 8 * c);
  };
  uint4 reg[2][2][NCH];   // [ring slot][K, V][chunk]
  auto load_tile = [&](int slot, int tile) {
    const int base = key_begin + 32 * tile;
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      const int idx = tid + 256 * j;
      const int kk = idx / CPR, c = idx - kk * CPR;
      reg[slot][0][j] = ld_kv(0, base + kk, c);
      reg[slot][1][j] = ld_kv(1, base + kk, c);
    }
  };
  auto store_tile = [&](int slot, int buf) {
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      const int idx = tid + 256 * j;
      const int kk = idx / CPR, c = idx - kk * CPR;
      *reinterpret_cast<uint4*>(&sm.k[buf][kk * KROW + 8 * c]) = reg[slot][0][j];
      *reinterpret_cast<uint4*>(&sm.v[buf][kk * VROW + 8 * c]) = reg[slot][1][j];
    }
  };

  // prefix tiles do not depend on earlier work: start them before the wait
  const bool pre0 = key_begin + 32 <= a.P, pre1 = key_begin + 64 <= a.P;
  if (n_tiles > 0 && pre0) load_tile(0, 0);
  if (n_tiles > 1 && pre1) load_tile(1, 1);
  if (!wait()) return false;
  if (n_tiles > 0 && !pre0) load_tile(0, 0);
  if (n_tiles > 1 && !pre1) load_tile(1, 1);

  // this wave's 16 query rows: Q^T fragments (B operand), one per k-step
  const int rt = min(4 * rb + w, n_rt - 1);
  const __amdgpu_buffer_rsrc_t rq =
      make_rsrc(a.q + (size_t)(bh * n_rt + rt) * NKS * 512, (size_t)NKS * kFragBytes);
  uint4 qf[NKS];
#pragma unroll
  for (int s = 0; s < NKS; ++s) qf[s] = buf_ld_act(rq, s * kFragBytes + l * 16);

  f32x4 o[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  __syncthreads();   // a previous task's readers of sm are done
  if (n_tiles > 0) {
    store_tile(0, 0);
    if (n_tiles > 2) load_tile(0, 2);
  }
  __syncthreads();

  // one 32-key tile; CUR (= it & 1) is a compile-time constant so that the
  // register ring stays in registers
  auto step = [&](int it, auto cur_c) {
    constexpr int cur = decltype(cur_c)::value;
    const int base = key_begin + 32 * it;
    // ---- S^T: lane holds S[row lr][key 16 mt + 4 lg + j]
    f32x4 s[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      s[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ksx = 0; ksx < NKS; ++ksx) {
        const uint4 kf = *reinterpret_cast<const uint4*>(&sm.k[cur][(16 * mt + lr) * KROW + 32 * ksx + 8 * lg]);
        s[mt] = mfma16(as_bf16x8(kf), as_bf16x8(qf[ksx]), s[mt]);
      }
    }
    float x[8];
    float mloc = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int key = base + 16 * mt + 4 * lg + j;
        const float v = key < key_end ? s[mt][j] * a.scale_log2 : -INFINITY;
        x[mt * 4 + j] = v;
        mloc = fmaxf(mloc, v);
      }
    mloc = fmaxf(mloc, __shfl_xor(mloc, 16));
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
    const float m_new = fmaxf(m_run, mloc);
    const float alpha = exp2f(m_run - m_new);
    float psum = 0.f;
    uint32_t pw[4];
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const float p0 = exp2f(x[e] - m_new);
      const float p1 = exp2f(x[e + 1] - m_new);
      psum += p0 + p1;
      pw[e / 2] = pack2(p0, p1);
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
    const bf16x8 pb = as_bf16x8(make_uint4(pw[0], pw[1], pw[2], pw[3]));

    // ---- O^T += V^T P^T
    const bf16_t* vt = &sm.v[cur][(4 * lg + (lr >> 2)) * VROW + 4 * (lr & 3)];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const uint2 lo = lds_tr16(vt + 16 * dt);
      const uint2 hi = lds_tr16(vt + 16 * VROW + 16 * dt);
      o[dt] = o[dt] * alpha;
      o[dt] = mfma16(as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y)), pb, o[dt]);
    }
    // ---- stage the next tile (its buffer was last read one tile ago) and
    //      start the loads of the tile after the next; tile t sits in ring
    //      slot t & 1
    if (it + 1 < n_tiles) {
      store_tile(cur ^ 1, cur ^ 1);
      if (it + 3 < n_tiles) load_tile(cur ^ 1, it + 3);
    }
    __syncthreads();
  };
  for (int it = 0; it < n_tiles; it += 2) {
    step(it, std::integral_constant<int, 0>{});
    if (it + 1 < n_tiles) step(it + 1, std::integral_constant<int, 1>{});
  }

  float l_tot = l_run;
  l_tot += __shfl_xor(l_tot, 16);
  l_tot += __shfl_xor(l_tot, 32);

  const int n_rb = (rows + 63) >> 6;
  const int rb_id = bh * n_rb + rb;
  const int MTo = mt_of(a.B * a.T);
  const int arow = 64 * rb + 16 * w + lr;

  if (a.splits == 1) {
    if (arow < rows) {
      const float inv = 1.f / l_tot;
      const int t = arow / G, h = hk * G + (arow - t * G);
      const int m = b * a.T + t;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
        st8c(a.o + fa_index(m, h * HD + 16 * dt + 4 * lg, MTo), pack2(o[dt][0] * inv, o[dt][1] * inv),
             pack2(o[dt][2] * inv, o[dt][3] * inv));
    }
    return true;
  }

  // ---- several key slices: publish (o / l, m, l); the last combines
  const int n_rbt = a.B * a.Hkv * n_rb;
  {
    const float inv = 1.f / l_tot;
    bf16_t* po = a.part_o + (((size_t)ks * n_rbt + rb_id) * 64 + 16 * w + lr) * HD + 4 * lg;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
      st8c(po + 16 * dt, pack2(o[dt][0] * inv, o[dt][1] * inv), pack2(o[dt][2] * inv, o[dt][3] * inv));
    if (lg == 0)
      st8c(a.part_ml + (((size_t)ks * n_rbt + rb_id) * 64 + 16 * w + lr) * 2, __float_as_uint(m_run),
           __float_as_uint(l_tot));
  }
  if (!arrive_last(&a.counters[rb_id], (unsigned)a.splits, &sm.last_flag)) return false;

  // 4 threads per row, HD / 4 columns each, in two halves; all slices' loads
  // of a half are in flight together
  constexpr int QC = HD / 4, HC = QC / 16;   // 16-byte chunks per half
  const int row = tid >> 2, qq = tid & 3;
  const int arow2 = 64 * rb + row;
  if (arow2 < rows) {
    float mx = -INFINITY;
    float2 ml[kAttnMaxSplits];
#pragma unroll
    for (int sp = 0; sp < kAttnMaxSplits; ++sp)
      if (sp < a.splits) {
        const uint2 u = ld8c(a.part_ml + (((size_t)sp * n_rbt + rb_id) * 64 + row) * 2);
        ml[sp] = make_float2(__uint_as_float(u.x), __uint_as_float(u.y));
        mx = fmaxf(mx, ml[sp].x);
      }
    float den = 0.f, wgt[kAttnMaxSplits];
#pragma unroll
    for (int sp = 0; sp < kAttnMaxSplits; ++sp)
      if (sp < a.splits) {
        wgt[sp] = ml[sp].y * exp2f(ml[sp].x - mx);
        den += wgt[sp];
      }
    const float inv = 1.f / den;
    const int t = arow2 / G, h = hk * G + (arow2 - t * G);
    const int m = b * a.T + t;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const int c0 = qq * QC + hf * (QC / 2);
      uint4 pv[kAttnMaxSplits][HC];
#pragma unroll
      for (int sp = 0; sp < kAttnMaxSplits; ++sp)
        if (sp < a.splits) {
          const bf16_t* po = a.part_o + (((size_t)sp * n_rbt + rb_id) * 64 + row) * HD + c0;
#pragma unroll
          for (int c = 0; c < HC; ++c) pv[sp][c] = ld16c(po + 8 * c);
        }
#pragma unroll
      for (int c = 0; c < HC; ++c) {
        float f[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int sp = 0; sp < kAttnMaxSplits; ++sp)
          if (sp < a.splits) {
            float x[8];
            unpack8(pv[sp][c], x);
#pragma unroll
            for (int e = 0; e < 8; ++e) f[e] = fmaf(wgt[sp], x[e], f[e]);
          }
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] *= inv;
        st16c(a.o + fa_index(m, h * HD + c0 + 8 * c, MTo), pack8(f));
      }
    }
  }
  return true;
}

}  // namespace blk
