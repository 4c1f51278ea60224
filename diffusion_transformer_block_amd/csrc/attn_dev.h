// Chunk attention task (device function) shared by the standalone kernel and
// the persistent stage kernel.  See attention.hip for the method notes.
#pragma once
#include "common.h"
#include "internal.h"

namespace blk {

constexpr int kKeyTile = 32;

template <int HD>
struct AttnSmem {
  bf16_t Ks[2][kKeyTile * (HD + 8)];
  bf16_t Vt[2][HD * 36];
  int last_flag;
};

// One (row block qb, stream x kv-head bh, key slice split) task.  Returns true
// if this workgroup wrote the rows' final output (no key split, or the last
// slice to arrive).
template <int HD>
__device__ bool attn_task(const AttnArgs& a, int qb, int bh, int split, AttnSmem<HD>& sm) {
  constexpr int KS_ROW = HD + 8;            // bf16 per K row in LDS
  constexpr int VT_ROW = 36;                // bf16 per transposed V row (72 B: conflict-free)
  constexpr int NKS = HD / 32;              // k-steps of S^T
  constexpr int NDT = HD / 16;              // 16-row tiles of O^T
  constexpr int KCH = kKeyTile * HD / 8 / 256;   // 16-byte K chunks per thread per tile
  constexpr int VITEMS = 16 * (HD / 8);          // (key pair, chunk) items per tile
  constexpr int VIT = (VITEMS + 255) / 256;       // per thread
  auto& Ks = sm.Ks;
  auto& Vt = sm.Vt;

  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63, lr = l & 15, lg = l >> 4;
  const int b = bh / a.Hkv, hk = bh - b * a.Hkv;
  const int G = a.Hq / a.Hkv;
  const int rows = G * a.T;
  const int L = a.P + a.T;
  const int key_begin = split * a.keys_per_split;
  const int key_end = min(L, key_begin + a.keys_per_split);

  // this lane's query row (B operand of S^T, and the owner of its softmax stats)
  const int qrow = qb * 64 + 16 * w + lr;
  const int qrc = min(qrow, rows - 1);
  const int qt = qrc / G, qh = hk * G + (qrc - qt * G);
  const bf16_t* qp = a.q + ((size_t)(b * a.T + qt) * a.Hq + qh) * HD + 8 * lg;
  uint4 qf[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) qf[ks] = ld_act16(qp + 32 * ks);

  const bf16_t* kpb = a.kp ? a.kp + (size_t)b * a.prefix_stride : nullptr;
  const bf16_t* vpb = a.vp ? a.vp + (size_t)b * a.prefix_stride : nullptr;
  const bf16_t* knb = a.kn + (size_t)b * a.new_stride;
  const bf16_t* vnb = a.vn + (size_t)b * a.new_stride;
  // prefix rows are read-only caller data; the chunk's own rows were written by
  // the QKV step (possibly earlier in the same kernel): coherent loads
  auto kv_load = [&](const bf16_t* pre, const bf16_t* own, int key, int off) -> uint4 {
    return key < a.P ? *reinterpret_cast<const uint4*>(pre + ((size_t)key * a.Hkv + hk) * HD + off)
                     : ld_act16(own + ((size_t)(key - a.P) * a.Hkv + hk) * HD + off);
  };

  // ---- tile staging: K row-major (coalesced 16-byte chunks), V as key pairs
  uint4 kreg[KCH], vreg[VIT][2];
  auto load_tile = [&](int base) {
#pragma unroll
    for (int q = 0; q < KCH; ++q) {
      const int cidx = tid + 256 * q;
      const int kk = cidx / (HD / 8);
      const int d0 = (cidx - kk * (HD / 8)) * 8;
      const int key = base + kk;
      kreg[q] = key < key_end ? kv_load(kpb, knb, key, d0) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int q = 0; q < VIT; ++q) {
      const int item = tid + 256 * q;
      const int kp = item & 15, c = item >> 4;     // key pair, 8-wide chunk of the head dim
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int key = base + 2 * kp + h;
        vreg[q][h] = (item < VITEMS && key < key_end) ? kv_load(vpb, vnb, key, 8 * c)
                                                      : make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int q = 0; q < KCH; ++q) {
      const int cidx = tid + 256 * q;
      const int kk = cidx / (HD / 8);
      const int d0 = (cidx - kk * (HD / 8)) * 8;
      *reinterpret_cast<uint4*>(&Ks[buf][kk * KS_ROW + d0]) = kreg[q];
    }
#pragma unroll
    for (int q = 0; q < VIT; ++q) {
      const int item = tid + 256 * q;
      if (VITEMS % 256 != 0 && item >= VITEMS) break;
      const int kp = item & 15, c = item >> 4;
      const uint32_t a0[4] = {vreg[q][0].x, vreg[q][0].y, vreg[q][0].z, vreg[q][0].w};
      const uint32_t a1[4] = {vreg[q][1].x, vreg[q][1].y, vreg[q][1].z, vreg[q][1].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        *reinterpret_cast<uint32_t*>(&Vt[buf][(8 * c + 2 * e) * VT_ROW + 2 * kp]) =
            (a0[e] & 0xffffu) | (a1[e] << 16);
        *reinterpret_cast<uint32_t*>(&Vt[buf][(8 * c + 2 * e + 1) * VT_ROW + 2 * kp]) =
            (a0[e] >> 16) | (a1[e] & 0xffff0000u);
      }
    }
  };

  f32x4 o[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  const int n_tiles = (key_end - key_begin + kKeyTile - 1) / kKeyTile;
  __syncthreads();   // a previous task's readers of sm are done
  if (n_tiles > 0) {
    load_tile(key_begin);
    store_tile(0);
    if (n_tiles > 1) load_tile(key_begin + kKeyTile);
  }
  __syncthreads();

  for (int it = 0; it < n_tiles; ++it) {
    const int cur = it & 1;
    const int base = key_begin + it * kKeyTile;
    // ---- S^T = K Q^T: lane holds S[query lr][key 16 mt + 4 lg + j]
    f32x4 s[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      s[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const uint4 kf = *reinterpret_cast<const uint4*>(&Ks[cur][(16 * mt + lr) * KS_ROW + 32 * ks + 8 * lg]);
        s[mt] = mfma16(as_bf16x8(kf), as_bf16x8(qf[ks]), s[mt]);
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

    // ---- O^T += V^T P^T; P^T slot e of lane group lg is key 4 lg + e (e < 4)
    //      or 16 + 4 lg + e - 4 (e >= 4), matching the S^T output layout.
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const bf16_t* vrow = &Vt[cur][(16 * dt + lr) * VT_ROW];
      const uint2 lo = *reinterpret_cast<const uint2*>(vrow + 4 * lg);
      const uint2 hi = *reinterpret_cast<const uint2*>(vrow + 16 + 4 * lg);
      o[dt] = o[dt] * alpha;
      o[dt] = mfma16(as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y)), pb, o[dt]);
    }
    // ---- stage the tile after next into the other buffer (last read one tile ago)
    if (it + 1 < n_tiles) {
      store_tile(cur ^ 1);
      if (it + 2 < n_tiles) load_tile(base + 2 * kKeyTile);
    }
    __syncthreads();
  }

  float l_tot = l_run;
  l_tot += __shfl_xor(l_tot, 16);
  l_tot += __shfl_xor(l_tot, 32);

  const int n_rb = (rows + 63) / 64;
  const size_t rb_id = (size_t)bh * n_rb + qb;   // row block id over all (b, hk)

  if (a.splits == 1) {
    if (qrow < rows) {
      const float inv = 1.f / l_tot;
      const int t = qrow / G, h = hk * G + (qrow - t * G);
      bf16_t* op = a.o + ((size_t)(b * a.T + t) * a.Hq + h) * HD + 4 * lg;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const uint64_t v = (uint64_t)pack2(o[dt][0] * inv, o[dt][1] * inv) |
                           ((uint64_t)pack2(o[dt][2] * inv, o[dt][3] * inv) << 32);
        __hip_atomic_store(reinterpret_cast<uint64_t*>(op + 16 * dt), v, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    return true;
  }

  // ---- split keys: publish partial (o, m, l), last workgroup combines in order
  const size_t n_rbt = (size_t)a.B * a.Hkv * n_rb;
  {
    float* po = a.part_o + ((size_t)split * n_rbt + rb_id) * 64 * HD + (size_t)(16 * w + lr) * HD + 4 * lg;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      st_dev2(po + 16 * dt, o[dt][0], o[dt][1]);
      st_dev2(po + 16 * dt + 2, o[dt][2], o[dt][3]);
    }
    if (lg == 0) {
      float* pm = a.part_ml + (((size_t)split * n_rbt + rb_id) * 64 + 16 * w + lr) * 2;
      st_dev2(pm, m_run, l_tot);
    }
  }
  if (!arrive_last(&a.counters[rb_id], (unsigned)a.splits, &sm.last_flag)) return false;

  // 4 threads per row, each HD/4 columns
  const int row = tid >> 2;
  const int qrow2 = qb * 64 + row;
  if (qrow2 < rows) {
    float mx = -INFINITY;
    for (int sp = 0; sp < a.splits; ++sp)
      mx = fmaxf(mx, ld_dev2(a.part_ml + (((size_t)sp * n_rbt + rb_id) * 64 + row) * 2).x);
    float den = 0.f;
    constexpr int QC = HD / 4;
    float num[QC];
#pragma unroll
    for (int c = 0; c < QC; ++c) num[c] = 0.f;
    for (int sp = 0; sp < a.splits; ++sp) {
      const float2 ml = ld_dev2(a.part_ml + (((size_t)sp * n_rbt + rb_id) * 64 + row) * 2);
      const float wgt = exp2f(ml.x - mx);
      den += wgt * ml.y;
      const float* po = a.part_o + ((size_t)sp * n_rbt + rb_id) * 64 * HD + (size_t)row * HD + (tid & 3) * QC;
#pragma unroll
      for (int c = 0; c < QC; c += 2) {
        const float2 v = ld_dev2(po + c);
        num[c] += wgt * v.x;
        num[c + 1] += wgt * v.y;
      }
    }
    const float inv = 1.f / den;
    const int t = qrow2 / G, h = hk * G + (qrow2 - t * G);
    bf16_t* op = a.o + ((size_t)(b * a.T + t) * a.Hq + h) * HD + (tid & 3) * QC;
#pragma unroll
    for (int c = 0; c < QC; c += 2)
      __hip_atomic_store(reinterpret_cast<uint32_t*>(op + c), pack2(num[c] * inv, num[c + 1] * inv),
                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  return true;
}

}  // namespace blk
