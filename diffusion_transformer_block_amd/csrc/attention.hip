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
// streamed in tiles of 32 through LDS.
//
// Per tile and wave:  S^T = K Q^T with MFMA 16x16x32 (K rows from LDS as the
// A operand, the wave's 16 query rows as the B operand kept in registers), so
// each lane holds 8 scores of ONE query row (lane % 16) -- exactly the B
// operand layout that O^T += V^T P^T needs, and the softmax statistics live
// in the same lane as that query's output columns: no shuffles besides the
// two cross-group max / sum steps.  V is written to LDS transposed so V^T's
// A fragments are two 8-byte reads.  Online softmax in base 2 (scale folded
// into log2(e) / sqrt(d)).
//
// Key slices: when (rows / 64) x streams x kv-heads is far below the number of
// compute units, keys are split across workgroups; each writes its unnormalised
// O, its running max and sum, and the last-arriving workgroup of a row block
// (device-scope counter, reset by that workgroup) combines the slices in order.
#include "common.h"
#include "internal.h"

namespace blk {

constexpr int kKeyTile = 32;

template <int HD>
__global__ __launch_bounds__(256) void chunk_attn_kernel(AttnArgs a) {
  constexpr int KS_ROW = HD + 8;            // bf16 per K row in LDS
  constexpr int VT_ROW = kKeyTile + 8;      // bf16 per transposed V row in LDS
  constexpr int NKS = HD / 32;              // k-steps of S^T
  constexpr int NDT = HD / 16;              // 16-row tiles of O^T
  constexpr int CH = kKeyTile * HD / 8;     // 16-byte chunks per K (or V) tile
  __shared__ __attribute__((aligned(16))) bf16_t Ks[kKeyTile * KS_ROW];
  __shared__ __attribute__((aligned(16))) bf16_t Vt[HD * VT_ROW];
  __shared__ int last_flag;

  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63, lr = l & 15, lg = l >> 4;
  const int qb = blockIdx.x;
  const int bh = blockIdx.y;               // b * Hkv + hk
  const int b = bh / a.Hkv, hk = bh - b * a.Hkv;
  const int split = blockIdx.z;
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
  for (int ks = 0; ks < NKS; ++ks) qf[ks] = *reinterpret_cast<const uint4*>(qp + 32 * ks);

  const bf16_t* kpb = a.kp ? a.kp + (size_t)b * a.prefix_stride : nullptr;
  const bf16_t* vpb = a.vp ? a.vp + (size_t)b * a.prefix_stride : nullptr;
  const bf16_t* knb = a.kn + (size_t)b * a.new_stride;
  const bf16_t* vnb = a.vn + (size_t)b * a.new_stride;

  f32x4 o[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  for (int base = key_begin; base < key_end; base += kKeyTile) {
    // ---- stage K (row-major) and V (transposed) of keys [base, base + 32)
#pragma unroll
    for (int q = 0; q < CH / 256; ++q) {
      const int cidx = tid + 256 * q;
      const int kk = cidx / (HD / 8);
      const int d0 = (cidx - kk * (HD / 8)) * 8;
      const int key = base + kk;
      uint4 kv = make_uint4(0, 0, 0, 0), vv = make_uint4(0, 0, 0, 0);
      if (key < key_end) {
        size_t off;
        const bf16_t *ks, *vs;
        if (key < a.P) {
          off = ((size_t)key * a.Hkv + hk) * HD + d0;
          ks = kpb;
          vs = vpb;
        } else {
          off = ((size_t)(key - a.P) * a.Hkv + hk) * HD + d0;
          ks = knb;
          vs = vnb;
        }
        kv = *reinterpret_cast<const uint4*>(ks + off);
        vv = *reinterpret_cast<const uint4*>(vs + off);
      }
      *reinterpret_cast<uint4*>(&Ks[kk * KS_ROW + d0]) = kv;
      const uint32_t vw[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        Vt[(d0 + 2 * e) * VT_ROW + kk] = (bf16_t)(vw[e] & 0xffffu);
        Vt[(d0 + 2 * e + 1) * VT_ROW + kk] = (bf16_t)(vw[e] >> 16);
      }
    }
    __syncthreads();

    // ---- S^T = K Q^T: lane holds S[query lr][key 16 mt + 4 lg + j]
    f32x4 s[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      s[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const uint4 kf = *reinterpret_cast<const uint4*>(&Ks[(16 * mt + lr) * KS_ROW + 32 * ks + 8 * lg]);
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
      const bf16_t* vrow = &Vt[(16 * dt + lr) * VT_ROW];
      const uint2 lo = *reinterpret_cast<const uint2*>(vrow + 4 * lg);
      const uint2 hi = *reinterpret_cast<const uint2*>(vrow + 16 + 4 * lg);
      const bf16x8 va = as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
      o[dt] = o[dt] * alpha;
      o[dt] = mfma16(va, pb, o[dt]);
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
        uint2 v;
        v.x = pack2(o[dt][0] * inv, o[dt][1] * inv);
        v.y = pack2(o[dt][2] * inv, o[dt][3] * inv);
        *reinterpret_cast<uint2*>(op + 16 * dt) = v;
      }
    }
    return;
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
  if (!arrive_last(&a.counters[rb_id], (unsigned)a.splits, &last_flag)) return;

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
      *reinterpret_cast<uint32_t*>(op + c) = pack2(num[c] * inv, num[c + 1] * inv);
  }
}

void attn_plan(int B, int T, int P, int Hq, int Hkv, int d, int* splits, int* keys_per_split) {
  (void)d;
  const int G = Hq / Hkv;
  const int n_rb = (G * T + 63) / 64;
  const long wgs = (long)n_rb * B * Hkv;
  const int L = P + T;
  int s = 1;
  if (wgs < 256) {
    s = (int)((512 + wgs - 1) / wgs);
    const int max_s = (L + 127) / 128;  // at least four key tiles per slice
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
