// Skinny GEMM task (M <= 64 rows) as a device function, shared by the
// standalone split-K kernel and the persistent stage kernel.
//
// [RT] = reading note on "Running VLAs at Real-time Speed" (Ma et al.,
// arXiv:2510.26742v1).  §5: bias / residual / activation merged into the GEMM
// tail; the gated FFN's two up-projections share one load of their input; the
// RMS statistic is consumed fused as a row scale; a partial split-K balances
// skinny shapes over the compute units; §6.2: at few tokens a GEMM is bound by
// reading its bf16 weights.
//
// One task = one 32-column group g (both 16-column tiles, as the fused QKV and
// gate/up epilogues need) over the K-range of split s.  The four waves split
// the K-range.  Each wave first issues all of its weight fragments for the
// task (16-byte streaming buffer loads, up to kMaxPrefetch k-tiles) -- weights
// do not depend on activations, so in the persistent kernel this happens
// before the wait for the producing step -- then streams the activation rows
// with device-coherent 16-byte buffer loads, four k-tiles per chunk, one chunk
// ahead of the MFMAs.  Buffer loads are bounds-checked by their descriptor
// (out-of-range reads return zero).  The waves reduce through LDS in a fixed
// order; with RMS the same pass sums x^2 of the rows it loaded.  K splits
// publish fp32 partials and the last workgroup of a group to arrive (device
// counter, reset by it) sums them in split order and runs the epilogue.
#pragma once
#include "common.h"
#include "internal.h"

namespace blk {

struct SkinnySmem {
  float red[4][4 * 2 * 256];  // [wave][(mt * 2 + i) * 64 + lane][4]
  float ssr[4][64];
  float rrow[64];
  int last_flag;
};

constexpr int kMaxPrefetch = 16;   // weight k-tiles per wave held in registers

__device__ __forceinline__ float sumsq8(uint4 v) {
  float s = 0.f;
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float lo = __uint_as_float(w[i] << 16);
    const float hi = __uint_as_float(w[i] & 0xffff0000u);
    s = fmaf(lo, lo, s);
    s = fmaf(hi, hi, s);
  }
  return s;
}

struct NoWait {
  __device__ __forceinline__ bool operator()() const { return true; }
};

// Computes the task and stores its outputs through `epi`.  `wait()` is called
// after the weight loads are issued and before the first activation load; it
// returns false to abandon the task (grid abort).  Returns false when the
// workgroup stops early (abandoned, or it only published a split partial).
template <int MT, bool RMS, class Epi, class Wait>
__device__ bool skinny_task(const GemmArgs& ga, const Epi& epi, int g, int s, SkinnySmem& sm,
                            Wait&& wait) {
  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63, lr = l & 15, lg = l >> 4;
  const int KT = ga.K >> 5;
  const int KTS = KT / ga.splits;
  const int KW = KTS >> 2;
  const int kt0 = s * KTS + w * KW;

  // ---- weights of this wave's k-range: fragments (g, kt, 0..1), all in flight
  const __amdgpu_buffer_rsrc_t rb =
      make_rsrc(ga.Bp + frag_offset(g, 0, 0, KT), (size_t)KT * 2 * kFragBytes);
  const int boff = (kt0 * 2) * kFragBytes + l * 16;
  uint4 bw[kMaxPrefetch][2];
  const int npf = KW < kMaxPrefetch ? KW : kMaxPrefetch;
#pragma unroll
  for (int q = 0; q < kMaxPrefetch; ++q)
    if (q < npf) {
      bw[q][0] = buf_ld_stream(rb, boff + q * 2 * kFragBytes);
      bw[q][1] = buf_ld_stream(rb, boff + q * 2 * kFragBytes + kFragBytes);
    }
  if (!wait()) return false;

  // ---- activations: rows 16 mt + lr, 8 consecutive k per lane group
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(ga.A, (size_t)ga.M * ga.lda * 2);
  int aoff[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int row = min(16 * mt + lr, ga.M - 1);
    aoff[mt] = (row * ga.lda + kt0 * 32 + 8 * lg) * 2;
  }

  f32x4 acc[MT][2];
  float ss[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    acc[mt][0] = f32x4{0.f, 0.f, 0.f, 0.f};
    acc[mt][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    ss[mt] = 0.f;
  }
  auto mma = [&](const uint4& a, int mt, const uint4& b0, const uint4& b1) {
    if (RMS) ss[mt] += sumsq8(a);
    acc[mt][0] = mfma16(as_bf16x8(a), as_bf16x8(b0), acc[mt][0]);
    acc[mt][1] = mfma16(as_bf16x8(a), as_bf16x8(b1), acc[mt][1]);
  };

  // chunks of 4 k-tiles; the next chunk's activations load while this one
  // multiplies.  Unrolled over the prefetch window so that every register
  // index is a compile-time constant.
  constexpr int CH = 4;
  if (KW <= kMaxPrefetch) {
    uint4 av[2][CH][MT];
    const int nfull = KW / CH;
    auto load_a = [&](int buf, int u0) {
#pragma unroll
      for (int q = 0; q < CH; ++q)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) av[buf][q][mt] = buf_ld_act(ra, aoff[mt] + (u0 + q) * 64);
    };
    if (nfull > 0) load_a(0, 0);
#pragma unroll
    for (int c = 0; c < kMaxPrefetch / CH; ++c) {
      if (c < nfull) {
        if (c + 1 < nfull) load_a((c + 1) & 1, (c + 1) * CH);
#pragma unroll
        for (int q = 0; q < CH; ++q)
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) mma(av[c & 1][q][mt], mt, bw[c * CH + q][0], bw[c * CH + q][1]);
      }
    }
#pragma unroll
    for (int u = 0; u < kMaxPrefetch; ++u) {   // tail k-tiles when KW is not a multiple of 4
      if (u >= nfull * CH && u < KW) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) mma(buf_ld_act(ra, aoff[mt] + u * 64), mt, bw[u][0], bw[u][1]);
      }
    }
  } else {
    // long K-ranges: the first kMaxPrefetch k-tiles come from the prefetch, the
    // rest stream one k-tile at a time
#pragma unroll
    for (int u = 0; u < kMaxPrefetch; ++u) {
      uint4 a[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) a[mt] = buf_ld_act(ra, aoff[mt] + u * 64);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) mma(a[mt], mt, bw[u][0], bw[u][1]);
    }
    for (int u = kMaxPrefetch; u < KW; ++u) {
      const uint4 b0 = buf_ld_stream(rb, boff + u * 2 * kFragBytes);
      const uint4 b1 = buf_ld_stream(rb, boff + u * 2 * kFragBytes + kFragBytes);
      uint4 a[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) a[mt] = buf_ld_act(ra, aoff[mt] + u * 64);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) mma(a[mt], mt, b0, b1);
    }
  }

  // ---- reduce the four waves' K ranges through LDS (a previous task's
  //      readers of sm must be done before it is overwritten)
  __syncthreads();
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int i = 0; i < 2; ++i)
      *reinterpret_cast<f32x4*>(&sm.red[w][((mt * 2 + i) * 64 + l) * 4]) = acc[mt][i];
  if (RMS) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      float v = ss[mt];
      v += __shfl_xor(v, 16);
      v += __shfl_xor(v, 32);
      if (lg == 0) sm.ssr[w][16 * mt + lr] = v;
    }
  }
  __syncthreads();

  float v[MT][2];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int ix = ((mt * 2 + i) * 64 + (tid >> 2)) * 4 + (tid & 3);
      v[mt][i] = ((sm.red[0][ix] + sm.red[1][ix]) + sm.red[2][ix]) + sm.red[3][ix];
    }
  float ssum = 0.f;
  if (RMS && tid < 16 * MT)
    ssum = ((sm.ssr[0][tid] + sm.ssr[1][tid]) + sm.ssr[2][tid]) + sm.ssr[3][tid];

  if (ga.splits > 1) {
    const size_t stride = (size_t)ga.n_groups * MT * 256 * 2;   // floats per split
    float* pbase = ga.part + ((size_t)g * MT * 256 + tid) * 2;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) st_dev2(pbase + s * stride + mt * 512, v[mt][0], v[mt][1]);
    if (RMS && tid < 16 * MT) st_dev(&ga.ss_part[((size_t)s * ga.n_groups + g) * 64 + tid], ssum);
    if (!arrive_last(&ga.counters[g], (unsigned)ga.splits, &sm.last_flag)) return false;
    float2 p[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      v[mt][0] = 0.f;
      v[mt][1] = 0.f;
    }
    ssum = 0.f;
    for (int s2 = 0; s2 < ga.splits; ++s2) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) p[mt] = ld_dev2(pbase + s2 * stride + mt * 512);
      const float sp = (RMS && tid < 16 * MT) ? ld_dev(&ga.ss_part[((size_t)s2 * ga.n_groups + g) * 64 + tid]) : 0.f;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        v[mt][0] += p[mt].x;
        v[mt][1] += p[mt].y;
      }
      ssum += sp;
    }
  }

  if (RMS) {
    if (tid < 16 * MT) sm.rrow[tid] = rsqrtf(ssum / (float)ga.K + ga.eps);
    __syncthreads();
  }
  const int c = (tid >> 2) & 15;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = 16 * mt + 4 * (tid >> 6) + (tid & 3);
    if (m < ga.M) {
      const float r = RMS ? sm.rrow[m] : (ga.r ? ga.r[m] : 1.f);
      epi.store(m, g, c, v[mt][0], v[mt][1], r);
    }
  }
  return true;
}

}  // namespace blk
