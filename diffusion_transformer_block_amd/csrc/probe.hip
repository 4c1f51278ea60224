// Measurement probes: the sustained HBM read bandwidth, the dense bf16 MFMA
// throughput and the shader clock of the device the caller's stream runs on.
// They are not part of the block stage: benchmarks report them beside the
// chip's nominal peaks (8 TB/s HBM3E, 2.5 PFLOP/s dense bf16 at 2.4 GHz), so
// a roofline fraction can be read against what the part sustains.
#include <hip/hip_runtime.h>

#include <string>

#include "../../include/blk.h"
#include "common.h"

namespace blk {

// A sink the probes write (through a pointer argument) only when an
// impossible value turns up, so the compiler keeps their loads and MFMAs;
// probe_clk receives the clock counters.
static __device__ unsigned probe_sink[4];
static __device__ unsigned long long probe_clk[2];

// HBM read: a grid-stride stream of 16-byte non-temporal loads, eight in
// flight per thread, folded into one word.
__global__ __launch_bounds__(256) void probe_read_kernel(const uint4* buf, size_t n16, unsigned* sink) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  unsigned acc = 0;
  for (; i + 7 * stride < n16; i += 8 * stride) {
    uint4 v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = ld_stream(buf + i + j * stride);
#pragma unroll
    for (int j = 0; j < 8; ++j) acc ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
  }
  for (; i < n16; i += stride) {
    const uint4 v = ld_stream(buf + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9e3779b9u) sink[0] = acc;
}

// Dense bf16 MFMA: every wave runs four independent chains of
// v_mfma_f32_32x32x16_bf16 on register operands.  Workgroup 0 records the
// shader-clock counter (s_memtime) and the 100 MHz constant counter
// (s_memrealtime) around its loop, which gives the clock under MFMA load.
__global__ __launch_bounds__(256) void probe_mfma_kernel(int iters, unsigned long long* clk, unsigned* sink) {
  typedef float f32x16 __attribute__((ext_vector_type(16)));
  const unsigned t = threadIdx.x + 1;
  const bf16x8 a = as_bf16x8(make_uint4(pack2(1.f / t, 0.5f), pack2(0.25f, 1.f), pack2(0.5f, 0.25f), pack2(1.f, 0.5f)));
  const bf16x8 b = as_bf16x8(make_uint4(pack2(0.5f, 1.f / t), pack2(1.f, 0.25f), pack2(0.25f, 0.5f), pack2(0.5f, 1.f)));
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  unsigned long long m0 = 0, r0 = 0;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    m0 = __builtin_readcyclecounter();
    r0 = __builtin_amdgcn_s_memrealtime();
  }
  for (int i = 0; i < iters; ++i) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    clk[0] = __builtin_readcyclecounter() - m0;
    clk[1] = __builtin_amdgcn_s_memrealtime() - r0;
  }
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < 16; ++e) s += c0[e] + c1[e] + c2[e] + c3[e];
  if (s == -1.f) sink[1] = 1u;
}

}  // namespace blk

using namespace blk;

namespace {
thread_local std::string g_probe_err;

int probe_fail(int code, const char* what, hipError_t e) {
  g_probe_err = std::string(what) + ": " + hipGetErrorString(e);
  return code;
}
#define PROBE_TRY(expr)                                            \
  do {                                                             \
    hipError_t e_ = (expr);                                        \
    if (e_ != hipSuccess) return probe_fail(BLK_EHIP, #expr, e_);  \
  } while (0)

// Elapsed milliseconds of `launch` run `reps` times on st, bracketed by events.
template <class F>
int time_on_stream(hipStream_t st, int reps, F&& launch, float* ms) {
  hipEvent_t e0 = nullptr, e1 = nullptr;
  PROBE_TRY(hipEventCreate(&e0));
  hipError_t e = hipEventCreate(&e1);
  if (e != hipSuccess) {
    (void)hipEventDestroy(e0);
    return probe_fail(BLK_EHIP, "hipEventCreate", e);
  }
  launch();   // warm-up
  e = hipEventRecord(e0, st);
  for (int r = 0; r < reps && e == hipSuccess; ++r) {
    launch();
    e = hipGetLastError();
  }
  if (e == hipSuccess) e = hipEventRecord(e1, st);
  if (e == hipSuccess) e = hipEventSynchronize(e1);
  if (e == hipSuccess) e = hipEventElapsedTime(ms, e0, e1);
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  if (e != hipSuccess) return probe_fail(BLK_EHIP, "probe timing", e);
  return BLK_OK;
}
}  // namespace

extern "C" {

const char* blk_probe_last_error(void) { return g_probe_err.c_str(); }

int blk_probe_hbm_read(const void* buf, size_t bytes, int reps, double* gb_per_s, void* stream) {
  g_probe_err.clear();
  if (!buf || !gb_per_s || reps <= 0 || bytes < (size_t(1) << 20) || bytes % 16 != 0 ||
      reinterpret_cast<uintptr_t>(buf) % 16 != 0)
    return (g_probe_err = "buf/gb_per_s NULL, reps <= 0, or bytes < 1 MiB / not a multiple of 16 / misaligned",
            BLK_EINVAL);
  hipStream_t st = (hipStream_t)stream;
  int dev = 0, cus = 0;
  PROBE_TRY(hipGetDevice(&dev));
  PROBE_TRY(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev));
  const unsigned grid = (unsigned)(cus > 0 ? cus : 256) * 8;
  const uint4* p = reinterpret_cast<const uint4*>(buf);
  const size_t n16 = bytes / 16;
  unsigned* sink = nullptr;
  PROBE_TRY(hipGetSymbolAddress(reinterpret_cast<void**>(&sink), HIP_SYMBOL(probe_sink)));
  float ms = 0.f;
  (void)hipGetLastError();
  const int rc = time_on_stream(st, reps, [&] { probe_read_kernel<<<grid, 256, 0, st>>>(p, n16, sink); }, &ms);
  if (rc) return rc;
  *gb_per_s = (double)bytes * reps / (ms * 1e-3) / 1e9;
  return BLK_OK;
}

int blk_probe_mfma_bf16(int iters, double* tflops, double* clock_ghz, void* stream) {
  g_probe_err.clear();
  if (!tflops || !clock_ghz || iters <= 0 || iters > (1 << 24))
    return (g_probe_err = "tflops/clock_ghz NULL or iters outside [1, 2^24]", BLK_EINVAL);
  hipStream_t st = (hipStream_t)stream;
  int dev = 0, cus = 0;
  PROBE_TRY(hipGetDevice(&dev));
  PROBE_TRY(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev));
  const unsigned grid = (unsigned)(cus > 0 ? cus : 256) * 2;   // two waves per SIMD
  unsigned long long* clk = nullptr;
  unsigned* sink = nullptr;
  PROBE_TRY(hipGetSymbolAddress(reinterpret_cast<void**>(&clk), HIP_SYMBOL(probe_clk)));
  PROBE_TRY(hipGetSymbolAddress(reinterpret_cast<void**>(&sink), HIP_SYMBOL(probe_sink)));
  float ms = 0.f;
  (void)hipGetLastError();
  const int reps = 3;
  const int rc = time_on_stream(st, reps, [&] { probe_mfma_kernel<<<grid, 256, 0, st>>>(iters, clk, sink); }, &ms);
  if (rc) return rc;
  unsigned long long c[2] = {0, 0};
  PROBE_TRY(hipMemcpy(c, clk, sizeof c, hipMemcpyDeviceToHost));
  const double flop = 2.0 * 32 * 32 * 16 * 4 * (double)iters * grid * 4 * reps;   // 4 waves per workgroup
  *tflops = flop / (ms * 1e-3) / 1e12;
  *clock_ghz = c[1] ? (double)c[0] / ((double)c[1] * 10.0) : 0.0;   // s_memrealtime ticks at 100 MHz
  return BLK_OK;
}

}  // extern "C"
