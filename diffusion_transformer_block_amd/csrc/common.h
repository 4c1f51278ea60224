// Shared device-side definitions for the block-stage kernels (gfx950 / CDNA4).
//
// Storage types: bf16 is carried as its 16-bit pattern (uint16_t); fp32 for
// gains, statistics, tables and accumulators.  MFMA operands are 8 x bf16 per
// lane (16 bytes), the operand width of v_mfma_f32_16x16x32_bf16.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace blk {

// Bytes that later kernels read, fetched by `wgs` extra workgroups of a
// launch while its tasks run.
struct Prefetch {
  const uint8_t* p = nullptr;
  size_t bytes = 0;
  int wgs = 0;
};

typedef uint16_t bf16_t;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// Streams of one call that may each have their own prefix length (a batch of
// chunks at different points of a history: [PS], section on same-block
// batching across chunks).  Kernels get a device pointer to the lengths
// (written into the workspace ahead of the block), or NULL when every stream
// has the call's P: a by-value table in the kernel arguments made the
// compiler serialize the argument loads of the kernels' prologues.
constexpr int kMaxVarStreams = 16;
__device__ __forceinline__ int stream_prefix(const int* plen, int P, int b) { return plen ? plen[b] : P; }

// ---------------------------------------------------------------- conversions
__device__ __forceinline__ float bf2f(bf16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// float -> bf16, round to nearest, ties to even; NaN stays NaN: gfx950's
// v_cvt_pk_bf16_f32, two per instruction (the first operand goes to the low
// half).  A two-lane vector conversion, not inline assembly: the compiler
// then inserts the wait states an MFMA result needs before this instruction
// reads it, which it cannot do for an assembly statement's inputs.
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
typedef float f32x2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2v{lo, hi}, bf16x2v));
}
__device__ __forceinline__ bf16_t f2bf(float f) { return (bf16_t)(pack2(f, 0.f) & 0xffffu); }

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

// 16-byte streaming load (read once: weights).
__device__ __forceinline__ uint4 ld_stream(const uint4* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// ---------------------------------------------------------------- cross-workgroup hand-off
// Partial results that another workgroup of the same kernel reads back go
// through device-coherent accesses (relaxed agent-scope atomics: sc1 loads and
// stores, coherent across the XCDs' L2 caches).  The writer waits for its
// stores to be acknowledged (vmcnt 0) before the workgroup bumps the arrival
// counter, so no device-wide fence -- an L2 write-back plus invalidate on this
// chip -- is needed.
__device__ __forceinline__ void st_dev(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev2(float* p, float a, float b) {
  const uint64_t v = (uint64_t)__float_as_uint(a) | ((uint64_t)__float_as_uint(b) << 32);
  __hip_atomic_store(reinterpret_cast<uint64_t*>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_dev(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float2 ld_dev2(const float* p) {
  const uint64_t v = __hip_atomic_load(reinterpret_cast<const uint64_t*>(p), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
  return make_float2(__uint_as_float((uint32_t)v), __uint_as_float((uint32_t)(v >> 32)));
}
__device__ __forceinline__ void wait_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Activations (bf16) produced by one workgroup and read by another within the
// same kernel: coherent 16-byte loads (two 8-byte agent-scope loads) and
// coherent 2-byte stores.
__device__ __forceinline__ uint4 ld_act16(const bf16_t* p) {
  const uint64_t* q = reinterpret_cast<const uint64_t*>(p);
  const uint64_t a = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint64_t b = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return make_uint4((uint32_t)a, (uint32_t)(a >> 32), (uint32_t)b, (uint32_t)(b >> 32));
}
__device__ __forceinline__ float ld_act(const bf16_t* p) {
  return bf2f(__hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}
__device__ __forceinline__ void st_act(bf16_t* p, float v) {
  __hip_atomic_store(p, f2bf(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_act_bits(bf16_t* p, bf16_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_f32c(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Publish this workgroup's partial (already stored with st_dev*) and report
// whether it is the last of `expected` workgroups to arrive at `counter`.  The
// last one resets the counter to zero for the next launch.  Call with every
// thread of the workgroup.
__device__ __forceinline__ bool arrive_last(unsigned* counter, unsigned expected, int* flag) {
  wait_stores();
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned old = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const bool last = old == expected - 1;
    if (last) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *flag = last;
  }
  __syncthreads();
  return *flag != 0;
}

// ---------------------------------------------------------------- LDS DMA
// s_waitcnt immediate that waits until at most n vector memory operations of
// the wave are outstanding (expcnt and lgkmcnt left free).
__host__ __device__ constexpr int vmcnt_imm(int n) {
  return 0x0F70 | (n & 15) | ((n >> 4) << 14);
}
// LDS byte address of a generic pointer into LDS: the shared aperture is
// 4 GiB aligned, so it is the pointer's low 32 bits (no address-space cast:
// the compiler's cast of a non-inlined generic pointer fails instruction
// selection in the persistent stage kernel).
__device__ __forceinline__ unsigned lds_u32(const void* p) { return (unsigned)(uintptr_t)p; }
// LDS DMA of 1 KiB per wave: lane l's 16 bytes at gp land at LDS byte
// address lds + 16 l (lds wave-uniform: read from the first lane).  Written
// as assembly so that the compiler adds no waits of its own for it (it would
// wait for the DMA before every later LDS read); callers wait (vmcnt) before
// the barrier that hands the data on.  The LDS address goes in as an M0
// operand (the compiler writes M0; the s_nop is the wait state before a DMA
// reads it).  Variants: default caching, streaming (nt: read once) and
// device-coherent (sc1: written earlier in the same launch).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(unsigned lds, const void* gp) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :: "{m0}"(__builtin_amdgcn_readfirstlane(lds)), "v"(gp) : "memory");
}
__device__ __forceinline__ void dma16_nt(unsigned lds, const void* gp) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %1, off nt"
               :: "{m0}"(__builtin_amdgcn_readfirstlane(lds)), "v"(gp) : "memory");
}
__device__ __forceinline__ void dma16_sc1(unsigned lds, const void* gp) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %1, off sc1"
               :: "{m0}"(__builtin_amdgcn_readfirstlane(lds)), "v"(gp) : "memory");
}
#pragma clang diagnostic pop

// ---------------------------------------------------------------- buffer resources
// Raw buffer accesses through a descriptor whose record count bounds the
// access: a load past the end returns zero, a store past the end is dropped.
typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, size_t bytes) {
  const int n = bytes > 0x7fffffffu ? 0x7fffffff : (int)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, 0x00020000);
}
// 16 bytes, device-coherent (sc1): data written by other workgroups of the
// same launch
__device__ __forceinline__ uint4 buf_ld_act(__amdgpu_buffer_rsrc_t r, int off) {
  const u32x4v v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 16);
  return make_uint4(v[0], v[1], v[2], v[3]);
}
// 16 bytes, streaming (nt): weights and caches read once
__device__ __forceinline__ uint4 buf_ld_stream(__amdgpu_buffer_rsrc_t r, int off) {
  const u32x4v v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 2);
  return make_uint4(v[0], v[1], v[2], v[3]);
}
// device-coherent 16 / 8-byte stores (sc1)
__device__ __forceinline__ void buf_st16(__amdgpu_buffer_rsrc_t r, int off, uint4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(u32x4v{v.x, v.y, v.z, v.w}, r, off, 0, 16);
}
__device__ __forceinline__ void buf_st8(__amdgpu_buffer_rsrc_t r, int off, uint32_t lo, uint32_t hi) {
  __builtin_amdgcn_raw_buffer_store_b64(u32x2v{lo, hi}, r, off, 0, 16);
}
__device__ __forceinline__ float buf_ld4_act(__amdgpu_buffer_rsrc_t r, int off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 16));
}
__device__ __forceinline__ void buf_st4(__amdgpu_buffer_rsrc_t r, int off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, off, 0, 16);
}
// Device-coherent 16 / 8-byte accesses through per-lane pointers, as relaxed
// agent-scope 64-bit atomics (global loads / stores with sc1).  A buffer
// descriptor must be wave-uniform, so the raw buffer forms above only serve
// accesses whose base is uniform.
__device__ __forceinline__ uint2 ld8c(const void* p) {
  const uint64_t v = __hip_atomic_load(reinterpret_cast<const uint64_t*>(p), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
  return make_uint2((uint32_t)v, (uint32_t)(v >> 32));
}
__device__ __forceinline__ uint4 ld16c(const void* p) {
  const uint2 a = ld8c(p);
  const uint2 b = ld8c(reinterpret_cast<const char*>(p) + 8);
  return make_uint4(a.x, a.y, b.x, b.y);
}
__device__ __forceinline__ void st8c(void* p, uint32_t lo, uint32_t hi) {
  __hip_atomic_store(reinterpret_cast<uint64_t*>(p), (uint64_t)lo | ((uint64_t)hi << 32),
                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st16c(void* p, uint4 v) {
  st8c(p, v.x, v.y);
  st8c(reinterpret_cast<char*>(p) + 8, v.z, v.w);
}

__device__ __forceinline__ uint4 pack8(const float* v) {
  return make_uint4(pack2(v[0], v[1]), pack2(v[2], v[3]), pack2(v[4], v[5]), pack2(v[6], v[7]));
}
__device__ __forceinline__ void unpack8(uint4 u, float* v) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

// ---------------------------------------------------------------- operand-order activations
// A small activation matrix X [M <= 64][K] (bf16) that a skinny MFMA GEMM
// reads as its row operand is stored in operand order: k-tile kt (32 columns)
// and row tile mt (16 rows) form one 1 KiB fragment at element
// ((kt * MT + mt) * 64 + lane) * 8, MT = ceil(M / 16), where lane
// r % 16 + 16 * ((c % 32) / 8) holds X[r][c .. c + 7] for c % 8 == 0.  A wave
// reads a fragment with one fully contiguous 16-byte load per lane (a
// row-major [M][K] matrix would need 16 rows x 64 bytes per load instead).
__host__ __device__ inline size_t fa_index(int r, int c, int MT) {
  return ((size_t)((c >> 5) * MT + (r >> 4)) * 64 + (r & 15) + 16 * ((c >> 3) & 3)) * 8 + (c & 7);
}
__host__ __device__ inline int mt_of(int M) { return (M + 15) >> 4; }

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// z sigmoid(z) with the hardware reciprocal (1 ulp) in place of an IEEE
// division: z -> -inf gives z * rcp(inf) = -0, z -> +inf gives z
__device__ __forceinline__ float silu(float z) { return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

// ---------------------------------------------------------------- packed weight fragments
//
// A weight matrix W [K x N] ([in, out], row-major) is stored as MFMA B-operand
// fragments.  Columns are taken in groups of 32 (two 16-column tiles); which
// logical columns form a group depends on the matrix (see col_of_group below).
// Fragment (group g, k-tile kt, tile i) holds W[32 kt + 8 (l/16) + e][col(g,i) + l%16]
// for lane l < 64, element e < 8, as 16 contiguous bytes at lane offset 16 l.
// Fragments are ordered [g][kt][i], 1 KiB each, so one wave reads one
// fragment with a single fully-coalesced 16-byte-per-lane load and the two
// tiles of a group over consecutive k-tiles are contiguous.
constexpr int kFragBytes = 1024;

__host__ __device__ inline size_t frag_offset(int g, int kt, int i, int KT) {
  return ((size_t)(g * KT + kt) * 2 + i) * kFragBytes;
}

// Column maps from a group index to the logical column of each of its tiles.
enum ColMap : int {
  kColPlain = 0,    // group g = columns [32g, 32g + 32)
  kColRopePairs = 1,// fused QKV: rotated heads pair column j with j + d/2 in one group
  kColGateUp = 2,   // fused gate/up: tile 0 = gate columns, tile 1 = up columns
};

struct ColMapArgs {
  int mode;
  int head_dim;   // kColRopePairs
  int n_rot;      // kColRopePairs: number of rotated columns ((Hq + Hkv) d)
  int half_n;     // kColGateUp: F (gate columns precede up columns)
};

// Logical column (in the concatenated source matrix) of tile i's first column.
__host__ __device__ inline int col_of_group(const ColMapArgs& m, int g, int i) {
  if (m.mode == kColRopePairs) {
    int gpr = m.head_dim / 32;            // groups per rotated head
    int n_rot_groups = m.n_rot / 32;
    if (g < n_rot_groups) {
      int head = g / gpr, t = g % gpr;
      return head * m.head_dim + 16 * t + i * (m.head_dim / 2);
    }
    return m.n_rot + 32 * (g - n_rot_groups) + 16 * i;
  }
  if (m.mode == kColGateUp) return i == 0 ? 16 * g : m.half_n + 16 * g;
  return 32 * g + 16 * i;
}

// An extra workgroup's share of the prefetch range: read (plain loads, so the
// lines allocate in the memory-side cache) and dropped.
__device__ inline void prefetch_range(const Prefetch& f, int i) {
  const size_t n16 = f.bytes / 16;
  const size_t per = (n16 + f.wgs - 1) / f.wgs;
  const size_t b0 = (size_t)i * per, b1 = min(n16, b0 + per);
  const uint4* p = reinterpret_cast<const uint4*>(f.p);
  unsigned x = 0;
  for (size_t j = b0 + threadIdx.x; j < b1; j += 256 * 8) {
    uint4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const size_t k = j + 256 * u;
      v[u] = k < b1 ? p[k] : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) x ^= v[u].x;
  }
  asm volatile("" ::"v"(x));
}

}  // namespace blk
