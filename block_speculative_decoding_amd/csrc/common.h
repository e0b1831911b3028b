// Shared device helpers and host-side launch plumbing for the dfspec library
// (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

namespace dfs {

typedef uint16_t bf16_t;                                   // bf16 bit pattern
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// ----------------------------------------------------------------- global loads
// 16-byte load through an explicit global (address space 1) pointer.  A load
// through a generic pointer may compile to a flat load, which also counts in
// the LDS/scalar counter: every wait for an LDS read would then drain all
// outstanding HBM loads.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) const u32x4 global_u32x4;
__device__ __forceinline__ uint4 ldg16(const void* p) { return __builtin_bit_cast(uint4, *(global_u32x4*)p); }
typedef __attribute__((address_space(1))) const bf16x8 global_bf16x8;
__device__ __forceinline__ bf16x8 ldg_bf16x8(const void* p) { return *(global_bf16x8*)p; }

// ----------------------------------------------------------------- scalar conversions

__device__ __forceinline__ float bf2f(bf16_t v) { return __uint_as_float(((uint32_t)v) << 16); }

// round to nearest, ties to even (gfx950 converts in hardware: v_cvt_pk_bf16_f32);
// NaN stays NaN
__device__ __forceinline__ bf16_t f2bf(float f) { return __builtin_bit_cast(bf16_t, (__bf16)f); }

template <typename T> struct Elem;
template <> struct Elem<float> {
  __device__ static __forceinline__ float load(const float* p, size_t i) { return p[i]; }
  __device__ static __forceinline__ void store(float* p, size_t i, float v) { p[i] = v; }
};
template <> struct Elem<bf16_t> {
  __device__ static __forceinline__ float load(const bf16_t* p, size_t i) { return bf2f(p[i]); }
  __device__ static __forceinline__ void store(bf16_t* p, size_t i, float v) { p[i] = f2bf(v); }
};

// ----------------------------------------------------------------- wave / block reductions

template <typename V>
__device__ __forceinline__ V wave_sum(V v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

// Sum over a block of NT threads (NT a multiple of 64); every thread gets the result.
template <int NT, typename V>
__device__ __forceinline__ V block_sum(V v, V* smem /* NT/64 entries */) {
  v = wave_sum(v);
  const int w = threadIdx.x / kWave;
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) smem[w] = v;
  __syncthreads();
  V t = smem[0];
#pragma unroll
  for (int i = 1; i < NT / kWave; ++i) t += smem[i];
  return t;
}

template <int NT>
__device__ __forceinline__ float block_max(float v, float* smem) {
  v = wave_max(v);
  const int w = threadIdx.x / kWave;
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) smem[w] = v;
  __syncthreads();
  float t = smem[0];
#pragma unroll
  for (int i = 1; i < NT / kWave; ++i) t = fmaxf(t, smem[i]);
  return t;
}

__host__ __device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }
__host__ __device__ __forceinline__ size_t align_up(size_t a, size_t b) { return (a + b - 1) / b * b; }

// Tile-packed activation layout (bf16, K a multiple of 64): the rows in groups
// of 16, each group's K in 64-wide tiles of 2 KB, a tile stored as [half h =
// 0..1][lane l = 0..63][8 values] with lane l holding row 16 g + (l % 16),
// columns 64 t + 32 h + 8 (l / 16) .. +7 — the matrix-core operand fragment
// order, so a wave loads a 16-row x 32-column half tile as one contiguous
// kilobyte.  Four consecutive columns k .. k+3 (k % 4 == 0) are contiguous.
// A buffer holds ceil(rows / 16) whole groups.
__host__ __device__ __forceinline__ size_t xpk_index(int m, int k, int K) {
  return ((size_t)(m >> 4) * (K >> 6) + (k >> 6)) * 1024 + ((k >> 5) & 1) * 512 + ((m & 15) + 16 * ((k >> 3) & 3)) * 8 +
         (k & 7);
}

// ----------------------------------------------------------------- host plumbing

// Profiling hooks (events around launches of one kernel group); see profile.cpp.
void prof_before(const char* group, hipStream_t s);
void prof_after(const char* group, hipStream_t s);

struct ProfScope {
  const char* g;
  hipStream_t s;
  ProfScope(const char* group, hipStream_t st) : g(group), s(st) { prof_before(g, s); }
  ~ProfScope() { prof_after(g, s); }
};

// Bump allocator over a caller-provided workspace (host-side offsets only).
struct Carver {
  char* base;
  size_t off = 0;
  explicit Carver(void* b) : base((char*)b) {}
  template <typename T>
  T* take(size_t count) {
    off = align_up(off, 256);
    T* p = base ? (T*)(base + off) : nullptr;
    off += count * sizeof(T);
    return p;
  }
};

}  // namespace dfs
