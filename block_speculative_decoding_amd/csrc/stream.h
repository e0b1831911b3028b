// Helpers shared by the vocabulary-streaming kernels (sampling and verify).
#pragma once

#include "kernels.h"

#include <math.h>

namespace dfs {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kPer = kChunk / 256;   // 16 consecutive elements per thread

__device__ __forceinline__ void load_run(const float* row, int V, int e0, bool vec, float* v) {
  if (vec && e0 + kPer <= V) {
#pragma unroll
    for (int q = 0; q < kPer / 4; ++q) {
      const float4 t = *(const float4*)(row + e0 + 4 * q);
      v[4 * q] = t.x;
      v[4 * q + 1] = t.y;
      v[4 * q + 2] = t.z;
      v[4 * q + 3] = t.w;
    }
  } else {
#pragma unroll
    for (int e = 0; e < kPer; ++e) v[e] = e0 + e < V ? row[e0 + e] : -INFINITY;
  }
}

// exclusive prefix sum over the 256 threads of a block (fp64)
__device__ __forceinline__ double block_exclusive_scan(double v, double* smem /*4*/, double* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  double inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const double t = __shfl_up(inc, o, 64);
    if (lane >= o) inc += t;
  }
  __syncthreads();
  if (lane == 63) smem[w] = inc;
  __syncthreads();
  double off = 0.0;
  for (int i = 0; i < w; ++i) off += smem[i];
  *total = smem[0] + smem[1] + smem[2] + smem[3];
  return off + inc - v;
}

// Inverse-CDF over chunks, by the whole block: chunk c (c < nch) has mass
// weight(c) >= 0; finds the first chunk whose running mass (chunks in order)
// exceeds t, else the last chunk with positive mass (rounding), else chunk 0.
// Returns the chunk and, in *before, the mass of the chunks ahead of it.  One
// thread per chunk (a thread takes consecutive chunks when nch > 256) and an
// fp64 block scan, instead of one thread walking every chunk.
template <typename ChunkWeight>
__device__ __forceinline__ int select_chunk(int nch, double t, ChunkWeight weight, double* before, double* smem,
                                            int* smemi) {
  const int tid = threadIdx.x;
  const int per = (nch + 255) / 256, c0 = tid * per;
  double w[4];                                   // per <= 4: nch <= 1024 chunks (V <= 4M)
  double loc = 0.0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    w[k] = (k < per && c0 + k < nch) ? weight(c0 + k) : 0.0;
    loc += w[k];
  }
  double total;
  double run = block_exclusive_scan(loc, smem, &total);
  int found = 0x7fffffff, last = -1;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    if (found == 0x7fffffff && w[k] > 0.0 && run + w[k] > t) found = c0 + k;
    if (w[k] > 0.0) last = c0 + k;
    run += w[k];
  }
  __syncthreads();
  if (tid == 0) {
    smemi[0] = 0x7fffffff;
    smemi[1] = -1;
  }
  __syncthreads();
  if (found != 0x7fffffff) atomicMin(&smemi[0], found);
  if (last >= 0) atomicMax(&smemi[1], last);
  __syncthreads();
  const int pick = smemi[0] != 0x7fffffff ? smemi[0] : (smemi[1] >= 0 ? smemi[1] : 0);
  // the owner of the picked chunk publishes its prefix mass
  __syncthreads();
  if (pick >= c0 && pick < c0 + per) {
    double r = 0.0;
    for (int k = 0; k < 4; ++k)
      if (k < per && c0 + k < pick) r += w[k];
    smem[0] = run - loc + r;   // exclusive prefix of this thread + its chunks before `pick`
  }
  __syncthreads();
  *before = smem[0];
  __syncthreads();
  return pick;
}

// Locate the token of an inverse-CDF draw inside one chunk (pick and verify).
// weights16(e0, w) fills the unnormalised weights (>= 0, 0 past V) of the 16
// consecutive elements e0 .. e0+15 a thread owns; `before` is the mass of all
// earlier chunks and `t` the threshold.  Returns the first element whose running
// sum exceeds t, else the last element of the chunk with positive weight
// (rounding), else -1.
template <typename Weights16>
__device__ __forceinline__ int chunk_search(int c, int V, double before, double t, Weights16 weights16, double* smem,
                                            int* smemi) {
  const int tid = threadIdx.x;
  const int e0 = c * kChunk + tid * kPer;
  double w[kPer];
  weights16(e0, w);
  double loc = 0.0;
#pragma unroll
  for (int e = 0; e < kPer; ++e) loc += w[e];
  double total;
  double run = before + block_exclusive_scan(loc, smem, &total);
  int found = 0x7fffffff, last_pos = -1;
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    run += w[e];
    if (found == 0x7fffffff && run > t) found = e0 + e;
    if (w[e] > 0.0) last_pos = e0 + e;
  }
  __syncthreads();
  if (tid == 0) {
    smemi[0] = 0x7fffffff;
    smemi[1] = -1;
  }
  __syncthreads();
  if (found != 0x7fffffff) atomicMin(&smemi[0], found);
  if (last_pos >= 0) atomicMax(&smemi[1], last_pos);
  __syncthreads();
  return smemi[0] != 0x7fffffff ? smemi[0] : smemi[1];
}

}  // namespace dfs
