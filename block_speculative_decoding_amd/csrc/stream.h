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

// Statistics of one 4096-token chunk of one logits row, by a 256-thread block
// (each thread 16 consecutive elements, one pass): T > 0: (max, sum exp((x -
// max) / T)) with the sum accumulated in fp64; T == 0: (max, index of the first
// maximum, or -1 when the chunk holds only -inf).  Every thread gets the result.
// With `sub` (T > 0): sub[j] = the same sum over the chunk's 64-token sub-chunk
// j (j = 0..63, relative to the chunk max), the same per-token terms.
constexpr int kSubTok = 64;                          // tokens per sub-chunk
constexpr int kSubPerChunk = kChunk / kSubTok;       // 64
__device__ __forceinline__ double2 chunk_stat_block(const float* row, int V, int c, bool vec, float T,
                                                    float* redf /*4*/, double* redd /*4*/, double* sub = nullptr) {
  const int tid = threadIdx.x;
  const int e0 = c * kChunk + tid * kPer;
  float v[kPer];
  load_run(row, V, e0, vec, v);
  float mx = v[0];
#pragma unroll
  for (int e = 1; e < kPer; ++e) mx = fmaxf(mx, v[e]);
  mx = block_max<256>(mx, redf);
  if (T == 0.f) {
    int first = 0x7fffffff;
#pragma unroll
    for (int e = kPer - 1; e >= 0; --e)
      if (v[e] == mx && e0 + e < V) first = e0 + e;
    // block min of indices through the float max helper on negated values
    float nf = -(float)first;
    nf = block_max<256>(first == 0x7fffffff ? -INFINITY : nf, redf);
    return make_double2((double)mx, nf == -INFINITY ? -1.0 : -(double)nf);
  }
  const float k = kLog2e / T;
  double s = 0.0;
  if (mx != -INFINITY) {
#pragma unroll
    for (int e = 0; e < kPer; ++e) s += (double)exp2f((v[e] - mx) * k);
  }
  if (sub) {   // the 4 threads of a sub-chunk, in token order: (t0 + t1) + (t2 + t3)
    double g = s + __shfl_xor(s, 1, 64);
    g += __shfl_xor(g, 2, 64);
    if ((tid & 3) == 0) sub[tid >> 2] = g;
  }
  s = block_sum<256>(s, redd);
  return make_double2((double)mx, s);
}

// One inverse-CDF step by a wave over 64 consecutive masses w >= 0 (lane order =
// token order): the first lane whose running mass (from `base`) exceeds t, else
// the last lane with positive mass, else -1; *before = the running mass ahead
// of the returned lane.
__device__ __forceinline__ double wave_exclusive_scan_f64(double v) {
  const int lane = threadIdx.x & 63;
  double inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const double t = __shfl_up(inc, o, 64);
    if (lane >= o) inc += t;
  }
  return inc - v;
}
__device__ __forceinline__ int wave_min_int(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ int wave_max_int(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ int wave_select(double w, double base, double t, double* before) {
  const int lane = threadIdx.x & 63;
  const double run = base + wave_exclusive_scan_f64(w);
  const int f = wave_min_int(w > 0.0 && run + w > t ? lane : 64);
  const int l = wave_max_int(w > 0.0 ? lane : -1);
  const int pick = f < 64 ? f : l;
  *before = __shfl(run, pick < 0 ? 0 : pick, 64);
  return pick;
}

// Inverse-CDF draw of one row by one wave from its chunk statistics and
// sub-chunk sums (T > 0): chunk, then 64-token sub-chunk, then token.  st
// [nch] (max, sum) and sub [nch][64] as chunk_stat_block wrote them; the
// weight of a token is exp2((x - m_c) log2e / T) * exp((m_c - M) / T) (m_c its
// chunk max, M the row max) — the terms of its chunk's and sub-chunk's sums
// scaled by the chunk's factor.  t = u * total.  Returns the token (-1 when the
// row has no mass); *M_out, *tot_out = the row max and total.
constexpr int kDrawChunksPerLane = 16;               // nch <= 1024
__device__ __forceinline__ int wave_draw(const float* row, int V, const double2* st, const double* sub, int nch,
                                         float T, double u, double* M_out, double* tot_out) {
  const int lane = threadIdx.x & 63;
  const int per = (nch + 63) / 64, c0 = lane * per;
  double2 cs[kDrawChunksPerLane];
  float mx = -INFINITY;
#pragma unroll
  for (int k = 0; k < kDrawChunksPerLane; ++k) {
    cs[k] = (k < per && c0 + k < nch) ? st[c0 + k] : make_double2(-INFINITY, 0.0);
    mx = fmaxf(mx, (float)cs[k].x);
  }
  mx = wave_max(mx);
  const double invT = 1.0 / (double)T;
  double wk[kDrawChunksPerLane], wl = 0.0;
#pragma unroll
  for (int k = 0; k < kDrawChunksPerLane; ++k) {
    wk[k] = cs[k].x == -INFINITY ? 0.0 : cs[k].y * exp((cs[k].x - (double)mx) * invT);
    wl += wk[k];
  }
  const double tot = wave_sum(wl);
  *M_out = mx;
  *tot_out = tot;
  const double t = u * tot;
  double before;
  const int ln = wave_select(wl, 0.0, t, &before);
  if (ln < 0) return -1;
  // the chunk inside lane ln's run
  double run = before, fb = 0.0, lb = 0.0, fm = 0.0, lm = 0.0;
  int f = -1, l = -1;
#pragma unroll
  for (int k = 0; k < kDrawChunksPerLane; ++k) {
    const double w = __shfl(wk[k], ln, 64), m = __shfl(cs[k].x, ln, 64);
    if (f < 0 && w > 0.0 && run + w > t) {
      f = k;
      fb = run;
      fm = m;
    }
    if (w > 0.0) {
      l = k;
      lb = run;
      lm = m;
    }
    run += w;
  }
  const int cstar = ln * per + (f >= 0 ? f : l);
  before = f >= 0 ? fb : lb;
  const double mc = f >= 0 ? fm : lm;
  const double scale = exp((mc - (double)mx) * invT);
  // sub-chunk, then token
  const int js = wave_select(sub[(size_t)cstar * kSubPerChunk + lane] * scale, before, t, &before);
  if (js < 0) return -1;
  const int v = cstar * kChunk + js * kSubTok + lane;
  const float k2 = kLog2e / T;
  const float x = v < V ? row[v] : -INFINITY;
  const double w = x == -INFINITY ? 0.0 : (double)exp2f((x - (float)mc) * k2) * scale;
  const int tl = wave_select(w, before, t, &before);
  return tl < 0 ? -1 : cstar * kChunk + js * kSubTok + tl;
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
