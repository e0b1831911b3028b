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
constexpr int kPickSubThreads = 512;                 // one row pick from sub-chunk statistics
constexpr int kPickSubPer = kPickSubMax / kPickSubThreads;   // sub-chunks per thread
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

// exclusive prefix sum over the NT threads of a block (fp64)
template <int NT = 256>
__device__ __forceinline__ double block_exclusive_scan(double v, double* smem /*NT/64*/, double* total) {
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
  double off = 0.0, tot = 0.0;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) {
    if (i < w) off += smem[i];
    tot += smem[i];
  }
  *total = tot;
  return off + inc - v;
}

}  // namespace dfs
