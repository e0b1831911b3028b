// Vocabulary-streaming kernels: chunked row statistics and inverse-CDF / argmax
// picks (DSpark page, section "Innowacje w tworzeniu tokenów": each position is
// sampled after the head's bias is added; the draw itself is plain inverse-CDF
// sampling with a supplied uniform).
//
// A row of V logits is cut into 4096-element chunks.  Pass 1 (one workgroup per
// (row, chunk), coalesced 16-byte loads, each logit read once) produces per
// chunk the local max and sum exp((x - max)/T) accumulated in fp64.  The pick
// (one workgroup per row) merges the chunk statistics, finds the chunk whose
// running mass crosses u * total, and re-reads only that chunk to locate the
// token (block-wide fp64 prefix sum over per-thread runs of 16 consecutive ids,
// so the scan follows increasing token id exactly).  Per row the pick reads
// one chunk: total traffic ~ one pass over the logits.
#include "stream.h"

namespace dfs {
namespace {

__global__ __launch_bounds__(256) void chunk_stats_kernel(const float* x, long row_stride, int V, float T,
                                                          double2* stats, int nch, bool vec) {
  __shared__ float redf[4];
  __shared__ double redd[4];
  const int c = blockIdx.x % nch, r = blockIdx.x / nch, tid = threadIdx.x;   // 1-D grid: rows may exceed 65535
  const float* row = x + (size_t)r * row_stride;
  const int e0 = c * kChunk + tid * kPer;
  float v[kPer];
  load_run(row, V, e0, vec, v);
  float mx = v[0];
#pragma unroll
  for (int e = 1; e < kPer; ++e) mx = fmaxf(mx, v[e]);
  mx = block_max<256>(mx, redf);
  double2 out;
  if (T == 0.f) {
    int first = 0x7fffffff;
#pragma unroll
    for (int e = kPer - 1; e >= 0; --e)
      if (v[e] == mx && e0 + e < V) first = e0 + e;
    // block min of indices through the float max helper on negated values
    float nf = -(float)first;
    nf = block_max<256>(first == 0x7fffffff ? -INFINITY : nf, redf);
    out = make_double2((double)mx, nf == -INFINITY ? -1.0 : -(double)nf);
  } else {
    const float k = kLog2e / T;
    double s = 0.0;
    if (mx != -INFINITY) {
#pragma unroll
      for (int e = 0; e < kPer; ++e) s += (double)exp2f((v[e] - mx) * k);
    }
    s = block_sum<256>(s, redd);
    out = make_double2((double)mx, s);
  }
  if (tid == 0) stats[(size_t)r * nch + c] = out;
}

// One wave per row (no workgroup barriers on the draw's critical path): merge
// the chunk statistics, draw with u, write the token and the row's (max, sum).
// Lane l owns chunks [l*per, l*per + per) (per = ceil(nch/64) <= 16), so a
// wave-wide exclusive scan of the lanes' masses gives every chunk's running
// mass in chunk order; the chosen chunk's 4096 logits are then rescanned with
// lane l owning elements 64 l .. 64 l + 63, again in token order.
constexpr int kPickPer = 16;                  // chunks per lane: nch <= 1024 (V <= 4M)
constexpr int kPickRun = kChunk / kWave;      // 64 consecutive elements per lane in the rescan

__device__ __forceinline__ double wave_exclusive_scan(double v) {
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

__global__ __launch_bounds__(64) void pick_kernel(PickArgs a, int nch, bool vec) {
  const int r = blockIdx.x, lane = threadIdx.x;
  const double2* st = a.stats + (size_t)r * nch;
  const float* row = a.x + (size_t)r * a.row_stride;
  const int per = (nch + 63) / 64, c0 = lane * per;
  double2 cs[kPickPer];
#pragma unroll
  for (int k = 0; k < kPickPer; ++k)
    cs[k] = (k < per && c0 + k < nch) ? st[c0 + k] : make_double2(-INFINITY, -1.0);
  float mx = -INFINITY;
#pragma unroll
  for (int k = 0; k < kPickPer; ++k) mx = fmaxf(mx, (float)cs[k].x);
  mx = wave_max(mx);
  if (a.temperature == 0.f) {
    // lowest index among the chunks holding the max
    int best = 0x7fffffff;
#pragma unroll
    for (int k = 0; k < kPickPer; ++k)
      if ((float)cs[k].x == mx && cs[k].y >= 0) best = min(best, (int)cs[k].y);
    best = wave_min_int(best);
    if (lane == 0) {
      a.tokens[(size_t)r * a.tok_stride] = best == 0x7fffffff ? 0 : best;
      if (a.row_stats) {
        a.row_stats[(size_t)r * a.rs_stride] = mx;
        a.row_stats[(size_t)r * a.rs_stride + 1] = 1.0;
      }
    }
    return;
  }
  const double T = a.temperature;
  // chunk masses relative to the row max, each computed once
  double w[kPickPer];
  double loc = 0.0;
#pragma unroll
  for (int k = 0; k < kPickPer; ++k) {
    const double m = cs[k].x;
    w[k] = m == -INFINITY ? 0.0 : cs[k].y * exp((m - (double)mx) / T);
    loc += w[k];
  }
  const double tot = wave_sum(loc);
  const double t = (double)a.u[(size_t)r * a.u_stride] * tot;
  // first chunk whose running mass exceeds t, else the last chunk with mass, else chunk 0
  double run = wave_exclusive_scan(loc);
  int found = 0x7fffffff, last = -1;
  double found_before = 0.0, last_before = 0.0;
#pragma unroll
  for (int k = 0; k < kPickPer; ++k) {
    if (found == 0x7fffffff && w[k] > 0.0 && run + w[k] > t) {
      found = c0 + k;
      found_before = run;
    }
    if (w[k] > 0.0) {
      last = c0 + k;
      last_before = run;
    }
    run += w[k];
  }
  const int f = wave_min_int(found), l = wave_max_int(last);
  const int cstar = f != 0x7fffffff ? f : (l >= 0 ? l : 0);
  // the owner lane publishes the mass ahead of the chosen chunk
  const int owner = min(cstar / per, 63);
  const double before = __shfl(f != 0x7fffffff ? found_before : last_before, owner, 64) *
                        (f != 0x7fffffff || l >= 0 ? 1.0 : 0.0);
  // rescan the chosen chunk in token order
  const float k2 = kLog2e / a.temperature;
  const int e0 = cstar * kChunk + lane * kPickRun;
  float v[kPickRun];
  if (vec && e0 + kPickRun <= a.V) {
#pragma unroll
    for (int q = 0; q < kPickRun / 4; ++q) {
      const float4 x4 = *(const float4*)(row + e0 + 4 * q);
      v[4 * q] = x4.x;
      v[4 * q + 1] = x4.y;
      v[4 * q + 2] = x4.z;
      v[4 * q + 3] = x4.w;
    }
  } else {
#pragma unroll
    for (int e = 0; e < kPickRun; ++e) v[e] = e0 + e < a.V ? row[e0 + e] : -INFINITY;
  }
  const float fmx = mx;
  double eloc = 0.0;
#pragma unroll
  for (int e = 0; e < kPickRun; ++e) eloc += v[e] == -INFINITY ? 0.0 : (double)exp2f((v[e] - fmx) * k2);
  double erun = before + wave_exclusive_scan(eloc);
  int tf = 0x7fffffff, tl = -1;
#pragma unroll
  for (int e = 0; e < kPickRun; ++e) {
    const double we = v[e] == -INFINITY ? 0.0 : (double)exp2f((v[e] - fmx) * k2);
    erun += we;
    if (tf == 0x7fffffff && erun > t) tf = e0 + e;
    if (we > 0.0) tl = e0 + e;
  }
  tf = wave_min_int(tf);
  tl = wave_max_int(tl);
  if (lane == 0) {
    const int tok = tf != 0x7fffffff ? tf : tl;
    a.tokens[(size_t)r * a.tok_stride] = tok < 0 ? 0 : tok;
    if (a.row_stats) {
      a.row_stats[(size_t)r * a.rs_stride] = mx;
      a.row_stats[(size_t)r * a.rs_stride + 1] = tot;
    }
  }
}

}  // namespace

hipError_t launch_chunk_stats(const float* x, long row_stride, int rows, int V, float temperature,
                              double2* stats, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  const int nch = ceil_div(V, kChunk);
  const bool vec = (row_stride % 4 == 0) && (((uintptr_t)x & 15) == 0);
  hipLaunchKernelGGL(chunk_stats_kernel, dim3(nch * rows), dim3(256), 0, s, x, row_stride, V, temperature,
                     stats, nch, vec);
  return hipGetLastError();
}

hipError_t launch_pick(const PickArgs& a, hipStream_t s) {
  if (a.rows <= 0) return hipSuccess;
  const int nch = ceil_div(a.V, kChunk);
  const bool vec = (a.row_stride % 4 == 0) && (((uintptr_t)a.x & 15) == 0);
  if (nch > 64 * kPickPer) return hipErrorInvalidValue;
  hipLaunchKernelGGL(pick_kernel, dim3(a.rows), dim3(64), 0, s, a, nch, vec);
  return hipGetLastError();
}

}  // namespace dfs
