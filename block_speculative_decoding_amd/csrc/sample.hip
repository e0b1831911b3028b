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

// One workgroup per row: merge chunk statistics, draw with u, write token and (max, sum).
__global__ __launch_bounds__(256) void pick_kernel(PickArgs a, int nch, bool vec) {
  __shared__ double redd[4];
  __shared__ float redf[4];
  __shared__ int smi[2];
  const int r = blockIdx.x, tid = threadIdx.x;
  const double2* st = a.stats + (size_t)r * nch;
  const float* row = a.x + (size_t)r * a.row_stride;
  float mx = -INFINITY;
  for (int c = tid; c < nch; c += 256) mx = fmaxf(mx, (float)st[c].x);
  mx = block_max<256>(mx, redf);
  if (a.temperature == 0.f) {
    float best = -INFINITY;   // lowest index among chunks holding the max (negated for max-reduction)
    for (int c = tid; c < nch; c += 256)
      if ((float)st[c].x == mx && st[c].y >= 0) best = fmaxf(best, -(float)st[c].y);
    best = block_max<256>(best, redf);
    if (tid == 0) {
      a.tokens[(size_t)r * a.tok_stride] = best == -INFINITY ? 0 : (int)(-best);
      if (a.row_stats) {
        a.row_stats[(size_t)r * a.rs_stride] = mx;
        a.row_stats[(size_t)r * a.rs_stride + 1] = 1.0;
      }
    }
    return;
  }
  const double T = a.temperature;
  // chunk masses relative to the row max
  double tot = 0.0;
  for (int c = tid; c < nch; c += 256) {
    const double m = st[c].x;
    if (m != -INFINITY) tot += st[c].y * exp((m - (double)mx) / T);
  }
  tot = block_sum<256>(tot, redd);
  const double u = a.u[(size_t)r * a.u_stride];
  const double t = u * tot;
  double before;
  const int cstar = select_chunk(
      nch, t,
      [&](int c) -> double {
        const double m = st[c].x;
        return m == -INFINITY ? 0.0 : st[c].y * exp((m - (double)mx) / T);
      },
      &before, redd, smi);
  const float k = kLog2e / a.temperature;
  const float fmx = mx;
  const int tok = chunk_search(
      cstar, a.V, before, t,
      [&](int e0, double* w) {
        float v[kPer];
        load_run(row, a.V, e0, vec, v);
#pragma unroll
        for (int e = 0; e < kPer; ++e) w[e] = v[e] == -INFINITY ? 0.0 : (double)exp2f((v[e] - fmx) * k);
      },
      redd, smi);
  if (tid == 0) {
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
  hipLaunchKernelGGL(pick_kernel, dim3(a.rows), dim3(256), 0, s, a, nch, vec);
  return hipGetLastError();
}

}  // namespace dfs
