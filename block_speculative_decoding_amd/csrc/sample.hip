// Vocabulary-streaming kernels: chunked row statistics and inverse-CDF / argmax
// picks (DSpark page, section "Innowacje w tworzeniu tokenów": each position is
// sampled after the head's bias is added; the draw itself is plain inverse-CDF
// sampling with a supplied uniform).
//
// A row of V logits is cut into 4096-token chunks.  Pass 1 (one workgroup per
// (row, chunk), coalesced 16-byte loads, each logit read once) produces per
// chunk the local max and sum exp((x - max)/T) accumulated in fp64, and the
// same sum over each 64-token sub-chunk.  The pick (one wave per row) merges
// the chunk statistics, finds the chunk whose running mass crosses u * total,
// then the sub-chunk inside it, then reads that sub-chunk's 64 logits (one per
// lane) to locate the token: three short dependent steps, scans in increasing
// token id.  Per row the pick reads 64 logits: total traffic ~ one pass over
// the logits.
#include "stream.h"

namespace dfs {
namespace {

__global__ __launch_bounds__(256) void chunk_stats_kernel(const float* x, long row_stride, int V, float T,
                                                          double2* stats, double* sub, int nch, bool vec) {
  __shared__ float redf[4];
  __shared__ double redd[4];
  const int c = blockIdx.x % nch, r = blockIdx.x / nch;   // 1-D grid: rows may exceed 65535
  const double2 out = chunk_stat_block(x + (size_t)r * row_stride, V, c, vec, T, redf, redd,
                                       sub && T != 0.f ? sub + ((size_t)r * nch + c) * kSubPerChunk : nullptr);
  if (threadIdx.x == 0) stats[(size_t)r * nch + c] = out;
}

// One wave per row (no workgroup barriers on the draw's critical path): the
// draw (T > 0: chunk, sub-chunk, token) or the argmax (T == 0), then the token
// and the row's (max, sum).
__global__ __launch_bounds__(64) void pick_kernel(PickArgs a, int nch) {
  const int r = blockIdx.x, lane = threadIdx.x;
  const double2* st = a.stats + (size_t)r * nch;
  if (a.temperature == 0.f) {
    // lowest index among the chunks holding the max
    const int per = (nch + 63) / 64, c0 = lane * per;
    float mx = -INFINITY;
    for (int k = 0; k < per && c0 + k < nch; ++k) mx = fmaxf(mx, (float)st[c0 + k].x);
    mx = wave_max(mx);
    int best = 0x7fffffff;
    for (int k = 0; k < per && c0 + k < nch; ++k)
      if ((float)st[c0 + k].x == mx && st[c0 + k].y >= 0) best = min(best, (int)st[c0 + k].y);
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
  double M, tot;
  const int tok = wave_draw(a.x + (size_t)r * a.row_stride, a.V, st, a.sub + (size_t)r * nch * kSubPerChunk, nch,
                            a.temperature, (double)a.u[(size_t)r * a.u_stride], &M, &tot);
  if (lane == 0) {
    a.tokens[(size_t)r * a.tok_stride] = tok < 0 ? 0 : tok;
    if (a.row_stats) {
      a.row_stats[(size_t)r * a.rs_stride] = M;
      a.row_stats[(size_t)r * a.rs_stride + 1] = tot;
    }
  }
}

}  // namespace

hipError_t launch_chunk_stats(const float* x, long row_stride, int rows, int V, float temperature,
                              double2* stats, double* sub, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  const int nch = ceil_div(V, kChunk);
  const bool vec = (row_stride % 4 == 0) && (((uintptr_t)x & 15) == 0);
  hipLaunchKernelGGL(chunk_stats_kernel, dim3(nch * rows), dim3(256), 0, s, x, row_stride, V, temperature,
                     stats, sub, nch, vec);
  return hipGetLastError();
}

hipError_t launch_pick(const PickArgs& a, hipStream_t s) {
  if (a.rows <= 0) return hipSuccess;
  const int nch = ceil_div(a.V, kChunk);
  if (nch > 64 * kDrawChunksPerLane) return hipErrorInvalidValue;
  hipLaunchKernelGGL(pick_kernel, dim3(a.rows), dim3(64), 0, s, a, nch);
  return hipGetLastError();
}

}  // namespace dfs
