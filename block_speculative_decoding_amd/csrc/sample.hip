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

// One workgroup per row from the head GEMM's sub-chunk statistics (max_j,
// sum_j) of its 64-token sub-chunks: the row max M; each sub-chunk's mass sum_j
// * exp2((max_j - M) log2e/T) (an fp32 exponential, the mass in fp64), thread t
// owning the run of sub-chunks [t*per, (t+1)*per); the sub-chunk whose running
// mass crosses u * total (the thread by a block scan, then inside its run); then
// the token among its 64, one logit per lane of wave 0, weighted exp2((x -
// max_j) log2e/T) times the sub-chunk's factor — its term of the sub-chunk's
// sum.  T == 0: the lowest column holding the row max.
__global__ __launch_bounds__(kPickSubThreads) void pick_sub_kernel(PickArgs a, const double2* subst, int nsub) {
  constexpr int NW = kPickSubThreads / 64;
  __shared__ float redf[NW];
  __shared__ double redd[NW];
  __shared__ int redi[2];
  __shared__ double bc[1];
  const int r = blockIdx.x, tid = threadIdx.x, lane = tid & 63;
  const double2* st = subst + (size_t)r * nsub;
  const int per = ceil_div(nsub, kPickSubThreads), j0 = tid * per;
  double2 cs[kPickSubPer];
  float mx = -INFINITY;
#pragma unroll
  for (int k = 0; k < kPickSubPer; ++k) {
    cs[k] = (k < per && j0 + k < nsub) ? st[j0 + k] : make_double2(-INFINITY, -1.0);
    mx = fmaxf(mx, (float)cs[k].x);
  }
  mx = block_max<kPickSubThreads>(mx, redf);
  if (tid == 0) {
    redi[0] = 0x7fffffff;
    redi[1] = -1;
  }
  __syncthreads();
  int tok;
  double tot = 1.0;
  if (a.temperature == 0.f) {
    int best = 0x7fffffff;
#pragma unroll
    for (int k = 0; k < kPickSubPer; ++k)
      if ((float)cs[k].x == mx && cs[k].y >= 0) best = min(best, (int)cs[k].y);
    best = wave_min_int(best);
    if (lane == 0 && best != 0x7fffffff) atomicMin(&redi[0], best);
    __syncthreads();
    tok = redi[0] == 0x7fffffff ? 0 : redi[0];
  } else {
    const float k2 = kLog2e / a.temperature;
    double wk[kPickSubPer], wl = 0.0;
#pragma unroll
    for (int k = 0; k < kPickSubPer; ++k) {
      wk[k] = cs[k].x == -INFINITY ? 0.0 : cs[k].y * (double)exp2f(((float)cs[k].x - mx) * k2);
      wl += wk[k];
    }
    const double run0 = block_exclusive_scan<kPickSubThreads>(wl, redd, &tot);
    const double t = (double)a.u[(size_t)r * a.u_stride] * tot;
    // in this thread's run: the first sub-chunk crossing t, and the last with mass
    int jf = 0x7fffffff, jl = -1;
    double run = run0;
#pragma unroll
    for (int k = 0; k < kPickSubPer; ++k) {
      if (jf == 0x7fffffff && wk[k] > 0.0 && run + wk[k] > t) jf = j0 + k;
      if (wk[k] > 0.0) jl = j0 + k;
      run += wk[k];
    }
    jf = wave_min_int(jf);
    jl = wave_max_int(jl);
    if (lane == 0) {
      if (jf != 0x7fffffff) atomicMin(&redi[0], jf);
      if (jl >= 0) atomicMax(&redi[1], jl);
    }
    __syncthreads();
    const int js = redi[0] != 0x7fffffff ? redi[0] : redi[1];
    // the owner of sub-chunk js publishes the mass ahead of it
    if (js >= 0 && js >= j0 && js < j0 + per) {
      double before = run0;
#pragma unroll
      for (int k = 0; k < kPickSubPer; ++k)
        if (j0 + k < js) before += wk[k];
      bc[0] = before;
    }
    __syncthreads();
    tok = -1;
    if (js >= 0 && tid < 64) {
      double before = bc[0];
      const float mj = (float)st[js].x;
      const double scale = (double)exp2f((mj - mx) * k2);
      const int v = js * 64 + lane;
      const float x = v < a.V ? a.x[(size_t)r * a.row_stride + v] : -INFINITY;
      const double w = x == -INFINITY ? 0.0 : (double)exp2f((x - mj) * k2) * scale;
      const int tl = wave_select(w, before, t, &before);
      tok = tl < 0 ? -1 : js * 64 + tl;
    }
  }
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

hipError_t launch_pick_sub(const PickArgs& a, const double2* subst, int nsub, hipStream_t s) {
  if (a.rows <= 0) return hipSuccess;
  if (nsub > kPickSubMax) return hipErrorInvalidValue;
  hipLaunchKernelGGL(pick_sub_kernel, dim3(a.rows), dim3(kPickSubThreads), 0, s, a, subst, nsub);
  return hipGetLastError();
}

}  // namespace dfs
