// Device-side bookkeeping between two cycles of the draft -> sample -> verify
// loop (DSpark page, section "Jak działa spekulatywne dekodowanie DSpark?": a
// cycle commits the longest valid prefix of the drafts plus one token; the
// DFlash latency paragraph counts tau as the accepted length including that
// token).  It turns spec_verify's outputs into the next dflash_draft_step's
// inputs on the device, so a chain of cycles needs no host synchronisation and
// can be captured into one HIP graph.
#include "kernels.h"

namespace dfs {
namespace {

// One thread per batch row.
__global__ __launch_bounds__(256) void advance_kernel(int B, int G, const int32_t* __restrict__ n_accepted,
                                                      const int32_t* __restrict__ out_tokens,
                                                      int32_t* __restrict__ n_new, int32_t* __restrict__ last_token,
                                                      int64_t* __restrict__ tau_sum) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  const int a = min(max(n_accepted[b], 0), G);        // accepted drafts this cycle
  n_new[b] = a + 1;                                    // committed rows the next call appends
  last_token[b] = out_tokens[(size_t)b * (G + 1) + a]; // the correction or bonus token
  if (tau_sum) tau_sum[b] += a + 1;
}

// ------------------------------------------------------------------ prefix scheduler
// Verify length per request (DSpark page, section "Optymalizacja weryfikacji i
// wydajności"; DeepSeek-V4.1 notes page, section "DSpark — le décodage
// spéculatif"): maximise SPS(N) * sum_b (1 + sum_{j < k_b} P[b, j]), P the
// prefix survival products of the per-position survival scores and N =
// sum_b (k_b + 1) the rows verified.  P does not increase along a request, so
// the optimum for M verified drafts takes the M largest P (ties: lower index
// first, which keeps every request's choice a prefix): sort, then scan M.  One
// workgroup; the running sum over the sorted values is taken by one thread in
// order (so the argmax — an integer decision — does not depend on a parallel
// summation order), the objective of every M is then evaluated in parallel and
// reduced to its first maximum.
constexpr int kSchedMax = 8192;

__device__ __forceinline__ bool sched_before(double va, int ka, double vb, int kb) {
  return va > vb || (va == vb && ka < kb);
}

__device__ double sched_sps(const SchedArgs& a, double n) {
  if (n <= (double)a.xs[0]) return a.ys[0];
  if (n >= (double)a.xs[a.ncurve - 1]) return a.ys[a.ncurve - 1];
  int i = 0;                                             // xs[i] <= n < xs[i+1]
  while ((double)a.xs[i + 1] <= n) ++i;
  const double x0 = a.xs[i], x1 = a.xs[i + 1], y0 = a.ys[i], y1 = a.ys[i + 1];
  return y0 + (y1 - y0) * ((n - x0) / (x1 - x0));
}

__global__ __launch_bounds__(1024) void schedule_kernel(SchedArgs a) {
  __shared__ double val[kSchedMax];
  __shared__ int key[kSchedMax];
  __shared__ int cnt[kSchedMax];
  __shared__ double red_v[16];
  __shared__ int red_m[16];
  const int tid = threadIdx.x, B = a.B, G = a.G, n = B * G;
  int np2 = 1;
  while (np2 < n) np2 <<= 1;
  for (int b = tid; b < B; b += 1024) {                  // prefix survival products, fp64
    double P = 1.0;
    for (int j = 0; j < G; ++j) {
      const float c = a.surv[(size_t)b * G + j];
      const double cc = c >= 0.f ? (c <= 1.f ? (double)c : 1.0) : 0.0;   // NaN -> 0
      P = P * cc;
      val[b * G + j] = P;
      key[b * G + j] = b * G + j;
    }
    cnt[b] = 0;
  }
  for (int i = n + tid; i < np2; i += 1024) {
    val[i] = -1.0;
    key[i] = 0x7fffffff;
  }
  __syncthreads();
  // bitonic sort into (value descending, index ascending)
  for (int k = 2; k <= np2; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = tid; i < np2; i += 1024) {
        const int ixj = i ^ j;
        if (ixj > i) {
          const bool up = (i & k) == 0;
          const bool swap = up ? sched_before(val[ixj], key[ixj], val[i], key[i])
                               : sched_before(val[i], key[i], val[ixj], key[ixj]);
          if (swap) {
            const double tv = val[i];
            val[i] = val[ixj];
            val[ixj] = tv;
            const int tk = key[i];
            key[i] = key[ixj];
            key[ixj] = tk;
          }
        }
      }
      __syncthreads();
    }
  }
  if (tid == 0) {                                        // running sums in place: val[m-1] = sum of the top m
    double acc = 0.0;
    for (int m = 0; m < n; ++m) {
      acc = acc + val[m];
      val[m] = acc;
    }
  }
  __syncthreads();
  // objective of every M = 0 .. n; first maximum (larger value, else smaller M)
  double bv = -1.0;
  int bmi = 0x7fffffff;
  for (int m = tid; m <= n; m += 1024) {
    const double o = sched_sps(a, (double)(B + m)) * ((double)B + (m > 0 ? val[m - 1] : 0.0));
    if (o > bv) {
      bv = o;
      bmi = m;
    }
  }
  for (int off = 32; off > 0; off >>= 1) {
    const double ov = __shfl_xor(bv, off, 64);
    const int om = __shfl_xor(bmi, off, 64);
    if (ov > bv || (ov == bv && om < bmi)) {
      bv = ov;
      bmi = om;
    }
  }
  if ((tid & 63) == 0) {
    red_v[tid >> 6] = bv;
    red_m[tid >> 6] = bmi;
  }
  __syncthreads();
  double best = red_v[0];
  int best_m = red_m[0];
  for (int w = 1; w < 16; ++w)
    if (red_v[w] > best || (red_v[w] == best && red_m[w] < best_m)) {
      best = red_v[w];
      best_m = red_m[w];
    }
  for (int r = tid; r < best_m; r += 1024) atomicAdd(&cnt[key[r] / G], 1);
  __syncthreads();
  for (int b = tid; b < B; b += 1024) a.n_verify[b] = cnt[b];
}

}  // namespace

hipError_t launch_schedule(const SchedArgs& a, hipStream_t s) {
  ProfScope ps("verify", s);
  if (a.B * a.G > kSchedMax || a.ncurve < 1 || a.ncurve > kSchedCurve) return hipErrorInvalidValue;
  hipLaunchKernelGGL(schedule_kernel, dim3(1), dim3(1024), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_advance(int B, int G, const int32_t* n_accepted, const int32_t* out_tokens, int32_t* n_new,
                          int32_t* last_token, int64_t* tau_sum, hipStream_t s) {
  ProfScope ps("verify", s);
  hipLaunchKernelGGL(advance_kernel, dim3((unsigned)((B + 255) / 256)), dim3(256), 0, s, B, G, n_accepted,
                     out_tokens, n_new, last_token, tau_sum);
  return hipGetLastError();
}

}  // namespace dfs
