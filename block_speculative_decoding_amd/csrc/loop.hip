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

}  // namespace

hipError_t launch_advance(int B, int G, const int32_t* n_accepted, const int32_t* out_tokens, int32_t* n_new,
                          int32_t* last_token, int64_t* tau_sum, hipStream_t s) {
  ProfScope ps("verify", s);
  hipLaunchKernelGGL(advance_kernel, dim3((unsigned)((B + 255) / 256)), dim3(256), 0, s, B, G, n_accepted,
                     out_tokens, n_new, last_token, tau_sum);
  return hipGetLastError();
}

}  // namespace dfs
