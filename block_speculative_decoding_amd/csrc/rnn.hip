// State update of the RNN sequential head (DSpark page, section "Innowacje w
// tworzeniu tokenów": an optional head that follows the whole block prefix; the
// page gives no structure, the cell is read as an Elman tanh cell):
//   h_i = tanh(U[prev_i] + A h_{i-1}),  h_0 = 0
// One workgroup per request: the previous state goes to LDS, each wave takes
// state elements j in turn and forms the dot product A[j, :] . h with its
// lanes over k (coalesced reads of A's row j), a wave-wide sum, then lane 0
// adds U[prev, j] and applies tanh.  The state stays fp32.  For the bf16
// output product it is also written as three bf16 terms hi + mid + lo
// (hi = bf16(h), mid = bf16(h - hi), lo = bf16(h - hi - mid)) whose sum
// carries h to about 2^-24 relative: three bf16 matrix-core passes over W then
// give W h at fp32 accuracy.
#include "kernels.h"

#include <math.h>

namespace dfs {
namespace {

template <typename T>
__global__ __launch_bounds__(256) void rnn_state_kernel(RnnArgs a) {
  __shared__ float hs[kRnnMaxRank];
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = a.r;
  float* h = a.h + (size_t)b * r;
  for (int k = tid; k < r; k += 256) hs[k] = a.first ? 0.f : h[k];
  __syncthreads();
  const int p = min(max(a.prev[(size_t)b * a.prev_stride], 0), a.V - 1);
  const T* U = (const T*)a.U + (size_t)p * r;
  const T* A = (const T*)a.A;
  for (int j = wave; j < r; j += 4) {
    float acc = 0.f;
    for (int k = lane; k < r; k += 64) acc = fmaf(Elem<T>::load(A, (size_t)j * r + k), hs[k], acc);
    acc = wave_sum(acc);
    if (lane == 0) {
      const float hv = tanhf(Elem<T>::load(U, j) + acc);
      h[j] = hv;
      if (a.split) {
        const bf16_t hi = f2bf(hv);
        const float r1 = hv - bf2f(hi);
        const bf16_t mid = f2bf(r1);
        const bf16_t lo = f2bf(r1 - bf2f(mid));
        const size_t o = (size_t)b * r + j, plane = (size_t)a.B * r;
        a.split[o] = hi;
        a.split[plane + o] = mid;
        a.split[2 * plane + o] = lo;
      }
    }
  }
}

}  // namespace

hipError_t launch_rnn_state(const RnnArgs& a, int dtype, hipStream_t s) {
  ProfScope ps("markov", s);
  if (a.r < 1 || a.r > kRnnMaxRank || a.B < 1) return hipErrorInvalidValue;
  if (dtype == 1) hipLaunchKernelGGL(rnn_state_kernel<bf16_t>, dim3(a.B), dim3(256), 0, s, a);
  else hipLaunchKernelGGL(rnn_state_kernel<float>, dim3(a.B), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace dfs
