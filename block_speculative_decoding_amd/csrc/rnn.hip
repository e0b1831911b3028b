// State update of the RNN sequential head (DSpark page, section "Innowacje w
// tworzeniu tokenów": an optional head that follows the whole block prefix; the
// page gives no structure, the cell is read as an Elman tanh cell):
//   h_i = tanh(U[prev_i] + A h_{i-1}),  h_0 = 0
// Grid (request, 64-element slice of the new state): wave w of a workgroup
// computes elements j = 64 * slice + 16 w .. +15.  The previous state goes to
// LDS; each lane covers k = 4 lane .. 4 lane + 3 (+ 256 t) of the dot products
// A[j, :] . h, all 16 rows' loads issued before any sum (one memory round
// trip per wave), then a wave-wide sum per row and lane 0 adds U[prev, j] and
// applies tanh.  The state stays fp32 and alternates between two buffers (every
// workgroup of a request reads the whole previous state).  For the bf16 output
// product the new state is also written as three bf16 terms hi + mid + lo
// (hi = bf16(h), mid = bf16(h - hi), lo = bf16(h - hi - mid)) whose sum carries
// h to about 2^-24 relative, side by side in one row of 3r values: one bf16
// matrix-core GEMM of K = 3r whose W column index wraps at r then gives W h at
// fp32 accuracy while streaming W once.
#include "kernels.h"

#include <math.h>

namespace dfs {
namespace {

template <typename T>
__global__ __launch_bounds__(256) void rnn_state_kernel(RnnArgs a) {
  constexpr int RW = 16;                                 // state elements per wave
  __shared__ float hs[kRnnMaxRank];
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = a.r;
  const float* hin = a.h_in + (size_t)b * r;
  for (int k = tid; k < r; k += 256) hs[k] = a.first ? 0.f : hin[k];
  __syncthreads();
  const int j0 = blockIdx.y * 64 + wave * RW;
  if (j0 >= r) return;                                   // uniform over the wave
  const T* A = (const T*)a.A;
  float acc[RW];
#pragma unroll
  for (int jj = 0; jj < RW; ++jj) acc[jj] = 0.f;
  if (!a.first) {
    for (int k0 = 4 * lane; k0 < r; k0 += 256) {
      float hk[4], av[RW][4];
#pragma unroll
      for (int e = 0; e < 4; ++e) hk[e] = k0 + e < r ? hs[k0 + e] : 0.f;
#pragma unroll
      for (int jj = 0; jj < RW; ++jj) {
        const size_t row = (size_t)min(j0 + jj, r - 1) * r;
#pragma unroll
        for (int e = 0; e < 4; ++e) av[jj][e] = k0 + e < r ? Elem<T>::load(A, row + k0 + e) : 0.f;
      }
#pragma unroll
      for (int jj = 0; jj < RW; ++jj)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[jj] = fmaf(av[jj][e], hk[e], acc[jj]);
    }
  }
  const int p = min(max(a.prev[(size_t)b * a.prev_stride], 0), a.V - 1);
  const T* U = (const T*)a.U + (size_t)p * r;
  float* hout = a.h_out + (size_t)b * r;
#pragma unroll
  for (int jj = 0; jj < RW; ++jj) {
    const float dot = wave_sum(acc[jj]);
    const int j = j0 + jj;
    if (lane == 0 && j < r) {
      const float hv = tanhf(Elem<T>::load(U, j) + dot);
      hout[j] = hv;
      if (a.split) {
        const bf16_t hi = f2bf(hv);
        const float r1 = hv - bf2f(hi);
        const bf16_t mid = f2bf(r1);
        const bf16_t lo = f2bf(r1 - bf2f(mid));
        bf16_t* row = a.split + (size_t)b * 3 * r + j;   // [b][term][j]
        row[0] = hi;
        row[r] = mid;
        row[2 * r] = lo;
      }
    }
  }
}

}  // namespace

hipError_t launch_rnn_state(const RnnArgs& a, int dtype, hipStream_t s) {
  ProfScope ps("markov", s);
  if (a.r < 1 || a.r > kRnnMaxRank || a.B < 1) return hipErrorInvalidValue;
  const dim3 grid(a.B, ceil_div(a.r, 64));
  if (dtype == 1) hipLaunchKernelGGL(rnn_state_kernel<bf16_t>, grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL(rnn_state_kernel<float>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace dfs
