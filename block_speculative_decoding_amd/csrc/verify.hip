// Rejection-sampling verification (DSpark page, section "Jak działa
// spekulatywne dekodowanie DSpark?": the longest valid prefix is kept and one
// more token appended, preserving the target distribution exactly).  The rule
// is the standard speculative-sampling one: accept d_i while
// u_i < p_i(d_i) / q_i(d_i); at the first rejection draw from
// normalise(max(0, p - q)); after a fully accepted block draw a bonus token
// from the next target distribution.
//
// Launch sequence (all on the caller's stream):
//   1. chunk statistics of every target row (and of the draft rows when the
//      sampler's row statistics are not supplied)            — streams [B, G+1, V]
//   2. decide: one workgroup per batch row, one wave per position, forms
//      p_i(d_i) and q_i(d_i) in fp64 for every position at once and keeps the
//      prefix up to the first rejection
//   3. fp64 exp-sums of the target and draft rows at each rejection (only B rows)
//   4. residual mass max(0, p - q) per chunk, with p and q normalised by (3)
//      (fp64 throughout: p - q cancels when the two are close)
//   5. final draw per row: residual (or p at the rejection when the residual has
//      no mass), or the bonus token from p_{G+1}
// Greedy (T == 0) finishes in step 2.
// A row may verify only its first k drafts (n_verify, the prefix scheduler's
// early stopping): the first rejection among them, else the bonus token from
// target row k — the same rule on a shorter draft, so still lossless.
#include "stream.h"

namespace dfs {
namespace {

// drafts verified in row b
__device__ __forceinline__ int verify_len(const VerifyArgs& a, int b) {
  return a.n_verify ? min(max(a.n_verify[b], 0), a.G) : a.G;
}

__device__ __forceinline__ void combine_chunks_wave(const double2* st, int nch, double T, double* M, double* S) {
  const int lane = threadIdx.x & 63;
  float mx = -INFINITY;
  for (int c = lane; c < nch; c += 64) mx = fmaxf(mx, (float)st[c].x);
  mx = wave_max(mx);
  double s = 0.0;
  for (int c = lane; c < nch; c += 64)
    if (st[c].x != -INFINITY) s += st[c].y * exp((st[c].x - (double)mx) / T);
  s = wave_sum(s);
  *M = mx;
  *S = s;
}

__device__ __forceinline__ int argmax_chunks_wave(const double2* st, int nch) {
  const int lane = threadIdx.x & 63;
  float mx = -INFINITY;
  for (int c = lane; c < nch; c += 64) mx = fmaxf(mx, (float)st[c].x);
  mx = wave_max(mx);
  float best = -INFINITY;
  for (int c = lane; c < nch; c += 64)
    if ((float)st[c].x == mx && st[c].y >= 0) best = fmaxf(best, -(float)st[c].y);
  best = wave_max(best);
  return best == -INFINITY ? 0 : (int)(-best);
}

// One workgroup (16 waves) per batch row; wave w takes positions w, w+16, ...
// (position G is the bonus row).  Per position: the target row's exact (max,
// sum) from its chunk statistics, the draft row's from the sampler (or its
// chunks), p(d) / q(d) in fp64, and the accept test; then the prefix.
constexpr int kDecideWaves = 16;
__global__ __launch_bounds__(1024) void decide_kernel(VerifyArgs a, int nch) {
  __shared__ int acc_sh[65];
  __shared__ double info_sh[65][4];
  __shared__ int arg_sh[65];
  const int b = blockIdx.x, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int G = a.G, V = a.V;
  const double T = a.temperature;
  for (int i = wave; i <= G; i += kDecideWaves) {
    const double2* pst = a.p_chunk + ((size_t)b * (G + 1) + i) * nch;
    if (a.temperature == 0.f) {
      const int arg = argmax_chunks_wave(pst, nch);
      if (lane == 0) {
        arg_sh[i] = arg;
        acc_sh[i] = i < G && a.drafts[(size_t)b * G + i] == arg;
      }
      continue;
    }
    double Mp, Sp, Mq = 0.0, Sq = 0.0;
    combine_chunks_wave(pst, nch, T, &Mp, &Sp);
    bool accept = false;
    if (i < G) {
      if (a.q_stats) {
        Mq = a.q_stats[((size_t)b * G + i) * 2];
        Sq = a.q_stats[((size_t)b * G + i) * 2 + 1];
      } else {
        combine_chunks_wave(a.q_chunk + ((size_t)b * G + i) * nch, nch, T, &Mq, &Sq);
      }
      const int d = a.drafts[(size_t)b * G + i];
      double r = 0.0;
      if (d >= 0 && d < V) {
        const double xp = a.p[((size_t)b * (G + 1) + i) * V + d];
        const double xq = a.q[((size_t)b * G + i) * V + d];
        const double pd = xp == -INFINITY ? 0.0 : exp((xp - Mp) / T) / Sp;
        const double qd = xq == -INFINITY ? 0.0 : exp((xq - Mq) / T) / Sq;
        r = qd > 0.0 ? pd / qd : (pd > 0.0 ? INFINITY : 0.0);
      }
      accept = (double)a.u_accept[(size_t)b * G + i] < r;
    }
    if (lane == 0) {
      acc_sh[i] = accept;
      info_sh[i][0] = Mp;
      info_sh[i][1] = Sp;
      info_sh[i][2] = Mq;
      info_sh[i][3] = Sq;
    }
  }
  __syncthreads();
  if (threadIdx.x != 0) return;
  const int kb = verify_len(a, b);
  int acc_end = kb;
  for (int i = 0; i < kb; ++i)
    if (!acc_sh[i]) {
      acc_end = i;
      break;
    }
  int32_t* out = a.out_tokens + (size_t)b * (G + 1);
  for (int i = 0; i < acc_end; ++i) out[i] = a.drafts[(size_t)b * G + i];
  if (a.temperature == 0.f) out[acc_end] = arg_sh[acc_end];   // correction or bonus: the target argmax
  for (int j = acc_end + 1; j <= G; ++j) out[j] = -1;
  a.state[b] = acc_end;
  a.n_accepted[b] = acc_end;
  if (a.temperature != 0.f)
    for (int k = 0; k < 4; ++k) a.rowinfo[b * 4 + k] = info_sh[acc_end][k];
}

// fp64 exp-sums over one chunk of the target and draft rows at the rejection
__global__ __launch_bounds__(256) void reject_sums_kernel(VerifyArgs a, int nch, bool vec) {
  __shared__ double red[4];
  const int c = blockIdx.x % nch, b = blockIdx.x / nch, tid = threadIdx.x;
  const int i = a.state[b];
  if (i >= verify_len(a, b)) return;
  const double T = a.temperature;
  const double Mp = a.rowinfo[b * 4], Mq = a.rowinfo[b * 4 + 2];
  const float* prow = a.p + ((size_t)b * (a.G + 1) + i) * a.V;
  const float* qrow = a.q + ((size_t)b * a.G + i) * a.V;
  const int e0 = c * kChunk + tid * kPer;
  float vp[kPer], vq[kPer];
  load_run(prow, a.V, e0, vec, vp);                  // -inf past V: no mass
  load_run(qrow, a.V, e0, vec, vq);
  const double invT = 1.0 / T;
  double sp = 0.0, sq = 0.0;
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    if (vp[e] != -INFINITY) sp += exp(((double)vp[e] - Mp) * invT);
    if (vq[e] != -INFINITY) sq += exp(((double)vq[e] - Mq) * invT);
  }
  sp = block_sum<256>(sp, red);
  sq = block_sum<256>(sq, red);
  if (tid == 0) a.sums[(size_t)b * nch + c] = make_double2(sp, sq);
}

// max(0, p - q) with p, q normalised in fp64, for the 16 elements e0 .. e0+15
__device__ __forceinline__ void residual16(const float* prow, const float* qrow, int V, int e0, bool vec, double Mp,
                                           double Mq, double Sp, double Sq, double T, double* w) {
  float vp[kPer], vq[kPer];
  load_run(prow, V, e0, vec, vp);
  load_run(qrow, V, e0, vec, vq);
  const double invT = 1.0 / T, invSp = 1.0 / Sp, invSq = 1.0 / Sq;
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    const double p = vp[e] == -INFINITY ? 0.0 : exp(((double)vp[e] - Mp) * invT) * invSp;
    const double q = vq[e] == -INFINITY ? 0.0 : exp(((double)vq[e] - Mq) * invT) * invSq;
    w[e] = p > q ? p - q : 0.0;
  }
}

// row totals (Sp, Sq) of the rejected position: block sum of the chunk sums
__device__ __forceinline__ void row_sums(const VerifyArgs& a, int b, int nch, double* Sp, double* Sq, double* red) {
  double sp = 0.0, sq = 0.0;
  for (int c = threadIdx.x; c < nch; c += 256) {
    sp += a.sums[(size_t)b * nch + c].x;
    sq += a.sums[(size_t)b * nch + c].y;
  }
  *Sp = block_sum<256>(sp, red);
  *Sq = block_sum<256>(sq, red);
}

__global__ __launch_bounds__(256) void residual_kernel(VerifyArgs a, int nch, bool vec) {
  __shared__ double red[4];
  const int c = blockIdx.x % nch, b = blockIdx.x / nch, tid = threadIdx.x;
  const int i = a.state[b];
  if (i >= verify_len(a, b)) return;
  double Sp, Sq;
  row_sums(a, b, nch, &Sp, &Sq, red);
  double w[kPer];
  residual16(a.p + ((size_t)b * (a.G + 1) + i) * a.V, a.q + ((size_t)b * a.G + i) * a.V, a.V,
             c * kChunk + tid * kPer, vec, a.rowinfo[b * 4], a.rowinfo[b * 4 + 2], Sp, Sq, a.temperature, w);
  double s = 0.0;
#pragma unroll
  for (int e = 0; e < kPer; ++e) s += w[e];
  s = block_sum<256>(s, red);
  if (tid == 0) a.r_chunk[(size_t)b * nch + c] = s;
}

// The one draw of a row: from the residual at the rejection (from p there when
// the residual has no mass), or the bonus token from p_{G+1}.
__global__ __launch_bounds__(256) void final_kernel(VerifyArgs a, int nch, bool vec) {
  __shared__ double red[4];
  __shared__ float redf[4];
  __shared__ int smi[2];
  const int b = blockIdx.x, tid = threadIdx.x;
  const int G = a.G;
  const int i = a.state[b];
  const double T = a.temperature;
  const double u = a.u_final[b];
  const double2* pst = a.p_chunk + ((size_t)b * (G + 1) + i) * nch;
  const bool rejected = i < verify_len(a, b);       // else: bonus token from target row i
  double W = 0.0;
  if (rejected) {
    for (int c = tid; c < nch; c += 256) W += a.r_chunk[(size_t)b * nch + c];
    W = block_sum<256>(W, red);
  }
  const bool use_resid = rejected && W > 0.0;
  float Mp = -INFINITY;
  if (!use_resid) {                                  // target row i (bonus: the row after the verified drafts)
    for (int c = tid; c < nch; c += 256) Mp = fmaxf(Mp, (float)pst[c].x);
    Mp = block_max<256>(Mp, redf);
    W = 0.0;
    for (int c = tid; c < nch; c += 256)
      if (pst[c].x != -INFINITY) W += pst[c].y * exp((pst[c].x - (double)Mp) / T);
    W = block_sum<256>(W, red);
  }
  const double t = u * W;
  double before;
  const int cstar = select_chunk(
      nch, t,
      [&](int c) -> double {
        if (use_resid) return a.r_chunk[(size_t)b * nch + c];
        return pst[c].x == -INFINITY ? 0.0 : pst[c].y * exp((pst[c].x - (double)Mp) / T);
      },
      &before, red, smi);
  const float* prow = a.p + ((size_t)b * (G + 1) + i) * a.V;
  int tok;
  if (use_resid) {
    double Sp, Sq;
    row_sums(a, b, nch, &Sp, &Sq, red);
    const float* qrow = a.q + ((size_t)b * G + i) * a.V;
    const double Mpr = a.rowinfo[b * 4], Mq = a.rowinfo[b * 4 + 2];
    tok = chunk_search(
        cstar, a.V, before, t,
        [&](int e0, double* w) { residual16(prow, qrow, a.V, e0, vec, Mpr, Mq, Sp, Sq, T, w); }, red, smi);
  } else {
    const float k = kLog2e / a.temperature;
    tok = chunk_search(
        cstar, a.V, before, t,
        [&](int e0, double* w) {
          float v[kPer];
          load_run(prow, a.V, e0, vec, v);
#pragma unroll
          for (int e = 0; e < kPer; ++e) w[e] = v[e] == -INFINITY ? 0.0 : (double)exp2f((v[e] - Mp) * k);
        },
        red, smi);
  }
  if (tid == 0) a.out_tokens[(size_t)b * (G + 1) + i] = tok < 0 ? 0 : tok;
}

}  // namespace

hipError_t launch_verify(const VerifyArgs& a, hipStream_t s) {
  ProfScope ps("verify", s);
  const int nch = ceil_div(a.V, kChunk);
  hipError_t e = launch_chunk_stats(a.p, a.V, a.B * (a.G + 1), a.V, a.temperature,
                                    const_cast<double2*>(a.p_chunk), s);
  if (e != hipSuccess) return e;
  if (!a.q_stats && a.temperature != 0.f) {
    e = launch_chunk_stats(a.q, a.V, a.B * a.G, a.V, a.temperature, const_cast<double2*>(a.q_chunk), s);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(decide_kernel, dim3(a.B), dim3(64 * kDecideWaves), 0, s, a, nch);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (a.temperature == 0.f) return hipSuccess;
  const bool vec = (a.V & 3) == 0 && ((uintptr_t)a.p & 15) == 0 && ((uintptr_t)a.q & 15) == 0;
  hipLaunchKernelGGL(reject_sums_kernel, dim3(nch * a.B), dim3(256), 0, s, a, nch, vec);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(residual_kernel, dim3(nch * a.B), dim3(256), 0, s, a, nch, vec);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(final_kernel, dim3(a.B), dim3(256), 0, s, a, nch, vec);
  return hipGetLastError();
}

}  // namespace dfs
