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
//   2. decide: one wave per batch row walks i = 1..G, forming p(d_i) and q(d_i)
//      in fp64 from the row statistics, and stops at the first rejection
//   3. fp64 exp-sums of the target and draft rows at each rejection (only B rows)
//   4. residual mass max(0, p - q) per chunk, with p and q normalised by (3)
//      (fp64 throughout: p - q cancels when the two are close)
//   5. final draw per row: residual (or p at the rejection when the residual has
//      no mass), or the bonus token from p_{G+1}
// Greedy (T == 0) finishes in step 2.
#include "stream.h"

namespace dfs {
namespace {

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

__global__ __launch_bounds__(64) void decide_kernel(VerifyArgs a, int nch) {
  const int b = blockIdx.x, lane = threadIdx.x;
  const int G = a.G, V = a.V;
  const double T = a.temperature;
  int acc_end = G;
  double info[4] = {0, 0, 0, 0};
  for (int i = 0; i < G; ++i) {
    const double2* pst = a.p_chunk + ((size_t)b * (G + 1) + i) * nch;
    const int d = a.drafts[(size_t)b * G + i];
    bool accept;
    if (a.temperature == 0.f) {
      const int arg = argmax_chunks_wave(pst, nch);
      accept = d == arg;
      if (!accept && lane == 0) a.out_tokens[(size_t)b * (G + 1) + i] = arg;
    } else {
      double Mp, Sp, Mq, Sq;
      combine_chunks_wave(pst, nch, T, &Mp, &Sp);
      if (a.q_stats) {
        Mq = a.q_stats[((size_t)b * G + i) * 2];
        Sq = a.q_stats[((size_t)b * G + i) * 2 + 1];
      } else {
        combine_chunks_wave(a.q_chunk + ((size_t)b * G + i) * nch, nch, T, &Mq, &Sq);
      }
      double r = 0.0;
      if (d >= 0 && d < V) {
        const double xp = a.p[((size_t)b * (G + 1) + i) * V + d];
        const double xq = a.q[((size_t)b * G + i) * V + d];
        const double pd = xp == -INFINITY ? 0.0 : exp((xp - Mp) / T) / Sp;
        const double qd = xq == -INFINITY ? 0.0 : exp((xq - Mq) / T) / Sq;
        r = qd > 0.0 ? pd / qd : (pd > 0.0 ? INFINITY : 0.0);
      }
      accept = (double)a.u_accept[(size_t)b * G + i] < r;
      info[0] = Mp;
      info[1] = Sp;
      info[2] = Mq;
      info[3] = Sq;
    }
    if (accept) {
      if (lane == 0) a.out_tokens[(size_t)b * (G + 1) + i] = d;
    } else {
      acc_end = i;
      break;
    }
  }
  if (acc_end == G) {
    const double2* pst = a.p_chunk + ((size_t)b * (G + 1) + G) * nch;
    if (a.temperature == 0.f) {
      const int arg = argmax_chunks_wave(pst, nch);
      if (lane == 0) a.out_tokens[(size_t)b * (G + 1) + G] = arg;
    } else {
      combine_chunks_wave(pst, nch, T, &info[0], &info[1]);
    }
  }
  if (lane == 0) {
    a.state[b] = acc_end;
    a.n_accepted[b] = acc_end;
    for (int j = acc_end + 1; j <= G; ++j) a.out_tokens[(size_t)b * (G + 1) + j] = -1;
#pragma unroll
    for (int k = 0; k < 4; ++k) a.rowinfo[b * 4 + k] = info[k];
  }
}

// fp64 exp-sums over one chunk of the target and draft rows at the rejection
__global__ __launch_bounds__(256) void reject_sums_kernel(VerifyArgs a, int nch) {
  __shared__ double red[4];
  const int c = blockIdx.x % nch, b = blockIdx.x / nch, tid = threadIdx.x;
  const int i = a.state[b];
  if (i >= a.G) return;
  const double T = a.temperature;
  const double Mp = a.rowinfo[b * 4], Mq = a.rowinfo[b * 4 + 2];
  const float* prow = a.p + ((size_t)b * (a.G + 1) + i) * a.V;
  const float* qrow = a.q + ((size_t)b * a.G + i) * a.V;
  double sp = 0.0, sq = 0.0;
  const int e0 = c * kChunk + tid * kPer;
  for (int e = e0; e < min(e0 + kPer, a.V); ++e) {
    const float xp = prow[e], xq = qrow[e];
    if (xp != -INFINITY) sp += exp(((double)xp - Mp) / T);
    if (xq != -INFINITY) sq += exp(((double)xq - Mq) / T);
  }
  sp = block_sum<256>(sp, red);
  sq = block_sum<256>(sq, red);
  if (tid == 0) a.sums[(size_t)b * nch + c] = make_double2(sp, sq);
}

struct ResidualWeight {
  const float* prow;
  const float* qrow;
  double Mp, Mq, Sp, Sq, T;
  __device__ double operator()(int e) const {
    const float xp = prow[e], xq = qrow[e];
    const double p = xp == -INFINITY ? 0.0 : exp(((double)xp - Mp) / T) / Sp;
    const double q = xq == -INFINITY ? 0.0 : exp(((double)xq - Mq) / T) / Sq;
    return p > q ? p - q : 0.0;
  }
};

__device__ __forceinline__ void row_sums(const VerifyArgs& a, int b, int nch, double* Sp, double* Sq) {
  double sp = 0.0, sq = 0.0;
  for (int c = 0; c < nch; ++c) {
    sp += a.sums[(size_t)b * nch + c].x;
    sq += a.sums[(size_t)b * nch + c].y;
  }
  *Sp = sp;
  *Sq = sq;
}

__global__ __launch_bounds__(256) void residual_kernel(VerifyArgs a, int nch) {
  __shared__ double red[4];
  const int c = blockIdx.x % nch, b = blockIdx.x / nch, tid = threadIdx.x;
  const int i = a.state[b];
  if (i >= a.G) return;
  ResidualWeight w;
  w.prow = a.p + ((size_t)b * (a.G + 1) + i) * a.V;
  w.qrow = a.q + ((size_t)b * a.G + i) * a.V;
  w.Mp = a.rowinfo[b * 4];
  w.Mq = a.rowinfo[b * 4 + 2];
  w.T = a.temperature;
  row_sums(a, b, nch, &w.Sp, &w.Sq);
  double s = 0.0;
  const int e0 = c * kChunk + tid * kPer;
  for (int e = e0; e < min(e0 + kPer, a.V); ++e) s += w(e);
  s = block_sum<256>(s, red);
  if (tid == 0) a.r_chunk[(size_t)b * nch + c] = s;
}

struct TargetWeight {
  const float* row;
  float M, k;
  __device__ double operator()(int e) const {
    const float x = row[e];
    return x == -INFINITY ? 0.0 : (double)exp2f((x - M) * k);
  }
};

__global__ __launch_bounds__(256) void final_kernel(VerifyArgs a, int nch) {
  __shared__ double red[4];
  __shared__ int smi[2];
  __shared__ double before_sh;
  __shared__ int c_sh, use_resid_sh;
  __shared__ double t_sh;
  const int b = blockIdx.x, tid = threadIdx.x;
  const int G = a.G;
  const int i = a.state[b];
  const double T = a.temperature;
  const double u = a.u_final[b];
  if (tid == 0) {
    // residual mass per chunk, or target row i (bonus: row G) chunk masses
    double W = 0.0;
    if (i < G)
      for (int c = 0; c < nch; ++c) W += a.r_chunk[(size_t)b * nch + c];
    const bool use_resid = i < G && W > 0.0;
    const double2* pst = a.p_chunk + ((size_t)b * (G + 1) + i) * nch;
    double Mp = -INFINITY;
    if (!use_resid) {
      for (int c = 0; c < nch; ++c) Mp = fmax(Mp, pst[c].x);
      W = 0.0;
      for (int c = 0; c < nch; ++c)
        if (pst[c].x != -INFINITY) W += pst[c].y * exp((pst[c].x - Mp) / T);
    }
    const double t = u * W;
    double before = 0.0, before_last = 0.0;
    int cstar = -1, lastpos = -1;
    for (int c = 0; c < nch; ++c) {
      const double w = use_resid ? a.r_chunk[(size_t)b * nch + c]
                                 : (pst[c].x == -INFINITY ? 0.0 : pst[c].y * exp((pst[c].x - Mp) / T));
      if (w > 0) {
        lastpos = c;
        before_last = before;
      }
      if (before + w > t) {
        cstar = c;
        break;
      }
      before += w;
    }
    if (cstar < 0) {
      cstar = lastpos < 0 ? 0 : lastpos;
      before = before_last;
    }
    c_sh = cstar;
    before_sh = before;
    use_resid_sh = use_resid;
    t_sh = t;
    if (!use_resid) a.rowinfo[b * 4] = Mp;    // exact row max for the target-row draw
  }
  __syncthreads();
  int tok;
  if (use_resid_sh) {
    ResidualWeight w;
    w.prow = a.p + ((size_t)b * (G + 1) + i) * a.V;
    w.qrow = a.q + ((size_t)b * G + i) * a.V;
    w.Mp = a.rowinfo[b * 4];
    w.Mq = a.rowinfo[b * 4 + 2];
    w.T = T;
    row_sums(a, b, nch, &w.Sp, &w.Sq);
    tok = chunk_search(c_sh, a.V, before_sh, t_sh, w, red, smi);
  } else {
    TargetWeight w;
    w.row = a.p + ((size_t)b * (G + 1) + i) * a.V;
    w.M = (float)a.rowinfo[b * 4];
    w.k = kLog2e / a.temperature;
    tok = chunk_search(c_sh, a.V, before_sh, t_sh, w, red, smi);
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
  hipLaunchKernelGGL(decide_kernel, dim3(a.B), dim3(64), 0, s, a, nch);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (a.temperature == 0.f) return hipSuccess;
  hipLaunchKernelGGL(reject_sums_kernel, dim3(nch * a.B), dim3(256), 0, s, a, nch);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(residual_kernel, dim3(nch * a.B), dim3(256), 0, s, a, nch);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(final_kernel, dim3(a.B), dim3(256), 0, s, a, nch);
  return hipGetLastError();
}

}  // namespace dfs
