// Rejection-sampling verification (DSpark page, section "Jak działa
// spekulatywne dekodowanie DSpark?": the longest valid prefix is kept and one
// more token appended, preserving the target distribution exactly).  The rule
// is the standard speculative-sampling one: accept d_i while
// u_i < p_i(d_i) / q_i(d_i); at the first rejection draw from
// normalise(max(0, p - q)); after a fully accepted block draw a bonus token
// from the next target distribution.
//
// Three launches on the caller's stream (T > 0):
//   1. statistics pass: per 4096-token chunk of every target row (and of every
//      draft row when the sampler's row statistics are not supplied) the chunk
//      max and sum exp((x - max)/T), and for the target rows the same sum per
//      64-token sub-chunk.  The one full read of the target logits.
//   2. resolve: 512-thread workgroups, each owning some chunks of one batch
//      row (one chunk each at small batches, several at large ones).  Every
//      workgroup of a row first takes the row's accept/reject decisions from
//      the chunk statistics (the same computation in each, so all agree on the
//      first rejected position a), then works on its own chunks of the rejected
//      target and draft rows in fp64: the exact sums of ep = exp((x_p - max)/T)
//      and eq = exp((x_q - max)/T), and per 64-token sub-chunk the sums of ep
//      and eq over the tokens where p > q under the statistics pass's
//      normalisers (the set P0 below).
//   3. draw: one wave per batch row.  Exact normalisers from the chunk sums,
//      then the inverse-CDF descent chunk -> sub-chunk -> token over the
//      residual masses (three short dependent reads, no full-chunk rescan); or
//      the bonus token from the target row after an accepted block (or from p_a
//      when the residual has no mass), by the same descent over the statistics
//      pass's chunk and sub-chunk sums of that row.
// Greedy (T == 0) decides from the argmax statistics in one second launch.
// A row may verify only its first k drafts (n_verify, the prefix scheduler's
// early stopping): the first rejection among them, else the bonus token from
// target row k — the same rule on a shorter draft, so still lossless.
//
// The residual masses: with p_v = a ep_v and q_v = b eq_v (ep, eq the exact
// fp64 weights, a = 1/Sp, b = 1/Sq exact), the mass of a range of tokens over
// the set P0 = {v : a0 ep_v > b0 eq_v} chosen with the statistics pass's
// normalisers (a0, b0; fp32 exponentials, ~1e-7 relative) is linear in (a, b):
// sum_{v in P0} (a ep_v - b eq_v) = a P - b Q, P and Q the sums of ep and eq
// over P0.  It equals the range's sum max(0, p - q) except for tokens whose p
// and q agree to ~1e-7 relative (which change side between the two
// normalisations; their residual is ~1e-7 of their mass); identical p and q
// rows give exactly zero.  The token-level step weighs the same P0.
#include "stream.h"

namespace dfs {
namespace {

// drafts verified in row b
__device__ __forceinline__ int verify_len(const VerifyArgs& a, int b) {
  return a.n_verify ? min(max(a.n_verify[b], 0), a.G) : a.G;
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

// Row (max, sum) from its chunk statistics, by a group of 16 lanes (lane `sub`
// takes chunks sub, sub + 16, ...): the float max over the group first, then
// each lane's sum of s_c exp((m_c - max)/T) and an fp64 sum over the group
// (fixed order).  Every lane of the group gets the result.
__device__ __forceinline__ void merge_group16(const double2* st, int nch, double invT, int sub, double* M, double* S) {
  float m = -INFINITY;
  for (int c = sub; c < nch; c += 16) m = fmaxf(m, (float)st[c].x);
#pragma unroll
  for (int o = 8; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  double s = 0.0;
  if (m != -INFINITY)
    for (int c = sub; c < nch; c += 16) {
      const double2 x = st[c];
      if (x.x != -INFINITY) s += x.y * exp((x.x - (double)m) * invT);
    }
#pragma unroll
  for (int o = 8; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);
  *M = m;
  *S = s;
}

// Accept/reject decisions of batch row b (T > 0) by a whole workgroup: 16 lanes
// per position, blockDim/16 positions at a time, each position's loads (its
// chunk statistics, the draft token and the two logits at it) issued together.
// Fills acc[i] and info[i] = (Mp, Sp, Mq, Sq) for i < kb; returns the first
// rejected position (kb when every verified draft is accepted).
__device__ __forceinline__ int decide_block(const VerifyArgs& a, int b, int kb, int nch, int* acc, double (*info)[4],
                                            int* first_sh) {
  const int tid = threadIdx.x, grp = tid >> 4, sub = tid & 15;
  const double invT = 1.0 / a.temperature;
  for (int i0 = 0; i0 < kb; i0 += (int)(blockDim.x >> 4)) {
    const int i = i0 + grp;
    if (i < kb) {                                          // uniform over the 16-lane group
      const int d = a.drafts[(size_t)b * a.G + i];
      const bool dv = d >= 0 && d < a.V;
      const double xp = dv ? (double)a.p[((size_t)b * (a.G + 1) + i) * a.V + d] : 0.0;
      const double xq = dv ? (double)a.q[((size_t)b * a.G + i) * a.V + d] : 0.0;
      double Mp, Sp, Mq, Sq;
      merge_group16(a.p_chunk + ((size_t)b * (a.G + 1) + i) * nch, nch, invT, sub, &Mp, &Sp);
      if (a.q_stats) {
        Mq = a.q_stats[((size_t)b * a.G + i) * 2];
        Sq = a.q_stats[((size_t)b * a.G + i) * 2 + 1];
      } else {
        merge_group16(a.q_chunk + ((size_t)b * a.G + i) * nch, nch, invT, sub, &Mq, &Sq);
      }
      double r = 0.0;
      if (dv) {
        const double pd = xp == -INFINITY ? 0.0 : exp((xp - Mp) * invT) / Sp;
        const double qd = xq == -INFINITY ? 0.0 : exp((xq - Mq) * invT) / Sq;
        r = qd > 0.0 ? pd / qd : (pd > 0.0 ? INFINITY : 0.0);
      }
      if (sub == 0) {
        acc[i] = (double)a.u_accept[(size_t)b * a.G + i] < r;
        info[i][0] = Mp;
        info[i][1] = Sp;
        info[i][2] = Mq;
        info[i][3] = Sq;
      }
    }
  }
  __syncthreads();
  if (tid == 0) {
    int e = kb;
    for (int i = 0; i < kb; ++i)
      if (!acc[i]) {
        e = i;
        break;
      }
    *first_sh = e;
  }
  __syncthreads();
  return *first_sh;
}

// Launch 1: chunk statistics of the p rows (then the q rows).
__global__ __launch_bounds__(256) void stats_kernel(VerifyArgs a, int nch, int p_rows, bool vec_p, bool vec_q) {
  __shared__ float redf[4];
  __shared__ double redd[4];
  const int c = blockIdx.x % nch, r = blockIdx.x / nch;
  const bool is_p = r < p_rows;
  const float* row = is_p ? a.p + (size_t)r * a.V : a.q + (size_t)(r - p_rows) * a.V;
  const double2 st =
      chunk_stat_block(row, a.V, c, is_p ? vec_p : vec_q, a.temperature, redf, redd,
                       is_p && a.temperature != 0.f ? a.p_sub + ((size_t)r * nch + c) * kSubPerChunk : nullptr);
  if (threadIdx.x == 0) {
    if (is_p) a.p_chunk[(size_t)r * nch + c] = st;
    else a.q_chunk[(size_t)(r - p_rows) * nch + c] = st;
  }
}

// Launch 2 (T > 0): 512-thread workgroups, nblk per batch row b, workgroup k
// owning chunks k, k + nblk, ...; in chunk c thread t owns tokens c*4096 + 8t ..
// +7, and each 8 consecutive threads one 64-token sub-chunk.
constexpr int kResThreads = 512;
constexpr int kResPer = kChunk / kResThreads;        // 8 tokens per thread
constexpr int kSubThreads = kSubTok / kResPer;       // threads per sub-chunk

__global__ __launch_bounds__(512) void resolve_kernel(VerifyArgs a, int nch, int nblk, bool vec) {
  __shared__ double4 red4[kResThreads / 64];
  __shared__ int acc_sh[64];
  __shared__ double info_sh[64][4];
  __shared__ int first_sh;
  const int b = blockIdx.x / nblk, c0 = blockIdx.x % nblk, tid = threadIdx.x;
  const int G = a.G, V = a.V;
  const double invT = 1.0 / a.temperature;
  const int kb = verify_len(a, b);
  float vp[kResPer], vq[kResPer];
  auto load_chunk = [&](int pos, int c) {
    const int e0 = c * kChunk + tid * kResPer;
    const float* pr = a.p + ((size_t)b * (G + 1) + pos) * V;
    const float* qr = a.q + ((size_t)b * G + pos) * V;
    if (vec && e0 + kResPer <= V) {
#pragma unroll
      for (int h = 0; h < kResPer / 4; ++h) {
        const float4 x = *(const float4*)(pr + e0 + 4 * h), y = *(const float4*)(qr + e0 + 4 * h);
        vp[4 * h] = x.x, vp[4 * h + 1] = x.y, vp[4 * h + 2] = x.z, vp[4 * h + 3] = x.w;
        vq[4 * h] = y.x, vq[4 * h + 1] = y.y, vq[4 * h + 2] = y.z, vq[4 * h + 3] = y.w;
      }
    } else {
#pragma unroll
      for (int e = 0; e < kResPer; ++e) {
        vp[e] = e0 + e < V ? pr[e0 + e] : -INFINITY;   // -inf past V: no mass
        vq[e] = e0 + e < V ? qr[e0 + e] : -INFINITY;
      }
    }
  };
  // the first chunk at the first position, loaded while the decisions are
  // taken: the usual rejected position when the draft and target disagree
  if (kb > 0) load_chunk(0, c0);
  const int ae = decide_block(a, b, kb, nch, acc_sh, info_sh, &first_sh);
  const bool rejected = ae < kb;
  if (c0 == 0) {   // the accepted prefix and the padding; out[ae] is the draw's
    int32_t* out = a.out_tokens + (size_t)b * (G + 1);
    for (int j = tid; j <= G; j += kResThreads)
      if (j != ae) out[j] = j < ae ? a.drafts[(size_t)b * G + j] : -1;
    if (tid == 0) {
      a.n_accepted[b] = ae;
      a.state[b] = ae;
      double* ri = a.rowinfo + (size_t)b * 4;
      if (rejected)
        for (int k = 0; k < 4; ++k) ri[k] = info_sh[ae][k];
    }
  }
  if (!rejected) return;                               // uniform: the draw reads the statistics only
  const double Mp = info_sh[ae][0], a0 = 1.0 / info_sh[ae][1];
  const double Mq = info_sh[ae][2], b0 = 1.0 / info_sh[ae][3];
  if (ae != 0) load_chunk(ae, c0);
  // this workgroup's chunks c0, c0 + nblk, ... of the rejected rows
  for (int c = c0; c < nch; c += nblk) {
    double sp = 0.0, sq = 0.0, P = 0.0, Q = 0.0;
#pragma unroll
    for (int e = 0; e < kResPer; ++e) {
      const double ep = vp[e] == -INFINITY ? 0.0 : exp(((double)vp[e] - Mp) * invT);
      const double eq = vq[e] == -INFINITY ? 0.0 : exp(((double)vq[e] - Mq) * invT);
      sp += ep;
      sq += eq;
      if (a0 * ep > b0 * eq) {
        P += ep;
        Q += eq;
      }
    }
    if (c + nblk < nch) load_chunk(ae, c + nblk);      // the next chunk's loads, during this one's sums
    // sub-chunk sums over the threads of the sub-chunk (fixed order)
#pragma unroll
    for (int o = kSubThreads / 2; o > 0; o >>= 1) {
      P += __shfl_xor(P, o, 64);
      Q += __shfl_xor(Q, o, 64);
    }
    double2* sub = a.sub + ((size_t)b * nch + c) * kSubPerChunk;
    if ((tid & (kSubThreads - 1)) == 0) sub[tid / kSubThreads] = make_double2(P, Q);
    if ((tid & (kSubThreads - 1)) != 0) P = Q = 0.0;  // each sub-chunk counted once below
    // the four chunk sums in one workgroup reduction (the shuffles of the four
    // run side by side)
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      sp += __shfl_xor(sp, o, 64);
      sq += __shfl_xor(sq, o, 64);
      P += __shfl_xor(P, o, 64);
      Q += __shfl_xor(Q, o, 64);
    }
    __syncthreads();                                   // red4 free (previous chunk read)
    if ((tid & 63) == 0) red4[tid >> 6] = make_double4(sp, sq, P, Q);
    __syncthreads();
    if (tid == 0) {
      double4 t = red4[0];
#pragma unroll
      for (int w = 1; w < kResThreads / 64; ++w) {
        t.x += red4[w].x;
        t.y += red4[w].y;
        t.z += red4[w].z;
        t.w += red4[w].w;
      }
      *(double4*)(a.res + ((size_t)b * nch + c) * 4) = t;
    }
  }
}

// Launch 3 (T > 0): one wave per batch row draws its one token.
__global__ __launch_bounds__(64) void draw_kernel(VerifyArgs a, int nch, bool vec) {
  const int b = blockIdx.x, lane = threadIdx.x;
  const int G = a.G, V = a.V;
  const double T = a.temperature, invT = 1.0 / T;
  const int ae = a.state[b];
  const bool rejected = ae < verify_len(a, b);
  const double u = a.u_final[b];
  const int per = (nch + 63) / 64, c0 = lane * per;
  const float* prow = a.p + ((size_t)b * (G + 1) + ae) * V;
  int tok = -1;
  bool use_resid = false;
  if (rejected) {
    const double* ri = a.rowinfo + (size_t)b * 4;
    const double Mp = ri[0], a0 = 1.0 / ri[1], Mq = ri[2], b0 = 1.0 / ri[3];
    const double* res = a.res + (size_t)b * nch * 4;
    double4 rc[kDrawChunksPerLane];
    double sp = 0.0, sq = 0.0;
#pragma unroll
    for (int k = 0; k < kDrawChunksPerLane; ++k) {
      rc[k] = (k < per && c0 + k < nch) ? *(const double4*)(res + (size_t)(c0 + k) * 4)
                                        : make_double4(0.0, 0.0, 0.0, 0.0);
      sp += rc[k].x;
      sq += rc[k].y;
    }
    sp = wave_sum(sp);
    sq = wave_sum(sq);
    const double a1 = 1.0 / sp, b1 = 1.0 / sq;
    double wl = 0.0, wk[kDrawChunksPerLane];
#pragma unroll
    for (int k = 0; k < kDrawChunksPerLane; ++k) {
      wk[k] = fmax(0.0, a1 * rc[k].z - b1 * rc[k].w);
      wl += wk[k];
    }
    const double W = wave_sum(wl);
    use_resid = W > 0.0;
    if (use_resid) {
      const double t = u * W;
      // chunk: the lane whose chunks cross t, then the chunk inside the lane
      double before;
      const int ln = wave_select(wl, 0.0, t, &before);
      int cstar = 0;
      if (ln >= 0) {
        double run = before;
        int f = -1, l = -1;
        double fb = 0.0, lb = 0.0;
#pragma unroll
        for (int k = 0; k < kDrawChunksPerLane; ++k) {
          const double w = __shfl(wk[k], ln, 64);
          if (f < 0 && w > 0.0 && run + w > t) {
            f = k;
            fb = run;
          }
          if (w > 0.0) {
            l = k;
            lb = run;
          }
          run += w;
        }
        cstar = ln * per + (f >= 0 ? f : l);
        before = f >= 0 ? fb : lb;
      }
      // sub-chunk, then token
      const double2 sb = a.sub[((size_t)b * nch + cstar) * kSubPerChunk + lane];
      const int js = wave_select(fmax(0.0, a1 * sb.x - b1 * sb.y), before, t, &before);
      const int v = cstar * kChunk + max(js, 0) * kSubTok + lane;
      const float* qrow = a.q + ((size_t)b * G + ae) * V;
      double w = 0.0;
      if (v < V) {
        const float xp = prow[v], xq = qrow[v];
        const double ep = xp == -INFINITY ? 0.0 : exp(((double)xp - Mp) * invT);
        const double eq = xq == -INFINITY ? 0.0 : exp(((double)xq - Mq) * invT);
        const double x = a1 * ep - b1 * eq;
        w = a0 * ep > b0 * eq && x > 0.0 ? x : 0.0;
      }
      const int tl = wave_select(w, before, t, &before);
      tok = tl >= 0 ? cstar * kChunk + max(js, 0) * kSubTok + tl : -1;
    }
  }
  if (!use_resid) {   // target row ae: the bonus row after an accepted block, or p_a without residual mass
    const size_t row = (size_t)b * (G + 1) + ae;
    double M, tot;
    tok = wave_draw(prow, V, a.p_chunk + row * nch, a.p_sub + row * nch * kSubPerChunk, nch, a.temperature, u, &M,
                    &tot);
  }
  if (lane == 0) a.out_tokens[(size_t)b * (G + 1) + ae] = tok < 0 ? 0 : tok;
}

// Launch 2 (T == 0): one workgroup (16 waves) per batch row; wave w takes
// positions w, w+16, ...: accept while the draft is the target's argmax (lowest
// index on ties), then emit the argmax at the first mismatch or the bonus row.
constexpr int kDecideWaves = 16;
__global__ __launch_bounds__(1024) void greedy_kernel(VerifyArgs a, int nch) {
  __shared__ int acc_sh[65];
  __shared__ int arg_sh[65];
  const int b = blockIdx.x, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int G = a.G;
  const int kb = verify_len(a, b);
  for (int i = wave; i <= kb; i += kDecideWaves) {
    const int arg = argmax_chunks_wave(a.p_chunk + ((size_t)b * (G + 1) + i) * nch, nch);
    if (lane == 0) {
      arg_sh[i] = arg;
      acc_sh[i] = i < kb && a.drafts[(size_t)b * G + i] == arg;
    }
  }
  __syncthreads();
  if (threadIdx.x != 0) return;
  int acc_end = kb;
  for (int i = 0; i < kb; ++i)
    if (!acc_sh[i]) {
      acc_end = i;
      break;
    }
  int32_t* out = a.out_tokens + (size_t)b * (G + 1);
  for (int i = 0; i < acc_end; ++i) out[i] = a.drafts[(size_t)b * G + i];
  out[acc_end] = arg_sh[acc_end];   // correction or bonus: the target argmax
  for (int j = acc_end + 1; j <= G; ++j) out[j] = -1;
  a.n_accepted[b] = acc_end;
}

}  // namespace

hipError_t launch_verify(const VerifyArgs& a, hipStream_t s) {
  ProfScope ps("verify", s);
  const int nch = ceil_div(a.V, kChunk);
  const int p_rows = a.B * (a.G + 1);
  const int q_rows = (!a.q_stats && a.temperature != 0.f) ? a.B * a.G : 0;
  const bool vec_p = (a.V & 3) == 0 && ((uintptr_t)a.p & 15) == 0;
  const bool vec_q = (a.V & 3) == 0 && ((uintptr_t)a.q & 15) == 0;
  hipLaunchKernelGGL(stats_kernel, dim3((unsigned)((size_t)(p_rows + q_rows) * nch)), dim3(256), 0, s, a, nch,
                     p_rows, vec_p, vec_q);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.temperature == 0.f) {
    hipLaunchKernelGGL(greedy_kernel, dim3(a.B), dim3(64 * kDecideWaves), 0, s, a, nch);
    return hipGetLastError();
  }
  // about two resident workgroups per CU: rows with many chunks per workgroup
  // at large batches (each workgroup repeats its row's decisions once)
  const int nblk = min(nch, max(1, ceil_div(512, a.B)));
  hipLaunchKernelGGL(resolve_kernel, dim3((unsigned)((size_t)a.B * nblk)), dim3(kResThreads), 0, s, a, nch, nblk,
                     vec_p && vec_q);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(draw_kernel, dim3(a.B), dim3(64), 0, s, a, nch, vec_p && vec_q);
  return hipGetLastError();
}

}  // namespace dfs
