// Block-vs-context attention of the drafter (DFlash page, architecture
// paragraph: full attention inside the block, causal toward the context — every
// context key precedes the block, so each block row sees all C_b context keys
// and all S block keys).
//
// bf16 path.  One wave owns one work unit (batch row b, key/value head g, key
// range).  Its queries are the R = (nq/nkv)*S rows of the GQA group (<= 64),
// held in registers for the whole unit.  Keys are walked 32 at a time:
//   S^T = K . Q^T    (v_mfma_f32_16x16x32_bf16; A = 16 keys x 32 dims read
//                     straight from the [slot][d] key cache)
//   online softmax in the exp2 domain, per query row (a row's 32 scores live in
//                     4 lanes: two cross-lane xor-shuffles reduce them)
//   O^T += V^T . P^T (A = 16 dims x 32 keys read straight from the transposed
//                     [d][slot] value cache; B = the probabilities exactly as the
//                     S^T step left them in registers)
// Key order inside a 32-key step is permuted for the S^T operand (A row c holds
// key 8*(c/4) + 4*t + c%4 of tile t) so that each lane ends up holding 8
// consecutive keys of one query row — the B-operand layout of the next MFMA —
// with no LDS round trip.  Context keys are split over units; one extra unit
// per (b, g) takes the S block keys; a combine kernel merges the units'
// (max, sum, O) partials.
//
// fp32 path: one workgroup per query row, two-pass chunked softmax on VALU.
#include "kernels.h"

#include <math.h>

namespace dfs {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ bf16x8 load8(const bf16_t* p) {
  return __builtin_bit_cast(bf16x8, ldg16(p));
}

__device__ __forceinline__ bf16x8 zero8() { return __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0)); }

template <int RT>
__global__ __launch_bounds__(64) void attn_bf16_d128(AttnArgs a) {
  constexpr int D = 128;
  const int lane = threadIdx.x, c = lane & 15, g4 = lane >> 4;
  const int unit = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int units = a.n_ctx_splits + 1;
  const size_t bg = (size_t)b * a.nkv + g;

  const bf16_t* K;
  const bf16_t* Vt;
  int ldv, k_begin, k_end;
  if (unit == a.n_ctx_splits) {              // the S block keys
    K = (const bf16_t*)a.k_blk + bg * 64 * D;
    Vt = (const bf16_t*)a.v_blk + bg * D * 64;
    ldv = 64;
    k_begin = 0;
    k_end = a.S;
  } else {                                   // context keys [unit*kps, (unit+1)*kps) ∩ [0, C_b)
    K = (const bf16_t*)a.k_cache + bg * a.max_ctx * D;
    Vt = (const bf16_t*)a.v_cache + bg * D * a.max_ctx;
    ldv = a.max_ctx;
    k_begin = unit * a.keys_per_split;
    k_end = min(min(a.ctx_len[b], a.ctx_bound), k_begin + a.keys_per_split);
  }

  // queries as the B operand of S^T: lane supplies row rt*16 + c, dims ds*32 + g4*8 .. +8
  const bf16_t* Q = (const bf16_t*)a.q + bg * a.Rpad * D;
  bf16x8 qf[RT][4];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int ds = 0; ds < 4; ++ds) {
      const int row = rt * 16 + c;
      qf[rt][ds] = row < a.R ? load8(Q + (size_t)row * D + ds * 32 + g4 * 8) : zero8();
    }

  f32x4 o[8][RT];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) o[dt][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run[RT], l_run[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    m_run[rt] = -INFINITY;
    l_run[rt] = 0.f;
  }
  const float sc = kLog2e * rsqrtf((float)D);

  // operand loads of one 32-key step starting at key k0
  bf16x8 kf[2][4], vf[8];
  auto load_step = [&](int k0) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int key = k0 + 8 * (c >> 2) + 4 * t + (c & 3);
#pragma unroll
      for (int ds = 0; ds < 4; ++ds) kf[t][ds] = load8(K + (size_t)key * D + ds * 32 + g4 * 8);
    }
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) vf[dt] = load8(Vt + (size_t)(dt * 16 + c) * ldv + k0 + g4 * 8);
  };

  if (k_begin < k_end) load_step(k_begin);
  for (int k0 = k_begin; k0 < k_end; k0 += 32) {
    bf16x8 kc[2][4], vc[8];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int ds = 0; ds < 4; ++ds) kc[t][ds] = kf[t][ds];
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) vc[dt] = vf[dt];
    if (k0 + 32 < k_end) load_step(k0 + 32);          // next step's loads in flight

    f32x4 s[2][RT];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ds = 0; ds < 4; ++ds)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kc[t][ds], qf[rt][ds], acc, 0, 0, 0);
        s[t][rt] = acc;
      }

    // this lane's scores are keys k0 + 8*g4 + 4*t + i of query row rt*16 + c
    const int kbase = k0 + 8 * g4;
    const int nvalid = k_end - kbase;                 // keys j < nvalid are real
    if (nvalid < 8) {
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        bf16_t e[8];
        *(uint4*)e = __builtin_bit_cast(uint4, vc[dt]);
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (j >= nvalid) e[j] = 0;
        vc[dt] = __builtin_bit_cast(bf16x8, *(uint4*)e);
      }
    }

    bf16x8 pf[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      float v[8];
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int j = 4 * t + i;
          v[j] = j < nvalid ? s[t][rt][i] * sc : -INFINITY;
        }
      float mx = v[0];
#pragma unroll
      for (int j = 1; j < 8; ++j) mx = fmaxf(mx, v[j]);
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_new = fmaxf(m_run[rt], mx);
      const bool none = m_new == -INFINITY;
      const float alpha = none ? 1.f : exp2f(m_run[rt] - m_new);
      bf16_t pb[8];
      float rs = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float p = none ? 0.f : exp2f(v[j] - m_new);
        pb[j] = f2bf(p);
        rs += bf2f(pb[j]);                            // normalise with the rounded weights
      }
      rs += __shfl_xor(rs, 16, 64);
      rs += __shfl_xor(rs, 32, 64);
      l_run[rt] = l_run[rt] * alpha + rs;
      m_run[rt] = m_new;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) o[dt][rt] *= alpha;
      pf[rt] = __builtin_bit_cast(bf16x8, *(uint4*)pb);
    }

#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
        o[dt][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vc[dt], pf[rt], o[dt][rt], 0, 0, 0);
  }

  // partial O^T tile (dt, rt): lane holds dims dt*16 + 4*g4 + i of row rt*16 + c
  const size_t ubase = (bg * units + unit) * a.Rpad;
  float* po = a.part_o + ubase * D;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int row = rt * 16 + c;
    if (row >= a.R) continue;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) *(f32x4*)(po + (size_t)row * D + dt * 16 + 4 * g4) = o[dt][rt];
    if (g4 == 0) {
      a.part_ml[(ubase + row) * 2 + 0] = m_run[rt];
      a.part_ml[(ubase + row) * 2 + 1] = l_run[rt];
    }
  }
}

// Merge the units of one (b, g, row): out = sum_u 2^(m_u - M) O_u / sum_u 2^(m_u - M) l_u
template <typename T>
__global__ __launch_bounds__(128) void attn_combine(AttnArgs a) {
  const int r = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int units = a.n_ctx_splits + 1;
  const size_t bg = (size_t)b * a.nkv + g;
  const float* ml = a.part_ml + (bg * units * a.Rpad + r) * 2;   // unit u at ml[u * Rpad * 2]
  const size_t ustride = (size_t)a.Rpad * 2;
  float M = -INFINITY;
  for (int u = 0; u < units; ++u) M = fmaxf(M, ml[u * ustride]);
  float den = 0.f;
  for (int u = 0; u < units; ++u) {
    const float m = ml[u * ustride];
    if (m != -INFINITY) den += exp2f(m - M) * ml[u * ustride + 1];
  }
  const int group = a.nq / a.nkv;
  const int hh = r / a.S, s = r % a.S, h = g * group + hh;
  const float inv = 1.f / den;
  for (int dd = threadIdx.x; dd < a.d; dd += blockDim.x) {
    float num = 0.f;
    for (int u = 0; u < units; ++u) {
      const float m = ml[u * ustride];
      if (m != -INFINITY)
        num += exp2f(m - M) * a.part_o[((bg * units + u) * a.Rpad + r) * a.d + dd];
    }
    Elem<T>::store((T*)a.out, (((size_t)b * a.S + s) * a.nq + h) * a.d + dd, num * inv);
  }
}

// fp32: one workgroup per (query row s, head h, batch b); keys in chunks of 256.
__global__ __launch_bounds__(256) void attn_f32(AttnArgs a) {
  constexpr int CH = 256;
  __shared__ float qs[256];
  __shared__ float ps[CH];
  __shared__ float red[4];
  const int s = blockIdx.x, h = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int group = a.nq / a.nkv, g = h / group, hh = h % group;
  const int d = a.d;
  const size_t bg = (size_t)b * a.nkv + g;
  const float* Q = (const float*)a.q + (bg * a.Rpad + hh * a.S + s) * d;
  for (int i = tid; i < d; i += 256) qs[i] = Q[i];
  __syncthreads();
  const int C = max(0, min(a.ctx_len[b], a.ctx_bound));
  const int total = C + a.S;
  const float scale = 1.f / sqrtf((float)d);
  float m_run = -INFINITY, l_run = 0.f, acc = 0.f;   // acc: output dim tid (tid < d)
  for (int k0 = 0; k0 < total; k0 += CH) {
    const int key = k0 + tid;
    float sv = -INFINITY;
    if (key < total) {
      const float* kr = key < C ? (const float*)a.k_cache + (bg * a.max_ctx + key) * d
                                : (const float*)a.k_blk + (bg * 64 + (key - C)) * d;
      float dot = 0.f;
      for (int i = 0; i < d; ++i) dot = fmaf(qs[i], kr[i], dot);
      sv = dot * scale;
    }
    const float mx = block_max<256>(sv, red);
    const float m_new = fmaxf(m_run, mx);
    const float p = key < total ? expf(sv - m_new) : 0.f;
    ps[tid] = p;
    const float sum = block_sum<256>(p, red);
    const float alpha = expf(m_run - m_new);
    l_run = l_run * alpha + sum;
    m_run = m_new;
    __syncthreads();
    if (tid < d) {
      float o = acc * alpha;
      const int n = min(CH, total - k0);
      for (int j = 0; j < n; ++j) {
        const int kk = k0 + j;
        const float v = kk < C ? ((const float*)a.v_cache)[(bg * d + tid) * a.max_ctx + kk]
                               : ((const float*)a.v_blk)[(bg * d + tid) * 64 + (kk - C)];
        o = fmaf(ps[j], v, o);
      }
      acc = o;
    }
    __syncthreads();
  }
  if (tid < d) ((float*)a.out)[(((size_t)b * a.S + s) * a.nq + h) * d + tid] = acc / l_run;
}

template <typename T>
__global__ __launch_bounds__(256) void attn_stage_kernel(const T* q, const T* k, const T* v, T* q_att, T* k_blk,
                                                         T* v_blk, int B, int S, int nq, int nkv, int d, int Rpad) {
  const int s = blockIdx.x, b = blockIdx.y;
  const int group = nq / nkv;
  for (int e = threadIdx.x; e < nq * d; e += 256) {
    const int h = e / d, dd = e % d, g = h / group, hh = h % group;
    q_att[(((size_t)b * nkv + g) * Rpad + hh * S + s) * d + dd] = q[(((size_t)b * S + s) * nq + h) * d + dd];
  }
  for (int e = threadIdx.x; e < nkv * d; e += 256) {
    const int g = e / d, dd = e % d;
    const size_t bg = (size_t)b * nkv + g;
    k_blk[(bg * 64 + s) * d + dd] = k[(((size_t)b * S + s) * nkv + g) * d + dd];
    v_blk[(bg * d + dd) * 64 + s] = v[(((size_t)b * S + s) * nkv + g) * d + dd];
  }
}

}  // namespace

hipError_t launch_attn_stage(const void* q, const void* k, const void* v, void* q_att, void* k_blk, void* v_blk,
                             int B, int S, int nq, int nkv, int d, int Rpad, int dtype, hipStream_t s) {
  if (dtype == 1)
    hipLaunchKernelGGL(attn_stage_kernel<bf16_t>, dim3(S, B), dim3(256), 0, s, (const bf16_t*)q, (const bf16_t*)k,
                       (const bf16_t*)v, (bf16_t*)q_att, (bf16_t*)k_blk, (bf16_t*)v_blk, B, S, nq, nkv, d, Rpad);
  else
    hipLaunchKernelGGL(attn_stage_kernel<float>, dim3(S, B), dim3(256), 0, s, (const float*)q, (const float*)k,
                       (const float*)v, (float*)q_att, (float*)k_blk, (float*)v_blk, B, S, nq, nkv, d, Rpad);
  return hipGetLastError();
}

AttnPlan attn_plan(int B, int nkv, int ctx_bound, int dtype) {
  AttnPlan p;
  if (dtype != 1) {
    p.keys_per_split = ctx_bound;
    p.n_ctx_splits = 0;
    return p;
  }
  const int pairs = B * nkv;
  int splits = ceil_div(512, pairs);
  const int max_splits = ceil_div(ctx_bound, 256);   // at least 256 keys per unit
  if (splits > max_splits) splits = max_splits;
  if (splits < 1) splits = 1;
  int kps = ceil_div(ceil_div(ctx_bound, splits), 64) * 64;
  if (kps < 64) kps = 64;
  p.keys_per_split = kps;
  p.n_ctx_splits = ceil_div(ctx_bound, kps);
  return p;
}

// Upper bound of the unit count over every ctx_bound <= max_ctx (the split
// count actually used never exceeds the target split count).
int attn_max_units(int B, int nkv, int max_ctx, int dtype) {
  if (dtype != 1) return 1;
  int splits = ceil_div(512, B * nkv);
  const int max_splits = ceil_div(max_ctx, 256);
  if (splits > max_splits) splits = max_splits;
  if (splits < 1) splits = 1;
  return splits + 1;
}

size_t attn_partial_elems(int units, int B, int nkv, int Rpad, int d) {
  return (size_t)B * nkv * units * Rpad * d;
}

hipError_t launch_attention(const AttnArgs& a, int dtype, hipStream_t s) {
  ProfScope ps("attention", s);
  if (dtype != 1) {
    hipLaunchKernelGGL(attn_f32, dim3(a.S, a.nq, a.B), dim3(256), 0, s, a);
    return hipGetLastError();
  }
  dim3 grid(a.n_ctx_splits + 1, a.nkv, a.B);
  const int rt = a.Rpad / 16;
  if (rt == 1) hipLaunchKernelGGL(attn_bf16_d128<1>, grid, dim3(64), 0, s, a);
  else if (rt == 2) hipLaunchKernelGGL(attn_bf16_d128<2>, grid, dim3(64), 0, s, a);
  else if (rt == 3) hipLaunchKernelGGL(attn_bf16_d128<3>, grid, dim3(64), 0, s, a);
  else hipLaunchKernelGGL(attn_bf16_d128<4>, grid, dim3(64), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_combine<bf16_t>, dim3(a.R, a.nkv, a.B), dim3(128), 0, s, a);
  return hipGetLastError();
}

}  // namespace dfs
