// Row-wise and element-wise kernels of the drafter: positions and rotary
// tables, embedding gather, RMSNorm (fused with the reduction of split-K GEMM
// partials and with the fp32 residual update), the Q/K/V epilogue (rotary
// embedding + KV injection into the caches + block K/V staging) and SwiGLU.
// All of them are HBM/latency bound and touch each byte once.
#include "kernels.h"

#include <math.h>

namespace dfs {
namespace {

// Rotary table of every row the call touches:
//   context row (b, j), j < n_new_max  -> position ctx_len[b] + j
//   block row (b, s), s < S            -> position C_b + s,  C_b = ctx_len[b] + n_new[b]
// Angles pos * theta^(-2i/d) are formed and evaluated in fp64 (positions reach
// 32K, where an fp32 angle would already be off by ~1e-3 rad), then stored fp32.
// Work block 0 also publishes per-row bookkeeping (clamped) of every batch row,
// its threads striding over the rows: base, appended rows, C_b.
__device__ __forceinline__ void prep_work(const MetaArgs& a, int blk, int nthr) {
  const int half = a.d / 2;
  const int Mc = a.B * a.n_new_max, Mx = Mc + a.B * a.S;
  const long idx = (long)blk * nthr + threadIdx.x;
  if (blk == 0) {
    for (int b = threadIdx.x; b < a.B; b += nthr) {
      const int base = min(max(a.ctx_len[b], 0), a.ctx_bound);
      const int nn = min(max(a.n_new[b], 0), a.n_new_max);
      const int cb = min(base + nn, a.ctx_bound);
      a.meta[b] = base;
      a.meta[a.B + b] = cb - base;
      a.meta[2 * a.B + b] = cb;
    }
  }
  if (!a.rope || idx >= (long)Mx * half) return;
  const int row = (int)(idx / half), i = (int)(idx % half);
  int b, pos;
  if (row < Mc) {
    b = row / a.n_new_max;
    pos = min(max(a.ctx_len[b], 0), a.ctx_bound) + row % a.n_new_max;
  } else {
    b = (row - Mc) / a.S;
    const int base = min(max(a.ctx_len[b], 0), a.ctx_bound);
    const int cb = min(base + min(max(a.n_new[b], 0), a.n_new_max), a.ctx_bound);
    pos = cb + (row - Mc) % a.S;
  }
  const double inv_freq = pow((double)a.theta, -2.0 * i / (double)a.d);
  const double ang = (double)pos * inv_freq;
  double sn, cs;
  sincos(ang, &sn, &cs);
  a.rope[idx] = make_float2((float)cs, (float)sn);
}

// RMSNorm of one row per workgroup (1024 threads), fused with the reduction of
// split-K GEMM partials and the fp32 residual update:
//   x = (resid or 0) + sum_z part[z]   (partials summed in z order after resid)
//   resid = x (when update_resid), out = T(x * rsqrt(mean(x^2)+eps) * g)
// or, for embedding rows, x = E[token] (stored to resid as well).
// Each thread holds up to two 4-element groups (H <= 8192); vector accesses
// when H is a multiple of 4.
// v += sum over z of the float4 at p + z * stride, z = 0 .. sp-1 in that order.  The
// loads go out in batches of 8 (then 4, then 1) before the adds, so a split-K sum
// costs one memory round trip per batch instead of one per partial.
__device__ __forceinline__ void add_partials4(const float* p, int sp, size_t stride, float* v) {
  int z = 0;
  for (; z + 8 <= sp; z += 8) {
    float4 t[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) t[j] = *(const float4*)(p + (z + j) * stride);
#pragma unroll
    for (int j = 0; j < 8; ++j) v[0] += t[j].x, v[1] += t[j].y, v[2] += t[j].z, v[3] += t[j].w;
  }
  for (; z + 4 <= sp; z += 4) {
    float4 t[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) t[j] = *(const float4*)(p + (z + j) * stride);
#pragma unroll
    for (int j = 0; j < 4; ++j) v[0] += t[j].x, v[1] += t[j].y, v[2] += t[j].z, v[3] += t[j].w;
  }
  for (; z < sp; ++z) {
    const float4 t = *(const float4*)(p + z * stride);
    v[0] += t.x, v[1] += t.y, v[2] += t.z, v[3] += t.w;
  }
}

// The same for two float4 runs (p into v, q into w) with their loads batched together.
__device__ __forceinline__ void add_partials4x2(const float* p, const float* q, int sp, size_t stride, float* v,
                                                float* w) {
  int z = 0;
  for (; z + 4 <= sp; z += 4) {
    float4 t[4], u[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      t[j] = *(const float4*)(p + (z + j) * stride);
      u[j] = *(const float4*)(q + (z + j) * stride);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[0] += t[j].x, v[1] += t[j].y, v[2] += t[j].z, v[3] += t[j].w;
      w[0] += u[j].x, w[1] += u[j].y, w[2] += u[j].z, w[3] += u[j].w;
    }
  }
  for (; z < sp; ++z) {
    const float4 t = *(const float4*)(p + z * stride), u = *(const float4*)(q + z * stride);
    v[0] += t.x, v[1] += t.y, v[2] += t.z, v[3] += t.w;
    w[0] += u.x, w[1] += u.y, w[2] += u.z, w[3] += u.w;
  }
}

constexpr int kNormThreads = 1024;
template <typename T>
__device__ __forceinline__ void norm_row(const NormArgs& a, int r, float* red) {
  const int tid = threadIdx.x;
  const bool vec = (a.H & 3) == 0;
  const size_t row0 = (size_t)r * a.H;
  const bool use_resid = a.resid && (a.update_resid || !a.part);
  const T* erow = nullptr;
  if (a.embed) {
    const int b = r / a.S, s = r % a.S;
    int tok = s == 0 ? a.last_token[b] : a.mask_id;
    tok = tok < 0 ? 0 : (tok >= a.V ? a.V - 1 : tok);
    erow = (const T*)a.embed + (size_t)tok * a.H;
  }
  float v[2][4];
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int h = 4 * (tid + i * kNormThreads);
#pragma unroll
    for (int e = 0; e < 4; ++e) v[i][e] = 0.f;
    if (h < a.H && erow) {
      if (vec) {
        if constexpr (sizeof(T) == 2) {   // 4 bf16: element h in the low half of the first word
          const uint2 w = *(const uint2*)(erow + h);
          v[i][0] = __uint_as_float(w.x << 16), v[i][1] = __uint_as_float(w.x & 0xFFFF0000u);
          v[i][2] = __uint_as_float(w.y << 16), v[i][3] = __uint_as_float(w.y & 0xFFFF0000u);
        } else {
          const float4 t = *(const float4*)(erow + h);
          v[i][0] = t.x, v[i][1] = t.y, v[i][2] = t.z, v[i][3] = t.w;
        }
        *(float4*)(a.resid + row0 + h) = make_float4(v[i][0], v[i][1], v[i][2], v[i][3]);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (h + e < a.H) {
            v[i][e] = Elem<T>::load(erow, h + e);
            a.resid[row0 + h + e] = v[i][e];
          }
      }
    } else if (h < a.H) {
      if (vec) {
        if (use_resid) {
          const float4 t = *(const float4*)(a.resid + row0 + h);
          v[i][0] = t.x, v[i][1] = t.y, v[i][2] = t.z, v[i][3] = t.w;
        }
        add_partials4(a.part ? a.part + row0 + h : nullptr, a.part ? a.sp : 0, a.part_stride, v[i]);
        if (a.part && a.update_resid) *(float4*)(a.resid + row0 + h) = make_float4(v[i][0], v[i][1], v[i][2], v[i][3]);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (h + e >= a.H) break;
          float x = use_resid ? a.resid[row0 + h + e] : 0.f;
          for (int z = 0; z < (a.part ? a.sp : 0); ++z) x += a.part[z * a.part_stride + row0 + h + e];
          if (a.part && a.update_resid) a.resid[row0 + h + e] = x;
          v[i][e] = x;
        }
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) ss += v[i][e] * v[i][e];
  }
  ss = block_sum<kNormThreads>(ss, red);
  const float rs = rsqrtf(ss / (float)a.H + a.eps);
  int orow = r;
  if (a.out_mode == 1) {
    const int s = r % a.S;
    if (s == 0) return;
    orow = (r / a.S) * (a.S - 1) + s - 1;
  }
  if constexpr (sizeof(T) == 2) {
    if (a.out_packed) {   // 4 consecutive columns are one 8-byte run of the packed layout
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int h = 4 * (tid + i * kNormThreads);
        if (h >= a.H) continue;
        uint32_t w[2];
#pragma unroll
        for (int e = 0; e < 4; e += 2)
          w[e / 2] = (uint32_t)f2bf(v[i][e] * rs * Elem<T>::load((const T*)a.gain, h + e)) |
                     ((uint32_t)f2bf(v[i][e + 1] * rs * Elem<T>::load((const T*)a.gain, h + e + 1)) << 16);
        *(uint2*)((bf16_t*)a.out + xpk_index(orow + a.out_row0, h, a.H)) = make_uint2(w[0], w[1]);
      }
      return;
    }
  }
  T* out = (T*)a.out + (size_t)orow * a.H;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int h = 4 * (tid + i * kNormThreads);
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (h + e < a.H) Elem<T>::store(out, h + e, v[i][e] * rs * Elem<T>::load((const T*)a.gain, h + e));
  }
}

template <typename T>
__global__ __launch_bounds__(1024) void norm_kernel(NormArgs a) {
  __shared__ float red[kNormThreads / 64];
  norm_row<T>(a, blockIdx.x, red);
}

// The start of a drafter call: workgroups [0, f.rows) normalise the context
// features, the next b.rows embed and normalise the block rows, the rest build
// the positions and rotary table (work block 0: the bookkeeping).  Independent
// rows, so one launch instead of three.
template <typename T>
__global__ __launch_bounds__(1024) void front_kernel(NormArgs f, NormArgs b, MetaArgs m) {
  __shared__ float red[kNormThreads / 64];
  const int r = blockIdx.x;
  if (r < f.rows) norm_row<T>(f, r, red);
  else if (r < f.rows + b.rows) norm_row<T>(b, r - f.rows, red);
  else prep_work(m, r - f.rows - b.rows, kNormThreads);
}

// Q/K/V epilogue: one workgroup per (row, head).  Sums the GEMM's split-K
// partials, applies the rotary embedding to queries and keys, and scatters:
//   context row -> K cache slot base+j (KV injection, layout [b][g][slot][d]),
//                  V cache [b][g][d][slot] (values transposed)
//   block row   -> queries [b][g][hh*S + s][d], block keys [b][g][s][d],
//                  block values [b][g][d][s]
template <typename T>
__global__ __launch_bounds__(64) void qkv_kernel(QkvArgs a) {
  const int row = blockIdx.x, hd = blockIdx.y;
  if (a.ctx_len_out && row == 0 && hd == 0)
    for (int b = threadIdx.x; b < a.B; b += 64) a.ctx_len_out[b] = a.meta[2 * a.B + b];
  const int d = a.d, half = d / 2;
  const int Mc = a.B * a.n_new_max;
  const int Nqkv = (a.nq + 2 * a.nkv) * d;
  const bool ctx = row < Mc;
  int b, j, pos_slot;
  if (ctx) {
    b = row / a.n_new_max;
    j = row % a.n_new_max;
    if (j >= a.meta[a.B + b] || hd < a.nq) return;     // not appended, or no query for context rows
    pos_slot = a.meta[b] + j;
  } else {
    b = (row - Mc) / a.S;
    j = (row - Mc) % a.S;
    pos_slot = j;
  }
  const int col0 = hd * d;
  const bool is_q = hd < a.nq, is_k = !is_q && hd < a.nq + a.nkv;
  const int g = is_q ? hd / (a.nq / a.nkv) : (is_k ? hd - a.nq : hd - a.nq - a.nkv);
  const size_t bg = (size_t)b * a.nkv + g;
  auto val = [&](int col) {
    float x = 0.f;
    const size_t off = (size_t)row * Nqkv + col0 + col;
    for (int z = 0; z < a.sp; ++z) x += a.part[z * a.part_stride + off];
    return x;
  };
  for (int i = threadIdx.x; i < half; i += 64) {
    float x1 = val(i), x2 = val(i + half);
    if ((is_q || is_k) && a.use_rope) {
      const float2 cs = a.rope[(size_t)row * half + i];
      const float y1 = x1 * cs.x - x2 * cs.y;
      const float y2 = x2 * cs.x + x1 * cs.y;
      x1 = y1;
      x2 = y2;
    }
    if (is_q) {
      const int hh = hd % (a.nq / a.nkv);
      T* dst = (T*)a.q_att + (bg * a.Rpad + hh * a.S + j) * d;
      Elem<T>::store(dst, i, x1);
      Elem<T>::store(dst, i + half, x2);
    } else if (is_k) {
      T* dst = ctx ? (T*)a.k_cache + (bg * a.max_ctx + pos_slot) * d : (T*)a.k_blk + (bg * 64 + j) * d;
      Elem<T>::store(dst, i, x1);
      Elem<T>::store(dst, i + half, x2);
    } else {
      const size_t ld = ctx ? (size_t)a.max_ctx : 64;
      T* dst = ctx ? (T*)a.v_cache + bg * d * ld : (T*)a.v_blk + bg * d * ld;
      Elem<T>::store(dst, (size_t)i * ld + pos_slot, x1);
      Elem<T>::store(dst, (size_t)(i + half) * ld + pos_slot, x2);
    }
  }
}

// The same epilogue for bf16 with d = 128, by tiles: one 256-thread workgroup per
// (batch row, tile of up to 16 consecutive rows of one segment — appended context
// rows, or block rows —, head).  Thread t takes row t/16 and dims 4*(t%16) .. +3
// plus the same four of the other rotary half: 16-byte loads of each split
// partial, 8-byte stores.  Values go through LDS and are written transposed so
// that each V^T cache row receives the tile's consecutive slots together.
__global__ __launch_bounds__(256) void qkv_tile_kernel(QkvArgs a) {
  constexpr int D = 128, HALF = 64, TR = 16;
  __shared__ bf16_t vt[D][TR + 2];
  const int tid = threadIdx.x, hd = blockIdx.y;
  if (a.ctx_len_out && blockIdx.x == 0 && hd == 0)
    for (int b = tid; b < a.B; b += 256) a.ctx_len_out[b] = a.meta[2 * a.B + b];
  const int ctx_tiles = (a.n_new_max + TR - 1) / TR, blk_tiles = (a.S + TR - 1) / TR;
  const int per_b = ctx_tiles + blk_tiles;
  const int b = blockIdx.x / per_b, tile = blockIdx.x % per_b;
  const bool ctx = tile < ctx_tiles;
  if (ctx && hd < a.nq) return;                          // no queries for context rows (uniform)
  const int j0 = (ctx ? tile : tile - ctx_tiles) * TR;   // first row of the tile within its segment
  const int nrows = ctx ? min(TR, a.meta[a.B + b] - j0) : min(TR, a.S - j0);   // appended / block rows
  if (nrows <= 0) return;
  const int Mc = a.B * a.n_new_max;
  const int Nqkv = (a.nq + 2 * a.nkv) * D;
  const bool is_q = hd < a.nq, is_k = !is_q && hd < a.nq + a.nkv;
  const int g = is_q ? hd / (a.nq / a.nkv) : (is_k ? hd - a.nq : hd - a.nq - a.nkv);
  const size_t bg = (size_t)b * a.nkv + g;
  const int r = tid >> 4, i0 = (tid & 15) * 4;
  const int j = j0 + r;
  const bool valid = r < nrows;
  const int row = ctx ? b * a.n_new_max + j : Mc + b * a.S + j;
  const int slot0 = ctx ? a.meta[b] + j0 : j0;           // cache slot (or block slot) of the tile's first row
  float x1[4] = {0.f, 0.f, 0.f, 0.f}, x2[4] = {0.f, 0.f, 0.f, 0.f};
  if (valid) {
    const size_t off = (size_t)row * Nqkv + hd * D + i0;
    add_partials4x2(a.part + off, a.part + off + HALF, a.sp, a.part_stride, x1, x2);
    if ((is_q || is_k) && a.use_rope) {
      const float4 c01 = *(const float4*)(a.rope + (size_t)row * HALF + i0);
      const float4 c23 = *(const float4*)(a.rope + (size_t)row * HALF + i0 + 2);
      const float cs[4][2] = {{c01.x, c01.y}, {c01.z, c01.w}, {c23.x, c23.y}, {c23.z, c23.w}};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float y1 = x1[e] * cs[e][0] - x2[e] * cs[e][1];
        const float y2 = x2[e] * cs[e][0] + x1[e] * cs[e][1];
        x1[e] = y1;
        x2[e] = y2;
      }
    }
  }
  auto pack4 = [](const float* v) {
    return make_uint2((uint32_t)f2bf(v[0]) | ((uint32_t)f2bf(v[1]) << 16),
                      (uint32_t)f2bf(v[2]) | ((uint32_t)f2bf(v[3]) << 16));
  };
  if (is_q || is_k) {
    if (!valid) return;
    bf16_t* dst;
    if (is_q) dst = (bf16_t*)a.q_att + (bg * a.Rpad + (hd % (a.nq / a.nkv)) * a.S + j) * D;
    else dst = ctx ? (bf16_t*)a.k_cache + (bg * a.max_ctx + slot0 + r) * D : (bf16_t*)a.k_blk + (bg * 64 + j) * D;
    *(uint2*)(dst + i0) = pack4(x1);
    *(uint2*)(dst + HALF + i0) = pack4(x2);
    return;
  }
  // values: transpose through LDS, then every lane group of 16 writes one dim's slots
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    vt[i0 + e][r] = f2bf(x1[e]);
    vt[HALF + i0 + e][r] = f2bf(x2[e]);
  }
  __syncthreads();
  const size_t ld = ctx ? (size_t)a.max_ctx : 64;
  bf16_t* dst = (ctx ? (bf16_t*)a.v_cache : (bf16_t*)a.v_blk) + bg * D * ld + slot0;
  const int rr = tid & 15;
  if (rr < nrows)
    for (int dim = tid >> 4; dim < D; dim += 16) dst[(size_t)dim * ld + rr] = vt[dim][rr];
}

// h = T(silu(gate) * up) with gate = sum_z part[z][m][f], up = sum_z part[z][m][F + f]
template <typename T>
__global__ __launch_bounds__(256) void swiglu_kernel(const float* part, int sp, size_t ps, int M, int F,
                                                     T* out) {
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (size_t)M * F) return;
  const size_t m = idx / F, f = idx % F;
  float gte = 0.f, up = 0.f;
  for (int z = 0; z < sp; ++z) {
    gte += part[z * ps + m * 2 * F + f];
    up += part[z * ps + m * 2 * F + F + f];
  }
  const float silu = gte / (1.f + expf(-gte));
  Elem<T>::store(out, idx, silu * up);
}

// out = (accumulate ? out : 0) + sum_z part[z]; split slices summed in z order.
__global__ __launch_bounds__(256) void reduce_kernel(const float* part, int sp, size_t ps, size_t n, float* out,
                                                     int accumulate) {
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= n) return;
  float x = accumulate ? out[idx] : 0.f;
  float y = 0.f;
  for (int z = 0; z < sp; ++z) y += part[z * ps + idx];
  out[idx] = x + y;
}

// float4 variant (n, ps multiples of 4 and 16-byte aligned buffers)
__global__ __launch_bounds__(256) void reduce4_kernel(const float4* part, int sp, size_t ps4, size_t n4, float4* out,
                                                      int accumulate) {
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= n4) return;
  float4 y = part[idx];
  for (int z = 1; z < sp; ++z) {
    const float4 t = part[z * ps4 + idx];
    y.x += t.x;
    y.y += t.y;
    y.z += t.z;
    y.w += t.w;
  }
  if (accumulate) {
    const float4 x = out[idx];
    y.x += x.x;
    y.y += x.y;
    y.z += x.z;
    y.w += x.w;
  }
  out[idx] = y;
}

}  // namespace

hipError_t launch_reduce(const float* part, int sp, size_t ps, size_t n, float* out, hipStream_t s,
                         int accumulate) {
  ProfScope pr("elementwise", s);
  const bool vec = n % 4 == 0 && ps % 4 == 0 && ((uintptr_t)part & 15) == 0 && ((uintptr_t)out & 15) == 0;
  if (vec && sp >= 1)
    hipLaunchKernelGGL(reduce4_kernel, dim3((unsigned)((n / 4 + 255) / 256)), dim3(256), 0, s, (const float4*)part,
                       sp, ps / 4, n / 4, (float4*)out, accumulate);
  else
    hipLaunchKernelGGL(reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, part, sp, ps, n, out,
                       accumulate);
  return hipGetLastError();
}

hipError_t launch_norm(const NormArgs& a, int dtype, hipStream_t s) {
  if (a.out_packed && (dtype != 1 || a.H % 64)) return hipErrorInvalidValue;
  ProfScope ps("elementwise", s);
  if (dtype == 1) hipLaunchKernelGGL(norm_kernel<bf16_t>, dim3(a.rows), dim3(kNormThreads), 0, s, a);
  else hipLaunchKernelGGL(norm_kernel<float>, dim3(a.rows), dim3(kNormThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_front(const NormArgs& f, const NormArgs& b, const MetaArgs& m, int dtype, hipStream_t s) {
  if ((f.out_packed && (dtype != 1 || f.H % 64)) || (b.out_packed && (dtype != 1 || b.H % 64)) || !b.embed ||
      !b.resid || b.part || b.out_mode != 0)
    return hipErrorInvalidValue;
  ProfScope ps("elementwise", s);
  const long n = (long)(m.B * m.n_new_max + m.B * m.S) * (m.d / 2);
  const int prep = m.rope && n > 0 ? (int)((n + kNormThreads - 1) / kNormThreads) : 1;
  const dim3 grid(f.rows + b.rows + prep);
  if (dtype == 1) hipLaunchKernelGGL(front_kernel<bf16_t>, grid, dim3(kNormThreads), 0, s, f, b, m);
  else hipLaunchKernelGGL(front_kernel<float>, grid, dim3(kNormThreads), 0, s, f, b, m);
  return hipGetLastError();
}

hipError_t launch_qkv_epilogue(const QkvArgs& a, int dtype, hipStream_t s) {
  ProfScope ps("elementwise", s);
  const bool aligned = (((uintptr_t)a.part | (uintptr_t)a.rope) & 15) == 0 && a.part_stride % 4 == 0;
  if (dtype == 1 && a.d == 128 && aligned) {
    const int tiles = (a.n_new_max + 15) / 16 + (a.S + 15) / 16;
    hipLaunchKernelGGL(qkv_tile_kernel, dim3(a.B * tiles, a.nq + 2 * a.nkv), dim3(256), 0, s, a);
    return hipGetLastError();
  }
  dim3 grid(a.B * a.n_new_max + a.B * a.S, a.nq + 2 * a.nkv);
  if (dtype == 1) hipLaunchKernelGGL(qkv_kernel<bf16_t>, grid, dim3(64), 0, s, a);
  else hipLaunchKernelGGL(qkv_kernel<float>, grid, dim3(64), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_swiglu(const float* part, int sp, size_t ps_, int M, int F, void* out, int dtype,
                         hipStream_t s) {
  ProfScope ps("elementwise", s);
  const int grid = ceil_div(M * F, 256);
  if (dtype == 1)
    hipLaunchKernelGGL(swiglu_kernel<bf16_t>, dim3(grid), dim3(256), 0, s, part, sp, ps_, M, F, (bf16_t*)out);
  else
    hipLaunchKernelGGL(swiglu_kernel<float>, dim3(grid), dim3(256), 0, s, part, sp, ps_, M, F, (float*)out);
  return hipGetLastError();
}

}  // namespace dfs
