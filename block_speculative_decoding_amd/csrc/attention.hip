// Block-vs-context attention of the drafter (DFlash page, architecture
// paragraph: full attention inside the block, causal toward the context — every
// context key precedes the block, so each block row sees all C_b context keys
// and all S block keys).
//
// bf16 path (matrix cores, v_mfma_f32_16x16x32_bf16).  The work unit is
// (batch row b, key/value head g, key range, group of 64 query rows); its
// queries are up to 64 of the R = (nq/nkv)*S rows of the GQA group (R > 64
// — long blocks — takes several groups, each reading the unit's keys).  A 4-wave workgroup streams the
// unit's K and V^T tiles through LDS once and each wave multiplies them against
// its own 16 query rows (details at the kernel).  Context keys are split over
// units so that the grid fills the GPU; one extra unit per (b, g) takes the S
// block keys; a combine kernel merges the units' (max, sum, O) partials.
//
// fp32 path: one workgroup per query row, two-pass chunked softmax on VALU.
#include "kernels.h"

#include <math.h>

namespace dfs {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNoMax = -1e30f;             // running max before the first key

// 2^x by the hardware exponential (results below 2^-126 flush to zero, which
// no softmax weight here can notice next to the running max's weight 1)
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
constexpr int kAttnTargetUnits = 256;        // context units per launch: one per CU

__device__ __forceinline__ bf16x8 load8(const bf16_t* p) {
  return __builtin_bit_cast(bf16x8, ldg16(p));
}

__device__ __forceinline__ bf16x8 zero8() { return __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0)); }

// One workgroup (4 waves) per unit: batch row b, key/value head g, key range.
// Wave w owns query rows [16w, 16w+16) of the GQA group (rows >= R idle).
// Keys are walked 64 at a time.  All 256 threads load the step's K tile
// (64 slots x 128 dims, contiguous in the [slot][d] cache) and V^T tile
// (128 dims x 64 slots of the transposed [d][slot] cache) into registers two
// steps ahead, then into double-buffered LDS; the 4 waves share both tiles.
//   S^T = K . Q^T    A = 16 keys x 32 dims from LDS; B = the wave's queries (registers)
//   online softmax in the exp2 domain (a row's 64 scores live in 4 lanes)
//   O^T += V^T . P^T A = 16 dims x 32 keys from LDS; B = the probabilities as the
//                    S^T step left them (key order permuted inside a step: A row c
//                    of key tile t is key 32*(t/2) + 8*(c/4) + 4*(t%2) + c%4, so
//                    each lane holds 8 consecutive keys of one query row)
// Value slots past the end of the range are zeroed on their way into LDS (slots
// past C_b may hold anything, including NaN); their scores are masked to -inf.
constexpr int kAttnKeys = 64;
constexpr int kKLd = 128 + 8;              // LDS row of the K tile (bf16 elements)
constexpr int kVLd = kAttnKeys + 8;        // LDS row of the V^T tile

// Grid: 1-D, the B*nkv*n_ctx_splits context units first and the B*nkv block-key
// units last, so that the (heavy) context units are dispatched one per CU ahead
// of the (tiny) block units instead of doubling up on some CUs.
__global__ __launch_bounds__(256) void attn_bf16_d128(AttnArgs a) {
  constexpr int D = 128, KS = kAttnKeys;
  __shared__ __attribute__((aligned(16))) bf16_t Ks[2][KS * kKLd];
  __shared__ __attribute__((aligned(16))) bf16_t Vs[2][D * kVLd];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, c = lane & 15, g4 = lane >> 4;
  const int pairs = a.B * a.nkv, rgs = a.row_groups, nctx = pairs * rgs * a.n_ctx_splits;
  const int id = blockIdx.x;
  const int unit = id < nctx ? id % a.n_ctx_splits : a.n_ctx_splits;
  const int rest = id < nctx ? id / a.n_ctx_splits : id - nctx;
  const int rg = rest % rgs, pair = rest / rgs;          // 64-row group of the R query rows
  const int g = pair % a.nkv, b = pair / a.nkv;
  const int units = a.n_ctx_splits + 1;
  const size_t bg = (size_t)b * a.nkv + g;
  // one context unit per (b, g, group) — the grid fills the GPU without splits —
  // also walks the S block keys and writes the normalised output itself (no
  // block units, no partials, no combine pass)
  const bool fused = a.n_ctx_splits == 1;

  const bf16_t* K;
  const bf16_t* Vt;
  int ldv, k_begin, k_end, k_lo = 0;
  if (unit == a.n_ctx_splits) {              // the S block keys
    K = (const bf16_t*)a.k_blk + bg * 64 * D;
    Vt = (const bf16_t*)a.v_blk + bg * D * 64;
    ldv = 64;
    k_begin = 0;
    k_end = a.S;
  } else {
    // context keys [unit*kps, (unit+1)*kps) ∩ [0, C_b): the row's own C_b split
    // evenly over the planned units (a loose host bound — a graph-captured loop
    // passes the cache capacity — then costs no imbalance)
    K = (const bf16_t*)a.k_cache + bg * a.max_ctx * D;
    Vt = (const bf16_t*)a.v_cache + bg * D * a.max_ctx;
    ldv = a.max_ctx;
    // with a sliding window only keys [C_b - window, C_b) count: the range starts
    // at that key rounded down to a 64-key step (aligned tiles), and the keys in
    // front of it inside the first step are masked
    const int cb = max(0, min(a.ctx_len[b], a.ctx_bound));
    k_lo = a.window > 0 ? max(0, cb - a.window) : 0;
    const int lo = k_lo / KS * KS;
    const int kps = (ceil_div(cb - lo, a.n_ctx_splits) + KS - 1) / KS * KS;
    k_begin = lo + unit * kps;
    k_end = min(cb, k_begin + kps);
  }
  int nsteps = k_end > k_begin ? (k_end - k_begin + KS - 1) / KS : 0;

  // staging: 16-byte chunks, 4 of K and 4 of V^T per thread per step
  //   K chunk q: slot q/16, dims (q%16)*8..+8      V chunk q: dim q/8, slots (q%8)*8..+8
  int kq_slot[4], kq_col[4], vq_row[4], vq_col[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int q = tid + 256 * i;
    kq_slot[i] = q >> 4;
    kq_col[i] = (q & 15) * 8;
    vq_row[i] = q >> 3;
    vq_col[i] = (q & 7) * 8;
  }
  uint4 kr0[4], vr0[4], kr1[4], vr1[4];
  auto issue = [&](int st, uint4* kr, uint4* vr) {
    const int k0 = k_begin + min(st, nsteps - 1) * KS;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      kr[i] = ldg16(K + (size_t)(k0 + kq_slot[i]) * D + kq_col[i]);
      vr[i] = ldg16(Vt + (size_t)vq_row[i] * ldv + k0 + vq_col[i]);
    }
  };
  // branch-free: no divergent control flow between loads and their waits
  auto keep = [](int nvalid, int w) -> unsigned {   // mask of the two bf16 in 32-bit word w
    return (2 * w < nvalid ? 0x0000FFFFu : 0u) | (2 * w + 1 < nvalid ? 0xFFFF0000u : 0u);
  };
  auto stage = [&](int st, const uint4* kr, const uint4* vr, int buf) {
    const int k0 = k_begin + st * KS;
    if (k0 + KS <= k_end) {                              // uniform: every value slot is real
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        *(uint4*)&Ks[buf][kq_slot[i] * kKLd + kq_col[i]] = kr[i];
        *(uint4*)&Vs[buf][vq_row[i] * kVLd + vq_col[i]] = vr[i];
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *(uint4*)&Ks[buf][kq_slot[i] * kKLd + kq_col[i]] = kr[i];
      const int nvalid = k_end - (k0 + vq_col[i]);   // value slots j < nvalid are real
      uint4 v = vr[i];
      v.x &= keep(nvalid, 0);
      v.y &= keep(nvalid, 1);
      v.z &= keep(nvalid, 2);
      v.w &= keep(nvalid, 3);
      *(uint4*)&Vs[buf][vq_row[i] * kVLd + vq_col[i]] = v;
    }
  };

  // this wave's queries as the B operand of S^T: row 64*rg + 16*wave + c, dims ds*32 + g4*8 .. +8
  const int row = rg * 64 + wave * 16 + c;
  const bool active = rg * 64 + wave * 16 < a.R;
  bf16x8 qf[4];
  const bf16_t* Q = (const bf16_t*)a.q + (bg * a.Rpad + min(row, a.Rpad - 1)) * D;
#pragma unroll
  for (int ds = 0; ds < 4; ++ds) {
    qf[ds] = __builtin_bit_cast(bf16x8, ldg16(Q + ds * 32 + g4 * 8));
    if (row >= a.R) qf[ds] = __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0));
  }
  f32x4 o[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  // m_run starts finite (far below any score) so that exp2(score - m_run) needs no
  // guard for masked (-inf) scores; a unit that saw no key reports -inf below
  float m_run = kNoMax, l_run = 0.f;
  const float sc = kLog2e * rsqrtf((float)D);

  auto compute = [&](int st, int buf) {
    const int k0 = k_begin + st * KS;
    const bf16_t* ks = Ks[buf];
    const bf16_t* vs = Vs[buf];
    f32x4 s[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int key = 32 * (t >> 1) + 8 * (c >> 2) + 4 * (t & 1) + (c & 3);
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ds = 0; ds < 4; ++ds)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*(const bf16x8*)&ks[key * kKLd + ds * 32 + g4 * 8], qf[ds],
                                                      acc, 0, 0, 0);
      s[t] = acc;
    }
    // lane's scores: tile t, reg i -> key k0 + 32*(t/2) + 8*g4 + 4*(t%2) + i of query row `row`
    float v[16];
    float mx = -INFINITY;
    if (k0 >= k_lo && k0 + KS <= k_end) {               // full step (uniform): no masking
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          v[4 * t + i] = s[t][i] * sc;
          mx = fmaxf(mx, v[4 * t + i]);
        }
    } else {
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = k0 + 32 * (t >> 1) + 8 * g4 + 4 * (t & 1) + i;
          v[4 * t + i] = key < k_end && key >= k_lo ? s[t][i] * sc : -INFINITY;
          mx = fmaxf(mx, v[4 * t + i]);
        }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    // Lazy rescaling: the reference m_run only moves when a row's maximum grows
    // by more than 2^8 (weights stay <= 256, exact in the fp32/bf16 range), so
    // the O rescale below is skipped by the whole wave on most steps.
    const bool grow = mx > m_run + 8.f;
    const float alpha = grow ? fast_exp2(m_run - mx) : 1.f;   // first key: 2^(kNoMax - mx) = 0
    if (grow) m_run = mx;
    // P enters the P.V product as two bf16 parts, hi = bf16(p) and lo = bf16(p - hi):
    // a single bf16 P (8 significant bits) costs ~1 bf16 ulp on every output element
    float rs = 0.f;
    bf16x8 pf[2], pl[2];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const float p = fast_exp2(v[j] - m_run);           // masked: 2^-inf = 0
      const __bf16 hi = (__bf16)p;
      pf[j >> 3][j & 7] = hi;
      pl[j >> 3][j & 7] = (__bf16)(p - (float)hi);
      rs += p;
    }
    rs += __shfl_xor(rs, 16, 64);
    rs += __shfl_xor(rs, 32, 64);
    l_run = l_run * alpha + rs;
    if (__any(grow)) {
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) o[dt] *= alpha;
    }
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {                     // keys 32*kh .. 32*kh+31
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const bf16x8 vf = *(const bf16x8*)&vs[(dt * 16 + c) * kVLd + 32 * kh + g4 * 8];
        o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[kh], o[dt], 0, 0, 0);
        o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pl[kh], o[dt], 0, 0, 0);
      }
    }
  };

  // Two steps per iteration, both always staged (a step past the end stages
  // clamped, fully masked tiles) so loads and waits sit in straight-line code;
  // only the math is skipped.
  auto walk = [&]() {
    if (nsteps > 0) {
      issue(0, kr0, vr0);
      issue(1, kr1, vr1);
      for (int it = 0; it < nsteps; it += 2) {
        stage(it, kr0, vr0, 0);
        __syncthreads();
        issue(it + 2, kr0, vr0);
        if (active) compute(it, 0);
        stage(it + 1, kr1, vr1, 1);
        __syncthreads();
        issue(it + 3, kr1, vr1);
        if (active && it + 1 < nsteps) compute(it + 1, 1);
      }
    }
  };
  walk();
  if (fused) {                               // then the block keys, same running softmax
    __syncthreads();                         // every wave is done with both LDS buffers
    K = (const bf16_t*)a.k_blk + bg * 64 * D;
    Vt = (const bf16_t*)a.v_blk + bg * D * 64;
    ldv = 64;
    k_begin = 0;
    k_end = a.S;
    k_lo = 0;
    nsteps = 1;
    walk();
  }
  if (!active || row >= a.R) return;

  if (fused) {
    // output tile dt: lane holds dims dt*16 + 4*g4 .. +3 of query row `row` = hh*S + s
    const int group = a.nq / a.nkv, hh = row / a.S, s = row % a.S, h = g * group + hh;
    const int orow = b * a.S + s;
    bf16_t* out = (bf16_t*)a.out + ((size_t)orow * a.nq + h) * D;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      bf16_t v4[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) v4[i] = f2bf(o[dt][i] / l_run);
      const int col = dt * 16 + 4 * g4;
      bf16_t* dst = a.out_packed ? (bf16_t*)a.out + xpk_index(orow, h * D + col, a.nq * D) : out + col;
      *(uint2*)dst = make_uint2((uint32_t)v4[0] | ((uint32_t)v4[1] << 16), (uint32_t)v4[2] | ((uint32_t)v4[3] << 16));
    }
    return;
  }

  // partial O^T tile dt: lane holds dims dt*16 + 4*g4 + i of row `row`
  const size_t ubase = (bg * units + unit) * a.Rpad;
  float* po = a.part_o + (ubase + row) * D;
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) *(f32x4*)(po + dt * 16 + 4 * g4) = o[dt];
  if (g4 == 0) {
    a.part_ml[(ubase + row) * 2 + 0] = l_run > 0.f ? m_run : -INFINITY;
    a.part_ml[(ubase + row) * 2 + 1] = l_run;
  }
}

// Merge the units of one (b, g, row): out = sum_u 2^(m_u - M) O_u / sum_u 2^(m_u - M) l_u.
// One thread per output element; with up to 8 units every load is issued at
// once (one memory round trip), otherwise the units are walked in groups of 8.
template <typename T>
__global__ __launch_bounds__(128) void attn_combine(AttnArgs a) {
  constexpr int U = 8;
  const int r = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int units = a.n_ctx_splits + 1;
  const size_t bg = (size_t)b * a.nkv + g;
  const float* ml = a.part_ml + (bg * units * a.Rpad + r) * 2;   // unit u at ml[u * Rpad * 2]
  const size_t ustride = (size_t)a.Rpad * 2;
  const int group = a.nq / a.nkv;
  const int hh = r / a.S, s = r % a.S, h = g * group + hh;
  for (int dd = threadIdx.x; dd < a.d; dd += blockDim.x) {
    const float* po = a.part_o + (bg * units * a.Rpad + r) * a.d + dd;   // unit u at po[u * Rpad * d]
    const size_t pstride = (size_t)a.Rpad * a.d;
    float M = -INFINITY, den = 0.f, num = 0.f;         // running merge over groups of U units
    for (int u0 = 0; u0 < units; u0 += U) {
      float m[U], l[U], o[U];
#pragma unroll
      for (int i = 0; i < U; ++i) {
        const int u = min(u0 + i, units - 1);
        m[i] = ml[u * ustride];
        l[i] = ml[u * ustride + 1];
        o[i] = po[u * pstride];
      }
      float mg = M;
#pragma unroll
      for (int i = 0; i < U; ++i)
        if (u0 + i < units) mg = fmaxf(mg, m[i]);
      if (mg == -INFINITY) continue;
      const float alpha = M == -INFINITY ? 0.f : exp2f(M - mg);
      den *= alpha;
      num *= alpha;
#pragma unroll
      for (int i = 0; i < U; ++i) {
        if (u0 + i >= units || m[i] == -INFINITY) continue;
        const float w = exp2f(m[i] - mg);
        den += w * l[i];
        num += w * o[i];
      }
      M = mg;
    }
    const int orow = b * a.S + s, col = h * a.d + dd;
    Elem<T>::store((T*)a.out, a.out_packed ? xpk_index(orow, col, a.nq * a.d) : (size_t)orow * a.nq * a.d + col,
                   num / den);
  }
}

// The same merge for d = 128, vectorised: 256 threads take 8 query rows, each
// thread four consecutive dims (16-byte partial loads, one 8-byte store), so
// the grid is a quarter of the size and each unit costs one load per thread.
// Per element the arithmetic is that of attn_combine, in the same order.
__global__ __launch_bounds__(256) void attn_combine4(AttnArgs a) {
  constexpr int U = 8, D = 128;
  const int r = blockIdx.x * 8 + (threadIdx.x >> 5), g = blockIdx.y, b = blockIdx.z;
  if (r >= a.R) return;
  const int dd = (threadIdx.x & 31) * 4;
  const int units = a.n_ctx_splits + 1;
  const size_t bg = (size_t)b * a.nkv + g;
  const float* ml = a.part_ml + (bg * units * a.Rpad + r) * 2;
  const size_t ustride = (size_t)a.Rpad * 2;
  const float* po = a.part_o + (bg * units * a.Rpad + r) * D + dd;
  const size_t pstride = (size_t)a.Rpad * D;
  float M = -INFINITY, den = 0.f, num[4] = {0.f, 0.f, 0.f, 0.f};
  for (int u0 = 0; u0 < units; u0 += U) {
    float m[U], l[U];
    float4 o[U];
#pragma unroll
    for (int i = 0; i < U; ++i) {
      const int u = min(u0 + i, units - 1);
      m[i] = ml[u * ustride];
      l[i] = ml[u * ustride + 1];
      o[i] = *(const float4*)(po + u * pstride);
    }
    float mg = M;
#pragma unroll
    for (int i = 0; i < U; ++i)
      if (u0 + i < units) mg = fmaxf(mg, m[i]);
    if (mg == -INFINITY) continue;
    const float alpha = M == -INFINITY ? 0.f : exp2f(M - mg);
    den *= alpha;
#pragma unroll
    for (int e = 0; e < 4; ++e) num[e] *= alpha;
#pragma unroll
    for (int i = 0; i < U; ++i) {
      if (u0 + i >= units || m[i] == -INFINITY) continue;
      const float w = exp2f(m[i] - mg);
      den += w * l[i];
      num[0] += w * o[i].x;
      num[1] += w * o[i].y;
      num[2] += w * o[i].z;
      num[3] += w * o[i].w;
    }
    M = mg;
  }
  const int group = a.nq / a.nkv, hh = r / a.S, s = r % a.S, h = g * group + hh;
  const int orow = b * a.S + s, col = h * D + dd;
  uint32_t w2[2];
#pragma unroll
  for (int e = 0; e < 4; e += 2)
    w2[e / 2] = (uint32_t)f2bf(num[e] / den) | ((uint32_t)f2bf(num[e + 1] / den) << 16);
  bf16_t* out = (bf16_t*)a.out + (a.out_packed ? xpk_index(orow, col, a.nq * D) : (size_t)orow * a.nq * D + col);
  *(uint2*)out = make_uint2(w2[0], w2[1]);
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
  const int lo = a.window > 0 ? max(0, C - a.window) : 0;   // first context key attended
  const float scale = 1.f / sqrtf((float)d);
  float m_run = -INFINITY, l_run = 0.f, acc = 0.f;   // acc: output dim tid (tid < d)
  for (int k0 = lo; k0 < total; k0 += CH) {
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

// ~one four-wave context unit per CU; long contexts (units of >= 2048 keys
// after the doubling) take a second resident unit per CU, which raised a
// 32K-token context from 4.4 to 4.9 TB/s, while shorter units only add
// partials and combine work
static int attn_target_splits(int pairs, int ctx) {
  int splits = ceil_div(kAttnTargetUnits, pairs);
  if (splits > 1 && ceil_div(ctx, 2 * splits) >= 2048) splits *= 2;
  return splits;
}

AttnPlan attn_plan(int B, int nkv, int ctx_bound, int dtype, int row_groups, int window) {
  if (window > 0 && window + 64 < ctx_bound) ctx_bound = window + 64;   // keys a row can attend (step-aligned)
  AttnPlan p;
  if (dtype != 1) {
    p.keys_per_split = ctx_bound;
    p.n_ctx_splits = 0;
    return p;
  }
  const int pairs = B * nkv * row_groups;
  int splits = attn_target_splits(pairs, ctx_bound);
  const int max_splits = ceil_div(ctx_bound, 256);   // at least 256 keys (4 steps) per unit
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
  int splits = 0;
  for (int rg = 1; rg <= 4; ++rg) splits = max(splits, attn_target_splits(B * nkv * rg, max_ctx));
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
  if (a.out_packed && (dtype != 1 || (a.nq * a.d) % 64)) return hipErrorInvalidValue;
  if (dtype != 1) {
    hipLaunchKernelGGL(attn_f32, dim3(a.S, a.nq, a.B), dim3(256), 0, s, a);
    return hipGetLastError();
  }
  // with a single context unit it takes the block keys too and writes the output
  const bool fused = a.n_ctx_splits == 1;
  const dim3 grid((unsigned)(a.B * a.nkv * a.row_groups * (fused ? 1 : a.n_ctx_splits + 1)));
  hipLaunchKernelGGL(attn_bf16_d128, grid, dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || fused) return e;
  if (a.d == 128 && ((uintptr_t)a.part_o & 15) == 0 && ((uintptr_t)a.out & 7) == 0)
    hipLaunchKernelGGL(attn_combine4, dim3((a.R + 7) / 8, a.nkv, a.B), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(attn_combine<bf16_t>, dim3(a.R, a.nkv, a.B), dim3(128), 0, s, a);
  return hipGetLastError();
}

}  // namespace dfs
