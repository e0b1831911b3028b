// Drafter GEMMs: Y = X . W^T with X [M, K] activations and W [N, K] weights
// ([out, in] storage, inputs contiguous), fp32 accumulation.
//
// bf16: a matrix-core kernel.  A workgroup of 4 waves owns a BM x BN output tile
// and walks K in steps of 64, staging both operand tiles in LDS (double
// buffered: the global loads of step k+1 are in flight while step k computes).
// Each wave computes a (BM/2) x (BN/2) sub-tile with v_mfma_f32_16x16x32_bf16;
// the "NT" operand layout means every lane feeds the matrix core 8 consecutive
// k values of one row with a single 16-byte LDS read, for X and for W alike.
// At the drafter's small M the kernel streams W from HBM once; K is split over
// workgroups (fp32 partial slices reduced by the consumer kernel) when there
// are too few output tiles to keep every CU loading.
//
// fp32: a plain LDS-tiled VALU kernel (the fp32 configuration is tiny).
#include "kernels.h"

namespace dfs {

namespace {

constexpr int BK = 64;
constexpr int LDK = BK + 8;   // padded LDS row (bf16 elements): 144 bytes

__device__ __forceinline__ const void* seg_row(const GemmArgs& a, int n, int es) {
  int s = 0;
  if (a.nseg > 1 && n >= a.seg[1].n0) s = 1;
  if (a.nseg > 2 && n >= a.seg[2].n0) s = 2;
  return (const char*)a.seg[s].w + (size_t)(n - a.seg[s].n0) * a.K * es;
}

__device__ __forceinline__ int x_row(const GemmArgs& a, int m) {
  if (!a.row_idx) return m;
  int r = a.row_idx[(size_t)m * a.row_idx_stride];
  return r < 0 ? 0 : (r >= a.x_rows ? a.x_rows - 1 : r);
}

template <int BM, int BN>
__global__ __launch_bounds__(256) void gemm_bf16_nt(GemmArgs a, int k_per_split) {
  constexpr int TM = BM / 32, TN = BN / 32;            // 16x16 tiles per wave (2x2 waves)
  constexpr int A_CH = BM * BK / 8 / 256;               // 16-byte chunks per thread
  constexpr int B_CH = BN * BK / 8 / 256;
  __shared__ __attribute__((aligned(16))) bf16_t As[2][BM * LDK];
  __shared__ __attribute__((aligned(16))) bf16_t Bs[2][BN * LDK];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int n0 = blockIdx.x * BN, m0 = blockIdx.y * BM, z = blockIdx.z;
  const int kbeg = z * k_per_split;
  const int kend = min(a.K, kbeg + k_per_split);
  const int nk = kend > kbeg ? (kend - kbeg) / BK : 0;

  const bf16_t* a_src[A_CH];
  bool a_ok[A_CH];
  int a_dst[A_CH];
#pragma unroll
  for (int i = 0; i < A_CH; ++i) {
    const int c = tid + i * 256, row = c >> 3, col = (c & 7) * 8, m = m0 + row;
    a_ok[i] = m < a.M;
    a_src[i] = (const bf16_t*)a.X + (size_t)x_row(a, a_ok[i] ? m : 0) * a.ldx + kbeg + col;
    a_dst[i] = row * LDK + col;
  }
  const bf16_t* b_src[B_CH];
  bool b_ok[B_CH];
  int b_dst[B_CH];
#pragma unroll
  for (int i = 0; i < B_CH; ++i) {
    const int c = tid + i * 256, row = c >> 3, col = (c & 7) * 8, n = n0 + row;
    b_ok[i] = n < a.N;
    b_src[i] = (const bf16_t*)seg_row(a, b_ok[i] ? n : 0, 2) + kbeg + col;
    b_dst[i] = row * LDK + col;
  }

  uint4 ra[A_CH], rb[B_CH];
  auto gload = [&](int kt) {
#pragma unroll
    for (int i = 0; i < A_CH; ++i)
      ra[i] = a_ok[i] ? *(const uint4*)(a_src[i] + kt * BK) : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < B_CH; ++i)
      rb[i] = b_ok[i] ? *(const uint4*)(b_src[i] + kt * BK) : make_uint4(0, 0, 0, 0);
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < A_CH; ++i) *(uint4*)&As[buf][a_dst[i]] = ra[i];
#pragma unroll
    for (int i = 0; i < B_CH; ++i) *(uint4*)&Bs[buf][b_dst[i]] = rb[i];
  };

  f32x4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (nk > 0) {
    gload(0);
    sstore(0);
  }
  __syncthreads();
  const int frag_row = lane & 15, frag_k = (lane >> 4) * 8;
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
#pragma unroll
    for (int ks = 0; ks < BK / 32; ++ks) {
      bf16x8 af[TM], bfg[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        af[i] = *(const bf16x8*)&As[buf][(wm * (BM / 2) + i * 16 + frag_row) * LDK + ks * 32 + frag_k];
#pragma unroll
      for (int j = 0; j < TN; ++j)
        bfg[j] = *(const bf16x8*)&Bs[buf][(wn * (BN / 2) + j * 16 + frag_row) * LDK + ks * 32 + frag_k];
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfg[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) sstore(buf ^ 1);
    __syncthreads();
  }

  // D layout of a 16x16 tile: lane holds column (lane & 15), rows 4*(lane >> 4) + r
  float* Y = a.Y + (size_t)z * a.y_split_stride;
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int n = n0 + wn * (BN / 2) + j * 16 + (lane & 15);
      if (n >= a.N) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + wm * (BM / 2) + i * 16 + (lane >> 4) * 4 + r;
        if (m >= a.M) continue;
        float* y = Y + (size_t)m * a.ldy + n;
        if (a.accumulate) *y = *y + acc[i][j][r];
        else *y = acc[i][j][r];
      }
    }
}

// fp32: 64x64 output tile, 256 threads each computing a 4x4 block, BK = 16.
__global__ __launch_bounds__(256) void gemm_f32_nt(GemmArgs a, int k_per_split) {
  constexpr int T = 64, KT = 16;
  __shared__ float As[KT][T + 1];
  __shared__ float Bs[KT][T + 1];
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;
  const int n0 = blockIdx.x * T, m0 = blockIdx.y * T, z = blockIdx.z;
  const int kbeg = z * k_per_split, kend = min(a.K, kbeg + k_per_split);
  float acc[4][4] = {};
  for (int k0 = kbeg; k0 < kend; k0 += KT) {
    for (int e = tid; e < T * KT; e += 256) {
      const int r = e / KT, kk = e % KT, k = k0 + kk;
      const int m = m0 + r, n = n0 + r;
      float xa = 0.f, wb = 0.f;
      if (m < a.M && k < kend) xa = ((const float*)a.X)[(size_t)x_row(a, m) * a.ldx + k];
      if (n < a.N && k < kend) wb = ((const float*)seg_row(a, n, 4))[k];
      As[kk][r] = xa;
      Bs[kk][r] = wb;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < KT; ++kk) {
      float xr[4], wr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) xr[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) wr[j] = Bs[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(xr[i], wr[j], acc[i][j]);
    }
    __syncthreads();
  }
  float* Y = a.Y + (size_t)z * a.y_split_stride;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int m = m0 + ty * 4 + i, n = n0 + tx * 4 + j;
      if (m < a.M && n < a.N) {
        float* y = Y + (size_t)m * a.ldy + n;
        if (a.accumulate) *y = *y + acc[i][j];
        else *y = acc[i][j];
      }
    }
}

}  // namespace

// Pick tile shape and K split.  Cost model (bytes-equivalent): weights once from
// HBM, X once per column tile (mostly from L2, weighted 1/4), fp32 partial
// slices written and read back (when split), scaled up when the grid is too
// small to keep ~2 workgroups on each of the 256 CUs.
GemmPlan gemm_plan(int M, int N, int K, int dtype, int force_splits) {
  GemmPlan best;
  if (dtype != 1) {   // fp32 VALU kernel
    best.bm = best.bn = 64;
    best.splits = 1;
    best.k_per_split = K;
    return best;
  }
  const int kb = K / BK;
  const int cand[4][2] = {{128, 128}, {128, 64}, {64, 128}, {64, 64}};
  double best_cost = 1e300;
  for (auto& c : cand) {
    const int bm = c[0], bn = c[1];
    const int mt = ceil_div(M, bm), nt = ceil_div(N, bn);
    for (int sp = 1; sp <= 32; ++sp) {
      if (force_splits && sp != force_splits) continue;
      const int kps_blocks = ceil_div(kb, sp);
      const int real_sp = ceil_div(kb, kps_blocks);
      if (real_sp != sp) continue;
      if (sp > 1 && kps_blocks < 4 && !force_splits) continue;
      const double w = 2.0 * N * K;
      const double x = 2.0 * (double)mt * bm * K * nt;                 // staged X bytes
      const double flops = 2.0 * (double)mt * bm * nt * bn * K;
      const double part = sp > 1 ? 8.0 * M * N * sp : 4.0 * M * N;
      const double wgs = (double)mt * nt * sp;
      const double fill = wgs >= 512 ? 1.0 : wgs / 512.0;
      const double mem = (w + 0.25 * x + part) / 8.0e12;
      const double cmp = flops / 1.2e15;                                  // ~half of dense peak
      const double cost = (mem > cmp ? mem : cmp) / fill;
      if (cost < best_cost * 0.999) {
        best_cost = cost;
        best.bm = bm;
        best.bn = bn;
        best.splits = sp;
        best.k_per_split = kps_blocks * BK;
      }
    }
  }
  if (best_cost == 1e300) {   // forced split count not representable: closest valid
    best.bm = 128;
    best.bn = 128;
    best.splits = 1;
    best.k_per_split = K;
  }
  return best;
}

size_t gemm_partial_elems(const GemmPlan& p, int M, int N) { return (size_t)p.splits * M * N; }

hipError_t launch_gemm(const GemmArgs& a, const GemmPlan& p, int dtype, hipStream_t s) {
  ProfScope ps("gemm", s);
  if (dtype != 1) {
    dim3 grid(ceil_div(a.N, 64), ceil_div(a.M, 64), p.splits);
    hipLaunchKernelGGL(gemm_f32_nt, grid, dim3(256), 0, s, a, p.k_per_split);
    return hipGetLastError();
  }
  dim3 grid(ceil_div(a.N, p.bn), ceil_div(a.M, p.bm), p.splits);
  if (p.bm == 128 && p.bn == 128)
    hipLaunchKernelGGL((gemm_bf16_nt<128, 128>), grid, dim3(256), 0, s, a, p.k_per_split);
  else if (p.bm == 128 && p.bn == 64)
    hipLaunchKernelGGL((gemm_bf16_nt<128, 64>), grid, dim3(256), 0, s, a, p.k_per_split);
  else if (p.bm == 64 && p.bn == 128)
    hipLaunchKernelGGL((gemm_bf16_nt<64, 128>), grid, dim3(256), 0, s, a, p.k_per_split);
  else
    hipLaunchKernelGGL((gemm_bf16_nt<64, 64>), grid, dim3(256), 0, s, a, p.k_per_split);
  return hipGetLastError();
}

}  // namespace dfs
