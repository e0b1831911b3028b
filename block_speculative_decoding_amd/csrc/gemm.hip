// Drafter GEMMs: Y = X . W^T with X [M, K] activations and W [N, K] weights
// ([out, in] storage, inputs contiguous), fp32 accumulation.
//
// bf16: one matrix-core kernel (v_mfma_f32_16x16x32_bf16) that streams W from
// HBM straight into MFMA operand registers while producer waves stage X tiles
// in LDS.  At the drafter's small M it reads W once and is bound by HBM; at
// M in the hundreds to thousands it runs 128 x 128 output tiles and is bound by
// the matrix cores.  K is split over workgroups (fp32 partial slices reduced by
// the consumer kernel) when there are too few output tiles to fill the chip.
//
// fp32: a plain LDS-tiled VALU kernel (the fp32 configuration is tiny).
#include "kernels.h"


namespace dfs {

namespace {

constexpr int BK = 64;
constexpr int LDK = BK + 8;   // padded LDS row (bf16 elements): 144 bytes
constexpr float kLog2eF = 1.4426950408889634f;

// columns of W: K, or wk when the K columns of X hold K / wk terms that all
// multiply the same W (GEMM column k uses W column k % wk)
__device__ __forceinline__ int w_cols(const GemmArgs& a) { return a.wk > 0 ? a.wk : a.K; }

__device__ __forceinline__ const void* seg_row(const GemmArgs& a, int n, int es) {
  int s = 0;
  if (a.nseg > 1 && n >= a.seg[1].n0) s = 1;
  if (a.nseg > 2 && n >= a.seg[2].n0) s = 2;
  return (const char*)a.seg[s].w + (size_t)(n - a.seg[s].n0) * w_cols(a) * es;
}

// first element of the packed 16-row tile group that holds logical W row n
constexpr int kTileElems = 16 * BK;   // one 16 x 64 tile (2 KB)
__device__ __forceinline__ const bf16_t* seg_tile(const GemmArgs& a, int n) {
  int s = 0;
  if (a.nseg > 1 && n >= a.seg[1].n0) s = 1;
  if (a.nseg > 2 && n >= a.seg[2].n0) s = 2;
  return (const bf16_t*)a.seg[s].w + (size_t)((n - a.seg[s].n0) >> 4) * (w_cols(a) / BK) * kTileElems;
}

__device__ __forceinline__ int x_row(const GemmArgs& a, int m) {
  if (!a.row_idx) return m;
  int r = a.row_idx[(size_t)m * a.row_idx_stride];
  return r < 0 ? 0 : (r >= a.x_rows ? a.x_rows - 1 : r);
}

// Weight-streaming kernel with producer/consumer waves.  A workgroup has 8 waves:
//   waves 4..7 (producers) stream the X tile (all BM rows x 64 k per step)
//     global -> registers -> LDS, XPD steps ahead;
//   waves 0..3 (consumers) stream their own 16*NW rows of W straight into MFMA
//     B-operand registers, PD steps ahead, and run the matrix-core math.
// Vector-memory counters are per wave and retire in order, so a wave that
// issued both operands would have to drain its deep W prefetch every time it
// waited for the (younger) X step; splitting the roles keeps every wave's
// waits on its own oldest loads only.  One barrier per k step; X is double
// buffered in LDS.
//
// Every load is unconditional (a predicated load becomes a branch, after which
// the compiler waits for everything): rows past M of X and past N of W read a
// valid row instead — output row m depends only on X row m and output column n
// only on W row n, and neither is stored — and steps past the end re-read the
// last step (cache hits) with the math skipped.
//
// Grid: 1-D over (m tile, n tile, k split), m tile fastest, remapped so that
// consecutive logical ids run on the same XCD (the hardware sends workgroup i
// to XCD i % 8): M tiles sharing one W slab then hit the same L2.
__device__ __forceinline__ int xcd_logical_id(int id, int total) {
  const int full = total & ~7;
  if (id >= full) return id;
  return (id & 7) * (full >> 3) + (id >> 3);
}

// Tile of a logical workgroup id: M tiles fastest, then N tiles, then K splits,
// over the computed tiles only.  The corner of the m_lo M tiles below skip_m
// and the n_lo N tiles left of skip_n is left out: the first n_lo N tiles have
// M tiles m_lo .. mtiles-1, the rest all mtiles (m_lo = 0 or n_lo = 0: every tile).
struct TileIdx {
  int m, n, z;
};
__device__ __forceinline__ TileIdx tile_of(int lid, int mtiles, int ntiles, int m_lo, int n_lo) {
  const int mq = mtiles - m_lo, corner = n_lo * mq;
  const int per = corner + (ntiles - n_lo) * mtiles;
  TileIdx t;
  t.z = lid / per;
  int r = lid - t.z * per;
  if (r < corner) {
    t.n = r / mq;
    t.m = m_lo + r % mq;
  } else {
    r -= corner;
    t.n = n_lo + r / mtiles;
    t.m = r % mtiles;
  }
  return t;
}

// GATED (NW = 2): the workgroup covers 64 output features; wave w streams the
// rows of features n0+16w .. +15 from W_gate (j = 0) and W_up (j = 1), so its
// epilogue holds gate and up of the same outputs and writes the SwiGLU product.
template <int MT, int NW, int PD, int XD, bool PACKED, bool GATED, int LB, int CW>
__global__ __launch_bounds__(64 * (CW + 4)) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gemm_stream_bf16(GemmArgs a, int k_per_split, int mtiles, int ntiles) {
  static_assert(CW == 3 || CW == 4, "consumer waves");
  static_assert(!GATED || NW == 2, "gated tiles pair gate and up");
  static_assert(LB == 8 || (LB == 4 && PD == 4), "loop body: 8 steps, or 4 (one turn of a 4-deep ring)");
  // W elements per k step and between the two 32-wide k halves of a step
  constexpr int WSTEP = PACKED ? kTileElems : BK, WKS = PACKED ? kTileElems / 2 : 32;
  // W offset of k step s of this split (relative to its first step): the
  // identity unless W is narrower than X (k wraps around W's columns)
  static_assert(PD == 4 || PD == 8, "ring depth divides the 8-step loop body");
  static_assert(XD == 2 || XD == PD, "X ring depth");
  constexpr int BM = 16 * MT, BN = GATED ? 16 * CW : 16 * CW * NW;
  constexpr int XCH = BM * BK / 8 / 256;                // 16-byte X chunks per producer lane per step
  static_assert(XCH >= 1, "tile too small");
  __shared__ __attribute__((aligned(16))) bf16_t Xs[2][BM * LDK];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const bool producer = wave >= CW;
  const int lid = xcd_logical_id(blockIdx.x, gridDim.x);
  const TileIdx tix = tile_of(lid, mtiles, ntiles, GATED ? 0 : min(a.skip_m / BM, mtiles),
                              GATED ? 0 : min(a.skip_n / BN, ntiles));
  const int n0 = tix.n * BN, m0 = tix.m * BM, z = tix.z;
  const int kbeg = z * k_per_split;
  const int kend = min(a.K, kbeg + k_per_split);
  const int nk = kend > kbeg ? (kend - kbeg) / BK : 0;
  if (nk == 0) return;                                   // uniform over the workgroup
  const int c = lane & 15, g4 = lane >> 4;
  const int kb0 = kbeg / BK, wsteps = w_cols(a) / BK;
  auto wofs = [&](int st) -> ptrdiff_t { return (ptrdiff_t)((kb0 + st) % wsteps - kb0) * WSTEP; };

  // producer state: X rows of this tile
  const bf16_t* x_src[XCH];
  int x_dst[XCH];
  // consumer state: W rows of this wave
  const bf16_t* w_src[NW];
  if (producer) {
    const int ptid = tid - 64 * CW;
#pragma unroll
    for (int i = 0; i < XCH; ++i) {
      const int ch = ptid + i * 256, row = ch >> 3, col = (ch & 7) * 8, m = min(m0 + row, a.M - 1);
      x_src[i] = (const bf16_t*)a.X + (size_t)x_row(a, m) * a.ldx + kbeg + col;
      x_dst[i] = row * LDK + col;
    }
  } else {
#pragma unroll
    for (int j = 0; j < NW; ++j) {
      if constexpr (GATED) {
        const int n = min(n0 + wave * 16 + c, a.N - 1);
        const bf16_t* w = (const bf16_t*)a.seg[j].w;
        if constexpr (PACKED)
          w_src[j] = w + ((size_t)(n >> 4) * (w_cols(a) / BK) + kbeg / BK) * kTileElems + lane * 8;
        else
          w_src[j] = w + (size_t)n * w_cols(a) + kbeg + g4 * 8;
      } else {
        const int n = min(n0 + wave * 16 * NW + j * 16 + c, a.N - 1);
        if constexpr (PACKED)   // the wave's 16 rows: one contiguous run of tiles
          w_src[j] = seg_tile(a, n) + (size_t)(kbeg / BK) * kTileElems + lane * 8;
        else
          w_src[j] = (const bf16_t*)seg_row(a, n, 2) + kbeg + g4 * 8;
      }
    }
  }

  // The two roles run separate loops with the same barrier sequence (one per k
  // step).  Steps are expanded by macro so every ring index is a constant.
  if (producer) {
    // X comes from L2, but behind the consumers' HBM misses in the same memory
    // pipeline, so it is prefetched XD steps ahead (XD = 2 or the W depth).
    uint4 xr[XD][XCH];
#pragma unroll
    for (int st = 0; st < XD; ++st) {
#pragma unroll
      for (int i = 0; i < XCH; ++i) xr[st][i] = ldg16(x_src[i] + min(st, nk - 1) * BK);
      __builtin_amdgcn_sched_barrier(0);   // oldest-first, as in the consumers
    }
#define DFS_PRODUCER_STEP(ST)                                                  \
  {                                                                            \
    const int kt = kb + ST;                                                    \
    {                                                                          \
      bf16_t* xs = Xs[ST & 1];                                                 \
      _Pragma("unroll") for (int i = 0; i < XCH; ++i) *(uint4*)&xs[x_dst[i]] = xr[ST % XD][i]; \
      __syncthreads();                                                         \
    }                                                                          \
    const int kk = min(kt + XD, nk - 1) * BK;                                  \
    _Pragma("unroll") for (int i = 0; i < XCH; ++i) xr[ST % XD][i] = ldg16(x_src[i] + kk);    \
  }
    // as many steps per iteration as the consumers run (same barrier sequence)
    for (int kb = 0; kb < nk; kb += LB) {
      DFS_PRODUCER_STEP(0)
      DFS_PRODUCER_STEP(1)
      DFS_PRODUCER_STEP(2)
      DFS_PRODUCER_STEP(3)
      if constexpr (LB == 8) {
        DFS_PRODUCER_STEP(4)
        DFS_PRODUCER_STEP(5)
        DFS_PRODUCER_STEP(6)
        DFS_PRODUCER_STEP(7)
      }
    }
#undef DFS_PRODUCER_STEP
    return;
  }

  f32x4 acc[MT][NW];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NW; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  bf16x8 wr[PD][NW][2];
#pragma unroll
  for (int st = 0; st < PD; ++st) {
#pragma unroll
    for (int j = 0; j < NW; ++j)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        wr[st][j][ks] = ldg_bf16x8(w_src[j] + wofs(min(st, nk - 1)) + ks * WKS);
    // keep the ring filled oldest-first: the loop's wait counts assume step 0
    // holds the oldest loads, also on entry
    __builtin_amdgcn_sched_barrier(0);
  }
#define DFS_CONSUMER_STEP(ST, R)                                                               \
  {                                                                                            \
    const int kt = kb + ST;                                                                    \
    __syncthreads();                                                                           \
    if (kt < nk) {                                                                             \
      const bf16_t* xs = Xs[ST & 1];                                                           \
      _Pragma("unroll") for (int ks = 0; ks < 2; ++ks) {                                       \
        bf16x8 bfg[NW];                                                                        \
        _Pragma("unroll") for (int j = 0; j < NW; ++j) bfg[j] = wr[R][j][ks];                 \
        _Pragma("unroll") for (int i = 0; i < MT; ++i) {                                       \
          const bf16x8 af = *(const bf16x8*)&xs[(i * 16 + c) * LDK + ks * 32 + g4 * 8];          \
          _Pragma("unroll") for (int j = 0; j < NW; ++j)                                       \
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bfg[j], af, acc[i][j], 0, 0, 0);   \
        }                                                                                      \
      }                                                                                        \
    }                                                                                          \
    __builtin_amdgcn_sched_barrier(0); /* keep the refill after this step's math */            \
    const ptrdiff_t kk = wofs(min(kt + PD, nk - 1));                                         \
    _Pragma("unroll") for (int j = 0; j < NW; ++j)                                             \
      _Pragma("unroll") for (int ks = 0; ks < 2; ++ks) wr[R][j][ks] = ldg_bf16x8(w_src[j] + kk + ks * WKS); \
  }
  // 8 steps (two turns of a 4-deep ring, one turn of an 8-deep one) per loop
  // iteration: the wait-count analysis is conservative across the loop back
  // edge, so cross it less often; a split whose step count is not a multiple
  // of 8 runs 4-step bodies instead (fewer idle steps past its end)
  for (int kb = 0; kb < nk; kb += LB) {
    DFS_CONSUMER_STEP(0, 0)
    DFS_CONSUMER_STEP(1, 1)
    DFS_CONSUMER_STEP(2, 2)
    DFS_CONSUMER_STEP(3, 3)
    if constexpr (LB == 8) {
      DFS_CONSUMER_STEP(4, 4 % PD)
      DFS_CONSUMER_STEP(5, 5 % PD)
      DFS_CONSUMER_STEP(6, 6 % PD)
      DFS_CONSUMER_STEP(7, 7 % PD)
    }
  }
#undef DFS_CONSUMER_STEP

  // W is the A operand and X the B operand, so each 16x16 tile comes out
  // transposed: lane (c, g4) holds output row m = c and the four consecutive
  // columns n = 4*g4 .. 4*g4+3 — one 16-byte store per tile and lane.
  if constexpr (GATED) {
    // h = bf16(silu(gate) * up) for features n .. n+3 of row m (one 8-byte store)
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      const int m = m0 + i * 16 + c, n = n0 + wave * 16 + g4 * 4;
      if (m >= a.M) continue;
      bf16_t* hrow = (bf16_t*)a.hout + (size_t)m * a.ldy;
      bf16_t h[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float g = acc[i][0][e], u = acc[i][1][e];
        h[e] = f2bf(g / (1.f + expf(-g)) * u);
      }
      bf16_t* dst = a.h_packed ? (bf16_t*)a.hout + xpk_index(m, n, a.N) : hrow + n;
      if (n + 3 < a.N) {
        *(uint2*)dst = make_uint2((uint32_t)h[0] | ((uint32_t)h[1] << 16), (uint32_t)h[2] | ((uint32_t)h[3] << 16));
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (n + e < a.N) dst[e] = h[e];
      }
    }
    return;
  }
  float* Y = a.Y + (size_t)z * a.y_split_stride;
  const bool vec = (a.ldy & 3) == 0 && ((uintptr_t)Y & 15) == 0;
#pragma unroll
  for (int i = 0; i < MT; ++i) {
    const int m = m0 + i * 16 + c;
    if (m >= a.M) continue;
    float* yrow = Y + (size_t)m * a.ldy;
#pragma unroll
    for (int j = 0; j < NW; ++j) {
      const int n = n0 + wave * 16 * NW + j * 16 + g4 * 4;
      if (vec && n + 3 < a.N) {
        f32x4 v = acc[i][j];
        if (a.accumulate) v += *(const f32x4*)(yrow + n);
        if (a.nt_store) __builtin_nontemporal_store(v, (f32x4*)(yrow + n));
        else *(f32x4*)(yrow + n) = v;
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if (n + r >= a.N) break;
          if (a.accumulate) yrow[n + r] += acc[i][j][r];
          else yrow[n + r] = acc[i][j][r];
        }
      }
    }
  }
}

// Matrix-core-bound GEMM for M in the hundreds to thousands: a BM x BN output
// tile per 512-thread workgroup (8 waves, 2 along M x 4 along N, all of them
// loading and multiplying).  K is walked in half steps of 32 through a ring of
// NS LDS stages filled by direct global->LDS loads (global_load_lds_dwordx4:
// each lane's 16 bytes land at lane*16 of a wave-uniform LDS address), issued
// NS-1 half steps ahead, so no registers hold operands in flight.
// A stage holds each operand in matrix-core fragment order: 16-row groups of
// 1 KB, lane l's 16 bytes being row l % 16, k 8*(l/16) .. +7 of the half step —
// one half of a tile-packed weight tile, copied verbatim; a row-major operand
// is gathered into it by per-lane addresses.  Every fragment read is one
// linear, conflict-free 16-byte LDS read per lane.
// Synchronisation per half step: each wave waits for its own loads of the
// stage (vmcnt counts them in issue order: (NS-2) half steps of younger loads
// may stay in flight), then a workgroup barrier; the stage read NS-1 half
// steps later is refilled only after that barrier.  The stages are distinct
// LDS arrays so that the compiler's own load/LDS-read ordering does not
// serialise the ring.
// W is the A operand (16 output columns) and X the B operand (16 rows), so a
// lane's result is 4 consecutive columns of one row, stored as one 16-byte
// vector as in the streaming kernel.
// GATED: the tile covers BN/2 features; each wave's BN/4 W rows are the gate
// rows of its BN/8 features followed by their up rows, so its epilogue holds
// gate and up of the same outputs and writes bf16(silu(gate) * up).
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

template <int BM, int BN, bool PACKED, bool GATED>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gemm_tile_bf16(GemmArgs a, int k_per_split, int mtiles, int ntiles) {
  constexpr int NS = 4;                                 // LDS ring depth (half steps)
  constexpr int NA = BN / 64, MB = BM / 32;             // 16-wide W / X fragments per wave
  constexpr int GW = BN / 16, GX = BM / 16;             // 1 KB units per half step
  constexpr int UPS = (GW + GX) / 8;                    // units per wave per half step
  constexpr int SE = (BN + BM) * 32;                    // stage size (bf16 elements)
  static_assert((GW % 8) == 0 && (GX % 8) == 0, "units split evenly over the waves");
  static_assert(!GATED || NA % 2 == 0, "gated tiles pair gate and up fragments");
  // a wave's vmcnt wait before reading a stage: younger half steps still in flight
  constexpr int kWait = (NS - 2) * UPS;
  static_assert(kWait < 16, "wait count fits the low vmcnt field");
  __shared__ __attribute__((aligned(1024))) bf16_t S0[SE];
  __shared__ __attribute__((aligned(1024))) bf16_t S1[SE];
  __shared__ __attribute__((aligned(1024))) bf16_t S2[SE];
  __shared__ __attribute__((aligned(1024))) bf16_t S3[SE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 2, wn = wave & 3;
  const int c = lane & 15, g4 = lane >> 4;
  const int lid = xcd_logical_id(blockIdx.x, gridDim.x);
  const TileIdx tix = tile_of(lid, mtiles, ntiles, GATED ? 0 : min(a.skip_m / BM, mtiles),
                              GATED ? 0 : min(a.skip_n / BN, ntiles));
  const int ntile = tix.n, z = tix.z;
  const int m0 = tix.m * BM;
  const int kbeg = z * k_per_split;
  const int kend = min(a.K, kbeg + k_per_split);
  const int nh = kend > kbeg ? (kend - kbeg) / 32 : 0;  // half steps
  if (nh == 0) return;                                   // uniform over the workgroup

  // Unit u = wave + 8*i of a half step: u < GW is W row group u, else X row
  // group u - GW.  src[i] is the lane's address at half step 0; hstep[i] the
  // advance per half step (elements); dsto[i] the unit's offset in a stage.
  const bf16_t* src[UPS];
  int dsto[UPS];
  int hstep[UPS];
#pragma unroll
  for (int i = 0; i < UPS; ++i) {
    const int u = wave + 8 * i;
    if (i < GW / 8) {
      const int g = u;
      if constexpr (GATED) {
        const int wg = g / NA, jj = g % NA;
        const int f = min(ntile * (BN / 2) + wg * (NA / 2) * 16 + (jj % (NA / 2)) * 16, (a.N - 1) & ~15);
        const bf16_t* w = (const bf16_t*)a.seg[jj < NA / 2 ? 0 : 1].w;
        if constexpr (PACKED)
          src[i] = w + ((size_t)(f >> 4) * (a.K / BK) + kbeg / BK) * kTileElems + lane * 8;
        else
          src[i] = w + (size_t)min(f + c, a.N - 1) * a.K + kbeg + g4 * 8;
      } else {
        const int n = min(ntile * BN + g * 16, (a.N - 1) & ~15);
        if constexpr (PACKED)
          src[i] = seg_tile(a, n) + (size_t)(kbeg / BK) * kTileElems + lane * 8;
        else
          src[i] = (const bf16_t*)seg_row(a, min(n + c, a.N - 1), 2) + kbeg + g4 * 8;
      }
      dsto[i] = g * 512;
      hstep[i] = PACKED ? kTileElems / 2 : 32;
    } else {
      const int g = u - GW;
      if (a.x_packed) {   // the 16-row group's tiles: one contiguous kilobyte per half step
        const int mg = min((m0 >> 4) + g, (a.M - 1) >> 4);
        src[i] = (const bf16_t*)a.X + ((size_t)mg * (a.K / BK) + kbeg / BK) * kTileElems + lane * 8;
        hstep[i] = kTileElems / 2;
      } else {
        const int m = min(m0 + g * 16 + c, a.M - 1);
        src[i] = (const bf16_t*)a.X + (size_t)x_row(a, m) * a.ldx + kbeg + g4 * 8;
        hstep[i] = 32;
      }
      dsto[i] = BN * 32 + g * 512;
    }
  }
  // a packed operand's half step h (of tile h/2) sits at h/2 * kTileElems + (h%2) * 512 = h * 512
  auto src_at = [&](int i, int h) -> const bf16_t* {
    if (PACKED && i < GW / 8) return src[i] + (size_t)h * (kTileElems / 2);
    return src[i] + (size_t)h * hstep[i];
  };
  auto fill = [&](bf16_t* stage, int h) {
    const int hh = min(h, nh - 1);                       // past the end: reload the last (unused)
#pragma unroll
    for (int i = 0; i < UPS; ++i)
      __builtin_amdgcn_global_load_lds((glb_void_t*)src_at(i, hh), (lds_void_t*)(stage + dsto[i]), 16, 0, 0);
  };

  f32x4 acc[NA][MB];
#pragma unroll
  for (int j = 0; j < NA; ++j)
#pragma unroll
    for (int i = 0; i < MB; ++i) acc[j][i] = f32x4{0.f, 0.f, 0.f, 0.f};

  fill(S0, 0);
  fill(S1, 1);
  fill(S2, 2);
#define DFS_TILE_STEP(CUR, NXT, H)                                                            \
  {                                                                                           \
    __builtin_amdgcn_s_waitcnt(0x0070 | kWait); /* own loads of stage H done; lgkm drained */ \
    __atomic_signal_fence(__ATOMIC_SEQ_CST);                                                  \
    __builtin_amdgcn_s_barrier();                                                             \
    __atomic_signal_fence(__ATOMIC_SEQ_CST);                                                  \
    fill(NXT, (H) + NS - 1);                                                                  \
    if ((H) < nh) {                                                                           \
      const bf16_t* ws = CUR + wn * NA * 512 + lane * 8;                                      \
      const bf16_t* xs = CUR + BN * 32 + wm * MB * 512 + lane * 8;                            \
      bf16x8 af[NA], bx[MB];                                                                  \
      _Pragma("unroll") for (int j = 0; j < NA; ++j) af[j] = *(const bf16x8*)(ws + j * 512);  \
      _Pragma("unroll") for (int i = 0; i < MB; ++i) bx[i] = *(const bf16x8*)(xs + i * 512);  \
      _Pragma("unroll") for (int i = 0; i < MB; ++i)                                          \
        _Pragma("unroll") for (int j = 0; j < NA; ++j)                                        \
          acc[j][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[j], bx[i], acc[j][i], 0, 0, 0); \
    }                                                                                         \
  }
  for (int h = 0; h < nh; h += NS) {
    DFS_TILE_STEP(S0, S3, h)
    DFS_TILE_STEP(S1, S0, h + 1)
    DFS_TILE_STEP(S2, S1, h + 2)
    DFS_TILE_STEP(S3, S2, h + 3)
  }
#undef DFS_TILE_STEP
  // drain the ring's trailing (unused) loads before the workgroup can exit
  __builtin_amdgcn_s_waitcnt(0x0070);

  if constexpr (GATED) {
    // h = bf16(silu(gate) * up) for features f .. f+3 of row m (one 8-byte store)
    constexpr int per = NA * 16 / 2;
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      const int m = m0 + (wm * MB + i) * 16 + c;
      if (m >= a.M) continue;
      bf16_t* hrow = (bf16_t*)a.hout + (size_t)m * a.ldy;
#pragma unroll
      for (int j = 0; j < NA / 2; ++j) {
        const int f = ntile * (BN / 2) + wn * per + j * 16 + g4 * 4;
        bf16_t hv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float g = acc[j][i][e], u = acc[j + NA / 2][i][e];
          hv[e] = f2bf(g / (1.f + expf(-g)) * u);
        }
        bf16_t* dst = a.h_packed ? (bf16_t*)a.hout + xpk_index(m, f, a.N) : hrow + f;
        if (f + 3 < a.N) {
          *(uint2*)dst =
              make_uint2((uint32_t)hv[0] | ((uint32_t)hv[1] << 16), (uint32_t)hv[2] | ((uint32_t)hv[3] << 16));
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (f + e < a.N) dst[e] = hv[e];
        }
      }
    }
    return;
  }
  float* Y = a.Y + (size_t)z * a.y_split_stride;
  const bool vec = (a.ldy & 3) == 0 && ((uintptr_t)Y & 15) == 0;
#pragma unroll
  for (int i = 0; i < MB; ++i) {
    const int m = m0 + (wm * MB + i) * 16 + c;
    if (m >= a.M) continue;
    float* yrow = Y + (size_t)m * a.ldy;
#pragma unroll
    for (int j = 0; j < NA; ++j) {
      const int n = ntile * BN + (wn * NA + j) * 16 + g4 * 4;
      if (vec && n + 3 < a.N) {
        f32x4 v = acc[j][i];
        if (a.accumulate) v += *(const f32x4*)(yrow + n);
        if (a.nt_store) __builtin_nontemporal_store(v, (f32x4*)(yrow + n));
        else *(f32x4*)(yrow + n) = v;
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if (n + r >= a.N) break;
          if (a.accumulate) yrow[n + r] += acc[j][i][r];
          else yrow[n + r] = acc[j][i][r];
        }
      }
    }
  }
}

// Short-K GEMM (K = 256, M <= 16*MT; the sequential head's per-position
// product at batches up to 128): a persistent grid where each workgroup stages all
// of X (M x 256, at most 64 KB) in LDS once, then each wave walks W row groups
// g, g + (waves in the grid), ...: one 8 KB contiguous load of the group's 16 W
// rows (packed) and of the Y values it accumulates into, issued one group
// ahead (two register buffers, unconditional loads: past the end the last group
// is re-read), 8*MT matrix-core products against X fragments from LDS, a
// 16-byte store per row.  No barrier after the X staging; nothing is re-read
// per k step.  Requires N % 4 == 0 and a 16-byte aligned Y with ldy % 4 == 0.
// T = 3: X holds three K = 256 terms side by side (wk = 256, the RNN head's state
// split hi | mid | lo); each W group is loaded once and multiplies all three.
template <int MT, bool PACKED, int T>
__global__ __launch_bounds__(256) void gemm_short_bf16(GemmArgs a) {
  constexpr int K = 4 * BK, KX = T * K, LDX = KX + 8;
  __shared__ __attribute__((aligned(16))) bf16_t Xs[16 * MT * LDX];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, c = lane & 15, g4 = lane >> 4;
  // X rows 0 .. 16*MT-1 (rows past M repeat row M-1; their results are not stored)
  for (int ch = tid; ch < 16 * MT * (KX / 8); ch += 256) {
    const int row = ch / (KX / 8), col = (ch % (KX / 8)) * 8;
    const int m = min(row, a.M - 1);
    *(uint4*)&Xs[row * LDX + col] = ldg16((const bf16_t*)a.X + (size_t)x_row(a, m) * a.ldx + col);
  }
  __syncthreads();
  const int ng = ceil_div(a.N, 16), tw = gridDim.x * 4;
  int g = blockIdx.x * 4 + wave;
  if (g >= ng) return;                                   // uniform over the wave; no barrier follows
  bf16x8 wf[2][8];
  f32x4 yv[2][MT];
  auto load = [&](int buf, int gg) {
    gg = min(gg, ng - 1);
    const int n0 = gg * 16;
    const bf16_t* w = PACKED ? (const bf16_t*)a.seg[0].w + (size_t)gg * 4 * kTileElems + lane * 8
                             : (const bf16_t*)a.seg[0].w + (size_t)min(n0 + c, a.N - 1) * K + g4 * 8;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        bf16x8 v = ldg_bf16x8(w + (PACKED ? (size_t)kt * kTileElems + h * 512 : (size_t)kt * BK + h * 32));
        if (buf == 0) wf[0][2 * kt + h] = v;
        else wf[1][2 * kt + h] = v;
      }
    const int n = min(n0 + 4 * g4, a.N - 4);
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      f32x4 y = f32x4{0.f, 0.f, 0.f, 0.f};
      if (a.accumulate) y = *(const f32x4*)(a.Y + (size_t)min(i * 16 + c, a.M - 1) * a.ldy + n);
      if (buf == 0) yv[0][i] = y;
      else yv[1][i] = y;
    }
  };
  auto compute_store = [&](int buf, int gg) {
    f32x4 acc[MT];
#pragma unroll
    for (int i = 0; i < MT; ++i) acc[i] = buf == 0 ? yv[0][i] : yv[1][i];
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const bf16x8 wa = buf == 0 ? wf[0][2 * kt + h] : wf[1][2 * kt + h];
#pragma unroll
          for (int i = 0; i < MT; ++i)
            acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                wa, *(const bf16x8*)&Xs[(i * 16 + c) * LDX + t * K + kt * BK + h * 32 + g4 * 8], acc[i], 0, 0, 0);
        }
    const int n = gg * 16 + 4 * g4;
    if (n >= a.N) return;
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      const int m = i * 16 + c;
      if (m < a.M) *(f32x4*)(a.Y + (size_t)m * a.ldy + n) = acc[i];
    }
  };
  load(0, g);
  while (true) {
    load(1, g + tw);
    compute_store(0, g);
    g += tw;
    if (g >= ng) break;
    load(0, g + tw);
    compute_store(1, g);
    g += tw;
    if (g >= ng) break;
  }
}

// The Markov head's per-position product with its sampling statistics in the
// epilogue (K = 256, M <= 128, one term): final = base + X . W^T written over
// the base logits, and for every row and 64-column sub-chunk of the output the
// sub-chunk's max and sum exp2((x - max) * k) (k = log2(e) / T, fp32
// exponentials summed in fp64), or for T == 0 (max, first column of the max).
// One workgroup per (pair of sub-chunks, chunk of 32 rows), one wave per
// 16-column W row group (waves 0-3 the first sub-chunk, 4-7 the second): each
// wave issues its whole group (8 KB of W, the base rows) before the X rows are
// staged in LDS — once for both sub-chunks, half the gathered-row traffic of one
// workgroup per sub-chunk — so a wave makes one memory round trip (about 60
// VGPRs a wave: at 32 rows the whole grid is resident at once).  The four waves
// of a sub-chunk combine its max, then its sum, through LDS.  The logits are read
// once and written once; no separate statistics pass re-reads them.
// sub[m * nsub + j] = (max, sum | first column).  The row chunks of a sub-chunk
// pair take consecutive logical ids, which the XCD remap puts on one XCD, so its
// W slab comes from HBM once and from that L2 after.
template <bool PACKED>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(8, 8)))
void head_gemm_stats_bf16(GemmArgs a, float T, double2* sub, int nsub, int nrc) {
  constexpr int K = 4 * BK, LDX = K + 8, MT = 2, R = 16 * MT;
  __shared__ __attribute__((aligned(16))) bf16_t Xs[R * LDX];
  __shared__ float smax[8][R];
  __shared__ double ssum[8][R];
  __shared__ int sfirst[8][R];
  const int tid = threadIdx.x, lane = tid & 63, wave8 = tid >> 6, c = lane & 15, g4 = lane >> 4;
  const int lid = nrc > 1 ? xcd_logical_id(blockIdx.x, gridDim.x) : blockIdx.x;
  const int hs = wave8 >> 2, wave = wave8 & 3;           // sub-chunk of the pair, wave in it
  const int u = 2 * (lid / nrc) + hs, m0 = (lid % nrc) * R, ng = ceil_div(a.N, 16);
  const int mr = a.M - m0;                               // rows of this chunk: min(mr, R)
  const int gw = 4 * u + wave;                           // this wave's W row group
  const bool live = gw < ng;                             // uniform over the wave
  const int g = min(gw, ng - 1);                         // past the end: the last group, nothing stored
  bf16x8 wf[8];
  {
    const bf16_t* w = PACKED ? (const bf16_t*)a.seg[0].w + (size_t)g * 4 * kTileElems + lane * 8
                             : (const bf16_t*)a.seg[0].w + (size_t)min(g * 16 + c, a.N - 1) * K + g4 * 8;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        wf[2 * kt + h] = ldg_bf16x8(w + (PACKED ? (size_t)kt * kTileElems + h * 512 : (size_t)kt * BK + h * 32));
  }
  f32x4 acc[MT];
  const int n = g * 16 + 4 * g4;                         // this lane's 4 columns (N % 4 == 0)
#pragma unroll
  for (int i = 0; i < MT; ++i)
    acc[i] = *(const f32x4*)(a.Y + (size_t)(m0 + min(i * 16 + c, mr - 1)) * a.ldy + min(n, a.N - 4));
  // X rows m0 .. m0+R-1 (rows past M repeat row M-1; their results are not stored)
  for (int ch = tid; ch < R * (K / 8); ch += 512) {
    const int row = ch / (K / 8), col = (ch % (K / 8)) * 8;
    const int m = m0 + min(row, mr - 1);
    *(uint4*)&Xs[row * LDX + col] = ldg16((const bf16_t*)a.X + (size_t)x_row(a, m) * a.ldx + col);
  }
  __syncthreads();
#pragma unroll
  for (int kt = 0; kt < 4; ++kt)
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < MT; ++i)
        acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            wf[2 * kt + h], *(const bf16x8*)&Xs[(i * 16 + c) * LDX + kt * BK + h * 32 + g4 * 8], acc[i], 0, 0, 0);
  const bool cols = live && n < a.N;                     // lane (c, g4) holds row 16 i + c, columns n .. n+3
#pragma unroll
  for (int i = 0; i < MT; ++i)
    if (cols && i * 16 + c < mr) *(f32x4*)(a.Y + (size_t)(m0 + i * 16 + c) * a.ldy + n) = acc[i];
  // the sub-chunk's max: over the 4 lanes g4 of a row, then over the 4 waves
#pragma unroll
  for (int i = 0; i < MT; ++i) {
    float mx = -INFINITY;
    if (cols)
#pragma unroll
      for (int e = 0; e < 4; ++e) mx = fmaxf(mx, acc[i][e]);
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    if (g4 == 0) smax[wave8][i * 16 + c] = mx;
  }
  __syncthreads();
  const float kk = T > 0.f ? kLog2eF / T : 0.f;
#pragma unroll
  for (int i = 0; i < MT; ++i) {
    const int row = i * 16 + c;
    const float mx = fmaxf(fmaxf(smax[4 * hs][row], smax[4 * hs + 1][row]), fmaxf(smax[4 * hs + 2][row], smax[4 * hs + 3][row]));
    if (T > 0.f) {
      double sl = 0.0;
      if (cols && mx != -INFINITY)
#pragma unroll
        for (int e = 0; e < 4; ++e) sl += (double)exp2f((acc[i][e] - mx) * kk);
      sl += __shfl_xor(sl, 16, 64);                      // g4 pairs (0,1), (2,3), then the two pairs
      sl += __shfl_xor(sl, 32, 64);
      if (g4 == 0) ssum[wave8][row] = sl;
    } else {
      int first = 0x7fffffff;
      if (cols)
#pragma unroll
        for (int e = 3; e >= 0; --e)
          if (acc[i][e] == mx) first = n + e;
      first = min(first, __shfl_xor(first, 16, 64));
      first = min(first, __shfl_xor(first, 32, 64));
      if (g4 == 0) sfirst[wave8][row] = first;
    }
  }
  __syncthreads();
  const int th = tid & 63, o = 4 * hs;                   // lanes of wave 0 (sub-chunk 0) and wave 4 (sub-chunk 1)
  if (wave == 0 && th < R && th < mr && u < nsub) {
    const float mx = fmaxf(fmaxf(smax[o][th], smax[o + 1][th]), fmaxf(smax[o + 2][th], smax[o + 3][th]));
    double r;
    if (T > 0.f) {
      r = (ssum[o][th] + ssum[o + 1][th]) + (ssum[o + 2][th] + ssum[o + 3][th]);
    } else {
      const int f = min(min(sfirst[o][th], sfirst[o + 1][th]), min(sfirst[o + 2][th], sfirst[o + 3][th]));
      r = f == 0x7fffffff ? -1.0 : (double)f;
    }
    sub[(size_t)(m0 + th) * nsub + u] = make_double2((double)mx, r);
  }
}

// Small-M GEMM (M <= 16 rows, K <= 512; the Markov head's per-position
// U[prev] . W product): every wave is independent — it owns 16 W rows, loads
// all their K at once (8 KB contiguous in the packed layout at K = 256), the
// rows it accumulates into and the few X rows (from L1/L2, as matrix-core
// fragments), then multiplies: one memory round trip per wave, no LDS, no
// barrier.  NKM = the largest K/64 the instance serves (4 or 8): at K <= 256
// few registers, so the whole grid of a 129280-row W is resident at once.
template <bool PACKED, int NKM>
__global__ __launch_bounds__(256) void gemm_rows_bf16(GemmArgs a) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int ng = blockIdx.x * 4 + wave;                  // 16-row group of W
  if (ng * 16 >= a.N) return;                            // uniform over the wave
  const int c = lane & 15, g4 = lane >> 4;
  const int nk = a.K / BK, wsteps = w_cols(a) / BK;     // 1 .. NKM
  const int n0 = ng * 16, n = n0 + 4 * g4;
  const bf16_t* wsrc = PACKED ? seg_tile(a, n0) + lane * 8
                              : (const bf16_t*)seg_row(a, min(n0 + c, a.N - 1), 2) + g4 * 8;
  bf16x8 wf[2 * NKM];
#pragma unroll
  for (int kt = 0; kt < NKM; ++kt) {
    if (kt >= nk) break;                                 // uniform
#pragma unroll
    for (int h = 0; h < 2; ++h)
      wf[2 * kt + h] = ldg_bf16x8(wsrc + (PACKED ? (size_t)(kt % wsteps) * kTileElems + h * 512
                                                 : (size_t)(kt % wsteps) * BK + h * 32));
  }
  // lane (c, g4) owns row m = c, columns n .. n+3; the values it adds to are
  // loaded in the same round trip as the operands
  const bool vec = (a.ldy & 3) == 0 && ((uintptr_t)a.Y & 15) == 0 && n + 3 < a.N;
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  if (a.accumulate && vec && c < a.M) acc = *(const f32x4*)(a.Y + (size_t)c * a.ldy + n);
  const bf16_t* xrow = (const bf16_t*)a.X + (size_t)x_row(a, min(c, a.M - 1)) * a.ldx + g4 * 8;
#pragma unroll
  for (int kt = 0; kt < NKM; ++kt) {
    if (kt >= nk) break;                                 // uniform
#pragma unroll
    for (int h = 0; h < 2; ++h)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[2 * kt + h], ldg_bf16x8(xrow + kt * BK + h * 32), acc, 0, 0, 0);
  }
  if (c >= a.M) return;
  float* yrow = a.Y + (size_t)c * a.ldy;
  if (vec) {
    *(f32x4*)(yrow + n) = acc;                           // includes the accumulated values
  } else {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (n + r >= a.N) break;
      if (a.accumulate) yrow[n + r] += acc[r];
      else yrow[n + r] = acc[r];
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

// Reorders a row-major bf16 [N, K] matrix into the tile-packed layout; one
// thread per 16-byte chunk of the output (grid-stride), rows past N zero.
__global__ __launch_bounds__(256) void pack_kernel(const bf16_t* __restrict__ src, bf16_t* __restrict__ dst, int N,
                                                   int K) {
  const int kb = K / BK;
  const size_t chunks = (size_t)ceil_div(N, 16) * 16 * K / 8;
  for (size_t c = (size_t)blockIdx.x * 256 + threadIdx.x; c < chunks; c += (size_t)gridDim.x * 256) {
    const size_t tile = c >> 7;
    const int q = (int)(c & 127), l = q & 63;
    const size_t nt = tile / kb;
    const int kt = (int)(tile % kb);
    const size_t row = nt * 16 + (l & 15);
    const int col = kt * BK + (q >> 6) * 32 + (l >> 4) * 8;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (row < (size_t)N) v = ldg16(src + row * K + col);
    *(uint4*)(dst + c * 8) = v;
  }
}

}  // namespace

// Kernel configurations the planner chooses from: weight streaming (kind 1)
// with BM = 16*MT rows and BN = 64*NW columns per workgroup, and the
// LDS-ring tile kernel (kind 3, 256 x 256) for M > 256.
struct Cand {
  int kind, bm, bn, mt, nw;
};
static const Cand kCands[] = {
    {1, 128, 128, 8, 2}, {1, 128, 64, 8, 1}, {1, 64, 128, 4, 2}, {1, 64, 64, 4, 1},
    {1, 32, 128, 2, 2},  {1, 32, 64, 2, 1},  {1, 256, 64, 16, 1}, {3, 256, 256, 0, 0},
    {1, 128, 96, 8, 2},  {1, 64, 96, 4, 2},   // 3 consumer waves: 96 columns per workgroup
    {1, 160, 128, 10, 2}, {1, 160, 96, 10, 2},  // 160-row tiles: M in (128, 160] in one M tile
};

// Cost model, two regimes.
// M <= 256 (HBM bound, weight streaming only): seconds at the HBM roofline for
// W (once per M tile, the M tiles of one W slab sharing an XCD's L2), staged X
// (mostly L2 hits, weighted 1/2) and the fp32 split partials (written and read
// back, mostly MALL resident), against the dense product at about half the
// bf16 peak.  The streaming kernel walks k in bodies of 8 steps (4 when the
// split's step count is not a multiple of 8), so a split's steps count rounded
// up to that body.  One workgroup occupies a CU: a grid of w < 256
// workgroups reaches about (w/256)^0.55 of the chip's bandwidth (a CU alone
// streams faster than its 1/256 share), a larger one runs in rounds of 256,
// each with a fixed ~1.5 us (pipeline ramp, epilogue).  Fitted to sweeps of the
// drafter shapes at M = 16 .. 256 (every pick within 3 % of the fastest
// measured configuration, the sum within 0.3 %).
// M > 256 (matrix-core bound): the 128 x 128 streaming tile at its measured
// ~0.85 PFLOP/s or the 256 x 256 LDS-ring tile (tile-packed inputs) at ~1.2
// PFLOP/s.  Compute time is counted in whole waves of 256 workgroups, plus a
// fixed ~4 us per wave; split partials cost a write and a read of M x N x
// splits fp32 on top.  Fitted to measurements of the drafter shapes at M = 320
// .. 2048, the cost of a split including its consumer's extra reads (the picks
// sum to within 1.2 % of the fastest configurations').
// With a skipped corner (no queries for the drafter's context rows) the n_lo
// N tiles left of skip_n hold only the M tiles from m_lo on: fewer tiles, and
// those weight rows are read by fewer M tiles.
static double plan_cost(const Cand& c, int sp, int M, int N, int K, int skip_m, int skip_n) {
  const bool big = M > 256;
  const int mt = ceil_div(M, c.bm), nt = ceil_div(N, c.bn);
  const int m_lo = min(skip_m / c.bm, mt), n_lo = min(skip_n / c.bn, nt);
  const int mq = mt - m_lo;
  const double tiles = (double)n_lo * mq + (double)(nt - n_lo) * mt;
  const double wgs = tiles * sp;
  // weight rows times the M tiles that read them (the first from HBM, the rest
  // mostly from L2 at half weight)
  const double nc = fmin((double)N, (double)n_lo * c.bn);
  const double wrows = nc * (mq > 0 ? 1.0 + 0.5 * (mq - 1) : 0.0) + (N - nc) * (1.0 + 0.5 * (mt - 1));
  // fp32 output: one slice, or sp slices written and read back by the consumer
  const double part = sp > 1 ? 1.5 * 4.0 * M * N * sp : 4.0 * M * N;
  if (!big) {
    const int kps = ceil_div(K / BK, sp);
    const double pad = (double)(kps % 8 == 0 ? kps : ceil_div(kps, 4) * 4) / kps;
    const double w = 2.0 * wrows * K * pad;
    const double x = 2.0 * tiles * c.bm * K * pad;
    const double flops = 2.0 * tiles * c.bm * c.bn * K;
    const double rounds = ceil(wgs / 256.0);
    const double fill = wgs < 256.0 ? pow(wgs / 256.0, 0.55) : wgs / (rounds * 256.0);
    return fmax((w + 0.5 * x + part) / 8.0e12, flops / 1.2e15) / fill + rounds * 1.5e-6;
  }
  const double w = 2.0 * wrows * K;
  const double x = 2.0 * tiles * c.bm * K;
  const double flops = 2.0 * tiles * c.bm * c.bn * K;
  const double fill = wgs >= 192.0 ? 1.0 : wgs / 192.0;
  const double mem = (w + 0.5 * x + part) / 8.0e12;
  const double waves = ceil(wgs / 256.0);
  const double rate = c.kind == 3 ? 1.2e15 : 0.85e15;
  const double cmp = flops / rate * (waves * 256.0 / wgs) + waves * 4.0e-6;
  // split partials are written in the epilogue and read back by the consumer:
  // neither overlaps the matrix-core work
  return fmax(mem / fill, cmp) + (sp > 1 ? 2.0 * 4.0 * M * N * sp / 8.0e12 : 0.0);
}

static bool plan_allows(const Cand& c, int M) {
  if (M > 256) return (c.kind == 1 && c.mt == 8 && c.nw == 2 && c.bn == 128) || c.kind == 3;
  return c.kind == 1;
}

static void plan_take(GemmPlan& p, const Cand& c, int sp, int kps_blocks) {
  p.kind = c.kind;
  p.bm = c.bm;
  p.bn = c.bn;
  p.mt = c.mt;
  p.nw = c.nw;
  p.splits = sp;
  p.k_per_split = kps_blocks * BK;
  // X prefetched as deep as W where that streaming variant is built (measured a little faster)
  p.xd = ((c.mt >= 8 && c.nw == 2) || (c.mt == 16 && c.nw == 1)) ? 4 : 2;
}

int gemm_tiles(const GemmPlan& p, int M, int N, int skip_m, int skip_n) {
  const int mt = ceil_div(M, p.bm), nt = ceil_div(N, p.bn);
  if (p.kind != 1 && p.kind != 3) return mt * nt;
  const int m_lo = min(skip_m / p.bm, mt), n_lo = min(skip_n / p.bn, nt);
  return n_lo * (mt - m_lo) + (nt - n_lo) * mt;
}

GemmPlan gemm_plan(int M, int N, int K, int dtype, int force_splits, int skip_m, int skip_n) {
  GemmPlan best;
  if (dtype != 1) {   // fp32 VALU kernel
    best.kind = 2;
    best.bm = best.bn = 64;
    best.splits = 1;
    best.k_per_split = K;
    return best;
  }
  const int kb = K / BK;
  // M <= 16, K <= 512 other than 256: one round of independent waves (1.5x faster
  // than the streaming kernel on a 4 x 129280 x 256 product; at 32 rows the
  // per-wave X fragments cost more than the streaming kernel's shared LDS tile)
  if (M <= 16 && K <= 8 * BK && K != 4 * BK && force_splits <= 1) {
    best.kind = 4;
    best.bm = 16 * ceil_div(M, 16);
    best.bn = 64;
    best.splits = 1;
    best.k_per_split = K;
    return best;
  }
  // K = 256 and up to 128 rows (the sequential head's product at batch <= 128):
  // the persistent short-K kernel (X staged once per workgroup; measured faster
  // than the small-M kernel too: 13.9 against 15.0 us at 4 rows)
  if (M <= 128 && K == 4 * BK && force_splits <= 1) {
    best.kind = 5;
    best.bm = 16 * ceil_div(M, 16);
    best.bn = 16;
    best.splits = 1;
    best.k_per_split = K;
    return best;
  }
  double best_cost = 1e300;
  for (const Cand& c : kCands) {
    if (!plan_allows(c, M)) continue;
    for (int sp = 1; sp <= 32; ++sp) {
      if (force_splits && sp != force_splits) continue;
      const int kps_blocks = ceil_div(kb, sp);
      const int real_sp = ceil_div(kb, kps_blocks);
      if (real_sp != sp) continue;
      if (sp > 1 && kps_blocks < 4 && !force_splits) continue;
      const double cost = plan_cost(c, sp, M, N, K, skip_m, skip_n);
      if (cost < best_cost * 0.999) {
        best_cost = cost;
        plan_take(best, c, sp, kps_blocks);
      }
    }
  }
  if (best_cost == 1e300) {   // forced split count not representable
    best.kind = 1;
    best.bm = 128;
    best.bn = 128;
    best.mt = 8;
    best.nw = 2;
    best.xd = 4;
    best.splits = 1;
    best.k_per_split = K;
  }
  return best;
}

// GEMM whose X holds K / wk terms against a W of wk columns (GemmArgs.wk):
// the persistent short-K kernel for three 256-wide terms and up to 32 rows,
// else the plan of the full-K product (the streaming kernels wrap k).
GemmPlan gemm_plan_wrapped(int M, int N, int K, int wk, int dtype) {
  if (dtype == 1 && wk == 4 * BK && K == 3 * wk && M <= 32) {
    GemmPlan p;
    p.kind = 5;
    p.bm = 16 * ceil_div(M, 16);
    p.bn = 16;
    p.splits = 1;
    p.k_per_split = K;
    return p;
  }
  return gemm_plan(M, N, K, dtype, 1);
}

// Gated gate|up GEMM (N = features): no K split (the SwiGLU needs complete
// sums).  Weight streaming with paired tiles (48 or 64 features per workgroup,
// 32/64/128 rows; only 128 rows above M = 256), or for M > 256 the tile kernel
// (128 features per workgroup) when the same cost model prefers it.  Fitted
// on the drafter's 12288 features at M = 64 .. 256: 48-feature tiles (256
// workgroups instead of 192) are 5-17 % faster, every pick within 6 % of the
// fastest measured.
GemmPlan gemm_plan_gated(int M, int N, int K, int dtype) {
  GemmPlan p;
  p.kind = -1;
  if (dtype != 1 || K % BK) return p;
  p.kind = 1;
  p.nw = 2;
  p.splits = 1;
  p.k_per_split = K;
  p.pd = 4;
  // streaming tiles of 16*mt rows x 48 or 64 features (3 or 4 consumer waves, each
  // with 16 gate + 16 up rows), priced by the same model on the 2N weight rows:
  // 48 features make 256 workgroups of the drafter's 12288 features
  double best = 1e300;
  for (int mt : {2, 4, 8, 10}) {
    if (M > 256 && mt != 8) continue;
    for (int fpt : {48, 64}) {
      const Cand c = {1, 16 * mt, 2 * fpt, mt, 2};
      const double cost = plan_cost(c, 1, M, 2 * N, K, 0, 0);
      if (cost < best * 0.999) {
        best = cost;
        p.mt = mt;
        p.bm = 16 * mt;
        p.bn = fpt;
        p.xd = mt >= 8 ? 4 : 2;
      }
    }
  }
  if (M > 256) {
    // both read 2N weight rows; the LDS tile covers 128 features
    const Cand tile = {3, 256, 256, 0, 0};
    if (plan_cost(tile, 1, M, 2 * N, K, 0, 0) < best) {
      p.kind = 3;
      p.bm = 256;
      p.bn = 256;
      p.mt = p.nw = 0;
    }
  }
  return p;
}

size_t gemm_partial_elems(const GemmPlan& p, int M, int N) { return (size_t)p.splits * M * N; }

template <int MT, int NW, int PD, int XD, int LB, int CW>
hipError_t launch_stream_lb(const GemmArgs& a, dim3 g1, int kps, int mtl, int ntl, hipStream_t s) {
  const dim3 blk(64 * (CW + 4));
  if constexpr (NW == 2) {
    if (a.gated) {
      if (a.packed)
        hipLaunchKernelGGL((gemm_stream_bf16<MT, NW, PD, XD, true, true, LB, CW>), g1, blk, 0, s, a, kps, mtl, ntl);
      else
        hipLaunchKernelGGL((gemm_stream_bf16<MT, NW, PD, XD, false, true, LB, CW>), g1, blk, 0, s, a, kps, mtl, ntl);
      return hipGetLastError();
    }
  }
  if (a.gated) return hipErrorInvalidValue;
  if (a.packed)
    hipLaunchKernelGGL((gemm_stream_bf16<MT, NW, PD, XD, true, false, LB, CW>), g1, blk, 0, s, a, kps, mtl, ntl);
  else
    hipLaunchKernelGGL((gemm_stream_bf16<MT, NW, PD, XD, false, false, LB, CW>), g1, blk, 0, s, a, kps, mtl, ntl);
  return hipGetLastError();
}

// CW consumer waves (4, or 3 for the gated tile of 48 features)
template <int MT, int NW, int PD, int XD, int CW = 4>
hipError_t launch_stream(const GemmArgs& a, dim3 g1, int kps, int mtl, int ntl, hipStream_t s) {
  if ((kps / BK) % 8 != 0) return launch_stream_lb<MT, NW, PD, XD, 4, CW>(a, g1, kps, mtl, ntl, s);
  return launch_stream_lb<MT, NW, PD, XD, 8, CW>(a, g1, kps, mtl, ntl, s);
}

template <int BM, int BN>
hipError_t launch_tile(const GemmArgs& a, dim3 g1, int kps, int mtl, int ntl, hipStream_t s) {
  if (a.gated) {
    if (a.packed)
      hipLaunchKernelGGL((gemm_tile_bf16<BM, BN, true, true>), g1, dim3(512), 0, s, a, kps, mtl, ntl);
    else
      hipLaunchKernelGGL((gemm_tile_bf16<BM, BN, false, true>), g1, dim3(512), 0, s, a, kps, mtl, ntl);
  } else {
    if (a.packed)
      hipLaunchKernelGGL((gemm_tile_bf16<BM, BN, true, false>), g1, dim3(512), 0, s, a, kps, mtl, ntl);
    else
      hipLaunchKernelGGL((gemm_tile_bf16<BM, BN, false, false>), g1, dim3(512), 0, s, a, kps, mtl, ntl);
  }
  return hipGetLastError();
}

hipError_t launch_gemm(const GemmArgs& a, const GemmPlan& p, int dtype, hipStream_t s) {
  ProfScope ps("gemm", s);
  // tile-packed X is read by the tile kernel only; a packed gated output needs whole 64-wide tiles
  if (a.x_packed && (dtype != 1 || p.kind != 3 || a.row_idx || a.K % BK || (a.wk > 0 && a.wk != a.K)))
    return hipErrorInvalidValue;
  if (a.h_packed && (!a.gated || a.N % BK)) return hipErrorInvalidValue;
  if (a.wk > 0 && a.wk != a.K) {
    // W narrower than X: only the bf16 weight-streaming and small-M kernels wrap k
    if (dtype != 1 || a.gated || a.wk % BK || a.K % a.wk) return hipErrorInvalidValue;
    if (p.kind == 3) {
      GemmPlan q = p;
      q.kind = 1;
      q.bm = 128;
      q.bn = 128;
      q.mt = 8;
      q.nw = 2;
      q.pd = 4;
      q.xd = 4;
      return launch_gemm(a, q, dtype, s);
    }
  }
  if (dtype != 1) {
    dim3 grid(ceil_div(a.N, 64), ceil_div(a.M, 64), p.splits);
    hipLaunchKernelGGL(gemm_f32_nt, grid, dim3(256), 0, s, a, p.k_per_split);
    return hipGetLastError();
  }
  const int kps = p.k_per_split;
  if (p.kind == 1) {
    const int mtl = ceil_div(a.M, p.bm), ntl = ceil_div(a.N, p.bn);
    const dim3 g1(gemm_tiles(p, a.M, a.N, a.gated ? 0 : a.skip_m, a.gated ? 0 : a.skip_n) * p.splits);
    if (g1.x == 0) return hipSuccess;   // the skipped corner is the whole output
#define DFS_STREAM(MT_, NW_, PD_, XD_)                                                                   \
  if (p.mt == MT_ && p.nw == NW_ && p.pd == PD_ && p.xd == XD_ && p.bn != 48 && p.bn != 96)              \
    return launch_stream<MT_, NW_, PD_, XD_>(a, g1, kps, mtl, ntl, s);
    DFS_STREAM(2, 2, 4, 2)
    DFS_STREAM(2, 1, 4, 2)
    DFS_STREAM(4, 2, 4, 2)
    DFS_STREAM(4, 1, 4, 2)
    DFS_STREAM(8, 1, 4, 2)
    DFS_STREAM(8, 2, 4, 4)
    DFS_STREAM(10, 2, 4, 4)
    DFS_STREAM(16, 1, 4, 4)
    // 96 columns per workgroup (3 consumer waves)
    if (!a.gated && p.bn == 96) {
      if (p.mt == 8 && p.nw == 2 && p.pd == 4 && p.xd == 4) return launch_stream<8, 2, 4, 4, 3>(a, g1, kps, mtl, ntl, s);
      if (p.mt == 10 && p.nw == 2 && p.pd == 4 && p.xd == 4) return launch_stream<10, 2, 4, 4, 3>(a, g1, kps, mtl, ntl, s);
      if (p.mt == 4 && p.nw == 2 && p.pd == 4 && p.xd == 2) return launch_stream<4, 2, 4, 2, 3>(a, g1, kps, mtl, ntl, s);
      return hipErrorInvalidValue;
    }
    // gated tiles of 48 features (3 consumer waves)
    if (a.gated && p.bn == 48) {
      if (p.mt == 8 && p.nw == 2 && p.pd == 4 && p.xd == 4) return launch_stream<8, 2, 4, 4, 3>(a, g1, kps, mtl, ntl, s);
      if (p.mt == 10 && p.nw == 2 && p.pd == 4 && p.xd == 4) return launch_stream<10, 2, 4, 4, 3>(a, g1, kps, mtl, ntl, s);
      if (p.mt == 4 && p.nw == 2 && p.pd == 4 && p.xd == 2) return launch_stream<4, 2, 4, 2, 3>(a, g1, kps, mtl, ntl, s);
      if (p.mt == 2 && p.nw == 2 && p.pd == 4 && p.xd == 2) return launch_stream<2, 2, 4, 2, 3>(a, g1, kps, mtl, ntl, s);
      return hipErrorInvalidValue;
    }
#undef DFS_STREAM
    return hipErrorInvalidValue;
  }
  if (p.kind == 5) {   // persistent short-K kernel, K = 256, M <= 128
    const bool three = a.wk == 4 * BK && a.K == 3 * a.wk;   // three terms against one W
    const bool ok = !a.gated && p.splits == 1 && (a.K == 4 * BK || three) && a.M <= (three ? 32 : 128) &&
                    a.N % 4 == 0 && (a.ldy & 3) == 0 && ((uintptr_t)a.Y & 15) == 0 && !a.x_packed &&
                    (three || a.wk == 0 || a.wk == a.K) && a.nseg == 1;
    if (!ok) {   // same product on the streaming kernel
      GemmPlan q = p;
      q.kind = 1;
      q.mt = a.M <= 32 ? 2 : (a.M <= 64 ? 4 : 8);
      q.bm = 16 * q.mt;
      q.bn = 128;
      q.nw = 2;
      q.pd = 4;
      q.xd = q.mt == 8 ? 4 : 2;
      return launch_gemm(a, q, dtype, s);
    }
    const int ng = ceil_div(a.N, 16);
    const int mt = ceil_div(a.M, 16);
    // resident at once: two workgroups per CU with 32 rows and one term, else one (registers)
    const dim3 g5(min(ceil_div(ng, 4), mt <= 2 && !three ? 512 : 256));
#define DFS_SHORT(MT_, T_)                                                                           \
  if (mt <= MT_) {                                                                                   \
    if (a.packed) hipLaunchKernelGGL((gemm_short_bf16<MT_, true, T_>), g5, dim3(256), 0, s, a);      \
    else hipLaunchKernelGGL((gemm_short_bf16<MT_, false, T_>), g5, dim3(256), 0, s, a);              \
    return hipGetLastError();                                                                        \
  }
    if (three) {
      DFS_SHORT(2, 3)
    } else {
      DFS_SHORT(2, 1)
      DFS_SHORT(4, 1)
      DFS_SHORT(8, 1)
    }
#undef DFS_SHORT
    return hipErrorInvalidValue;
  }
  if (p.kind == 4) {   // independent waves, 16 W rows each, M <= 16, K <= 512
    if (a.gated || a.M > 16 || a.K > 8 * BK || p.splits > 1) return hipErrorInvalidValue;
    const dim3 g4(ceil_div(a.N, 64));
    const bool short_k = a.K <= 4 * BK;
    if (a.packed) {
      if (short_k) hipLaunchKernelGGL((gemm_rows_bf16<true, 4>), g4, dim3(256), 0, s, a);
      else hipLaunchKernelGGL((gemm_rows_bf16<true, 8>), g4, dim3(256), 0, s, a);
    } else {
      if (short_k) hipLaunchKernelGGL((gemm_rows_bf16<false, 4>), g4, dim3(256), 0, s, a);
      else hipLaunchKernelGGL((gemm_rows_bf16<false, 8>), g4, dim3(256), 0, s, a);
    }
    return hipGetLastError();
  }
  if (p.kind == 3) {   // LDS-ring tile kernel; gated tiles cover bn/2 features
    // its direct-to-LDS loads take 16-byte aligned rows; otherwise the 128 x 128
    // streaming tile with the same split count (same workspace)
    bool aligned = ((uintptr_t)a.X & 15) == 0 && (a.x_packed || (a.ldx & 7) == 0);
    for (int i = 0; i < (a.gated ? 2 : a.nseg); ++i) aligned = aligned && ((uintptr_t)a.seg[i].w & 15) == 0;
    if (!aligned) {
      if (a.x_packed) return hipErrorInvalidValue;
      GemmPlan q = p;
      q.kind = 1;
      q.bm = 128;
      q.bn = a.gated ? 64 : 128;
      q.mt = 8;
      q.nw = 2;
      q.pd = 4;
      q.xd = 4;
      return launch_gemm(a, q, dtype, s);
    }
    const int mtl = ceil_div(a.M, p.bm), ntl = ceil_div(a.N, a.gated ? p.bn / 2 : p.bn);
    const dim3 g1((a.gated ? mtl * ntl : gemm_tiles(p, a.M, a.N, a.skip_m, a.skip_n)) * p.splits);
    if (g1.x == 0) return hipSuccess;   // the skipped corner is the whole output
    if (p.bm == 256 && p.bn == 256) return launch_tile<256, 256>(a, g1, kps, mtl, ntl, s);
    return hipErrorInvalidValue;
  }
  return hipErrorInvalidValue;
}

hipError_t launch_head_gemm_stats(const GemmArgs& a, float temperature, double2* sub, hipStream_t s) {
  const bool ok = !a.gated && a.nseg == 1 && a.K == 4 * BK && a.M >= 1 && a.M <= 128 && a.N % 4 == 0 &&
                  (a.ldy & 3) == 0 && ((uintptr_t)a.Y & 15) == 0 && !a.x_packed && (a.wk == 0 || a.wk == a.K) &&
                  a.accumulate;
  if (!ok) return hipErrorInvalidValue;
  const int nsub = ceil_div(a.N, 64), nrc = ceil_div(a.M, 32);
  const dim3 grid(ceil_div(nsub, 2) * nrc);
  if (a.packed) hipLaunchKernelGGL(head_gemm_stats_bf16<true>, grid, dim3(512), 0, s, a, temperature, sub, nsub, nrc);
  else hipLaunchKernelGGL(head_gemm_stats_bf16<false>, grid, dim3(512), 0, s, a, temperature, sub, nsub, nrc);
  return hipGetLastError();
}

size_t packed_matrix_elems(int N, int K) { return (size_t)ceil_div(N, 16) * 16 * K; }

hipError_t launch_pack(const void* src, void* dst, int N, int K, hipStream_t s) {
  const size_t chunks = packed_matrix_elems(N, K) / 8;
  const size_t need = (chunks + 255) / 256;
  const unsigned blocks = (unsigned)(need < 16384 ? need : 16384);
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(pack_kernel, dim3(blocks), dim3(256), 0, s, (const bf16_t*)src, (bf16_t*)dst, N, K);
  return hipGetLastError();
}

}  // namespace dfs
