// Internal host-side launchers shared between the translation units of the
// dfspec library.  Not part of the C ABI.
#pragma once

#include "common.h"

namespace dfs {

// ------------------------------------------------------------------ GEMM
// Y[z][m][n] (+)= sum_{k in split z} X[row(m)][k] * W[n][k]
// W is the row-concatenation of up to three [n_i, K] segments (e.g. wq|wk|wv).
struct GemmSeg {
  const void* w = nullptr;
  int n0 = 0;   // first logical row of W held by this segment
};

struct GemmArgs {
  const void* X = nullptr;
  int ldx = 0;                        // elements between X rows
  const int32_t* row_idx = nullptr;   // optional row gather: X row of m = row_idx[m * row_idx_stride]
  int row_idx_stride = 1;
  int x_rows = 0;                     // rows of X (gathered indices are clamped to it)
  int M = 0, N = 0, K = 0;
  GemmSeg seg[3];
  int nseg = 1;
  float* Y = nullptr;
  long ldy = 0;
  size_t y_split_stride = 0;          // elements between split slices of Y
  int accumulate = 0;                 // 1: Y += acc (single split only)
  int packed = 0;                     // 1: W segments tile-packed (bf16; see packed_matrix_elems)
  // gated (SwiGLU) output: seg[0] = W_gate, seg[1] = W_up, both [N, K]; the kernel
  // writes hout[m][n] = bf16(silu(gate) * up) (row stride ldy) instead of Y
  int gated = 0;
  void* hout = nullptr;
  int nt_store = 0;                   // 1: results written with non-temporal stores (not re-read soon)
  // > 0 and < K: W has wk columns and GEMM column k multiplies W column k % wk
  // (X's K columns hold K / wk terms of one operand; bf16 streaming / rows kernels)
  int wk = 0;
  int x_packed = 0;                   // 1: X in the tile-packed layout (xpk_index; tile kernel only)
  int h_packed = 0;                   // 1: gated output hout written tile-packed (K = N features)
  // output tiles whose rows all lie below skip_m and whose columns all lie below
  // skip_n are not computed and their Y is left untouched (the drafter's Q|K|V
  // product: no queries for the context rows); the weight-streaming and LDS-ring
  // kernels honour it, the others compute those tiles too
  int skip_m = 0, skip_n = 0;
};

struct GemmPlan {
  int kind = 1;            // 1: bf16 weight streaming, 3: bf16 LDS-ring tile, 4: bf16 small-M rows,
                           // 5: bf16 persistent short-K (K = 256, M <= 128), 2: fp32 VALU
  int bm = 128, bn = 128, mt = 8, nw = 2, splits = 1, k_per_split = 0;
  int pd = 4, xd = 2;      // weight-streaming kernel: k steps of W / X in flight per wave
};

GemmPlan gemm_plan(int M, int N, int K, int dtype, int force_splits = 0, int skip_m = 0, int skip_n = 0);
// output tiles of a plan's grid per K split, the skipped corner (GemmArgs.skip_m/n) left out
int gemm_tiles(const GemmPlan& p, int M, int N, int skip_m, int skip_n);
// plan of a single-split GEMM whose X holds K / wk terms against W's wk columns
GemmPlan gemm_plan_wrapped(int M, int N, int K, int wk, int dtype);
// plan of a gated gate|up GEMM (N = features), or kind < 0 when no gated kernel fits
GemmPlan gemm_plan_gated(int M, int N, int K, int dtype);
// Tile-packed bf16 weights: [ceil(N/16)][K/64] tiles of 16 rows x 64 columns,
// each 2 KB tile stored in matrix-core operand order [ks 0..1][lane 0..63][8]:
// lane l holds row 16*nt + (l % 16), columns 64*kt + 32*ks + 8*(l / 16) .. +7.
// Rows past N are zero.  A wave loads one k step of 16 rows as 2 contiguous KB.
size_t packed_matrix_elems(int N, int K);
hipError_t launch_pack(const void* src, void* dst, int N, int K, hipStream_t s);
size_t gemm_partial_elems(const GemmPlan& p, int M, int N);   // sp * M * N
hipError_t launch_gemm(const GemmArgs& a, const GemmPlan& p, int dtype, hipStream_t s);

// ------------------------------------------------------------------ attention
struct AttnArgs {
  const void* q;        // [B][nkv][Rpad][d]  rows r = hh * S + s
  const void* k_blk;    // [B][nkv][64][d]
  const void* v_blk;    // [B][nkv][d][64]   (transposed)
  const void* k_cache;  // [B][nkv][max_ctx][d]   (one layer)
  const void* v_cache;  // [B][nkv][d][max_ctx]   (one layer, transposed)
  const int32_t* ctx_len;   // [B] context keys per row (already clamped)
  void* out;            // [B][S][nq][d]
  float* part_o;        // [B][nkv][nunits][Rpad][d]
  float* part_ml;       // [B][nkv][nunits][Rpad][2]
  int B, S, nq, nkv, d, max_ctx, ctx_bound;
  int R, Rpad;          // rows per kv head = (nq/nkv)*S, padded to 16
  int n_ctx_splits;     // units = n_ctx_splits + 1 (last = block keys); a row's C_b is split evenly
  int row_groups = 1;   // bf16: the R rows in groups of 64, one workgroup per (unit, group)
  int window = 0;       // > 0: only the last `window` of a row's C_b context keys are attended
  int out_packed = 0;   // bf16: out written tile-packed as rows b*S + s of nq*d columns (xpk_index)
};
struct AttnPlan {
  int keys_per_split, n_ctx_splits;
};
AttnPlan attn_plan(int B, int nkv, int ctx_bound, int dtype, int row_groups = 1, int window = 0);
int attn_max_units(int B, int nkv, int max_ctx, int dtype);
size_t attn_partial_elems(int units, int B, int nkv, int Rpad, int d);
hipError_t launch_attention(const AttnArgs& a, int dtype, hipStream_t s);
// Re-layout of plain [B, S, nq, d] queries and [B, S, nkv, d] keys/values into
// the attention kernel's operand layouts (used by the stand-alone attention entry).
hipError_t launch_attn_stage(const void* q, const void* k, const void* v, void* q_att, void* k_blk,
                             void* v_blk, int B, int S, int nq, int nkv, int d, int Rpad, int dtype,
                             hipStream_t s);

// ------------------------------------------------------------------ drafter elementwise
struct MetaArgs {
  const int32_t* ctx_len;   // [B] in
  const int32_t* n_new;     // [B] in
  int32_t* meta;            // [3][B]: base, nn, C_b
  float2* rope;             // [(B*n_new_max + B*S)][d/2] (cos, sin)
  int B, S, n_new_max, d, ctx_bound;
  float theta;
};
// out[row_map(r)] = T( RMSNorm( in[r] (+= sum_z part[z][r]) ; gain ) )
struct NormArgs {
  float* resid = nullptr;         // [rows][H] fp32 residual (updated when part != null and update_resid)
  const float* part = nullptr;    // [sp][rows][H] partials to reduce (nullable)
  int sp = 0;
  size_t part_stride = 0;
  int update_resid = 0;           // 1: resid += sum(part), then normalise resid
  const void* gain = nullptr;     // [H] dtype
  void* out = nullptr;            // dtype
  int rows = 0, H = 0;
  float eps = 0.f;
  int out_mode = 0;               // 0: out row = r; 1: only rows with r % S != 0 -> b*(S-1) + s-1
  int S = 1;
  int out_packed = 0;             // bf16: out tile-packed (xpk_index), output row + out_row0 in it
  int out_row0 = 0;
  // embedding rows (embed != null): row r = b*S + s is E[token], token = last_token[b]
  // at s == 0 else mask_id (clamped to [0, V)), written to resid, then normalised
  const void* embed = nullptr;    // [V][H] dtype
  const int32_t* last_token = nullptr;
  int mask_id = 0, V = 0;
};
hipError_t launch_norm(const NormArgs& a, int dtype, hipStream_t s);
// The start of a drafter call in one launch: the context features' RMSNorm
// (feat, rows may be 0), the block rows' embedding and first pre-norm (blk), and
// the positions, rotary table and per-row bookkeeping (m; meta[2B + b] = C_b).
hipError_t launch_front(const NormArgs& feat, const NormArgs& blk, const MetaArgs& m, int dtype, hipStream_t s);

struct QkvArgs {
  const float* part;     // [sp][Mx][Nqkv]
  int sp;
  size_t part_stride;
  const int32_t* meta;   // [3][B]
  const float2* rope;    // [Mx][d/2]
  int use_rope;
  void* k_cache;         // layer base [B][nkv][max_ctx][d]
  void* v_cache;         // layer base [B][nkv][d][max_ctx]
  void* q_att;           // [B][nkv][Rpad][d]
  void* k_blk;           // [B][nkv][64][d]
  void* v_blk;           // [B][nkv][d][64]
  int B, S, n_new_max, nq, nkv, d, max_ctx, Rpad;
  int32_t* ctx_len_out = nullptr;   // when set: ctx_len_out[b] = meta C_b (the caller's context lengths advanced)
};
hipError_t launch_qkv_epilogue(const QkvArgs& a, int dtype, hipStream_t s);

hipError_t launch_reduce(const float* part, int sp, size_t part_stride, size_t n, float* out, hipStream_t s,
                         int accumulate = 0);

hipError_t launch_swiglu(const float* part, int sp, size_t part_stride, int M, int F, void* out,
                         int dtype, hipStream_t s);

// ------------------------------------------------------------------ sampling / verify
// Chunked row statistics: per (row, chunk): (max, sum exp((x-max)/T)) in fp64, or for
// T == 0 (max, index of the first maximum).
constexpr int kChunk = 4096;
// sub (nullable, used when temperature > 0): [rows][nch][64] fp64 sums of each
// 64-token sub-chunk relative to its chunk max
hipError_t launch_chunk_stats(const float* x, long row_stride, int rows, int V, float temperature,
                              double2* stats, double* sub, hipStream_t s);

struct PickArgs {
  const float* x;          // logits rows
  long row_stride;
  int rows, V;
  float temperature;
  const double2* stats;    // [rows][nchunks]
  const double* sub;       // [rows][nchunks][64] sub-chunk sums (T > 0)
  const float* u;          // [rows] (stride u_stride)
  long u_stride;
  int32_t* tokens;         // [rows] (stride tok_stride)
  long tok_stride;
  double* row_stats;       // [rows][2] (stride rs_stride doubles), nullable
  long rs_stride;
};
hipError_t launch_pick(const PickArgs& a, hipStream_t s);
// The Markov head's product Y += X . W^T (K = 256, M <= 128, accumulate) with, per
// row and 64-column sub-chunk, (max, sum exp((x - max)/T)) or for T == 0 (max,
// first column of the max) in sub [M][ceil(N/64)].
hipError_t launch_head_gemm_stats(const GemmArgs& a, float temperature, double2* sub, hipStream_t s);
// One workgroup per row: inverse-CDF draw / argmax from those sub-chunk
// statistics (subst [rows][nsub], row r at subst + r * nsub, nsub <=
// kPickSubMax); PickArgs.stats/.sub unused.
constexpr int kPickSubMax = 4096;                    // V <= 262144 on the fused head path
hipError_t launch_pick_sub(const PickArgs& a, const double2* subst, int nsub, hipStream_t s);

struct VerifyArgs {
  const float* q;          // draft logits [B][G][V]
  const float* p;          // target logits [B][G+1][V]
  const int32_t* drafts;   // [B][G]
  const float* u_accept;   // [B][G]
  const float* u_final;    // [B]
  const int32_t* n_verify; // [B] drafts verified per row (clamped to [0, G]), or null = G
  float temperature;
  const double* q_stats;   // [B][G][2] (max, sum) of the draft rows, or null -> q_chunk
  double2* q_chunk;        // [B*G][nch]
  double2* p_chunk;        // [B*(G+1)][nch]
  double* p_sub;           // [B*(G+1)][nch][64] sub-chunk sums of the target rows
  double* rowinfo;         // [B][4]: (Mp, Sp, Mq, Sq) at the rejected position, statistics-pass normalisers
  int32_t* state;          // [B]: first rejected position (= the verify length when all are accepted)
  double* res;             // [B][nch][4]: per chunk of the rejected rows, fp64 sums (see verify.hip)
  double2* sub;            // [B][nch][64]: per 64-token sub-chunk of the rejected rows, fp64 sums
  int32_t* out_tokens;     // [B][G+1]
  int32_t* n_accepted;     // [B]
  int B, G, V;
};
hipError_t launch_verify(const VerifyArgs& a, hipStream_t s);

// ------------------------------------------------------------------ cycle bookkeeping
hipError_t launch_advance(int B, int G, const int32_t* n_accepted, const int32_t* out_tokens, int32_t* n_new,
                          int32_t* last_token, int64_t* tau_sum, hipStream_t s);

constexpr int kSchedCurve = 32;   // throughput-curve points passed by value
struct SchedArgs {
  const float* surv;       // [B][G] per-position survival scores
  int32_t* n_verify;       // [B] out: drafts to verify per request
  int B, G, ncurve;
  float xs[kSchedCurve];   // rows in the verify batch, increasing
  float ys[kSchedCurve];   // verify passes per second at xs
};
hipError_t launch_schedule(const SchedArgs& a, hipStream_t s);

// ------------------------------------------------------------------ RNN sequential head
constexpr int kRnnMaxRank = 1024;
struct RnnArgs {
  const void* U;           // [V][r] input factor (dtype)
  const void* A;           // [r][r] recurrent matrix (dtype), row j -> state element j
  const int32_t* prev;     // previous token of request b at prev[b * prev_stride]
  long prev_stride;
  const float* h_in;       // [B][r] fp32 previous state (ignored when first)
  float* h_out;            // [B][r] fp32 new state (a different buffer)
  bf16_t* split;           // [B][3][r] bf16 terms hi, mid, lo of the new state, or null
  int first;               // 1: previous state is zero (first position of the block)
  int B, V, r;
};
hipError_t launch_rnn_state(const RnnArgs& a, int dtype, hipStream_t s);

}  // namespace dfs
