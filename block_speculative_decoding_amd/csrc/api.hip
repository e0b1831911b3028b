// C ABI of the dfspec library: host-side validation, workspace carving and the
// launch sequence of each entry point.  See include/dfspec.h for the contract.
#include "../../include/dfspec.h"
#include "kernels.h"

#include <mutex>

using namespace dfs;

namespace {

// ------------------------------------------------------------------ static scratch
// The scratch of spec_verify_static: a file-scope device array, one copy per
// GPU the library runs on, held until the process ends.  Host code reaches it
// only through the device address that hipGetSymbolAddress returns for the
// current device (the array's own name is a host-side stand-in); the address
// of each device is looked up once, on that device's first call.
constexpr size_t kStaticScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) char scratch[kStaticScratchBytes];
constexpr int kMaxDevices = 64;
void* g_scratch_dev[kMaxDevices];
std::mutex g_scratch_mu;

int static_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return DFS_EHIP;
  if (dev >= kMaxDevices) return DFS_EUNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return DFS_EHIP;
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return DFS_OK;
}

#define DFS_TRY(expr)                          \
  do {                                         \
    if ((expr) != hipSuccess) return DFS_EHIP; \
  } while (0)

size_t dtype_size(int dt) { return dt == DFS_BF16 ? 2 : 4; }

// the vocabulary-streaming kernels select among at most 1024 chunks of 4096 tokens
constexpr int kMaxVocab = 1024 * kChunk;

struct DraftDims {
  int L, H, nq, nkv, d, F, V, nT, S, G, max_ctx, group, R, Rpad;
  int B, nmax, Mc, Mb, Mx, Nqkv;
  size_t es;
};

int check_cfg(const dfs_drafter_cfg* c) {
  if (!c) return DFS_EINVAL;
  if (c->n_layers < 1 || c->hidden < 1 || c->n_q_heads < 1 || c->n_kv_heads < 1 || c->head_dim < 2 ||
      c->mlp_dim < 1 || c->vocab < 1 || c->n_target_layers < 1 || c->block < 2 || c->max_ctx < 1)
    return DFS_EINVAL;
  if (c->n_q_heads % c->n_kv_heads != 0 || c->head_dim % 2 != 0) return DFS_EINVAL;
  if (c->mask_token_id < 0 || c->mask_token_id >= c->vocab) return DFS_EINVAL;
  if (c->dtype != DFS_F32 && c->dtype != DFS_BF16) return DFS_EINVAL;
  if (!(c->rms_eps >= 0.f) || c->window < 0) return DFS_EINVAL;
  if (c->max_ctx % 64 != 0 || c->block > 64 || c->hidden > 8192) return DFS_EUNSUPPORTED;
  const long R = (long)(c->n_q_heads / c->n_kv_heads) * c->block;
  if (c->dtype == DFS_BF16) {
    if (c->head_dim != 128 || c->hidden % 64 || (c->n_q_heads * c->head_dim) % 64 || c->mlp_dim % 64 ||
        ((long)c->n_target_layers * c->hidden) % 64 || R > 256)
      return DFS_EUNSUPPORTED;
  } else {
    if (c->head_dim > 256 || R > 256) return DFS_EUNSUPPORTED;
  }
  return DFS_OK;
}

DraftDims dims_of(const dfs_drafter_cfg* c, int B, int nmax) {
  DraftDims d;
  d.L = c->n_layers;
  d.H = c->hidden;
  d.nq = c->n_q_heads;
  d.nkv = c->n_kv_heads;
  d.d = c->head_dim;
  d.F = c->mlp_dim;
  d.V = c->vocab;
  d.nT = c->n_target_layers;
  d.S = c->block;
  d.G = c->block - 1;
  d.max_ctx = c->max_ctx;
  d.group = d.nq / d.nkv;
  d.R = d.group * d.S;
  d.Rpad = (d.R + 15) / 16 * 16;
  d.B = B;
  d.nmax = nmax;
  d.Mc = B * nmax;
  d.Mb = B * d.S;
  d.Mx = d.Mc + d.Mb;
  d.Nqkv = (d.nq + 2 * d.nkv) * d.d;
  d.es = dtype_size(c->dtype);
  return d;
}

struct DraftWs {
  int32_t* meta;
  float2* rope;
  char* xs;
  float* resid;
  char* mlp_in;
  char* attn_o;
  char* hmid;
  char* z;
  char* q_att;
  char* k_blk;
  char* v_blk;
  float* part;
  float* apart_o;
  float* apart_ml;
  size_t resid_off, mlp_in_off, hmid_off;   // byte offsets in the workspace (trace hook)
  size_t bytes;
};

DraftWs carve_draft(void* base, const DraftDims& d, int dtype) {
  Carver cv(base);
  DraftWs w;
  w.meta = cv.take<int32_t>(3 * (size_t)d.B);
  w.rope = cv.take<float2>((size_t)d.Mx * (d.d / 2));
  // GEMM inputs: whole 16-row groups (room for the tile-packed layout)
  auto r16 = [](int m) { return (size_t)ceil_div(m, 16) * 16; };
  w.xs = cv.take<char>(r16(d.Mx) * d.H * d.es);
  w.resid = cv.take<float>((size_t)d.Mb * d.H);
  w.resid_off = cv.off - (size_t)d.Mb * d.H * sizeof(float);
  w.mlp_in = cv.take<char>(r16(d.Mb) * d.H * d.es);
  w.mlp_in_off = cv.off - r16(d.Mb) * d.H * d.es;
  w.attn_o = cv.take<char>(r16(d.Mb) * d.nq * d.d * d.es);
  w.hmid = cv.take<char>(r16(d.Mb) * d.F * d.es);
  w.hmid_off = cv.off - r16(d.Mb) * d.F * d.es;
  w.z = cv.take<char>(r16(d.B * d.G) * d.H * d.es);
  w.q_att = cv.take<char>((size_t)d.B * d.nkv * d.Rpad * d.d * d.es);
  w.k_blk = cv.take<char>((size_t)d.B * d.nkv * 64 * d.d * d.es);
  w.v_blk = cv.take<char>((size_t)d.B * d.nkv * d.d * 64 * d.es);
  size_t part = 0;
  auto upd = [&](int M, int N, int K, int skip_m = 0, int skip_n = 0) {
    if (M <= 0) return;
    const GemmPlan p = gemm_plan(M, N, K, dtype, 0, skip_m, skip_n);
    const size_t e = gemm_partial_elems(p, M, N);
    if (e > part) part = e;
  };
  upd(d.Mc, d.H, d.nT * d.H);
  upd(d.Mx, d.Nqkv, d.H, d.Mc, d.nq * d.d);
  upd(d.Mb, d.H, d.nq * d.d);
  upd(d.Mb, 2 * d.F, d.H);
  upd(d.Mb, d.H, d.F);
  w.part = cv.take<float>(part);
  const int units = attn_max_units(d.B, d.nkv, d.max_ctx, dtype);
  w.apart_o = cv.take<float>(attn_partial_elems(units, d.B, d.nkv, d.Rpad, d.d));
  w.apart_ml = cv.take<float>((size_t)d.B * d.nkv * units * d.Rpad * 2);
  w.bytes = cv.off + 256;
  return w;
}

// Whether the GEMM's X is produced in the tile-packed layout: the LDS-ring tile
// kernel loads a packed half tile as one contiguous kilobyte per wave instead of
// gathering 16 row pieces (bf16 activations this library writes itself).
bool pack_x(int M, int N, int K, int dtype, int force_splits = 0, int skip_m = 0, int skip_n = 0) {
  return dtype == DFS_BF16 && M > 0 && K % 64 == 0 &&
         gemm_plan(M, N, K, dtype, force_splits, skip_m, skip_n).kind == 3;
}

// skip_m, skip_n: output tiles entirely inside rows [0, skip_m) x columns
// [0, skip_n) are not computed (GemmArgs.skip_m)
hipError_t run_gemm(const void* X, int ldx, int M, int N, int K, const void* w0, const void* w1, int n1,
                    const void* w2, int n2, float* Y, int dtype, int packed, hipStream_t s, int* splits_out,
                    size_t* stride_out, int force_splits = 0, long ldy = 0, int nt_store = 0, int x_packed = 0,
                    int skip_m = 0, int skip_n = 0) {
  GemmArgs a;
  a.skip_m = skip_m;
  a.skip_n = skip_n;
  a.packed = packed;
  a.nt_store = nt_store;
  a.x_packed = x_packed;
  a.X = X;
  a.ldx = ldx;
  a.x_rows = M;
  a.M = M;
  a.N = N;
  a.K = K;
  a.seg[0].w = w0;
  a.seg[0].n0 = 0;
  a.nseg = 1;
  if (w1) {
    a.seg[1].w = w1;
    a.seg[1].n0 = n1;
    a.nseg = 2;
  }
  if (w2) {
    a.seg[2].w = w2;
    a.seg[2].n0 = n2;
    a.nseg = 3;
  }
  const GemmPlan p = gemm_plan(M, N, K, dtype, force_splits, skip_m, skip_n);
  a.Y = Y;
  a.ldy = ldy ? ldy : N;
  a.y_split_stride = (size_t)M * N;
  if (splits_out) *splits_out = p.splits;
  if (stride_out) *stride_out = (size_t)M * N;
  return launch_gemm(a, p, dtype, s);
}

// SwiGLU MLP input: hout[m][f] = bf16(silu(X.Wg^T) * (X.Wu^T)) in one weight pass
hipError_t run_gemm_gated(const void* X, int ldx, int M, int F, int K, const void* wg, const void* wu, void* hout,
                          int packed, const GemmPlan& p, hipStream_t s, int x_packed = 0, int h_packed = 0) {
  GemmArgs a;
  a.x_packed = x_packed;
  a.h_packed = h_packed;
  a.X = X;
  a.ldx = ldx;
  a.x_rows = M;
  a.M = M;
  a.N = F;
  a.K = K;
  a.seg[0].w = wg;
  a.seg[1].w = wu;
  a.nseg = 2;
  a.ldy = F;
  a.packed = packed;
  a.gated = 1;
  a.hout = hout;
  return launch_gemm(a, p, DFS_BF16, s);
}

template <typename P>
const char* at(const P* base, size_t off) {
  return (const char*)base + off;
}

}  // namespace

extern "C" {

const char* dfs_status_string(int st) {
  switch (st) {
    case DFS_OK: return "ok";
    case DFS_EINVAL: return "invalid argument";
    case DFS_EUNSUPPORTED: return "unsupported shape or dtype";
    case DFS_EHIP: return "HIP launch failed";
    case DFS_EWORKSPACE: return "workspace too small";
    default: return "unknown status";
  }
}

size_t dflash_draft_workspace_size(const dfs_drafter_cfg* cfg, int32_t batch, int32_t n_new_max) {
  if (check_cfg(cfg) != DFS_OK || batch < 1 || n_new_max < 0) return 0;
  const DraftDims d = dims_of(cfg, batch, n_new_max);
  return carve_draft(nullptr, d, cfg->dtype).bytes;
}

int dfs_draft_trace_layout(const dfs_drafter_cfg* cfg, int32_t batch, int32_t n_new_max, size_t* offsets,
                           int32_t* packed) {
  if (!offsets || !packed || batch < 1 || n_new_max < 0) return DFS_EINVAL;
  const int st = check_cfg(cfg);
  if (st != DFS_OK) return st;
  const DraftDims d = dims_of(cfg, batch, n_new_max);
  const int dt = cfg->dtype;
  const DraftWs w = carve_draft(nullptr, d, dt);
  // the same layout decisions as dflash_draft_step's
  const GemmPlan gated = gemm_plan_gated(d.Mb, d.F, d.H, dt);
  offsets[0] = w.resid_off;
  offsets[1] = w.mlp_in_off;
  offsets[2] = w.hmid_off;
  packed[0] = 0;
  packed[1] = dt == DFS_BF16 && gated.kind == 3;
  packed[2] = gated.kind > 0 && pack_x(d.Mb, d.H, d.F, dt);
  return DFS_OK;
}

int dflash_draft_step(const dfs_drafter_cfg* cfg, const dfs_drafter_weights* wt, int32_t batch,
                      const void* hidden_new, const int32_t* n_new, int32_t n_new_max, int32_t ctx_bound,
                      void* k_cache, void* v_cache, int32_t* ctx_len, const int32_t* last_token,
                      float* base_logits, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_cfg(cfg);
  if (st != DFS_OK) return st;
  if (!wt || batch < 1 || n_new_max < 0 || !n_new || !k_cache || !v_cache || !ctx_len || !last_token ||
      !base_logits || !workspace)
    return DFS_EINVAL;
  if (n_new_max > 0 && !hidden_new) return DFS_EINVAL;
  if (ctx_bound < 1 || ctx_bound > cfg->max_ctx) return DFS_EINVAL;
  if (batch > 65535) return DFS_EUNSUPPORTED;   // batch is a grid dimension of the attention kernels
  if (!wt->embed || !wt->fc || !wt->fc_norm || !wt->final_norm || !wt->lm_head || !wt->attn_norm || !wt->wq ||
      !wt->wk || !wt->wv || !wt->wo || !wt->mlp_norm || !wt->w_gate || !wt->w_up || !wt->w_down)
    return DFS_EINVAL;
  for (int l = 0; l < cfg->n_layers; ++l)
    if (!wt->attn_norm[l] || !wt->wq[l] || !wt->wk[l] || !wt->wv[l] || !wt->wo[l] || !wt->mlp_norm[l] ||
        !wt->w_gate[l] || !wt->w_up[l] || !wt->w_down[l])
      return DFS_EINVAL;
  const DraftDims d = dims_of(cfg, batch, n_new_max);
  const int dt = cfg->dtype;
  const int pk = wt->packed;
  if (pk != 0 && pk != 1) return DFS_EINVAL;
  if (pk && dt != DFS_BF16) return DFS_EUNSUPPORTED;
  const DraftWs w = carve_draft(workspace, d, dt);
  if (workspace_bytes < w.bytes) return DFS_EWORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  const size_t es = d.es;

  // positions, rotary table, bookkeeping
  MetaArgs ma;
  ma.ctx_len = ctx_len;
  ma.n_new = n_new;
  ma.meta = w.meta;
  ma.rope = cfg->rope_theta > 0.f ? w.rope : nullptr;
  ma.B = d.B;
  ma.S = d.S;
  ma.n_new_max = d.nmax;
  ma.d = d.d;
  ma.ctx_bound = ctx_bound;
  ma.theta = cfg->rope_theta;

  int sp;
  size_t pst;
  // which GEMM inputs are written tile-packed (those read by the LDS-ring tile kernel)
  const GemmPlan gated = gemm_plan_gated(d.Mb, d.F, d.H, dt);
  // no queries are needed for the context rows: the Q|K|V product skips those tiles
  const int qkv_skip_m = d.Mc, qkv_skip_n = d.nq * d.d;
  const int xp_qkv = pack_x(d.Mx, d.Nqkv, d.H, dt, 0, qkv_skip_m, qkv_skip_n);
  const int xp_o = pack_x(d.Mb, d.H, d.nq * d.d, dt);
  const int xp_mlp = dt == DFS_BF16 && gated.kind == 3;
  const int xp_down = gated.kind > 0 && pack_x(d.Mb, d.H, d.F, dt);
  const int xp_lm = pack_x(d.B * d.G, d.V, d.H, dt, 1);
  // 1. context features f = RMSNorm(concat(h) . fc^T) -> xs rows [0, Mc); in the
  //    same launch the block embedding [last, MASK x gamma] with layer 0's
  //    attention pre-norm, and the positions / rotary table / bookkeeping
  NormArgs nf;
  if (d.Mc > 0) {
    DFS_TRY(run_gemm(hidden_new, d.nT * d.H, d.Mc, d.H, d.nT * d.H, wt->fc, nullptr, 0, nullptr, 0, w.part, dt, pk, s,
                     &sp, &pst));
    nf.part = w.part;
    nf.sp = sp;
    nf.part_stride = pst;
    nf.gain = wt->fc_norm;
    nf.out = w.xs;
    nf.out_packed = xp_qkv;
    nf.rows = d.Mc;
    nf.H = d.H;
    nf.eps = cfg->rms_eps;
  }
  // block rows of xs: rows Mc.. (packed: same buffer, row offset Mc)
  char* xs_blk = xp_qkv ? w.xs : w.xs + (size_t)d.Mc * d.H * es;
  {
    NormArgs nb;
    nb.resid = w.resid;
    nb.embed = wt->embed;
    nb.last_token = last_token;
    nb.mask_id = cfg->mask_token_id;
    nb.V = d.V;
    nb.S = d.S;
    nb.gain = wt->attn_norm[0];
    nb.out = xs_blk;
    nb.out_packed = xp_qkv;
    nb.out_row0 = xp_qkv ? d.Mc : 0;
    nb.rows = d.Mb;
    nb.H = d.H;
    nb.eps = cfg->rms_eps;
    DFS_TRY(launch_front(nf, nb, ma, dt, s));
  }
  const int rgs = dt == DFS_BF16 ? ceil_div(d.R, 64) : 1;   // 64-row groups of the R query rows
  const AttnPlan ap = attn_plan(d.B, d.nkv, ctx_bound, dt, rgs, cfg->window);
  const size_t layer_cache = (size_t)d.B * d.nkv * d.max_ctx * d.d * es;
  for (int l = 0; l < d.L; ++l) {
    // 2. Q|K|V of [features ; block rows] in one pass over wq|wk|wv
    DFS_TRY(run_gemm(w.xs, d.H, d.Mx, d.Nqkv, d.H, wt->wq[l], wt->wk[l], d.nq * d.d, wt->wv[l],
                     (d.nq + d.nkv) * d.d, w.part, dt, pk, s, &sp, &pst, 0, 0, 0, xp_qkv, qkv_skip_m, qkv_skip_n));
    QkvArgs qa;
    qa.part = w.part;
    qa.sp = sp;
    qa.part_stride = pst;
    qa.meta = w.meta;
    qa.rope = w.rope;
    qa.use_rope = cfg->rope_theta > 0.f;
    qa.k_cache = (char*)k_cache + l * layer_cache;
    qa.v_cache = (char*)v_cache + l * layer_cache;
    qa.q_att = w.q_att;
    qa.k_blk = w.k_blk;
    qa.v_blk = w.v_blk;
    qa.B = d.B;
    qa.S = d.S;
    qa.n_new_max = d.nmax;
    qa.nq = d.nq;
    qa.nkv = d.nkv;
    qa.d = d.d;
    qa.max_ctx = d.max_ctx;
    qa.Rpad = d.Rpad;
    qa.ctx_len_out = l == 0 ? ctx_len : nullptr;   // every read of the caller's lengths is behind us
    DFS_TRY(launch_qkv_epilogue(qa, dt, s));
    // 3. block attention over [context keys ; block keys]
    AttnArgs aa;
    aa.q = w.q_att;
    aa.k_blk = w.k_blk;
    aa.v_blk = w.v_blk;
    aa.k_cache = qa.k_cache;
    aa.v_cache = qa.v_cache;
    aa.ctx_len = w.meta + 2 * d.B;
    aa.out = w.attn_o;
    aa.part_o = w.apart_o;
    aa.part_ml = w.apart_ml;
    aa.B = d.B;
    aa.S = d.S;
    aa.nq = d.nq;
    aa.nkv = d.nkv;
    aa.d = d.d;
    aa.max_ctx = d.max_ctx;
    aa.ctx_bound = ctx_bound;
    aa.R = d.R;
    aa.Rpad = d.Rpad;
    aa.n_ctx_splits = ap.n_ctx_splits;
    aa.row_groups = rgs;
    aa.window = cfg->window;
    aa.out_packed = xp_o;
    DFS_TRY(launch_attention(aa, dt, s));
    // 4. O projection, residual add, MLP pre-norm
    DFS_TRY(run_gemm(w.attn_o, d.nq * d.d, d.Mb, d.H, d.nq * d.d, wt->wo[l], nullptr, 0, nullptr, 0, w.part, dt,
                     pk, s, &sp, &pst, 0, 0, 0, xp_o));
    {
      NormArgs na;
      na.resid = w.resid;
      na.part = w.part;
      na.sp = sp;
      na.part_stride = pst;
      na.update_resid = 1;
      na.gain = wt->mlp_norm[l];
      na.out = w.mlp_in;
      na.out_packed = xp_mlp;
      na.rows = d.Mb;
      na.H = d.H;
      na.eps = cfg->rms_eps;
      DFS_TRY(launch_norm(na, dt, s));
    }
    // 5. SwiGLU MLP: gate and up in one weight pass (the product formed in the
    //    GEMM epilogue when a gated plan fits, else by a separate pass over the
    //    fp32 results), then down, residual add, next pre-norm
    if (gated.kind > 0) {
      DFS_TRY(run_gemm_gated(w.mlp_in, d.H, d.Mb, d.F, d.H, wt->w_gate[l], wt->w_up[l], w.hmid, pk, gated, s,
                             xp_mlp, xp_down));
    } else {
      DFS_TRY(run_gemm(w.mlp_in, d.H, d.Mb, 2 * d.F, d.H, wt->w_gate[l], wt->w_up[l], d.F, nullptr, 0, w.part, dt,
                       pk, s, &sp, &pst));
      DFS_TRY(launch_swiglu(w.part, sp, pst, d.Mb, d.F, w.hmid, dt, s));
    }
    DFS_TRY(run_gemm(w.hmid, d.F, d.Mb, d.H, d.F, wt->w_down[l], nullptr, 0, nullptr, 0, w.part, dt, pk, s,
                     &sp, &pst, 0, 0, 0, xp_down));
    {
      NormArgs na;
      na.resid = w.resid;
      na.part = w.part;
      na.sp = sp;
      na.part_stride = pst;
      na.update_resid = 1;
      na.rows = d.Mb;
      na.H = d.H;
      na.eps = cfg->rms_eps;
      if (l + 1 < d.L) {
        na.gain = wt->attn_norm[l + 1];
        na.out = xs_blk;
        na.out_packed = xp_qkv;
        na.out_row0 = xp_qkv ? d.Mc : 0;
      } else {   // final norm of the mask rows only -> z [B*(S-1), H]
        na.gain = wt->final_norm;
        na.out = w.z;
        na.out_mode = 1;
        na.S = d.S;
        na.out_packed = xp_lm;
      }
      DFS_TRY(launch_norm(na, dt, s));
    }
  }
  // 6. LM head on the mask rows -> base logits [B, S-1, V]
  // (the logits are not re-read before the sampler's pass: non-temporal stores)
  DFS_TRY(run_gemm(w.z, d.H, d.B * d.G, d.V, d.H, wt->lm_head, nullptr, 0, nullptr, 0, base_logits, dt, pk, s,
                   &sp, &pst, 1, 0, 1, xp_lm));
  return DFS_OK;
}

// ------------------------------------------------------------------ Markov head + sampling

// Draw position i of every request from its final logits: chunk statistics,
// then the inverse-CDF (or greedy) pick; writes d_i and the row's (max, sum).
static hipError_t sample_position(int batch, int n_draft, int vocab, int i, const float* logits,
                                  const float* u_draft, float temperature, int32_t* draft_tokens,
                                  double* row_stats, double2* stats, double* sub, hipStream_t s) {
  const long rowV = (long)n_draft * vocab;
  const hipError_t e =
      launch_chunk_stats(logits + (size_t)i * vocab, rowV, batch, vocab, temperature, stats, sub, s);
  if (e != hipSuccess) return e;
  PickArgs pa;
  pa.x = logits + (size_t)i * vocab;
  pa.row_stride = rowV;
  pa.rows = batch;
  pa.V = vocab;
  pa.temperature = temperature;
  pa.stats = stats;
  pa.sub = sub;
  pa.u = u_draft + i;
  pa.u_stride = n_draft;
  pa.tokens = draft_tokens + i;
  pa.tok_stride = n_draft;
  pa.row_stats = row_stats ? row_stats + 2 * i : nullptr;
  pa.rs_stride = 2 * (long)n_draft;
  return launch_pick(pa, s);
}

// statistics of every sampled row: per chunk (max, sum) and per 64-token sub-chunk sums
static size_t sample_carve(int B, int G, int V, void* base, double2** stats, double** sub,
                           double2** head_sub = nullptr) {
  Carver cv(base);
  const size_t nch = (size_t)ceil_div(V, kChunk);
  double2* st = cv.take<double2>((size_t)B * G * nch);
  double* sb = cv.take<double>((size_t)B * G * nch * 64);
  double2* hs = cv.take<double2>((size_t)B * ceil_div(V, 64));   // one position's head statistics
  if (stats) *stats = st;
  if (sub) *sub = sb;
  if (head_sub) *head_sub = hs;
  return cv.off + 256;
}

size_t markov_bias_sample_workspace_size(int32_t batch, int32_t n_draft, int32_t vocab) {
  if (batch < 1 || n_draft < 1 || vocab < 1) return 0;
  return sample_carve(batch, n_draft, vocab, nullptr, nullptr, nullptr);
}

int markov_bias_sample(int32_t batch, int32_t n_draft, int32_t vocab, int32_t rank, float* logits, const void* U,
                       const void* Wt, int32_t uw_dtype, const int32_t* last_token, const float* u_draft,
                       float temperature, int32_t* draft_tokens, double* row_stats, void* workspace,
                       size_t workspace_bytes, void* stream) {
  if (batch < 1 || n_draft < 1 || vocab < 1 || rank < 0 || !logits || !last_token || !u_draft || !draft_tokens ||
      !workspace)
    return DFS_EINVAL;
  if (vocab > kMaxVocab) return DFS_EUNSUPPORTED;
  if (!(temperature >= 0.f)) return DFS_EINVAL;
  if (rank > 0 && (!U || !Wt)) return DFS_EINVAL;
  if (rank > 0 && uw_dtype != DFS_F32 && uw_dtype != DFS_BF16 && uw_dtype != DFS_BF16_PACKED) return DFS_EINVAL;
  if (rank > 0 && uw_dtype != DFS_F32 && rank % 64 != 0) return DFS_EUNSUPPORTED;
  const int uw_packed = uw_dtype == DFS_BF16_PACKED;
  if (uw_packed) uw_dtype = DFS_BF16;
  if (workspace_bytes < markov_bias_sample_workspace_size(batch, n_draft, vocab)) return DFS_EWORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  double2* stats;
  double* sub;
  double2* head_sub;
  sample_carve(batch, n_draft, vocab, workspace, &stats, &sub, &head_sub);
  const long rowV = (long)n_draft * vocab;
  if (rank == 0) {
    ProfScope ps("sample", s);
    DFS_TRY(launch_chunk_stats(logits, vocab, batch * n_draft, vocab, temperature, stats, sub, s));
    PickArgs pa;
    pa.x = logits;
    pa.row_stride = vocab;
    pa.rows = batch * n_draft;
    pa.V = vocab;
    pa.temperature = temperature;
    pa.stats = stats;
    pa.sub = sub;
    pa.u = u_draft;
    pa.u_stride = 1;
    pa.tokens = draft_tokens;
    pa.tok_stride = 1;
    pa.row_stats = row_stats;
    pa.rs_stride = 2;
    DFS_TRY(launch_pick(pa, s));
    return DFS_OK;
  }
  ProfScope ps("markov", s);
  const GemmPlan plan = gemm_plan(batch, vocab, rank, uw_dtype, 1);
  // rank 256, up to 128 rows, bf16: the product writes the per-64-token statistics
  // the draw needs (2 launches per position instead of 3)
  const bool fused = uw_dtype == DFS_BF16 && rank == 256 && batch <= 128 && vocab % 4 == 0 &&
                     ceil_div(vocab, 64) <= kPickSubMax && ((uintptr_t)logits & 15) == 0;
  for (int i = 0; i < n_draft; ++i) {
    // final_i = base_i + U[prev] . W   (rows gathered by the previous token)
    GemmArgs ga;
    ga.X = U;
    ga.ldx = rank;
    ga.row_idx = i == 0 ? last_token : draft_tokens + (i - 1);
    ga.row_idx_stride = i == 0 ? 1 : n_draft;
    ga.x_rows = vocab;
    ga.M = batch;
    ga.N = vocab;
    ga.K = rank;
    ga.seg[0].w = Wt;
    ga.nseg = 1;
    ga.Y = logits + (size_t)i * vocab;
    ga.ldy = rowV;
    ga.y_split_stride = 0;
    ga.accumulate = 1;
    ga.packed = uw_packed;
    if (fused) {   // product + per-64-token statistics in one launch, then the draw
      DFS_TRY(launch_head_gemm_stats(ga, temperature, head_sub, s));
      PickArgs pa;
      pa.x = logits + (size_t)i * vocab;
      pa.row_stride = rowV;
      pa.rows = batch;
      pa.V = vocab;
      pa.temperature = temperature;
      pa.u = u_draft + i;
      pa.u_stride = n_draft;
      pa.tokens = draft_tokens + i;
      pa.tok_stride = n_draft;
      pa.row_stats = row_stats ? row_stats + 2 * i : nullptr;
      pa.rs_stride = 2 * (long)n_draft;
      DFS_TRY(launch_pick_sub(pa, head_sub, ceil_div(vocab, 64), s));
      continue;
    }
    DFS_TRY(launch_gemm(ga, plan, uw_dtype, s));
    DFS_TRY(sample_position(batch, n_draft, vocab, i, logits, u_draft, temperature, draft_tokens, row_stats, stats,
                            sub, s));
  }
  return DFS_OK;
}

// ------------------------------------------------------------------ RNN head + sampling

static size_t rnn_carve(int B, int G, int V, int r, void* base, double2** stats, double** sub, float** h,
                        bf16_t** split) {
  Carver cv(base);
  double2* st = cv.take<double2>((size_t)B * G * ceil_div(V, kChunk));
  double* sb = cv.take<double>((size_t)B * G * ceil_div(V, kChunk) * 64);
  float* hh = cv.take<float>((size_t)2 * B * r);   // two state buffers, alternating by position
  bf16_t* sp = cv.take<bf16_t>((size_t)3 * B * r);
  if (stats) *stats = st;
  if (sub) *sub = sb;
  if (h) *h = hh;
  if (split) *split = sp;
  return cv.off + 256;
}

size_t rnn_bias_sample_workspace_size(int32_t batch, int32_t n_draft, int32_t vocab, int32_t rank) {
  if (batch < 1 || n_draft < 1 || vocab < 1 || rank < 1 || rank > kRnnMaxRank) return 0;
  return rnn_carve(batch, n_draft, vocab, rank, nullptr, nullptr, nullptr, nullptr, nullptr);
}

int rnn_bias_sample(int32_t batch, int32_t n_draft, int32_t vocab, int32_t rank, float* logits, const void* U,
                    const void* Wt, const void* A, int32_t uw_dtype, const int32_t* last_token, const float* u_draft,
                    float temperature, int32_t* draft_tokens, double* row_stats, void* workspace,
                    size_t workspace_bytes, void* stream) {
  if (batch < 1 || n_draft < 1 || vocab < 1 || rank < 1 || !logits || !U || !Wt || !A || !last_token ||
      !u_draft || !draft_tokens || !workspace)
    return DFS_EINVAL;
  if (!(temperature >= 0.f)) return DFS_EINVAL;
  if (uw_dtype != DFS_F32 && uw_dtype != DFS_BF16 && uw_dtype != DFS_BF16_PACKED) return DFS_EINVAL;
  if (vocab > kMaxVocab || rank > kRnnMaxRank) return DFS_EUNSUPPORTED;
  if (uw_dtype != DFS_F32 && rank % 64 != 0) return DFS_EUNSUPPORTED;
  const int uw_packed = uw_dtype == DFS_BF16_PACKED;
  if (uw_packed) uw_dtype = DFS_BF16;
  if (workspace_bytes < rnn_bias_sample_workspace_size(batch, n_draft, vocab, rank)) return DFS_EWORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  double2* stats;
  double* sub;
  float* h;
  bf16_t* split;
  rnn_carve(batch, n_draft, vocab, rank, workspace, &stats, &sub, &h, &split);
  const bool bf = uw_dtype == DFS_BF16;
  const long rowV = (long)n_draft * vocab;
  ProfScope ps("markov", s);
  // bf16: X rows [hi | mid | lo] of the state (K = 3 rank) against W (rank columns, wrapping)
  const int kx = bf ? 3 * rank : rank;
  const GemmPlan plan = gemm_plan_wrapped(batch, vocab, kx, rank, uw_dtype);
  for (int i = 0; i < n_draft; ++i) {
    // h_i = tanh(U[prev_i] + A h_{i-1}), then final_i = base_i + W h_i
    RnnArgs ra;
    ra.U = U;
    ra.A = A;
    ra.prev = i == 0 ? last_token : draft_tokens + (i - 1);
    ra.prev_stride = i == 0 ? 1 : n_draft;
    float* h_new = h + (size_t)(i & 1) * batch * rank;
    ra.h_in = h + (size_t)((i + 1) & 1) * batch * rank;
    ra.h_out = h_new;
    ra.split = bf ? split : nullptr;
    ra.first = i == 0;
    ra.B = batch;
    ra.V = vocab;
    ra.r = rank;
    DFS_TRY(launch_rnn_state(ra, uw_dtype, s));
    // fp32: the state itself; bf16: its three bf16 terms in one pass over W
    GemmArgs ga;
    ga.X = bf ? (const void*)split : (const void*)h_new;
    ga.ldx = kx;
    ga.x_rows = batch;
    ga.M = batch;
    ga.N = vocab;
    ga.K = kx;
    ga.wk = rank;
    ga.seg[0].w = Wt;
    ga.nseg = 1;
    ga.Y = logits + (size_t)i * vocab;
    ga.ldy = rowV;
    ga.y_split_stride = 0;
    ga.accumulate = 1;
    ga.packed = uw_packed;
    DFS_TRY(launch_gemm(ga, plan, uw_dtype, s));
    DFS_TRY(sample_position(batch, n_draft, vocab, i, logits, u_draft, temperature, draft_tokens, row_stats, stats,
                            sub, s));
  }
  return DFS_OK;
}

// ------------------------------------------------------------------ verify

static size_t verify_carve(int B, int G, int V, void* base, VerifyArgs* a) {
  Carver cv(base);
  const size_t nch = (size_t)ceil_div(V, kChunk);
  double2* p_chunk = cv.take<double2>((size_t)B * (G + 1) * nch);
  double* p_sub = cv.take<double>((size_t)B * (G + 1) * nch * 64);
  double2* q_chunk = cv.take<double2>((size_t)B * G * nch);
  double* rowinfo = cv.take<double>((size_t)B * 4);
  int32_t* state = cv.take<int32_t>(B);
  double* res = cv.take<double>((size_t)B * nch * 4);
  double2* sub = cv.take<double2>((size_t)B * nch * 64);
  if (a) {
    a->p_chunk = p_chunk;
    a->p_sub = p_sub;
    a->q_chunk = q_chunk;
    a->rowinfo = rowinfo;
    a->state = state;
    a->res = res;
    a->sub = sub;
  }
  return cv.off + 256;
}

size_t spec_verify_workspace_size(int32_t batch, int32_t n_draft, int32_t vocab) {
  if (batch < 1 || n_draft < 1 || vocab < 1) return 0;
  return verify_carve(batch, n_draft, vocab, nullptr, nullptr);
}

static int verify_check(int32_t batch, int32_t n_draft, int32_t vocab, const float* draft_logits,
                        const float* target_logits, const int32_t* draft_tokens, const float* u_accept,
                        const float* u_final, float temperature, int32_t* out_tokens, int32_t* n_accepted) {
  if (batch < 1 || n_draft < 1 || vocab < 1 || !draft_logits || !target_logits || !draft_tokens || !u_accept ||
      !u_final || !out_tokens || !n_accepted)
    return DFS_EINVAL;
  if (vocab > kMaxVocab || n_draft > 64) return DFS_EUNSUPPORTED;   // one decide slot per position
  // the statistics pass runs one workgroup per (row, chunk) of the target and draft rows
  if ((size_t)batch * (2 * n_draft + 1) * ceil_div(vocab, kChunk) > 0x7fffffffu) return DFS_EUNSUPPORTED;
  if (!(temperature >= 0.f)) return DFS_EINVAL;
  return DFS_OK;
}

static int verify_run(int32_t batch, int32_t n_draft, int32_t vocab, const float* draft_logits,
                      const float* target_logits, const int32_t* draft_tokens, const float* u_accept,
                      const float* u_final, float temperature, const double* draft_row_stats, const int32_t* n_verify,
                      int32_t* out_tokens, int32_t* n_accepted, void* workspace, void* stream) {
  VerifyArgs a;
  verify_carve(batch, n_draft, vocab, workspace, &a);
  a.q = draft_logits;
  a.p = target_logits;
  a.drafts = draft_tokens;
  a.u_accept = u_accept;
  a.u_final = u_final;
  a.temperature = temperature;
  a.q_stats = draft_row_stats;
  a.n_verify = n_verify;
  a.out_tokens = out_tokens;
  a.n_accepted = n_accepted;
  a.B = batch;
  a.G = n_draft;
  a.V = vocab;
  DFS_TRY(launch_verify(a, (hipStream_t)stream));
  return DFS_OK;
}

int spec_verify(int32_t batch, int32_t n_draft, int32_t vocab, const float* draft_logits,
                const float* target_logits, const int32_t* draft_tokens, const float* u_accept,
                const float* u_final, float temperature, const double* draft_row_stats, const int32_t* n_verify,
                int32_t* out_tokens, int32_t* n_accepted, void* workspace, size_t workspace_bytes, void* stream) {
  const int st = verify_check(batch, n_draft, vocab, draft_logits, target_logits, draft_tokens, u_accept, u_final,
                              temperature, out_tokens, n_accepted);
  if (st != DFS_OK) return st;
  if (!workspace) return DFS_EINVAL;
  if (workspace_bytes < spec_verify_workspace_size(batch, n_draft, vocab)) return DFS_EWORKSPACE;
  return verify_run(batch, n_draft, vocab, draft_logits, target_logits, draft_tokens, u_accept, u_final, temperature,
                    draft_row_stats, n_verify, out_tokens, n_accepted, workspace, stream);
}

int spec_verify_static(int32_t batch, int32_t n_draft, int32_t vocab, const float* draft_logits,
                       const float* target_logits, const int32_t* draft_tokens, const float* u_accept,
                       const float* u_final, float temperature, const double* draft_row_stats,
                       const int32_t* n_verify, int32_t* out_tokens, int32_t* n_accepted, void* stream) {
  const int st = verify_check(batch, n_draft, vocab, draft_logits, target_logits, draft_tokens, u_accept, u_final,
                              temperature, out_tokens, n_accepted);
  if (st != DFS_OK) return st;
  if (spec_verify_workspace_size(batch, n_draft, vocab) > kStaticScratchBytes) return DFS_EWORKSPACE;
  void* ws = nullptr;
  const int sc = static_scratch(&ws);
  if (sc != DFS_OK) return sc;
  return verify_run(batch, n_draft, vocab, draft_logits, target_logits, draft_tokens, u_accept, u_final, temperature,
                    draft_row_stats, n_verify, out_tokens, n_accepted, ws, stream);
}

// ------------------------------------------------------------------ multi-step loop

int spec_cycle_advance(int32_t batch, int32_t n_draft, const int32_t* n_accepted, const int32_t* out_tokens,
                       int32_t* n_new, int32_t* last_token, int64_t* tau_sum, void* stream) {
  if (batch < 1 || n_draft < 0 || !n_accepted || !out_tokens || !n_new || !last_token) return DFS_EINVAL;
  if (n_draft > 64) return DFS_EUNSUPPORTED;
  DFS_TRY(launch_advance(batch, n_draft, n_accepted, out_tokens, n_new, last_token, tau_sum, (hipStream_t)stream));
  return DFS_OK;
}

int spec_schedule_verify(int32_t batch, int32_t n_draft, const float* survival, int32_t n_curve,
                         const float* curve_rows, const float* curve_sps, int32_t* n_verify, void* stream) {
  if (batch < 1 || n_draft < 1 || !survival || !curve_rows || !curve_sps || !n_verify || n_curve < 1)
    return DFS_EINVAL;
  if ((long)batch * n_draft > 8192 || n_curve > kSchedCurve) return DFS_EUNSUPPORTED;
  SchedArgs a;
  a.surv = survival;
  a.n_verify = n_verify;
  a.B = batch;
  a.G = n_draft;
  a.ncurve = n_curve;
  for (int i = 0; i < n_curve; ++i) {
    if (!(curve_sps[i] >= 0.f) || !(curve_rows[i] > 0.f)) return DFS_EINVAL;
    if (i > 0 && !(curve_rows[i] > curve_rows[i - 1])) return DFS_EINVAL;
    a.xs[i] = curve_rows[i];
    a.ys[i] = curve_sps[i];
  }
  DFS_TRY(launch_schedule(a, (hipStream_t)stream));
  return DFS_OK;
}

// ------------------------------------------------------------------ kernel-level hooks

size_t dfs_block_attention_workspace_size(int32_t batch, int32_t block, int32_t n_q_heads, int32_t n_kv_heads,
                                          int32_t head_dim, int32_t ctx_bound, int32_t dtype) {
  if (batch < 1 || block < 1 || block > 64 || n_q_heads < 1 || n_kv_heads < 1 || head_dim < 2 || ctx_bound < 1)
    return 0;
  const int R = n_q_heads / n_kv_heads * block, Rpad = (R + 15) / 16 * 16;
  const size_t es = dtype_size(dtype);
  Carver cv(nullptr);
  cv.take<char>((size_t)batch * n_kv_heads * Rpad * head_dim * es);
  cv.take<char>((size_t)batch * n_kv_heads * 64 * head_dim * es);
  cv.take<char>((size_t)batch * n_kv_heads * head_dim * 64 * es);
  const int rgs = dtype == DFS_BF16 ? ceil_div(R, 64) : 1;   // 64-row groups of the R query rows
  const AttnPlan ap = attn_plan(batch, n_kv_heads, ctx_bound, dtype, rgs);
  cv.take<float>(attn_partial_elems(ap.n_ctx_splits + 1, batch, n_kv_heads, Rpad, head_dim));
  cv.take<float>((size_t)batch * n_kv_heads * (ap.n_ctx_splits + 1) * Rpad * 2);
  return cv.off + 256;
}

int dfs_block_attention(int32_t batch, int32_t block, int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                        int32_t max_ctx, int32_t ctx_bound, int32_t dtype, int32_t window, const void* q,
                        const void* k_blk, const void* v_blk, const void* k_cache, const void* v_cache,
                        const int32_t* ctx_len, void* out, void* workspace, size_t workspace_bytes, void* stream) {
  if (!q || !k_blk || !v_blk || !k_cache || !v_cache || !ctx_len || !out || !workspace) return DFS_EINVAL;
  if (batch < 1 || block < 1 || n_q_heads < 1 || n_kv_heads < 1 || n_q_heads % n_kv_heads || max_ctx < 1 ||
      ctx_bound < 1 || ctx_bound > max_ctx || (dtype != DFS_F32 && dtype != DFS_BF16) || window < 0)
    return DFS_EINVAL;
  const int R = n_q_heads / n_kv_heads * block, Rpad = (R + 15) / 16 * 16;
  if (block > 64 || max_ctx % 64 || batch > 65535) return DFS_EUNSUPPORTED;
  if (dtype == DFS_BF16 && (head_dim != 128 || R > 256)) return DFS_EUNSUPPORTED;
  if (dtype == DFS_F32 && (head_dim > 256 || R > 256)) return DFS_EUNSUPPORTED;
  if (workspace_bytes <
      dfs_block_attention_workspace_size(batch, block, n_q_heads, n_kv_heads, head_dim, ctx_bound, dtype))
    return DFS_EWORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  const size_t es = dtype_size(dtype);
  Carver cv(workspace);
  char* q_att = cv.take<char>((size_t)batch * n_kv_heads * Rpad * head_dim * es);
  char* kb = cv.take<char>((size_t)batch * n_kv_heads * 64 * head_dim * es);
  char* vb = cv.take<char>((size_t)batch * n_kv_heads * head_dim * 64 * es);
  const int rgs = dtype == DFS_BF16 ? ceil_div(R, 64) : 1;   // 64-row groups of the R query rows
  const AttnPlan ap = attn_plan(batch, n_kv_heads, ctx_bound, dtype, rgs, window);
  float* po = cv.take<float>(attn_partial_elems(ap.n_ctx_splits + 1, batch, n_kv_heads, Rpad, head_dim));
  float* pml = cv.take<float>((size_t)batch * n_kv_heads * (ap.n_ctx_splits + 1) * Rpad * 2);
  DFS_TRY(launch_attn_stage(q, k_blk, v_blk, q_att, kb, vb, batch, block, n_q_heads, n_kv_heads, head_dim, Rpad,
                            dtype, s));
  AttnArgs aa;
  aa.q = q_att;
  aa.k_blk = kb;
  aa.v_blk = vb;
  aa.k_cache = k_cache;
  aa.v_cache = v_cache;
  aa.ctx_len = ctx_len;
  aa.out = out;
  aa.part_o = po;
  aa.part_ml = pml;
  aa.B = batch;
  aa.S = block;
  aa.nq = n_q_heads;
  aa.nkv = n_kv_heads;
  aa.d = head_dim;
  aa.max_ctx = max_ctx;
  aa.ctx_bound = ctx_bound;
  aa.R = R;
  aa.Rpad = Rpad;
  aa.n_ctx_splits = ap.n_ctx_splits;
  aa.row_groups = rgs;
  aa.window = window;
  DFS_TRY(launch_attention(aa, dtype, s));
  return DFS_OK;
}

size_t dfs_gemm_workspace_size(int32_t M, int32_t N, int32_t K, int32_t dtype, int32_t splits) {
  if (M < 1 || N < 1 || K < 1) return 0;
  const GemmPlan p = gemm_plan(M, N, K, dtype, splits);
  return p.splits > 1 ? align_up(gemm_partial_elems(p, M, N) * sizeof(float), 256) + 256 : 256;
}

int dfs_gemm(int32_t M, int32_t N, int32_t K, int32_t dtype, const void* X, const void* W, float* Y,
             int32_t splits, int32_t w_packed, void* workspace, size_t workspace_bytes, void* stream) {
  return dfs_gemm_skip(M, N, K, dtype, X, W, Y, splits, w_packed, 0, 0, workspace, workspace_bytes, stream);
}

int dfs_gemm_skip(int32_t M, int32_t N, int32_t K, int32_t dtype, const void* X, const void* W, float* Y,
                  int32_t splits, int32_t w_packed, int32_t skip_m, int32_t skip_n, void* workspace,
                  size_t workspace_bytes, void* stream) {
  if (M < 1 || N < 1 || K < 1 || !X || !W || !Y || splits < 0 || (dtype != DFS_F32 && dtype != DFS_BF16) ||
      (w_packed != 0 && w_packed != 1) || skip_m < 0 || skip_m > M || skip_n < 0 || skip_n > N)
    return DFS_EINVAL;
  if ((skip_m > 0 || skip_n > 0) && splits < 1) return DFS_EINVAL;   // the workspace size needs the split count
  if (dtype == DFS_BF16 && K % 64) return DFS_EUNSUPPORTED;
  if (w_packed && dtype != DFS_BF16) return DFS_EUNSUPPORTED;
  if (workspace_bytes < dfs_gemm_workspace_size(M, N, K, dtype, splits) || !workspace) return DFS_EWORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  const GemmPlan p = gemm_plan(M, N, K, dtype, splits, skip_m, skip_n);
  float* target = p.splits > 1 ? (float*)workspace : Y;
  int sp;
  size_t pst;
  DFS_TRY(run_gemm(X, K, M, N, K, W, nullptr, 0, nullptr, 0, target, dtype, w_packed, s, &sp, &pst, splits, 0, 0, 0,
                   skip_m, skip_n));
  if (sp > 1) DFS_TRY(launch_reduce(target, sp, pst, (size_t)M * N, Y, s));
  return DFS_OK;
}

int dfs_gemm_swiglu(int32_t M, int32_t F, int32_t K, const void* X, const void* Wg, const void* Wu, void* H,
                    int32_t w_packed, void* stream) {
  if (M < 1 || F < 1 || K < 1 || !X || !Wg || !Wu || !H || (w_packed != 0 && w_packed != 1)) return DFS_EINVAL;
  if (K % 64) return DFS_EUNSUPPORTED;
  const GemmPlan p = gemm_plan_gated(M, F, K, DFS_BF16);
  if (p.kind < 0) return DFS_EUNSUPPORTED;
  DFS_TRY(run_gemm_gated(X, K, M, F, K, Wg, Wu, H, w_packed, p, (hipStream_t)stream));
  return DFS_OK;
}

size_t dfs_packed_matrix_bytes(int32_t rows, int32_t cols) {
  if (rows < 1 || cols < 64 || cols % 64) return 0;
  return packed_matrix_elems(rows, cols) * sizeof(bf16_t);
}

int dfs_pack_matrix(int32_t rows, int32_t cols, const void* src, void* dst, void* stream) {
  if (rows < 1 || cols < 1 || !src || !dst || src == dst) return DFS_EINVAL;
  if (cols % 64) return DFS_EUNSUPPORTED;
  DFS_TRY(launch_pack(src, dst, rows, cols, (hipStream_t)stream));
  return DFS_OK;
}

}  // extern "C"
