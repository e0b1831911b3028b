/*
 * dfspec.h — C ABI of one block-parallel speculative draft-and-verify step on
 * AMD Instinct MI355X (gfx950).
 *
 * Three entry points, called in this order for one cycle:
 *
 *   dflash_draft_step   DFlash-style drafter forward pass.  Page "DFlash —
 *                       диффузионный метод спекулятивного декодинга"
 *                       (telemetr.me), architecture paragraph: hidden states of
 *                       several target layers are concatenated, linearly
 *                       projected and normalised into context features; the same
 *                       features enter every drafter layer as keys/values ("KV
 *                       injection"); the block is the last decoded token plus
 *                       mask tokens, predicted in one pass; attention is full
 *                       inside the block and causal toward the context.
 *   markov_bias_sample  DSpark sequential head + sampling.  Page "DeepSeek
 *                       prezentuje DSpark: przyspieszenie generowania
 *                       DeepSeek-V4 o 60-85%" (aigest.pl), section "Innowacje w
 *                       tworzeniu tokenów": a light sequential head adds a bias
 *                       that depends on the previous token (Markov head,
 *                       low-rank factorisation, rank 256) to each position's base
 *                       logits before that position is sampled.
 *   rnn_bias_sample     The optional RNN sequential head of the same section
 *                       (it follows the whole block prefix), same sampling.
 *   spec_verify         Rejection-sampling verification.  Same DSpark page,
 *                       section "Jak działa spekulatywne dekodowanie DSpark?":
 *                       the target keeps the longest valid prefix and adds one
 *                       token, exactly preserving the target distribution.  The
 *                       rule is the standard speculative-sampling one: accept
 *                       draft d_i while u_i < p_i(d_i)/q_i(d_i); at the first
 *                       rejection draw from normalise(max(0, p - q)); after a
 *                       fully accepted block draw one bonus token from p.
 *
 * Conventions for every function below
 *  - Tensor pointers are DEVICE pointers unless marked "host".  All tensors are
 *    dense, row-major, in the layouts stated.  The caller owns every buffer,
 *    including the workspace; the library allocates no device memory, never
 *    synchronises, and enqueues all work on `stream` (a hipStream_t; NULL = the
 *    null stream).  Results are valid once the caller has synchronised with
 *    that stream.  Its mutable global state is the opt-in timing hook
 *    dfs_profile_begin/end (process-wide, not thread-safe; disarmed by default,
 *    when it costs one flag test per launch) and the per-GPU static scratch of
 *    spec_verify_static (below).
 *  - Return value: DFS_OK (0) or a negative dfs_status.  Every shape, pointer
 *    and size check is done on the host before anything is enqueued; on error
 *    nothing is enqueued and no output is touched.  DFS_EHIP reports a failed
 *    launch (hipGetLastError), in which case outputs are unspecified.
 *  - Device-resident integers (token ids, lengths) are not visible to the host
 *    checks.  Kernels clamp them so that no access leaves its buffer: an
 *    out-of-range last token is clamped to [0, V-1]; an out-of-range draft token
 *    is treated as rejected by spec_verify.
 *  - Calls on one stream are ordered; concurrent calls on different streams
 *    must not share a workspace or any output buffer.
 */
#ifndef DFSPEC_H
#define DFSPEC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DFS_OK = 0,
  DFS_EINVAL = -1,        /* null pointer, negative or inconsistent size */
  DFS_EUNSUPPORTED = -2,  /* valid but outside what the kernels implement (see each call) */
  DFS_EHIP = -3,          /* a HIP launch failed */
  DFS_EWORKSPACE = -4     /* workspace smaller than the matching *_workspace_size() */
} dfs_status;

typedef enum {
  DFS_F32 = 0,
  DFS_BF16 = 1,
  DFS_BF16_PACKED = 2   /* a bf16 weight matrix in the tile-packed layout of dfs_pack_matrix */
} dfs_dtype;

/* Drafter shape.  B (batch) and the per-call row counts are arguments of the
 * calls, not part of the configuration. */
typedef struct {
  int32_t n_layers;        /* L >= 1 */
  int32_t hidden;          /* H */
  int32_t n_q_heads;       /* nq, a multiple of n_kv_heads */
  int32_t n_kv_heads;      /* nkv */
  int32_t head_dim;        /* d, even */
  int32_t mlp_dim;         /* F (SwiGLU width) */
  int32_t vocab;           /* V */
  int32_t n_target_layers; /* nT: target layers whose hidden states are concatenated */
  int32_t block;           /* S = 1 last decoded token + (S-1) mask tokens, S >= 2 */
  int32_t max_ctx;         /* cache slots per sequence, a multiple of 64; preferably not a
                              multiple of 1024: at a large power-of-two stride every (row,
                              head) cache block starts on the same HBM channels (measured
                              ~10 % slower attention at 2048 than at 2112 slots) */
  int32_t mask_token_id;   /* embedding row used for every mask slot, in [0, V) */
  float rms_eps;           /* RMSNorm: y = x / sqrt(mean(x^2) + eps) * g */
  float rope_theta;        /* rotate-half rotary base; <= 0 disables rotary embedding */
  int32_t dtype;           /* dfs_dtype of weights, hidden states, caches and activations */
  int32_t window;          /* > 0: block rows attend only the last `window` context keys (the
                              DSpark drafter's sliding window, DeepSeek-V4.1 notes page, section
                              "DSpark — le décodage spéculatif"); 0: the whole context */
} dfs_drafter_cfg;

/* Drafter weights, all in cfg.dtype, matrices stored [out, in] (row = output
 * feature, inputs contiguous), or — with packed = 1, bf16 only — every matrix
 * except the embedding in the tile-packed layout written by dfs_pack_matrix
 * (the layout the matrix-core kernels stream at full HBM bandwidth; pack once
 * at load time).  The per-layer members point to HOST arrays of L device
 * pointers.  The embedding and LM head are the target's, reused (DSpark page,
 * section "Optymalizacja weryfikacji i wydajności"). */
typedef struct {
  const void* embed;       /* [V, H] */
  const void* fc;          /* [H, nT*H]; input = target hiddens concatenated in ascending layer order */
  const void* fc_norm;     /* [H] RMSNorm gain of the context features */
  const void* final_norm;  /* [H] */
  const void* lm_head;     /* [V, H] */
  const void* const* attn_norm; /* L x [H] */
  const void* const* wq;        /* L x [nq*d, H] */
  const void* const* wk;        /* L x [nkv*d, H] */
  const void* const* wv;        /* L x [nkv*d, H] */
  const void* const* wo;        /* L x [H, nq*d] */
  const void* const* mlp_norm;  /* L x [H] */
  const void* const* w_gate;    /* L x [F, H] */
  const void* const* w_up;      /* L x [F, H] */
  const void* const* w_down;    /* L x [H, F] */
  int32_t packed;               /* 0: row-major matrices; 1: tile-packed (fc, wq, wk, wv, wo, w_gate,
                                   w_up, w_down, lm_head), DFS_EUNSUPPORTED for fp32 */
} dfs_drafter_weights;

/* ------------------------------------------------------------------ draft */

/* Bytes of workspace dflash_draft_step needs for this batch and n_new_max.
 * Returns 0 for an invalid configuration. */
size_t dflash_draft_workspace_size(const dfs_drafter_cfg* cfg, int32_t batch, int32_t n_new_max);

/* One drafter call.
 *
 * 1. Context features of the rows the target committed since the previous
 *    call: f = RMSNorm(hidden_new[b, j] . fc^T; fc_norm) for j < n_new[b].
 * 2. KV injection: for every layer l, K = RoPE(f . wk[l]^T), V = f . wv[l]^T are
 *    written to cache slots ctx_len[b] + j (positions ctx_len[b] + j).
 * 3. The block [last_token[b], mask x (S-1)] at positions C_b .. C_b+S-1, where
 *    C_b = ctx_len[b] + n_new[b], runs through the L pre-norm layers
 *    (attention over the C_b cached keys — the last min(C_b, cfg.window) of them
 *    when cfg.window > 0 — and the S block keys, full inside the block; then a
 *    SwiGLU MLP; fp32 residual stream).
 * 4. base_logits[b, j-1] = RMSNorm(x_j; final_norm) . lm_head^T for mask slot
 *    j = 1..S-1 (slot j predicts the token at slot j).
 * 5. ctx_len[b] is advanced to C_b.
 *
 * hidden_new  [B, n_new_max, nT*H] cfg.dtype; rows j >= n_new[b] are ignored.
 * n_new       [B] int32 (device), values clamped to [0, n_new_max].  A prefill
 *             is a call (or several) with large n_new_max.
 * n_new_max   host, >= 0.
 * ctx_bound   host, 1 <= ctx_bound <= max_ctx, and ctx_bound >= ctx_len[b] +
 *             n_new[b] for every b (used to size the attention grid).  A row
 *             that breaks it is computed with C_b clamped to ctx_bound (memory
 *             safe, result unspecified).
 * k_cache     [L, B, nkv, max_ctx, d] cfg.dtype, in/out, keys after RoPE.
 * v_cache     [L, B, nkv, d, max_ctx] cfg.dtype, in/out — values stored
 *             transposed (slots contiguous) so the attention kernel reads them
 *             as matrix-core operands straight from memory.
 *             Slots >= C_b are never read (they may hold anything).
 * ctx_len     [B] int32 (device), in/out.
 * last_token  [B] int32 (device).
 * base_logits [B, S-1, V] fp32, out.
 *
 * DFS_EUNSUPPORTED for cfg.dtype == DFS_BF16 unless head_dim == 128,
 * hidden, nq*d, mlp_dim, nT*H are multiples of 64 and (nq/nkv)*S <= 256;
 * for DFS_F32 unless head_dim <= 256 and (nq/nkv)*S <= 256.
 */
int dflash_draft_step(const dfs_drafter_cfg* cfg, const dfs_drafter_weights* weights,
                      int32_t batch, const void* hidden_new, const int32_t* n_new,
                      int32_t n_new_max, int32_t ctx_bound, void* k_cache, void* v_cache,
                      int32_t* ctx_len, const int32_t* last_token, float* base_logits,
                      void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------ Markov + sample */

size_t markov_bias_sample_workspace_size(int32_t batch, int32_t n_draft, int32_t vocab);

/* Sequential head and sampling of the gamma = n_draft draft positions.
 *
 * For i = 1..gamma (prev_1 = last_token[b], prev_i = d_{i-1}):
 *   final_i = base_i + U[prev_i] . W      (rank > 0; W stored transposed as Wt)
 *   d_i     = inverse-CDF draw from softmax(final_i / T) with u_draft[b, i]
 *             (token ids scanned in increasing order; first k whose running
 *             sum exceeds u * total), or the lowest-index argmax when T == 0.
 * With rank == 0 there is no head and all positions are drawn independently.
 *
 * logits      [B, gamma, V] fp32, in: base logits, out: final logits (in place).
 * U, Wt       [V, rank] in uw_dtype (NULL when rank == 0).  uw_dtype =
 *             DFS_BF16_PACKED: U row-major bf16, Wt tile-packed by dfs_pack_matrix.
 * last_token  [B] int32; out-of-range previous tokens are clamped to [0, V-1].
 * u_draft     [B, gamma] fp32 in [0, 1).
 * temperature host, >= 0.
 * draft_tokens[B, gamma] int32 out.
 * row_stats   [B, gamma, 2] fp64 out, may be NULL: (max, sum exp((x - max)/T))
 *             of each final row (T == 0: (max, 1)); spec_verify can reuse them.
 *
 * DFS_EUNSUPPORTED for a bf16 head unless rank is a multiple of 64, and for
 * vocab > 4194304.
 */
int markov_bias_sample(int32_t batch, int32_t n_draft, int32_t vocab, int32_t rank,
                       float* logits, const void* U, const void* Wt, int32_t uw_dtype,
                       const int32_t* last_token, const float* u_draft, float temperature,
                       int32_t* draft_tokens, double* row_stats, void* workspace,
                       size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------- RNN + sample */

size_t rnn_bias_sample_workspace_size(int32_t batch, int32_t n_draft, int32_t vocab, int32_t rank);

/* The optional RNN sequential head of the same DSpark page and section ("Innowacje
 * w tworzeniu tokenów": a head that follows the whole block prefix instead of the
 * previous token only).  The page gives no structure; the cell implemented is an
 * Elman tanh cell whose state has the head's rank r, fed the previous token
 * through the Markov head's input factor:
 *   h_0 = 0,  h_i = tanh(U[prev_i] + A h_{i-1}),  final_i = base_i + W h_i
 * (prev_1 = last_token[b], prev_i = d_{i-1}), each d_i drawn as in
 * markov_bias_sample.  The state is kept in fp32; with bf16 factors W h_i is
 * formed from three bf16 terms of h_i (hi + mid + lo) in one matrix-core pass
 * over W, i.e. to fp32 accuracy.
 *
 * logits, last_token, u_draft, temperature, draft_tokens, row_stats: as for
 *             markov_bias_sample.
 * U, Wt       [V, rank] in uw_dtype (DFS_F32, DFS_BF16, or DFS_BF16_PACKED: Wt
 *             tile-packed by dfs_pack_matrix, U row-major bf16).
 * A           [rank, rank] row-major, fp32 for DFS_F32 else bf16; A[j][k]
 *             weights state element k of h_{i-1} into element j of h_i.
 * workspace   rnn_bias_sample_workspace_size bytes (holds the state between
 *             positions; nothing persists across calls).
 *
 * DFS_EINVAL for rank < 1 or null pointers; DFS_EUNSUPPORTED for rank > 1024,
 * a bf16 head unless rank is a multiple of 64, and vocab > 4194304.
 */
int rnn_bias_sample(int32_t batch, int32_t n_draft, int32_t vocab, int32_t rank, float* logits,
                    const void* U, const void* Wt, const void* A, int32_t uw_dtype,
                    const int32_t* last_token, const float* u_draft, float temperature,
                    int32_t* draft_tokens, double* row_stats, void* workspace,
                    size_t workspace_bytes, void* stream);

/* ----------------------------------------------------------------- verify */

size_t spec_verify_workspace_size(int32_t batch, int32_t n_draft, int32_t vocab);

/* Rejection-sampling verification of gamma = n_draft draft tokens per row.
 *
 * p_i = softmax(target_logits[b, i] / T), q_i = softmax(draft_logits[b, i] / T).
 * For i = 1..gamma: accept d_i iff u_accept[b, i] < p_i(d_i) / q_i(d_i)
 * (q = 0 counts as +inf when p > 0, else 0; an out-of-range d_i is rejected).
 * At the first rejection a: out token = inverse-CDF draw with u_final[b] from
 * max(0, p_a - q_a) (from p_a if that has no mass).  If all are accepted: bonus
 * token = draw from p_{gamma+1} with u_final[b].  T == 0: greedy (accept while
 * d_i equals the target argmax, emit the argmax).
 *
 * draft_logits   [B, gamma, V] fp32 (the final logits the drafts were drawn from).
 * target_logits  [B, gamma+1, V] fp32.
 * draft_tokens   [B, gamma] int32.
 * u_accept       [B, gamma] fp32; u_final [B] fp32.
 * draft_row_stats[B, gamma, 2] fp64 from markov_bias_sample, or NULL to recompute.
 *                They hold the draft rows' (max, sum exp((x - max)/T)) at the
 *                temperature of the markov_bias_sample call that wrote them, so
 *                they may only be passed when that call used the same
 *                temperature as this one (pass NULL otherwise); T == 0 stats
 *                (max, 1) are not used by greedy verification.
 * n_verify       [B] int32 or NULL: row b verifies only its first k_b = n_verify[b]
 *                drafts (clamped to [0, gamma]; NULL = gamma) — the prefix
 *                scheduler's early stopping (same DSpark page, section
 *                "Optymalizacja weryfikacji i wydajności": per-request verify
 *                length, losslessness kept).  If those k_b are all accepted the
 *                bonus token is drawn from target row k_b, so target_logits rows
 *                0..k_b must be valid; the rule is the one above on a k_b-draft
 *                block, hence still exact.
 * out_tokens     [B, gamma+1] int32 out: accepted drafts, the correction or bonus
 *                token, then -1.
 * n_accepted     [B] int32 out, in [0, k_b]; the cycle yields n_accepted + 1 tokens.
 *
 * DFS_EUNSUPPORTED for vocab > 4194304 or n_draft > 64.
 */
int spec_verify(int32_t batch, int32_t n_draft, int32_t vocab, const float* draft_logits,
                const float* target_logits, const int32_t* draft_tokens, const float* u_accept,
                const float* u_final, float temperature, const double* draft_row_stats,
                const int32_t* n_verify, int32_t* out_tokens, int32_t* n_accepted, void* workspace,
                size_t workspace_bytes, void* stream);

/* spec_verify for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * arguments and results as spec_verify without the workspace.  Its scratch is a
 * static device array of 64 MiB inside the library, one copy per GPU the library
 * runs on, held until the process ends; the call allocates nothing (no
 * hipMalloc, hipFree or allocating library routine).  Every call on one GPU
 * shares that GPU's array, so calls that overlap on one GPU (different streams,
 * threads or processes sharing the library instance) race and must be ordered by
 * the caller; nothing in the array needs to start at zero and each call
 * overwrites what it reads.  DFS_EWORKSPACE when spec_verify_workspace_size()
 * of the arguments exceeds 64 MiB; otherwise the checks and errors of
 * spec_verify, plus DFS_EHIP if the array's device address cannot be obtained. */
int spec_verify_static(int32_t batch, int32_t n_draft, int32_t vocab, const float* draft_logits,
                       const float* target_logits, const int32_t* draft_tokens, const float* u_accept,
                       const float* u_final, float temperature, const double* draft_row_stats,
                       const int32_t* n_verify, int32_t* out_tokens, int32_t* n_accepted, void* stream);

/* ------------------------------------------------------------ multi-step loop */

/* Device-side bookkeeping between two cycles, so that draft -> sample -> verify
 * -> advance -> draft ... runs on one stream with no host synchronisation (and
 * can be captured into a HIP graph).  Same DSpark page, section "Jak działa
 * spekulatywne dekodowanie DSpark?": a cycle commits the accepted prefix plus
 * one token, tau = n_accepted + 1 tokens; the committed tokens are what the
 * next drafter call appends as context (their target hidden states) and the
 * last of them starts the next block.  For each row b, a = n_accepted[b]
 * clamped to [0, n_draft]:
 *   n_new[b]       = a + 1              (rows the next dflash_draft_step appends)
 *   last_token[b]  = out_tokens[b, a]   (the correction or bonus token)
 *   tau_sum[b]    += a + 1              (running count of committed tokens)
 * n_accepted [B] int32, out_tokens [B, n_draft+1] int32 (spec_verify's outputs,
 * may alias nothing written here); n_new, last_token [B] int32 out; tau_sum [B]
 * int64 in/out, or NULL.  No workspace.  DFS_EINVAL for null required pointers,
 * batch < 1 or n_draft < 0; DFS_EUNSUPPORTED for n_draft > 64.
 * A graph-captured chain needs host-side bounds that hold for every captured
 * cycle: dflash_draft_step's n_new_max = S and ctx_bound = the cache capacity. */
int spec_cycle_advance(int32_t batch, int32_t n_draft, const int32_t* n_accepted, const int32_t* out_tokens,
                       int32_t* n_new, int32_t* last_token, int64_t* tau_sum, void* stream);

/* Hardware-aware prefix scheduler: a verify length per request (same DSpark
 * page, section "Optymalizacja weryfikacji i wydajności": the verify length of
 * each request is set from a throughput curve SPS(B) profiled once at startup,
 * more tokens when the GPUs are idle and fewer when busy, losslessness kept by
 * early stopping; DeepSeek-V4.1 notes page, section "DSpark — le décodage
 * spéculatif": prefix survival probabilities combined with the measured curve to
 * maximise the expected system throughput).
 * survival [B, n_draft] fp32 (device): per-position survival scores c[b, i] (the
 *   chance that draft i survives given its predecessors did), clipped to [0, 1],
 *   NaN = 0; P[b, j] = c[b, 0] * ... * c[b, j] (fp64).
 * curve_rows, curve_sps [n_curve] (HOST, copied at the call; 1 <= n_curve <= 32):
 *   verify passes per second at that many rows in the verify batch; rows strictly
 *   increasing and > 0, sps >= 0; linear between points, constant past the ends.
 * n_verify [B] int32 out (device): k_b in [0, n_draft] maximising
 *   SPS(sum_b (k_b + 1)) * sum_b (1 + sum_{j < k_b} P[b, j]) — exact: P does not
 *   increase along a request, so the best k for M verified drafts take the M
 *   largest P (ties: lower request, then lower position) and M is scanned; the
 *   first maximum wins.  Feed n_verify to spec_verify.
 * DFS_EINVAL for null pointers, batch or n_draft < 1, a bad curve;
 * DFS_EUNSUPPORTED for batch * n_draft > 8192 or n_curve > 32. */
int spec_schedule_verify(int32_t batch, int32_t n_draft, const float* survival, int32_t n_curve,
                         const float* curve_rows, const float* curve_sps, int32_t* n_verify, void* stream);

/* ------------------------------------------------------------------ misc */

const char* dfs_status_string(int status);

/* Kernel-level hooks used by tests and the benchmark. */

/* Block attention alone, same math and layouts as inside dflash_draft_step:
 * q [B, S, nq, d], k_blk [B, S, nkv, d], v_blk [B, S, nkv, d] (all cfg dtype),
 * caches as above for ONE layer ([B, nkv, max_ctx, d] and [B, nkv, d, max_ctx]),
 * ctx_len [B] int32 = context keys of each row, out [B, S, nq, d] cfg dtype;
 * window > 0 restricts each row to its last `window` context keys (cfg.window). */
size_t dfs_block_attention_workspace_size(int32_t batch, int32_t block, int32_t n_q_heads,
                                          int32_t n_kv_heads, int32_t head_dim, int32_t ctx_bound,
                                          int32_t dtype);
int dfs_block_attention(int32_t batch, int32_t block, int32_t n_q_heads, int32_t n_kv_heads,
                        int32_t head_dim, int32_t max_ctx, int32_t ctx_bound, int32_t dtype, int32_t window,
                        const void* q, const void* k_blk, const void* v_blk, const void* k_cache,
                        const void* v_cache, const int32_t* ctx_len, void* out, void* workspace,
                        size_t workspace_bytes, void* stream);

/* Where dflash_draft_step leaves three intermediates of its LAST layer in the
 * workspace, for stage-by-stage parity tests (run the call with a prefix of the
 * layers to see any layer).  After a call, at byte offsets[k] of the workspace:
 *   k = 0  the fp32 residual stream [B*S, H] after the layer (the input of the
 *          next layer, or of the final norm);
 *   k = 1  the MLP input m = RMSNorm(x + attention output) [B*S, H] in cfg dtype;
 *   k = 2  the gated product silu(m Wg^T) * (m Wu^T) [B*S, F] in cfg dtype.
 * packed[k] = 1 when that tensor is stored in the tile-packed activation layout
 * (rows in groups of 16, each group's columns in 64-wide 2 KB tiles in
 * matrix-core operand order: element (r, c) of a tensor with C columns at
 * ((r/16)*(C/64) + c/64)*1024 + ((c/32)%2)*512 + (r%16 + 16*((c/8)%4))*8 + c%8),
 * else 0 (row-major).  offsets [3] and packed [3] are HOST arrays.
 * DFS_EINVAL / DFS_EUNSUPPORTED as for dflash_draft_workspace_size's inputs. */
int dfs_draft_trace_layout(const dfs_drafter_cfg* cfg, int32_t batch, int32_t n_new_max, size_t* offsets,
                           int32_t* packed);

/* Y[M, N] fp32 = X[M, K] . W[N, K]^T, both in `dtype`; the matrix-core kernel of
 * the drafter (split over K when `splits` > 1; splits = 0 picks automatically).
 * w_packed = 1: W is tile-packed (bf16 only). */
size_t dfs_gemm_workspace_size(int32_t M, int32_t N, int32_t K, int32_t dtype, int32_t splits);
int dfs_gemm(int32_t M, int32_t N, int32_t K, int32_t dtype, const void* X, const void* W,
             float* Y, int32_t splits, int32_t w_packed, void* workspace, size_t workspace_bytes,
             void* stream);

/* dfs_gemm with a skipped corner, the form dflash_draft_step's Q|K|V product takes
 * (the new context rows need keys and values only, no queries): output tiles lying
 * entirely inside rows [0, skip_m) x columns [0, skip_n) may be left uncomputed.
 * Y outside that corner is X . W^T as for dfs_gemm; inside it Y is unspecified (untouched by the
 * tiles the kernels skip, overwritten by a split-K reduction or by kernels that
 * compute every tile).  0 <= skip_m <= M, 0 <= skip_n <= N; with a skipped corner
 * `splits` must be >= 1 (the split count dfs_gemm_workspace_size was asked for).
 * DFS_EINVAL otherwise; the other errors as for dfs_gemm. */
int dfs_gemm_skip(int32_t M, int32_t N, int32_t K, int32_t dtype, const void* X, const void* W,
                  float* Y, int32_t splits, int32_t w_packed, int32_t skip_m, int32_t skip_n,
                  void* workspace, size_t workspace_bytes, void* stream);

/* H[M, F] bf16 = silu(X . Wg^T) * (X . Wu^T), the gated gate|up product of the
 * drafter's SwiGLU MLP (the layer form read for the DFlash drafter: pre-norm
 * attention then a SwiGLU MLP), computed in the epilogue of the drafter's
 * matrix-core GEMM: fp32 sums, silu and product in fp32, one rounding to bf16.
 * X [M, K] bf16 row-major; Wg, Wu [F, K] bf16, both row-major or both
 * tile-packed (w_packed = 1, see below); H [M, F] bf16 row-major.  All device
 * pointers, caller-owned, no workspace; runs on `stream`.  DFS_EINVAL for null
 * pointers or non-positive sizes, DFS_EUNSUPPORTED unless K is a multiple of 64. */
int dfs_gemm_swiglu(int32_t M, int32_t F, int32_t K, const void* X, const void* Wg, const void* Wu,
                    void* H, int32_t w_packed, void* stream);

/* Weight layout for the matrix-core kernels.  A bf16 matrix W [rows, cols]
 * (cols a multiple of 64) becomes ceil(rows/16) x (cols/64) tiles of 16 rows x
 * 64 columns, row-tile major; each 2 KB tile holds [half h = 0..1][lane l =
 * 0..63][8 values]: row 16*t + (l % 16), columns 64*c + 32*h + 8*(l / 16) .. +7,
 * i.e. exactly the operand fragment each lane of a wave feeds the 16x16x32
 * matrix instruction; rows past `rows` are zero.  One k step of 16 rows is
 * then two contiguous kilobytes, the access pattern HBM streams best.
 * dfs_packed_matrix_bytes returns 0 for unsupported shapes.  dfs_pack_matrix
 * reads src (row-major, device) and writes dst (device, that many bytes, not
 * overlapping src) on `stream`. */
size_t dfs_packed_matrix_bytes(int32_t rows, int32_t cols);
int dfs_pack_matrix(int32_t rows, int32_t cols, const void* src, void* dst, void* stream);

/* Per-kernel timing with HIP events recorded around every launch of the named
 * kernel group on the launching stream ("gemm", "attention", "sample", "verify",
 * "markov", "elementwise").  dfs_profile_begin arms recording for at most
 * max_launches launches (host allocates the events once, outside any timed
 * region); dfs_profile_end synchronises the events and returns the number of
 * launches recorded and their summed duration in milliseconds. */
int dfs_profile_begin(const char* group, int32_t max_launches);
int dfs_profile_end(int32_t* launches, double* total_ms);

#ifdef __cplusplus
}
#endif
#endif /* DFSPEC_H */
