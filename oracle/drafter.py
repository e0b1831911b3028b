"""Oracle of the DFlash-style block drafter forward pass.

[DFlash] architecture paragraph: the drafter is a small transformer.  Context
features are the hidden states of several target-model layers, concatenated,
linearly projected and normalised; the same features feed every drafter layer
("KV injection": each layer projects them to its keys and values, and only the
block's own states change from layer to layer).  The first layer receives the
last decoded token followed by mask tokens, all predicted in one forward pass.
Attention is full inside the block and causal toward the preceding context.
[DSpark] "Optymalizacja weryfikacji i wydajności": the drafter reuses the
target's embedding and output head.  [DSpark] "Innowacje w tworzeniu tokenów"
and [DSpark-fr] table "Ce que fait DSpark": one pass yields the base logits of
every block position.

Readings where the pages leave a step open (each is listed with its reason in
the design notes of the repository):

* normalisation = RMSNorm with gain g and epsilon eps: y = x / sqrt(mean(x^2) + eps) * g;
* each layer applies its own Wk, Wv (the ones used for block rows) to the
  features; the features are not re-normalised per layer;
* layer form: pre-norm; attention then SwiGLU MLP, each added to an fp32
  residual stream; no biases; score scale 1/sqrt(d); final RMSNorm before the
  LM head; grouped-query attention, query head h uses key/value head h // (nq/nkv);
* positions: rotate-half rotary embedding on queries and keys with base theta
  (theta <= 0 disables it); context row j of a sequence sits at position j,
  the block's last decoded token at C_b (the context length after the append)
  and mask token j at C_b + j;
* mask slot j (j = 1..S-1) predicts the token at slot j; slot 0 (the last
  decoded token) produces no logits;
* the mask token is a row of the shared embedding (mask_token_id);
* sliding window (the DSpark drafter variant of the DeepSeek-V4.1 notes page,
  section "DSpark — le décodage spéculatif": a 128-token window): with
  window > 0 a block row attends the last min(C_b, window) context keys and all
  S block keys; every appended row is still cached; positions are unchanged.

Storage boundaries (rounded exactly where the GPU path stores a tensor):
features, K/V, attention inputs/outputs, MLP input and SwiGLU product in the
weight dtype; residual stream and logits in fp32.

Arithmetic is float64 throughout.  ``arith=np.float32`` evaluates the same
steps with every operation in fp32 instead (storage roundings unchanged); the
gap between the two evaluations measures how far any correct fp32 evaluation
of this network can drift from the float64 one, and is used only as a
yardstick of conditioning.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .rounding import round_to, as_f64, round_f32, f64_to_bf16_bits


@dataclass(frozen=True)
class DrafterShape:
    n_layers: int
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    mlp_dim: int
    vocab: int
    n_target_layers: int
    block: int
    max_ctx: int
    mask_token_id: int
    rms_eps: float
    rope_theta: float
    dtype: str
    window: int = 0          # > 0: the block sees only the last `window` context keys

    @classmethod
    def of(cls, w) -> "DrafterShape":
        """Build from any object carrying the same attribute names."""
        return cls(**{f: getattr(w, f) for f in cls.__dataclass_fields__})


def rmsnorm(x, gain, eps, arith=np.float64):
    """y = x / sqrt(mean(x^2) + eps) * gain along the last axis."""
    x = np.asarray(x, dtype=arith)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + arith(eps)) * np.asarray(gain, dtype=arith)


def rope_rotate(x, positions, theta, arith=np.float64):
    """Rotate-half rotary embedding.

    x: [..., n_heads, d]; ``positions`` has shape x.shape[:-2] (one position
    per row, shared by its heads).  Pair (i, i + d/2) of every head is rotated
    by the angle pos * theta**(-2i/d) (angles and their sines in float64).
    """
    x = np.asarray(x, dtype=arith)
    if theta <= 0:
        return x.copy()
    d = x.shape[-1]
    half = d // 2
    inv_freq = theta ** (-np.arange(half, dtype=np.float64) * 2.0 / d)
    ang = np.asarray(positions, dtype=np.float64)[..., None] * inv_freq      # [..., half]
    cos = np.cos(ang).astype(arith)[..., None, :]
    sin = np.sin(ang).astype(arith)[..., None, :]
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * cos - x2 * sin, x2 * cos + x1 * sin], axis=-1)


def block_attention(q, k_ctx, v_ctx, k_blk, v_blk, arith=np.float64):
    """Attention of the block rows, by definition.

    q [S, nq, d]; k_ctx, v_ctx [C_b, nkv, d]; k_blk, v_blk [S, nkv, d].
    Every context key precedes every block row, so "causal toward the context"
    lets each block row see all C_b context keys, and "full inside the block"
    lets it see all S block keys.  Returns o [S, nq, d].
    """
    q = np.asarray(q, arith)
    keys = np.concatenate([np.asarray(k_ctx, arith), np.asarray(k_blk, arith)], 0)
    vals = np.concatenate([np.asarray(v_ctx, arith), np.asarray(v_blk, arith)], 0)
    S, nq, d = q.shape
    nkv = keys.shape[1]
    group = nq // nkv
    o = np.empty_like(q)
    for h in range(nq):
        g = h // group
        s = q[:, h, :] @ keys[:, g, :].T / arith(np.sqrt(d))   # [S, C_b + S]
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p /= p.sum(axis=1, keepdims=True)
        o[:, h, :] = p @ vals[:, g, :]
    return o


def _w(weights, name, dtype, arith=np.float64):
    return as_f64(weights[name], dtype).astype(arith, copy=False)


def context_features(shape: DrafterShape, weights, hidden_rows, arith=np.float64):
    """f = RMSNorm(concat_t(h_t) . W_fc^T; g_fc), rounded to the weight dtype.

    hidden_rows [n, nT*H] already concatenated in ascending target-layer order.
    """
    dt = shape.dtype
    h = as_f64(hidden_rows, dt).astype(arith, copy=False)
    y = h @ _w(weights, "fc", dt, arith).T
    return round_to(rmsnorm(y, _w(weights, "fc_norm", dt, arith), shape.rms_eps, arith), dt).astype(arith)


def draft_step(shape: DrafterShape, weights, hidden_new, n_new, k_cache, v_cache,
               ctx_len, last_token, batch_rows=None, arith=np.float64):
    """One drafter call: append the newly committed context rows, then draft a block.

    Arguments mirror the library entry point, in logical layouts:
      hidden_new [B, n_new_max, nT*H] (weight dtype storage), n_new [B],
      k_cache, v_cache [L, B, max_ctx, nkv, d] (weight dtype storage; modified
      in place at slots ctx_len[b] .. ctx_len[b]+n_new[b]-1), ctx_len [B]
      (not modified; the new lengths are returned), last_token [B].
    ``batch_rows`` restricts the work to some batch rows (others are skipped
    and their logits left as NaN).  ``arith``: float64, or float32 for the
    conditioning yardstick described in the module notes.
    Returns (base_logits [B, S-1, V] float32, new_ctx_len [B]).
    """
    sh = shape
    dt = sh.dtype
    B = len(n_new)
    S = sh.block
    nq, nkv, d, H = sh.n_q_heads, sh.n_kv_heads, sh.head_dim, sh.hidden
    rows = range(B) if batch_rows is None else list(batch_rows)
    F = arith

    def rnd(v):                     # storage rounding, back in the arithmetic type
        return round_to(v, dt).astype(F)

    def wt(name):
        return _w(weights, name, dt, F)

    new_len = np.asarray(ctx_len, np.int64) + np.asarray(n_new, np.int64)
    if np.any(new_len > sh.max_ctx):
        raise ValueError("context overflow")

    def store(cache, l, b, pos, val):
        # cache holds storage-format values; val is float64 already rounded to dt
        if dt == "bf16":
            cache[l, b, pos] = f64_to_bf16_bits(val)
        else:
            cache[l, b, pos] = val.astype(np.float32)

    # 1) context features of the newly committed rows, and 2) their K/V per layer
    feats = {}
    for b in rows:
        nb = int(n_new[b])
        if nb > 0:
            feats[b] = context_features(sh, weights, hidden_new[b, :nb], F)
    for l in range(sh.n_layers):
        wk = wt(f"layers.{l}.wk")
        wv = wt(f"layers.{l}.wv")
        for b, f in feats.items():
            pos = int(ctx_len[b]) + np.arange(f.shape[0])
            k = rope_rotate((f @ wk.T).reshape(-1, nkv, d), pos, sh.rope_theta, F)
            v = (f @ wv.T).reshape(-1, nkv, d)
            store(k_cache, l, b, pos, round_to(k, dt))
            store(v_cache, l, b, pos, round_to(v, dt))

    # 3) block: [last decoded token, MASK x (S-1)] at positions C_b .. C_b+S-1
    rows = list(rows)
    tok = np.full((len(rows), S), sh.mask_token_id, np.int64)
    tok[:, 0] = np.clip(np.asarray(last_token)[rows], 0, sh.vocab - 1)
    emb = wt("embed")
    x = round_f32(emb[tok]).astype(F)                         # [R, S, H] residual stream
    for l in range(sh.n_layers):
        x = drafter_layer(sh, weights, l, x, k_cache, v_cache, new_len, rows, arith)
    out = np.full((B, S - 1, sh.vocab), np.nan, np.float32)
    out[rows] = block_logits(sh, weights, x, arith)
    return out, new_len.astype(np.int32)


def drafter_layer(shape: DrafterShape, weights, l, x, k_cache, v_cache, new_len, rows, arith=np.float64):
    """Layer l of the drafter on the block rows' residual stream.

    x [R, S, H] (fp32 values) is the residual stream of batch rows ``rows`` on
    entry; k_cache, v_cache [L, B, max_ctx, nkv, d] hold every cached context row
    (the step's own appended rows included) and new_len [B] the context lengths
    after the append (the block sits at positions new_len[b] .. new_len[b]+S-1).
    Pre-norm attention over [cached context keys ; block keys], residual, pre-norm
    SwiGLU MLP, residual.  Returns the residual stream after the layer."""
    x1 = attention_half(shape, weights, l, x, k_cache, v_cache, new_len, rows, arith)
    m = mlp_input(shape, weights, l, x1, arith)
    return mlp_residual(shape, weights, l, x1, swiglu_product(shape, weights, l, m, arith), arith)


def attention_half(shape: DrafterShape, weights, l, x, k_cache, v_cache, new_len, rows, arith=np.float64):
    """x + Attention(RMSNorm(x)) . Wo of layer l (arguments as drafter_layer)."""
    sh = shape
    dt = sh.dtype
    S = sh.block
    nq, nkv, d = sh.n_q_heads, sh.n_kv_heads, sh.head_dim
    F = arith
    rows = list(rows)

    def rnd(v):                     # storage rounding, back in the arithmetic type
        return round_to(v, dt).astype(F)

    def wt(name):
        return _w(weights, name, dt, F)

    x = np.asarray(x, F)
    pos = np.asarray(new_len)[rows][:, None] + np.arange(S)[None, :]      # [R, S]
    p = f"layers.{l}."
    a = rnd(rmsnorm(x, wt(p + "attn_norm"), sh.rms_eps, F))
    q = rnd(rope_rotate((a @ wt(p + "wq").T).reshape(-1, S, nq, d), pos, sh.rope_theta, F))
    k = rnd(rope_rotate((a @ wt(p + "wk").T).reshape(-1, S, nkv, d), pos, sh.rope_theta, F))
    v = rnd((a @ wt(p + "wv").T).reshape(-1, S, nkv, d))
    o = np.empty_like(q)
    for i, b in enumerate(rows):
        cb = int(new_len[b])
        lo = max(0, cb - sh.window) if sh.window > 0 else 0     # sliding window: the last `window` keys
        kc = as_f64(k_cache[l, b, lo:cb], dt)
        vc = as_f64(v_cache[l, b, lo:cb], dt)
        o[i] = block_attention(q[i], kc, vc, k[i], v[i], F)
    o = rnd(o).reshape(-1, S, nq * d)
    return round_f32(x + o @ wt(p + "wo").T).astype(F)


def mlp_input(shape: DrafterShape, weights, l, x1, arith=np.float64):
    """m = RMSNorm(x1; g_mlp) of layer l, rounded to the weight dtype."""
    return round_to(rmsnorm(np.asarray(x1, arith), _w(weights, f"layers.{l}.mlp_norm", shape.dtype, arith),
                            shape.rms_eps, arith), shape.dtype).astype(arith)


def swiglu_product(shape: DrafterShape, weights, l, m, arith=np.float64):
    """silu(m . Wg^T) * (m . Wu^T) of layer l, rounded to the weight dtype."""
    F = arith
    m = np.asarray(m, F)
    g = m @ _w(weights, f"layers.{l}.w_gate", shape.dtype, F).T
    u = m @ _w(weights, f"layers.{l}.w_up", shape.dtype, F).T
    with np.errstate(over="ignore"):
        return round_to(g / (F(1) + np.exp(-g)) * u, shape.dtype).astype(F)       # silu(g) * u


def mlp_residual(shape: DrafterShape, weights, l, x1, hmid, arith=np.float64):
    """x1 + hmid . Wd^T of layer l, stored fp32."""
    F = arith
    return round_f32(np.asarray(x1, F) + np.asarray(hmid, F) @ _w(weights, f"layers.{l}.w_down", shape.dtype,
                                                                   F).T).astype(F)


def block_logits(shape: DrafterShape, weights, x, arith=np.float64):
    """Final RMSNorm of the mask rows (slots 1..S-1) and the LM head:
    x [R, S, H] residual stream -> base logits [R, S-1, V] float32."""
    sh = shape
    dt = sh.dtype
    F = arith
    z = round_to(rmsnorm(np.asarray(x, F)[:, 1:, :], _w(weights, "final_norm", dt, F), sh.rms_eps, F),
                 dt).astype(F)
    out = np.empty((z.shape[0], sh.block - 1, sh.vocab), np.float32)
    lm = weights["lm_head"]
    chunk = 16384
    for v0 in range(0, sh.vocab, chunk):
        wl = as_f64(lm[v0:v0 + chunk], dt).astype(F, copy=False)
        out[:, :, v0:v0 + chunk] = (z @ wl.T).astype(np.float32)
    return out
