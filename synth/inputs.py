"""Synthetic inputs of the draft-and-verify step (seeded; no method arithmetic).

Distributions (per workload, see ``configs.Workload``):
  weights (embedding, feature projection, Q/K/V/O, gate/up/down, LM head) ~ N(0, 0.02^2),
      stored in the workload dtype (bf16 rounded to nearest even, or fp32);
  norm gains 1 (or 1 + N(0, gain_std^2) for tests that must see the gain);
  target hidden states ~ N(0, 1); Markov factors U, Wt [V, r] ~ N(0, std^2);
  K/V cache prefix ~ N(0, kv_std^2) (the spread of K = f Wk^T for unit-RMS f
      and 0.02 weights at H = 4096: 0.02 * 64 = 1.28);
  target logits ~ N(0, std^2) fp32, or draft logits + N(0, noise^2);
  uniforms U[0, 1) fp32; last decoded token uniform in [0, V-1).
Layouts are the logical ones: caches [L, B, max_ctx, nkv, d]; weight matrices
[out, in].
"""
from __future__ import annotations

import numpy as np

from . import rng
from .configs import Workload


def drafter_weights(w: Workload, seed: int, gain_std: float = 0.0, layers=None) -> dict:
    dt = w.dtype
    H, nq, nkv, d, F, V, nT = (w.hidden, w.n_q_heads, w.n_kv_heads, w.head_dim, w.mlp_dim,
                               w.vocab, w.n_target_layers)
    s = w.weight_std
    out = {
        "embed": rng.normal(seed, "embed", (V, H), s, dtype=dt),
        "fc": rng.normal(seed, "fc", (H, nT * H), s, dtype=dt),
        "fc_norm": rng.gains(seed, "fc_norm", H, gain_std, dt),
        "final_norm": rng.gains(seed, "final_norm", H, gain_std, dt),
        "lm_head": rng.normal(seed, "lm_head", (V, H), s, dtype=dt),
    }
    for l in (range(w.n_layers) if layers is None else layers):
        p = f"layers.{l}."
        out[p + "attn_norm"] = rng.gains(seed, p + "attn_norm", H, gain_std, dt)
        out[p + "wq"] = rng.normal(seed, p + "wq", (nq * d, H), s, dtype=dt)
        out[p + "wk"] = rng.normal(seed, p + "wk", (nkv * d, H), s, dtype=dt)
        out[p + "wv"] = rng.normal(seed, p + "wv", (nkv * d, H), s, dtype=dt)
        out[p + "wo"] = rng.normal(seed, p + "wo", (H, nq * d), s, dtype=dt)
        out[p + "mlp_norm"] = rng.gains(seed, p + "mlp_norm", H, gain_std, dt)
        out[p + "w_gate"] = rng.normal(seed, p + "w_gate", (F, H), s, dtype=dt)
        out[p + "w_up"] = rng.normal(seed, p + "w_up", (F, H), s, dtype=dt)
        out[p + "w_down"] = rng.normal(seed, p + "w_down", (H, F), s, dtype=dt)
    return out


def step_inputs(w: Workload, seed: int, n_new=None, ctx_len=None, n_new_max=None) -> dict:
    """hidden_new [B, n_new_max, nT*H], n_new [B], ctx_len [B] (before the append),
    last_token [B].  Default: every row appends S rows onto C - S cached rows."""
    B = w.batch
    n_new = np.full(B, w.block, np.int32) if n_new is None else np.asarray(n_new, np.int32)
    ctx_len = (np.full(B, w.ctx - w.block, np.int32) if ctx_len is None
               else np.asarray(ctx_len, np.int32))
    nmax = int(n_new.max()) if n_new_max is None else int(n_new_max)
    nmax = max(nmax, 1)
    hid = rng.normal(seed, "hidden_new", (B, nmax, w.n_target_layers * w.hidden),
                     w.hidden_std, dtype=w.dtype)
    last = rng.integers(seed, "last_token", (B,), 0, w.vocab - 1)
    return {"hidden_new": hid, "n_new": n_new, "ctx_len": ctx_len, "last_token": last,
            "n_new_max": nmax}


def cache_prefix(w: Workload, seed: int, ctx_len, kv_std: float = 1.28, garbage=None):
    """K and V caches [L, B, max_ctx, nkv, d] holding synthetic rows below ctx_len[b].

    Slots at or above ctx_len[b] hold zeros, or ``garbage`` ("nan" / "big") for
    tests that check those slots are never read.
    """
    L, B, M, nkv, d = w.n_layers, w.batch, w.max_ctx, w.n_kv_heads, w.head_dim
    shape = (L, B, M, nkv, d)
    k = rng.normal(seed, "k_cache", shape, kv_std, dtype="f32")
    v = rng.normal(seed, "v_cache", shape, kv_std, dtype="f32")
    fill = {None: 0.0, "nan": np.nan, "big": 1e4}[garbage]
    ctx_len = np.asarray(ctx_len)
    for b in range(B):
        k[:, b, int(ctx_len[b]):] = fill
        v[:, b, int(ctx_len[b]):] = fill
    if w.dtype == "bf16":
        # NaN survives: its quiet bit pattern is kept by the truncation below
        kb = rng.to_bf16_bits(np.nan_to_num(k, nan=0.0))
        vb = rng.to_bf16_bits(np.nan_to_num(v, nan=0.0))
        if garbage == "nan":
            for b in range(B):
                kb[:, b, int(ctx_len[b]):] = 0x7FC0
                vb[:, b, int(ctx_len[b]):] = 0x7FC0
        return kb, vb
    return k, v


def uniforms(w: Workload, seed: int, batch=None):
    B = w.batch if batch is None else batch
    G = w.gamma
    return (rng.uniform01(seed, "u_draft", (B, G)),
            rng.uniform01(seed, "u_accept", (B, G)),
            rng.uniform01(seed, "u_final", (B,)))


def markov_factors(w: Workload, seed: int, std=None, rank=None, dtype=None):
    r = w.markov_rank if rank is None else rank
    dt = w.dtype if dtype is None else dtype
    s = w.markov_factor_std if std is None else std
    return (rng.normal(seed, "markov_U", (w.vocab, r), s, dtype=dt),
            rng.normal(seed, "markov_Wt", (w.vocab, r), s, dtype=dt))


def rnn_recurrence(w: Workload, seed: int, std=None, rank=None, dtype=None):
    """[r, r] recurrent matrix of the RNN sequential head, N(0, (0.5/sqrt(r))^2)
    entries (spectral radius about 1/2: the state neither dies out nor saturates)."""
    r = w.markov_rank if rank is None else rank
    dt = w.dtype if dtype is None else dtype
    s = 0.5 / r ** 0.5 if std is None else std
    return rng.normal(seed, "rnn_A", (r, r), s, dtype=dt)


def base_logits(w: Workload, seed: int, std=None, batch=None):
    B = w.batch if batch is None else batch
    s = w.base_logit_std if std is None else std
    return rng.normal(seed, "base_logits", (B, w.gamma, w.vocab), s, dtype="f32")


def target_logits(w: Workload, seed: int, draft_logits=None, batch=None):
    """[B, S, V] fp32.  With ``draft_logits`` [B, S-1, V] and a workload noise std,
    rows 0..S-2 are draft + N(0, noise^2) and the bonus row is N(0, std^2)."""
    B = w.batch if batch is None else batch
    t = rng.normal(seed, "target_logits", (B, w.block, w.vocab), w.target_logit_std, dtype="f32")
    if draft_logits is not None and w.target_noise_std > 0:
        noise = rng.normal(seed, "target_noise", (B, w.gamma, w.vocab), w.target_noise_std,
                           dtype="f32")
        t[:, :w.gamma] = np.asarray(draft_logits, np.float32) + noise
    return t


def cycle_inputs(w: Workload, seed: int, cycle: int, batch=None) -> dict:
    """Inputs of cycle ``cycle`` of a multi-step loop, independent across cycles:
    hidden_new [B, S, nT*H] (target hidden states of the rows the previous cycle
    committed; rows >= n_new[b] unused), uniforms u_draft, u_accept [B, gamma] and
    u_final [B], target logits [B, S, V] ~ N(0, std^2), noise [B, S, V] ~ N(0, 1)
    for targets built from the draft logits (draft + noise_std * noise), and
    per-position survival scores [B, gamma] ~ U[0, 1) standing in for a
    confidence head."""
    B = w.batch if batch is None else batch
    G, S = w.gamma, w.block
    k = f"cycle{cycle}."
    return {
        "hidden_new": rng.normal(seed, k + "hidden_new", (B, S, w.n_target_layers * w.hidden), w.hidden_std,
                                 dtype=w.dtype),
        "u_draft": rng.uniform01(seed, k + "u_draft", (B, G)),
        "u_accept": rng.uniform01(seed, k + "u_accept", (B, G)),
        "u_final": rng.uniform01(seed, k + "u_final", (B,)),
        "target_logits": rng.normal(seed, k + "target_logits", (B, S, w.vocab), w.target_logit_std, dtype="f32"),
        "noise": rng.normal(seed, k + "target_noise", (B, S, w.vocab), 1.0, dtype="f32"),
        "survival": rng.uniform01(seed, k + "survival", (B, G)),
    }
