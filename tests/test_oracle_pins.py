"""Pins of the CPU oracle against what the pages and mathematics fix (no GPU).

Each test checks the oracle against something other than itself: a closed
form, a textbook or library routine, an invariant, brute force on tiny inputs,
or a value the pages print.
"""
import json
import os

import numpy as np
import pytest
from scipy import special, stats

import oracle
from oracle import drafter as od
from synth import TINY, inputs, rng

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- rounding

def test_bf16_rounding_ties_and_ranges():
    r = oracle.round_bf16
    assert r(1.0) == 1.0
    assert r(1 + 2.0 ** -8) == 1.0                      # tie -> even mantissa
    assert r(1 + 3 * 2.0 ** -8) == 1 + 2.0 ** -6         # tie -> even (upward)
    assert r(1 + 2.0 ** -8 + 2.0 ** -30) == 1 + 2.0 ** -7
    assert r(-2.5) == -2.5
    assert r(float.fromhex("0x1.fep127")) == float.fromhex("0x1.fep127")
    assert np.isinf(r(float.fromhex("0x1.ffp127")))       # rounds past the largest finite
    assert r(2.0 ** -133) == 2.0 ** -133                 # smallest subnormal
    assert r(2.0 ** -134) == 0.0                         # tie with zero -> even (zero)
    assert np.isnan(r(np.nan))


def test_bf16_rounding_matches_bit_trick_on_fp32():
    # textbook route for fp32 inputs: add 0x7FFF + lsb to the bits, truncate
    x = np.random.default_rng(0).standard_normal(200_000).astype(np.float32) * 10
    b = x.view(np.uint32).astype(np.uint64)
    bits = ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)
    np.testing.assert_array_equal(oracle.f64_to_bf16_bits(x.astype(np.float64)), bits)
    back = oracle.bf16_bits_to_f64(bits)
    np.testing.assert_array_equal(back, oracle.round_bf16(x.astype(np.float64)))
    assert oracle.bf16_bits_to_f64(np.uint16(0x3F80)) == 1.0
    assert oracle.bf16_bits_to_f64(np.uint16(0xC000)) == -2.0


# ---------------------------------------------------------------- RMSNorm

def test_rmsnorm_closed_forms():
    y = od.rmsnorm(np.array([3.0, 4.0]), np.ones(2), 0.0)
    np.testing.assert_allclose(y, np.array([3.0, 4.0]) / np.sqrt(12.5), rtol=1e-15)
    x = np.random.default_rng(1).standard_normal((7, 64)) * 5
    y = od.rmsnorm(x, np.ones(64), 0.0)
    np.testing.assert_allclose(np.sqrt(np.mean(y * y, axis=1)), 1.0, rtol=1e-12)   # unit RMS
    np.testing.assert_allclose(od.rmsnorm(3.7 * x, np.ones(64), 0.0), y, rtol=1e-12)  # scale free
    g = np.linspace(0.5, 2.0, 64)
    np.testing.assert_allclose(od.rmsnorm(x, g, 0.0), y * g, rtol=1e-12)
    # eps: a zero row stays zero instead of dividing by zero
    assert np.all(od.rmsnorm(np.zeros(8), np.ones(8), 1e-6) == 0)


# ---------------------------------------------------------------- RoPE

def _rope_complex(x, pos, theta):
    """Rotary embedding as complex multiplication: (x_i + i x_{i+d/2}) * exp(i pos w_i)."""
    d = x.shape[-1]
    half = d // 2
    w = theta ** (-np.arange(half) * 2.0 / d)
    z = (x[..., :half] + 1j * x[..., half:]) * np.exp(1j * np.asarray(pos)[..., None, None] * w)
    return np.concatenate([z.real, z.imag], axis=-1)


def test_rope_is_complex_rotation():
    g = np.random.default_rng(2)
    x = g.standard_normal((5, 3, 16))
    pos = np.array([0, 1, 7, 300, 32767])
    out = od.rope_rotate(x, pos, 1e6)
    np.testing.assert_allclose(out, _rope_complex(x, pos, 1e6), atol=1e-12)
    np.testing.assert_allclose(out[0], x[0], atol=0)                           # position 0
    np.testing.assert_allclose(np.linalg.norm(out, axis=-1), np.linalg.norm(x, axis=-1),
                               rtol=1e-12)
    # d = 2: a plain 2-D rotation by pos radians
    v = np.array([[[1.0, 0.0]]])
    np.testing.assert_allclose(od.rope_rotate(v, np.array([np.pi / 2]), 10.0), [[[0.0, 1.0]]],
                               atol=1e-15)
    assert np.array_equal(od.rope_rotate(x, pos, 0.0), x)                      # disabled


def test_rope_scores_depend_on_relative_position():
    g = np.random.default_rng(3)
    q = g.standard_normal((1, 1, 32))
    k = g.standard_normal((1, 1, 32))
    s = [float(np.sum(od.rope_rotate(q, np.array([m + t]), 1e4) *
                      od.rope_rotate(k, np.array([n + t]), 1e4)))
         for (m, n, t) in [(10, 3, 0), (10, 3, 1000), (10, 3, 77)]]
    np.testing.assert_allclose(s, s[0], rtol=1e-10)


# ---------------------------------------------------------------- attention

def _bruteforce_block_attention(q, k_ctx, v_ctx, k_blk, v_blk, window=0):
    """Whole sequence [context ; block] with an explicit 0/-inf mask matrix built
    from the rule: full attention inside the block, causal toward the context
    (with a sliding window: only the last `window` context keys)."""
    C = k_ctx.shape[0]
    S, nq, d = q.shape
    nkv = k_ctx.shape[1]
    n = C + S
    keys = np.concatenate([k_ctx, k_blk])
    vals = np.concatenate([v_ctx, v_blk])
    rep = nq // nkv
    keys = np.repeat(keys, rep, axis=1)          # [n, nq, d]
    vals = np.repeat(vals, rep, axis=1)
    mask = np.full((n, n), -np.inf)
    for i in range(n):
        for j in range(n):
            in_block_i, in_block_j = i >= C, j >= C
            if in_block_i and in_block_j:
                mask[i, j] = 0.0                 # full attention inside the block
            elif j <= i and not in_block_j and (window <= 0 or j >= C - window):
                mask[i, j] = 0.0                 # causal toward the (earlier) context, within the window
    qfull = np.zeros((n, nq, d))
    qfull[C:] = q
    out = np.zeros((S, nq, d))
    for h in range(nq):
        s = qfull[:, h] @ keys[:, h].T / np.sqrt(d) + mask
        p = special.softmax(s[C:], axis=1)
        out[:, h] = p @ vals[:, h]
    return out


@pytest.mark.parametrize("C,S,nq,nkv", [(37, 5, 6, 2), (0, 4, 4, 4), (9, 1, 8, 2), (64, 16, 4, 1)])
def test_block_attention_matches_bruteforce_mask(C, S, nq, nkv):
    g = np.random.default_rng(C * 100 + S)
    d = 16
    q = g.standard_normal((S, nq, d))
    kc, vc = g.standard_normal((C, nkv, d)), g.standard_normal((C, nkv, d))
    kb, vb = g.standard_normal((S, nkv, d)), g.standard_normal((S, nkv, d))
    np.testing.assert_allclose(od.block_attention(q, kc, vc, kb, vb),
                               _bruteforce_block_attention(q, kc, vc, kb, vb), atol=1e-12)


def test_block_attention_special_cases():
    g = np.random.default_rng(5)
    C, S, nq, nkv, d = 20, 3, 4, 2, 8
    q = g.standard_normal((S, nq, d))
    kc, vc = g.standard_normal((C, nkv, d)), g.standard_normal((C, nkv, d))
    kb, vb = g.standard_normal((S, nkv, d)), g.standard_normal((S, nkv, d))
    o = od.block_attention(q, kc, vc, kb, vb)
    # GQA == MHA with each key/value head repeated for its query group
    o_mha = od.block_attention(q, np.repeat(kc, 2, 1), np.repeat(vc, 2, 1),
                               np.repeat(kb, 2, 1), np.repeat(vb, 2, 1))
    np.testing.assert_allclose(o, o_mha, atol=1e-12)
    # permuting the context rows (no positions involved here) changes nothing
    perm = g.permutation(C)
    np.testing.assert_allclose(od.block_attention(q, kc[perm], vc[perm], kb, vb), o, atol=1e-12)
    # zero queries: uniform weights over all C + S visible keys
    o0 = od.block_attention(np.zeros_like(q), kc, vc, kb, vb)
    mean_v = np.concatenate([vc, vb]).mean(0)                       # [nkv, d]
    np.testing.assert_allclose(o0, np.broadcast_to(np.repeat(mean_v, 2, 0), o0.shape), atol=1e-12)
    # S = 1: plain decode attention of one query over C + 1 keys
    o1 = od.block_attention(q[:1], kc, vc, kb[:1], vb[:1])
    keys = np.concatenate([kc, kb[:1]])[:, 0]
    vals = np.concatenate([vc, vb[:1]])[:, 0]
    w = special.softmax(keys @ q[0, 0] / np.sqrt(d))
    np.testing.assert_allclose(o1[0, 0], w @ vals, atol=1e-12)


# ---------------------------------------------------------------- drafter

def _tiny(**kw):
    base = dict(batch=2, block=4, ctx=24, n_layers=1, hidden=32, n_q_heads=4, n_kv_heads=2,
                head_dim=8, mlp_dim=48, vocab=50, n_target_layers=3, markov_rank=4)
    base.update(kw)
    return TINY.with_(name="pin", **base)


def _shape(w):
    return od.DrafterShape.of(w)


def _run(w, weights, step, kc, vc):
    kc, vc = kc.copy(), vc.copy()
    logits, new_len = od.draft_step(_shape(w), weights, step["hidden_new"], step["n_new"], kc, vc,
                                    step["ctx_len"], step["last_token"])
    return logits, new_len, kc, vc


def test_kv_injection_context_kv_independent_of_block_and_shared_across_layers():
    w = _tiny(n_layers=3)
    weights = inputs.drafter_weights(w, 0, gain_std=0.1)
    for l in (1, 2):                                      # same Wk, Wv in every layer
        weights[f"layers.{l}.wk"] = weights["layers.0.wk"]
        weights[f"layers.{l}.wv"] = weights["layers.0.wv"]
    step = inputs.step_inputs(w, 0)
    kc, vc = inputs.cache_prefix(w, 0, step["ctx_len"])
    _, _, k1, v1 = _run(w, weights, step, kc, vc)
    step2 = dict(step, last_token=(step["last_token"] + 7) % (w.vocab - 1))
    _, _, k2, v2 = _run(w, weights, step2, kc, vc)
    assert np.array_equal(k1, k2) and np.array_equal(v1, v2)    # block tokens do not matter
    for b in range(w.batch):                                    # same features in every layer
        c = step["ctx_len"][b]
        new = slice(c, c + w.block)
        for l in (1, 2):
            assert np.array_equal(k1[l, b, new], k1[0, b, new])
            assert np.array_equal(v1[l, b, new], v1[0, b, new])
    # the appended slots are exactly ctx_len .. ctx_len + n_new - 1
    for b in range(w.batch):
        c = step["ctx_len"][b]
        assert np.array_equal(k1[:, b, :c], kc[:, b, :c])
        assert not np.array_equal(k1[:, b, c:c + w.block], kc[:, b, c:c + w.block])
        assert np.array_equal(k1[:, b, c + w.block:], kc[:, b, c + w.block:])


def test_drafter_closed_form_without_attention_and_mlp_output():
    # Wo = 0 and W_down = 0: the residual stream stays at the embeddings, so every
    # mask row's logits are RMSNorm(E[MASK]) . W_lm^T whatever the context
    w = _tiny()
    weights = inputs.drafter_weights(w, 1, gain_std=0.1)
    weights["layers.0.wo"] = np.zeros_like(weights["layers.0.wo"])
    weights["layers.0.w_down"] = np.zeros_like(weights["layers.0.w_down"])
    step = inputs.step_inputs(w, 1)
    kc, vc = inputs.cache_prefix(w, 1, step["ctx_len"])
    logits, _, _, _ = _run(w, weights, step, kc, vc)
    e = weights["embed"][w.mask_token_id].astype(np.float64)
    g = weights["final_norm"].astype(np.float64)
    z = e / np.sqrt(np.mean(e * e) + w.rms_eps) * g
    z = z.astype(np.float32).astype(np.float64)
    want = (weights["lm_head"].astype(np.float64) @ z).astype(np.float32)
    for b in range(w.batch):
        for j in range(w.gamma):
            np.testing.assert_array_equal(logits[b, j], want)


def _rms(x, g, eps):
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * g


def _bruteforce_one_layer_drafter(w, weights, hidden_all, last_token):
    """Sequence-level formulation of a 1-layer drafter with its MLP switched off:
    every context row j (features at position j) and every block row (position
    C + j) projects its own keys and values; only block rows query; an explicit
    mask implements full-in-block / causal-to-context.  fp32 storage throughout."""
    f32 = lambda a: np.asarray(a, np.float64).astype(np.float32).astype(np.float64)
    W = {k: np.asarray(v, np.float64) for k, v in weights.items()}
    C = hidden_all.shape[0]
    S, H, nq, nkv, d = w.block, w.hidden, w.n_q_heads, w.n_kv_heads, w.head_dim
    feats = f32(_rms(hidden_all @ W["fc"].T, W["fc_norm"], w.rms_eps))
    toks = [last_token] + [w.mask_token_id] * (S - 1)
    x = f32(W["embed"][toks])
    a = f32(_rms(x, W["layers.0.attn_norm"], w.rms_eps))
    rows = np.concatenate([feats, a])                           # [C + S, H]
    pos = np.arange(C + S)
    k = f32(_rope_complex((rows @ W["layers.0.wk"].T).reshape(-1, nkv, d), pos, w.rope_theta))
    v = f32((rows @ W["layers.0.wv"].T).reshape(-1, nkv, d))
    q = f32(_rope_complex((a @ W["layers.0.wq"].T).reshape(-1, nq, d), pos[C:], w.rope_theta))
    o = _bruteforce_block_attention(q, k[:C], v[:C], k[C:], v[C:], window=w.window)
    x = f32(x + f32(o).reshape(S, nq * d) @ W["layers.0.wo"].T)
    z = f32(_rms(x[1:], W["final_norm"], w.rms_eps))
    return (z @ W["lm_head"].T).astype(np.float32)


@pytest.mark.parametrize("split,arith,window", [(None, np.float64, 0), (9, np.float64, 0), (None, np.float32, 0),
                                                (None, np.float64, 6), (9, np.float64, 6), (None, np.float64, 30)])
def test_drafter_matches_sequence_level_bruteforce(split, arith, window):
    # one layer, MLP output off, fp32 storage; the context is appended in one
    # call (prefill) or in two calls; positions come out of the cache
    # bookkeeping.  The fp32-arithmetic evaluation computes the same function.
    # window > 0: the sliding-window variant (30 > C: the whole context)
    w = _tiny(batch=1, ctx=21, dtype="f32", rope_theta=100.0, window=window)
    weights = inputs.drafter_weights(w, 2, gain_std=0.1)
    weights["layers.0.w_down"] = np.zeros_like(weights["layers.0.w_down"])
    C = 17
    hid = rng.normal(2, "pin_hidden", (1, C, w.n_target_layers * w.hidden), 1.0)
    last = np.array([5], np.int32)
    sh = _shape(w)
    kc = np.zeros((1, 1, w.max_ctx, w.n_kv_heads, w.head_dim), np.float32)
    vc = np.zeros_like(kc)
    ctx = np.zeros(1, np.int32)
    for lo, hi in ([(0, C)] if split is None else [(0, split), (split, C)]):
        logits, ctx = od.draft_step(sh, weights, hid[:, lo:hi], np.array([hi - lo]), kc, vc,
                                    ctx, last, arith=arith)
    assert ctx[0] == C
    want = _bruteforce_one_layer_drafter(w, weights, hid[0].astype(np.float64), 5)
    np.testing.assert_allclose(logits[0], want, atol=2e-6 if arith is np.float64 else 1e-4, rtol=0)


def _torch_swiglu(m, w_gate, w_up, w_down):
    """SwiGLU MLP through torch's own SiLU (CPU, float64): (silu(m Wg^T) * (m Wu^T)) Wd^T,
    with the gated product stored in fp32 as the drafter stores it."""
    import torch
    import torch.nn.functional as Fn
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))
    mt = t(m)
    h = Fn.silu(mt @ t(w_gate).T) * (mt @ t(w_up).T)
    h = h.to(torch.float32).to(torch.float64)
    return (h @ t(w_down).T).numpy()


def _bruteforce_drafter(w, weights, hidden_all, last_token):
    """Sequence-level formulation of an L-layer drafter with its MLP on.

    The sequence is [context rows ; block rows].  KV injection: a context row's
    state is its feature vector at EVERY layer (only the block rows evolve), and
    layer l's keys/values of every row come from that layer's own Wk, Wv.  Only
    block rows query; the explicit mask gives full-in-block / causal-to-context.
    Each layer: pre-norm attention, residual, pre-norm SwiGLU MLP (torch's SiLU),
    residual.  fp32 storage throughout, float64 arithmetic."""
    f32 = lambda a: np.asarray(a, np.float64).astype(np.float32).astype(np.float64)
    W = {k: np.asarray(v, np.float64) for k, v in weights.items()}
    C = hidden_all.shape[0]
    S, nq, nkv, d = w.block, w.n_q_heads, w.n_kv_heads, w.head_dim
    feats = f32(_rms(hidden_all @ W["fc"].T, W["fc_norm"], w.rms_eps))
    toks = [last_token] + [w.mask_token_id] * (S - 1)
    x = f32(W["embed"][toks])
    pos = np.arange(C + S)
    for l in range(w.n_layers):
        p = f"layers.{l}."
        a = f32(_rms(x, W[p + "attn_norm"], w.rms_eps))
        rows = np.concatenate([feats, a])                       # layer-l states of the whole sequence
        k = f32(_rope_complex((rows @ W[p + "wk"].T).reshape(-1, nkv, d), pos, w.rope_theta))
        v = f32((rows @ W[p + "wv"].T).reshape(-1, nkv, d))
        q = f32(_rope_complex((a @ W[p + "wq"].T).reshape(-1, nq, d), pos[C:], w.rope_theta))
        o = _bruteforce_block_attention(q, k[:C], v[:C], k[C:], v[C:], window=w.window)
        x = f32(x + f32(o).reshape(S, nq * d) @ W[p + "wo"].T)
        m = f32(_rms(x, W[p + "mlp_norm"], w.rms_eps))
        x = f32(x + _torch_swiglu(m, W[p + "w_gate"], W[p + "w_up"], W[p + "w_down"]))
    z = f32(_rms(x[1:], W["final_norm"], w.rms_eps))
    return (z @ W["lm_head"].T).astype(np.float32)


def _strong_mlp(weights, w, seed):
    """Gate/up weights wide enough that SiLU works in its curved range (|g| ~ 3)
    and a down projection that makes the MLP a large share of the residual."""
    out = dict(weights)
    for l in range(w.n_layers):
        p = f"layers.{l}."
        out[p + "w_gate"] = rng.normal(seed, p + "w_gate_strong", (w.mlp_dim, w.hidden), 0.5)
        out[p + "w_up"] = rng.normal(seed, p + "w_up_strong", (w.mlp_dim, w.hidden), 0.5)
        out[p + "w_down"] = rng.normal(seed, p + "w_down_strong", (w.hidden, w.mlp_dim), 0.01)
    return out


@pytest.mark.parametrize("n_layers,split", [(2, None), (3, None), (2, 9)])
def test_drafter_mlp_and_layer_stacking_match_sequence_level_bruteforce(n_layers, split):
    # L layers with the SwiGLU MLP on and distinct random norm gains per layer: a
    # gate/up swap, sigmoid in place of SiLU, a dropped residual or a layer reading
    # another layer's weights or gains changes the logits far beyond the bar
    w = _tiny(batch=1, ctx=21, dtype="f32", rope_theta=100.0, n_layers=n_layers)
    weights = _strong_mlp(inputs.drafter_weights(w, 11, gain_std=0.3), w, 11)
    C = 17
    hid = rng.normal(11, "pin_hidden_mlp", (1, C, w.n_target_layers * w.hidden), 1.0)
    last = np.array([7], np.int32)
    sh = _shape(w)
    kc = np.zeros((n_layers, 1, w.max_ctx, w.n_kv_heads, w.head_dim), np.float32)
    vc = np.zeros_like(kc)
    ctx = np.zeros(1, np.int32)
    for lo, hi in ([(0, C)] if split is None else [(0, split), (split, C)]):
        logits, ctx = od.draft_step(sh, weights, hid[:, lo:hi], np.array([hi - lo]), kc, vc, ctx, last)
    want = _bruteforce_drafter(w, weights, hid[0].astype(np.float64), 7)
    np.testing.assert_allclose(logits[0], want, atol=2e-6, rtol=0)
    # the MLP matters at this scale: switching it off moves the logits by far more
    off = dict(weights)
    for l in range(n_layers):
        off[f"layers.{l}.w_down"] = np.zeros_like(weights[f"layers.{l}.w_down"])
    kc2, vc2 = np.zeros_like(kc), np.zeros_like(vc)
    l_off, _ = od.draft_step(sh, off, hid, np.array([C]), kc2, vc2, np.zeros(1, np.int32), last)
    assert np.abs(l_off[0] - want).max() > 1e-2


def test_drafter_swiglu_gate_and_up_roles():
    # one layer, attention output off (Wo = 0), so a mask row's state after the
    # layer is e + MLP(m) with e = E[MASK] and m = RMSNorm(e; g_mlp)
    w = _tiny(dtype="f32", rope_theta=100.0)
    base = _strong_mlp(inputs.drafter_weights(w, 12, gain_std=0.3), w, 12)
    base["layers.0.wo"] = np.zeros_like(base["layers.0.wo"])
    step = inputs.step_inputs(w, 12)
    kc, vc = inputs.cache_prefix(w, 12, step["ctx_len"])

    def run(**over):
        wt = dict(base)
        wt.update({f"layers.0.{k}": v for k, v in over.items()})
        return _run(w, wt, step, kc, vc)[0]

    Fd, H = w.mlp_dim, w.hidden
    no_mlp = run(w_down=np.zeros((H, Fd), np.float32))
    # silu(g) * 0 and silu(0) * u are exactly zero: the MLP adds nothing
    np.testing.assert_array_equal(run(w_up=np.zeros((Fd, H), np.float32)), no_mlp)
    np.testing.assert_array_equal(run(w_gate=np.zeros((Fd, H), np.float32)), no_mlp)
    # a gate row g_f = lam for every feature of the mask rows: silu(lam) ~ lam when
    # lam >> 0 and ~ 0 when lam << 0 (a gate/up swap would give silu(u) * lam instead)
    e = base["embed"][w.mask_token_id].astype(np.float64)
    m = (e / np.sqrt(np.mean(e * e) + w.rms_eps) * base["layers.0.mlp_norm"]).astype(np.float32)
    m = m.astype(np.float64)
    unit = np.broadcast_to(m / (m @ m), (Fd, H))
    np.testing.assert_allclose(run(w_gate=(-60.0 * unit).astype(np.float32)), no_mlp, atol=1e-9, rtol=0)
    lam = 60.0
    wg = (lam * unit).astype(np.float32)
    g = wg.astype(np.float64) @ m                                 # ~ lam for every feature
    u = base["layers.0.w_up"].astype(np.float64) @ m
    hmid = (g * u).astype(np.float32).astype(np.float64)          # silu(g) = g to ~1e-24 here
    x = (e + hmid @ base["layers.0.w_down"].astype(np.float64).T).astype(np.float32).astype(np.float64)
    z = (x / np.sqrt(np.mean(x * x) + w.rms_eps) * base["final_norm"]).astype(np.float32).astype(np.float64)
    want = (base["lm_head"].astype(np.float64) @ z).astype(np.float32)
    got = run(w_gate=wg)
    for b in range(w.batch):
        for j in range(w.gamma):
            np.testing.assert_allclose(got[b, j], want, atol=2e-6, rtol=0)


def test_drafter_batch_rows_independent_and_garbage_slots_ignored():
    w = _tiny(n_layers=2, ctx=40)
    weights = inputs.drafter_weights(w, 3, gain_std=0.1)
    step = inputs.step_inputs(w, 3, ctx_len=[20, 30], n_new=[4, 2], n_new_max=4)
    kc, vc = inputs.cache_prefix(w, 3, step["ctx_len"])
    kg, vg = inputs.cache_prefix(w, 3, step["ctx_len"], garbage="big")
    l1, n1, _, _ = _run(w, weights, step, kc, vc)
    l2, n2, _, _ = _run(w, weights, step, kg, vg)
    np.testing.assert_array_equal(l1, l2)
    np.testing.assert_array_equal(n1, [24, 32])
    # changing batch row 1's inputs leaves row 0 alone
    step3 = dict(step, last_token=np.array([step["last_token"][0], 3], np.int32))
    l3, _, _, _ = _run(w, weights, step3, kc, vc)
    np.testing.assert_array_equal(l3[0], l1[0])
    assert not np.array_equal(l3[1], l1[1])


def test_mask_rows_identical_without_positions():
    # with rotary embedding off nothing distinguishes the mask rows: full
    # attention inside the block gives them identical outputs
    w = _tiny(rope_theta=0.0)
    weights = inputs.drafter_weights(w, 4, gain_std=0.1)
    step = inputs.step_inputs(w, 4)
    kc, vc = inputs.cache_prefix(w, 4, step["ctx_len"])
    logits, _, _, _ = _run(w, weights, step, kc, vc)
    for j in range(1, w.gamma):
        np.testing.assert_array_equal(logits[:, j], logits[:, 0])


# ---------------------------------------------------------------- sampling

def test_inverse_cdf_hand_examples():
    assert oracle.inverse_cdf([1, 2, 3, 4], 0.25) == (1, pytest.approx(0.05))
    assert oracle.inverse_cdf([0, 0, 5, 1], 0.0)[0] == 2                 # u = 0: first positive
    assert oracle.inverse_cdf([0, 0, 0, 1, 0], 0.7)[0] == 3              # one-hot
    assert oracle.inverse_cdf([1, 1, 1, 0], 1 - 2 ** -24)[0] == 2        # top end
    assert oracle.argmax_with_gap([1.0, 3.0, 3.0, 2.0]) == (1, 0.0)      # lowest index on ties


def test_inverse_cdf_equals_searchsorted():
    g = np.random.default_rng(6)
    for _ in range(200):
        w = g.exponential(size=int(g.integers(1, 40)))
        u = g.random()
        k, _ = oracle.inverse_cdf(w, u)
        assert k == int(np.searchsorted(np.cumsum(w), u * w.sum(), side="right"))


def test_softmax_weights_normalise_to_scipy_softmax():
    g = np.random.default_rng(7)
    x = g.standard_normal((3, 100)) * 3
    for T in (1.0, 0.5, 2.0):
        w = oracle.softmax_weights(x, T)
        np.testing.assert_allclose(w / w.sum(1, keepdims=True), special.softmax(x / T, axis=1),
                                   rtol=1e-12)


def _chi2_pvalue(counts, probs):
    exp = probs * counts.sum()
    keep = exp >= 5
    obs = np.append(counts[keep], counts[~keep].sum())
    ex = np.append(exp[keep], exp[~keep].sum())
    if ex[-1] == 0:
        obs, ex = obs[:-1], ex[:-1]
    return stats.chisquare(obs, ex).pvalue


def test_sampler_chi_square():
    g = np.random.default_rng(8)
    x = g.standard_normal(8)
    q = special.softmax(x)
    us = rng.uniform01(8, "chi_u", (40_000,))
    counts = np.bincount([oracle.sample_row(x, u, 1.0)[0] for u in us], minlength=8)
    assert _chi2_pvalue(counts, q) > 1e-4


# ---------------------------------------------------------------- Markov head

def test_markov_bias_is_row_of_low_rank_bigram_table():
    V, r, G = 12, 3, 4
    g = np.random.default_rng(9)
    U = g.standard_normal((V, r)).astype(np.float32)
    Wt = g.standard_normal((V, r)).astype(np.float32)
    table = U.astype(np.float64) @ Wt.astype(np.float64).T       # dense V x V bigram bias
    assert np.linalg.matrix_rank(table) == r
    base = g.standard_normal((2, G, V)).astype(np.float32)
    last = np.array([3, 11])
    u = rng.uniform01(9, "mk", (2, G))
    final, tok, _ = oracle.markov_sample(base, U, Wt, "f32", last, u, 1.0)
    for b in range(2):
        prev = last[b]
        for i in range(G):
            np.testing.assert_allclose(final[b, i].astype(np.float64) - base[b, i],
                                       table[prev], atol=2e-6)
            prev = tok[b, i]
    # rank 0: no head, positions are sampled independently from the base logits
    f0, t0, _ = oracle.markov_sample(base, None, None, "f32", last, u, 1.0)
    assert np.array_equal(f0, base)
    for b in range(2):
        for i in range(G):
            assert t0[b, i] == oracle.sample_row(base[b, i], u[b, i], 1.0)[0]


def test_markov_sequence_distribution_chi_square():
    # V = 8, gamma = 3: the empirical distribution of drafted sequences equals
    # prod_i softmax(base_i + table[d_{i-1}])(d_i), enumerated over all 8^3 sequences
    V, G, r, N = 8, 3, 4, 30_000
    g = np.random.default_rng(10)
    U = (g.standard_normal((V, r)) * r ** -0.25).astype(np.float32)
    Wt = (g.standard_normal((V, r)) * r ** -0.25).astype(np.float32)
    base1 = g.standard_normal((G, V)).astype(np.float32)
    table = U.astype(np.float64) @ Wt.astype(np.float64).T
    last = 2
    probs = np.zeros(V ** G)
    for idx in range(V ** G):
        seq = np.unravel_index(idx, (V,) * G)
        pr, prev = 1.0, last
        for i in range(G):
            pr *= special.softmax(base1[i] + table[prev])[seq[i]]
            prev = seq[i]
        probs[idx] = pr
    base = np.broadcast_to(base1, (N, G, V))
    u = rng.uniform01(10, "mk_seq", (N, G))
    _, tok, _ = oracle.markov_sample(base, U, Wt, "f32", np.full(N, last), u, 1.0)
    idx = np.ravel_multi_index(tuple(tok.T), (V,) * G)
    assert _chi2_pvalue(np.bincount(idx, minlength=V ** G), probs) > 1e-4


# ---------------------------------------------------------------- RNN head

def _torch_elman_states(U, A, prev_tokens):
    """States of torch.nn.RNN (tanh, no bias) on one-hot inputs, float64."""
    import torch
    V, r = U.shape
    cell = torch.nn.RNN(V, r, nonlinearity="tanh", bias=False, dtype=torch.float64)
    with torch.no_grad():
        cell.weight_ih_l0.copy_(torch.from_numpy(np.asarray(U, np.float64).T.copy()))
        cell.weight_hh_l0.copy_(torch.from_numpy(np.asarray(A, np.float64)))
        x = torch.nn.functional.one_hot(torch.as_tensor(np.asarray(prev_tokens, np.int64)), V).double()
        out, _ = cell(x[:, None, :])
    return out[:, 0, :].numpy()


def test_rnn_head_states_equal_a_library_elman_rnn():
    # the head's recurrence is an Elman cell fed one-hot previous tokens: torch's
    # RNN with W_ih = U^T and W_hh = A must produce the same states, and the
    # bias added to each position must be W h of that state
    V, r, G, B = 11, 5, 6, 3
    g = np.random.default_rng(21)
    U = (g.standard_normal((V, r)) * 0.8).astype(np.float32)
    Wt = g.standard_normal((V, r)).astype(np.float32)
    A = (g.standard_normal((r, r)) * 0.7).astype(np.float32)
    base = g.standard_normal((B, G, V)).astype(np.float32)
    last = np.array([0, 7, 10])
    u = rng.uniform01(21, "rnn", (B, G))
    final, tok, _, states = oracle.rnn_sample(base, U, Wt, A, "f32", last, u, 1.0)
    for b in range(B):
        prev = np.concatenate([[last[b]], tok[b, :-1]])
        ref = _torch_elman_states(U, A, prev)
        np.testing.assert_allclose(states[b], ref, rtol=0, atol=1e-13)
        np.testing.assert_allclose(oracle.rnn_states(U, A, "f32", prev), ref, rtol=0, atol=1e-13)
        bias = ref @ Wt.astype(np.float64).T
        np.testing.assert_allclose(final[b].astype(np.float64) - base[b], bias, atol=2e-6)
    # A transposed is a different head: the states must tell them apart
    prev = np.concatenate([[last[0]], tok[0, :-1]])
    assert np.abs(_torch_elman_states(U, A.T, prev) - states[0]).max() > 1e-3


def test_rnn_head_sequence_distribution_chi_square():
    # V = 6, gamma = 3: drafted sequences follow prod_i softmax(base_i + W h_i)(d_i)
    # with h_i the library RNN's state on the sequence's own prefix
    V, G, r, N = 6, 3, 4, 30_000
    g = np.random.default_rng(22)
    U = (g.standard_normal((V, r)) * 0.9).astype(np.float32)
    Wt = (g.standard_normal((V, r)) * 0.9).astype(np.float32)
    A = (g.standard_normal((r, r)) * 0.6).astype(np.float32)
    base1 = (g.standard_normal((G, V)) * 0.5).astype(np.float32)
    last = 4
    probs = np.zeros(V ** G)
    for idx in range(V ** G):
        seq = np.unravel_index(idx, (V,) * G)
        h = _torch_elman_states(U, A, [last] + list(seq[:-1]))
        pr = 1.0
        for i in range(G):
            pr *= special.softmax(base1[i] + h[i] @ Wt.astype(np.float64).T)[seq[i]]
        probs[idx] = pr
    base = np.broadcast_to(base1, (N, G, V))
    u = rng.uniform01(22, "rnn_seq", (N, G))
    _, tok, _, _ = oracle.rnn_sample(base, U, Wt, A, "f32", np.full(N, last), u, 1.0)
    idx = np.ravel_multi_index(tuple(tok.T), (V,) * G)
    assert _chi2_pvalue(np.bincount(idx, minlength=V ** G), probs) > 1e-4


def test_rnn_head_degenerate_cases():
    V, r, G = 9, 4, 5
    g = np.random.default_rng(23)
    U = g.standard_normal((V, r)).astype(np.float32)
    Wt = g.standard_normal((V, r)).astype(np.float32)
    base = g.standard_normal((2, G, V)).astype(np.float32)
    last = np.array([1, 8])
    u = rng.uniform01(23, "rnn_deg", (2, G))
    # no recurrence: the head is a Markov head whose input factor is tanh(U)
    f0, t0, m0, _ = oracle.rnn_sample(base, U, Wt, np.zeros((r, r), np.float32), "f32", last, u, 1.0)
    f1, t1, m1 = oracle.markov_sample(base, np.tanh(U.astype(np.float64)).astype(np.float32), Wt, "f32", last, u, 1.0)
    np.testing.assert_allclose(f0, f1, atol=1e-5)
    ok = (m0 > 1e-5) & (m1 > 1e-5)
    assert np.array_equal(t0[ok], t1[ok]) and ok.mean() > 0.9
    # zero input factor: the state stays 0 and positions are independent draws
    f2, t2, _, st = oracle.rnn_sample(base, np.zeros_like(U), Wt, g.standard_normal((r, r)).astype(np.float32),
                                      "f32", last, u, 1.0)
    assert not st.any() and np.array_equal(f2, base)
    for b in range(2):
        for i in range(G):
            assert t2[b, i] == oracle.sample_row(base[b, i], u[b, i], 1.0)[0]


# ---------------------------------------------------------------- verify

def _verify_trials(p_logits, q_logits, N, seed, temperature=1.0):
    """Drafts sampled from q by the oracle sampler, then verified against p."""
    G = q_logits.shape[0]
    ud = rng.uniform01(seed, "vt_draft", (N, G))
    ua = rng.uniform01(seed, "vt_acc", (N, G))
    uf = rng.uniform01(seed, "vt_fin", (N,))
    qw = special.softmax(q_logits.astype(np.float64) / temperature, axis=1)
    cum = np.cumsum(qw, axis=1)
    drafts = np.array([[int(np.searchsorted(cum[i], ud[n, i] * cum[i, -1], side="right"))
                        for i in range(G)] for n in range(N)], np.int32)
    ql = np.broadcast_to(q_logits, (N,) + q_logits.shape)
    pl = np.broadcast_to(p_logits, (N,) + p_logits.shape)
    out, nacc, _ = oracle.verify(ql, pl, drafts, ua, uf, temperature)
    return out, nacc, drafts


def test_verify_is_lossless_chi_square_and_acceptance_matches_tv():
    V, G, N = 8, 3, 20_000
    g = np.random.default_rng(11)
    p_logits = g.standard_normal((G + 1, V)).astype(np.float32)
    q_logits = g.standard_normal((G, V)).astype(np.float32)
    out, nacc, _ = _verify_trials(p_logits, q_logits, N, 11)
    p = special.softmax(p_logits.astype(np.float64), axis=1)
    q = special.softmax(q_logits.astype(np.float64), axis=1)
    for i in range(G + 1):
        reached = nacc >= i
        assert _chi2_pvalue(np.bincount(out[reached, i], minlength=V), p[i]) > 1e-4
    alphas = [oracle.acceptance_rate(p[i], q[i]) for i in range(G)]
    assert np.isclose(alphas[0], 1 - 0.5 * np.abs(p[0] - q[0]).sum())        # 1 - TV
    acc1 = np.mean(nacc >= 1)
    assert abs(acc1 - alphas[0]) < 4 * np.sqrt(alphas[0] * (1 - alphas[0]) / N)
    tau = oracle.tau_from_accepted(nacc)
    et = oracle.expected_tau_independent(alphas)
    assert abs(tau.mean() - et) < 4 * tau.std() / np.sqrt(N)
    assert np.all((tau >= 1) & (tau <= G + 1))
    for n in range(N):                                   # -1 padding after the last token
        assert np.all(out[n, nacc[n] + 1:] == -1) and np.all(out[n, :nacc[n] + 1] >= 0)


def test_verify_early_stopping_is_the_rule_on_the_truncated_block():
    # n_verify = k: the outcome equals verifying the k-draft block (drafts and
    # draft rows 0..k-1, target rows 0..k, row k acting as the bonus row);
    # n_verify = gamma reproduces the unbounded call
    g = np.random.default_rng(21)
    B, G, V = 40, 4, 12
    q = g.standard_normal((B, G, V)).astype(np.float32)
    p = g.standard_normal((B, G + 1, V)).astype(np.float32)
    d = g.integers(0, V, (B, G)).astype(np.int32)
    ua = g.random((B, G)).astype(np.float32)
    uf = g.random(B).astype(np.float32)
    full = oracle.verify(q, p, d, ua, uf, 1.0)
    same = oracle.verify(q, p, d, ua, uf, 1.0, n_verify=np.full(B, G))
    assert np.array_equal(full[0], same[0]) and np.array_equal(full[1], same[1])
    kv = g.integers(-1, G + 2, B)                        # includes out-of-range lengths (clamped)
    out, nacc, _ = oracle.verify(q, p, d, ua, uf, 1.0, n_verify=kv)
    for b in range(B):
        k = int(np.clip(kv[b], 0, G))
        o1, n1, _ = oracle.verify(q[b:b + 1, :k] if k else np.zeros((1, 0, V), np.float32), p[b:b + 1, :k + 1],
                                  d[b:b + 1, :k], ua[b:b + 1, :k], uf[b:b + 1], 1.0)
        assert nacc[b] == n1[0] and nacc[b] <= k
        assert np.array_equal(out[b, :k + 1], o1[0]) and np.all(out[b, k + 1:] == -1)
    for T in (0.0,):                                     # greedy: the same truncation
        o0, n0, _ = oracle.verify(q, p, d, ua, uf, T, n_verify=kv)
        assert np.all(n0 <= np.clip(kv, 0, G))


def test_verify_early_stopping_stays_lossless_chi_square():
    # random verify lengths per trial (0..gamma): the first emitted token is still
    # distributed as the target's first row
    V, G, N = 8, 3, 20_000
    g = np.random.default_rng(12)
    p_logits = g.standard_normal((G + 1, V)).astype(np.float32)
    q_logits = g.standard_normal((G, V)).astype(np.float32)
    ud = rng.uniform01(12, "es_draft", (N, G))
    qw = special.softmax(q_logits.astype(np.float64), axis=1)
    cum = np.cumsum(qw, axis=1)
    drafts = np.array([[int(np.searchsorted(cum[i], ud[n, i] * cum[i, -1], side="right")) for i in range(G)]
                       for n in range(N)], np.int32)
    kv = g.integers(0, G + 1, N)
    out, nacc, _ = oracle.verify(np.broadcast_to(q_logits, (N, G, V)), np.broadcast_to(p_logits, (N, G + 1, V)),
                                 drafts, rng.uniform01(12, "es_acc", (N, G)), rng.uniform01(12, "es_fin", (N,)),
                                 1.0, n_verify=kv)
    p = special.softmax(p_logits.astype(np.float64), axis=1)
    assert _chi2_pvalue(np.bincount(out[:, 0], minlength=V), p[0]) > 1e-4
    assert np.all(nacc <= kv)
    assert np.all(nacc[kv == 0] == 0)


def test_verify_identical_and_disjoint_distributions():
    V, G, N = 8, 3, 2000
    g = np.random.default_rng(12)
    lg = g.standard_normal((G + 1, V)).astype(np.float32)
    out, nacc, drafts = _verify_trials(lg, lg[:G], N, 12)
    assert np.all(nacc == G)                             # q == p: everything accepted
    assert np.array_equal(out[:, :G], drafts)
    # disjoint supports: q only on 0..3, p only on 4..7 -> reject at once, draw from p
    q = np.full((G, V), -np.inf, np.float32); q[:, :4] = g.standard_normal((G, 4))
    p = np.full((G + 1, V), -np.inf, np.float32); p[:, 4:] = g.standard_normal((G + 1, 4))
    out, nacc, _ = _verify_trials(p, q, 20_000, 13)
    assert np.all(nacc == 0)
    assert _chi2_pvalue(np.bincount(out[:, 0], minlength=V),
                        special.softmax(p[0].astype(np.float64))) > 1e-4


def test_verify_greedy_and_out_of_range():
    V, G = 10, 4
    g = np.random.default_rng(14)
    pl = g.standard_normal((1, G + 1, V)).astype(np.float32)
    ql = g.standard_normal((1, G, V)).astype(np.float32)
    arg = pl[0].argmax(1)
    drafts = arg[:G].copy()[None].astype(np.int32)
    drafts[0, 2] = (arg[2] + 1) % V                         # first mismatch at position 3
    out, nacc, _ = oracle.verify(ql, pl, drafts, np.zeros((1, G)), np.zeros(1), 0.0)
    assert nacc[0] == 2 and list(out[0]) == [arg[0], arg[1], arg[2], -1, -1]
    drafts = arg[:G][None].astype(np.int32)
    out, nacc, _ = oracle.verify(ql, pl, drafts, np.zeros((1, G)), np.zeros(1), 0.0)
    assert nacc[0] == G and out[0, G] == arg[G]             # bonus = argmax of the last row
    bad = np.array([[V + 3, 0, 0, 0]], np.int32)            # out-of-range draft: rejected
    out, nacc, _ = oracle.verify(ql, pl, bad, np.zeros((1, G)), np.full(1, 0.5), 1.0)
    assert nacc[0] == 0 and 0 <= out[0, 0] < V


def test_verify_with_markov_drafts_matches_enumerated_expected_tau():
    V, G, r, N = 6, 3, 3, 20_000
    g = np.random.default_rng(15)
    U = (g.standard_normal((V, r)) * r ** -0.25).astype(np.float32)
    Wt = (g.standard_normal((V, r)) * r ** -0.25).astype(np.float32)
    base1 = g.standard_normal((G, V)).astype(np.float32)
    p_logits = g.standard_normal((G + 1, V)).astype(np.float32)
    last = 1
    ud = rng.uniform01(15, "mv_d", (N, G))
    ua = rng.uniform01(15, "mv_a", (N, G))
    uf = rng.uniform01(15, "mv_f", (N,))
    final, tok, _ = oracle.markov_sample(np.broadcast_to(base1, (N, G, V)), U, Wt, "f32",
                                         np.full(N, last), ud, 1.0)
    out, nacc, _ = oracle.verify(final, np.broadcast_to(p_logits, (N, G + 1, V)), tok, ua, uf, 1.0)
    table = U.astype(np.float64) @ Wt.astype(np.float64).T
    p = special.softmax(p_logits[:G].astype(np.float64), axis=1)
    q_first = special.softmax(base1[0] + table[last])
    q_next = np.stack([special.softmax(base1[i][None, :] + table, axis=1) for i in range(1, G)])
    et = oracle.expected_tau_markov(p, q_first, q_next)
    tau = oracle.tau_from_accepted(nacc)
    assert abs(tau.mean() - et) < 4 * tau.std() / np.sqrt(N)
    pf = special.softmax(p_logits.astype(np.float64), axis=1)
    for i in range(G + 1):                               # lossless with a Markov draft too
        reached = nacc >= i
        assert _chi2_pvalue(np.bincount(out[reached, i], minlength=V), pf[i]) > 1e-4


# ---------------------------------------------------------------- bookkeeping

def test_latency_bookkeeping_closed_forms_and_page_figures():
    assert oracle.latency_per_token(3.0, 5.0, 4.0) == 2.0
    assert oracle.expected_tau_independent([1, 1, 1]) == 4.0
    assert oracle.expected_tau_independent([0, 1, 1]) == 1.0
    a, G = 0.7, 5
    assert np.isclose(oracle.expected_tau_independent([a] * G), (1 - a ** (G + 1)) / (1 - a))
    # prefix-independent draft distributions: the Markov enumeration reduces to the product form
    g = np.random.default_rng(16)
    p = special.softmax(g.standard_normal((3, 4)), axis=1)
    q = special.softmax(g.standard_normal((3, 4)), axis=1)
    q_next = np.stack([np.broadcast_to(q[i], (4, 4)) for i in (1, 2)])
    alphas = [oracle.acceptance_rate(p[i], q[i]) for i in range(3)]
    assert np.isclose(oracle.expected_tau_markov(p, q[0], q_next),
                      oracle.expected_tau_independent(alphas))
    # the DSpark page's figures: +0.2-1.3 % per round for +30 % accepted length
    fx = json.load(open(os.path.join(GOLDEN, "dspark_head_latency.json")))
    lo, hi = fx["round_latency_overhead"]
    gain = fx["accepted_length_gain"]
    t_round, tau0 = 1.0, 2.0
    base_L = oracle.latency_per_token(0.3 * t_round, 0.7 * t_round, tau0)
    for ov in (lo, hi):
        L = oracle.latency_per_token(0.3 * (1 + ov), 0.7 * (1 + ov), tau0 * (1 + gain))
        assert np.isclose(L / base_L, (1 + ov) / (1 + gain))
    assert 0.770 < (1 + lo) / (1 + gain) < (1 + hi) / (1 + gain) < 0.780


# ---------------------------------------------------------------- multi-step loop

def test_loop_advance_hand_cases():
    from oracle import loop
    # gamma = 3: out_tokens = accepted drafts, then the correction/bonus token, then -1
    out = np.array([[7, -1, -1, -1],        # rejected at the first draft: correction 7
                    [4, 5, 6, 9],           # all three accepted: bonus 9
                    [4, 5, 8, -1],          # two accepted, correction 8
                    [3, -1, -1, -1]])       # an out-of-range count (-2) is clamped to 0
    n_new, last, tau = loop.advance(np.array([0, 3, 2, -2]), out, 3)
    assert n_new.tolist() == [1, 4, 3, 1]
    assert last.tolist() == [7, 9, 8, 3]
    assert tau.tolist() == [1, 4, 3, 1]
    # a count above gamma is clamped to gamma (the bonus slot)
    n_new, last, _ = loop.advance(np.array([5]), np.array([[1, 2, 3, 4]]), 3)
    assert n_new.tolist() == [4] and last.tolist() == [4]


def _loop_setup(cycles, seed=3):
    w = TINY.with_(batch=2)
    weights = inputs.drafter_weights(w, seed, gain_std=0.1)
    ctx0 = np.array([100, 61], np.int32)                 # room for every cycle's append below max_ctx
    kc, vc = inputs.cache_prefix(w, seed, ctx0)
    U, Wt = inputs.markov_factors(w, seed, std=w.markov_rank ** -0.25)
    last0 = rng.integers(seed, "last_token", (w.batch,), 0, w.vocab - 1)
    n0 = np.full(w.batch, w.block, np.int32)
    cins = [inputs.cycle_inputs(w, seed, c) for c in range(cycles)]
    return w, weights, ctx0, kc, vc, U, Wt, last0, n0, cins


def test_loop_identical_distributions_commit_the_whole_block_each_cycle():
    # target rows = the final draft rows (p = q): every draft is accepted, each
    # cycle commits S tokens, the next block starts from the bonus token and the
    # context grows by S per cycle (closed form of the loop under p = q)
    from oracle import loop
    w, weights, ctx0, kc, vc, U, Wt, last0, n0, cins = _loop_setup(3)
    S, G = w.block, w.gamma

    def same(c, final):
        t = cins[c]["target_logits"].copy()
        t[:, :G] = final
        return t

    recs = loop.run_cycles(od.DrafterShape.of(w), weights, U, Wt, "f32", kc, vc, ctx0, last0, n0, cins, 1.0,
                           target_fn=same)
    for c, r in enumerate(recs):
        assert r["n_accepted"].tolist() == [G, G]
        assert np.array_equal(r["out_tokens"][:, :G], r["draft_tokens"])
        assert r["n_new"].tolist() == [S, S] and r["tau"].tolist() == [S, S]
        assert np.array_equal(r["last_token"], r["out_tokens"][:, G])
        assert np.array_equal(r["ctx_len"], ctx0 + S * (c + 1))     # the first cycle appends n0 = S rows
    # the state each cycle starts from is what the previous cycle left
    assert np.array_equal(recs[0]["last_token_in"], last0) and np.array_equal(recs[0]["n_new_in"], n0)
    for prev, nxt in zip(recs, recs[1:]):
        assert np.array_equal(nxt["last_token_in"], prev["last_token"])
        assert np.array_equal(nxt["n_new_in"], prev["n_new"])


def test_loop_point_mass_target_commits_one_token_per_cycle():
    # target = a point mass on token t*: a first draft other than t* is rejected
    # (p = 0), the residual max(0, p - q) is the point mass, so the cycle commits
    # exactly t*, n_new = 1 and the next block starts from t*
    from oracle import loop
    w, weights, ctx0, kc, vc, U, Wt, last0, n0, cins = _loop_setup(3, seed=4)
    t_star = 17

    def point(c, final):
        t = np.full((w.batch, w.block, w.vocab), -np.inf, np.float32)
        t[:, :, t_star] = 0.0
        return t

    recs = loop.run_cycles(od.DrafterShape.of(w), weights, U, Wt, "f32", kc, vc, ctx0, last0, n0, cins, 1.0,
                           target_fn=point)
    ctx = ctx0 + n0
    for r in recs:
        for b in range(w.batch):
            if r["draft_tokens"][b, 0] != t_star:
                assert r["n_accepted"][b] == 0 and r["out_tokens"][b, 0] == t_star
                assert r["n_new"][b] == 1 and r["last_token"][b] == t_star
        assert np.array_equal(r["ctx_len"], ctx)
        ctx = ctx + r["n_new"]


# ---------------------------------------------------------------- prefix scheduler

def test_scheduler_scan_finds_the_brute_force_optimum():
    from oracle import scheduler as osch
    g = np.random.default_rng(31)
    for trial in range(60):
        B, G = int(g.integers(1, 4)), int(g.integers(1, 4))
        c = g.random((B, G)).astype(np.float32)
        xs = np.sort(g.choice(np.arange(1, 20), size=int(g.integers(2, 6)), replace=False)).astype(np.float32)
        shape = trial % 3       # decreasing (busy), increasing then flat (idle: batching helps), random
        if shape == 0:
            ys = (100.0 / (1.0 + 0.3 * xs)).astype(np.float32)
        elif shape == 1:
            ys = np.minimum(10.0 * xs, 40.0).astype(np.float32)
        else:
            ys = (g.random(len(xs)) * 50 + 1).astype(np.float32)
        k = osch.schedule(c, xs, ys)
        P = osch.prefix_survival(c)
        assert np.all((k >= 0) & (k <= G))
        assert np.isclose(osch.objective(k, P, xs, ys), osch.brute_force(c, xs, ys), rtol=1e-12, atol=0)


def test_scheduler_idle_verifies_everything_busy_verifies_less():
    from oracle import scheduler as osch
    g = np.random.default_rng(32)
    B, G = 16, 7
    c = (0.2 + 0.8 * g.random((B, G))).astype(np.float32)
    xs = np.array([1, 1000], np.float32)
    assert np.array_equal(osch.schedule(c, xs, np.array([50, 50], np.float32)), np.full(B, G))   # flat curve
    totals = []
    for alpha in (0.0, 0.01, 0.05, 0.2, 1.0, 5.0):          # SPS(N) = 1 / (1 + alpha N): heavier load
        xs = np.arange(1, B * (G + 1) + 2, dtype=np.float32)
        ys = (1.0 / (1.0 + alpha * xs)).astype(np.float32)
        totals.append(int(osch.schedule(c, xs, ys).sum()))
    assert totals[0] == B * G and all(a >= b for a, b in zip(totals, totals[1:])) and totals[-1] < totals[0]
    # nothing survives: nothing is verified
    assert np.array_equal(osch.schedule(np.zeros((B, G), np.float32), xs, ys), np.zeros(B))
