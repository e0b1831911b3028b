"""Oracle of draft-token sampling and of the Markov sequential head.

[DSpark] "Innowacje w tworzeniu tokenów": a heavy parallel core emits base
logits for every block position; a light sequential head then adds a
prefix-dependent bias before each token is sampled.  The default head is the
Markov head, which looks only at the immediately preceding token, and keeps its
cost low at large vocabularies through a rank-256 factorisation.  Written out,
with U [V, r] and W [r, V] the two factors (W is stored transposed as Wt [V, r]):

    final_i = base_i + U[prev_i] . W        prev_1 = last decoded token, prev_i = d_{i-1}
    d_i ~ softmax(final_i / T)

Readings: the bias is applied at every position including the first (whose
previous token is the last decoded token), with no scale or nonlinearity; the
sum is rounded to fp32 (the logits' storage precision) before sampling.

Sampling (T > 0) is inverse-CDF sampling with a supplied uniform u in [0, 1):
token ids are scanned in increasing order with unnormalised weights
w_v = exp((x_v - max x) / T); the drawn token is the first k whose running sum
exceeds u * sum(w) (strictly); if rounding leaves no such k, the last token with
w > 0.  T == 0 means greedy: the lowest index among the maxima.

Every draw also returns a *margin*: how far, as a fraction of the total mass,
the threshold lies from the nearest boundary of the chosen token's interval
(greedy: the gap between the largest and second largest logit).  A draw with a
margin below 1e-6 may legitimately differ between two correct implementations
whose roundings differ; tests exclude such draws.
"""
from __future__ import annotations

import numpy as np

from .rounding import as_f64, round_f32


def softmax_weights(logits, temperature):
    """Unnormalised weights exp((x - max) / T) in float64 along the last axis."""
    x = np.asarray(logits, np.float64)
    return np.exp((x - x.max(axis=-1, keepdims=True)) / temperature)


def inverse_cdf(w, u):
    """Inverse-CDF draw from unnormalised non-negative weights w with uniform u.

    Returns (token, margin).
    """
    w = np.asarray(w, np.float64)
    total = float(np.sum(w))
    t = float(u) * total
    cum = np.cumsum(w)
    hit = np.nonzero(cum > t)[0]
    if hit.size:
        k = int(hit[0])
    else:
        k = int(np.nonzero(w > 0)[0][-1])
    lo = cum[k - 1] if k > 0 else 0.0
    margin = min(t - lo, cum[k] - t) / total
    return k, float(margin)


def argmax_with_gap(logits):
    x = np.asarray(logits, np.float64)
    k = int(np.argmax(x))                   # first index among equal maxima
    if x.size == 1:
        return k, np.inf
    top2 = np.partition(x, -2)[-2:]
    return k, float(top2[1] - top2[0])


def sample_row(logits, u, temperature):
    """One draw from softmax(logits / T) (T > 0) or greedy (T == 0)."""
    if temperature == 0:
        return argmax_with_gap(logits)
    return inverse_cdf(softmax_weights(logits, temperature), u)


def markov_sample(base_logits, U, Wt, uw_dtype, last_token, u_draft, temperature):
    """Sequential sampling of the gamma draft positions with the Markov head.

    base_logits [B, gamma, V] fp32; U, Wt [V, r] in ``uw_dtype`` storage (None or
    rank 0 = no head, positions independent); last_token [B]; u_draft [B, gamma].
    Returns (final_logits [B, gamma, V] float32, tokens [B, gamma] int32,
    margins [B, gamma] float64).  Out-of-range previous tokens are clamped.
    """
    base = np.asarray(base_logits, np.float32)
    B, G, V = base.shape
    final = base.copy()
    tokens = np.zeros((B, G), np.int32)
    margins = np.zeros((B, G), np.float64)
    has_head = U is not None and np.asarray(U).size > 0
    if has_head:
        Uf = as_f64(U, uw_dtype)
        Wf = as_f64(Wt, uw_dtype)
    for b in range(B):
        prev = int(last_token[b])
        for i in range(G):
            row = base[b, i].astype(np.float64)
            if has_head:
                p = min(max(prev, 0), V - 1)
                bias = round_f32(Wf @ Uf[p])            # U[prev] . W, one value per vocab entry
                row = round_f32(row + bias)
                final[b, i] = row.astype(np.float32)
            k, m = sample_row(row, u_draft[b, i], temperature)
            tokens[b, i] = k
            margins[b, i] = m
            prev = k
    return final, tokens, margins


def rnn_states(U, A, uw_dtype, prev_tokens):
    """States of the RNN sequential head along one block (float64).

    [DSpark] "Innowacje w tworzeniu tokenów": besides the default Markov head
    the page names an optional RNN head that follows the whole block prefix
    (with only a marginal gain over the Markov head).  It gives no structure, so
    the cell is a reading: an Elman cell whose state has the head's rank r,

        h_0 = 0,   h_i = tanh(U[prev_i] + A h_{i-1})      i = 1 .. gamma

    with the Markov head's input factor U [V, r] as the input embedding (so the
    i-th input is the same previous token the Markov head looks up), a
    recurrent matrix A [r, r] (row j holds the weights into state element j),
    no bias; the state is kept in full precision.  prev_tokens [gamma] are the
    previous tokens prev_1 .. prev_gamma (clamped to the vocabulary).
    Returns [gamma, r].
    """
    Uf = as_f64(U, uw_dtype)
    Af = as_f64(A, uw_dtype)
    V, r = Uf.shape
    h = np.zeros(r)
    out = np.zeros((len(prev_tokens), r))
    for i, p in enumerate(prev_tokens):
        p = min(max(int(p), 0), V - 1)
        h = np.tanh(Uf[p] + Af @ h)
        out[i] = h
    return out


def rnn_sample(base_logits, U, Wt, A, uw_dtype, last_token, u_draft, temperature):
    """Sequential sampling of the gamma draft positions with the RNN head.

    final_i = base_i + W h_i (the Markov head's output factor, Wt [V, r]; the
    bias rounded to fp32, then the sum, as for the Markov head), h_i from
    ``rnn_states`` with prev_1 = last decoded token and prev_i = d_{i-1}; each
    draw as in ``sample_row``.  Returns (final_logits [B, gamma, V] float32,
    tokens [B, gamma] int32, margins [B, gamma] float64, states [B, gamma, r]).
    """
    base = np.asarray(base_logits, np.float32)
    B, G, V = base.shape
    Uf = as_f64(U, uw_dtype)
    Wf = as_f64(Wt, uw_dtype)
    Af = as_f64(A, uw_dtype)
    r = Uf.shape[1]
    final = base.copy()
    tokens = np.zeros((B, G), np.int32)
    margins = np.zeros((B, G), np.float64)
    states = np.zeros((B, G, r))
    for b in range(B):
        prev = int(last_token[b])
        h = np.zeros(r)
        for i in range(G):
            p = min(max(prev, 0), V - 1)
            h = np.tanh(Uf[p] + Af @ h)
            states[b, i] = h
            bias = round_f32(Wf @ h)
            row = round_f32(base[b, i].astype(np.float64) + bias)
            final[b, i] = row.astype(np.float32)
            k, m = sample_row(row, u_draft[b, i], temperature)
            tokens[b, i] = k
            margins[b, i] = m
            prev = k
    return final, tokens, margins, states
