"""Oracle of rejection-sampling verification.

[DSpark] "Jak działa spekulatywne dekodowanie DSpark?": the target model checks
the drafted block in one pass; rejection sampling keeps the longest valid
prefix and adds one more token, which exactly preserves the target
distribution.  The acceptance rule itself is [SpecSampling]:

  for i = 1 .. gamma:   p_i = softmax(target_i / T), q_i = softmax(draft_i / T)
      r_i = p_i(d_i) / q_i(d_i)      (q = 0: +inf when p > 0, else 0)
      accept d_i iff u_accept_i < r_i
  at the first rejection a: emit a token drawn from normalise(max(0, p_a - q_a))
      with u_final (if that residual has no mass, draw from p_a instead) and stop;
  if every draft is accepted: emit a bonus token drawn from p_{gamma+1} with u_final.

T == 0 is greedy verification: accept while d_i equals the target argmax;
emit the target argmax at the first mismatch, or the bonus argmax.

Readings: the comparison is strict (u in [0,1), so r >= 1 always accepts); a
draft token outside [0, V) is rejected; the draws use the inverse-CDF
convention of ``sampling.inverse_cdf``.

Output per batch row: out_tokens [gamma+1] = accepted drafts, then the
correction or bonus token, then -1; n_accepted = number of accepted drafts;
tau = n_accepted + 1 tokens are produced.
"""
from __future__ import annotations

import numpy as np

from .sampling import softmax_weights, inverse_cdf, argmax_with_gap


def verify(draft_logits, target_logits, draft_tokens, u_accept, u_final, temperature, n_verify=None):
    """Returns (out_tokens [B, gamma+1] int32, n_accepted [B] int32,
    margins [B, gamma+1] float64 (accept tests, then the final draw in the last
    column; inf for positions not reached)).

    ``n_verify`` [B] (optional): row b verifies only its first k_b drafts
    (clamped to [0, gamma]) — the prefix scheduler's early stopping ([DSpark]
    "Optymalizacja weryfikacji i wydajności"); if all k_b are accepted the bonus
    token is drawn from target row k_b.  The rule on a k_b-draft block."""
    q_all = np.asarray(draft_logits, np.float32)
    p_all = np.asarray(target_logits, np.float32)
    B, G, V = q_all.shape
    out = np.full((B, G + 1), -1, np.int32)
    n_acc = np.zeros(B, np.int32)
    margins = np.full((B, G + 1), np.inf)
    for b in range(B):
        kb = G if n_verify is None else int(np.clip(n_verify[b], 0, G))
        a = kb
        for i in range(kb):
            d = int(draft_tokens[b, i])
            if temperature == 0:
                t_arg, gap = argmax_with_gap(p_all[b, i])
                margins[b, i] = gap
                if d == t_arg:
                    out[b, i] = d
                    continue
                out[b, i] = t_arg
                a = i
                break
            wp = softmax_weights(p_all[b, i], temperature)
            wq = softmax_weights(q_all[b, i], temperature)
            p = wp / wp.sum()
            q = wq / wq.sum()
            if 0 <= d < V:
                if q[d] > 0:
                    r = p[d] / q[d]
                else:
                    r = np.inf if p[d] > 0 else 0.0
            else:
                r = 0.0
            u = float(u_accept[b, i])
            margins[b, i] = abs(u - min(r, 1.0))
            if u < r:
                out[b, i] = d
                continue
            resid = np.maximum(0.0, p - q)
            if resid.sum() > 0:
                tok, m = inverse_cdf(resid, u_final[b])
            else:
                tok, m = inverse_cdf(p, u_final[b])
            out[b, i] = tok
            margins[b, G] = m
            a = i
            break
        if a == kb:                                   # every verified draft accepted: bonus from row kb
            if temperature == 0:
                tok, m = argmax_with_gap(p_all[b, kb])
            else:
                tok, m = inverse_cdf(softmax_weights(p_all[b, kb], temperature), u_final[b])
            out[b, kb] = tok
            margins[b, G] = m
        n_acc[b] = a
    return out, n_acc, margins
