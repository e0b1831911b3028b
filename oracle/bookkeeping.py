"""Oracle of the cycle bookkeeping.

[DSpark] "Jak działa spekulatywne dekodowanie DSpark?": per-token latency
L = (T_draft + T_verify) / tau, tau = tokens accepted per cycle.  [DFlash]
first paragraph states the same quantity with tau = mean accepted length
including the bonus token.  [DSpark] "Optymalizacja weryfikacji i wydajności":
minimising the total-variation loss directly maximises the acceptance rate;
the per-position acceptance probability is alpha = sum_v min(p(v), q(v)) =
1 - TV(p, q) [SpecSampling].
"""
from __future__ import annotations

import itertools

import numpy as np


def tau_from_accepted(n_accepted):
    """Tokens produced per cycle: accepted drafts plus the correction/bonus token."""
    return np.asarray(n_accepted, np.int64) + 1


def latency_per_token(t_draft, t_verify, tau):
    """L = (T_draft + T_verify) / tau (tau = mean tokens per cycle)."""
    return (np.asarray(t_draft, np.float64) + np.asarray(t_verify, np.float64)) / np.asarray(tau, np.float64)


def acceptance_rate(p, q):
    """Probability that one draft drawn from q survives verification against p."""
    p = np.asarray(p, np.float64)
    q = np.asarray(q, np.float64)
    return float(np.minimum(p, q).sum())


def expected_tau_independent(alphas):
    """E[tau] when position i is accepted with probability alpha_i independently of
    the prefix: sum_{k=0}^{gamma} prod_{i<=k} alpha_i (empty product = 1)."""
    a = np.asarray(alphas, np.float64)
    return float(1.0 + np.sum(np.cumprod(a)))


def expected_tau_markov(p, q_first, q_next):
    """Exact E[tau] by enumeration for a Markov draft distribution.

    p [gamma, V]: target distribution per position (prefix independent);
    q_first [V]: draft distribution of position 1; q_next [gamma-1, V, V]:
    q_next[i-1, prev, v] = draft distribution of position i+1 given d_i = prev.
    The draft prefix d_1..d_k survives with probability
    prod_i q_i(d_i | d_{i-1}) min(1, p_i(d_i) / q_i(d_i | d_{i-1}))
    = prod_i min(q_i(d_i | d_{i-1}), p_i(d_i)).
    """
    p = np.asarray(p, np.float64)
    G, V = p.shape
    et = 1.0
    for k in range(1, G + 1):
        tot = 0.0
        for seq in itertools.product(range(V), repeat=k):
            pr = min(q_first[seq[0]], p[0, seq[0]])
            for i in range(1, k):
                pr *= min(q_next[i - 1, seq[i - 1], seq[i]], p[i, seq[i]])
            tot += pr
        et += tot
    return et
