"""Oracle of the hardware-aware prefix scheduler (TEST INFRASTRUCTURE ONLY).

[DSpark] "Optymalizacja weryfikacji i wydajności": a confidence head scores each
draft position with its chance of surviving verification given accepted
predecessors; a hardware-aware prefix scheduler sets the verify length of each
request from a throughput curve SPS(B) profiled once at startup — more tokens
when the GPUs are idle, fewer when they are busy — and keeps losslessness by
early stopping.  [DSpark-fr] "DSpark — le décodage spéculatif": the scheduler
combines the prefix survival probabilities with the measured throughput curves
to maximise the expected system throughput under the current load.

Readings (listed with their reasons in the design notes):

* c[b, i] is the conditional survival of draft i of request b (clipped to
  [0, 1]; NaN counts as 0); prefix survival P[b, k] = c[b, 0] * ... * c[b, k]
  (probability that the first k+1 drafts all survive), products in float64;
* verifying k_b drafts of request b puts k_b + 1 rows into the verify batch and
  commits 1 + sum_{j < k_b} P[b, j] tokens in expectation;
* the curve gives verify passes per second as a function of the rows N in the
  batch, linear between its points and constant beyond its ends;
* the scheduler maximises SPS(N) * sum_b (1 + sum_{j < k_b} P[b, j]) over the
  lengths k_b in [0, gamma]; the first maximum in the order below wins.

Because P[b, j] does not increase along j, the best lengths for a given number
M of verified drafts take the M largest P values (ties: lower request, then
lower position first), which are prefixes of each request; scanning M therefore
finds the exact optimum, and ``brute_force`` checks that on small cases.
"""
from __future__ import annotations

import itertools

import numpy as np


def prefix_survival(c):
    c = np.asarray(c, np.float32).astype(np.float64)
    c = np.where(np.isnan(c), 0.0, np.clip(c, 0.0, 1.0))
    out = np.empty_like(c)
    for b in range(c.shape[0]):
        acc = 1.0
        for j in range(c.shape[1]):
            acc = acc * c[b, j]
            out[b, j] = acc
    return out


def sps_at(n, xs, ys):
    """Throughput curve at n rows: linear between points, constant past the ends."""
    xs = np.asarray(xs, np.float32).astype(np.float64)
    ys = np.asarray(ys, np.float32).astype(np.float64)
    n = float(n)
    if n <= xs[0]:
        return ys[0]
    if n >= xs[-1]:
        return ys[-1]
    i = int(np.searchsorted(xs, n, side="right")) - 1
    return ys[i] + (ys[i + 1] - ys[i]) * ((n - xs[i]) / (xs[i + 1] - xs[i]))


def objective(k, P, xs, ys):
    k = np.asarray(k, np.int64)
    B = P.shape[0]
    tokens = sum(1.0 + P[b, :k[b]].sum() for b in range(B))
    return sps_at(int(k.sum()) + B, xs, ys) * tokens


def schedule(c, xs, ys):
    """Verify lengths k [B] (int32) maximising the expected throughput."""
    P = prefix_survival(c)
    B, G = P.shape
    order = sorted(range(B * G), key=lambda e: (-P.flat[e], e))
    best, best_m = sps_at(B, xs, ys) * B, 0
    acc = 0.0
    for m in range(1, B * G + 1):
        acc = acc + P.flat[order[m - 1]]
        o = sps_at(B + m, xs, ys) * (B + acc)
        if o > best:
            best, best_m = o, m
    k = np.zeros(B, np.int32)
    for e in order[:best_m]:
        k[e // G] += 1
    return k


def brute_force(c, xs, ys):
    """All (gamma+1)^B length vectors (small cases only): the best objective."""
    P = prefix_survival(c)
    B, G = P.shape
    return max(objective(k, P, xs, ys) for k in itertools.product(range(G + 1), repeat=B))
