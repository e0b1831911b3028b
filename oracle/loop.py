"""Oracle of the multi-step draft -> sample -> verify loop (TEST INFRASTRUCTURE ONLY).

[DSpark] "Jak działa spekulatywne dekodowanie DSpark?": each cycle the target
keeps the longest valid prefix of the drafts and adds one token, so a cycle
commits tau = accepted + 1 tokens; [DFlash] latency paragraph counts the same
tau (accepted length including the bonus token).  [DFlash] architecture
paragraph: the drafter conditions on the context features of the tokens the
target has committed, and its block starts from the last decoded token.

Readings (listed with their reasons in the design notes):

* the rows the next drafter call appends are exactly the tokens committed by
  the last cycle, n_new = accepted + 1, and their target hidden states are an
  input of that call (the target model is not part of the loop; tests and the
  benchmark draw them from a seeded pool);
* the next block's first slot is the last committed token, i.e. the correction
  token at the first rejection or the bonus token after a fully accepted block;
* an out-of-range accepted count is clamped to [0, gamma].
"""
from __future__ import annotations

import numpy as np

from . import drafter as od
from .sampling import markov_sample, rnn_sample
from .scheduler import schedule
from .verify import verify


def advance(n_accepted, out_tokens, n_draft):
    """Device-side bookkeeping between two cycles.

    n_accepted [B]; out_tokens [B, n_draft + 1] (accepted drafts, then the
    correction or bonus token).  Returns (n_new [B], last_token [B], tau [B]):
    the rows the next drafter call appends, the next block's first token, and
    the tokens this cycle committed."""
    out_tokens = np.asarray(out_tokens, np.int64)
    a = np.clip(np.asarray(n_accepted, np.int64), 0, n_draft)
    last = out_tokens[np.arange(len(a)), a]
    return (a + 1).astype(np.int32), last.astype(np.int32), a + 1


def run_cycles(shape, weights, U, Wt, uw_dtype, k_cache, v_cache, ctx_len, last_token, n_new, cycles,
               temperature, target_fn=None, curve=None, A=None):
    """Run len(cycles) cycles of draft -> Markov sample -> verify -> advance
    (with the RNN head's recurrent matrix ``A``: RNN-head sampling instead).

    ``cycles[c]`` holds that cycle's inputs: hidden_new [B, S, nT*H] (rows
    < n_new[b] used), u_draft [B, gamma], u_accept [B, gamma], u_final [B], and
    target_logits [B, S, V] unless ``target_fn(c, final_draft_logits)`` supplies
    them.  With ``curve`` = (rows, passes per second) each cycle's ``survival``
    [B, gamma] goes through the prefix scheduler and only the chosen drafts are
    verified.  k_cache, v_cache (logical layout) are updated in place; ctx_len,
    last_token, n_new are the state before the first cycle.  Returns one record
    per cycle with everything either side emits plus the draws' margins."""
    G = shape.block - 1
    ctx = np.asarray(ctx_len, np.int64).copy()
    last = np.asarray(last_token, np.int32).copy()
    nn = np.asarray(n_new, np.int32).copy()
    out = []
    for c, cin in enumerate(cycles):
        last_in, n_new_in = last.copy(), nn.copy()
        base, ctx = od.draft_step(shape, weights, cin["hidden_new"], nn, k_cache, v_cache, ctx, last)
        if A is not None:
            final, tokens, m_draft, _ = rnn_sample(base, U, Wt, A, uw_dtype, last, cin["u_draft"], temperature)
        else:
            final, tokens, m_draft = markov_sample(base, U, Wt, uw_dtype, last, cin["u_draft"], temperature)
        target = target_fn(c, final) if target_fn is not None else cin["target_logits"]
        n_verify = None
        if curve is not None:
            n_verify = schedule(cin["survival"], curve[0], curve[1])
        out_tok, n_acc, m_ver = verify(final, target, tokens, cin["u_accept"], cin["u_final"], temperature,
                                       n_verify=n_verify)
        nn, last, tau = advance(n_acc, out_tok, G)
        out.append(dict(draft_tokens=tokens, n_accepted=n_acc, out_tokens=out_tok, n_new=nn, last_token=last,
                        tau=tau, ctx_len=ctx.copy(), margins_draft=m_draft, margins_verify=m_ver,
                        final_logits=final, last_token_in=last_in, n_new_in=n_new_in, n_verify=n_verify))
    return out
