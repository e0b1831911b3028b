"""Multi-step draft -> sample -> verify loop on one stream, with no host synchronisation.

Every step of a cycle runs in the library's kernels: ``dflash_draft_step`` appends
the rows the previous cycle committed and drafts a block, ``markov_bias_sample``
draws the drafts, the caller supplies the target logits (the target model is not
part of this library), ``spec_verify`` accepts or rejects, and
``spec_cycle_advance`` turns its outputs into the next call's n_new and last
token on the device (DSpark page, section "Jak działa spekulatywne dekodowanie
DSpark?": each cycle commits the accepted prefix plus one token).  The host only
enqueues work, so a chain of cycles can be captured into one HIP graph
(``torch.cuda.graph``) and replayed.

This module only holds buffers and passes pointers; it computes nothing itself.
"""
from __future__ import annotations

import torch

from . import dfspec as D


class SpecLoop:
    """State and buffers of a chain of cycles for one batch.

    k_cache, v_cache: the library's cache layouts with room for every cycle's
    append; ctx_len, last_token, n_new: device int32 [B], the state before the
    first cycle (updated in place by every cycle).  The host-side bounds passed
    to the drafter hold for any cycle: n_new_max = S and ctx_bound = the cache
    capacity, so the same enqueued work is valid whatever the device-side state."""

    def __init__(self, cfg: D.DrafterConfig, weights: D.DrafterWeights, k_cache, v_cache, ctx_len, last_token, n_new,
                 temperature: float = 1.0, U=None, Wt=None, wt_packed: bool = False, curve=None, A=None):
        """curve: optional (rows, passes per second) throughput table for the prefix
        scheduler; with it, a cycle given survival scores verifies per request only
        the drafts spec_schedule_verify picks.  A: the RNN head's recurrent matrix
        [r, r]; with it the drafts come from rnn_bias_sample instead of the Markov
        head."""
        B = ctx_len.numel()
        S, V = cfg.block, cfg.vocab
        G = S - 1
        dev = ctx_len.device
        self.cfg, self.weights, self.B, self.S, self.G, self.V = cfg, weights, B, S, G, V
        self.k_cache, self.v_cache = k_cache, v_cache
        self.ctx_len, self.last_token, self.n_new = ctx_len, last_token, n_new
        self.temperature = float(temperature)
        self.U, self.Wt, self.wt_packed, self.A = U, Wt, wt_packed, A
        self.logits = torch.empty((B, G, V), dtype=torch.float32, device=dev)
        self.tokens = torch.empty((B, G), dtype=torch.int32, device=dev)
        self.row_stats = torch.empty((B, G, 2), dtype=torch.float64, device=dev)
        self.target = torch.empty((B, S, V), dtype=torch.float32, device=dev)
        self.out_tokens = torch.empty((B, S), dtype=torch.int32, device=dev)
        self.n_accepted = torch.empty(B, dtype=torch.int32, device=dev)
        self.tau_sum = torch.zeros(B, dtype=torch.int64, device=dev)
        self.curve = curve
        self.n_verify = torch.full((B,), G, dtype=torch.int32, device=dev)
        self.ws_draft = torch.empty(D.dflash_draft_workspace_size(cfg, B, S), dtype=torch.uint8, device=dev)
        ws_head = (D.rnn_bias_sample_workspace_size(B, G, V, U.shape[1]) if A is not None
                   else D.markov_bias_sample_workspace_size(B, G, V))
        self.ws_markov = torch.empty(ws_head, dtype=torch.uint8, device=dev)
        self.ws_verify = torch.empty(D.spec_verify_workspace_size(B, G, V), dtype=torch.uint8, device=dev)

    def cycle(self, hidden_new, u_draft, u_accept, u_final, target_fn, survival=None):
        """Enqueue one cycle.  hidden_new [B, S, nT*H]: target hidden states of the
        rows committed by the previous cycle (rows >= n_new[b] ignored); u_draft,
        u_accept [B, gamma], u_final [B]; target_fn(final_draft_logits, target)
        enqueues the target logits [B, S, V] into ``target``; survival [B, gamma]
        (device fp32, with a curve): per-position survival scores for the
        scheduler."""
        D.dflash_draft_step(self.cfg, self.weights, hidden_new, self.n_new, self.S, self.cfg.max_ctx, self.k_cache,
                            self.v_cache, self.ctx_len, self.last_token, self.logits, self.ws_draft)
        if self.A is not None:
            D.rnn_bias_sample(self.logits, self.U, self.Wt, self.A, self.last_token, u_draft, self.temperature,
                              self.tokens, self.row_stats, self.ws_markov, wt_packed=self.wt_packed)
        else:
            D.markov_bias_sample(self.logits, self.U, self.Wt, self.last_token, u_draft, self.temperature,
                                 self.tokens, self.row_stats, self.ws_markov, wt_packed=self.wt_packed)
        target_fn(self.logits, self.target)
        nv = None
        if survival is not None and self.curve is not None:
            D.spec_schedule_verify(survival, self.curve[0], self.curve[1], self.n_verify)
            nv = self.n_verify
        D.spec_verify(self.logits, self.target, self.tokens, u_accept, u_final, self.temperature, self.row_stats,
                      self.out_tokens, self.n_accepted, self.ws_verify, n_verify=nv)
        D.spec_cycle_advance(self.n_accepted, self.out_tokens, self.n_new, self.last_token, self.tau_sum)
