"""CPU oracle for one block-parallel speculative draft-and-verify step.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product path
(the HIP library and its Python binding) never calls it, and it never calls the
product path: the two share no code.  The only module both sides use is
``synth`` (seeded input generation, which contains none of the method's
arithmetic).

Everything is plain NumPy in float64.  Values are rounded to the declared
storage precision (bf16 or fp32) at the same tensor boundaries as the storage
the GPU path uses, so that both sides compute the same function; inside one
boundary the oracle keeps full float64.  (``draft_step`` can also evaluate the
same steps in fp32 arithmetic; tests use that only to measure how far any
fp32 evaluation drifts from the float64 one.)

Citation key (the pages, by title; sections are named as they appear):

* [DFlash]  "DFlash — диффузионный метод спекулятивного декодинга", Душный NLP
  channel post (telemetr.me/content/stuffynlp).  Paragraphs used: latency per
  token (verify + draft time over mean accepted length incl. the bonus token),
  architecture (five-layer transformer; first layer gets the last decoded token
  plus mask tokens; context features = hidden states of several target layers,
  concatenated, linearly projected and normalised; the same features enter
  every layer: "KV injection"; full attention inside the block, causal toward
  the previous context).
* [DSpark]  "DeepSeek prezentuje DSpark: przyspieszenie generowania
  DeepSeek-V4 o 60-85%" (aigest.pl).  Sections: "Jak działa spekulatywne
  dekodowanie DSpark?" (rejection sampling keeps the longest valid prefix plus
  one token and exactly preserves the target distribution; latency
  L = (T_draft + T_verify) / tau), "Innowacje w tworzeniu tokenów" (parallel
  core emits base logits per position; light sequential head adds a
  prefix-dependent bias before each token is sampled; Markov head = previous
  token only, rank-256 factorisation; an optional RNN head follows the whole
  block prefix), "Optymalizacja weryfikacji i wydajności"
  (total-variation loss <-> acceptance rate), "Wyniki i zastosowania
  produkcyjne" (draft length 4 -> 16 costs 0.2-1.3 % latency per round for
  +30 % accepted length).
* [DSpark-fr]  "Single-Pass mHC, Engram et DSpark" (mkdocs.reaper.mx, DeepSeek
  V4.1-Flash architecture notes), section "DSpark — le décodage spéculatif",
  table "Ce que fait DSpark" (one pass gives the base logits of all block
  positions; Markov head models dependencies between draft tokens).
* [SpecSampling] the standard speculative-sampling acceptance rule the pages
  name but do not print: accept draft d_i while u_i < p_i(d_i) / q_i(d_i); at
  the first rejection sample from normalise(max(0, p_i - q_i)); if every draft
  is accepted append one bonus token drawn from the next target distribution.

Functions without an independent pin are marked "parity unpinned" in their
docstrings; at present there are none.
"""
from .rounding import round_bf16, round_f32, bf16_bits_to_f64, f64_to_bf16_bits, round_to
from .drafter import (rmsnorm, rope_rotate, block_attention, context_features,
                      draft_step, DrafterShape)
from .sampling import (softmax_weights, inverse_cdf, argmax_with_gap, sample_row,
                       markov_sample, rnn_states, rnn_sample)
from .verify import verify
from .bookkeeping import (tau_from_accepted, latency_per_token, acceptance_rate,
                          expected_tau_independent, expected_tau_markov)

__all__ = [
    "round_bf16", "round_f32", "bf16_bits_to_f64", "f64_to_bf16_bits", "round_to",
    "rmsnorm", "rope_rotate", "block_attention", "context_features", "draft_step",
    "DrafterShape", "softmax_weights", "inverse_cdf", "argmax_with_gap", "sample_row",
    "markov_sample", "rnn_states", "rnn_sample", "verify", "tau_from_accepted", "latency_per_token",
    "acceptance_rate", "expected_tau_independent", "expected_tau_markov",
]
