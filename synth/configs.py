"""Workload shapes for the block speculative draft-and-verify step.

Pure data: sizes, dtypes and the distributions the synthetic inputs are drawn
from.  Nothing here computes any part of the method.

Names follow the pages' notation: B batch, S block (1 last decoded token plus
gamma = S-1 mask tokens), C context length, L drafter layers, H hidden, nq/nkv
query/key-value heads of width d, F MLP width, V vocabulary, nT target layers
whose hidden states are concatenated, r Markov-head rank, T temperature.
"""
from __future__ import annotations

from dataclasses import dataclass, replace


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    block: int
    ctx: int                 # context keys a block row attends to after the step's append
    n_layers: int
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    mlp_dim: int
    vocab: int
    n_target_layers: int
    markov_rank: int          # 0 = no Markov head (independent positions)
    dtype: str                # "f32" or "bf16": weights, hiddens, K/V cache, GEMM inputs
    target_logit_std: float   # std of synthetic target logits
    target_noise_std: float = 0.0   # >0: target logits = draft logits + N(0, std^2)
    temperature: float = 1.0
    rms_eps: float = 1e-6
    rope_theta: float = 1e6
    weight_std: float = 0.02
    hidden_std: float = 1.0
    base_logit_std: float = 1.28    # std of synthetic base logits fed to the sampler alone
    markov_factor_std: float = 0.02
    window: int = 0                 # > 0: block rows attend only the last `window` context keys

    @property
    def gamma(self) -> int:
        return self.block - 1

    @property
    def mask_token_id(self) -> int:
        return self.vocab - 1

    @property
    def max_ctx(self) -> int:
        # cache capacity: the context rounded up to 64 slots plus one more 64-slot
        # step (room for the next append; it also keeps the per-head slot stride off
        # large powers of two, which would put every head's block on the same HBM
        # channels)
        return (self.ctx + 63) // 64 * 64 + 64

    @property
    def ctx_before(self) -> int:
        """Context length before the step appends the S newly committed rows."""
        return self.ctx - self.block

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


_BIG = dict(n_layers=5, hidden=4096, n_q_heads=32, n_kv_heads=8, head_dim=128,
            mlp_dim=12288, n_target_layers=5, dtype="bf16")

TINY = Workload("tiny_fp32_b1_s4_c128", batch=1, block=4, ctx=128, n_layers=2, hidden=256,
                n_q_heads=4, n_kv_heads=4, head_dim=64, mlp_dim=1024, vocab=1000,
                n_target_layers=3, markov_rank=16, dtype="f32", target_logit_std=2.0)
DFLASH = Workload("dflash_bf16_b8_s16_c4096_v151936", batch=8, block=16, ctx=4096,
                  vocab=151936, markov_rank=0, target_logit_std=3.0, **_BIG)
DSPARK = Workload("dspark_markov_bf16_b32_s16_c4096_v129280", batch=32, block=16, ctx=4096,
                  vocab=129280, markov_rank=256, target_logit_std=3.0, **_BIG)
LONGCTX = Workload("longctx_bf16_b4_s16_c32768_v151936", batch=4, block=16, ctx=32768,
                   vocab=151936, markov_rank=256, target_logit_std=3.0, **_BIG)
HIGHBATCH = Workload("highbatch_bf16_b128_s8_c2048_v129280", batch=128, block=8, ctx=2048,
                     vocab=129280, markov_rank=256, target_logit_std=3.0,
                     target_noise_std=1.0, **_BIG)

# the DSpark drafter variant: 3 layers attending a 128-token window of the
# context, 5-token block (1 last token + 4 drafts), otherwise as C2
DSPARK_WINDOW = Workload("dspark_window_bf16_b32_s5_c4096_w128_v129280", batch=32, block=5, ctx=4096,
                         vocab=129280, markov_rank=256, target_logit_std=3.0,
                         **{**_BIG, "n_layers": 3}, window=128)

WORKLOADS = {"C0": TINY, "C1": DFLASH, "C2": DSPARK, "C3": LONGCTX, "C4": HIGHBATCH, "C5": DSPARK_WINDOW}

# a bf16 drafter with the big configs' structure (GQA 32/8 x 128) at a size the
# oracle finishes in seconds, spanning several GEMM and attention tiles with ragged tails
MEDIUM = Workload("medium_bf16_b3_s16_c300", batch=3, block=16, ctx=300, n_layers=2, hidden=512,
                  n_q_heads=8, n_kv_heads=2, head_dim=128, mlp_dim=1536, vocab=5000,
                  n_target_layers=3, markov_rank=64, dtype="bf16", target_logit_std=3.0)
