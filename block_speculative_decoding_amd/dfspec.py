"""ctypes binding of libdfspec.so (argument marshalling only).

Every function here takes torch tensors that already live on the GPU, checks
their dtype/shape/contiguity, and passes raw pointers and sizes to the C ABI of
``include/dfspec.h`` on torch's current HIP stream.  No arithmetic of the step
happens in Python.  If the library is missing, importing this module raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdfspec.so")

DFS_OK, DFS_EINVAL, DFS_EUNSUPPORTED, DFS_EHIP, DFS_EWORKSPACE = 0, -1, -2, -3, -4
DFS_F32, DFS_BF16, DFS_BF16_PACKED = 0, 1, 2

EXPORTS = [
    "dflash_draft_workspace_size", "dflash_draft_step",
    "markov_bias_sample_workspace_size", "markov_bias_sample", "rnn_bias_sample_workspace_size", "rnn_bias_sample",
    "spec_verify_workspace_size", "spec_verify", "dfs_status_string",
    "dfs_block_attention_workspace_size", "dfs_block_attention",
    "dfs_gemm_workspace_size", "dfs_gemm", "dfs_profile_begin", "dfs_profile_end",
    "dfs_packed_matrix_bytes", "dfs_pack_matrix", "dfs_gemm_swiglu", "spec_cycle_advance", "spec_schedule_verify",
    "dfs_draft_trace_layout", "spec_verify_static", "dfs_gemm_skip",
]


class DfsError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} ({status})")


class CDrafterCfg(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "n_layers", "hidden", "n_q_heads", "n_kv_heads", "head_dim", "mlp_dim", "vocab",
        "n_target_layers", "block", "max_ctx", "mask_token_id")] + [
        ("rms_eps", ctypes.c_float), ("rope_theta", ctypes.c_float), ("dtype", ctypes.c_int32),
        ("window", ctypes.c_int32)]


_PP = ctypes.POINTER(ctypes.c_void_p)


class CDrafterWeights(ctypes.Structure):
    _fields_ = [("embed", ctypes.c_void_p), ("fc", ctypes.c_void_p), ("fc_norm", ctypes.c_void_p),
                ("final_norm", ctypes.c_void_p), ("lm_head", ctypes.c_void_p)] + [
        (n, _PP) for n in ("attn_norm", "wq", "wk", "wv", "wo", "mlp_norm", "w_gate", "w_up",
                           "w_down")] + [("packed", ctypes.c_int32)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built: run `python -m block_speculative_decoding_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    sig = {
        "dflash_draft_workspace_size": (sz, [vp, i32, i32]),
        "dflash_draft_step": (ctypes.c_int, [vp, vp, i32, vp, vp, i32, i32, vp, vp, vp, vp, vp, vp, sz, vp]),
        "markov_bias_sample_workspace_size": (sz, [i32, i32, i32]),
        "markov_bias_sample": (ctypes.c_int, [i32, i32, i32, i32, vp, vp, vp, i32, vp, vp, f32, vp, vp,
                                              vp, sz, vp]),
        "rnn_bias_sample_workspace_size": (sz, [i32, i32, i32, i32]),
        "rnn_bias_sample": (ctypes.c_int, [i32, i32, i32, i32, vp, vp, vp, vp, i32, vp, vp, f32, vp, vp,
                                           vp, sz, vp]),
        "spec_verify_workspace_size": (sz, [i32, i32, i32]),
        "spec_verify": (ctypes.c_int, [i32, i32, i32, vp, vp, vp, vp, vp, f32, vp, vp, vp, vp, vp, sz, vp]),
        "spec_verify_static": (ctypes.c_int, [i32, i32, i32, vp, vp, vp, vp, vp, f32, vp, vp, vp, vp, vp]),
        "dfs_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "dfs_block_attention_workspace_size": (sz, [i32, i32, i32, i32, i32, i32, i32]),
        "dfs_block_attention": (ctypes.c_int, [i32, i32, i32, i32, i32, i32, i32, i32, i32, vp, vp, vp, vp,
                                               vp, vp, vp, vp, sz, vp]),
        "dfs_gemm_workspace_size": (sz, [i32, i32, i32, i32, i32]),
        "dfs_gemm": (ctypes.c_int, [i32, i32, i32, i32, vp, vp, vp, i32, i32, vp, sz, vp]),
        "dfs_gemm_skip": (ctypes.c_int, [i32, i32, i32, i32, vp, vp, vp, i32, i32, i32, i32, vp, sz, vp]),
        "dfs_gemm_swiglu": (ctypes.c_int, [i32, i32, i32, vp, vp, vp, vp, i32, vp]),
        "spec_cycle_advance": (ctypes.c_int, [i32, i32, vp, vp, vp, vp, vp, vp]),
        "spec_schedule_verify": (ctypes.c_int, [i32, i32, vp, i32, ctypes.POINTER(f32), ctypes.POINTER(f32), vp,
                                                vp]),
        "dfs_packed_matrix_bytes": (sz, [i32, i32]),
        "dfs_draft_trace_layout": (ctypes.c_int, [vp, i32, i32, ctypes.POINTER(sz), ctypes.POINTER(i32)]),
        "dfs_pack_matrix": (ctypes.c_int, [i32, i32, vp, vp, vp]),
        "dfs_profile_begin": (ctypes.c_int, [ctypes.c_char_p, i32]),
        "dfs_profile_end": (ctypes.c_int, [ctypes.POINTER(i32), ctypes.POINTER(ctypes.c_double)]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


LIB = _load()


def status_string(st: int) -> str:
    return LIB.dfs_status_string(st).decode()


def _check(st: int, where: str):
    if st != DFS_OK:
        raise DfsError(st, where)


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _ptr(t, dtype=None, numel=None, name="tensor"):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} must have {numel} elements, got {t.numel()}")
    return ctypes.c_void_p(t.data_ptr())


def torch_dtype(dt: int):
    return torch.bfloat16 if dt == DFS_BF16 else torch.float32


@dataclass
class DrafterConfig:
    n_layers: int
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    mlp_dim: int
    vocab: int
    n_target_layers: int
    block: int
    max_ctx: int
    mask_token_id: int
    rms_eps: float
    rope_theta: float
    dtype: int          # DFS_F32 / DFS_BF16
    window: int = 0     # > 0: sliding attention window over the context (DSpark drafter variant)

    @classmethod
    def of(cls, w) -> "DrafterConfig":
        """From any object with the same attribute names (dtype "f32"/"bf16" accepted)."""
        kw = {f: getattr(w, f) for f in cls.__dataclass_fields__}
        if isinstance(kw["dtype"], str):
            kw["dtype"] = DFS_BF16 if kw["dtype"] == "bf16" else DFS_F32
        return cls(**kw)

    def c(self) -> CDrafterCfg:
        return CDrafterCfg(self.n_layers, self.hidden, self.n_q_heads, self.n_kv_heads, self.head_dim,
                           self.mlp_dim, self.vocab, self.n_target_layers, self.block, self.max_ctx,
                           self.mask_token_id, self.rms_eps, self.rope_theta, self.dtype, self.window)


class DrafterWeights:
    """Device tensors of the drafter keyed like the synthetic generator
    ("embed", "fc", ..., "layers.{l}.wq", ...), plus the C struct pointing at them.
    packed=True (bf16) packs every matrix but the embedding with dfs_pack_matrix
    (new device tensors; the row-major ones are not kept)."""

    PER_LAYER = ("attn_norm", "wq", "wk", "wv", "wo", "mlp_norm", "w_gate", "w_up", "w_down")
    PACKED = ("fc", "lm_head", "wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down")

    def __init__(self, cfg: DrafterConfig, tensors: dict, packed: bool = False):
        self.cfg = cfg
        dt = torch_dtype(cfg.dtype)
        for k, v in tensors.items():
            if v.dtype != dt or not v.is_cuda or not v.is_contiguous():
                raise TypeError(f"weight {k} must be a contiguous {dt} CUDA tensor")
        if packed:
            if cfg.dtype != DFS_BF16:
                raise ValueError("packed weights need bf16")
            tensors = {k: (pack_matrix(v) if k.split(".")[-1] in self.PACKED else v) for k, v in tensors.items()}
        self.t = tensors
        self.packed = bool(packed)
        L = cfg.n_layers
        self._arrays = {}
        for n in self.PER_LAYER:
            arr = (ctypes.c_void_p * L)(*[tensors[f"layers.{l}.{n}"].data_ptr() for l in range(L)])
            self._arrays[n] = arr
        self.c = CDrafterWeights(
            tensors["embed"].data_ptr(), tensors["fc"].data_ptr(), tensors["fc_norm"].data_ptr(),
            tensors["final_norm"].data_ptr(), tensors["lm_head"].data_ptr(),
            *[ctypes.cast(self._arrays[n], _PP) for n in self.PER_LAYER], int(self.packed))


    def layer_prefix(self, n: int) -> "DrafterWeights":
        """The same device tensors as a drafter of only the first n layers."""
        from dataclasses import replace
        if not 1 <= n <= self.cfg.n_layers:
            raise ValueError(f"layer prefix {n} outside 1..{self.cfg.n_layers}")
        out = object.__new__(DrafterWeights)
        out.cfg = replace(self.cfg, n_layers=n)
        out.t = self.t
        out.packed = self.packed
        out._arrays = {k: (ctypes.c_void_p * n)(*list(v)[:n]) for k, v in self._arrays.items()}
        out.c = CDrafterWeights(
            self.t["embed"].data_ptr(), self.t["fc"].data_ptr(), self.t["fc_norm"].data_ptr(),
            self.t["final_norm"].data_ptr(), self.t["lm_head"].data_ptr(),
            *[ctypes.cast(out._arrays[k], _PP) for k in self.PER_LAYER], int(self.packed))
        return out


# ------------------------------------------------------------------ entry points

def dflash_draft_workspace_size(cfg: DrafterConfig, batch: int, n_new_max: int) -> int:
    c = cfg.c()
    return int(LIB.dflash_draft_workspace_size(ctypes.byref(c), batch, n_new_max))


def dflash_draft_step(cfg: DrafterConfig, weights: DrafterWeights, hidden_new, n_new, n_new_max: int,
                      ctx_bound: int, k_cache, v_cache, ctx_len, last_token, base_logits, workspace,
                      stream=None):
    B = ctx_len.numel()
    dt = torch_dtype(cfg.dtype)
    c = cfg.c()
    L, nkv, d, M = cfg.n_layers, cfg.n_kv_heads, cfg.head_dim, cfg.max_ctx
    st = LIB.dflash_draft_step(
        ctypes.byref(c), ctypes.byref(weights.c), B,
        _ptr(hidden_new, dt, B * n_new_max * cfg.n_target_layers * cfg.hidden, "hidden_new") if n_new_max else None,
        _ptr(n_new, torch.int32, B, "n_new"), n_new_max, ctx_bound,
        _ptr(k_cache, dt, L * B * nkv * M * d, "k_cache"), _ptr(v_cache, dt, L * B * nkv * M * d, "v_cache"),
        _ptr(ctx_len, torch.int32, B, "ctx_len"), _ptr(last_token, torch.int32, B, "last_token"),
        _ptr(base_logits, torch.float32, B * (cfg.block - 1) * cfg.vocab, "base_logits"),
        _ptr(workspace, torch.uint8, None, "workspace"), workspace.numel(), _stream(stream))
    _check(st, "dflash_draft_step")


def draft_trace_layout(cfg: DrafterConfig, batch: int, n_new_max: int):
    """Workspace byte offsets and tile-packed flags of the last layer's residual
    stream, MLP input and gated product left by dflash_draft_step (test hook)."""
    c = cfg.c()
    off = (ctypes.c_size_t * 3)()
    pk = (ctypes.c_int32 * 3)()
    _check(LIB.dfs_draft_trace_layout(ctypes.byref(c), batch, n_new_max, off, pk), "dfs_draft_trace_layout")
    return list(off), list(pk)


def markov_bias_sample_workspace_size(batch: int, n_draft: int, vocab: int) -> int:
    return int(LIB.markov_bias_sample_workspace_size(batch, n_draft, vocab))


def markov_bias_sample(logits, U, Wt, last_token, u_draft, temperature: float, draft_tokens,
                       row_stats, workspace, stream=None, wt_packed: bool = False):
    """wt_packed: Wt was packed by pack_matrix (bf16)."""
    B, G, V = logits.shape
    rank = 0 if U is None else U.shape[1]
    uw_dtype = DFS_F32
    if U is not None:
        uw_dtype = DFS_BF16 if U.dtype == torch.bfloat16 else DFS_F32
        _ptr(U, torch_dtype(uw_dtype), V * rank, "U")
        if wt_packed:
            if uw_dtype != DFS_BF16:
                raise ValueError("a packed Wt must be bf16")
            _ptr(Wt, torch.bfloat16, packed_matrix_bytes(V, rank) // 2, "Wt")
            uw_dtype = DFS_BF16_PACKED
        else:
            _ptr(Wt, torch_dtype(uw_dtype), V * rank, "Wt")
    st = LIB.markov_bias_sample(
        B, G, V, rank, _ptr(logits, torch.float32, B * G * V, "logits"),
        _ptr(U, name="U"), _ptr(Wt, name="Wt"), uw_dtype,
        _ptr(last_token, torch.int32, B, "last_token"), _ptr(u_draft, torch.float32, B * G, "u_draft"),
        float(temperature), _ptr(draft_tokens, torch.int32, B * G, "draft_tokens"),
        _ptr(row_stats, torch.float64, B * G * 2, "row_stats") if row_stats is not None else None,
        _ptr(workspace, torch.uint8, None, "workspace"), workspace.numel(), _stream(stream))
    _check(st, "markov_bias_sample")


def rnn_bias_sample_workspace_size(batch: int, n_draft: int, vocab: int, rank: int) -> int:
    return int(LIB.rnn_bias_sample_workspace_size(batch, n_draft, vocab, rank))


def rnn_bias_sample(logits, U, Wt, A, last_token, u_draft, temperature: float, draft_tokens, row_stats,
                    workspace, stream=None, wt_packed: bool = False):
    """RNN sequential head + sampling; U, Wt [V, r] and A [r, r] all bf16 or all fp32.
    wt_packed: Wt was packed by pack_matrix (bf16)."""
    B, G, V = logits.shape
    rank = U.shape[1]
    uw_dtype = DFS_BF16 if U.dtype == torch.bfloat16 else DFS_F32
    dt = torch_dtype(uw_dtype)
    _ptr(U, dt, V * rank, "U")
    _ptr(A, dt, rank * rank, "A")
    if wt_packed:
        if uw_dtype != DFS_BF16:
            raise ValueError("a packed Wt must be bf16")
        _ptr(Wt, torch.bfloat16, packed_matrix_bytes(V, rank) // 2, "Wt")
        uw_dtype = DFS_BF16_PACKED
    else:
        _ptr(Wt, dt, V * rank, "Wt")
    st = LIB.rnn_bias_sample(
        B, G, V, rank, _ptr(logits, torch.float32, B * G * V, "logits"), _ptr(U, name="U"), _ptr(Wt, name="Wt"),
        _ptr(A, name="A"), uw_dtype, _ptr(last_token, torch.int32, B, "last_token"),
        _ptr(u_draft, torch.float32, B * G, "u_draft"), float(temperature),
        _ptr(draft_tokens, torch.int32, B * G, "draft_tokens"),
        _ptr(row_stats, torch.float64, B * G * 2, "row_stats") if row_stats is not None else None,
        _ptr(workspace, torch.uint8, None, "workspace"), workspace.numel(), _stream(stream))
    _check(st, "rnn_bias_sample")


def spec_verify_workspace_size(batch: int, n_draft: int, vocab: int) -> int:
    return int(LIB.spec_verify_workspace_size(batch, n_draft, vocab))


def spec_verify(draft_logits, target_logits, draft_tokens, u_accept, u_final, temperature: float,
                draft_row_stats, out_tokens, n_accepted, workspace, stream=None, n_verify=None):
    """n_verify: optional device int32 [B], drafts verified per row (early stopping)."""
    B, G, V = draft_logits.shape
    st = LIB.spec_verify(
        B, G, V, _ptr(draft_logits, torch.float32, B * G * V, "draft_logits"),
        _ptr(target_logits, torch.float32, B * (G + 1) * V, "target_logits"),
        _ptr(draft_tokens, torch.int32, B * G, "draft_tokens"), _ptr(u_accept, torch.float32, B * G, "u_accept"),
        _ptr(u_final, torch.float32, B, "u_final"), float(temperature),
        _ptr(draft_row_stats, torch.float64, B * G * 2, "draft_row_stats") if draft_row_stats is not None else None,
        _ptr(n_verify, torch.int32, B, "n_verify"),
        _ptr(out_tokens, torch.int32, B * (G + 1), "out_tokens"), _ptr(n_accepted, torch.int32, B, "n_accepted"),
        _ptr(workspace, torch.uint8, None, "workspace"), workspace.numel(), _stream(stream))
    _check(st, "spec_verify")


def spec_verify_static(draft_logits, target_logits, draft_tokens, u_accept, u_final, temperature: float,
                       draft_row_stats, out_tokens, n_accepted, stream=None, n_verify=None):
    """spec_verify on the library's static per-GPU scratch (no workspace, no allocation)."""
    B, G, V = draft_logits.shape
    st = LIB.spec_verify_static(
        B, G, V, _ptr(draft_logits, torch.float32, B * G * V, "draft_logits"),
        _ptr(target_logits, torch.float32, B * (G + 1) * V, "target_logits"),
        _ptr(draft_tokens, torch.int32, B * G, "draft_tokens"), _ptr(u_accept, torch.float32, B * G, "u_accept"),
        _ptr(u_final, torch.float32, B, "u_final"), float(temperature),
        _ptr(draft_row_stats, torch.float64, B * G * 2, "draft_row_stats") if draft_row_stats is not None else None,
        _ptr(n_verify, torch.int32, B, "n_verify"),
        _ptr(out_tokens, torch.int32, B * (G + 1), "out_tokens"), _ptr(n_accepted, torch.int32, B, "n_accepted"),
        _stream(stream))
    _check(st, "spec_verify_static")


def dfs_block_attention_workspace_size(batch, block, nq, nkv, d, ctx_bound, dtype) -> int:
    return int(LIB.dfs_block_attention_workspace_size(batch, block, nq, nkv, d, ctx_bound, dtype))


def dfs_block_attention(q, k_blk, v_blk, k_cache, v_cache, ctx_len, out, max_ctx: int, ctx_bound: int,
                        workspace, stream=None, window: int = 0):
    B, S, nq, d = q.shape
    nkv = k_blk.shape[2]
    dtype = DFS_BF16 if q.dtype == torch.bfloat16 else DFS_F32
    dt = q.dtype
    st = LIB.dfs_block_attention(
        B, S, nq, nkv, d, max_ctx, ctx_bound, dtype, int(window), _ptr(q, dt, name="q"), _ptr(k_blk, dt, name="k_blk"),
        _ptr(v_blk, dt, name="v_blk"), _ptr(k_cache, dt, B * nkv * max_ctx * d, "k_cache"),
        _ptr(v_cache, dt, B * nkv * max_ctx * d, "v_cache"), _ptr(ctx_len, torch.int32, B, "ctx_len"),
        _ptr(out, dt, B * S * nq * d, "out"), _ptr(workspace, torch.uint8, None, "workspace"),
        workspace.numel(), _stream(stream))
    _check(st, "dfs_block_attention")


def dfs_gemm_workspace_size(M, N, K, dtype, splits=0) -> int:
    return int(LIB.dfs_gemm_workspace_size(M, N, K, dtype, splits))


def dfs_gemm(X, W, Y, splits: int, workspace, stream=None, w_packed: bool = False):
    """Y = X . W^T; with w_packed, W is pack_matrix(W') of a [N, K] matrix and N = Y.shape[1]."""
    M, K = X.shape
    N = Y.shape[1] if w_packed else W.shape[0]
    dtype = DFS_BF16 if X.dtype == torch.bfloat16 else DFS_F32
    wn = packed_matrix_bytes(N, K) // 2 if w_packed else N * K
    st = LIB.dfs_gemm(M, N, K, dtype, _ptr(X, X.dtype, name="X"), _ptr(W, X.dtype, wn, "W"),
                      _ptr(Y, torch.float32, M * N, "Y"), splits, int(w_packed),
                      _ptr(workspace, torch.uint8, None, "workspace"), workspace.numel(), _stream(stream))
    _check(st, "dfs_gemm")


def dfs_gemm_skip(X, W, Y, splits: int, skip_m: int, skip_n: int, workspace, stream=None, w_packed: bool = False):
    """dfs_gemm whose output tiles inside rows [0, skip_m) x columns [0, skip_n) may be
    left uncomputed (Y there unspecified); splits >= 1 when a corner is skipped."""
    M, K = X.shape
    N = Y.shape[1] if w_packed else W.shape[0]
    dtype = DFS_BF16 if X.dtype == torch.bfloat16 else DFS_F32
    wn = packed_matrix_bytes(N, K) // 2 if w_packed else N * K
    st = LIB.dfs_gemm_skip(M, N, K, dtype, _ptr(X, X.dtype, name="X"), _ptr(W, X.dtype, wn, "W"),
                           _ptr(Y, torch.float32, M * N, "Y"), splits, int(w_packed), skip_m, skip_n,
                           _ptr(workspace, torch.uint8, None, "workspace"), workspace.numel(), _stream(stream))
    _check(st, "dfs_gemm_skip")


def dfs_gemm_swiglu(X, Wg, Wu, H, stream=None, w_packed: bool = False):
    """H = bf16(silu(X . Wg^T) * (X . Wu^T)); X [M, K], H [M, F] bf16; Wg, Wu [F, K]
    bf16, or with w_packed their pack_matrix copies."""
    M, K = X.shape
    F = H.shape[1]
    if X.dtype != torch.bfloat16 or H.dtype != torch.bfloat16 or H.shape[0] != M:
        raise TypeError("dfs_gemm_swiglu takes bf16 X [M, K] and H [M, F]")
    wn = packed_matrix_bytes(F, K) // 2 if w_packed else F * K
    st = LIB.dfs_gemm_swiglu(M, F, K, _ptr(X, torch.bfloat16, M * K, "X"), _ptr(Wg, torch.bfloat16, wn, "Wg"),
                             _ptr(Wu, torch.bfloat16, wn, "Wu"), _ptr(H, torch.bfloat16, M * F, "H"),
                             int(w_packed), _stream(stream))
    _check(st, "dfs_gemm_swiglu")


def spec_cycle_advance(n_accepted, out_tokens, n_new, last_token, tau_sum=None, stream=None):
    """Next cycle's n_new = n_accepted + 1 and last_token = out_tokens[b, n_accepted]
    (device, no sync); tau_sum (int64, optional) accumulates n_accepted + 1."""
    B = n_accepted.numel()
    G = out_tokens.shape[1] - 1
    st = LIB.spec_cycle_advance(B, G, _ptr(n_accepted, torch.int32, B, "n_accepted"),
                                _ptr(out_tokens, torch.int32, B * (G + 1), "out_tokens"),
                                _ptr(n_new, torch.int32, B, "n_new"), _ptr(last_token, torch.int32, B, "last_token"),
                                _ptr(tau_sum, torch.int64, B, "tau_sum"), _stream(stream))
    _check(st, "spec_cycle_advance")


def spec_schedule_verify(survival, curve_rows, curve_sps, n_verify, stream=None):
    """Verify lengths per request (device int32 [B] out) from survival scores
    [B, gamma] (device fp32) and a host throughput curve (rows, passes/s)."""
    B, G = survival.shape
    xs = [float(x) for x in curve_rows]
    ys = [float(y) for y in curve_sps]
    if len(xs) != len(ys):
        raise ValueError("curve_rows and curve_sps differ in length")
    FA = ctypes.c_float * len(xs)
    st = LIB.spec_schedule_verify(B, G, _ptr(survival, torch.float32, B * G, "survival"), len(xs), FA(*xs), FA(*ys),
                                  _ptr(n_verify, torch.int32, B, "n_verify"), _stream(stream))
    _check(st, "spec_schedule_verify")


def packed_matrix_bytes(rows: int, cols: int) -> int:
    return int(LIB.dfs_packed_matrix_bytes(rows, cols))


def pack_matrix(w, stream=None):
    """Tile-packed copy of a row-major bf16 [rows, cols] device matrix (flat bf16 tensor)."""
    if w.dim() != 2 or w.dtype != torch.bfloat16:
        raise TypeError("pack_matrix takes a 2-D bf16 tensor")
    rows, cols = w.shape
    n = packed_matrix_bytes(rows, cols)
    if n == 0:
        raise ValueError(f"cannot pack a [{rows}, {cols}] matrix (cols must be a multiple of 64)")
    out = torch.empty(n // 2, dtype=torch.bfloat16, device=w.device)
    _check(LIB.dfs_pack_matrix(rows, cols, _ptr(w, torch.bfloat16, rows * cols, "w"),
                               _ptr(out, torch.bfloat16, n // 2, "out"), _stream(stream)), "dfs_pack_matrix")
    return out


def dfs_profile_begin(group: str, max_launches: int):
    _check(LIB.dfs_profile_begin(group.encode(), max_launches), "dfs_profile_begin")


def dfs_profile_end():
    n = ctypes.c_int32(0)
    ms = ctypes.c_double(0.0)
    _check(LIB.dfs_profile_end(ctypes.byref(n), ctypes.byref(ms)), "dfs_profile_end")
    return int(n.value), float(ms.value)


# ------------------------------------------------------------------ layout helpers (host side)

def cache_from_logical(k_logical, v_logical):
    """[L, B, max_ctx, nkv, d] logical caches -> the library's layouts
    K [L, B, nkv, max_ctx, d] and V [L, B, nkv, d, max_ctx] (values transposed)."""
    k = k_logical.permute(0, 1, 3, 2, 4).contiguous()
    v = v_logical.permute(0, 1, 3, 4, 2).contiguous()
    return k, v


def cache_to_logical(k, v):
    return k.permute(0, 1, 3, 2, 4).contiguous(), v.permute(0, 1, 4, 2, 3).contiguous()
