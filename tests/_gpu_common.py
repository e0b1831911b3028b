"""Helpers of the GPU parity tests: device upload/download and flag-aware
comparison of draws.  Imported only by tests marked ``gpu``."""
import sys

import numpy as np
import torch

DEV = "cuda"
FLAG = 1e-6          # draws whose oracle margin is below this may legitimately differ


def flag_budget(V, n_draws):
    """Upper bound on flagged draws: a threshold u*S lands within FLAG*S of one of
    the (up to V) interval ends with probability sum_k min(2*FLAG, p_k) <= 2*FLAG*V."""
    return 3 + int(3 * 2 * FLAG * V * n_draws)


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def up(arr, kind):
    a = np.ascontiguousarray(arr)
    if kind == "bf16":
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(DEV)
    if kind == "f32":
        return torch.from_numpy(a.astype(np.float32, copy=False)).to(DEV)
    if kind == "i32":
        return torch.from_numpy(a.astype(np.int32, copy=False)).to(DEV)
    if kind == "f64":
        return torch.from_numpy(a.astype(np.float64, copy=False)).to(DEV)
    raise ValueError(kind)


def down(t):
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def as_f64(arr, kind):
    if kind == "bf16":
        b = np.asarray(arr, np.uint16).astype(np.uint32) << 16
        return b.view(np.float32).astype(np.float64)
    return np.asarray(arr, np.float64)


def workspace(nbytes):
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=DEV)


def compare_sequential_draws(gpu, ora, margins, what):
    """Rows of sequential draws: equal until the first flagged draw of a row
    (that draw and everything after it in the row are excluded)."""
    gpu = np.asarray(gpu)
    ora = np.asarray(ora)
    n_cmp = n_flag = 0
    for b in range(ora.shape[0]):
        for i in range(ora.shape[1]):
            if margins[b, i] < FLAG:
                n_flag += 1
                break
            assert gpu[b, i] == ora[b, i], f"{what}: row {b} position {i}: gpu {gpu[b, i]} oracle {ora[b, i]}"
            n_cmp += 1
    return n_cmp, n_flag


def upload_weights(w, np_weights, packed=False):
    from block_speculative_decoding_amd import dfspec as D
    cfg = D.DrafterConfig.of(w)
    t = {k: up(v, w.dtype) for k, v in np_weights.items()}
    return cfg, D.DrafterWeights(cfg, t, packed=packed)


def unpack_activations(buf, rows, cols):
    """Row-major [rows, cols] from a tile-packed activation buffer (rows in groups
    of 16, each group's columns in 64-wide 2 KB tiles in matrix-core operand
    order; the layout the library's header states for its trace hook)."""
    r = np.arange(rows)[:, None]
    c = np.arange(cols)[None, :]
    idx = (((r >> 4) * (cols >> 6) + (c >> 6)) * 1024 + ((c >> 5) & 1) * 512 + ((r & 15) + 16 * ((c >> 3) & 3)) * 8
           + (c & 7))
    return np.asarray(buf).reshape(-1)[idx]


def draft_trace(D, cfg, batch, n_new_max, ws, dtype):
    """The last layer's residual stream [B*S, H] (fp32), MLP input [B*S, H] and
    gated product [B*S, F] (storage dtype) that dflash_draft_step left in ws."""
    off, packed = D.draft_trace_layout(cfg, batch, n_new_max)
    M, H, F = batch * cfg.block, cfg.hidden, cfg.mlp_dim
    es = 2 if dtype == "bf16" else 4
    host = down(ws).view(np.uint8)

    def grab(k, cols, kind):
        rows = (M + 15) // 16 * 16 if packed[k] else M
        raw = host[off[k]:off[k] + rows * cols * (4 if kind == "f32" else es)]
        arr = raw.view(np.float32 if kind == "f32" or es == 4 else np.uint16)
        if packed[k]:
            return unpack_activations(arr, M, cols)
        return arr.reshape(M, cols)

    return grab(0, H, "f32"), grab(1, H, dtype), grab(2, F, dtype)
