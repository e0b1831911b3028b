"""GPU parity of the kernel-level pieces through the C ABI, at sizes the oracle
finishes in seconds that span several tiles and ragged tails."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

import oracle
from oracle import drafter as od
from synth import rng

from _gpu_common import (DEV, FLAG, as_f64, compare_sequential_draws, down, flag_budget, say, up,
                         workspace)


@pytest.fixture(scope="module")
def D():
    import torch
    assert torch.cuda.is_available()
    from block_speculative_decoding_amd import dfspec
    return dfspec


# ---------------------------------------------------------------- GEMM (matrix cores)

# M > 256 with enough columns is planned onto the LDS-ring tile kernel (256 x 256
# tiles): (640, 8200, 1024) with its automatic 2-way K split and a forced 3-way
# one, (600, 16400, 512) unsplit; ragged in both M and N.  M <= 16 with K <= 512
# ((5, 3001, 512), (1, 64, 64)) runs the independent-wave small-M kernel, ragged N; K = 256 with
# M <= 128 ((16, 1000, 256), (32, 1000, 256), (120, 300, 256)) the persistent short-K kernel.
# (100, 6000, 1024 / 2048) get 96-column streaming tiles (3 consumer waves, 64 and 128 rows).
# M in (128, 160] runs one 160-row M tile: (150, 4096, 4096) with 128 columns and 8 splits
# (ragged M), forced to 3 splits with 96 columns, and (160, 6000, 2048) with 96 columns.
@pytest.mark.parametrize("M,N,K,splits", [(1, 64, 64, 0), (120, 300, 256, 0), (120, 300, 256, 3),
                                          (256, 1000, 512, 7), (64, 128, 4096, 0), (130, 4096, 1024, 0),
                                          (640, 8200, 1024, 0), (640, 8200, 1024, 3), (600, 16400, 512, 0),
                                          (32, 1000, 256, 0), (5, 3001, 512, 0), (16, 1000, 256, 0), (17, 129, 192, 0),
                                          (100, 6000, 1024, 0), (100, 6000, 2048, 0),
                                          (150, 4096, 4096, 0), (150, 4096, 4096, 3), (160, 6000, 2048, 0)])
def test_gemm_bf16_matches_fp64_product(D, M, N, K, splits):
    say(f"gemm bf16 M={M} N={N} K={K} splits={splits}")
    X = rng.normal(1, "gx", (M, K), 1.0, dtype="bf16")
    W = rng.normal(1, "gw", (N, K), 0.05, dtype="bf16")
    Y = __import__("torch").empty((M, N), dtype=__import__("torch").float32, device=DEV)
    ws = workspace(D.dfs_gemm_workspace_size(M, N, K, D.DFS_BF16, splits))
    D.dfs_gemm(up(X, "bf16").view(M, K), up(W, "bf16").view(N, K), Y, splits, ws)
    want = as_f64(X, "bf16") @ as_f64(W, "bf16").T
    got = down(Y).astype(np.float64)
    np.testing.assert_allclose(got, want, atol=2e-5 * np.sqrt(K), rtol=1e-5)


# The skipped corner of the drafter's Q|K|V product (no queries for the context rows):
# (300, 1000, 512) unsplit on 128 x 128 streaming tiles (one M tile and four N tiles
# skipped, the corner ending inside the next tiles), (700, 3000, 1024) with 2 splits,
# (2048, 6144, 4096) with 2 splits on the LDS-ring tile kernel (the C4 shape, checked on
# sampled rows).  Every element outside the corner matches the fp64 product; in the
# unsplit case the skipped tiles keep the NaN the output was filled with.
@pytest.mark.parametrize("M,N,K,splits,skip_m,skip_n,rows", [
    (300, 1000, 512, 1, 150, 512, None), (700, 3000, 1024, 2, 300, 2000, None),
    (2048, 6144, 4096, 2, 1024, 4096, (0, 255, 256, 1023, 1024, 1500, 2047))])
def test_gemm_skipped_corner(D, M, N, K, splits, skip_m, skip_n, rows):
    import torch
    say(f"gemm skip M={M} N={N} K={K} splits={splits} corner {skip_m} x {skip_n}")
    X = rng.normal(11, "kx", (M, K), 1.0, dtype="bf16")
    W = rng.normal(11, "kw", (N, K), 0.05, dtype="bf16")
    Wd = up(W, "bf16").view(N, K)
    Y = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
    ws = workspace(D.dfs_gemm_workspace_size(M, N, K, D.DFS_BF16, splits))
    D.dfs_gemm_skip(up(X, "bf16").view(M, K), D.pack_matrix(Wd), Y, splits, skip_m, skip_n, ws, w_packed=True)
    got = down(Y).astype(np.float64)
    r = np.arange(M) if rows is None else np.array(rows)
    want = as_f64(X, "bf16")[r] @ as_f64(W, "bf16").T
    keep = ~((r[:, None] < skip_m) & (np.arange(N)[None, :] < skip_n))
    np.testing.assert_allclose(got[r][keep], want[keep], atol=2e-5 * np.sqrt(K), rtol=1e-5)
    if M == 300:
        # the tiles wholly inside the corner (128 x 128 streaming tiles here) are never written
        assert np.isnan(got[:skip_m // 128 * 128, :skip_n // 128 * 128]).all()


def _packed_reference(W):
    """The tile-packed layout written out from its definition: tiles of 16 rows x 64
    columns, row-tile major; inside a tile [half h][lane l][8 values] = row
    16t + l % 16, columns 64c + 32h + 8(l // 16) .. +7; rows past N zero."""
    N, K = W.shape
    nt = -(-N // 16)
    Wp = np.zeros((nt * 16, K), W.dtype)
    Wp[:N] = W
    out = np.empty((nt, K // 64, 2, 64, 8), W.dtype)
    for l in range(64):
        for h in range(2):
            cols = np.arange(8) + 32 * h + 8 * (l // 16)
            # [nt, K//64, 8]: row 16t + l%16, column 64c + cols
            out[:, :, h, l, :] = Wp[l % 16::16].reshape(nt, K // 64, 64)[:, :, cols]
    return out.reshape(-1)


@pytest.mark.parametrize("N,K", [(16, 64), (100, 192), (1000, 512)])
def test_pack_matrix_layout(D, N, K):
    W = rng.integers(9, "packw", (N, K), 0, 65535).astype(np.uint16)     # arbitrary bit patterns
    got = down(D.pack_matrix(up(W, "bf16").view(N, K)))
    np.testing.assert_array_equal(got.view(np.uint16), _packed_reference(W))


@pytest.mark.parametrize("M,N,K,splits", [(1, 64, 64, 0), (120, 300, 256, 3), (128, 1000, 512, 0),
                                          (256, 1000, 512, 7), (300, 200, 256, 0), (130, 4096, 1024, 0),
                                          (640, 8200, 1024, 0), (16, 1000, 256, 0), (3, 100, 64, 0), (100, 6000, 2048, 0),
                                          (150, 4096, 4096, 0), (160, 6000, 2048, 0)])
def test_gemm_packed_weights_bit_identical(D, M, N, K, splits):
    # same operands in the same order: the packed and row-major kernels agree bit for bit
    import torch
    say(f"gemm packed M={M} N={N} K={K} splits={splits}")
    X = rng.normal(1, "gx", (M, K), 1.0, dtype="bf16")
    W = rng.normal(1, "gw", (N, K), 0.05, dtype="bf16")
    Wd = up(W, "bf16").view(N, K)
    Y0 = torch.empty((M, N), dtype=torch.float32, device=DEV)
    Y1 = torch.empty((M, N), dtype=torch.float32, device=DEV)
    ws = workspace(D.dfs_gemm_workspace_size(M, N, K, D.DFS_BF16, splits))
    D.dfs_gemm(up(X, "bf16").view(M, K), Wd, Y0, splits, ws)
    D.dfs_gemm(up(X, "bf16").view(M, K), D.pack_matrix(Wd), Y1, splits, ws, w_packed=True)
    assert np.array_equal(down(Y0).view(np.uint32), down(Y1).view(np.uint32))
    want = as_f64(X, "bf16") @ as_f64(W, "bf16").T
    np.testing.assert_allclose(down(Y1).astype(np.float64), want, atol=2e-5 * np.sqrt(K), rtol=1e-5)


# (48, 1000, 256) and (320, 1536, 512) run the weight-streaming kernel with paired
# gate/up tiles; (150, 6144, 1024) and (150, 16384, 1024) its 160-row tiles of 48 and
# 64 features (ragged M); (700, 8200, 1024) is planned onto the LDS-ring tile kernel
# (ragged M, and F not a multiple of 16).
@pytest.mark.parametrize("M,F,K", [(48, 1000, 256), (320, 1536, 512), (150, 6144, 1024), (150, 16384, 1024),
                                   (700, 8200, 1024)])
def test_gemm_swiglu_matches_fp64(D, M, F, K):
    import torch
    say(f"gemm swiglu M={M} F={F} K={K}")
    X = rng.normal(3, "sx", (M, K), 1.0, dtype="bf16")
    Wg = rng.normal(3, "sg", (F, K), 0.05, dtype="bf16")
    Wu = rng.normal(3, "su", (F, K), 0.05, dtype="bf16")
    Xd, Wgd, Wud = up(X, "bf16").view(M, K), up(Wg, "bf16").view(F, K), up(Wu, "bf16").view(F, K)
    H0 = torch.full((M, F), float("nan"), dtype=torch.bfloat16, device=DEV)
    H1 = torch.full((M, F), float("nan"), dtype=torch.bfloat16, device=DEV)
    D.dfs_gemm_swiglu(Xd, Wgd, Wud, H0)
    D.dfs_gemm_swiglu(Xd, D.pack_matrix(Wgd), D.pack_matrix(Wud), H1, w_packed=True)
    torch.cuda.synchronize()
    # same sums in the same order: packed and row-major agree bit for bit
    assert torch.equal(H0.view(torch.int16), H1.view(torch.int16))
    x = as_f64(X, "bf16")
    g = x @ as_f64(Wg, "bf16").T
    u = x @ as_f64(Wu, "bf16").T
    want = g / (1.0 + np.exp(-g)) * u
    got = H0.float().cpu().numpy().astype(np.float64)
    # one bf16 rounding (<= 2^-9 relative) of a value whose fp32 sums carry ~1e-6 relative error
    np.testing.assert_allclose(got, want, rtol=2.0 ** -8, atol=3e-4)


def test_gemm_f32(D):
    import torch
    M, N, K = 5, 70, 48
    X = rng.normal(2, "gx32", (M, K), 1.0)
    W = rng.normal(2, "gw32", (N, K), 0.1)
    Y = torch.empty((M, N), dtype=torch.float32, device=DEV)
    D.dfs_gemm(up(X, "f32"), up(W, "f32"), Y, 0, workspace(D.dfs_gemm_workspace_size(M, N, K, 0, 0)))
    np.testing.assert_allclose(down(Y), X.astype(np.float64) @ W.astype(np.float64).T, atol=1e-5)


# ---------------------------------------------------------------- block attention

@pytest.mark.parametrize("dtype,B,S,nq,nkv,d,max_ctx,ctx,window", [
    ("bf16", 3, 16, 8, 2, 128, 640, [600, 37, 0], 0),
    ("bf16", 2, 8, 8, 2, 128, 2112, [2100, 1031], 0),
    ("bf16", 2, 4, 4, 4, 128, 128, [128, 65], 0),
    ("bf16", 2, 32, 8, 2, 128, 640, [600, 37], 0),      # R = 128 query rows per kv head: two 64-row groups
    ("bf16", 1, 24, 8, 2, 128, 256, [200], 0),          # R = 96: a partial second group
    ("f32", 2, 4, 4, 4, 64, 128, [124, 50], 0),
    ("f32", 1, 5, 6, 2, 32, 320, [300], 0),
    # sliding window: first key not step-aligned (600 - 128 = 472), shorter and empty contexts
    ("bf16", 3, 16, 8, 2, 128, 640, [600, 37, 0], 128),
    ("bf16", 2, 8, 8, 2, 128, 2112, [2100, 1031], 100),
    ("bf16", 2, 32, 8, 2, 128, 640, [600, 37], 64),
    ("f32", 2, 4, 4, 4, 64, 128, [124, 50], 30),
    # the full workload shapes: 8 rows x 4096 context keys (4 key chunks per row and
    # kv head, merged), and 4 rows x 32768 keys (long-context plan: two resident units per CU)
    ("bf16", 8, 16, 32, 8, 128, 4160, [4096] * 8, 0),
    ("bf16", 4, 16, 32, 8, 128, 32832, [32768, 32768, 30001, 32768], 0),
])
def test_block_attention_matches_oracle(D, dtype, B, S, nq, nkv, d, max_ctx, ctx, window):
    import torch
    say(f"attention {dtype} B={B} S={S} nq={nq} nkv={nkv} ctx={ctx} window={window}")
    ctx = np.array(ctx, np.int32)
    q = rng.normal(3, "aq", (B, S, nq, d), 1.0, dtype=dtype)
    kb = rng.normal(3, "akb", (B, S, nkv, d), 1.0, dtype=dtype)
    vb = rng.normal(3, "avb", (B, S, nkv, d), 1.0, dtype=dtype)
    kc = rng.normal(3, "akc", (B, nkv, max_ctx, d), 1.0, dtype=dtype)
    vc = rng.normal(3, "avc", (B, nkv, d, max_ctx), 1.0, dtype=dtype)
    nan = np.uint16(0x7FC0) if dtype == "bf16" else np.float32(np.nan)
    for b in range(B):                                        # slots >= ctx_len are never read
        kc[b, :, ctx[b]:] = nan
        vc[b, :, :, ctx[b]:] = nan
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    out = torch.empty((B, S, nq, d), dtype=tdt, device=DEV)
    ws = workspace(D.dfs_block_attention_workspace_size(B, S, nq, nkv, d, int(ctx.max()),
                                                        1 if dtype == "bf16" else 0))
    D.dfs_block_attention(up(q, dtype), up(kb, dtype), up(vb, dtype), up(kc, dtype), up(vc, dtype),
                          up(ctx, "i32"), out, max_ctx, int(max(ctx.max(), 1)), ws, window=window)
    got = as_f64(down(out), dtype)
    tol = 2e-2 if dtype == "bf16" else 1e-4
    for b in range(B):
        c = ctx[b]
        lo = max(0, c - window) if window > 0 else 0
        want = od.block_attention(as_f64(q[b], dtype), as_f64(kc[b, :, lo:c], dtype).transpose(1, 0, 2),
                                  as_f64(vc[b, :, :, lo:c], dtype).transpose(2, 0, 1),
                                  as_f64(kb[b], dtype), as_f64(vb[b], dtype))
        np.testing.assert_allclose(got[b], want, atol=tol, rtol=0)


@pytest.mark.parametrize("B,S,nq,nkv,ctx", [(3, 16, 8, 2, [600, 37, 300]),   # 64 rows per kv head
                                            (2, 5, 4, 4, [700, 290])])          # 5 rows: a partial row group
def test_attention_combine_paths_agree(D, B, S, nq, nkv, ctx):
    """The key-chunk merge has a vectorised kernel (8-byte aligned output) and a
    one-thread-per-dim kernel (any alignment; here the output sits 2 bytes off);
    both do the same fp32 arithmetic in the same order, so the outputs agree
    bit for bit.  Contexts of several hundred keys split into key chunks."""
    import torch
    d, max_ctx = 128, 704
    say(f"attention combine paths B={B} S={S} nq={nq} nkv={nkv} ctx={ctx}")
    ctx = np.array(ctx, np.int32)
    args = [up(rng.normal(4, "cq", (B, S, nq, d), 1.0, dtype="bf16"), "bf16"),
            up(rng.normal(4, "ckb", (B, S, nkv, d), 1.0, dtype="bf16"), "bf16"),
            up(rng.normal(4, "cvb", (B, S, nkv, d), 1.0, dtype="bf16"), "bf16"),
            up(rng.normal(4, "ckc", (B, nkv, max_ctx, d), 1.0, dtype="bf16"), "bf16"),
            up(rng.normal(4, "cvc", (B, nkv, d, max_ctx), 1.0, dtype="bf16"), "bf16"),
            up(ctx, "i32")]
    n = B * S * nq * d
    aligned = torch.empty(n, dtype=torch.bfloat16, device=DEV)
    shifted = torch.empty(n + 1, dtype=torch.bfloat16, device=DEV)[1:]
    assert aligned.data_ptr() % 8 == 0 and shifted.data_ptr() % 8 == 2
    ws = workspace(D.dfs_block_attention_workspace_size(B, S, nq, nkv, d, int(ctx.max()), 1))
    for out in (aligned, shifted):
        D.dfs_block_attention(*args, out.view(B, S, nq, d), max_ctx, int(ctx.max()), ws)
    torch.cuda.synchronize()
    assert torch.equal(aligned.view(torch.int16), shifted.view(torch.int16))


# ---------------------------------------------------------------- sampling (no head)

# the largest vocabulary the library takes (1024 chunks of 4096 tokens; the pick merges
# exactly that many per row), also ragged (V % 4 != 0: scalar loads, a partial last chunk)
MAX_V = 1024 * 4096


@pytest.mark.parametrize("V,T", [(1000, 1.0), (10000, 0.7), (10000, 0.0), (8, 1.0),
                                 (MAX_V, 1.0), (MAX_V - 3, 0.8), (MAX_V, 0.0)])
def test_parallel_sampling_matches_oracle(D, V, T):
    import torch
    B, G = (6, 5) if V < MAX_V - 3 else (2, 2)
    say(f"sampling V={V} T={T}")
    logits = rng.normal(4, f"sl{V}", (B, G, V), 3.0)
    u = rng.uniform01(4, f"su{V}", (B, G))
    lt = up(logits, "f32")
    tok = torch.empty((B, G), dtype=torch.int32, device=DEV)
    rs = torch.empty((B, G, 2), dtype=torch.float64, device=DEV)
    ws = workspace(D.markov_bias_sample_workspace_size(B, G, V))
    D.markov_bias_sample(lt, None, None, up(np.zeros(B, np.int32), "i32"), up(u, "f32"), T, tok, rs, ws)
    got = down(tok)
    rows = down(rs)
    flagged = 0
    for b in range(B):
        for i in range(G):
            k, m = oracle.sample_row(logits[b, i], u[b, i], T)
            if m < FLAG:
                flagged += 1
                continue
            assert got[b, i] == k, (b, i, got[b, i], k)
            if T > 0:
                x = logits[b, i].astype(np.float64)
                np.testing.assert_allclose(rows[b, i, 0], x.max())
                np.testing.assert_allclose(rows[b, i, 1], np.exp((x - x.max()) / T).sum(), rtol=1e-6)
    assert flagged <= flag_budget(V, B * G)
    np.testing.assert_array_equal(down(lt), logits)          # no head: logits untouched


# ---------------------------------------------------------------- Markov head

# rank 256 with up to 128 rows runs the fused product + per-64-token statistics kernel
# (32-row chunks) and the draw from those statistics (20 rows, V = 9000: a partial last
# sub-chunk; T = 0.7 and greedy; 33 and 100 rows: a ragged last row chunk; V = 68 and 4:
# two sub-chunks, the second of 4 tokens, and a single partial one); 129 rows the
# product, then the separate statistics pass
@pytest.mark.parametrize("dtype,B,G,V,r,T", [("f32", 2, 3, 1000, 16, 1.0), ("bf16", 4, 15, 5000, 64, 1.0),
                                             ("bf16", 33, 7, 9000, 256, 1.0), ("bf16", 20, 5, 9000, 256, 1.0),
                                             ("bf16", 20, 5, 9000, 256, 0.7), ("bf16", 20, 5, 9000, 256, 0.0),
                                             ("bf16", 3, 4, 9004, 256, 1.0), ("bf16", 1, 4, 9000, 256, 1.0),
                                             ("bf16", 100, 3, 9000, 256, 0.7), ("bf16", 5, 3, 68, 256, 1.0),
                                             ("bf16", 2, 2, 4, 256, 0.0),
                                             ("bf16", 129, 2, 5000, 256, 1.0)])
def test_markov_head_matches_oracle(D, dtype, B, G, V, r, T):
    import torch
    say(f"markov {dtype} B={B} G={G} V={V} r={r} T={T}")
    base = rng.normal(5, f"mb{V}", (B, G, V), 1.5)
    U = rng.normal(5, f"mU{V}", (V, r), r ** -0.25, dtype=dtype)
    Wt = rng.normal(5, f"mW{V}", (V, r), r ** -0.25, dtype=dtype)
    last = rng.integers(5, f"ml{V}", (B,), 0, V - 1)
    u = rng.uniform01(5, f"mu{V}", (B, G))
    lt = up(base, "f32")
    tok = torch.empty((B, G), dtype=torch.int32, device=DEV)
    rs = torch.empty((B, G, 2), dtype=torch.float64, device=DEV)
    ws = workspace(D.markov_bias_sample_workspace_size(B, G, V))
    D.markov_bias_sample(lt, up(U, dtype), up(Wt, dtype), up(last, "i32"), up(u, "f32"), T, tok, rs, ws)
    final, otok, margins = oracle.markov_sample(base, U, Wt, dtype, last, u, T)
    got_tok = down(tok)
    got_final = down(lt)
    got_rs = down(rs)
    n_cmp, n_flag = compare_sequential_draws(got_tok, otok, margins, "markov tokens")
    # final logits and row statistics where both sides used the same previous token
    for b in range(B):
        for i in range(G):
            if i > 0 and got_tok[b, i - 1] != otok[b, i - 1]:
                break
            np.testing.assert_allclose(got_final[b, i], final[b, i], atol=1e-4, rtol=0)
            x = final[b, i].astype(np.float64)
            np.testing.assert_allclose(got_rs[b, i, 0], x.max(), atol=1e-4)
            if T > 0:
                np.testing.assert_allclose(got_rs[b, i, 1], np.exp((x - x.max()) / T).sum(), rtol=1e-4)
    assert n_flag <= flag_budget(V, B * G)
    say(f"  compared {n_cmp} draws, {n_flag} flagged")


def test_markov_head_packed_wt_bit_identical(D):
    import torch
    B, G, V, r = 5, 4, 3000, 64
    base = rng.normal(6, "pmb", (B, G, V), 1.5)
    U = rng.normal(6, "pmU", (V, r), r ** -0.25, dtype="bf16")
    Wt = rng.normal(6, "pmW", (V, r), r ** -0.25, dtype="bf16")
    last = up(rng.integers(6, "pml", (B,), 0, V - 1), "i32")
    u = up(rng.uniform01(6, "pmu", (B, G)), "f32")
    outs = []
    for packed in (False, True):
        lt = up(base, "f32")
        tok = torch.empty((B, G), dtype=torch.int32, device=DEV)
        wt = up(Wt, "bf16").view(V, r)
        D.markov_bias_sample(lt, up(U, "bf16"), D.pack_matrix(wt) if packed else wt, last, u, 1.0, tok, None,
                             workspace(D.markov_bias_sample_workspace_size(B, G, V)), wt_packed=packed)
        outs.append((down(lt), down(tok)))
    assert np.array_equal(outs[0][0].view(np.uint32), outs[1][0].view(np.uint32))
    assert np.array_equal(outs[0][1], outs[1][1])


# ---------------------------------------------------------------- RNN head

def _rnn_inputs(seed, dtype, B, G, V, r):
    base = rng.normal(seed, f"rb{V}", (B, G, V), 1.5)
    U = rng.normal(seed, f"rU{V}", (V, r), 0.6, dtype=dtype)
    Wt = rng.normal(seed, f"rW{V}", (V, r), r ** -0.25, dtype=dtype)
    A = rng.normal(seed, f"rA{r}", (r, r), 0.5 / np.sqrt(r), dtype=dtype)
    last = rng.integers(seed, f"rl{V}", (B,), 0, V - 1)
    u = rng.uniform01(seed, f"ru{V}", (B, G))
    return base, U, Wt, A, last, u


# rank 256 runs W h on the persistent short-K kernel up to 32 rows (B = 20 here, and the last case:
# the DSpark 5-token block at the full vocabulary with packed W), on the streaming kernel above
@pytest.mark.parametrize("dtype,B,G,V,r,packed", [("f32", 2, 3, 1000, 16, False), ("bf16", 4, 15, 5000, 64, False),
                                                  ("bf16", 33, 7, 9000, 256, False), ("bf16", 20, 5, 9000, 256, False),
                                                  ("bf16", 32, 4, 129280, 256, True)])
def test_rnn_head_matches_oracle(D, dtype, B, G, V, r, packed):
    import torch
    say(f"rnn {dtype} B={B} G={G} V={V} r={r} packed={packed}")
    base, U, Wt, A, last, u = _rnn_inputs(7, dtype, B, G, V, r)
    lt = up(base, "f32")
    tok = torch.empty((B, G), dtype=torch.int32, device=DEV)
    rs = torch.empty((B, G, 2), dtype=torch.float64, device=DEV)
    ws = workspace(D.rnn_bias_sample_workspace_size(B, G, V, r))
    wt = up(Wt, dtype)
    if packed:
        wt = D.pack_matrix(wt.view(V, r))
    D.rnn_bias_sample(lt, up(U, dtype), wt, up(A, dtype), up(last, "i32"), up(u, "f32"), 1.0, tok, rs, ws,
                      wt_packed=packed)
    final, otok, margins, _ = oracle.rnn_sample(base, U, Wt, A, dtype, last, u, 1.0)
    got_tok = down(tok)
    got_final = down(lt)
    n_cmp, n_flag = compare_sequential_draws(got_tok, otok, margins, "rnn tokens")
    # final logits (and row statistics) where both sides used the same prefix
    got_rs = down(rs)
    for b in range(B):
        for i in range(G):
            if i > 0 and got_tok[b, i - 1] != otok[b, i - 1]:
                break
            np.testing.assert_allclose(got_final[b, i], final[b, i], atol=1e-4, rtol=0)
            x = final[b, i].astype(np.float64)
            np.testing.assert_allclose(got_rs[b, i, 0], x.max(), atol=1e-4)
            np.testing.assert_allclose(got_rs[b, i, 1], np.exp(x - x.max()).sum(), rtol=1e-4)
    assert n_flag <= flag_budget(V, B * G)
    say(f"  compared {n_cmp} draws, {n_flag} flagged")


def test_rnn_head_repeat_calls_identical_and_zero_recurrence_is_markov_on_tanh_u(D):
    # the state lives in the workspace only for one call: a second call on the same
    # workspace gives bit-identical results; with A = 0 the head equals the Markov
    # head whose input factor is tanh(U) (fp32 factors, same kernels for W h)
    import torch
    B, G, V, r = 6, 5, 3000, 32
    base, U, Wt, A, last, u = _rnn_inputs(8, "f32", B, G, V, r)
    ws = workspace(D.rnn_bias_sample_workspace_size(B, G, V, r))
    outs = []
    for _ in range(2):
        lt = up(base, "f32")
        tok = torch.empty((B, G), dtype=torch.int32, device=DEV)
        D.rnn_bias_sample(lt, up(U, "f32"), up(Wt, "f32"), up(A, "f32"), up(last, "i32"), up(u, "f32"), 1.0, tok,
                          None, ws)
        outs.append((down(lt), down(tok)))
    assert np.array_equal(outs[0][0].view(np.uint32), outs[1][0].view(np.uint32))
    assert np.array_equal(outs[0][1], outs[1][1])
    lt = up(base, "f32")
    tok = torch.empty((B, G), dtype=torch.int32, device=DEV)
    D.rnn_bias_sample(lt, up(U, "f32"), up(Wt, "f32"), up(np.zeros((r, r), np.float32), "f32"), up(last, "i32"),
                      up(u, "f32"), 1.0, tok, None, ws)
    _, otok, margins = oracle.markov_sample(base, np.tanh(U.astype(np.float64)).astype(np.float32), Wt, "f32",
                                            last, u, 1.0)
    compare_sequential_draws(down(tok), otok, margins, "rnn A=0 vs markov(tanh U)")


# ---------------------------------------------------------------- verify

def _drafts_from_q(q_logits, ud, T):
    """Draft tokens drawn from q by plain inverse CDF (test input generation)."""
    B, G, V = q_logits.shape
    out = np.zeros((B, G), np.int32)
    for b in range(B):
        for i in range(G):
            if T == 0:
                out[b, i] = int(np.argmax(q_logits[b, i]))
            else:
                w = np.exp((q_logits[b, i] - q_logits[b, i].max()) / T)
                out[b, i] = int(np.searchsorted(np.cumsum(w), ud[b, i] * w.sum(), side="right"))
    return np.minimum(out, V - 1)


# early: every row verifies only its first n_verify[b] drafts (random in -1 .. G+1,
# clamped), the prefix scheduler's early stopping
@pytest.mark.parametrize("B,G,V,T,with_stats,early", [(2, 2, MAX_V, 1.0, False, False), (2, 3, MAX_V - 3, 0.9, True, False),
                                                      (64, 7, 3000, 1.0, False, False), (16, 15, 20000, 1.0, True, False),
                                                      (32, 7, 3000, 0.0, False, False), (8, 3, 8, 1.0, False, False),
                                                      (16, 5, 4096, 0.8, False, False), (64, 7, 3000, 1.0, False, True),
                                                      (16, 15, 20000, 1.0, True, True), (32, 7, 3000, 0.0, False, True)])
def test_verify_matches_oracle(D, B, G, V, T, with_stats, early):
    import torch
    say(f"verify B={B} G={G} V={V} T={T} stats={with_stats} early={early}")
    q = rng.normal(6, f"vq{V}", (B, G, V), 2.0)
    p = np.empty((B, G + 1, V), np.float32)
    p[:, :G] = q + rng.normal(6, f"vn{V}", (B, G, V), 1.0)
    p[:, G] = rng.normal(6, f"vb{V}", (B, V), 2.0)
    ud = rng.uniform01(6, f"vud{V}", (B, G))
    ua = rng.uniform01(6, f"vua{V}", (B, G))
    uf = rng.uniform01(6, f"vuf{V}", (B,))
    drafts = _drafts_from_q(q, ud, T)
    drafts[0, 0] = V + 5 if B > 1 else drafts[0, 0]          # out-of-range draft: rejected
    stats = None
    if with_stats:
        x = q.astype(np.float64)
        mx = x.max(-1)
        stats = np.stack([mx, np.exp((x - mx[..., None]) / T).sum(-1)], -1)
    out = torch.empty((B, G + 1), dtype=torch.int32, device=DEV)
    nacc = torch.empty((B,), dtype=torch.int32, device=DEV)
    ws = workspace(D.spec_verify_workspace_size(B, G, V))
    nv = rng.integers(6, f"vnv{V}", (B,), -1, G + 2).astype(np.int32) if early else None
    D.spec_verify(up(q, "f32"), up(p, "f32"), up(drafts, "i32"), up(ua, "f32"), up(uf, "f32"), T,
                  up(stats, "f64") if stats is not None else None, out, nacc, ws,
                  n_verify=up(nv, "i32") if early else None)
    oout, onacc, margins = oracle.verify(q, p, drafts, ua, uf, T, n_verify=nv)
    gout, gnacc = down(out), down(nacc)
    flagged = 0
    for b in range(B):
        reached = list(range(min(onacc[b], G - 1) + 1)) + [G]
        if any(margins[b, i] < FLAG for i in reached if np.isfinite(margins[b, i])):
            flagged += 1
            continue
        assert gnacc[b] == onacc[b], (b, gnacc[b], onacc[b])
        np.testing.assert_array_equal(gout[b], oout[b])
    assert flagged <= flag_budget(V, B)
    assert gnacc[0] == 0 if B > 1 and T > 0 else True


def test_verify_identical_distributions_accept_everything(D):
    import torch
    B, G, V = 32, 7, 5000
    q = rng.normal(7, "vi", (B, G + 1, V), 2.0)
    drafts = _drafts_from_q(q[:, :G], rng.uniform01(7, "vid", (B, G)), 1.0)
    out = torch.empty((B, G + 1), dtype=torch.int32, device=DEV)
    nacc = torch.empty((B,), dtype=torch.int32, device=DEV)
    D.spec_verify(up(np.ascontiguousarray(q[:, :G]), "f32"), up(q, "f32"), up(drafts, "i32"),
                  up(rng.uniform01(7, "via", (B, G)), "f32"), up(rng.uniform01(7, "vif", (B,)), "f32"), 1.0,
                  None, out, nacc, workspace(D.spec_verify_workspace_size(B, G, V)))
    assert np.all(down(nacc) == G)
    np.testing.assert_array_equal(down(out)[:, :G], drafts)


def test_verify_is_lossless_on_gpu_chi_square(D):
    """The batch dimension as trials: V = 8, 200 000 rows; each emitted token at a
    reached position follows the target distribution."""
    import torch
    from scipy import special, stats
    B, G, V = 200_000, 3, 8
    g = np.random.default_rng(8)
    q1 = g.standard_normal((G, V)).astype(np.float32)
    p1 = g.standard_normal((G + 1, V)).astype(np.float32)
    qv = np.broadcast_to(q1, (B, G, V)).copy()
    pv = np.broadcast_to(p1, (B, G + 1, V)).copy()
    ud = rng.uniform01(8, "cu_d", (B, G))
    qp = special.softmax(q1.astype(np.float64), axis=1)
    drafts = np.stack([np.minimum(np.searchsorted(np.cumsum(qp[i]), ud[:, i], side="right"), V - 1)
                       for i in range(G)], 1).astype(np.int32)
    out = torch.empty((B, G + 1), dtype=torch.int32, device=DEV)
    nacc = torch.empty((B,), dtype=torch.int32, device=DEV)
    D.spec_verify(up(qv, "f32"), up(pv, "f32"), up(drafts, "i32"), up(rng.uniform01(8, "cu_a", (B, G)), "f32"),
                  up(rng.uniform01(8, "cu_f", (B,)), "f32"), 1.0, None, out, nacc,
                  workspace(D.spec_verify_workspace_size(B, G, V)))
    o, n = down(out), down(nacc)
    pp = special.softmax(p1.astype(np.float64), axis=1)
    for i in range(G + 1):
        sel = o[n >= i, i]
        cnt = np.bincount(sel, minlength=V)
        assert stats.chisquare(cnt, pp[i] * cnt.sum()).pvalue > 1e-4
    alpha1 = np.minimum(pp[0], qp[0]).sum()
    assert abs(np.mean(n >= 1) - alpha1) < 4 * np.sqrt(alpha1 * (1 - alpha1) / B)


# ---------------------------------------------------------------- verify / sampling edge cases

U_TOP = 1.0 - 2.0 ** -24          # the largest uniform below 1 in fp32


def _verify_case(name, B, G, V):
    """Inputs of one verify edge case: q [B, G, V], p [B, G+1, V] (fp32, -inf where
    masked), drafts, u_accept, u_final, and which of them are decided by construction."""
    q = rng.normal(9, f"eq_{name}", (B, G, V), 2.0)
    p = rng.normal(9, f"ep_{name}", (B, G + 1, V), 2.0)
    ua = rng.uniform01(9, f"ea_{name}", (B, G))
    uf = rng.uniform01(9, f"ef_{name}", (B,))
    ud = rng.uniform01(9, f"ed_{name}", (B, G))
    drafts = None
    if name == "disjoint":             # target on even ids in [17, V - 23], draft on odd ids: p(d) = 0,
        p[:, :, 1::2] = -np.inf        # residual = p, drawn at u_final 0 (first id 18), just below 1, random
        p[:, :, :17] = -np.inf
        p[:, :, V - 22:] = -np.inf
        q[:, :, 0::2] = -np.inf
        uf[0::4] = 0.0
        uf[1::4] = U_TOP
    elif name == "point_mass":         # every target row one finite logit: the emitted token is forced
        t = rng.integers(9, "ept", (B, G + 1), 0, V)
        p[:] = -np.inf
        for b in range(B):
            for i in range(G + 1):
                p[b, i, t[b, i]] = 0.5
        drafts = _drafts_from_q(q, ud, 1.0)
        drafts[::2, :] = t[::2, :G]    # even rows draft the target's token: accepted (p(d) = 1 >= q(d))
    elif name == "q_zero":             # drafts where q is -inf and p finite: p/q = +inf, always accepted
        drafts = rng.integers(9, "eqd", (B, G), 0, V).astype(np.int32)
        for b in range(B):
            for i in range(G):
                q[b, i, drafts[b, i]] = -np.inf
    elif name == "zero_residual":      # p = q and an out-of-range draft: rejected with no residual mass
        p[:, :G] = q
        drafts = _drafts_from_q(q, ud, 1.0)
        drafts[:, 0] = V + 3
    elif name == "u_edges":            # u_accept 0: accepted while p/q > 0, so every block is; the
        ua[:] = 0.0                    # bonus token at u_final 0 (the first token) or just below 1
        uf[0::2] = 0.0
        uf[1::2] = U_TOP
    if drafts is None:
        drafts = _drafts_from_q(np.where(np.isinf(q), -1e30, q), ud, 1.0)
    return q, p, np.asarray(drafts, np.int32), ua, uf


@pytest.mark.parametrize("name", ["disjoint", "point_mass", "q_zero", "zero_residual", "u_edges"])
@pytest.mark.parametrize("with_stats", [False, True])
def test_verify_edge_cases_match_oracle(D, name, with_stats):
    """-inf-masked logits (disjoint supports, a point-mass target, q(d) = 0 < p(d)),
    the residual with no mass (falls back to p), and the extreme uniforms.  Draws
    whose threshold sits exactly at an end of the distribution (u = 0, u just below
    1) are decided by the inverse-CDF convention itself, not by rounding, so they
    are compared without the flag exclusion."""
    import torch
    B, G, V = 16, 4, 9000
    say(f"verify edge case {name} stats={with_stats}")
    q, p, drafts, ua, uf = _verify_case(name, B, G, V)
    stats = None
    if with_stats:
        x = q.astype(np.float64)
        mx = x.max(-1)
        stats = np.stack([mx, np.exp(x - mx[..., None]).sum(-1)], -1)
    out = torch.empty((B, G + 1), dtype=torch.int32, device=DEV)
    nacc = torch.empty((B,), dtype=torch.int32, device=DEV)
    D.spec_verify(up(q, "f32"), up(p, "f32"), up(drafts, "i32"), up(ua, "f32"), up(uf, "f32"), 1.0,
                  up(stats, "f64") if stats is not None else None, out, nacc,
                  workspace(D.spec_verify_workspace_size(B, G, V)))
    oout, onacc, margins = oracle.verify(q, p, drafts, ua, uf, 1.0)
    gout, gnacc = down(out), down(nacc)
    edge_final = (uf == 0.0) | (uf == np.float32(U_TOP))
    flagged = 0
    for b in range(B):
        reached = list(range(min(onacc[b], G - 1) + 1))
        tests = [margins[b, i] for i in reached if np.isfinite(margins[b, i])]
        if not edge_final[b]:
            tests.append(margins[b, G])
        if any(m < FLAG for m in tests):                     # a random uniform next to a threshold
            flagged += 1
            continue
        assert gnacc[b] == onacc[b], (name, b, gnacc[b], onacc[b])
        np.testing.assert_array_equal(gout[b], oout[b])
    assert flagged <= flag_budget(V, B)
    # what the construction forces, independently of the oracle
    if name == "disjoint":
        assert np.all(gnacc == 0) and np.all(gout[:, 0] % 2 == 0) and np.all(gout[0::4, 0] == 18)
    elif name == "point_mass":
        for b in range(B):
            a = gnacc[b]
            assert gout[b, a] == int(np.argmax(p[b, a]))
        assert np.all(gnacc[::2] == G)
    elif name == "q_zero":
        assert np.all(gnacc == G)
    elif name == "zero_residual":
        assert np.all(gnacc == 0)
    elif name == "u_edges":
        assert np.all(gnacc == G) and np.all(gout[0::2, G] == 0)   # p/q > 0 everywhere; u = 0: token 0


@pytest.mark.parametrize("T", [1.0, 0.0])
def test_sampling_masked_logits_and_extreme_uniforms(D, T):
    """Rank-0 sampling of rows with -inf entries (a one-hot row, a row with only
    its odd ids finite, an unmasked row) at u = 0 (the first token with mass),
    u just below 1 (the last one) and ordinary uniforms."""
    import torch
    B, G, V = 4, 6, 9000
    logits = rng.normal(10, "sm", (B, G, V), 3.0)
    logits[0, :] = -np.inf
    logits[0, :, 4321] = 1.0                                  # one-hot rows
    logits[1, :, 0::2] = -np.inf                              # odd ids only
    u = rng.uniform01(10, "smu", (B, G))
    u[:, 0] = 0.0
    u[:, 1] = U_TOP
    tok = torch.empty((B, G), dtype=torch.int32, device=DEV)
    ws = workspace(D.markov_bias_sample_workspace_size(B, G, V))
    D.markov_bias_sample(up(logits, "f32"), None, None, up(np.zeros(B, np.int32), "i32"), up(u, "f32"), T, tok,
                         None, ws)
    got = down(tok)
    for b in range(B):
        for i in range(G):
            k, m = oracle.sample_row(logits[b, i], u[b, i], T)
            if i >= 2:
                assert m >= FLAG
            assert got[b, i] == k, (b, i, got[b, i], k)
    assert np.all(got[0] == 4321) and np.all(got[1] % 2 == 1)
    if T > 0:
        assert got[2, 0] == 0 and got[3, 0] == 0              # u = 0: the first token (all finite)
        assert got[1, 0] == 1                                 # the first finite id
