"""GPU parity of dflash_draft_step against the oracle on the same seeded inputs:
the tiny fp32 workload, and a bf16 drafter with the big workloads' structure
(GQA 4:1, head dim 128) at a size that spans several GEMM/attention tiles,
with ragged context lengths, ragged appends, a prefill call, and NaN in every
cache slot the step must not read."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

import oracle
from oracle import drafter as od
from synth import MEDIUM, TINY, inputs

WIDE = MEDIUM.with_(name="wide_bf16_l1_h4096", hidden=4096, n_q_heads=32, n_kv_heads=8, mlp_dim=12288, n_layers=1,
                    vocab=9000, n_target_layers=2)

from _gpu_common import DEV, as_f64, down, say, up, upload_weights, workspace

CASES = {
    # name: (workload, seed, ctx_len, n_new, n_new_max)
    "tiny": (TINY, 0, None, None, None),
    "tiny_ragged": (TINY.with_(batch=3), 1, [124, 60, 3], [4, 1, 0], 4),
    "medium": (MEDIUM, 2, None, None, None),
    "medium_ragged": (MEDIUM, 3, [284, 131, 7], [16, 5, 0], 16),
    "medium_prefill": (MEDIUM.with_(batch=2), 4, [0, 0], [284, 150], 284),
    "medium_b1_s8": (MEDIUM.with_(batch=1, block=8, ctx=1000), 5, None, None, None),
    # weights in the tile-packed layout (V = 5000 leaves a partial last row tile)
    "medium_packed": (MEDIUM, 2, None, None, None, True),
    "medium_ragged_packed": (MEDIUM, 3, [284, 131, 7], [16, 5, 0], 16, True),
    # 320 block rows: every GEMM in its matrix-core-bound plan (128-row tiles,
    # ragged last tile), the gated MLP GEMM over three M tiles
    "medium_b20_packed": (MEDIUM.with_(batch=20), 6, None, None, None, True),
    # a 32-token block: 128 query rows per kv head, attention in two 64-row groups
    "medium_s32": (MEDIUM.with_(batch=2, block=32), 7, None, None, None),
    # sliding-window drafter (64 context keys): ragged contexts above and below the window
    "medium_window": (MEDIUM.with_(window=64), 9, [284, 131, 7], [16, 5, 0], 16),
    "medium_window_packed": (MEDIUM.with_(window=100), 9, [284, 131, 7], [16, 5, 0], 16, True),
    # one full-width layer (H 4096, 32/8 heads, F 12288) at batches where the planner
    # gives the LDS-ring tile kernel the O, gate|up and down GEMMs (B = 20) or the
    # Q|K|V, gate|up and down GEMMs (B = 24): their inputs are written tile-packed
    "wide_b20_packed": (WIDE.with_(batch=20), 10, None, None, None, True),
    "wide_b24_packed": (WIDE.with_(batch=24), 11, None, None, None, True),
    # more batch rows than one workgroup has threads: every row's bookkeeping
    # (base, appended count, new length) must still be published
    "tiny_b300_ragged": (TINY.with_(batch=300), 12, [(37 * b) % 125 for b in range(300)],
                         [b % 5 for b in range(300)], 4),
    # no context rows appended at all (n_new_max = 0: no feature projection; the call
    # still embeds, normalises and advances nothing)
    "tiny_no_append": (TINY.with_(batch=2), 13, [50, 20], [0, 0], 0),
    "medium_no_append": (MEDIUM.with_(batch=2), 14, [300, 9], [0, 0], 0),
    # a hidden size that is not a multiple of 4: the scalar paths of the embedding
    # and the RMSNorm rows
    "tiny_h250": (TINY.with_(batch=2, hidden=250), 15, None, None, None),
}


@pytest.fixture(scope="module")
def D():
    import torch
    assert torch.cuda.is_available()
    from block_speculative_decoding_amd import dfspec
    return dfspec


def run_case(D, w, seed, ctx_len, n_new, nmax, packed=False, gain_std=0.1):
    import torch
    weights = inputs.drafter_weights(w, seed, gain_std=gain_std)
    step = inputs.step_inputs(w, seed, n_new=n_new, ctx_len=ctx_len, n_new_max=nmax)
    kc, vc = inputs.cache_prefix(w, seed, step["ctx_len"], garbage="nan")
    B, G = w.batch, w.gamma
    cfg, wdev = upload_weights(w, weights, packed=packed)
    kdev, vdev = D.cache_from_logical(up(kc, w.dtype), up(vc, w.dtype))
    ctx_dev = up(step["ctx_len"], "i32")
    logits = torch.full((B, G, w.vocab), float("nan"), dtype=torch.float32, device=DEV)
    ctx_bound = int((step["ctx_len"] + step["n_new"]).max())
    lib_nmax = 0 if nmax == 0 else step["n_new_max"]   # the generators keep one (unused) row
    ws = workspace(D.dflash_draft_workspace_size(cfg, B, lib_nmax))
    D.dflash_draft_step(cfg, wdev, up(step["hidden_new"], w.dtype) if lib_nmax else None, up(step["n_new"], "i32"),
                        lib_nmax, ctx_bound, kdev, vdev, ctx_dev, up(step["last_token"], "i32"),
                        logits, ws)
    torch.cuda.synchronize()
    k_log, v_log = D.cache_to_logical(kdev, vdev)
    gpu = dict(logits=down(logits), ctx=down(ctx_dev), k=down(k_log), v=down(v_log))
    ko, vo = kc.copy(), vc.copy()
    ologits, onew = od.draft_step(od.DrafterShape.of(w), weights, step["hidden_new"], step["n_new"], ko, vo,
                                  step["ctx_len"], step["last_token"])
    ora = dict(logits=ologits, ctx=onew, k=ko, v=vo)
    if w.hidden >= 4096:   # the same steps in fp32 arithmetic: the spread any fp32 evaluation shows
        ora["logits32"], _ = od.draft_step(od.DrafterShape.of(w), weights, step["hidden_new"], step["n_new"],
                                           kc.copy(), vc.copy(), step["ctx_len"], step["last_token"],
                                           arith=np.float32)
    return gpu, ora, step


@pytest.mark.parametrize("name", list(CASES))
def test_draft_step_matches_oracle(D, name):
    w, seed, ctx_len, n_new, nmax, *packed = CASES[name]
    say(f"draft step {name}: {w.name} B={w.batch} S={w.block}")
    gpu, ora, step = run_case(D, w, seed, ctx_len, n_new, nmax, packed=bool(packed and packed[0]))
    tol = 1e-4 if w.dtype == "f32" else 2e-2
    np.testing.assert_array_equal(gpu["ctx"], ora["ctx"])
    err = np.abs(gpu["logits"].astype(np.float64) - ora["logits"])
    say(f"  logits max abs err {err.max():.3g} (tol {tol})")
    if "logits32" in ora:
        # full width (H = 4096, F = 12288): every bf16 storage rounding can flip by
        # an ulp on a sub-ulp difference, so the logits are held to the yardstick of
        # the full-size tests — within 1.5x the fp32-arithmetic oracle's own max and
        # mean departure from the float64 oracle, never tighter than 2e-2 max
        spread = np.abs(ora["logits32"].astype(np.float64) - ora["logits"])
        say(f"  fp32 oracle max {spread.max():.4f} mean {spread.mean():.5f}; GPU mean {err.mean():.5f}")
        assert err.max() <= max(tol, 1.5 * spread.max())
        assert err.mean() <= 1.5 * spread.mean()
    else:
        assert err.max() <= tol
    # cache: appended slots within tolerance, every other slot bit-identical (NaN stays NaN)
    for b in range(w.batch):
        c0, c1 = int(step["ctx_len"][b]), int(ora["ctx"][b])
        for key in ("k", "v"):
            g, o = gpu[key][:, b], ora[key][:, b]
            # bf16-stored values: 2e-2 abs, or one bf16 ulp of the value where larger
            np.testing.assert_allclose(as_f64(g[:, c0:c1], w.dtype), as_f64(o[:, c0:c1], w.dtype), atol=tol,
                                       rtol=0 if w.dtype == "f32" else 2.0 ** -7)
            untouched = np.concatenate([g[:, :c0].ravel(), g[:, c1:].ravel()])
            expect = np.concatenate([o[:, :c0].ravel(), o[:, c1:].ravel()])
            assert np.array_equal(untouched.view(np.uint8), expect.view(np.uint8))


def test_draft_step_is_deterministic(D):
    w, seed, ctx_len, n_new, nmax = CASES["medium"]
    a, _, _ = run_case(D, w, seed, ctx_len, n_new, nmax)
    b, _, _ = run_case(D, w, seed, ctx_len, n_new, nmax)
    assert np.array_equal(a["logits"].view(np.uint32), b["logits"].view(np.uint32))


def test_draft_packed_weights_bit_identical_to_row_major(D):
    w, seed, ctx_len, n_new, nmax = CASES["medium_ragged"]
    a, _, _ = run_case(D, w, seed, ctx_len, n_new, nmax, packed=False)
    b, _, _ = run_case(D, w, seed, ctx_len, n_new, nmax, packed=True)
    assert np.array_equal(a["logits"].view(np.uint32), b["logits"].view(np.uint32))
    for key in ("k", "v"):
        assert np.array_equal(a[key].view(np.uint8), b[key].view(np.uint8))
