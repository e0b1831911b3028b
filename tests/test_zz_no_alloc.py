"""The allocation-free verify entry point (spec_verify_static, for callers that
cannot allocate device memory) against spec_verify with a caller workspace, on
the same inputs: two calls in a row on the shared static scratch, the second
with a smaller input, both identical to spec_verify bit for bit (same kernels,
same arithmetic); an input whose scratch would exceed the static array is
rejected on the host."""
import ctypes

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

from synth import rng

from _gpu_common import DEV, down, say, up, workspace


def _inputs(seed, B, G, V, T):
    q = rng.normal(seed, f"na_q{V}", (B, G, V), 2.0)
    p = np.empty((B, G + 1, V), np.float32)
    p[:, :G] = q + rng.normal(seed, f"na_n{V}", (B, G, V), 1.0)
    p[:, G] = rng.normal(seed, f"na_b{V}", (B, V), 2.0)
    ud = rng.uniform01(seed, f"na_ud{V}", (B, G))
    drafts = np.zeros((B, G), np.int32)
    for b in range(B):
        for i in range(G):
            x = q[b, i].astype(np.float64)
            w = np.exp((x - x.max()) / max(T, 1e-3))
            drafts[b, i] = min(int(np.searchsorted(np.cumsum(w), ud[b, i] * w.sum(), side="right")), V - 1)
    ua = rng.uniform01(seed, f"na_ua{V}", (B, G))
    uf = rng.uniform01(seed, f"na_uf{V}", (B,))
    stats = None
    if T > 0:
        x = q.astype(np.float64)
        mx = x.max(-1)
        stats = np.stack([mx, np.exp((x - mx[..., None]) / T).sum(-1)], -1)
    return q, p, drafts, ua, uf, stats


def _call(D, static, q, p, drafts, ua, uf, T, stats):
    import torch
    B, G, V = q.shape
    out = torch.full((B, G + 1), -7, dtype=torch.int32, device=DEV)
    nacc = torch.full((B,), -7, dtype=torch.int32, device=DEV)
    args = [B, G, V, up(q, "f32"), up(p, "f32"), up(drafts, "i32"), up(ua, "f32"), up(uf, "f32")]
    ptrs = [ctypes.c_void_p(a.data_ptr()) if hasattr(a, "data_ptr") else a for a in args]
    st_t = up(stats, "f64") if stats is not None else None
    tail = [ctypes.c_float(T), ctypes.c_void_p(st_t.data_ptr()) if st_t is not None else None, None,
            ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(nacc.data_ptr())]
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if static:
        rc = D.LIB.spec_verify_static(*ptrs, *tail, stream)
    else:
        ws = workspace(D.spec_verify_workspace_size(B, G, V))
        rc = D.LIB.spec_verify(*ptrs, *tail, ctypes.c_void_p(ws.data_ptr()), ws.numel(), stream)
    assert rc == 0, (static, rc)
    torch.cuda.synchronize()
    return down(out), down(nacc)


@pytest.fixture(scope="module")
def D():
    import torch
    assert torch.cuda.is_available()
    from block_speculative_decoding_amd import dfspec
    return dfspec


def test_static_verify_matches_workspace_verify_twice(D):
    for (B, G, V, T, seed) in [(24, 7, 20000, 1.0, 1), (3, 3, 5000, 0.8, 2), (5, 4, 3000, 0.0, 3)]:
        say(f"static-scratch verify B={B} G={G} V={V} T={T}")
        inp = _inputs(seed, B, G, V, T)
        want = _call(D, False, *inp[:5], T, inp[5])
        got = _call(D, True, *inp[:5], T, inp[5])
        np.testing.assert_array_equal(got[0], want[0])
        np.testing.assert_array_equal(got[1], want[1])
        assert np.all(want[1] >= 0) and np.all(want[1] <= G)


def test_static_verify_rejects_inputs_beyond_the_scratch(D):
    # 512 rows x 64 drafts at V = 151936 need far more than 64 MiB of scratch:
    # rejected on the host before anything runs
    B, G, V = 512, 63, 151936
    assert D.spec_verify_workspace_size(B, G, V) > 64 << 20
    dummy = ctypes.c_void_p(16)
    rc = D.LIB.spec_verify_static(B, G, V, dummy, dummy, dummy, dummy, dummy, ctypes.c_float(1.0), None, None,
                                  dummy, dummy, None)
    assert rc == D.DFS_EWORKSPACE
