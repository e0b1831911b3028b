"""Host-side checks of the C ABI (no GPU): the library loads, exports every
function include/dfspec.h declares, sizes its workspaces, and rejects invalid
arguments before enqueueing anything."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dfspec.h")
LIB = os.path.join(ROOT, "block_speculative_decoding_amd", "libdfspec.so")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", src)) - {"if", "sizeof"})


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libdfspec.so is not built (run python -m block_speculative_decoding_amd.build)")
    return ctypes.CDLL(LIB)


def test_every_declared_symbol_is_exported(lib):
    names = _declared()
    assert {"dflash_draft_step", "markov_bias_sample", "spec_verify"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


class Cfg(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "n_layers", "hidden", "n_q_heads", "n_kv_heads", "head_dim", "mlp_dim", "vocab",
        "n_target_layers", "block", "max_ctx", "mask_token_id")] + [
        ("rms_eps", ctypes.c_float), ("rope_theta", ctypes.c_float), ("dtype", ctypes.c_int32),
        ("window", ctypes.c_int32)]


def _cfg(**kw):
    base = dict(n_layers=5, hidden=4096, n_q_heads=32, n_kv_heads=8, head_dim=128, mlp_dim=12288,
                vocab=151936, n_target_layers=5, block=16, max_ctx=4096, mask_token_id=151935,
                rms_eps=1e-6, rope_theta=1e6, dtype=1, window=0)
    base.update(kw)
    return Cfg(**base)


def test_workspace_sizes(lib):
    lib.dflash_draft_workspace_size.restype = ctypes.c_size_t
    lib.markov_bias_sample_workspace_size.restype = ctypes.c_size_t
    lib.spec_verify_workspace_size.restype = ctypes.c_size_t
    c = _cfg()
    ws = lib.dflash_draft_workspace_size(ctypes.byref(c), 8, 16)
    assert 10 << 20 < ws < 1 << 30
    assert lib.dflash_draft_workspace_size(ctypes.byref(c), 8, 64) > ws      # grows with rows
    assert lib.dflash_draft_workspace_size(ctypes.byref(_cfg(head_dim=64)), 8, 16) == 0   # bf16 needs d=128
    assert lib.dflash_draft_workspace_size(ctypes.byref(_cfg(max_ctx=100)), 8, 16) == 0
    assert lib.dflash_draft_workspace_size(ctypes.byref(_cfg(n_q_heads=30)), 8, 16) == 0
    assert lib.dflash_draft_workspace_size(ctypes.byref(_cfg(window=-1)), 8, 16) == 0     # window >= 0
    assert lib.dflash_draft_workspace_size(ctypes.byref(_cfg(window=128)), 8, 16) > 0
    assert lib.dflash_draft_workspace_size(ctypes.byref(_cfg(block=32)), 8, 16) > 0      # R = 128 rows
    assert lib.dflash_draft_workspace_size(ctypes.byref(_cfg(block=64, n_q_heads=40)), 8, 16) == 0   # R > 256
    assert lib.dflash_draft_workspace_size(None, 8, 16) == 0
    assert lib.markov_bias_sample_workspace_size(32, 15, 129280) > 0
    assert lib.markov_bias_sample_workspace_size(0, 15, 129280) == 0
    assert lib.spec_verify_workspace_size(8, 15, 151936) > 0
    assert lib.spec_verify_workspace_size(8, 0, 151936) == 0


def test_invalid_arguments_rejected_on_host(lib):
    c = _cfg()
    fake = ctypes.c_void_p(0x1000)       # device pointers: never dereferenced, validation fails first
    empty_weights = (ctypes.c_void_p * 14)()                  # host struct with null members
    lib.dflash_draft_step.restype = ctypes.c_int
    args = [ctypes.byref(c), ctypes.byref(empty_weights), 8, fake, fake, 16, 4096, fake, fake, fake,
            fake, fake, fake, ctypes.c_size_t(16), None]
    assert lib.dflash_draft_step(*args) == -1                 # weights struct not filled in
    a2 = list(args); a2[6] = 5000                             # ctx_bound > max_ctx
    assert lib.dflash_draft_step(*a2) == -1
    a3 = list(args); a3[2] = 0
    assert lib.dflash_draft_step(*a3) == -1
    bad = _cfg(block=80)
    a4 = list(args); a4[0] = ctypes.byref(bad)
    assert lib.dflash_draft_step(*a4) == -2
    # markov: rank 32 bf16 unsupported; too-small workspace
    lib.markov_bias_sample.argtypes = [ctypes.c_int32] * 4 + [ctypes.c_void_p] * 3 + [ctypes.c_int32] + \
        [ctypes.c_void_p] * 2 + [ctypes.c_float] + [ctypes.c_void_p] * 3 + [ctypes.c_size_t, ctypes.c_void_p]
    assert lib.markov_bias_sample(4, 3, 1000, 32, fake, fake, fake, 1, fake, fake, 1.0, fake, None,
                                  fake, 1 << 20, None) == -2
    assert lib.markov_bias_sample(4, 3, 1000, 0, fake, None, None, 1, fake, fake, 1.0, fake, None,
                                  fake, 8, None) == -4
    assert lib.markov_bias_sample(4, 3, 1000, 0, fake, None, None, 1, fake, fake, -1.0, fake, None,
                                  fake, 1 << 20, None) == -1
    lib.spec_verify.argtypes = [ctypes.c_int32] * 3 + [ctypes.c_void_p] * 5 + [ctypes.c_float] + \
        [ctypes.c_void_p] * 5 + [ctypes.c_size_t, ctypes.c_void_p]
    assert lib.spec_verify(4, 3, 1000, fake, fake, None, fake, fake, 1.0, None, None, fake, fake, fake,
                           1 << 20, None) == -1
    assert lib.spec_verify(4, 3, 1000, fake, fake, fake, fake, fake, 1.0, None, None, fake, fake, fake,
                           16, None) == -4
    # RNN head: a state is needed (rank >= 1), rank <= 1024, bf16 rank a multiple of 64
    lib.rnn_bias_sample_workspace_size.restype = ctypes.c_size_t
    assert lib.rnn_bias_sample_workspace_size(4, 3, 1000, 0) == 0
    assert lib.rnn_bias_sample_workspace_size(4, 3, 1000, 2048) == 0
    assert lib.rnn_bias_sample_workspace_size(4, 3, 1000, 64) > lib.markov_bias_sample_workspace_size(4, 3, 1000)
    lib.rnn_bias_sample.argtypes = [ctypes.c_int32] * 4 + [ctypes.c_void_p] * 4 + [ctypes.c_int32] + \
        [ctypes.c_void_p] * 2 + [ctypes.c_float] + [ctypes.c_void_p] * 3 + [ctypes.c_size_t, ctypes.c_void_p]
    rnn = lambda rank, dt, a, wsb, T=1.0: lib.rnn_bias_sample(4, 3, 1000, rank, fake, fake, fake, a, dt, fake, fake, T,
                                                              fake, None, fake, wsb, None)
    assert rnn(0, 0, fake, 1 << 20) == -1
    assert rnn(64, 1, None, 1 << 20) == -1                     # A missing
    assert rnn(64, 1, fake, 1 << 20, T=-1.0) == -1
    assert rnn(32, 1, fake, 1 << 20) == -2                     # bf16 rank not a multiple of 64
    assert rnn(2048, 0, fake, 1 << 30) == -2
    assert rnn(64, 1, fake, 16) == -4
    # vocabulary limit: 1024 chunks of 4096 tokens
    assert lib.markov_bias_sample(4, 3, 4194305, 0, fake, None, None, 1, fake, fake, 1.0, fake, None,
                                  fake, 1 << 30, None) == -2
    assert lib.markov_bias_sample_workspace_size(2, 2, 4194304) > 0
    # GEMM with a skipped corner: corner inside the matrix, a split count when a corner is skipped
    lib.dfs_gemm_skip.argtypes = [ctypes.c_int32] * 4 + [ctypes.c_void_p] * 3 + [ctypes.c_int32] * 4 + \
        [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    gs = lambda sp, sm, sn, wsb=1 << 30: lib.dfs_gemm_skip(300, 1000, 512, 1, fake, fake, fake, sp, 0, sm, sn,
                                                            fake, wsb, None)
    assert gs(1, 301, 0) == -1                                 # skip_m > M
    assert gs(1, 0, 1001) == -1                                # skip_n > N
    assert gs(1, -1, 0) == -1
    assert gs(0, 150, 512) == -1                               # automatic split count with a corner
    assert gs(2, 150, 512, wsb=16) == -4
    lib.dfs_status_string.restype = ctypes.c_char_p
    assert lib.dfs_status_string(-4) == b"workspace too small"


def test_packed_matrix_sizes_and_rejections(lib):
    lib.dfs_packed_matrix_bytes.restype = ctypes.c_size_t
    # rows rounded up to whole 16-row tiles, 2 bytes per value
    assert lib.dfs_packed_matrix_bytes(100, 128) == 112 * 128 * 2
    assert lib.dfs_packed_matrix_bytes(151936, 4096) == 151936 * 4096 * 2
    assert lib.dfs_packed_matrix_bytes(16, 96) == 0          # columns must be whole 64-wide tiles
    assert lib.dfs_packed_matrix_bytes(0, 64) == 0
    lib.dfs_pack_matrix.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                                    ctypes.c_void_p]
    fake = ctypes.c_void_p(0x1000)
    assert lib.dfs_pack_matrix(16, 64, None, fake, None) == -1
    assert lib.dfs_pack_matrix(16, 64, fake, fake, None) == -1     # in place is not allowed
    assert lib.dfs_pack_matrix(16, 96, fake, ctypes.c_void_p(0x2000), None) == -2
