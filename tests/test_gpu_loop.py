"""GPU tests of the multi-step loop: draft -> Markov sample -> verify -> advance,
chained on one stream with the accepted count driving the next append on the
device; against the oracle's loop, and graph replay against eager execution."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

from oracle import drafter as od
from oracle import loop as ol
from synth import MEDIUM, TINY, inputs, rng

from _gpu_common import DEV, FLAG, down, flag_budget, say, up, upload_weights


@pytest.fixture(scope="module")
def D():
    import torch
    assert torch.cuda.is_available()
    from block_speculative_decoding_amd import dfspec
    return dfspec


def test_cycle_advance_matches_oracle(D):
    import torch
    B, G = 1000, 15
    n_acc = rng.integers(5, "adv_n", (B,), -3, G + 5).astype(np.int32)      # includes out-of-range counts
    out = rng.integers(5, "adv_out", (B, G + 1), 0, 151936).astype(np.int32)
    tau0 = rng.integers(5, "adv_tau", (B,), 0, 1000).astype(np.int64)
    n_new = torch.full((B,), -7, dtype=torch.int32, device=DEV)
    last = torch.full((B,), -7, dtype=torch.int32, device=DEV)
    tau = torch.from_numpy(tau0.copy()).to(DEV)
    D.spec_cycle_advance(up(n_acc, "i32"), up(out, "i32"), n_new, last, tau)
    torch.cuda.synchronize()
    want_n, want_last, want_tau = ol.advance(n_acc, out, G)
    assert np.array_equal(down(n_new), want_n)
    assert np.array_equal(down(last), want_last)
    assert np.array_equal(down(tau), tau0 + want_tau)


@pytest.mark.parametrize("B,G,curve", [(32, 15, "busy"), (128, 7, "rising"), (1, 64, "busy"), (8, 3, "flat"),
                                       (128, 64, "busy"), (40, 15, "random")])
def test_schedule_matches_oracle(D, B, G, curve):
    # the verify lengths are integers decided in fp64 on both sides: bit-exact
    import torch
    from oracle import scheduler as osch
    g = np.random.default_rng(B * 100 + G)
    c = rng.uniform01(9, f"surv{B}_{G}", (B, G))
    c[0, :2] = [np.nan, 1.5] if G >= 2 else c[0, :2]         # NaN -> 0, above 1 -> 1
    n_max = B * (G + 1)
    if curve == "busy":       # throughput falls with the batch
        xs = np.array([1, 8, 64, n_max + 1], np.float32)
        ys = (1000.0 / (1.0 + 0.02 * xs)).astype(np.float32)
    elif curve == "rising":   # batching helps up to a point
        xs = np.array([1, n_max // 3 + 1, n_max + 1], np.float32)
        ys = np.array([10, 400, 420], np.float32)
    elif curve == "flat":
        xs, ys = np.array([1.0], np.float32), np.array([100.0], np.float32)
    else:
        xs = np.sort(g.choice(np.arange(1, n_max + 8), size=12, replace=False)).astype(np.float32)
        ys = (g.random(12) * 500 + 1).astype(np.float32)
    nv = torch.full((B,), -9, dtype=torch.int32, device=DEV)
    D.spec_schedule_verify(up(c, "f32").view(B, G), xs, ys, nv)
    torch.cuda.synchronize()
    want = osch.schedule(c, xs, ys)
    got = down(nv)
    say(f"schedule B={B} G={G} {curve}: verified {int(got.sum())} of {B * G} drafts")
    assert np.array_equal(got, want)


def _state(w, seed, ctx0, packed=False):
    """Device state of a loop over workload w: weights, caches, Markov factors."""
    import torch
    weights = inputs.drafter_weights(w, seed, gain_std=0.1)
    kc, vc = inputs.cache_prefix(w, seed, ctx0)
    U, Wt = inputs.markov_factors(w, seed, std=w.markov_rank ** -0.25)
    last0 = rng.integers(seed, "last_token", (w.batch,), 0, w.vocab - 1).astype(np.int32)
    cfg, wdev = upload_weights(w, weights, packed=packed)
    kd, vd = D_cache(w, kc, vc)
    Ud = up(U, w.dtype)
    Wd = up(Wt, w.dtype)
    if packed:
        from block_speculative_decoding_amd import dfspec
        Wd = dfspec.pack_matrix(Wd.view(w.vocab, w.markov_rank))
    return dict(weights=weights, kc=kc, vc=vc, U=U, Wt=Wt, last0=last0, cfg=cfg, wdev=wdev, kd=kd, vd=vd,
                Ud=Ud.view(w.vocab, w.markov_rank), Wd=Wd if packed else Wd.view(w.vocab, w.markov_rank))


def D_cache(w, kc, vc):
    from block_speculative_decoding_amd import dfspec
    return dfspec.cache_from_logical(up(kc, w.dtype), up(vc, w.dtype))


@pytest.mark.parametrize("targets", ["independent", "draft_plus_noise", "scheduled", "rnn_head"])
def test_loop_tiny_matches_oracle(D, targets):
    # four cycles of the tiny fp32 drafter with the Markov head.  Targets either
    # independent random rows each cycle (mostly one committed token), or each
    # side's own final draft rows plus the same seeded N(0, 0.5^2) noise and a
    # random bonus row (long accepted prefixes): the accepted count, hence the
    # next append, varies from cycle to cycle
    import torch
    from block_speculative_decoding_amd.loop import SpecLoop
    w = TINY.with_(batch=2)
    seed, cycles = 3, 4
    ctx0 = np.array([100, 61], np.int32)
    n0 = np.full(w.batch, w.block, np.int32)
    st = _state(w, seed, ctx0)
    cins = [inputs.cycle_inputs(w, seed, c) for c in range(cycles)]
    say(f"loop tiny: {cycles} cycles")
    # scheduled: draft + noise targets, and the prefix scheduler picks per-request
    # verify lengths from seeded survival scores and a falling throughput curve
    curve = (np.array([1, 4, 16], np.float32), np.array([100, 60, 20], np.float32)) if targets == "scheduled" else None
    # rnn_head: draft + noise targets, drafts from the RNN sequential head
    A = inputs.rnn_recurrence(w, seed) if targets == "rnn_head" else None
    lp = SpecLoop(st["cfg"], st["wdev"], st["kd"], st["vd"], up(ctx0, "i32"), up(st["last0"], "i32"), up(n0, "i32"),
                  1.0, st["Ud"], st["Wd"], curve=curve, A=None if A is None else up(A, "f32"))
    gpu = []
    sigma = 0.5
    for c in range(cycles):
        t = up(cins[c]["target_logits"], "f32").view(w.batch, w.block, w.vocab)
        nz = up(cins[c]["noise"], "f32").view(w.batch, w.block, w.vocab)

        def tgt(final, target, t=t, nz=nz):
            target.copy_(t)
            if targets != "independent":
                target[:, :w.gamma].copy_(final)
                target[:, :w.gamma].add_(nz[:, :w.gamma], alpha=sigma)
        lp.cycle(up(cins[c]["hidden_new"], "f32"), up(cins[c]["u_draft"], "f32"), up(cins[c]["u_accept"], "f32"),
                 up(cins[c]["u_final"], "f32"), tgt,
                 survival=up(cins[c]["survival"], "f32").view(w.batch, w.gamma) if curve else None)
        torch.cuda.synchronize()
        gpu.append({k: down(getattr(lp, a)).copy() for k, a in (("draft_tokens", "tokens"), ("n_accepted", "n_accepted"),
                    ("out_tokens", "out_tokens"), ("n_new", "n_new"), ("last_token", "last_token"),
                    ("ctx_len", "ctx_len"), ("n_verify", "n_verify"))})
    kc, vc = st["kc"].copy(), st["vc"].copy()
    def ora_target(c, final):
        t = cins[c]["target_logits"].copy()
        if targets != "independent":         # the oracle's own final rows, the same noise (fp32 add)
            t[:, :w.gamma] = (final.astype(np.float32) + np.float32(sigma) * cins[c]["noise"][:, :w.gamma]
                              ).astype(np.float32)
        return t
    ora = ol.run_cycles(od.DrafterShape.of(w), st["weights"], st["U"], st["Wt"], "f32", kc, vc, ctx0, st["last0"], n0,
                        cins, 1.0, target_fn=ora_target, curve=curve, A=A)
    alive = np.ones(w.batch, bool)
    n_cmp = n_flag = 0
    for c in range(cycles):
        g, o = gpu[c], ora[c]
        if curve is not None:                    # scheduler decisions: same inputs, exact
            assert np.array_equal(g["n_verify"], o["n_verify"]), f"cycle {c} verify lengths"
        for b in range(w.batch):
            if not alive[b]:
                continue
            for i in range(w.gamma):
                if o["margins_draft"][b, i] < FLAG:
                    alive[b] = False
                    n_flag += 1
                    break
                assert g["draft_tokens"][b, i] == o["draft_tokens"][b, i], f"cycle {c} row {b} draft {i}"
            if not alive[b]:
                continue
            if np.any(o["margins_verify"][b] < FLAG):
                alive[b] = False
                n_flag += 1
                continue
            for k in ("n_accepted", "n_new", "last_token", "ctx_len"):
                assert g[k][b] == o[k][b], f"cycle {c} row {b} {k}: gpu {g[k][b]} oracle {o[k][b]}"
            assert np.array_equal(g["out_tokens"][b], o["out_tokens"][b]), f"cycle {c} row {b} out_tokens"
            n_cmp += 1
    assert n_flag <= flag_budget(w.vocab, cycles * w.batch * w.block)
    assert n_cmp >= cycles                       # the comparison is not vacuous
    say(f"  compared {n_cmp} row-cycles, flagged {n_flag}; taus {[o['tau'].tolist() for o in ora]}")
    # the caches rows every surviving row appended, within the fp32 tolerance
    k_log, v_log = D.cache_to_logical(lp.k_cache, lp.v_cache)
    kg, vg = down(k_log), down(v_log)
    for b in np.nonzero(alive)[0]:
        n = int(gpu[-1]["ctx_len"][b])
        np.testing.assert_allclose(kg[:, b, :n], kc[:, b, :n], atol=1e-4, rtol=1e-4)
        np.testing.assert_allclose(vg[:, b, :n], vc[:, b, :n], atol=1e-4, rtol=1e-4)


def _medium_loop(D, packed=True, curve=None):
    from block_speculative_decoding_amd.loop import SpecLoop
    w = MEDIUM
    seed = 8
    ctx0 = np.array([200, 150, 100], np.int32)
    n0 = np.full(w.batch, w.block, np.int32)
    st = _state(w, seed, ctx0, packed=packed)
    lp = SpecLoop(st["cfg"], st["wdev"], st["kd"], st["vd"], up(ctx0, "i32"), up(st["last0"], "i32"), up(n0, "i32"),
                  1.0, st["Ud"], st["Wd"], wt_packed=packed, curve=curve)
    return w, seed, lp


def test_loop_identical_distributions_commit_every_draft(D):
    # target rows = the final draft rows: every draft is accepted each cycle, the
    # next block starts from the bonus token and the context grows by S per cycle
    import torch
    w, seed, lp = _medium_loop(D)
    cins = [inputs.cycle_inputs(w, seed, c) for c in range(3)]
    ctx = down(lp.ctx_len).astype(np.int64) + w.block
    for c in range(3):
        bonus = up(cins[c]["target_logits"], "f32").view(w.batch, w.block, w.vocab)[:, w.gamma]

        def same(final, target, bonus=bonus):
            target[:, :w.gamma].copy_(final)
            target[:, w.gamma].copy_(bonus)
        lp.cycle(up(cins[c]["hidden_new"], w.dtype).view(w.batch, w.block, -1), up(cins[c]["u_draft"], "f32"),
                 up(cins[c]["u_accept"], "f32"), up(cins[c]["u_final"], "f32"), same)
        torch.cuda.synchronize()
        assert down(lp.n_accepted).tolist() == [w.gamma] * w.batch
        assert np.array_equal(down(lp.out_tokens)[:, :w.gamma], down(lp.tokens))
        assert np.array_equal(down(lp.last_token), down(lp.out_tokens)[:, w.gamma])
        assert down(lp.n_new).tolist() == [w.block] * w.batch
        assert np.array_equal(down(lp.ctx_len), ctx)
        ctx = ctx + w.block
    assert down(lp.tau_sum).tolist() == [3 * w.block] * w.batch


@pytest.mark.parametrize("scheduled", [False, True])
def test_loop_graph_replay_matches_eager(D, scheduled):
    # three cycles with targets = draft + N(0, 1) noise (partial acceptance), run
    # eagerly and as one captured HIP graph replayed twice from the same start;
    # scheduled: the prefix scheduler sets the verify lengths inside the graph
    import torch
    curve = (np.array([4, 16, 49], np.float32), np.array([300, 200, 90], np.float32)) if scheduled else None
    w, seed, lp = _medium_loop(D, curve=curve)
    G = w.gamma
    cyc = [inputs.cycle_inputs(w, seed, c) for c in range(3)]
    dev_in = [dict(h=up(ci["hidden_new"], w.dtype).view(w.batch, w.block, -1), ud=up(ci["u_draft"], "f32"),
                   ua=up(ci["u_accept"], "f32"), uf=up(ci["u_final"], "f32"),
                   nz=up(ci["noise"], "f32").view(w.batch, w.block, w.vocab),
                   sv=up(ci["survival"], "f32").view(w.batch, G)) for ci in cyc]

    def run():
        for d in dev_in:
            def tgt(final, target, nz=d["nz"]):
                target[:, :G].copy_(final)
                target[:, :G].add_(nz[:, :G])
                target[:, G].copy_(nz[:, G])
                target[:, G].mul_(3.0)
            lp.cycle(d["h"], d["ud"], d["ua"], d["uf"], tgt, survival=d["sv"] if scheduled else None)

    state = (lp.k_cache, lp.v_cache, lp.ctx_len, lp.last_token, lp.n_new, lp.tau_sum)
    start = [t.clone() for t in state]
    outs = (lp.k_cache, lp.v_cache, lp.ctx_len, lp.last_token, lp.n_new, lp.tau_sum, lp.logits, lp.tokens,
            lp.out_tokens, lp.n_accepted, lp.n_verify)

    def restore():
        for t, s0 in zip(state, start):
            t.copy_(s0)

    def snap():
        return [down(t).copy() for t in outs]

    run()
    torch.cuda.synchronize()
    eager = snap()
    taus = down(lp.tau_sum)
    say(f"loop graph: eager taus over 3 cycles {taus.tolist()}")
    assert np.all(taus >= 3) and np.all(taus <= 3 * w.block)
    restore()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            run()
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(2):
        restore()
        torch.cuda.synchronize()
        x = torch.randn(512, 512, device=DEV)
        (x @ x).sum().item()                     # unrelated eager work between replays
        g.replay()
        torch.cuda.synchronize()
        got = snap()
        for a, b in zip(got, eager):
            assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), f"graph replay {rep} differs from eager"
