"""The chained launch (muon_plan_set_chained): every Gram, poly and update
tile of the k Newton-Schulz steps in one launch, each tile waiting on its
matrix's completion counter, all tiles of a matrix on one XCD.

The chained and the separate launches run the same tile code on the same
operands in the same order within each matrix, so they must agree bitwise:
outputs, momentum buffers, applied weights. Parity of the chained path with
the float64 oracle is covered by the full-set tests of test_gpu_parity.py,
which run the plans' default (chained) path. The failure path is forced
from the host: a wait bound of zero makes every wait that is not already
satisfied give up, and the launch must end early and report it.
"""
import pytest
import torch

from workloads import CONFIGS, make_gradients

pytestmark = pytest.mark.gpu

mu = pytest.importorskip("muon_newton_schulz_04_amd")
DEV = "cuda"
QUINTIC = CONFIGS["gpt2_124m_matrix_set"].coeffs


def say(msg):
    print(msg, flush=True)


def mixed_set(seed):
    """Twelve 768 x 768 and four wide/tall 768 x 1024 matrices (chained:
    sixteen matrices over the eight XCDs, no split Gram tiles)."""
    g = torch.Generator().manual_seed(seed)
    shapes = [(768, 768)] * 12 + [(768, 1024), (1024, 768)] * 2
    return [(torch.randn(r, c, generator=g) * 0.02).to(torch.bfloat16).to(DEV) for r, c in shapes]


def run(grads, cfg, chained, calls, weights=None, noalloc=False):
    bufs = [torch.zeros_like(x) for x in grads]
    outs = [torch.empty_like(x) for x in grads]
    plan = mu.MuonPlan(grads, bufs, outs)
    plan.set_chained(chained)
    ws = torch.empty(plan.workspace_bytes, dtype=torch.uint8, device=DEV)
    ws_list = None
    if weights is not None:
        ws_list = [w.clone() for w in weights]
        plan.set_weights(ws_list, [1.0 + 0.25 * (i % 3) for i in range(len(grads))],
                         [0.5 + 0.5 * (i % 2) for i in range(len(grads))])
    res = []
    for _ in range(calls):
        if weights is not None:
            plan.step_apply(cfg, 0.02, 0.01, ws)
        elif noalloc:
            plan.step_noalloc(cfg)
        else:
            plan.step(cfg, ws)
        torch.cuda.synchronize()
        res.append([o.clone() for o in (ws_list if weights is not None else outs)] +
                   [b.clone() for b in bufs])
    state = plan.chain_state()
    plan.destroy()
    return res, state


def assert_same(a, b):
    assert len(a) == len(b)
    for call, (ra, rb) in enumerate(zip(a, b)):
        for t, (x, y) in enumerate(zip(ra, rb)):
            if not torch.equal(x, y):
                d = (x.float() - y.float()).abs()
                raise AssertionError(f"call {call}, tensor {t} {tuple(x.shape)}: "
                                     f"{int((d > 0).sum())} elements differ, max {float(d.max()):.3g}")


@pytest.mark.parametrize("name", ["gpt2_124m_matrix_set", "gpt2_350m_matrix_set"])
def test_chained_step_matches_separate_launches(name):
    wl = CONFIGS[name]
    grads = [x.to(DEV) for x in make_gradients(wl, step=4)]
    cfg = mu.make_config(*wl.coeffs, wl.steps, wl.momentum, wl.nesterov, wl.eps)
    say(f"chained {name}")
    a, sa = run(grads, cfg, True, 3)
    say(f"separate {name}")
    b, sb = run(grads, cfg, False, 3)
    assert sa == (1, 0) and sb == (0, 0)
    assert_same(a, b)


@pytest.mark.parametrize("steps", [1, 2, 3, 5])
def test_chained_step_counts(steps):
    """k = 1 (the first update is also the last), 2, 3 and 5 on a mixed set, four
    calls each."""
    grads = mixed_set(11)
    cfg = mu.make_config(*QUINTIC, steps, 0.95, True, 1e-7)
    say(f"chained mixed set, k = {steps}")
    a, sa = run(grads, cfg, True, 4)
    b, sb = run(grads, cfg, False, 4)
    assert sa == (1, 0) and sb == (0, 0)
    assert_same(a, b)


def test_chained_ragged_set_matches_separate_launches():
    """Sides that are not multiples of the 256-wide tile (padding tiles,
    odd tile counts, tall and wide matrices) through the chained launch."""
    shapes = [(300, 700), (700, 300), (520, 520), (257, 1000), (1000, 257), (640, 900), (900, 640),
              (333, 333)] * 2
    assert len(mu.muon_schedule_query(shapes, mu.MUON_BF16, 7)) > 0
    g = torch.Generator().manual_seed(16)
    grads = [(torch.randn(r, c, generator=g) * 0.02).to(torch.bfloat16).to(DEV) for r, c in shapes]
    cfg = mu.make_config(*QUINTIC, 5, 0.95, True, 1e-7)
    say("chained ragged set")
    a, sa = run(grads, cfg, True, 3)
    b, sb = run(grads, cfg, False, 3)
    assert sa == (1, 0) and sb == (0, 0)
    assert_same(a, b)


def test_chained_apply_matches_separate_launches():
    grads = mixed_set(12)
    g = torch.Generator().manual_seed(5)
    weights = [torch.randn(x.shape, generator=g).to(torch.bfloat16).to(DEV) for x in grads]
    cfg = mu.make_config(*QUINTIC, 5, 0.95, True, 1e-7)
    say("chained weight application")
    a, sa = run(grads, cfg, True, 2, weights=weights)
    b, _ = run(grads, cfg, False, 2, weights=weights)
    assert sa == (1, 0)
    assert_same(a, b)


def test_chained_noalloc_matches_separate_launches():
    """The no-allocation entry point on a chained set (its counters live in
    the fixed scratch array like the rest of the workspace)."""
    grads = mixed_set(13)
    cfg = mu.make_config(*QUINTIC, 5, 0.95, True, 1e-7)
    say("chained, no-allocation entry point")
    a, sa = run(grads, cfg, True, 2, noalloc=True)
    b, _ = run(grads, cfg, False, 2)
    assert sa == (1, 0)
    assert_same(a, b)


def test_chained_wait_bound_ends_the_launch_and_reports():
    """A zero wait bound: the tiles whose inputs are not ready when their
    workgroup starts give up; the launch ends, the plan reports error 1,
    and with the bound restored the next calls are exact again."""
    grads = mixed_set(14)
    cfg = mu.make_config(*QUINTIC, 5, 0.95, True, 1e-7)
    bufs = [torch.zeros_like(x) for x in grads]
    outs = [torch.empty_like(x) for x in grads]
    plan = mu.MuonPlan(grads, bufs, outs)
    ws = torch.empty(plan.workspace_bytes, dtype=torch.uint8, device=DEV)
    say("chained launch with a zero wait bound")
    plan.set_chain_timeout(0)
    plan.step(cfg, ws)
    torch.cuda.synchronize()
    assert plan.chain_state() == (1, 1)
    assert plan.chain_state() == (1, 0)          # reading clears the word
    with pytest.raises(mu.MuonError):
        plan.set_chain_timeout(-1)
    plan.set_chain_timeout(2_000_000)
    for b in bufs:
        b.zero_()
    say("chained launch, bound restored")
    got = []
    for _ in range(2):
        plan.step(cfg, ws)
        torch.cuda.synchronize()
        got.append([o.clone() for o in outs] + [b.clone() for b in bufs])
    assert plan.chain_state() == (1, 0)
    plan.destroy()
    want, _ = run(grads, cfg, False, 2)
    assert_same(got, want)


def test_timing_as_run_reports_the_chained_launch():
    """Timing mode 2 brackets the momentum slot, the normalise slot and the
    chained launch as the step runs (the per-kernel counts of Gram, poly and
    update stay zero); results are bitwise those of untimed steps. On a plan
    without a chained launch, mode 2 times each kernel as mode 1 does."""
    grads = mixed_set(15)
    cfg = mu.make_config(*QUINTIC, 5, 0.95, True, 1e-7)
    want, _ = run(grads, cfg, True, 3)
    bufs = [torch.zeros_like(x) for x in grads]
    outs = [torch.empty_like(x) for x in grads]
    plan = mu.MuonPlan(grads, bufs, outs)
    ws = torch.empty(plan.workspace_bytes, dtype=torch.uint8, device=DEV)
    with pytest.raises(mu.MuonError):
        plan.set_timing(3)
    say("timing as run, chained")
    plan.set_timing(2)
    got = []
    for _ in range(3):
        plan.step(cfg, ws)
        torch.cuda.synchronize()
        got.append([o.clone() for o in outs] + [b.clone() for b in bufs])
    kt = plan.kernel_times()
    ms, n = plan.chain_times()
    assert n == 3 and ms > 0
    assert kt["momentum"][1] == 3 and kt["normalize"][1] == 3
    assert kt["gram"][1] == kt["poly"][1] == kt["update"][1] == 0
    assert plan.chain_times() == (0.0, 0)          # reading resets
    assert_same(got, want)
    say("timing as run, separate launches")
    plan.set_chained(False)
    plan.step(cfg, ws)
    kt = plan.kernel_times()
    assert kt["gram"][1] == 5 and kt["update"][1] == 5 and plan.chain_times() == (0.0, 0)
    plan.set_timing(0)
    plan.destroy()


def test_chained_orthogonalize_matches_separate_launches():
    """muon_orthogonalize (u = G, no momentum state) on a chained set, whose
    cached plan runs chained, against a plan without momentum forced to the
    separate launches."""
    grads = mixed_set(17)
    cfg = mu.make_config(*QUINTIC, 5, 0.0, False, 1e-7)
    say("chained orthogonalisation")
    outs_a = [torch.empty_like(x) for x in grads]
    mu.muon_orthogonalize(grads, outs_a, cfg)
    outs_b = [torch.empty_like(x) for x in grads]
    plan = mu.MuonPlan(grads, None, outs_b)
    plan.set_chained(False)
    plan.step(cfg)
    torch.cuda.synchronize()
    plan.destroy()
    assert_same([outs_a], [outs_b])


def test_two_chained_plans_on_concurrent_streams():
    """Two chained plans stepping at the same time on two streams (their
    persistent workgroups share the CUs; each launch only ever waits on its
    own running workgroups): outputs and buffers bitwise those of the same
    steps run one plan after the other."""
    sets = [mixed_set(21), mixed_set(22)]
    cfg = mu.make_config(*QUINTIC, 5, 0.95, True, 1e-7)
    want = [run(g, cfg, True, 2)[0] for g in sets]
    plans, state = [], []
    for g in sets:
        bufs = [torch.zeros_like(x) for x in g]
        outs = [torch.empty_like(x) for x in g]
        plan = mu.MuonPlan(g, bufs, outs)
        ws = torch.empty(plan.workspace_bytes, dtype=torch.uint8, device=DEV)
        plans.append(plan)
        state.append((bufs, outs, ws))
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    say("two chained plans, concurrent streams")
    got = [[], []]
    for _ in range(2):
        for i in range(2):
            plans[i].step(cfg, state[i][2], streams[i])
        torch.cuda.synchronize()
        for i in range(2):
            got[i].append([o.clone() for o in state[i][1]] + [b.clone() for b in state[i][0]])
    for i in range(2):
        assert plans[i].chain_state() == (1, 0)
        assert_same(got[i], want[i])
        plans[i].destroy()
