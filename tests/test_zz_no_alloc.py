"""muon_plan_step_noalloc (the library's fixed device scratch array as the
workspace) against muon_plan_step on the same inputs, through the C ABI:
calls in a row on sets of different sizes (the second smaller, then the
first again over the array's stale contents), outputs and momentum buffers
bitwise equal to the workspace path's and within the oracle's bar; a set
that needs more workspace than the array holds is refused."""
import numpy as np
import pytest
import torch

import oracle
from workloads import CONFIGS, make_gradients, to_f64

pytestmark = pytest.mark.gpu

mu = pytest.importorskip("muon_newton_schulz_04_amd")
DEV = "cuda"
WL = CONFIGS["gpt2_small_block"]


def f32(x):
    return float(np.float32(x))


def noalloc_matches_plan_step(shapes, seed):
    print(f"no-alloc step vs plan step: shapes {shapes} seed {seed}", flush=True)
    grads = [g.to(DEV) for g in make_gradients(WL, step=seed, shapes=shapes)]
    bufs0 = [(0.5 * g.float()).to(g.dtype) for g in grads]     # a nonzero momentum state
    cfg = mu.make_config(*WL.coeffs, WL.steps, WL.momentum, WL.nesterov, WL.eps)
    b_ref, o_ref = [b.clone() for b in bufs0], [torch.empty_like(g) for g in grads]
    ref = mu.MuonPlan(grads, b_ref, o_ref)
    assert ref.workspace_bytes <= mu.MUON_SCRATCH_BYTES
    ref.step(cfg)
    b_na, o_na = [b.clone() for b in bufs0], [torch.full_like(g, 7.0) for g in grads]
    na = mu.MuonPlan(grads, b_na, o_na)
    na.step_noalloc(cfg)
    torch.cuda.synchronize()
    for x, y in zip(o_ref + b_ref, o_na + b_na):
        assert torch.equal(x, y)
    a, b, c = (f32(x) for x in WL.coeffs)
    for g, b0, o in zip(grads, bufs0, o_na):
        want, _ = oracle.muon_update(to_f64(g), to_f64(b0), a=a, b=b, c=c, steps=WL.steps,
                                     mu=f32(WL.momentum), nesterov=WL.nesterov, eps=f32(WL.eps))
        got = to_f64(o)
        assert np.linalg.norm(got - want) / np.linalg.norm(want) < WL.tol
    ref.destroy()
    na.destroy()


def test_noalloc_two_calls_second_smaller():
    big = list(WL.shapes)                                   # one GPT-2 block, about 50 MB
    small = [(200, 333), (333, 200), (5, 1)]
    noalloc_matches_plan_step(big, seed=1)
    noalloc_matches_plan_step(small, seed=2)
    noalloc_matches_plan_step(big, seed=3)                  # over the smaller set's leftovers


def test_noalloc_refuses_sets_beyond_the_array():
    wl = CONFIGS["gpt2_124m_matrix_set"]                    # about 600 MB of workspace
    grads = [torch.zeros(r, c, dtype=torch.bfloat16, device=DEV) for r, c in wl.shapes]
    bufs = [torch.zeros_like(g) for g in grads]
    outs = [torch.full_like(g, 3.0) for g in grads]
    plan = mu.MuonPlan(grads, bufs, outs)
    assert plan.workspace_bytes > mu.MUON_SCRATCH_BYTES
    cfg = mu.make_config(*wl.coeffs, wl.steps, wl.momentum, wl.nesterov, wl.eps)
    with pytest.raises(mu.MuonError) as exc:
        plan.step_noalloc(cfg)
    assert exc.value.code == 9                              # MUON_E_SCRATCH
    torch.cuda.synchronize()
    assert all(bool((o == 3.0).all()) for o in outs)        # nothing was enqueued
    plan.destroy()
