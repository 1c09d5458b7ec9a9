"""Weight application fused into the last update (muon_plan_step_apply),
through the C ABI, against the float64 oracle.

W' = W (1 - lr' wd') - lr' X with lr' = lr lr_mul, wd' = wd wd_mul. The
GPU's X carries the update's own error (bar 2e-2 for bf16 sets, 1e-4 for
fp32 sets, relative Frobenius),
and each side rounds W' once to the set's dtype, so per matrix
  ||W'_gpu - W'_oracle||_F <= bar * ||lr lr_mul X||_F + 2^-p ||W'||_F
with 2^-p the distance two round-to-nearest results of one value can be
apart (2^-8 for bf16, 2^-23 for fp32, relative).
"""
import numpy as np
import pytest
import torch

import oracle
from workloads import CONFIGS, make_gradients, to_f64

pytestmark = pytest.mark.gpu

mu = pytest.importorskip("muon_newton_schulz_04_amd")
DEV = "cuda"
QUINTIC = CONFIGS["gpt2_small_block"].coeffs
TDT = {"bf16": torch.bfloat16, "fp32": torch.float32}
BAR = {"bf16": 2e-2, "fp32": 1e-4}
ROUND = {"bf16": 2.0 ** -8, "fp32": 2.0 ** -23}


def f32(x):
    return float(np.float32(x))


def say(msg):
    print(msg, flush=True)


def make_set(shapes, dtype, seed):
    grads = [g.to(TDT[dtype]).to(DEV) for g in
             make_gradients(CONFIGS["gpt2_small_block"], step=seed, shapes=shapes)]
    gen = torch.Generator().manual_seed(seed)
    bufs = [(0.1 * torch.randn(g.shape, generator=gen)).to(TDT[dtype]).to(DEV) for g in grads]
    ws = [(0.05 * torch.randn(g.shape, generator=gen)).to(TDT[dtype]).to(DEV) for g in grads]
    return grads, bufs, ws


def run_apply(grads, bufs, ws, steps, lr, wd, lr_mul, wd_mul, momentum=0.95, nesterov=True):
    outs = [torch.full_like(g, 7.0) for g in grads]  # sentinel: must stay untouched
    plan = mu.MuonPlan(grads, bufs, outs)
    plan.set_weights(ws, lr_mul, wd_mul)
    cfg = mu.make_config(*QUINTIC, steps, momentum, nesterov, 1e-7)
    plan.step_apply(cfg, lr, wd)
    torch.cuda.synchronize()
    plan.destroy()
    return outs


def oracle_apply(g64, b64, w64, steps, lr, wd, lr_mul, wd_mul, dtype, momentum=0.95,
                 nesterov=True):
    a, b, c = (f32(x) for x in QUINTIC)
    x, nb = oracle.muon_update(g64, b64, a=a, b=b, c=c, steps=steps, mu=f32(momentum),
                               nesterov=nesterov, eps=f32(1e-7), buf_dtype=dtype)
    w_new = oracle.apply_weight(w64, x, lr=f32(lr), wd=f32(wd), lr_mul=f32(lr_mul),
                                wd_mul=f32(wd_mul), dtype=dtype)
    return w_new, x, nb


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("steps", [5, 0])
def test_apply_matches_oracle(dtype, steps):
    shapes = [(768, 768), (256, 1024), (1024, 256), (300, 500), (517, 260), (0, 64), (64, 64)]
    grads, bufs, ws = make_set(shapes, dtype, seed=11)
    g64 = [to_f64(g) for g in grads]
    b64 = [to_f64(b) for b in bufs]
    w64 = [to_f64(w) for w in ws]
    lr, wd = 0.5, 0.1
    lr_mul = [1.0, 0.5, 2.0, 1.5, 0.25, 1.0, 3.0]
    wd_mul = [1.0, 0.0, 2.0, 0.5, 1.0, 1.0, 0.0]
    say(f"apply parity {dtype} steps={steps}")
    outs = run_apply(grads, bufs, ws, steps, lr, wd, lr_mul, wd_mul)
    for i, (r, c) in enumerate(shapes):
        if r == 0 or c == 0:
            continue
        want, x, nb = oracle_apply(g64[i], b64[i], w64[i], steps, lr, wd, lr_mul[i], wd_mul[i],
                                   dtype)
        got = to_f64(ws[i])
        bound = BAR[dtype] * np.linalg.norm(f32(lr) * f32(lr_mul[i]) * x) + \
            ROUND[dtype] * np.linalg.norm(want)
        err = np.linalg.norm(got - want)
        assert err <= bound, (i, err, bound)
        assert np.array_equal(to_f64(bufs[i]), nb)              # momentum as in a plain step
        assert torch.all(outs[i] == 7.0)                        # out untouched


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_apply_exact_special_cases(dtype):
    """A zero effective rate leaves W bitwise unchanged: lr = 0, or
    lr_mul = 0 for some matrices (whatever wd, wd_mul and X are)."""
    shapes = [(512, 768), (768, 512), (130, 70)]
    grads, bufs, ws = make_set(shapes, dtype, seed=3)
    w0 = [w.clone() for w in ws]
    run_apply(grads, bufs, ws, 5, lr=0.0, wd=0.3, lr_mul=[1.0] * 3, wd_mul=[1.0] * 3)
    for w, w_ref in zip(ws, w0):
        assert torch.equal(w, w_ref)
    run_apply(grads, bufs, ws, 5, lr=0.25, wd=1.0, lr_mul=[0.0, 1.0, 0.0], wd_mul=[2.0] * 3)
    assert torch.equal(ws[0], w0[0]) and torch.equal(ws[2], w0[2])
    assert not torch.equal(ws[1], w0[1])


def test_apply_gpt2_block_set():
    """The GPT-2 block set (4 x 768^2, 768 x 3072, 3072 x 768) with Adam-like
    multipliers; all matrices against the oracle."""
    wl = CONFIGS["gpt2_small_block"]
    grads, bufs, ws = make_set(wl.shapes, "bf16", seed=5)
    g64 = [to_f64(g) for g in grads]
    b64 = [to_f64(b) for b in bufs]
    w64 = [to_f64(w) for w in ws]
    n = len(grads)
    lr_mul, wd_mul = [1.0] * n, [1.0] * n
    say("apply gpt2 block set")
    run_apply(grads, bufs, ws, wl.steps, 0.05, 0.1, lr_mul, wd_mul)
    for i in range(n):
        want, x, _ = oracle_apply(g64[i], b64[i], w64[i], wl.steps, 0.05, 0.1, 1.0, 1.0, "bf16")
        bound = BAR["bf16"] * np.linalg.norm(f32(0.05) * x) + ROUND["bf16"] * np.linalg.norm(want)
        assert np.linalg.norm(to_f64(ws[i]) - want) <= bound


def test_apply_validation():
    shapes = [(256, 512), (0, 8), (128, 128)]
    grads, bufs, ws = make_set(shapes, "bf16", seed=1)
    outs = [torch.empty_like(g) for g in grads]
    plan = mu.MuonPlan(grads, bufs, outs)
    cfg = mu.make_config(*QUINTIC, 5, 0.95, True, 1e-7)

    def code(fn):
        with pytest.raises(mu.MuonError) as e:
            fn()
        return e.value.code

    assert code(lambda: plan.step_apply(cfg, 0.1, 0.1)) == 1            # no weights attached
    with pytest.raises(ValueError):
        plan.set_weights(ws[:2])                                       # one per matrix
    assert code(lambda: plan.set_weights([ws[0], None, None])) == 1     # NULL for a non-empty matrix
    assert code(lambda: plan.set_weights([grads[0], None, ws[2]])) == 1  # overlaps a grad
    big = torch.empty(256 * 512 + 1, dtype=torch.bfloat16, device=DEV)
    mis = big[1:].view(256, 512)                                       # 2-byte aligned: legal
    plan.set_weights([mis, None, ws[2]])
    assert code(lambda: plan.step_apply(cfg, float("nan"), 0.1)) == 1   # non-finite lr
    plan.set_weights([ws[0], None, ws[2]], lr_mul=[1.0, 1.0, 1.0], wd_mul=[0.0, 0.0, 0.0])
    plan.step_apply(cfg, 0.1, 0.1)
    torch.cuda.synchronize()
    plan.destroy()


def test_apply_without_momentum_state():
    """A plan without momentum buffers (mu = 0) applies X0's orthogonalisation
    of the raw gradient; checked against the oracle with mu = 0."""
    shapes = [(384, 640), (640, 384)]
    grads, _, ws = make_set(shapes, "bf16", seed=8)
    g64 = [to_f64(g) for g in grads]
    w64 = [to_f64(w) for w in ws]
    outs = [torch.empty_like(g) for g in grads]
    plan = mu.MuonPlan(grads, None, outs)
    plan.set_weights(ws, [1.0, 2.0], [1.0, 0.0])
    plan.step_apply(mu.make_config(*QUINTIC, 5, 0.0, False, 1e-7), 0.3, 0.2)
    torch.cuda.synchronize()
    plan.destroy()
    for i, (lm, wm) in enumerate([(1.0, 1.0), (2.0, 0.0)]):
        want, x, _ = oracle_apply(g64[i], None, w64[i], 5, 0.3, 0.2, lm, wm, "bf16", momentum=0.0,
                                  nesterov=False)
        bound = BAR["bf16"] * np.linalg.norm(f32(0.3) * f32(lm) * x) + ROUND["bf16"] * np.linalg.norm(want)
        assert np.linalg.norm(to_f64(ws[i]) - want) <= bound
