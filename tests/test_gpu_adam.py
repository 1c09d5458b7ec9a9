"""The Adam branch (include/muon_adam.h) through the C ABI against the
float64 oracle.

Both sides keep m and v as float32 and p at its dtype. The GPU computes in
fp32 and the oracle in float64 from its own state, so per element
  |m_gpu - m_orc| <= 2^-21 (beta1 |m_prev| + (1 - beta1) |g|): a few fp32
    roundings of the two terms (the sum itself may cancel), the same for v;
  |p_gpu - p_orc| <= ulp(p) + 1e-5 lr' : one rounding step of p apart at most,
    plus the fp32 error of the step itself (|step| <= ~lr' when |m_hat| ~
    sqrt(v_hat)).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from workloads import (gpt2_124m_adam_multipliers, gpt2_124m_adam_shapes, make_adam_state,
                       new_grads, to_f64)

pytestmark = pytest.mark.gpu

mu = pytest.importorskip("muon_newton_schulz_04_amd")
DEV = "cuda"
TDT = {"bf16": torch.bfloat16, "fp32": torch.float32}
HP = dict(lr=1e-3, beta1=0.9, beta2=0.99, eps=1e-8, wd=0.1)


def f32(x):
    return float(np.float32(x))


def say(msg):
    print(msg, flush=True)


def ulp(x, dtype):
    """Spacing of the dtype's values at |x| (normals)."""
    bits = 8 if dtype == "bf16" else 24
    e = np.floor(np.log2(np.maximum(np.abs(x), 1e-38)))
    return np.ldexp(1.0, (e - (bits - 1)).astype(int))


def check_moments(m, v, m_o, v_o, m_prev, v_prev, g):
    b1, b2 = HP["beta1"], HP["beta2"]
    assert np.all(np.abs(m - m_o) <= 2.0 ** -21 * (b1 * np.abs(m_prev) + (1 - b1) * np.abs(g)))
    assert np.all(np.abs(v - v_o) <= 2.0 ** -21 * (b2 * v_prev + (1 - b2) * g * g))


def check(p_gpu, m_gpu, v_gpu, p_o, m_o, v_o, dtype, lr_eff, m_prev, v_prev, g):
    p, m, v = to_f64(p_gpu).ravel(), to_f64(m_gpu).ravel(), to_f64(v_gpu).ravel()
    check_moments(m, v, m_o, v_o, m_prev, v_prev, g)
    assert np.all(np.abs(p - p_o) <= ulp(p_o, dtype) + 1e-5 * lr_eff)


def views_with_odd_offsets(shapes, dtype, seed):
    """Tensors whose storage starts one element into a buffer (no 16-byte
    alignment: the scalar path)."""
    params, grads, ms, vs = make_adam_state(shapes, TDT[dtype], seed, DEV)
    out = []
    for group in (params, grads, ms, vs):
        lst = []
        for t in group:
            buf = torch.empty(t.numel() + 1, dtype=t.dtype, device=DEV)
            view = buf[1:].view(t.shape)
            view.copy_(t)
            lst.append(view)
        out.append(lst)
    return out


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("aligned", [True, False])
def test_adam_matches_oracle(dtype, aligned):
    shapes = [(1,), (7,), (8,), (768,), (2304,), (16384,), (16389,), (100003,), (4096, 768), (0,)]
    if aligned:
        params, grads, ms, vs = make_adam_state(shapes, TDT[dtype], 4, DEV)
    else:
        params, grads, ms, vs = views_with_odd_offsets(shapes, dtype, 4)
    lr_mul = [1.0, 0.5, 2.0, 1.0, 0.1, 1.0, 3.0, 1.0, 0.25, 1.0]
    wd_mul = [0.0, 1.0, 1.0, 0.0, 2.0, 1.0, 0.0, 1.0, 1.0, 1.0]
    plan = mu.AdamPlan(params, grads, ms, vs, lr_mul, wd_mul)
    for t in range(1, 4):
        if t > 1:
            new_grads(grads, 100 + t)
        # each step is compared from the state the GPU holds before it
        state = [[to_f64(x).ravel() for x in (p, m, v)] for p, m, v in zip(params, ms, vs)]
        say(f"adam parity {dtype} aligned={aligned} step {t}")
        plan.step(step=t, **HP)
        torch.cuda.synchronize()
        for i in range(len(shapes)):
            if params[i].numel() == 0:
                continue
            g = to_f64(grads[i]).ravel()
            m_prev, v_prev = state[i][1], state[i][2]
            p_o, m_o, v_o = oracle.adam_update(
                state[i][0], g, m_prev, v_prev, lr=f32(HP["lr"]),
                beta1=f32(HP["beta1"]), beta2=f32(HP["beta2"]), eps=f32(HP["eps"]),
                wd=f32(HP["wd"]), step=t, lr_mul=f32(lr_mul[i]), wd_mul=f32(wd_mul[i]),
                dtype=dtype)
            check(params[i], ms[i], vs[i], p_o, m_o, v_o, dtype, HP["lr"] * lr_mul[i],
                  m_prev, v_prev, g)
    plan.destroy()


def test_adam_zero_rate_keeps_params():
    """lr = 0: parameters bitwise unchanged (whatever wd), moments updated."""
    shapes = [(16389,), (512, 768)]
    params, grads, ms, vs = make_adam_state(shapes, torch.bfloat16, 9, DEV)
    p0 = [p.clone() for p in params]
    m0 = [m.clone() for m in ms]
    plan = mu.AdamPlan(params, grads, ms, vs)
    plan.step(lr=0.0, beta1=0.9, beta2=0.99, eps=1e-8, wd=0.5, step=1)
    torch.cuda.synchronize()
    for p, q, m, n in zip(params, p0, ms, m0):
        assert torch.equal(p, q)
        assert not torch.equal(m, n)
    plan.destroy()


def test_adam_gpt2_124m_set_sampled():
    """The full GPT-2 124M Adam set (39.5 M elements, bf16 parameters): one
    step, checked against the oracle on a seeded sample of elements of every
    tensor (the update is elementwise)."""
    shapes = gpt2_124m_adam_shapes()
    lr_mul, wd_mul = gpt2_124m_adam_multipliers(shapes)
    params, grads, ms, vs = make_adam_state(shapes, torch.bfloat16, 21, DEV)
    rng = np.random.default_rng(0)
    picks = [rng.choice(p.numel(), size=min(p.numel(), 4096), replace=False) for p in params]
    before = [[to_f64(t).ravel()[k] for t in (p, g, m, v)]
              for p, g, m, v, k in zip(params, grads, ms, vs, picks)]
    plan = mu.AdamPlan(params, grads, ms, vs, lr_mul, wd_mul)
    say("adam gpt2 124m set")
    plan.step(step=5, **HP)
    torch.cuda.synchronize()
    for i, k in enumerate(picks):
        p, g, m, v = before[i]
        p_o, m_o, v_o = oracle.adam_update(p, g, m, v, lr=f32(HP["lr"]), beta1=f32(HP["beta1"]),
                                           beta2=f32(HP["beta2"]), eps=f32(HP["eps"]),
                                           wd=f32(HP["wd"]), step=5, lr_mul=lr_mul[i],
                                           wd_mul=wd_mul[i], dtype="bf16")
        got = [to_f64(t).ravel()[k] for t in (params[i], ms[i], vs[i])]
        check_moments(got[1], got[2], m_o, v_o, m, v, g)
        assert np.all(np.abs(got[0] - p_o) <= ulp(p_o, "bf16") + 1e-5 * HP["lr"])
    plan.destroy()


def test_adam_validation():
    params, grads, ms, vs = make_adam_state([(1000,), (64,)], torch.bfloat16, 2, DEV)

    def code(fn):
        with pytest.raises(mu.MuonError) as e:
            fn()
        return e.value.code

    # the second tensor's first moment inside the first tensor's
    assert code(lambda: mu.AdamPlan(params, grads, [ms[0], ms[0][100:164]], vs)) == 1
    plan = mu.AdamPlan(params, grads, ms, vs)
    assert code(lambda: plan.step(lr=1e-3, beta1=0.9, beta2=0.99, eps=1e-8, wd=0.0, step=0)) == 1
    assert code(lambda: plan.step(lr=1e-3, beta1=1.0, beta2=0.99, eps=1e-8, wd=0.0, step=1)) == 1
    assert code(lambda: plan.step(lr=math.inf, beta1=0.9, beta2=0.99, eps=1e-8, wd=0.0,
                                  step=1)) == 1
    plan.step(lr=1e-3, beta1=0.9, beta2=0.99, eps=1e-8, wd=0.0, step=1)
    torch.cuda.synchronize()
    plan.destroy()


def test_adam_empty_and_zero_sized_lists():
    """An empty list and a list of only empty tensors plan and step as no-ops."""
    plan = mu.AdamPlan([], [], [], [])
    plan.step(lr=1e-3, beta1=0.9, beta2=0.99, eps=1e-8, wd=0.0, step=1)
    plan.destroy()
    e = [torch.empty(0, dtype=torch.bfloat16, device=DEV)]
    m = [torch.empty(0, dtype=torch.float32, device=DEV)]
    plan = mu.AdamPlan(e, e, m, m)
    plan.step(lr=1e-3, beta1=0.9, beta2=0.99, eps=1e-8, wd=0.0, step=1)
    torch.cuda.synchronize()
    plan.destroy()
