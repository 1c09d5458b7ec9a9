"""Parity of the HIP path (through the C ABI) with the float64 oracle.

Bar (per matrix, relative Frobenius error): 2e-2 for bf16 sets, 1e-4 for
fp32 sets; momentum buffers bitwise equal to the oracle's (the exact
mu * buf + g rounded once). The full matrix sets also hold every 256 x 256
tile of every matrix (rows <= cols orientation) to the same relative bar,
and the largest elementwise error to 2e-2 of the largest entry.
The oracle receives the same seeded inputs and the float32 values of the
scalars the C ABI takes (a, b, c, mu, eps are floats there).
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from workloads import CONFIGS, make_gradients, to_f64

pytestmark = pytest.mark.gpu

mu = pytest.importorskip("muon_newton_schulz_04_amd")
DEV = "cuda"
QUINTIC = CONFIGS["gpt2_small_block"].coeffs
CUBIC = (1.5, -0.5, 0.0)
TOL = {"bf16": 2e-2, "fp32": 1e-4}
TDT = {"bf16": torch.bfloat16, "fp32": torch.float32}


def f32(x):
    return float(np.float32(x))


def rel(got, want):
    nw = np.linalg.norm(want)
    return float(np.linalg.norm(got - want) / (nw if nw > 0 else 1.0))


def say(msg):
    print(msg, flush=True)


def gpu_call(grads, bufs, coeffs, steps, momentum=0.0, nesterov=False, eps=1e-7,
             ortho=False, outs=None):
    """grads/bufs: device tensors. Returns (outs, bufs) as float64 arrays."""
    if outs is None:
        outs = [torch.empty_like(g) for g in grads]
    cfg = mu.make_config(*coeffs, steps, momentum, nesterov, eps)
    if ortho:
        mu.muon_orthogonalize(grads, outs, cfg)
    else:
        mu.muon_step(grads, bufs, outs, cfg)
    torch.cuda.synchronize()
    return [to_f64(o) for o in outs], (None if bufs is None else [to_f64(b) for b in bufs])


def oracle_call(grads64, bufs64, coeffs, steps, momentum=0.0, nesterov=False, eps=1e-7,
                buf_dtype="bf16"):
    a, b, c = (f32(x) for x in coeffs)
    outs, nbs = [], []
    for i, g in enumerate(grads64):
        o, nb = oracle.muon_update(g, None if bufs64 is None else bufs64[i], a=a, b=b, c=c,
                                   steps=steps, mu=f32(momentum), nesterov=nesterov,
                                   eps=f32(eps), buf_dtype=buf_dtype)
        outs.append(o)
        nbs.append(nb)
    return outs, nbs


def check_buffers(got, want, dtype, equal_nan=False):
    for gb, wb in zip(got, want):
        assert np.array_equal(gb, wb, equal_nan=equal_nan), float(np.mean(gb != wb))


# ------------------------------------------------------------------ tiny fp32

def test_tiny_fp32_cubic_polar():
    cfg = CONFIGS["tiny_fp32_64x128_cubic"]
    g = make_gradients(cfg)[0]
    say(f"tiny fp32 {tuple(g.shape)} cubic k={cfg.steps}")
    outs, _ = gpu_call([g.to(DEV)], None, cfg.coeffs, cfg.steps, ortho=True)
    want, _ = oracle_call([to_f64(g)], None, cfg.coeffs, cfg.steps)
    assert rel(outs[0], want[0]) < 1e-4
    U, _, Vt = np.linalg.svd(to_f64(g), full_matrices=False)
    assert rel(outs[0], U @ Vt) < 1e-3


# ------------------------------------------------------- sub-steps, ragged

RAGGED = [(200, 333), (333, 200), (129, 257), (64, 128), (1, 5), (5, 1), (128, 128),
          (300, 300), (7, 1000), (1000, 7)]
CASES = {
    "x0_only": (QUINTIC, 0),
    "identity": ((1.0, 0.0, 0.0), 1),
    "gram_times_x": ((0.0, 1.0, 0.0), 1),
    "gram_sq_times_x": ((0.0, 0.0, 1.0), 1),
    "quintic5": (QUINTIC, 5),
    "cubic3": (CUBIC, 3),
}


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("case", list(CASES))
def test_substeps_ragged(dtype, case):
    coeffs, steps = CASES[case]
    wl = CONFIGS["gpt2_small_block"]
    grads = make_gradients(wl, step=3, shapes=RAGGED)
    grads = [g.to(TDT[dtype]) for g in grads]
    bufs = [torch.randn(g.shape, generator=torch.Generator().manual_seed(i)).to(g.dtype)
            for i, g in enumerate(grads)]
    say(f"substeps {dtype} {case} shapes={RAGGED}")
    outs, nbufs = gpu_call([g.to(DEV) for g in grads], [b.to(DEV) for b in bufs], coeffs, steps,
                           momentum=0.9, nesterov=True)
    want, wbufs = oracle_call([to_f64(g) for g in grads], [to_f64(b) for b in bufs], coeffs,
                              steps, momentum=0.9, nesterov=True, buf_dtype=dtype)
    for shp, o, w in zip(RAGGED, outs, want):
        assert o.shape == w.shape
        e = rel(o, w)
        assert e < TOL[dtype], (shp, e)
    check_buffers(nbufs, wbufs, dtype)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_plain_momentum_and_no_momentum(dtype):
    wl = CONFIGS["gpt2_small_block"]
    shapes = [(256, 384), (384, 256)]
    grads = [g.to(TDT[dtype]) for g in make_gradients(wl, step=4, shapes=shapes)]
    bufs = [(0.5 * g.float()).to(g.dtype) for g in grads]
    for momentum, nesterov in [(0.8, False), (0.0, False)]:
        say(f"momentum={momentum} nesterov={nesterov} {dtype}")
        outs, nb = gpu_call([g.to(DEV) for g in grads], [b.to(DEV) for b in bufs], QUINTIC, 5,
                            momentum=momentum, nesterov=nesterov)
        want, wb = oracle_call([to_f64(g) for g in grads], [to_f64(b) for b in bufs], QUINTIC, 5,
                               momentum=momentum, nesterov=nesterov, buf_dtype=dtype)
        for o, w in zip(outs, want):
            assert rel(o, w) < TOL[dtype]
        if momentum:
            check_buffers(nb, wb, dtype)
        else:
            for b0, b1 in zip(bufs, nb):      # untouched without momentum
                assert np.array_equal(to_f64(b0), b1)


# ------------------------------------------------------------ GPU invariants

def unpanel(flat, rows, cols):
    """Row-major view of a 16-bit operand stored in 32-column panels
    (element (r, c) at ((c // 32) * rows + r) * 32 + c % 32)."""
    return flat.view(cols // 32, rows, 32).permute(1, 0, 2).reshape(rows, cols)


def test_gram_is_bitwise_symmetric_and_padding_zero():
    shapes = [(200, 333), (333, 200), (256, 512)]
    grads = [g.to(DEV) for g in make_gradients(CONFIGS["gpt2_small_block"], step=5, shapes=shapes)]
    outs = [torch.empty_like(g) for g in grads]
    plan = mu.MuonPlan(grads, None, outs)
    ws = plan.step(mu.make_config(*QUINTIC, 1))
    torch.cuda.synchronize()
    for i in range(len(shapes)):
        info = plan.buffer_info(i)
        mp, m = info["mp"], info["m"]
        for key in ("gram", "poly"):
            off = info[key]
            A = unpanel(ws[off: off + mp * mp * 2].view(torch.float16), mp, mp).float().cpu()
            assert torch.equal(A, A.t()), key
            assert torch.count_nonzero(A[m:, :]) == 0 and torch.count_nonzero(A[:, m:]) == 0
        # trace(A) = ||X0||_F^2 = (||u|| / (||u|| + eps))^2 ~ 1
        off = info["gram"]
        A = unpanel(ws[off: off + mp * mp * 2].view(torch.float16), mp, mp).double().cpu()
        assert abs(float(torch.trace(A)) - 1.0) < 1e-2
    plan.destroy()


def test_split_gram_tiles():
    """A small set of wide and tall matrices (ragged m) whose Gram tiles are
    split into parts and summed in a second pass: parity with the oracle,
    bitwise determinism, and the same result on the transposed inputs."""
    shapes = [(100, 3000), (3000, 100), (256, 4096), (40, 8192)]
    red = mu.muon_schedule_query(shapes, mu.MUON_BF16, 5)
    assert (red[:, 0] >= 0).sum() > 0, "this set splits its Gram tiles"
    grads = [g.to(DEV) for g in make_gradients(CONFIGS["gpt2_small_block"], step=11, shapes=shapes)]
    bufs = [torch.zeros_like(g) for g in grads]
    say("split gram")
    got, nb = gpu_call(grads, bufs, QUINTIC, 5, momentum=0.95, nesterov=True)
    want, wb = oracle_call([to_f64(g) for g in grads], [np.zeros(g.shape) for g in grads], QUINTIC, 5,
                           momentum=0.95, nesterov=True)
    for o, w in zip(got, want):
        assert rel(o, w) < TOL["bf16"]
    check_buffers(nb, wb, "bf16")
    again, _ = gpu_call(grads, None, QUINTIC, 5, ortho=True)
    again2, _ = gpu_call(grads, None, QUINTIC, 5, ortho=True)
    for a, b in zip(again, again2):
        assert np.array_equal(a, b)
    tr, _ = gpu_call([g.t().contiguous() for g in grads], None, QUINTIC, 5, ortho=True)
    for a, t in zip(again, tr):
        assert rel(t.T, a) < 1e-2


@pytest.mark.parametrize("seed", [7, 8, 9])
def test_random_small_sets(seed):
    """Seeded random sets of 2 to 4 bf16 matrices (any orientation, ragged
    sides up to 1200 x 4000; most of them split Gram tiles) against the
    oracle, with momentum."""
    rng = np.random.default_rng(seed)
    shapes = [(int(rng.integers(1, 1200)), int(rng.integers(1, 4000))) for _ in range(int(rng.integers(2, 5)))]
    shapes = [(r, c) if rng.random() < 0.5 else (c, r) for r, c in shapes]
    grads = [g.to(DEV) for g in make_gradients(CONFIGS["gpt2_small_block"], step=seed, shapes=shapes)]
    bufs = [torch.zeros_like(g) for g in grads]
    say(f"random set seed={seed} shapes={shapes}")
    got, nb = gpu_call(grads, bufs, QUINTIC, 5, momentum=0.95, nesterov=True)
    want, wb = oracle_call([to_f64(g) for g in grads], [np.zeros(g.shape) for g in grads], QUINTIC, 5,
                           momentum=0.95, nesterov=True)
    for shp, o, w in zip(shapes, got, want):
        assert rel(o, w) < TOL["bf16"], shp
    check_buffers(nb, wb, "bf16")


def low_rank(rng, rows, cols, k):
    """rows x cols of rank k: Haar U, V (QR with the signs of diag(R)
    folded in), singular values linspace(1, 0.5, k)."""
    def haar(n, r):
        q, rr = np.linalg.qr(rng.standard_normal((n, r)))
        return q * np.sign(np.diag(rr))
    return haar(rows, k) @ np.diag(np.linspace(1.0, 0.5, k)) @ haar(cols, k).T


def test_low_rank_and_power_law_inputs():
    """Rank-deficient gradients (rank 1, 2 and 8, both orientations) and a
    1/i power-law spectrum. The polynomial's slope at 0 is a, so rounding
    noise in X0 along the zero singular directions grows by up to a^5 ~ 485
    over five steps; X0's low byte (and every later iterate's) keeps it
    under the bar. Relative Frobenius error and the largest elementwise
    error over the largest entry, both within 2e-2, with Nesterov momentum
    from a zero buffer (u = g + 0.95 g in fp32: bits beyond fp16)."""
    rng = np.random.default_rng(31)
    specs = [(4, 300, 1), (300, 4, 1), (8, 100, 2), (64, 256, 1), (256, 1024, 8), (1024, 256, 8)]
    mats = [low_rank(rng, r, c, k) for r, c, k in specs]
    q1 = np.linalg.qr(rng.standard_normal((512, 512)))[0]
    q2 = np.linalg.qr(rng.standard_normal((2048, 512)))[0]
    mats.append(q1 @ np.diag(1.0 / np.arange(1, 513)) @ q2.T)
    grads = [torch.from_numpy(g).to(torch.bfloat16).to(DEV) for g in mats]
    bufs = [torch.zeros_like(g) for g in grads]
    say("low-rank and power-law inputs")
    got, _ = gpu_call(grads, bufs, QUINTIC, 5, momentum=0.95, nesterov=True)
    want, _ = oracle_call([to_f64(g) for g in grads], [np.zeros(g.shape) for g in grads], QUINTIC, 5,
                          momentum=0.95, nesterov=True)
    for g, o, w in zip(grads, got, want):
        assert rel(o, w) < TOL["bf16"], tuple(g.shape)
        assert np.max(np.abs(o - w)) < TOL["bf16"] * np.max(np.abs(w)), tuple(g.shape)


def lo_byte_index(mp, np_):
    """Byte offset of X(m, n) in the fp16 path's low-byte layout: per 256 x 256
    tile (row-major over tiles), per 32-row block u, per 64-column wave
    column wn and 32-column block j, 64 lanes x 16 bytes; lane l32 + 32 lh
    holds row 32 u + l32, columns 64 wn + 32 j + 8 g + 4 lh + r at byte
    4 g + r."""
    m = np.arange(mp)[:, None]
    n = np.arange(np_)[None, :]
    tile = (m // 256) * (np_ // 256) + n // 256
    mm, nn = m % 256, n % 256
    lane = mm % 32 + 32 * ((nn // 4) % 2)
    return (((((tile * 8 + mm // 32) * 4 + nn // 64) * 2 + (nn // 32) % 2) * 64 + lane) * 16
            + ((nn // 8) % 4) * 4 + nn % 4)


def x0_record(ws, info):
    """{sigma, p, p guessed, rewrite flag} of a matrix (x0_scale)."""
    off = info["x0_scale"]
    return ws[off: off + 16].view(torch.float32).cpu().numpy().astype(np.float64)


def test_x0_operand_and_scale():
    """After a one-step call the workspace still holds X0 (the momentum pass
    writes it, the last update only reads it): U = u p with p the power of
    two that puts max |u| in [2^12, 2^13), as its fp16 rounding hi (x_op0)
    plus the e4m3 byte of (U - hi) 2^5 (x_lo), and sigma (hi + byte 2^-5) is
    the oracle's X0 = u / (||u|| + eps) to the format's precision: |error| <=
    2^-15 |x| (the byte's 4 significant bits below hi's last one; the fp32
    norm adds about 2^-20) plus sigma 2^-14 (the byte's smallest step). A
    fresh plan has no guess of p (guessed 1); the second call on the same
    inputs guesses right. With Nesterov momentum u = g + mu buf' carries
    fp32 bits that fp16 drops, so the byte is exercised (for a bf16 u, U is
    exact in fp16 and the byte is zero)."""
    shapes = [(200, 333), (333, 200), (256, 512), (40, 700)]
    grads = [g.to(DEV) for g in make_gradients(CONFIGS["gpt2_small_block"], step=9, shapes=shapes)]
    gen = torch.Generator().manual_seed(3)
    buf0 = [torch.randn(g.shape, generator=gen).to(torch.bfloat16).to(DEV) for g in grads]
    outs = [torch.empty_like(g) for g in grads]
    bufs = [b.clone() for b in buf0]
    plan = mu.MuonPlan(grads, bufs, outs)
    cfg = mu.make_config(*QUINTIC, 1, 0.95, True)
    for call in range(2):
        for b, b0 in zip(bufs, buf0):
            b.copy_(b0)
        ws = plan.step(cfg)
        torch.cuda.synchronize()
        for i, g in enumerate(grads):
            info = plan.buffer_info(i)
            m, n, mp, np_ = info["m"], info["n"], info["mp"], info["np"]
            u, _ = oracle.momentum_update(to_f64(g), to_f64(buf0[i]), f32(0.95), True, "bf16")
            x0 = oracle.frobenius_normalize(u, 1e-7)
            if g.shape[0] > g.shape[1]:
                x0 = x0.T
            want = np.zeros((mp, np_))
            want[:m, :n] = x0
            sigma, p, guess, flag = x0_record(ws, info)
            frac, _ = np.frexp(p)
            assert frac == 0.5, "p is a power of two"
            assert guess == (1.0 if call == 0 else p)
            assert flag == (1.0 if guess != p else 0.0)
            off = info["x_op0"]
            hi = unpanel(ws[off: off + mp * np_ * 2].view(torch.float16), mp, np_).double().cpu().numpy()
            top = np.abs(hi).max()
            assert 2.0 ** 12 * (1 - 2.0 ** -11) <= top <= 2.0 ** 13, top
            lob = ws[info["x_lo"]: info["x_lo"] + mp * np_].cpu().numpy()[lo_byte_index(mp, np_)]
            lo = torch.from_numpy(np.ascontiguousarray(lob)).view(torch.float8_e4m3fn).double().numpy()
            assert np.all(np.abs(lo) <= 64)
            got = sigma * (hi + lo * 2.0 ** -5)
            bound = (2.0 ** -15 + 2.0 ** -19) * np.abs(want) + sigma * 2.0 ** -14
            err = np.abs(got - want)
            assert np.all(err <= bound), (i, float(np.max(err / bound)))
            # the byte carries what fp16 drops: hi alone is off by up to 2^-11
            assert np.max(np.abs(sigma * hi - want)) > 4 * np.max(err)
            assert not np.any(hi[m:, :]) and not np.any(hi[:, n:])   # padding stays zero
            assert not np.any(lo[m:, :]) and not np.any(lo[:, n:])
    plan.destroy()


def test_x1_low_bytes_are_residuals():
    """After a two-step call, X1 is in x_op1 (fp16 hi) and x_lo (e4m3 bytes
    in the update's accumulator order): every byte, read through that
    layout, must be the rounded residual of its own element, |lo 2^-18| <=
    (1 + 2^-3) ulp16(hi) / 2 (plus e4m3's smallest step, 2^-27), with most
    bytes nonzero, zero padding, and hi + lo 2^-18 within the bf16 bar of the
    oracle's X1."""
    shapes = [(200, 333), (333, 200), (256, 512)]
    grads = [g.to(DEV) for g in make_gradients(CONFIGS["gpt2_small_block"], step=4, shapes=shapes)]
    outs = [torch.empty_like(g) for g in grads]
    plan = mu.MuonPlan(grads, None, outs)
    ws = plan.step(mu.make_config(*QUINTIC, 2))
    torch.cuda.synchronize()
    a, b, c = (f32(x) for x in QUINTIC)
    for i, g in enumerate(grads):
        info = plan.buffer_info(i)
        m, n, mp, np_ = info["m"], info["n"], info["mp"], info["np"]
        x0 = oracle.frobenius_normalize(to_f64(g), 1e-7)
        x1 = oracle.newton_schulz(x0.T if g.shape[0] > g.shape[1] else x0, a, b, c, 1)
        off = info["x_op1"]
        hi = unpanel(ws[off: off + mp * np_ * 2].view(torch.float16), mp, np_).double().cpu().numpy()
        lob = ws[info["x_lo"]: info["x_lo"] + mp * np_].cpu().numpy()[lo_byte_index(mp, np_)]
        lo = torch.from_numpy(np.ascontiguousarray(lob)).view(torch.float8_e4m3fn).double().numpy()
        r = lo * 2.0 ** -18
        ah = np.abs(hi)
        ulp = np.where(ah >= 2.0 ** -14, 2.0 ** (np.floor(np.log2(np.maximum(ah, 2.0 ** -14))) - 10),
                       2.0 ** -24)
        assert np.all(np.abs(r) <= (1 + 2.0 ** -3) * ulp / 2 + 2.0 ** -27)
        assert np.count_nonzero(lo[:m, :n]) > 0.5 * m * n
        assert not np.any(hi[m:, :]) and not np.any(hi[:, n:])
        assert not np.any(lo[m:, :]) and not np.any(lo[:, n:])
        assert rel((hi + r)[:m, :n], x1) < TOL["bf16"]
    plan.destroy()


def test_x0_guess_never_changes_results():
    """X0's power of two is guessed from the plan's previous call and
    corrected by the scale pass: a plan that has seen other gradient scales
    (smaller by 2^-20, where guesses miss and operands are rewritten, larger
    by 3, the same again, far larger) gives bitwise the outputs and momentum
    buffers of a fresh plan on each call's inputs."""
    shapes = [(200, 333), (333, 200), (64, 1100), (520, 96)]
    base = [g.to(DEV) for g in make_gradients(CONFIGS["gpt2_small_block"], step=21, shapes=shapes)]
    grads = [g.clone() for g in base]
    bufs = [torch.zeros_like(g) for g in grads]
    outs = [torch.empty_like(g) for g in grads]
    cfg = mu.make_config(*QUINTIC, 5, 0.95, True)
    plan = mu.MuonPlan(grads, bufs, outs)
    for call, f in enumerate((1.0, 2.0 ** -20, 3.0, 3.0, 1e4)):
        say(f"x0 guess: call {call}, gradient scale {f}")
        for g, b0 in zip(grads, base):
            g.copy_((b0.float() * f).to(torch.bfloat16))
        bufs_fresh = [b.clone() for b in bufs]
        ws = plan.step(cfg)
        torch.cuda.synchronize()
        rec = [x0_record(ws, plan.buffer_info(i)) for i in range(len(shapes))]
        # the flag marks exactly the matrices whose guess missed; the call
        # after the 2^-20 scaling (u shrinks to about mu^2 / (1 + mu) of its
        # size: the buffer still holds the large gradient) rewrites some
        assert all(r[3] == (1.0 if r[1] != r[2] else 0.0) for r in rec)
        if call == 1:
            assert any(r[3] == 1 for r in rec), "the rewrite path ran"
        got_o = [o.clone() for o in outs]
        got_b = [b.clone() for b in bufs]
        outs_fresh = [torch.empty_like(g) for g in grads]
        fresh = mu.MuonPlan(grads, bufs_fresh, outs_fresh)
        fresh.step(cfg)
        torch.cuda.synchronize()
        fresh.destroy()
        for a, b in zip(got_o + got_b, outs_fresh + bufs_fresh):
            assert torch.equal(a, b)
    plan.destroy()


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_deterministic_odd_and_scale_invariant(dtype):
    shapes = [(256, 640), (640, 256)]
    grads = [g.to(TDT[dtype]).to(DEV) for g in
             make_gradients(CONFIGS["gpt2_small_block"], step=6, shapes=shapes)]
    o1, _ = gpu_call(grads, None, QUINTIC, 5, ortho=True)
    o2, _ = gpu_call(grads, None, QUINTIC, 5, ortho=True)
    on, _ = gpu_call([-g for g in grads], None, QUINTIC, 5, ortho=True)
    o4, _ = gpu_call([g * 4 for g in grads], None, QUINTIC, 5, ortho=True)  # exact scaling
    for a, b, n, s in zip(o1, o2, on, o4):
        assert np.array_equal(a, b)
        if dtype == "fp32":
            assert np.array_equal(n, -a)          # fp32 matrix cores round symmetrically
        else:
            # the 16-bit-input matrix-core sums are not sign-symmetric in their
            # last bit; oddness holds to rounding
            assert rel(n, -a) < 5e-3
        assert rel(s, a) < (1e-5 if dtype == "fp32" else 5e-3)


def test_grouped_concurrent_run_matches_timed_whole_set_run():
    """Without the chained launch, large sets run as concurrent groups; with
    per-kernel timing on, every kernel runs over the whole set in one launch.
    Same kernels, same tiles: the results must be bitwise equal (momentum
    buffers included)."""
    wl = CONFIGS["gpt2_124m_matrix_set"]
    grads = [g.to(DEV) for g in make_gradients(wl, step=9)]
    res = []
    for timing in (False, True):
        bufs = [torch.zeros_like(g) for g in grads]
        outs = [torch.empty_like(g) for g in grads]
        plan = mu.MuonPlan(grads, bufs, outs)
        plan.set_chained(False)
        ws = torch.empty(plan.workspace_bytes, dtype=torch.uint8, device=DEV)
        cfg = mu.make_config(*wl.coeffs, wl.steps, wl.momentum, wl.nesterov, wl.eps)
        plan.set_timing(timing)
        for _ in range(2):
            plan.step(cfg, ws)
        torch.cuda.synchronize()
        if timing:
            ms, n = plan.kernel_times()["update"]
            assert n == 2 * wl.steps and ms > 0
        res.append(([o.clone() for o in outs], [b.clone() for b in bufs]))
        plan.destroy()
    for a, b in zip(res[0][0] + res[0][1], res[1][0] + res[1][1]):
        assert torch.equal(a, b)


def test_zero_matrix_empty_matrix_and_aliasing():
    g = [torch.zeros(130, 70, dtype=torch.bfloat16, device=DEV),
         torch.empty(0, 64, dtype=torch.bfloat16, device=DEV),
         torch.randn(96, 160, device=DEV).to(torch.bfloat16)]
    g_copy = [x.clone() for x in g]
    outs = [torch.full_like(x, 7.0) for x in g]
    outs[2] = g[2]                      # out aliases grad
    bufs = [torch.zeros_like(x) for x in g]
    cfg = mu.make_config(*QUINTIC, 5, 0.95, True)
    mu.muon_step(g, bufs, outs, cfg)
    torch.cuda.synchronize()
    assert torch.count_nonzero(outs[0]) == 0 and torch.isfinite(outs[0].float()).all()
    want, _ = oracle_call([to_f64(g_copy[2])], [np.zeros((96, 160))], QUINTIC, 5, 0.95, True)
    assert rel(to_f64(outs[2]), want[0]) < 2e-2


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("pad", [8, 3], ids=["ld16B", "ld_unaligned"])
def test_strided_rows(dtype, pad):
    """Matrices that are column slices of wider buffers (row stride ld = cols
    + pad): pad 8 keeps 16-byte rows for bf16, pad 3 does not (scalar
    paths). Wide and tall, ragged against the tiles. The columns beyond
    `cols` of grad, momentum and out must stay untouched."""
    wl = CONFIGS["gpt2_small_block"]
    shapes = [(200, 333), (333, 200), (64, 520)]
    grads = [g.to(TDT[dtype]) for g in make_gradients(wl, step=6, shapes=shapes)]
    bufs0 = [(0.3 * g.float()).to(g.dtype) for g in grads]
    say(f"strided rows {dtype} pad {pad}")
    g_dev, b_dev, o_dev, parents = [], [], [], []
    for g, b in zip(grads, bufs0):
        r, c = g.shape
        pg = torch.full((r, c + pad), 5.0, dtype=g.dtype, device=DEV)
        pb = torch.full((r, c + pad), 6.0, dtype=g.dtype, device=DEV)
        po = torch.full((r, c + pad), 7.0, dtype=g.dtype, device=DEV)
        pg[:, :c] = g.to(DEV)
        pb[:, :c] = b.to(DEV)
        parents.append((pg, pb, po))
        g_dev.append(pg[:, :c])
        b_dev.append(pb[:, :c])
        o_dev.append(po[:, :c])
    cfg = mu.make_config(*QUINTIC, 5, 0.95, True, 1e-7)
    mu.muon_step(g_dev, b_dev, o_dev, cfg)
    torch.cuda.synchronize()
    want, wb = oracle_call([to_f64(g) for g in grads], [to_f64(b) for b in bufs0], QUINTIC, 5,
                           momentum=0.95, nesterov=True, buf_dtype=dtype)
    for i, (pg, pb, po) in enumerate(parents):
        c = shapes[i][1]
        e = rel(to_f64(o_dev[i]), want[i])
        say(f"  matrix {shapes[i]} rel err {e:.3e}")
        assert e < TOL[dtype], (i, e)
        check_buffers([to_f64(b_dev[i])], [wb[i]], dtype)
        assert torch.equal(pg[:, c:].float().cpu(), torch.full((shapes[i][0], pad), 5.0))
        assert torch.equal(pb[:, c:].float().cpu(), torch.full((shapes[i][0], pad), 6.0))
        assert torch.equal(po[:, c:].float().cpu(), torch.full((shapes[i][0], pad), 7.0))


# ------------------------------------------------------ full configurations

TILE = 256


def tile_errors(got, want):
    """Largest relative Frobenius error over the 256 x 256 tiles of the
    rows <= cols orientation (edge tiles ragged), so that one wrong tile or
    mirrored strip cannot hide in the norm of a large matrix."""
    if got.shape[0] > got.shape[1]:
        got, want = got.T, want.T
    worst = 0.0
    for i in range(0, got.shape[0], TILE):
        for j in range(0, got.shape[1], TILE):
            worst = max(worst, rel(got[i:i + TILE, j:j + TILE], want[i:i + TILE, j:j + TILE]))
    return worst


def report(name, rows):
    """Writes the measured errors of a configuration (per shape group:
    matrices compared, max and median relative Frobenius error, worst tile,
    worst elementwise error over the largest entry) as a markdown table to
    $MUON_PARITY_REPORT/<name>.md when that variable names a directory."""
    out = os.environ.get("MUON_PARITY_REPORT")
    if not out:
        return
    os.makedirs(out, exist_ok=True)
    groups = {}
    for r in rows:
        groups.setdefault((tuple(r["shape"]), r["step"]), []).append(r)
    lines = [f"### {name}", "",
             "| step | shape | matrices | max rel Frobenius | median | worst 256x256 tile | "
             "max abs err / max abs |", "|---|---|---|---|---|---|---|"]
    for (shp, st), rs in sorted(groups.items(), key=lambda kv: (kv[0][1], kv[0][0])):
        e = np.array([r["rel"] for r in rs])
        lines.append(f"| {st} | {shp[0]}x{shp[1]} | {len(rs)} | {e.max():.3e} | {np.median(e):.3e} | "
                     f"{max(r['tile'] for r in rs):.3e} | {max(r['maxabs'] for r in rs):.3e} |")
    with open(os.path.join(out, f"{name}.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    with open(os.path.join(out, f"{name}.json"), "w") as f:
        json.dump(rows, f)


def run_config(name, step_seeds=(0,), sample=None, device_gen="cpu"):
    """One muon_step per seed (fresh gradients, the momentum buffers carried
    over) on a whole workload; every matrix (or the listed sample) against
    the oracle: buffers bitwise, the output per matrix, per tile and
    elementwise. Every matrix is also checked finite and bounded."""
    wl = CONFIGS[name]
    say(f"config {name}: {wl.n_matrices} matrices, steps {step_seeds}")
    bufs = outs = buf64 = None
    idx = list(range(wl.n_matrices)) if sample is None else sorted(sample)
    cfg = mu.make_config(*wl.coeffs, wl.steps, wl.momentum, wl.nesterov, wl.eps)
    a, b, c = (f32(x) for x in wl.coeffs)
    rows = []
    for t, s in enumerate(step_seeds):
        grads = make_gradients(wl, step=s, device=device_gen)
        grads_dev = [g.to(DEV) for g in grads]
        if bufs is None:
            bufs = [torch.zeros_like(g) for g in grads_dev]
            outs = [torch.empty_like(g) for g in grads_dev]
            buf64 = {i: np.zeros(grads[i].shape) for i in idx}
        g64 = {i: to_f64(grads[i]) for i in idx}
        del grads
        mu.muon_step(grads_dev, bufs, outs, cfg)
        torch.cuda.synchronize()
        for i in idx:
            want, nb = oracle.muon_update(g64[i], buf64[i], a=a, b=b, c=c, steps=wl.steps,
                                          mu=f32(wl.momentum), nesterov=wl.nesterov, eps=f32(wl.eps))
            got_buf = to_f64(bufs[i])
            check_buffers([got_buf], [nb], wl.dtype)
            buf64[i] = nb
            got = to_f64(outs[i])
            e, et = rel(got, want), tile_errors(got, want)
            ea = float(np.max(np.abs(got - want)) / np.max(np.abs(want)))
            rows.append({"step": t, "matrix": i, "shape": list(wl.shapes[i]), "rel": e, "tile": et,
                         "maxabs": ea})
            if i in (idx[0], idx[-1]) or e > 0.5 * wl.tol:
                say(f"  step {t} matrix {i} {wl.shapes[i]} rel {e:.3e} tile {et:.3e} maxabs {ea:.3e}")
            assert e < wl.tol, (t, i, e)
            assert et < wl.tol, (t, i, "tile", et)
            assert ea < wl.tol, (t, i, "max abs", ea)
        for i in range(len(outs)):        # every matrix: finite, singular values bounded
            o = outs[i].float()
            assert torch.isfinite(o).all()
            m = min(o.shape)
            assert float(torch.linalg.matrix_norm(o)) <= 1.21 * m ** 0.5
        del grads_dev
    report(name, rows)
    return rows


def test_config_gpt2_small_block_two_steps():
    run_config("gpt2_small_block", step_seeds=(0, 1))


def test_config_gpt2_124m_matrix_set_two_steps():
    run_config("gpt2_124m_matrix_set", step_seeds=(0, 1))


@pytest.mark.slow
def test_config_gpt2_350m_matrix_set():
    run_config("gpt2_350m_matrix_set")


@pytest.mark.slow
def test_config_wide_powerlaw():
    """The 64-matrix 2048 x 8192 / 8192 x 2048 set: the first and last
    matrix of each orientation and 16 more drawn with a fixed seed (the
    oracle takes seconds per matrix)."""
    wl = CONFIGS["wide_2048x8192_powerlaw"]
    rng = np.random.default_rng(2048)
    pick = set(rng.choice(np.arange(1, wl.n_matrices - 1), 16, replace=False).tolist())
    pick |= {0, wl.n_matrices // 2 - 1, wl.n_matrices // 2, wl.n_matrices - 1}
    run_config("wide_2048x8192_powerlaw", sample=pick, device_gen=DEV)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("steps", [0, 5])
def test_extreme_gradient_scales(dtype, steps):
    """Gradients scaled by 2^100 and 2^-20 (exact scalings of both dtypes).
    A plain fp32 sum of u^2 overflows once entries pass about 2^60, which
    would turn out into zeros; the partial sums are kept relative to a power
    of two, so the norm and out match the oracle on the scaled inputs, with
    Nesterov momentum from a zero buffer. (Inputs whose norm falls below eps
    are another matter: X0 = u / (||u|| + eps) is then tiny, and the fp16
    iterates of bf16 sets flush it.)"""
    shapes = [(200, 333), (333, 200), (64, 1100)]
    base = make_gradients(CONFIGS["gpt2_small_block"], step=17, shapes=shapes)
    for scale in (2.0 ** 100, 2.0 ** -20):
        grads = [(g.double() * scale).to(TDT[dtype]).to(DEV) for g in base]
        bufs = [torch.zeros_like(g) for g in grads]
        say(f"scale 2^{int(np.log2(scale))} {dtype} k={steps}")
        got, _ = gpu_call(grads, bufs, QUINTIC, steps, momentum=0.95, nesterov=True)
        want, _ = oracle_call([to_f64(g) for g in grads], [np.zeros(s) for s in shapes], QUINTIC, steps,
                              momentum=0.95, nesterov=True, buf_dtype=dtype)
        for shp, o, w in zip(shapes, got, want):
            assert np.all(np.isfinite(o)), shp
            assert rel(o, w) < TOL[dtype], (shp, scale, rel(o, w))


def test_nan_and_inf_propagate():
    """NaN and Inf in a gradient propagate to that matrix's whole output
    (a NaN or infinite norm makes every entry of X0 NaN or zero times
    infinity), stay in its buffer at their own positions only, and leave the
    other matrices of the set untouched (their parity with the oracle)."""
    shapes = [(96, 160), (160, 96), (128, 300)]
    grads = [g.to(DEV) for g in make_gradients(CONFIGS["gpt2_small_block"], step=13, shapes=shapes)]
    grads[0][5, 7] = float("nan")
    grads[1][40, 3] = float("inf")
    bufs = [torch.zeros_like(g) for g in grads]
    say("nan / inf propagation")
    got, nb = gpu_call(grads, bufs, QUINTIC, 5, momentum=0.95, nesterov=True)
    want, wb = oracle_call([to_f64(g) for g in grads], [np.zeros(s) for s in shapes], QUINTIC, 5,
                           momentum=0.95, nesterov=True)
    assert np.isnan(got[0]).all() and np.isnan(got[1]).all()
    check_buffers(nb, wb, "bf16", equal_nan=True)
    assert np.isnan(nb[0]).sum() == 1 and np.isinf(nb[1]).sum() == 1
    assert rel(got[2], want[2]) < TOL["bf16"]


# ------------------------------------------------------------ maximum sizes

@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_max_dims(dtype):
    """One side at the largest dimension the ABI accepts (65536), wide and
    tall: a Gram matrix of 64 x 64 over k = 65536 (long k loops, split Gram
    tiles for bf16 sets)."""
    wl = CONFIGS["gpt2_small_block"]
    shapes = [(64, 65536), (65536, 64)]
    grads = [g.to(TDT[dtype]) for g in make_gradients(wl, step=9, shapes=shapes)]
    say(f"max dims {dtype}")
    outs, _ = gpu_call([g.to(DEV) for g in grads], None, QUINTIC, 5, ortho=True)
    for i, g in enumerate(grads):
        want = oracle.orthogonalize(to_f64(g), *(f32(x) for x in QUINTIC), 5, eps=f32(1e-7))
        e = rel(outs[i], want)
        say(f"  matrix {shapes[i]} rel err {e:.3e}")
        assert e < TOL[dtype], (i, e)


def orthonormal_rows(m, n, seed):
    """m x n (n = 4 m) with orthonormal rows, on the GPU: row i holds +-1/2
    at columns i, i + m, i + 2m, i + 3m (disjoint supports, exact in bf16).
    Returns the matrix and its nonzero mask."""
    gen = torch.Generator(device="cpu").manual_seed(seed)
    signs = (torch.randint(0, 2, (4, m), generator=gen) * 2 - 1).to(torch.bfloat16).to(DEV)
    q = torch.zeros(m, n, dtype=torch.bfloat16, device=DEV)
    rows = torch.arange(m, device=DEV)
    for t in range(4):
        q[rows, rows + t * m] = 0.5 * signs[t]
    return q


@pytest.mark.slow
@pytest.mark.parametrize("tall", [False, True], ids=["wide", "tall"])
def test_max_elements_orthonormal_rows(tall):
    """A matrix of 2^30 elements (16384 x 65536, the largest the ABI
    accepts; byte offsets beyond 2^31). Its rows are orthonormal, so every
    singular value of X0 is sigma0 = 1 / (sqrt(m) + eps) and the exact output
    is p^5(sigma0) Q, p^5 from the oracle's iteration on the 1 x 1 matrix
    [[sigma0]] (the iteration acts on singular values only). The zero pattern
    must come out exactly (every product of a misplaced index would land on
    a zero), and every nonzero within 2e-2 of the value."""
    m, n = 16384, 65536
    q = orthonormal_rows(m, n, seed=11)
    g = q.t().contiguous() if tall else q
    del q
    say(f"max elements {'tall' if tall else 'wide'} {tuple(g.shape)}")
    out = torch.empty_like(g)
    cfg = mu.make_config(*QUINTIC, 5, 0.0, False, 1e-7)
    mu.muon_orthogonalize([g], [out], cfg)
    torch.cuda.synchronize()
    sigma0 = 1.0 / (np.sqrt(m) + f32(1e-7))
    p5 = float(oracle.newton_schulz(np.array([[sigma0]]), *(f32(x) for x in QUINTIC), 5)[0, 0])
    mask = g != 0
    assert int(torch.count_nonzero(out[~mask])) == 0
    ratio = (out[mask].float() / g[mask].float()).double()       # = p5 for every entry
    lo, hi = float(ratio.min()), float(ratio.max())
    say(f"  p5 {p5:.6f}: output / input in [{lo:.6f}, {hi:.6f}]")
    assert abs(lo - p5) < 2e-2 * p5 and abs(hi - p5) < 2e-2 * p5
    assert int(mask.sum()) == 4 * m


# ------------------------------------------------------------ HIP graphs

@pytest.mark.parametrize("chained", [True, False], ids=["chained", "groups"])
def test_graph_capture_replays_match_eager(chained):
    """A whole step of the GPT-2-124M set (the chained launch, or groups of
    matrices forked onto their own streams and joined back) captured once as
    a HIP graph: three replays, with eager work and synchronisations in
    between, give bitwise the outputs and momentum buffers of three eager
    steps from the same state."""
    wl = CONFIGS["gpt2_124m_matrix_set"]
    grads = [g.to(DEV) for g in make_gradients(wl, step=0)]
    bufs = [torch.zeros_like(g) for g in grads]
    outs = [torch.empty_like(g) for g in grads]
    plan = mu.MuonPlan(grads, bufs, outs)
    plan.set_chained(chained)
    ws = torch.empty(plan.workspace_bytes, dtype=torch.uint8, device=DEV)
    cfg = mu.make_config(*wl.coeffs, wl.steps, wl.momentum, wl.nesterov, wl.eps)
    say("graph capture: eager reference")
    ref = []
    for _ in range(3):
        plan.step(cfg, ws)
        torch.cuda.synchronize()
        ref.append(([o.clone() for o in outs], [b.clone() for b in bufs]))
    for b in bufs:
        b.zero_()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        plan.step(cfg, ws)
    torch.cuda.synchronize()
    for b in bufs:                      # capture runs nothing; start again from zero
        b.zero_()
    for o in outs:
        o.fill_(3.0)
    torch.cuda.synchronize()
    for k in range(3):
        say(f"graph replay {k}")
        graph.replay()
        torch.cuda.synchronize()
        _ = (grads[0].float() * 2).sum().item()   # eager work between replays
        for o, r in zip(outs, ref[k][0]):
            assert torch.equal(o, r)
        for b, r in zip(bufs, ref[k][1]):
            assert torch.equal(b, r)
    assert plan.chain_state() == ((1 if chained else 0), 0)
    del graph
    plan.destroy()
