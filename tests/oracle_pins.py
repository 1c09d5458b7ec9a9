"""Pins of the float64 oracle against facts fixed by the mathematics.

Each pin takes an ``impl`` object exposing the oracle's functions and raises
AssertionError when the implementation disagrees with an independent fact:
  * the SVD closed form  out = U p^k(S / (||u||_F + eps)) V^T  (LAPACK SVD);
  * the cubic (1.5, -0.5, 0) iteration tends to the polar factor U V^T
    (scipy.linalg.polar);
  * exact rational closed forms for diagonal inputs (tests/golden);
  * all singular values equal -> out = p^k(1/sqrt(m)) G/||G|| with p^k in
    exact rational arithmetic;
  * a naive pure-Python loop implementation on tiny inputs;
  * invariants (scale, sign, transpose, orthogonal equivariance, rank, zero);
  * momentum closed forms; the buffer's single rounding against exact
    rational arithmetic; bf16 rounding against torch's float32 -> bfloat16
    cast and hand-made ties.
``test_oracle.py`` runs every pin on the oracle; ``test_oracle_mutations.py``
plants mistakes in copies of the oracle and checks a pin catches each one.
"""
from __future__ import annotations

import json
import math
import os
from fractions import Fraction

import numpy as np
import scipy.linalg
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
QUINTIC = (3.4445, -4.7750, 2.0315)
CUBIC = (1.5, -0.5, 0.0)
EPS = 1e-7


def rel_fro(x, y):
    return float(np.linalg.norm(np.asarray(x) - np.asarray(y)) / max(np.linalg.norm(y), 1e-300))


def p_scalar(x, a, b, c, k):
    for _ in range(k):
        x = a * x + b * x ** 3 + c * x ** 5
    return x


def closed_form(u, a, b, c, k, eps=EPS):
    """U p^k(S / (||u||_F + eps)) V^T via LAPACK SVD."""
    U, S, Vt = np.linalg.svd(u, full_matrices=False)
    s = S / (np.linalg.norm(u) + eps)
    return (U * p_scalar(s, a, b, c, k)[None, :]) @ Vt


# ---------------------------------------------------------------- pins

def pin_closed_form(impl):
    rng = np.random.default_rng(11)
    for (r, c_), coeffs, k in [((24, 40), QUINTIC, 5), ((40, 24), QUINTIC, 5),
                               ((32, 32), QUINTIC, 5), ((17, 60), CUBIC, 7),
                               ((60, 17), (2.0, -1.5, 0.5), 3), ((9, 9), QUINTIC, 1)]:
        g = rng.standard_normal((r, c_))
        g[:, 0] *= 30.0                     # spread the spectrum
        out = impl.orthogonalize(g, *coeffs, k, EPS)
        ref = closed_form(g, *coeffs, k)
        assert out.shape == g.shape
        assert rel_fro(out, ref) < 1e-11, (r, c_, rel_fro(out, ref))


def pin_closed_form_with_momentum(impl):
    """Two momentum steps from a zero buffer, then the SVD closed form of the
    u given by the momentum recurrence written out by hand."""
    rng = np.random.default_rng(5)
    mu = 0.95
    for shape in [(20, 36), (36, 20)]:
        g1 = rng.standard_normal(shape)
        g2 = rng.standard_normal(shape)
        buf = np.zeros(shape)
        out1, buf = impl.muon_update(g1, buf, a=QUINTIC[0], b=QUINTIC[1], c=QUINTIC[2], steps=5,
                                     mu=mu, nesterov=True, eps=EPS, buf_dtype="f64")
        assert rel_fro(out1, closed_form((1 + mu) * g1, *QUINTIC, 5)) < 1e-11
        out2, buf = impl.muon_update(g2, buf, a=QUINTIC[0], b=QUINTIC[1], c=QUINTIC[2], steps=5,
                                     mu=mu, nesterov=True, eps=EPS, buf_dtype="f64")
        u2 = g2 + mu * (mu * g1 + g2)
        assert rel_fro(buf, mu * g1 + g2) < 1e-15
        assert rel_fro(out2, closed_form(u2, *QUINTIC, 5)) < 1e-11
        # plain (non-Nesterov) momentum: u = buf'
        out3, buf3 = impl.muon_update(g2, mu * 0 + g1, a=1.5, b=-0.5, c=0.0, steps=4,
                                      mu=mu, nesterov=False, eps=EPS, buf_dtype="f64")
        assert rel_fro(buf3, mu * g1 + g2) < 1e-15
        assert rel_fro(out3, closed_form(mu * g1 + g2, 1.5, -0.5, 0.0, 4)) < 1e-11


def exact_round(v: Fraction, sig_bits: int) -> float:
    """Round the rational v to the nearest value with `sig_bits` significant
    bits and float32's exponent range (bf16: 8, fp32: 24), ties to even,
    by exact rational arithmetic: normal exponents from -126, a fixed
    spacing of 2**(-126 - sig_bits + 1) below 2**-126, +-inf from 2**128."""
    if v == 0:
        return 0.0
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()   # 2**e <= a < 2**(e+2)
    if Fraction(2) ** e > a:
        e -= 1
    if Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)
    ulp = Fraction(2) ** (e - sig_bits + 1)
    q = a / ulp
    n = q.numerator // q.denominator
    rem = q - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    r = n * ulp
    out = math.inf if r >= Fraction(2) ** 128 else float(r)
    return -out if v < 0 else out


def pin_momentum_bf16_state(impl):
    """The stored buffer is the exact mu*buf + g rounded once to the buffer's
    dtype (checked against exact rational arithmetic), and the Nesterov
    vector uses that rounded buffer."""
    rng = np.random.default_rng(3)
    mu = float(np.float32(0.95))         # the library's mu is a float32
    g1 = torch.tensor(rng.standard_normal((8, 12)), dtype=torch.bfloat16).double().numpy()
    g2 = torch.tensor(rng.standard_normal((8, 12)), dtype=torch.bfloat16).double().numpy()
    u1, b1 = impl.momentum_update(g1, np.zeros_like(g1), mu, True, "bf16")
    assert np.array_equal(b1, g1) and np.array_equal(u1, g1 + mu * g1)   # u = (1+mu) g
    u2, b2 = impl.momentum_update(g2, b1, mu, True, "bf16")
    want_b2 = np.array([exact_round(Fraction(mu) * Fraction(x) + Fraction(y), 8)
                        for x, y in zip(b1.ravel().tolist(), g2.ravel().tolist())]).reshape(b1.shape)
    assert np.array_equal(b2, want_b2)
    assert np.array_equal(u2, g2 + mu * want_b2)
    assert not np.array_equal(b2, mu * g1 + g2)   # rounding actually happened
    # many random bf16 (buf, g) pairs with a float32 mu, exponents up to 2**+-40
    # apart, for bf16 and fp32 state: a single rounding of the exact value
    mu32 = mu
    n = 6000
    bb = torch.tensor(rng.standard_normal(n) * 2.0 ** rng.integers(-40, 40, n),
                      dtype=torch.bfloat16).double().numpy()
    gg = torch.tensor(rng.standard_normal(n) * 2.0 ** rng.integers(-40, 40, n),
                      dtype=torch.bfloat16).double().numpy()
    bb[: n // 2] = torch.tensor(rng.standard_normal(n // 2), dtype=torch.bfloat16).double().numpy()
    gg[: n // 2] = torch.tensor(rng.standard_normal(n // 2), dtype=torch.bfloat16).double().numpy()
    for fmt, bits in (("bf16", 8), ("fp32", 24)):
        _, nb = impl.momentum_update(gg, bb, mu32, False, fmt)
        want = [exact_round(Fraction(mu32) * Fraction(x) + Fraction(y), bits)
                for x, y in zip(bb.tolist(), gg.tolist())]
        assert np.array_equal(nb, np.array(want)), fmt
    # a case where rounding through float32 would differ: mu32*b + g lies
    # just below the bf16 halfway point 2.0234375 and its float32 rounding
    # lands on it (ties to even would then give 2.03125); the exact value
    # rounds down to 2.015625
    mu9 = float(np.float32(0.9))
    b, g = np.array([0.078125]), np.array([1.953125])     # both bfloat16 values
    exact = mu9 * b + g
    assert exact[0] < 2.0234375 and np.float32(exact[0]) == np.float32(2.0234375)
    _, nb = impl.momentum_update(g, b, mu9, False, "bf16")
    assert nb[0] == 2.015625
    # a case where the float64 sum itself is inexact: mu*b = 1 + 2**-8 is the
    # bf16 halfway point between 1 and 1 + 2**-7, and g = 2**-80 puts the
    # exact value above it (the float64 sum drops g and would tie to 1)
    _, nb = impl.momentum_update(np.array([2.0 ** -80, -(2.0 ** -80)]),
                                 np.array([2.0 + 2 ** -7, 2.0 + 2 ** -7]), 0.5, False, "bf16")
    assert nb[0] == 1.0 + 2 ** -7 and nb[1] == 1.0
    u0, b0 = impl.momentum_update(g2, None, 0.0, True, "bf16")
    assert b0 is None and np.array_equal(u0, g2)
    try:                                  # a float64 mu would make mu*buf inexact
        impl.momentum_update(g2, b1, 0.95, True, "bf16")
    except ValueError:
        pass
    else:
        raise AssertionError("a mu that is not a float32 value must be refused")


def pin_polar_limit(impl):
    """Cubic coefficients drive X0 to the polar factor U V^T."""
    rng = np.random.default_rng(0)
    g = rng.standard_normal((64, 128))          # the tiny fp32 check's draw
    g32 = g.astype(np.float32).astype(np.float64)
    U, _, Vt = np.linalg.svd(g32, full_matrices=False)
    polar = U @ Vt
    e10 = rel_fro(impl.orthogonalize(g32, *CUBIC, 10, EPS), polar)
    assert 1e-4 < e10 < 1e-3, e10        # 10 steps: close but not converged
    e30 = rel_fro(impl.orthogonalize(g32, *CUBIC, 30, EPS), polar)
    assert e30 < 1e-12, e30
    wp, _ = scipy.linalg.polar(g32.T)           # right polar of the tall transpose
    assert rel_fro(impl.orthogonalize(g32.T, *CUBIC, 30, EPS), wp) < 1e-12


def pin_equal_singular_values(impl):
    """G with orthonormal rows (times 7): every normalised singular value is
    1/sqrt(m)/(1 + eps/(7 sqrt m)) so out = p^k(s) G / 7; p^k exact."""
    for m, n, want in [(768, 768, 1.0835945714), (64, 256, None)]:
        q, _ = np.linalg.qr(np.random.default_rng(m).standard_normal((n, m)))
        g = 7.0 * q.T                                   # m x n, orthonormal rows
        fro = 7.0 * math.sqrt(m)
        s = Fraction(7) / (Fraction(fro) + Fraction(EPS))
        a, b, c = (Fraction(str(x)) for x in QUINTIC)
        pk = float(p_scalar(s, a, b, c, 5))
        if want is not None:
            assert abs(pk - want) < 1e-9                # p^5 at s = 1/sqrt(768), to 10 digits
        out = impl.orthogonalize(g, *QUINTIC, 5, EPS)
        assert rel_fro(out, pk * q.T) < 1e-11


def pin_golden_diagonal(impl):
    with open(os.path.join(GOLDEN, "diag_closed_forms.json")) as f:
        gold = json.load(f)
    for case in gold["cases"]:
        r, c_ = case["rows"], case["cols"]
        for transpose in (False, True):
            g = np.zeros((r, c_))
            for i, d in enumerate(case["diag"]):
                g[i, i] = d
            want = np.zeros((r, c_))
            for i, d in enumerate(case["out_diag"]):
                want[i, i] = d
            if transpose:
                g, want = g.T, want.T
            out = impl.orthogonalize(g, *case["coeffs"], case["steps"], gold["eps"])
            assert out.shape == want.shape
            assert np.max(np.abs(out - want)) < 1e-12, (case["name"], transpose)


def naive_update(g, buf, a, b, c, k, mu, nesterov, eps):
    """The whole update with Python lists and loops only (no numpy)."""
    rows, cols = len(g), len(g[0])
    if mu:
        nb = [[mu * buf[i][j] + g[i][j] for j in range(cols)] for i in range(rows)]
        u = [[(g[i][j] + mu * nb[i][j]) if nesterov else nb[i][j] for j in range(cols)]
             for i in range(rows)]
    else:
        u = [row[:] for row in g]
    ss = 0.0
    for i in range(rows):
        for j in range(cols):
            ss += u[i][j] * u[i][j]
    nrm = math.sqrt(ss) + eps
    x = [[u[i][j] / nrm for j in range(cols)] for i in range(rows)]
    tall = rows > cols
    if tall:
        x = [[x[i][j] for i in range(rows)] for j in range(cols)]
    m, n = len(x), len(x[0])
    for _ in range(k):
        A = [[sum(x[i][t] * x[j][t] for t in range(n)) for j in range(m)] for i in range(m)]
        AA = [[sum(A[i][t] * A[t][j] for t in range(m)) for j in range(m)] for i in range(m)]
        B = [[b * A[i][j] + c * AA[i][j] for j in range(m)] for i in range(m)]
        x = [[a * x[i][j] + sum(B[i][t] * x[t][j] for t in range(m)) for j in range(n)]
             for i in range(m)]
    if tall:
        x = [[x[i][j] for i in range(m)] for j in range(n)]
    return x


def pin_brute_force(impl):
    rng = np.random.default_rng(7)
    for (r, c_), mu, nest, k in [((2, 3), 0.0, False, 5), ((5, 3), 0.9, True, 5),
                                 ((8, 8), 0.5, False, 3), ((16, 40), 0.95, True, 2),
                                 ((40, 16), 0.95, True, 2)]:
        g = rng.standard_normal((r, c_))
        buf = rng.standard_normal((r, c_)) if mu else None
        want = np.array(naive_update(g.tolist(), None if buf is None else buf.tolist(),
                                     *QUINTIC, k, mu, nest, EPS))
        out, _ = impl.muon_update(g, buf, a=QUINTIC[0], b=QUINTIC[1], c=QUINTIC[2], steps=k,
                                  mu=mu, nesterov=nest, eps=EPS, buf_dtype="f64")
        assert rel_fro(out, want) < 1e-12, ((r, c_), rel_fro(out, want))


def pin_invariants(impl):
    rng = np.random.default_rng(13)
    g = rng.standard_normal((24, 56))
    f = lambda x, k=5, abc=QUINTIC: impl.orthogonalize(x, *abc, k, 0.0)   # noqa: E731
    base = f(g)
    assert rel_fro(f(3.5 * g), base) < 1e-12                # scale
    assert np.array_equal(f(-g), -base)                      # odd
    assert rel_fro(f(g.T), base.T) < 1e-12                   # transpose
    P, _ = np.linalg.qr(rng.standard_normal((24, 24)))
    Q, _ = np.linalg.qr(rng.standard_normal((56, 56)))
    assert rel_fro(f(P @ g @ Q), P @ base @ Q) < 1e-11       # orthogonal equivariance
    low = rng.standard_normal((24, 3)) @ rng.standard_normal((3, 56))
    sv = np.linalg.svd(f(low), compute_uv=False)
    assert np.all(sv[3:] < 1e-12) and np.all(sv[:3] > 0.1)   # rank kept
    z = impl.orthogonalize(np.zeros((5, 7)), *QUINTIC, 5, EPS)
    assert np.all(z == 0) and np.all(np.isfinite(z))         # zero -> zero, no NaN
    x0 = g / (np.linalg.norm(g) + EPS)
    assert rel_fro(impl.orthogonalize(g, *QUINTIC, 0, EPS), x0) < 1e-15   # k = 0
    assert rel_fro(impl.orthogonalize(g, 1.0, 0.0, 0.0, 4, EPS), x0) < 1e-15  # identity map
    # (0,1,0): one step gives (X X^T) X
    assert rel_fro(impl.orthogonalize(g, 0.0, 1.0, 0.0, 1, EPS), x0 @ x0.T @ x0) < 1e-12
    A = x0 @ x0.T
    assert rel_fro(impl.orthogonalize(g, 0.0, 0.0, 1.0, 1, EPS), A @ A @ x0) < 1e-12


def pin_bf16_rounding(impl):
    rng = np.random.default_rng(17)
    x32 = np.concatenate([
        rng.standard_normal(20000).astype(np.float32),
        (rng.standard_normal(2000) * 1e-39).astype(np.float32),     # subnormals
        (rng.standard_normal(2000) * 1e37).astype(np.float32),
        np.array([3.3895e38, -3.3900e38, 3.4e38, 0.0, -0.0], np.float32),
    ])
    want = torch.from_numpy(x32).to(torch.bfloat16).double().numpy()
    got = impl.bf16_round(x32.astype(np.float64))
    assert np.array_equal(got, want)
    # ties to even, by hand: 1 + 2^-8 -> 1, 1 + 3*2^-8 -> 1 + 2^-6
    one = 1.0
    assert impl.bf16_round(np.array([one + 2 ** -8]))[0] == 1.0
    assert impl.bf16_round(np.array([one + 3 * 2 ** -8]))[0] == 1.0 + 2 ** -6
    assert impl.bf16_round(np.array([one + 2 ** -8 + 2 ** -30]))[0] == 1.0 + 2 ** -7
    assert impl.bf16_round(np.array([-(one + 2 ** -8)]))[0] == -1.0
    assert impl.bf16_round(np.array([2.0 ** -134]))[0] == 0.0            # subnormal tie -> 0
    assert impl.bf16_round(np.array([3 * 2.0 ** -134]))[0] == 2.0 ** -132
    assert np.isinf(impl.bf16_round(np.array([2.0 ** 128 * (1 - 2 ** -9)]))[0])
    assert np.isnan(impl.bf16_round(np.array([np.nan]))[0])


def pin_apply_weight(impl):
    """Weight application W' = W (1 - lr' wd') - lr' X (lr' = lr lr_mul,
    wd' = wd wd_mul), pinned by special cases with exact answers (dyadic
    scalars keep float64 exact)."""
    rng = np.random.default_rng(23)
    W = impl.bf16_round(rng.standard_normal((6, 10)))
    X = rng.standard_normal((6, 10))
    # lr = 0: the weight is untouched, bit for bit, whatever X and wd are
    for dt in ("bf16", "fp32", "f64"):
        assert np.array_equal(impl.apply_weight(W, X, lr=0.0, wd=3.0, lr_mul=2.0, wd_mul=5.0,
                                                dtype=dt), W)
    # step equal to the kept fraction and X = W: the result is exactly zero.
    # lr' = 0.25 * 2 = 0.5, wd' = 0.25 * 4 = 1: keep = 1 - 0.5 = 0.5 = lr';
    # ignoring wd_mul or lr_mul, swapping them, leaving lr out of the decay
    # or flipping a sign all miss 0
    Z = impl.apply_weight(W, W, lr=0.25, wd=0.25, lr_mul=2.0, wd_mul=4.0, dtype="f64")
    assert np.array_equal(Z, np.zeros_like(W))
    # pure decay (X = 0) applied k times: the exact geometric sequence
    # (1 - 1/8)^k W (lr' wd' = 0.25 * 0.5), in rational arithmetic on dyadic
    # entries
    Wd = np.array([[0.5, -1.25], [3.0, 0.0]])
    cur = Wd.copy()
    for _ in range(4):
        cur = impl.apply_weight(cur, np.zeros_like(Wd), lr=0.125, wd=0.25, lr_mul=2.0,
                                wd_mul=2.0, dtype="f64")
    want = [[float(Fraction(7, 8) ** 4 * Fraction(v)) for v in row] for row in Wd.tolist()]
    assert np.array_equal(cur, np.array(want))
    # no decay: the step is -lr*lr_mul*X exactly (dyadic values)
    Xd = np.array([[1.0, -2.0], [0.25, 4.0]])
    got = impl.apply_weight(Wd, Xd, lr=0.125, wd=0.0, lr_mul=2.0, wd_mul=9.0, dtype="f64")
    assert np.array_equal(got - Wd, -0.25 * Xd)
    # affine in (W, X) separately: superposition of the two parts
    a1 = impl.apply_weight(W, X, lr=0.3, wd=0.7, lr_mul=1.1, wd_mul=0.9, dtype="f64")
    a2 = impl.apply_weight(W, np.zeros_like(X), lr=0.3, wd=0.7, lr_mul=1.1, wd_mul=0.9, dtype="f64")
    a3 = impl.apply_weight(np.zeros_like(W), X, lr=0.3, wd=0.7, lr_mul=1.1, wd_mul=0.9, dtype="f64")
    assert np.allclose(a1, a2 + a3, rtol=0, atol=1e-14)
    # stored at the weight's dtype: bf16 / fp32 rounding of the float64 value
    b = impl.apply_weight(W, X, lr=0.3, wd=0.7, lr_mul=1.1, wd_mul=0.9, dtype="bf16")
    assert np.array_equal(b, torch.from_numpy(a1).float().to(torch.bfloat16).double().numpy()) or \
        np.max(np.abs(b - a1) / np.maximum(np.abs(a1), 1e-30)) <= 2.0 ** -9
    assert np.array_equal(impl.bf16_round(b), b)


def pin_adam(impl):
    """Adam with bias correction and decoupled decay, pinned by closed forms
    that hold exactly for dyadic betas and inputs:
      * from a zero state, with a constant gradient and eps = 0, the bias-
        corrected moments are exactly g and g^2, so every step moves p by
        -lr' sign(g) (lr' = lr lr_mul);
      * a zero gradient leaves only the decay p (1 - lr' wd') and shrinks the
        moments by beta1 and beta2;
      * with beta1 = beta2 = 0 the step is lr' g / (|g| + eps);
    plus the storage formats of the state (float32) and of p."""
    b1, b2 = 0.5, 15.0 / 16.0      # (1 - b1) = 1/2 and sqrt(1 - b2) = 1/4 differ
    g = np.array([0.5, -2.0, 0.25, -0.125, 4.0])
    p0 = np.array([1.0, -0.5, 0.0, 2.0, -3.0])
    z = np.zeros_like(g)
    p, m, v = p0.copy(), z.copy(), z.copy()
    for t in range(1, 5):
        p, m, v = impl.adam_update(p, g, m, v, lr=0.0625, beta1=b1, beta2=b2, eps=0.0, wd=0.0,
                                   step=t, lr_mul=2.0, wd_mul=3.0, dtype="fp32")
        assert np.array_equal(p, p0 - t * 0.125 * np.sign(g)), t
        assert np.array_equal(m, (1 - b1 ** t) * g) and np.array_equal(v, (1 - b2 ** t) * g * g)
    # zero gradient and zero first moment: decay only, p (1 - lr' wd') with
    # lr' wd' = (0.0625 * 2) * (1 * 4) = 1/2; the moments shrink by the betas
    m0 = np.array([0.5, -1.0, 0.25, 2.0, 0.0])
    v0 = np.array([1.0, 0.25, 4.0, 0.5, 0.0])
    p1, m1, v1 = impl.adam_update(p0, z, z, v0, lr=0.0625, beta1=b1, beta2=b2, eps=1e-3, wd=1.0,
                                  step=3, lr_mul=2.0, wd_mul=4.0, dtype="fp32")
    assert np.array_equal(p1, 0.5 * p0) and np.array_equal(m1, z) and np.array_equal(v1, b2 * v0)
    _, m2, _ = impl.adam_update(p0, z, m0, v0, lr=0.0625, beta1=b1, beta2=b2, eps=1e-3, wd=1.0,
                                step=3, dtype="fp32")
    assert np.array_equal(m2, b1 * m0)
    # no averaging: the step is lr' g / (|g| + eps) whatever the state
    p2, _, _ = impl.adam_update(p0, g, m0, v0, lr=0.5, beta1=0.0, beta2=0.0, eps=0.25, wd=0.0,
                                step=7, dtype="fp32")
    want = p0 - 0.5 * g / (np.abs(g) + 0.25)
    assert np.allclose(p2, want, rtol=2 ** -23, atol=0)
    # storage: moments are float32 values, p at its dtype
    rng = np.random.default_rng(5)
    gg, pp = rng.standard_normal(64), rng.standard_normal(64)
    pb, mb, vb = impl.adam_update(pp, gg, np.zeros(64), np.zeros(64), lr=0.01, beta1=0.9,
                                  beta2=0.99, eps=1e-8, wd=0.1, step=1, dtype="bf16")
    assert np.array_equal(impl.fp32_round(mb), mb) and np.array_equal(impl.fp32_round(vb), vb)
    assert np.array_equal(impl.bf16_round(pb), pb)
    assert not np.array_equal(pb, pp)


ALL_PINS = [pin_closed_form, pin_closed_form_with_momentum, pin_momentum_bf16_state,
            pin_polar_limit, pin_equal_singular_values, pin_golden_diagonal, pin_brute_force,
            pin_invariants, pin_bf16_rounding, pin_apply_weight, pin_adam]
