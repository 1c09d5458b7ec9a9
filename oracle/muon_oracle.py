"""Float64 CPU oracle of the Muon update: momentum, Frobenius normalisation,
and the odd-polynomial Newton-Schulz iteration.

TEST INFRASTRUCTURE ONLY. This module is the reference the HIP path is checked
against. Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` may import it. It shares no code with the HIP library
(``muon_newton_schulz_04_amd/``) and imports nothing from it.

Sources (the pages are prose; none prints the iteration or code):
  [MUON]  blog.hotdry.top, "How to train a GPT model in 3 minutes: an analysis
          of modded-nanogpt's optimizations", section 2 (algorithm and
          architecture innovations), item "customised Muon optimizer": Muon
          comes from spectral gradient descent and replaces the SVD-like step
          of a conventional optimizer by a Newton-Schulz iteration; it keeps
          less optimizer state than AdamW (one momentum buffer).
  [GREEN] yongjin360.com, Modded-NanoGPT green-AI article, section
          "technical evolution": Muon's Newton-Schulz orthogonalisation.
The pages leave the iteration's form, coefficients, step count, normalisation,
transpose rule, momentum form and precision open. The readings taken here:
  * momentum (SGD form)  buf' = mu*buf + g, buf' stored at the buffer's dtype
    (round to nearest, ties to even); u = g + mu*buf' (Nesterov) or u = buf';
  * X0 = u / (||u||_F + eps);
  * work on X0^T when rows > cols so the Gram matrix is min(rows,cols) square;
  * k times: A = X X^T, B = b A + c A A, X = a X + B X; transpose back.
Every step is computed in float64 with dense matrix products, no blocking,
no symmetry tricks and no batching.

Parity of every function here is pinned by ``tests/test_oracle.py`` against
the SVD closed form, the polar factor, exact rational arithmetic and naive
loops (no function is parity unpinned).
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "bf16_round",
    "fp32_round",
    "two_sum",
    "round_exact_sum",
    "momentum_update",
    "frobenius_normalize",
    "ns_polynomial_step",
    "newton_schulz",
    "orthogonalize",
    "muon_update",
    "apply_weight",
    "adam_update",
    "falg_flops",
]


# ---------------------------------------------------------------------------
# Storage rounding of the optimizer state (the momentum buffer).
# ---------------------------------------------------------------------------

def bf16_round(x) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 value, ties to even.

    bfloat16 has float32's exponent range (normals down to 2**-126,
    subnormals spaced 2**-133) and 8 significant bits. Written out from that
    definition: split x = f * 2**e with 0.5 <= |f| < 1, keep 8 bits of f with
    round-half-even, and use the fixed subnormal spacing below 2**-126.
    Values whose rounding reaches 2**128 become +-inf; NaN stays NaN.
    [MUON]: the optimizer's one state tensor is the momentum buffer; the
    buffer's storage type is a bf16 tensor in the GPT-2 workloads.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    finite = np.isfinite(x)
    out[~finite] = x[~finite]
    xf = x[finite]
    f, e = np.frexp(xf)                      # xf = f * 2**e, 0.5 <= |f| < 1
    normal = np.abs(xf) >= 2.0 ** -126
    r = np.empty_like(xf)
    # normal range: 8 significant bits -> f scaled to [128, 256)
    r[normal] = np.ldexp(np.rint(np.ldexp(f[normal], 8)), e[normal] - 8)
    # subnormal range: absolute spacing 2**-133
    r[~normal] = np.ldexp(np.rint(np.ldexp(xf[~normal], 133)), -133)
    r[np.abs(r) >= 2.0 ** 128] = np.copysign(np.inf, r[np.abs(r) >= 2.0 ** 128])
    out[finite] = r
    return out


def fp32_round(x) -> np.ndarray:
    """Round float64 values to the nearest float32 (numpy's IEEE cast)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


_ROUND = {"bf16": bf16_round, "fp32": fp32_round, "f64": lambda x: np.asarray(x, np.float64)}


def two_sum(a, b):
    """Error-free sum of two float64 arrays (Knuth's TwoSum): returns (s, e)
    with s = fl(a + b) and s + e == a + b exactly (round to nearest, no
    overflow)."""
    s = a + b
    bb = s - a
    e = (a - (s - bb)) + (b - bb)
    return s, e


def round_exact_sum(hi, lo, fmt: str) -> np.ndarray:
    """Round the exact real value hi + lo (an unevaluated float64 sum with
    hi = fl(hi + lo)) to the storage format ``fmt`` ("bf16" or "fp32"),
    round to nearest, ties to even.

    Every value and every halfway point of bf16 and fp32 is a float64, and
    rounding to float64 is monotone, so hi lies on the same side of each
    halfway point as hi + lo unless hi *is* a halfway point. Only then does
    lo decide: a positive lo moves the value above the halfway point, a
    negative one below it; lo == 0 is a true tie (ties to even).
    """
    rnd = _ROUND[fmt]
    hi = np.asarray(hi, dtype=np.float64)
    lo = np.asarray(lo, dtype=np.float64)
    r = rnd(hi)
    up = rnd(np.nextafter(hi, np.inf))
    down = rnd(np.nextafter(hi, -np.inf))
    tie = (up != down) & np.isfinite(hi) & (lo != 0)
    return np.where(tie, np.where(lo > 0, up, down), r)


# ---------------------------------------------------------------------------
# The update, step by step.
# ---------------------------------------------------------------------------

def momentum_update(g, buf, mu: float, nesterov: bool, buf_dtype: str = "bf16"):
    """Momentum step of the Muon update. Returns (u, new_buf).

    buf' = mu * buf + g, the exact real value rounded once to the buffer's
    storage dtype (round to nearest, ties to even); the vector that is
    orthogonalised is u = g + mu * buf' (Nesterov) or u = buf'.
    With mu == 0 (no momentum state) u = g and buf is ignored.
    [MUON]: Muon keeps a single momentum buffer per hidden matrix.

    For bf16 and fp32 state with a float32 mu the product mu * buf has at
    most 48 significant bits, so it is exact in float64; the sum with g is
    carried exactly as a float64 pair (two_sum) and rounded once.
    """
    g = np.asarray(g, dtype=np.float64)
    if mu == 0.0 or buf is None:
        return g.copy(), None
    buf = np.asarray(buf, dtype=np.float64)
    if buf_dtype in ("bf16", "fp32"):
        if float(np.float32(mu)) != float(mu):
            raise ValueError("mu must be a float32 value for bf16/fp32 state")
        hi, lo = two_sum(mu * buf, g)
        new_buf = round_exact_sum(hi, lo, buf_dtype)
    else:
        new_buf = mu * buf + g
    u = g + mu * new_buf if nesterov else new_buf.copy()
    return u, new_buf


def frobenius_normalize(u, eps: float):
    """X0 = u / (||u||_F + eps), ||u||_F = sqrt(sum of squares of all entries).

    The normalisation puts every singular value of X0 in [0, 1], the range on
    which the Newton-Schulz polynomial is designed to act ([MUON], [GREEN]).
    """
    u = np.asarray(u, dtype=np.float64)
    return u / (np.sqrt(np.sum(u * u)) + eps)


def ns_polynomial_step(x, a: float, b: float, c: float):
    """One Newton-Schulz step X <- a X + b (X X^T) X + c (X X^T)^2 X.

    Computed as A = X X^T, B = b A + c A A, X <- a X + B X (the same
    polynomial, grouped so that only m x m products are formed, m = rows).
    On singular values this maps sigma -> a sigma + b sigma^3 + c sigma^5
    and leaves the singular vectors unchanged ([MUON]: the iteration stands in
    for the SVD of spectral descent).
    """
    A = x @ x.T
    B = b * A + c * (A @ A)
    return a * x + B @ x


def newton_schulz(x0, a: float, b: float, c: float, steps: int):
    """k Newton-Schulz steps on X0, on the transpose when rows > cols.

    Working on the orientation with rows <= cols keeps the Gram matrix
    min(rows, cols) square; the result is transposed back, so the output has
    X0's shape ([MUON]).
    """
    x = np.asarray(x0, dtype=np.float64)
    tall = x.shape[0] > x.shape[1]
    if tall:
        x = x.T
    for _ in range(int(steps)):
        x = ns_polynomial_step(x, a, b, c)
    return x.T.copy() if tall else x.copy()


def orthogonalize(g, a: float, b: float, c: float, steps: int, eps: float = 1e-7):
    """Normalise then iterate, with no momentum state (u = g)."""
    return newton_schulz(frobenius_normalize(g, eps), a, b, c, steps)


def muon_update(g, buf, *, a: float, b: float, c: float, steps: int, mu: float,
                nesterov: bool, eps: float = 1e-7, buf_dtype: str = "bf16"):
    """The whole Muon update of one matrix. Returns (out, new_buf).

    out = NS_k( u / (||u||_F + eps) ) with u from ``momentum_update``.
    """
    u, new_buf = momentum_update(g, buf, mu, nesterov, buf_dtype)
    return newton_schulz(frobenius_normalize(u, eps), a, b, c, steps), new_buf


def apply_weight(w, x, *, lr: float, wd: float, lr_mul: float = 1.0, wd_mul: float = 1.0,
                 dtype: str = "bf16") -> np.ndarray:
    """Moves the weight against the orthogonalised update, with decoupled
    weight decay:  W' = W * (1 - lr' * wd') - lr' * X  where lr' = lr*lr_mul
    and wd' = wd*wd_mul, in float64, then stored at the weight's dtype (round
    to nearest even).

    Sources: mhpq.cn, modded-nanogpt track_1_short technical guide, section
    6.2 (training hyper-parameters): each parameter group has its own
    learning-rate and weight-decay multipliers (lr_mul, wd_mul);
    yongjin360.com, Modded-NanoGPT green-AI article, hyper-parameter
    paragraph: weight decay is part of the training recipe. The pages state
    neither the schedule nor the form of the decay; the plainest reading is
    the decoupled form above (the decay proportional to the effective rate,
    as in decoupled-decay Adam) with every scalar supplied by the caller.
    """
    w = np.asarray(w, dtype=np.float64)
    x = np.asarray(x, dtype=np.float64)
    lr_eff = float(lr) * float(lr_mul)
    wd_eff = float(wd) * float(wd_mul)
    res = w * (1.0 - lr_eff * wd_eff) - lr_eff * x
    if dtype == "bf16":
        return bf16_round(res)
    if dtype == "fp32":
        return fp32_round(res)
    return res


def adam_update(p, g, m, v, *, lr: float, beta1: float, beta2: float, eps: float, wd: float,
                step: int, lr_mul: float = 1.0, wd_mul: float = 1.0, dtype: str = "bf16"):
    """One Adam update of a parameter tensor off the Muon path, in float64.

    Source: mhpq.cn, modded-nanogpt track_1_short technical guide, section
    6.2 (training hyper-parameters): the parameter groups that are not
    projection matrices run Adam with betas (0.9, 0.99) and their own lr_mul,
    with wd_mul = 0 for biases and scales. The pages do not write Adam out;
    this is the textbook update with bias correction and decoupled weight
    decay, the multipliers scaling the rate and the decay:
        m <- beta1 m + (1 - beta1) g;   v <- beta2 v + (1 - beta2) g^2
        m_hat = m / (1 - beta1^t);      v_hat = v / (1 - beta2^t)
        p <- p (1 - lr' wd') - lr' m_hat / (sqrt(v_hat) + eps)
    with lr' = lr*lr_mul, wd' = wd*wd_mul and t = step (1-based). The moments
    are stored as float32 and p at its dtype (round to nearest even); those
    stored values are returned (p, m, v).
    """
    p = np.asarray(p, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    m = np.asarray(m, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    t = int(step)
    m_new = fp32_round(beta1 * m + (1.0 - beta1) * g)
    v_new = fp32_round(beta2 * v + (1.0 - beta2) * g * g)
    m_hat = m_new / (1.0 - beta1 ** t)
    v_hat = v_new / (1.0 - beta2 ** t)
    rate = float(lr) * float(lr_mul)
    decay = float(wd) * float(wd_mul)
    p_new = p * (1.0 - rate * decay) - rate * m_hat / (np.sqrt(v_hat) + eps)
    p_new = bf16_round(p_new) if dtype == "bf16" else fp32_round(p_new)
    return p_new, m_new, v_new


def falg_flops(rows: int, cols: int, steps: int) -> int:
    """Algorithmic flops of k steps on one matrix (m = min, n = max side):
    m(m+1)n for the symmetric Gram, m^2(m+1) for the symmetric A^2 and
    2 m^2 n for B X, per step. Used only to express oracle time as a rate."""
    m, n = min(rows, cols), max(rows, cols)
    return steps * (m * (m + 1) * n + m * m * (m + 1) + 2 * m * m * n)
