"""Plain fp64 CPU oracle of the LoGRA sketch hot path.

TEST INFRASTRUCTURE ONLY.  This module is the slow, obviously-correct
reference that the HIP library is checked against.  Only tests, the smoke
check and the benchmark's CPU-baseline leg may import it; the product path
never calls it and shares no code with it.

Sources (cited by page title and section):
  [paper]   "LoGRA: Scaling LLM Reinforcement Learning with Low-Rank Gradient
            Sketches", paper text on paperpeel.com.
  [zh]      Chinese review of the paper on shibing624.github.io
            (ai-paper-analysis), section "梯度速写怎么工作" and "Predicted-KL 步长控制".
  [ko]      Korean summary of the paper on onedev.kr, sections "어떻게 동작하나"
            and "무엇과 다른가".
  [rgc]     "Randomized Gradient Compression" blog (iluvatarlabs), section
            "How it works" -- a different method, used only for the
            orientation of the contraction and the meaning of stochastic
            rounding.
  [summary] paperlayer.ai section summary of the paper, "B. RowAdam" and
            "D.1 Main mathematical-reasoning experiments".

Arithmetic is fp64 on the exactly decoded bf16/fp32 inputs.  The merged
weight is formed in fp64 and rounded once, straight to the weight's type
(nearest-even, or stochastically with the fraction of the gap taken from the
fp64 value); the library forms it in fp32 first, which may move a result by
one bf16 unit where the value sits within fp32 rounding of a tie or a
stochastic threshold -- inside the merge's 1-ulp contract.

Parity status of every function is stated in its docstring; all are pinned by
the CPU tests except the placement of RowAdam's relative epsilon, whose
effect is below every tolerance ("parity unpinned" for that detail only).
"""
from __future__ import annotations

import math

import numpy as np

from . import philox

# ---------------------------------------------------------------------------
# bf16 / fp32 encodings (plain format definitions)
# ---------------------------------------------------------------------------


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Decode bf16 bit patterns (uint16) to fp64: a bf16 is the top half of an fp32."""
    u32 = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):  # a signalling NaN widens to a quiet NaN of its sign
        return u32.view(np.float32).astype(np.float64)


def f32_to_bf16_rne(x32: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 with round-to-nearest-even; returns uint16 bits.

    Truncating the fp32 pattern to its top 16 bits gives the bf16 value ``a``
    nearer to zero; ``b`` is the next bf16 away from zero.  The discarded
    16 bits are the distance to ``a`` in units of 2^-16 of the gap: above half
    picks ``b``, below half ``a``, exactly half picks the one with an even
    last bit.  NaN becomes a quiet NaN of the same sign.
    """
    u = np.asarray(x32, dtype=np.float32).view(np.uint32)
    hi = (u >> np.uint32(16)).astype(np.uint32)
    low = u & np.uint32(0xFFFF)
    up = (low > 0x8000) | ((low == 0x8000) & ((hi & np.uint32(1)) == 1))
    out = np.where(up, hi + np.uint32(1), hi)
    nan = np.isnan(np.asarray(x32, dtype=np.float32))
    out = np.where(nan, (hi & np.uint32(0x8000)) | np.uint32(0x7FC0), out)
    return out.astype(np.uint16)


def f32_to_bf16_stochastic(x32: np.ndarray, u: np.ndarray) -> np.ndarray:
    """Stochastic rounding of fp32 values to bf16 with 16-bit draws ``u``.

    [rgc] "How it works": a value a fraction f of the way across the gap
    between its two bf16 neighbours moves to the far neighbour with
    probability f.  With ``a`` the neighbour nearer zero, ``b`` the one
    away from zero and f = (|x| - |a|) / (|b| - |a|), the result is ``b``
    iff floor(f * 2^16) + u >= 2^16, else ``a``.  For an fp32 input,
    f * 2^16 is an integer, so the mean over all 2^16 draws is exactly x.
    Non-finite inputs are returned as their nearest-even rounding.
    """
    x = np.asarray(x32, dtype=np.float32)
    ubits = x.view(np.uint32)
    a_bits = ubits & np.uint32(0xFFFF0000)          # bf16 neighbour nearer zero
    b_bits = a_bits + np.uint32(0x10000)            # next bf16 magnitude, same sign
    a = a_bits.view(np.float32).astype(np.float64)
    ax = np.abs(x.astype(np.float64))
    with np.errstate(invalid="ignore", over="ignore", divide="ignore"):
        # bf16 spacing in the binade of x (8 significant bits; subnormal
        # spacing 2^-133).  Above the largest finite bf16 the far neighbour
        # is infinity and the spacing of the last binade is used.
        _, e = np.frexp(np.where(np.isfinite(ax), ax, 0.0))
        gap = np.ldexp(1.0, np.maximum(e - 1, -126) - 7)
        f = (ax - np.abs(a)) / gap
        fscaled = np.floor(f * 65536.0)
    take_b = (fscaled + np.asarray(u, dtype=np.float64)) >= 65536.0
    take_b &= np.isfinite(x)
    out = np.where(take_b, b_bits >> np.uint32(16), a_bits >> np.uint32(16)).astype(np.uint16)
    nonfinite = ~np.isfinite(x)
    return np.where(nonfinite, f32_to_bf16_rne(x), out).astype(np.uint16)


def ulp_bf16(x: np.ndarray) -> np.ndarray:
    """Spacing of consecutive bf16 values at |x|.

    bf16 keeps 8 significant bits, so in the binade [2^e, 2^(e+1)) (e >= -126)
    the spacing is 2^(e-7); below 2^-126 (subnormals, and zero) it is 2^-133.
    At a power of two the spacing above it, the larger one, is returned.  The
    binade is read with frexp, which is exact (a logarithm can round a value
    just below a power of two up into the next binade).  Non-finite inputs
    give NaN.
    """
    ax = np.abs(np.asarray(x, dtype=np.float64))
    finite = np.isfinite(ax)
    _, e = np.frexp(np.where(finite, ax, 0.0))      # ax = m 2^e, m in [0.5, 1)
    sp = np.ldexp(1.0, np.maximum(e - 1, -126) - 7)
    sp = np.where(ax < 2.0 ** -126, 2.0 ** -133, sp)
    return np.where(finite, sp, np.nan)


def _bf16_neighbours(x: np.ndarray):
    """For finite fp64 x: the bf16 bit patterns a (nearer zero) and b (next away from
    zero, infinity past the largest finite value) around x, and the fraction
    f = (|x| - |a|) / (|b| - |a|) of the gap, all exact in fp64."""
    ax = np.minimum(np.abs(x), 2.0 ** 128)         # at 2^128 and above: a = infinity
    gap = ulp_bf16(ax)
    a = np.floor(ax / gap) * gap                    # truncation to the bf16 grid (exact)
    f = np.where(ax < 2.0 ** 128, (ax - a) / gap, 0.0)
    with np.errstate(over="ignore"):
        a_mag = (a.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint32)
    sign = np.where(np.signbit(x), np.uint32(0x8000), np.uint32(0))
    a_bits = a_mag | sign
    b_bits = (a_mag + np.uint32(1)) | sign          # 0x7F7F + 1 = 0x7F80, infinity
    return a_bits, b_bits, f


def f64_to_bf16_rne(x64: np.ndarray) -> np.ndarray:
    """Round fp64 values to bf16 once, nearest with ties to even; uint16 bits.

    The result is the bf16 neighbour of x nearer to it; at exactly half the gap
    the neighbour whose last significand bit is 0.  Values from half a gap past
    the largest finite bf16 round to infinity; +-0 keep their sign; NaN gives a
    quiet NaN.
    """
    x = np.asarray(x64, dtype=np.float64)
    finite = np.isfinite(x)
    xf = np.where(finite, x, 0.0)
    a_bits, b_bits, f = _bf16_neighbours(xf)
    up = (f > 0.5) | ((f == 0.5) & ((a_bits & np.uint32(1)) == 1))
    out = np.where(up, b_bits, a_bits)
    inf_bits = np.where(np.signbit(x), np.uint32(0xFF80), np.uint32(0x7F80))
    nan_bits = np.where(np.signbit(x), np.uint32(0xFFC0), np.uint32(0x7FC0))
    out = np.where(np.isinf(x), inf_bits, out)
    out = np.where(np.isnan(x), nan_bits, out)
    return out.astype(np.uint16)


def f64_to_bf16_stochastic(x64: np.ndarray, u: np.ndarray) -> np.ndarray:
    """Stochastic rounding of fp64 values to bf16 with 16-bit draws ``u``; uint16 bits.

    [rgc] "How it works": the far neighbour b is taken with probability equal
    to the fraction f of the gap that x has crossed: b iff
    floor(f * 2^16) + u >= 2^16, else the neighbour a nearer zero.  f comes
    from the fp64 value itself.  Non-finite inputs round to nearest.
    """
    x = np.asarray(x64, dtype=np.float64)
    finite = np.isfinite(x)
    xf = np.where(finite, x, 0.0)
    a_bits, b_bits, f = _bf16_neighbours(xf)
    take_b = (np.floor(f * 65536.0) + np.asarray(u, dtype=np.float64)) >= 65536.0
    out = np.where(take_b, b_bits, a_bits).astype(np.uint16)
    return np.where(finite, out, f64_to_bf16_rne(x)).astype(np.uint16)


# ---------------------------------------------------------------------------
# Projection A (Rademacher, seed-regenerated)
# ---------------------------------------------------------------------------


def c_r(r: int) -> float:
    """Scale of the Rademacher entries, 1/sqrt(r) ([zh] and [ko]: entries +-1/sqrt(r);
    the paper's §3.4.1 prints "+-1/r" with the root lost in extraction)."""
    return 1.0 / math.sqrt(r)


def c_r_f32(r: int) -> np.float32:
    """1/sqrt(r) rounded once to fp32 (the scale the fp32 output of A carries)."""
    return np.float32(1.0 / math.sqrt(r))


def sigma(seed: int, matrix_id: int, step: int, r: int, k: int) -> np.ndarray:
    """Sign matrix sigma in {+1,-1}^{r x k} of projection (seed, matrix_id, step), int8.

    [paper] §2.2: each weight matrix has its own A, refreshed each update
    (fixed basis = keep ``step`` constant); §2.2 "Memory and synchronization":
    the rollout engine regenerates A from its seed.  Bit layout: oracle.philox.
    """
    bits = philox.sign_bits(seed, matrix_id, step, r, k)
    return (1 - 2 * bits.astype(np.int16)).astype(np.int8)


def regen_A(seed: int, matrix_id: int, step: int, r: int, k: int, kind: str = "f64"):
    """Materialise A [r x k].

    kind "i8": the signs sigma (int8); "f32": sigma * fl32(1/sqrt(r));
    "f64": sigma / sqrt(r) (used by the other oracle functions).
    [paper] §2.1 (A in R^{r x k}); [zh]/[ko] (+-1/sqrt(r) entries).
    """
    s = sigma(seed, matrix_id, step, r, k)
    if kind == "i8":
        return s
    if kind == "f32":
        return (s.astype(np.float32) * c_r_f32(r)).astype(np.float32)
    if kind == "f64":
        return s.astype(np.float64) * c_r(r)
    raise ValueError(kind)


def gaussian_A(seed: int, matrix_id: int, step: int, r: int, k: int, kind: str = "f64"):
    """Gaussian projection A [r x k] with entries z / sqrt(r), z standard normal
    (the variant the pages ablate against Rademacher signs: [paper] §3.4.1 and
    App. D.3; E[A^T A] = I as for the Rademacher A).  kind "f64" or "f32" (the
    fp64 value rounded once)."""
    a = philox.gaussian_normals(seed, matrix_id, step, r, k) / math.sqrt(r)
    if kind == "f64":
        return a
    if kind == "f32":
        return a.astype(np.float32)
    raise ValueError(kind)


# ---------------------------------------------------------------------------
# The sketch path
# ---------------------------------------------------------------------------


def project(X: np.ndarray, A: np.ndarray) -> np.ndarray:
    """Projected input X A^T [T x r].

    [paper] §2.1: the inputs of the weight-gradient product are projected
    before they meet the backward derivatives; [rgc] "How it works": the
    layer saves X P (here P = A^T) instead of X.
    """
    return np.asarray(X, np.float64) @ np.asarray(A, np.float64).T


def accumulate(S: np.ndarray, D: np.ndarray, XAt: np.ndarray) -> np.ndarray:
    """One microbatch of the sketch: S + D^T (X A^T) [d x r].

    [paper] §2.1: S = G A^T with G = D^T X the weight gradient (the sketch
    named Equation 2 there), accumulated microbatch by microbatch in fp32
    without forming G; [rgc] "How it works": C += D^T (X P).
    """
    return np.asarray(S, np.float64) + np.asarray(D, np.float64).T @ np.asarray(XAt, np.float64)


def dense_gradient(D: np.ndarray, X: np.ndarray) -> np.ndarray:
    """Dense weight gradient G = D^T X (only for brute-force checks, [paper] §2.1)."""
    return np.asarray(D, np.float64).T @ np.asarray(X, np.float64)


def reconstruct(S: np.ndarray, A: np.ndarray) -> np.ndarray:
    """Low-rank gradient estimate S A [d x k] ([paper] §2.1, 'A low-rank weight update')."""
    return np.asarray(S, np.float64) @ np.asarray(A, np.float64)


def reconstruction_cosine(G: np.ndarray, A: np.ndarray) -> float:
    """Frobenius cosine between G and (G A^T) A ([paper] App. D.3 'Reconstruction heatmaps')."""
    G = np.asarray(G, np.float64)
    Gh = (G @ A.T) @ A
    return float((G * Gh).sum() / (np.linalg.norm(G) * np.linalg.norm(Gh)))


def sketch_bytes(d: int, r: int) -> int:
    """fp32 storage of one sketch, 4*d*r bytes ([paper] §2.2 'Memory and synchronization')."""
    return 4 * d * r


# ---------------------------------------------------------------------------
# Sketch optimiser
# ---------------------------------------------------------------------------


def rowadam(S: np.ndarray, v: np.ndarray, t: int, beta: float, eps: float):
    """RowAdam: row-wise second-moment scaling of S into U, Frobenius norm restored.

    [summary] "B. RowAdam": each sketch row is scaled by a running estimate
    of its squared magnitude (no first moment), then the sketch's Frobenius
    norm is restored; the d row statistics persist across projection
    refreshes.  [paper] App. D.1 Table 4: beta2 = 0.95, no first moment,
    epsilon 1e-8 *relative*.  Reading taken where the pages are silent:

        m_i   = sum_j S_ij^2                       (row squared magnitude)
        v_i  <- beta v_i + (1 - beta) m_i          (v starts at 0; t = 1, 2, ...)
        vh_i  = v_i / (1 - beta^t)                 (Adam-style bias correction)
        rho   = sqrt(mean_i vh_i)                  (scale the relative eps refers to)
        Ut_ij = S_ij / (sqrt(vh_i) + eps * rho)
        U     = Ut * ||S||_F / ||Ut||_F            (U = 0 when Ut = 0)

    Bias correction and sum-vs-mean over a row are uniform factors that the
    norm restoration cancels exactly under a relative eps; only the eps
    placement is a free choice (parity unpinned for that detail: with
    eps = 1e-8 it moves U by ~1e-8 relative, far below the tolerance).
    Returns (U, v_new) in fp64.
    """
    if t < 1:
        raise ValueError("t counts updates from 1")
    S = np.asarray(S, np.float64)
    v = np.asarray(v, np.float64)
    m = (S * S).sum(axis=1)
    v_new = beta * v + (1.0 - beta) * m
    vh = v_new / (1.0 - beta ** t)
    rho = math.sqrt(vh.mean()) if vh.size else 0.0
    denom = np.sqrt(vh) + eps * rho
    with np.errstate(invalid="ignore", divide="ignore"):
        Ut = np.where(denom[:, None] > 0, S / np.where(denom > 0, denom, 1.0)[:, None], 0.0)
    nS = np.linalg.norm(S)
    nU = np.linalg.norm(Ut)
    U = Ut * (nS / nU) if nU > 0 else np.zeros_like(S)
    return U, v_new


# ---------------------------------------------------------------------------
# Predicted-KL step control
# ---------------------------------------------------------------------------


def _log_softmax(x: np.ndarray) -> np.ndarray:
    x = np.asarray(x, np.float64)
    m = x.max(axis=-1, keepdims=True)
    return x - m - np.log(np.exp(x - m).sum(axis=-1, keepdims=True))


def predicted_kl_q(z: np.ndarray, zdot: np.ndarray, tau: float) -> float:
    """q(D) = 1/(2|P| tau^2) * sum_s Var_{v ~ p(s)}[zdot_v(s)], p(s) = softmax(z(s)/tau).

    [paper] §2.3 (the coefficient named Equation 6 there) and App. A.1: the
    second derivative of the per-context KL along the update is the
    p-weighted variance of the logit change rates divided by tau^2, and the
    KL is half of it times alpha^2.  Computed per context with a centred
    two-pass variance.
    """
    z = np.asarray(z, np.float64)
    zdot = np.asarray(zdot, np.float64)
    P = z.shape[0]
    p = np.exp(_log_softmax(z / tau))
    mu = (p * zdot).sum(axis=1)
    var = (p * (zdot - mu[:, None]) ** 2).sum(axis=1)
    return float(var.sum() / (2.0 * P * tau * tau))


def exact_kl_mean(z: np.ndarray, zdot: np.ndarray, alpha: float, tau: float) -> float:
    """Mean over contexts of KL(softmax(z/tau) || softmax((z + alpha zdot)/tau)).

    [paper] §2.3 (average KL over the context set; Equation 5 approximates it
    by alpha^2 q) and App. A.1 (K_s(a) along the update, logits linear in a).
    """
    lp = _log_softmax(np.asarray(z, np.float64) / tau)
    lq = _log_softmax((np.asarray(z, np.float64) + alpha * np.asarray(zdot, np.float64)) / tau)
    # an entry of probability 0 (logit -inf, masked) adds 0 log 0 = 0 to the sum
    with np.errstate(invalid="ignore"):
        terms = np.where(np.isneginf(lp), 0.0, np.exp(lp) * (lp - lq))
    return float(terms.sum(axis=1).mean())


def step_alpha(q: float, delta: float, alpha_max: float) -> float:
    """alpha = min(alpha_max, sqrt(delta / q)).

    [paper] §2.3 and App. A.2 print delta/q with the root lost; the root is
    restored from the requirement alpha^2 q <= delta ([paper] §2.3), [zh]
    and [ko] (which also state q = 4 delta gives half the step).  q = 0 gives
    alpha_max (the limit); negative or NaN q, delta <= 0 or alpha_max <= 0
    are errors.
    """
    if not (delta > 0) or not (alpha_max > 0):
        raise ValueError("delta and alpha_max must be positive")
    if math.isnan(q) or q < 0:
        raise ValueError("q must be >= 0")
    if q == 0:
        return float(alpha_max)
    return float(min(alpha_max, math.sqrt(delta / q)))


# ---------------------------------------------------------------------------
# Merge
# ---------------------------------------------------------------------------


def merge(W: np.ndarray, U: np.ndarray, A: np.ndarray, scale: float, *,
          w_dtype: str, mode: str = "nearest", u_draws: np.ndarray | None = None):
    """In-place merge W <- round(W - scale * U A).

    [paper] §2.1 (W <- W - alpha eta U A, "Equation 4" position) and §2.2
    (merged into the weights, no adapter branch); §2.2 "Memory and
    synchronization": the rollout side applies the received alpha*eta*U with
    A regenerated from its seed (scale = 1 there).  [rgc] "How it works":
    bf16 weights kept without an fp32 copy, updated with stochastic rounding.

    The updated weight is formed in fp64 and rounded once, straight to the
    weight's type: to fp32 (nearest) for ``w_dtype == "f32"``, to bf16
    nearest-even or stochastically with ``u_draws`` for ``"bf16"``.
    ``W`` holds the decoded weights (fp64); the result is fp32 values for
    ``"f32"`` and uint16 bf16 bits for ``"bf16"``.
    """
    x64 = np.asarray(W, np.float64) - float(scale) * (np.asarray(U, np.float64) @ np.asarray(A, np.float64))
    if w_dtype == "f32":
        if mode != "nearest":
            raise ValueError("stochastic rounding is defined for bf16 weights only")
        return x64.astype(np.float32)
    if w_dtype != "bf16":
        raise ValueError(w_dtype)
    if mode == "nearest":
        return f64_to_bf16_rne(x64)
    if mode == "stochastic":
        if u_draws is None:
            raise ValueError("stochastic rounding needs draws")
        return f64_to_bf16_stochastic(x64, u_draws)
    raise ValueError(mode)


# ---------------------------------------------------------------------------
# KL budget schedule (the scalar steps either side of alpha)
# ---------------------------------------------------------------------------


def kl_budget(u: int, H: int, delta_max: float, delta_min: float) -> float:
    """Cosine-annealed budget delta_u for update u = 1, 2, ... ([paper] App. D.1 'KL budget').

    delta_u = delta_min + (delta_max - delta_min)/2 * (1 + cos(pi (u-1)/(H-1)))
    for u <= H, held at delta_min afterwards ([paper] App. D.2: annealed over
    the horizon, then held constant).
    """
    if u < 1 or H < 2:
        raise ValueError("u >= 1 and H >= 2")
    if u >= H:
        return float(delta_min)
    return float(delta_min + 0.5 * (delta_max - delta_min) * (1.0 + math.cos(math.pi * (u - 1) / (H - 1))))


def mismatch_ema(kappa_prev, measurement, weight: float = 0.3):
    """Smoothed rollout-vs-trainer log-prob mismatch ([summary] D.1).

    The new measurement enters with ``weight``; the estimate is clamped at 0;
    with no valid measurement (None or NaN) the previous estimate is kept.
    Returns None until a first valid measurement exists.
    """
    if measurement is None or (isinstance(measurement, float) and math.isnan(measurement)):
        return kappa_prev
    m = float(measurement)
    k = m if kappa_prev is None else weight * m + (1.0 - weight) * float(kappa_prev)
    return max(0.0, k)


def effective_budget(delta_u: float, kappa) -> float:
    """delta_eff = max(delta_u - kappa, 0.5 delta_u); no subtraction without kappa
    ([paper] App. D.1, budget floor 50% in Table 4; [summary] D.1)."""
    if kappa is None:
        return float(delta_u)
    return float(max(delta_u - float(kappa), 0.5 * delta_u))
