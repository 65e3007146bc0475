"""Per-block denoising update, fp64 (oracle).

Block-wise denoising ("Minute-Long Videos with Dual Parallelisms", Abstract)
keeps the queued blocks at progressively decreasing noise levels; per the
pith.science verdict (pith_extraction.key_machinery) each step moves every
queued block one level down, each block at its own timestep.  The pages name
the schedule family only by the titles they build on, so the update is the
plain reading: an epsilon-prediction DDIM step (eta = 0) on the DDPM linear
beta schedule, restated from those published methods:

  beta_s    = beta_start + (beta_end - beta_start) * (s - 1) / (T - 1),  s = 1..T
  abar_t    = prod_{s <= t} (1 - beta_s),  abar_0 = 1
  t'        = max(t - stride, 0)
  x0_hat    = (x - sqrt(1 - abar_t) * eps) / sqrt(abar_t)
  x'        = sqrt(abar_t') * x0_hat + sqrt(1 - abar_t') * eps

The result is rounded to bf16 once, from fp64, at the very end.

Variant: velocity-prediction flow matching.  The generator the DualParal page
evaluates on (Wan2.1) is a flow-matching model, and the pages name that family
only through titles ("... Guidance for Flow Matching Models", "... Velocity
for Accelerating Flow Matching Inference").  The plain reading is rectified
flow: x_sigma = (1 - sigma) x0 + sigma eps, velocity v = eps - x0, and one
Euler step of the probability-flow ODE,

  u         = t / T,  sigma(t) = shift * u / (1 + (shift - 1) * u)
  x'        = x + (sigma(t') - sigma(t)) * v

(shift = 1 gives the linear schedule; a shift > 1 spends more steps at high
noise, the time shift of published flow-matching samplers).
"""
import numpy as np

from .numerics import f64_to_bf16_bits, bf16_bits_to_f64

DEFAULT = dict(T=1000, beta_start=1e-4, beta_end=0.02, stride=20)


def betas(T, beta_start, beta_end):
    """beta_1 .. beta_T, evenly spaced (index 0 holds beta_1)."""
    return np.linspace(beta_start, beta_end, T, dtype=np.float64)


def alpha_bar(T, beta_start, beta_end):
    """abar_0 .. abar_T (index t holds abar_t; abar_0 = 1)."""
    ab = np.ones(T + 1)
    acc = 1.0
    b = betas(T, beta_start, beta_end)
    for s in range(1, T + 1):
        acc *= 1.0 - b[s - 1]
        ab[s] = acc
    return ab


def prev_timestep(t, stride):
    return max(int(t) - int(stride), 0)


def ddim_step(x, eps, t, t_prev, ab):
    """One deterministic DDIM step from t to t_prev (fp64 in, fp64 out)."""
    x = np.asarray(x, dtype=np.float64)
    eps = np.asarray(eps, dtype=np.float64)
    a_t, a_p = ab[t], ab[t_prev]
    x0 = (x - np.sqrt(1.0 - a_t) * eps) / np.sqrt(a_t)
    return np.sqrt(a_p) * x0 + np.sqrt(1.0 - a_p) * eps


def ddim_coefficients(t, t_prev, ab):
    """(c1, c2) with x' = c1 x + c2 eps, the same step folded into two numbers."""
    a_t, a_p = ab[t], ab[t_prev]
    c1 = np.sqrt(a_p / a_t)
    c2 = np.sqrt(1.0 - a_p) - np.sqrt(a_p) * np.sqrt(1.0 - a_t) / np.sqrt(a_t)
    return c1, c2


def flow_sigma(t, T, shift=1.0):
    """Noise level of timestep t under the (shifted) linear flow schedule."""
    u = float(t) / float(T)
    return shift * u / (1.0 + (shift - 1.0) * u)


def flow_step(x, v, t, t_prev, T, shift=1.0):
    """One Euler step of the flow from t to t_prev (fp64 in, fp64 out)."""
    x = np.asarray(x, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    return x + (flow_sigma(t_prev, T, shift) - flow_sigma(t, T, shift)) * v


def flow_coefficients(t, t_prev, T, shift=1.0):
    """(c1, c2) with x' = c1 x + c2 v."""
    return 1.0, flow_sigma(t_prev, T, shift) - flow_sigma(t, T, shift)


def block_update_ref(x_bits, eps_bits, t_per_block, T=1000, beta_start=1e-4,
                     beta_end=0.02, stride=20, kind="ddim", shift=1.0):
    """x_bits, eps_bits: [n_blocks][elems] bf16 patterns -> updated bf16 patterns.
    kind "ddim": eps_bits is the predicted noise; "flow": the predicted velocity."""
    x = bf16_bits_to_f64(x_bits)
    e = bf16_bits_to_f64(eps_bits)
    out = np.empty(np.shape(x_bits), dtype=np.uint16)
    ab = alpha_bar(T, beta_start, beta_end) if kind == "ddim" else None
    for b, t in enumerate(t_per_block):
        tp = prev_timestep(t, stride)
        if kind == "ddim":
            y = ddim_step(x[b], e[b], int(t), tp, ab)
        elif kind == "flow":
            y = flow_step(x[b], e[b], int(t), tp, T, shift)
        else:
            raise ValueError(kind)
        out[b] = f64_to_bf16_bits(y)
    return out
