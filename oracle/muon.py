"""Oracle for one Muon step on one weight matrix (test infrastructure only).

Follows the DeepSeek-V4 Algorithm 1 as printed on the deep-dive page
("V4 的完整更新公式，逐行拆解") and as expanded in the DeepSeek-V4 book,
ch. 6, §5 (which writes the Frobenius normalisation and the two-stage
Newton–Schulz loop out explicitly).  For each independent weight W (n x m)
with gradient G and momentum buffer M:

    M_t = mu * M_{t-1} + G_t                 momentum accumulate
    N_t = mu * M_t + G_t                     Nesterov look-ahead (one buffer)
    X   = N_t / ||N_t||_F                    normalise into the NS domain
    repeat 8x with (3.4445, -4.7750, 2.0315), then 2x with (2, -1.5, 0.5):
        X = a X + b (X X^T) X + c (X X^T)^2 X
    O_t = X * sqrt(max(n, m)) * gamma        rescale the update RMS
    W_t = (1 - lr * wd) W_{t-1} - lr * O_t   decoupled decay + update

Readings taken where the pages leave a step open (each is listed with its
reason in the design notes of the repository):

* The Gram matrix is formed on the smaller side: if n > m the iteration runs
  on N^T and the result is transposed back (the deep-dive page's cost formula
  in "收益与代价" assumes m <= n).  For n == m no transpose is taken.
* ||N||_F == 0 gives X = 0, i.e. a decay-only update (no epsilon is printed).
* The three-term polynomial is evaluated as (a I + b A + c A A) X with
  A = X X^T; that is the printed expression with (X X^T)^2 X written as
  (A A) X and the common right factor X taken out.
* Momentum and the Nesterov input are float32 with one rounding per
  operation, in the order the formulas are written; the decay and update
  given an float32 X use d = fl32(1 - lr*wd) and s = fl32(lr*gamma*sqrt(max))
  computed in float64 and rounded once.
"""

import math

import numpy as np

from .bf16 import bf16_round_f32

_AGGRESSIVE = (3.4445, -4.7750, 2.0315)
_STANDARD = (2.0, -1.5, 0.5)

# Hybrid two-stage schedule: 8 aggressive steps, then 2 standard steps
# (DeepSeek-V4 book ch. 6, §4 and §5; the deep-dive page's description of
# the "deepseekv4" coefficient set in the Megatron-Bridge section).
DEEPSEEK_V4_SCHEDULE = (_AGGRESSIVE,) * 8 + (_STANDARD,) * 2

# Five-step quintic schedule with the aggressive coefficients (the deep-dive
# page, "系数怎么调出来的" and the "quintic" recipe, muon_num_ns_steps=5).
QUINTIC5_SCHEDULE = (_AGGRESSIVE,) * 5


def nesterov_momentum_f32(m, g, mu, nesterov=True):
    """Momentum accumulate and Nesterov input in float32.

    m: previous momentum buffer (float32); g: gradient (float32 or the float32
    widening of a bfloat16 gradient).  Returns (M_t, N_t).  With
    nesterov=False the NS input is M_t itself ("momentum before
    orthogonalisation", deep-dive page, "Muon 的定义").
    """
    m = np.asarray(m, dtype=np.float32)
    g = np.asarray(g, dtype=np.float32)
    muf = np.float32(mu)
    m_new = (muf * m) + g
    if nesterov:
        n = (muf * m_new) + g
    else:
        n = m_new.copy()
    return m_new.astype(np.float32), n.astype(np.float32)


def newton_schulz(n_mat, schedule=DEEPSEEK_V4_SCHEDULE):
    """Normalise by the Frobenius norm and run the NS quintic iterations.

    float64 throughout.  Returns O'_t (same shape as n_mat), whose singular
    values approach 1 (DeepSeek-V4 book ch. 6, §3 and §5 lines 8-14 of its
    expanded algorithm).
    """
    x = np.array(n_mat, dtype=np.float64)
    transposed = x.shape[0] > x.shape[1]
    if transposed:
        x = x.T.copy()
    nrm = math.sqrt(float(np.sum(x * x)))
    if nrm == 0.0:
        out = np.zeros_like(x)
        return out.T.copy() if transposed else out
    x = x / nrm
    for a, b, c in schedule:
        gram = x @ x.T
        poly = b * gram + c * (gram @ gram)
        x = a * x + poly @ x
    return x.T.copy() if transposed else x


def orthogonalized_update(n_mat, gamma, schedule=DEEPSEEK_V4_SCHEDULE):
    """O_t = NS(N_t) * sqrt(max(n, m)) * gamma, in float64."""
    rows, cols = np.shape(n_mat)
    return newton_schulz(n_mat, schedule) * (math.sqrt(max(rows, cols)) * gamma)


def unit_rms_factor(x, gamma):
    """Scale of the unit-RMS mode: O = X * gamma / RMS(X), RMS(X) = ||X||_F / sqrt(n m).

    The deep-dive page's Megatron-Bridge recipe (muon_scale_mode
    "unit_rms_norm" with muon_extra_scale_factor 0.2, and the remark below it
    that contrasts it with V4's sqrt(max) rule) divides the update by its own
    RMS and multiplies by the extra factor; gamma plays that factor here.
    X = 0 has no RMS to divide by: the factor is 0 (a decay-only update, as
    for ||N|| = 0).  Computed in float64 from the values given.
    """
    x = np.asarray(x, dtype=np.float64)
    rows, cols = x.shape
    ss = float(np.sum(x * x))
    if ss == 0.0:
        return 0.0
    return gamma * math.sqrt(float(rows) * float(cols)) / math.sqrt(ss)


def update_scale(x, gamma, scale_mode="sqrt_max"):
    """The factor O_t / O'_t: sqrt(max(n, m)) * gamma (V4, Algorithm 1) or the
    unit-RMS factor of `unit_rms_factor`."""
    rows, cols = np.shape(x)
    if scale_mode == "sqrt_max":
        return math.sqrt(max(rows, cols)) * gamma
    if scale_mode == "unit_rms":
        return unit_rms_factor(x, gamma)
    raise ValueError(f"unknown scale mode {scale_mode!r}")


def muon_scalars_f32(lr, weight_decay, gamma, rows, cols, x32=None, scale_mode="sqrt_max"):
    """Host scalars of the decay + update: (d, s) as float32.

    d = 1 - lr*wd and s = lr * gamma * sqrt(max(rows, cols)) (unit-RMS mode:
    s = lr * unit_rms_factor(x32, gamma), which needs the float32 X), each
    computed in float64 and rounded once to float32.
    """
    d = np.float32(1.0 - lr * weight_decay)
    if scale_mode == "unit_rms":
        s = np.float32(lr * unit_rms_factor(x32, gamma))
    else:
        s = np.float32(lr * gamma * math.sqrt(float(max(rows, cols))))
    return d, s


def apply_update_f32(w, x32, lr, weight_decay, gamma, param_bf16, scale_mode="sqrt_max"):
    """W_t = (1 - lr*wd) W_{t-1} - lr * scale * X, float32 ops.

    w: parameter values as float32 (bfloat16 values widened exactly when
    param_bf16).  x32: the float32 orthogonalised update O'_t (unscaled).
    scale = sqrt(max) * gamma, or gamma / RMS(x32) in the unit-RMS mode.
    Computes fl(fl(d*w) - fl(s*x)); rounds the result to bfloat16 (RNE) when
    the parameter is bfloat16.
    """
    w = np.asarray(w, dtype=np.float32)
    x32 = np.asarray(x32, dtype=np.float32)
    rows, cols = w.shape
    d, s = muon_scalars_f32(lr, weight_decay, gamma, rows, cols, x32, scale_mode)
    return apply_update_ds_f32(w, x32, d, s, param_bf16)


def apply_update_ds_f32(w, x32, d, s, param_bf16):
    """fl(fl(d*w) - fl(s*x)) in float32 for given float32 scalars d and s, rounded
    to bfloat16 (RNE) when the parameter is bfloat16 (the decay + update step of
    Algorithm 1 with its scalars already formed)."""
    w = np.asarray(w, dtype=np.float32)
    x32 = np.asarray(x32, dtype=np.float32)
    d, s = np.float32(d), np.float32(s)
    out = (d * w) - (s * x32)
    out = out.astype(np.float32)
    if param_bf16:
        out = bf16_round_f32(out)
    return out


def muon_step(w, g, m, lr=0.02, momentum=0.95, weight_decay=0.1, gamma=0.2,
              nesterov=True, schedule=DEEPSEEK_V4_SCHEDULE, param_bf16=False, scale_mode="sqrt_max"):
    """One full Muon step on one matrix.

    Returns a dict with
      m_new : float32 M_t (bit-exact target)
      n     : float32 N_t (the NS input)
      x     : float64 O'_t (NS output, unscaled)
      o     : float64 O_t = O'_t * scale (the parity object); scale is
              sqrt(max) * gamma, or gamma / RMS(O'_t) when scale_mode is
              "unit_rms"
      w_new : float32 W_t computed from fl32(O'_t) (bfloat16-rounded if the
              parameter is bfloat16)
    """
    m_new, n = nesterov_momentum_f32(m, g, momentum, nesterov)
    x = newton_schulz(n, schedule)
    rows, cols = np.shape(w)
    o = x * update_scale(x, gamma, scale_mode)
    w_new = apply_update_f32(w, x.astype(np.float32), lr, weight_decay, gamma, param_bf16, scale_mode)
    return {"m_new": m_new, "n": n, "x": x, "o": o, "w_new": w_new}


def ns_flops_dense(rows, cols, steps):
    """NS FLOPs by the deep-dive page's count 2(2 n m^2 + m^3) per step, m <= n."""
    big, small = max(rows, cols), min(rows, cols)
    return steps * 2 * (2 * big * small * small + small ** 3)


def ns_flops_algorithmic(rows, cols, steps):
    """FLOPs the method must do per matrix, using the symmetry of A and A^2.

    Per step: X X^T needs only one triangle (l * s * (s+1) FLOPs), A A only
    one triangle (s^2 * (s+1)), and (aI + bA + cA^2) X is a full s x s by
    s x l product (2 s^2 l).
    """
    big, small = max(rows, cols), min(rows, cols)
    return steps * (big * small * (small + 1) + small * small * (small + 1)
                    + 2 * small * small * big)
