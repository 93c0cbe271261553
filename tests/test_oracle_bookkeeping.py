"""Pins of the oracle's elementwise bookkeeping (CPU only): momentum and the
Nesterov input against torch's SGD, AdamW against torch's AdamW, bfloat16
rounding against torch's conversion, and the decay + update against exact
dyadic arithmetic and the singular-value closed form of a full step."""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle import adamw_step_f32, apply_update_f32, bf16_round_f32, nesterov_momentum_f32


def _rng(seed):
    return np.random.default_rng(seed)


# ------------------------------------------------------------------------- bfloat16


def test_bf16_rounding_matches_torch():
    r = _rng(1)
    x = np.concatenate([
        r.standard_normal(20000).astype(np.float32) * np.float32(3.0),
        (r.standard_normal(2000) * 1e-39).astype(np.float32),      # subnormals
        np.array([0.0, -0.0, np.inf, -np.inf, 3.4e38, -3.4e38, 1e-45], np.float32),
    ])
    # exact ties: low half == 0x8000 with even and odd kept parts
    ties = (np.arange(0x3F800000, 0x3F800000 + 64 * 0x10000, 0x10000, dtype=np.uint32)
            | np.uint32(0x8000)).view(np.float32)
    x = np.concatenate([x, ties])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    got = bf16_round_f32(x)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    assert np.all(np.isnan(bf16_round_f32(np.array([np.nan], np.float32))))


# ------------------------------------------------------------------ momentum + Nesterov


@pytest.mark.parametrize("nesterov", [True, False])
def test_momentum_matches_torch_sgd_float64(nesterov):
    """M_t = mu M + G and N_t = mu M_t + G equal torch SGD's momentum buffer and
    its Nesterov direction (dampening 0)."""
    r = _rng(2)
    shape = (33, 65)
    m0 = r.standard_normal(shape)
    g = r.standard_normal(shape)
    p = torch.zeros(shape, dtype=torch.float64, requires_grad=True)
    opt = torch.optim.SGD([p], lr=1.0, momentum=0.95, dampening=0.0, nesterov=nesterov)
    opt.state[p]["momentum_buffer"] = torch.from_numpy(m0.copy())
    p.grad = torch.from_numpy(g.copy())
    opt.step()
    ref_m = opt.state[p]["momentum_buffer"].numpy()
    ref_n = -p.detach().numpy()          # p was 0 and lr 1, so p = -direction
    # oracle in float64 arithmetic: feed float64 through the same formulas
    mu = 0.95
    m_new = mu * m0 + g
    n = mu * m_new + g if nesterov else m_new
    assert np.allclose(ref_m, m_new, rtol=0, atol=1e-15)
    assert np.allclose(ref_n, n, rtol=0, atol=1e-15)
    # and the float32 oracle agrees with torch's float32 run to one ulp
    m32, n32 = nesterov_momentum_f32(m0.astype(np.float32), g.astype(np.float32), mu, nesterov)
    p32 = torch.zeros(shape, dtype=torch.float32, requires_grad=True)
    opt32 = torch.optim.SGD([p32], lr=1.0, momentum=0.95, dampening=0.0, nesterov=nesterov)
    opt32.state[p32]["momentum_buffer"] = torch.from_numpy(m0.astype(np.float32))
    p32.grad = torch.from_numpy(g.astype(np.float32))
    opt32.step()
    ulp = np.spacing(np.abs(m32)).astype(np.float64)
    assert np.all(np.abs(opt32.state[p32]["momentum_buffer"].numpy() - m32) <= ulp)
    # torch may fuse g + mu*buf into one rounding; both results lie within half an ulp
    # of the result plus half an ulp of the product of the exact value.
    big = np.abs(np.float32(mu) * m32)
    tol = (np.spacing(np.abs(n32)) + np.spacing(big)).astype(np.float64)
    assert np.all(np.abs(-p32.detach().numpy() - n32) <= tol)


def test_nesterov_expansion_identity():
    """mu (mu M + G) + G = (1 + mu) G + mu^2 M (the deep-dive page, Nesterov step)."""
    r = _rng(3)
    m0, g = r.standard_normal((7, 9)), r.standard_normal((7, 9))
    mu = 0.95
    lhs = mu * (mu * m0 + g) + g
    rhs = (1 + mu) * g + mu ** 2 * m0
    assert np.allclose(lhs, rhs, rtol=1e-14, atol=1e-15)
    # The float32 oracle follows the two-step form with the single buffer M_t.
    m32, n32 = nesterov_momentum_f32(m0.astype(np.float32), g.astype(np.float32), mu)
    assert np.allclose(n32, rhs, rtol=1e-5, atol=1e-6)


def test_momentum_exact_dyadic():
    # mu = 0.5 and dyadic inputs: every float32 op is exact
    m0 = np.array([[1.0, -2.0], [0.25, 0.0]], np.float32)
    g = np.array([[0.5, 0.5], [-1.0, 3.0]], np.float32)
    m1, n1 = nesterov_momentum_f32(m0, g, 0.5)
    assert np.array_equal(m1, np.array([[1.0, -0.5], [-0.875, 3.0]], np.float32))
    assert np.array_equal(n1, np.array([[1.0, 0.25], [-1.4375, 4.5]], np.float32))


# -------------------------------------------------------------------- decay + update


def test_update_exact_dyadic():
    """W' = (1 - lr wd) W - lr gamma sqrt(max(n,m)) X with values where float32 is exact."""
    r = _rng(4)
    w = (r.integers(-64, 64, (16, 16)) / 64.0).astype(np.float32)
    x = (r.integers(-64, 64, (16, 16)) / 64.0).astype(np.float32)
    lr, wd, gamma = 0.5, 0.5, 0.25                    # d = 0.75, s = 0.5*0.25*4 = 0.5
    got = apply_update_f32(w, x, lr, wd, gamma, param_bf16=False)
    assert np.array_equal(got, (0.75 * w.astype(np.float64) - 0.5 * x).astype(np.float32))
    d, s = oracle.muon_scalars_f32(lr, wd, gamma, 16, 16)
    assert d == np.float32(0.75) and s == np.float32(0.5)


def test_update_scalars_use_max_side():
    d, s = oracle.muon_scalars_f32(0.02, 0.1, 0.2, 2048, 7168)
    assert s == np.float32(0.02 * 0.2 * math.sqrt(7168.0))
    assert d == np.float32(1.0 - 0.002)
    d2, s2 = oracle.muon_scalars_f32(0.02, 0.1, 0.2, 7168, 2048)
    assert (d, s) == (d2, s2)


def test_update_bf16_param_rounds_once():
    r = _rng(5)
    w = bf16_round_f32((r.standard_normal((8, 24)) * 0.02).astype(np.float32))
    x = r.standard_normal((8, 24)).astype(np.float32)
    got = apply_update_f32(w, x, 0.02, 0.1, 0.2, param_bf16=True)
    d, s = oracle.muon_scalars_f32(0.02, 0.1, 0.2, 8, 24)
    f32 = (d * w) - (s * x)
    ref = torch.from_numpy(f32).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(got, ref)


def test_full_step_closed_form():
    """W_t = (1 - lr wd) W - lr gamma sqrt(l) U f(sigma/||N||) V^T with N = mu M_t + G."""
    r = _rng(6)
    rows, cols = 12, 20
    w = (r.standard_normal((rows, cols)) * 0.02).astype(np.float32)
    g = r.standard_normal((rows, cols)).astype(np.float32)
    m0 = r.standard_normal((rows, cols)).astype(np.float32)
    res = oracle.muon_step(w, g, m0, lr=0.02, momentum=0.95, weight_decay=0.1, gamma=0.2)
    u, s, vt = np.linalg.svd(res["n"].astype(np.float64), full_matrices=False)
    xs = s / math.sqrt(float(np.sum(s * s)))
    for a, b, c in oracle.DEEPSEEK_V4_SCHEDULE:
        xs = a * xs + b * xs ** 3 + c * xs ** 5
    o_ref = (u * xs) @ vt * (math.sqrt(cols) * 0.2)
    assert np.linalg.norm(res["o"] - o_ref) <= 1e-11 * np.linalg.norm(o_ref)
    w_ref = (1 - 0.02 * 0.1) * w.astype(np.float64) - 0.02 * o_ref
    assert np.max(np.abs(res["w_new"] - w_ref)) < 1e-7


def test_zero_gradient_is_decay_only():
    w = (_rng(7).standard_normal((5, 9)) * 0.02).astype(np.float32)
    z = np.zeros((5, 9), np.float32)
    res = oracle.muon_step(w, z, z)
    assert not np.any(res["x"])
    d, _ = oracle.muon_scalars_f32(0.02, 0.1, 0.2, 5, 9)
    assert np.array_equal(res["w_new"], (d * w).astype(np.float32))


# ------------------------------------------------------------------------------ AdamW


def _torch_adamw(p, g, m, v, step, lr, b1, b2, eps, wd, dtype):
    t = torch.tensor(p, dtype=dtype, requires_grad=True)
    opt = torch.optim.AdamW([t], lr=lr, betas=(b1, b2), eps=eps, weight_decay=wd)
    if step > 1:
        st = opt.state[t]
        st["step"] = torch.tensor(float(step - 1))
        st["exp_avg"] = torch.tensor(m, dtype=dtype)
        st["exp_avg_sq"] = torch.tensor(v, dtype=dtype)
    t.grad = torch.tensor(g, dtype=dtype)
    opt.step()
    st = opt.state[t]
    return t.detach().numpy(), st["exp_avg"].numpy(), st["exp_avg_sq"].numpy()


@pytest.mark.parametrize("step", [1, 2, 10])
def test_adamw_matches_torch_float64(step):
    r = _rng(10 + step)
    n = 4096
    p = (r.standard_normal(n) * 0.02).astype(np.float32)
    g = r.standard_normal(n).astype(np.float32)
    if step == 1:
        m = np.zeros(n, np.float32)
        v = np.zeros(n, np.float32)
    else:
        m = (r.standard_normal(n) * 0.1).astype(np.float32)
        v = (np.abs(r.standard_normal(n)) * 1e-2).astype(np.float32)
    hp = dict(lr=0.02, b1=0.9, b2=0.95, eps=1e-8, wd=0.1)
    ref_p, ref_m, ref_v = _torch_adamw(p.astype(np.float64), g.astype(np.float64),
                                       m.astype(np.float64), v.astype(np.float64), step,
                                       dtype=torch.float64, **hp)
    got_p, got_m, got_v = adamw_step_f32(p, g, m, v, 0.02, 0.9, 0.95, 1e-8, 0.1, step)
    # float32 rounding bound: a few units of 2^-24 of the magnitudes that are summed
    eps = 2.0 ** -24
    m64, v64, g64 = m.astype(np.float64), v.astype(np.float64), g.astype(np.float64)
    assert np.all(np.abs(got_m - ref_m) <= 4 * eps * (0.9 * np.abs(m64) + 0.1 * np.abs(g64)))
    assert np.all(np.abs(got_v - ref_v) <= 4 * eps * (0.95 * v64 + 0.05 * g64 * g64))
    m_mag = (0.9 * np.abs(m64) + 0.1 * np.abs(g64)) / (1 - 0.9 ** step)
    step_mag = 0.02 * m_mag / (np.sqrt(ref_v / (1 - 0.95 ** step)) + 1e-8)
    assert np.all(np.abs(got_p - ref_p) <= 8 * eps * (np.abs(p) + step_mag))
    # and the formula itself: a wrong bias correction or decay would be off by >> that
    assert np.max(np.abs(got_p - ref_p)) < 1e-7


def test_adamw_first_step_is_sign_step():
    """At t = 1 the bias-corrected ratio is g / (|g| + eps): a signed lr step."""
    g = np.array([1.0, -2.0, 0.5, -0.25], np.float32)
    p = np.zeros(4, np.float32)
    z = np.zeros(4, np.float32)
    got_p, _, _ = adamw_step_f32(p, g, z, z, 0.01, 0.9, 0.95, 1e-8, 0.0, 1)
    assert np.allclose(got_p, -0.01 * np.sign(g), rtol=1e-6)


def test_adamw_rejects_step_zero():
    z = np.zeros(2, np.float32)
    with pytest.raises(ValueError):
        adamw_step_f32(z, z, z, z, 0.01, 0.9, 0.95, 1e-8, 0.1, 0)
