"""Pins for the oracle's gate activation (no GPU).

g = -exp(A_log) * softplus(x + dt_bias) and beta = sigmoid(b) (GDN pool-mode
digest, sglang PR 30169, key-code test; KDA prefill digest, sglang PR 27488,
extend wrapper taking A_log and dt_bias).  The pins tie the fp64 activation to
library routines (numpy's logaddexp, scipy's expit), to the closed form the
pages' own parameter recipe implies (dt_bias is the inverse softplus of dt, so
a zero raw input gives g = -A dt), and to invariants, and check that a wrong
activation (sign, a missing exp on A_log, a missing dt_bias, the channel and
head axes swapped) fails at least one of them.
"""
import math

import numpy as np
import pytest
import scipy.special
import torch

import kda_workloads as W


def test_softplus_matches_logaddexp(oracle):
    """softplus(z) = log(e^0 + e^z), numpy's logaddexp(0, z)."""
    z = np.concatenate([np.linspace(-80.0, 80.0, 4001), [-745.0, -1e-300, 0.0, 1e-300, 700.0]])
    np.testing.assert_allclose(oracle.softplus(z), np.logaddexp(0.0, z), rtol=1e-14, atol=0)


def test_sigmoid_matches_expit(oracle):
    b = np.concatenate([np.linspace(-60.0, 60.0, 2401), [-800.0, 0.0, 800.0]])
    np.testing.assert_allclose(oracle.sigmoid(b), scipy.special.expit(b), rtol=1e-14, atol=0)


def test_softplus_sigmoid_invariants(oracle):
    """softplus(z) - softplus(-z) = z, sigmoid(b) + sigmoid(-b) = 1,
    softplus(0) = ln 2, and softplus' = sigmoid (central difference)."""
    z = np.linspace(-30.0, 30.0, 601)
    np.testing.assert_allclose(oracle.softplus(z) - oracle.softplus(-z), z, rtol=0, atol=1e-13)
    np.testing.assert_allclose(oracle.sigmoid(z) + oracle.sigmoid(-z), 1.0, rtol=0, atol=1e-15)
    assert abs(oracle.softplus(np.array([0.0]))[0] - math.log(2.0)) < 1e-16
    h = 1e-5
    deriv = (oracle.softplus(z + h) - oracle.softplus(z - h)) / (2 * h)
    np.testing.assert_allclose(deriv, oracle.sigmoid(z), rtol=0, atol=1e-9)


def _page_head_params(seed, hv):
    """The pages' per-head parameter recipe: A ~ U(0, 16), A_log = log A,
    dt log-uniform on [1e-3, 1e-1] clamped at 1e-4, dt_bias the inverse
    softplus of dt (GDN pool-mode digest, key-code test)."""
    gen = torch.Generator().manual_seed(seed)
    A = torch.rand(hv, generator=gen, dtype=torch.float64) * 16.0
    lo, hi = math.log(1e-3), math.log(1e-1)
    dt = torch.exp(torch.rand(hv, generator=gen, dtype=torch.float64) * (hi - lo) + lo).clamp_min(1e-4)
    dt_bias = dt + torch.log(-torch.expm1(-dt))
    return A.numpy(), np.log(A.numpy()), dt.numpy(), dt_bias.numpy()


def test_zero_input_gives_minus_A_dt(oracle):
    """With x = 0, softplus(dt_bias) = dt, so g = -A * dt exactly (up to
    rounding), per head (scalar gate) and per channel."""
    A, A_log, dt, dt_bias = _page_head_params(3, 8)
    g = oracle.gate_activation(np.zeros((5, 8)), A_log, dt_bias)
    np.testing.assert_allclose(g, np.broadcast_to(-A * dt, (5, 8)), rtol=1e-12, atol=0)
    # per channel: a different (A, dt) in every channel of a head
    A2, A_log2, dt2, dt_bias2 = _page_head_params(4, 8 * 6)
    g2 = oracle.gate_activation(np.zeros((3, 8, 6)), A_log2.reshape(8, 6), dt_bias2.reshape(8, 6))
    np.testing.assert_allclose(g2, np.broadcast_to((-A2 * dt2).reshape(8, 6), (3, 8, 6)), rtol=1e-12, atol=0)


def test_large_input_is_linear(oracle):
    """softplus(z) = z + log1p(e^-z): for z = 40 the gate is -exp(A_log)(x + dt_bias)
    to within e^-40 relative."""
    A_log = np.array([[0.5, -1.0], [2.0, 0.0]])
    dt_bias = np.array([[1.0, -2.0], [0.25, 3.0]])
    x = 40.0 - dt_bias[None] + np.zeros((2, 2, 2))
    g = oracle.gate_activation(x, A_log, dt_bias)
    np.testing.assert_allclose(g, -np.exp(A_log)[None] * 40.0 * np.ones((2, 2, 2)), rtol=1e-15, atol=0)


def test_gate_axes(oracle):
    """A_log and dt_bias are indexed [value head, key channel]: a one-hot
    A_log changes exactly one (head, channel) column of g."""
    x = np.random.default_rng(5).standard_normal((4, 3, 5))
    base = oracle.gate_activation(x, np.zeros((3, 5)), np.zeros((3, 5)))
    bump = np.zeros((3, 5))
    bump[1, 3] = math.log(2.0)
    g = oracle.gate_activation(x, bump, np.zeros((3, 5)))
    diff = g != base
    assert diff[:, 1, 3].all() and diff.sum() == 4
    np.testing.assert_allclose(g[:, 1, 3], 2.0 * base[:, 1, 3], rtol=1e-15)


def test_fused_gate_prefill_is_activation_then_recurrence(oracle):
    """prefill_fused_gate equals the plain recurrence fed with gates computed
    by library routines (logaddexp, expit), per channel and scalar."""
    for scalar in (False, True):
        inp = W.make_prefill(61, [23, 5], 1, 2, 8, 4, io="f32", gate="realistic",
                             scalar_gate=scalar, h0="random")
        x, A_log, dtb, b = (t.double().numpy() for t in (inp.gx, inp.A_log, inp.dt_bias, inp.bx))
        g_lib = -np.exp(A_log)[None] * np.logaddexp(0.0, x + dtb[None])
        beta_lib = scipy.special.expit(b)
        o, ht = oracle.prefill_fused_gate(inp.q, inp.k, inp.v, inp.gx, inp.A_log, inp.dt_bias, inp.bx,
                                          inp.cu_seqlens, h0=inp.h0)
        o2, ht2 = oracle.prefill(inp.q, inp.k, inp.v, g_lib, beta_lib, inp.cu_seqlens, h0=inp.h0)
        np.testing.assert_allclose(o, o2, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(ht, ht2, rtol=1e-12, atol=1e-13)


def test_raw_inputs_reproduce_the_generated_gates(oracle):
    """In fp32 io the raw draws are exact, so the activation reproduces the
    generator's g and beta (which torch computed in fp32) to fp32 rounding."""
    inp = W.make_prefill(62, [40], 1, 2, 16, 8, io="f32", gate="realistic")
    g = oracle.gate_activation(inp.gx, inp.A_log, inp.dt_bias)
    np.testing.assert_allclose(g, inp.g.double().numpy(), rtol=2e-6, atol=1e-30)
    np.testing.assert_allclose(oracle.sigmoid(inp.bx), inp.beta.double().numpy(), rtol=2e-6, atol=0)


# ---- planted mistakes (in copies of the oracle's activation, on the CPU) ----

def _wrong(kind):
    def softplus(z):
        return np.maximum(z, 0.0) + np.log1p(np.exp(-np.abs(z)))

    def act(x, A_log, dt_bias):
        x, A_log, dt_bias = (np.asarray(t, np.float64) for t in (x, A_log, dt_bias))
        if kind == "sign":
            return np.exp(A_log)[None] * softplus(x + dt_bias[None])
        if kind == "no_exp":
            return -A_log[None] * softplus(x + dt_bias[None])
        if kind == "no_dt_bias":
            return -np.exp(A_log)[None] * softplus(x)
        if kind == "exp_not_softplus":
            return -np.exp(A_log)[None] * np.exp(x + dt_bias[None])
        if kind == "axes_swapped":
            return -np.exp(A_log.T.reshape(A_log.shape))[None] * softplus(x + dt_bias[None])
        raise ValueError(kind)
    return act


@pytest.mark.parametrize("kind", ["sign", "no_exp", "no_dt_bias", "exp_not_softplus", "axes_swapped"])
def test_pins_reject_wrong_activation(oracle, monkeypatch, kind):
    monkeypatch.setattr(oracle, "gate_activation", _wrong(kind))
    pins = [test_zero_input_gives_minus_A_dt, test_large_input_is_linear, test_gate_axes,
            test_fused_gate_prefill_is_activation_then_recurrence]
    caught = []
    for pin in pins:
        try:
            pin(oracle)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, kind
