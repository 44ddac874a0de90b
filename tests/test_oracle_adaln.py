"""Pins of the AdaLN + residual oracle against things it does not compute itself."""
import numpy as np
import pytest
import torch

import oracle
import oracle.adaln as oadaln


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def test_layer_norm_matches_torch_layer_norm():
    """A library routine: torch.nn.functional.layer_norm in float64 on the CPU (no affine)."""
    x = _rand((3, 17, 256), 0) * 3.0 + 1.5
    for eps in (1e-5, 1e-2):
        ref = torch.nn.functional.layer_norm(torch.from_numpy(x), (256,), eps=eps).numpy()
        assert np.allclose(oracle.layer_norm(x, eps), ref, rtol=0, atol=1e-12)


def test_normalised_rows_have_zero_mean_and_the_closed_form_variance():
    x = _rand((4, 9, 512), 1) * 2.0 - 0.7
    eps = 1e-3
    xh = oracle.layer_norm(x, eps)
    var = x.var(axis=-1)
    assert np.allclose(xh.mean(axis=-1), 0.0, atol=1e-13)
    assert np.allclose(xh.var(axis=-1), var / (var + eps), rtol=1e-12)


def test_biased_variance_closed_form():
    """Row (1, -1, 1, -1, ...): mean 0, biased variance exactly 1, so xhat = x / sqrt(1 + eps)
    (an unbiased variance, C / (C - 1), would give a different value)."""
    C, eps = 256, 1e-5
    x = np.tile([1.0, -1.0], C // 2)[None, None]
    xh = oracle.layer_norm(x, eps)
    assert np.allclose(xh, x / np.sqrt(1.0 + eps), rtol=1e-15)


def test_constant_rows_give_residual_plus_beta():
    x = np.full((2, 5, 256), 3.25)
    res, beta = _rand((2, 5, 256), 2), _rand((2, 256), 3)
    out = oracle.adaln_residual(x, res, _rand((2, 256), 4), beta, 1e-5)
    assert np.array_equal(out, res + beta[:, None, :])


def test_shift_and_scale_invariance():
    x = _rand((2, 7, 512), 5)
    xh = oracle.layer_norm(x, 1e-12)
    assert np.allclose(oracle.layer_norm(3.5 * x - 11.0, 1e-12 * 3.5 ** 2), xh, atol=1e-9)


def test_film_and_residual_terms():
    """out - res - beta is gamma times the normalised row: linear in gamma, per batch element."""
    B, T, C, eps = 2, 6, 256, 1e-5
    x, res = _rand((B, T, C), 6), _rand((B, T, C), 7)
    g, b = _rand((B, C), 8), _rand((B, C), 9)
    out = oracle.adaln_residual(x, res, g, b, eps)
    xh = oracle.layer_norm(x, eps)
    for bi in range(B):
        assert np.allclose(out[bi] - res[bi] - b[bi], g[bi] * xh[bi], atol=1e-13)
    # gamma = 1, beta = 0, res = 0 reduces to the library LayerNorm
    ref = torch.nn.functional.layer_norm(torch.from_numpy(x), (C,), eps=eps).numpy()
    assert np.allclose(oracle.adaln_residual(x, np.zeros_like(x), np.ones((B, C)), np.zeros((B, C)), eps),
                       ref, atol=1e-12)


def _mutant_layer_norm(mutation):
    def bad_ln(x, eps):
        x = np.asarray(x, dtype=np.float64)
        mean = x.mean(axis=-1, keepdims=True)
        if mutation == "unbiased":
            return (x - mean) / np.sqrt(x.var(axis=-1, ddof=1, keepdims=True) + eps)
        if mutation == "eps_outside":
            return (x - mean) / (np.sqrt(x.var(axis=-1, keepdims=True)) + eps)
        assert mutation == "no_center"
        return x / np.sqrt(x.var(axis=-1, keepdims=True) + eps)
    return bad_ln


def _mutant_adaln(mutation):
    def bad_adaln(x, res, gamma, beta, eps):
        xhat = oadaln.layer_norm(x, eps)
        g = np.asarray(gamma, dtype=np.float64)[:, None, :]
        b = np.asarray(beta, dtype=np.float64)[:, None, :]
        r = np.asarray(res, dtype=np.float64)
        if mutation == "beta_before_gamma":
            return r + g * (xhat + b)
        if mutation == "no_residual":
            return g * xhat + b
        assert mutation == "gamma_of_batch_0"
        return r + g[:1] * xhat + b
    return bad_adaln


PINS = [test_layer_norm_matches_torch_layer_norm, test_normalised_rows_have_zero_mean_and_the_closed_form_variance,
        test_biased_variance_closed_form, test_constant_rows_give_residual_plus_beta,
        test_shift_and_scale_invariance, test_film_and_residual_terms]


@pytest.mark.parametrize("mutation", ["unbiased", "eps_outside", "no_center", "beta_before_gamma", "no_residual",
                                      "gamma_of_batch_0"])
def test_mutations_are_caught(mutation, monkeypatch):
    """A plausible mistake planted in oracle.adaln (in place of its LayerNorm or its FiLM /
    residual step, also where the package re-exports it) makes at least one pin above fail."""
    if mutation in ("unbiased", "eps_outside", "no_center"):
        bad = _mutant_layer_norm(mutation)
        monkeypatch.setattr(oadaln, "layer_norm", bad)
        monkeypatch.setattr(oracle, "layer_norm", bad)
    else:
        bad = _mutant_adaln(mutation)
        monkeypatch.setattr(oadaln, "adaln_residual", bad)
        monkeypatch.setattr(oracle, "adaln_residual", bad)
    failed = []
    for pin in PINS:
        try:
            pin()
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"no pin catches the {mutation} mutation"
