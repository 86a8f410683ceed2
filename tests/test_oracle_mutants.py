"""Each plausible mistake, planted in a copy of the oracle on the CPU, must be caught
by at least one pin. This shows the pins constrain the oracle where it matters: tap
direction, where the padding sits, W layout, residual, bias, eps placement, biased
variance, group layout and the affine shift."""
import numpy as np
import pytest

import oracle
from oracle import reference as R
from pins import BLOCK_PINS, EXT_PINS, GN_PINS, TRAIN_PINS


def _m_tap_reversed(x, rm, rv, g, b_, eps, W, b, d):
    return oracle.prenorm_block(x, rm, rv, g, b_, eps, np.asarray(W)[:, :, ::-1], b, d)


def _m_w_transposed(x, rm, rv, g, b_, eps, W, b, d):
    return oracle.prenorm_block(x, rm, rv, g, b_, eps, np.asarray(W).transpose(1, 0, 2), b, d)


def _m_pad_before_bn(x, rm, rv, g, b_, eps, W, b, d):
    x = R._f64(x)
    xpad = R.zero_pad_time(x, d)
    zpad = R.bn_eval_relu(xpad, rm, rv, g, b_, eps)      # padding then BN: wrong
    return x + R.conv1d_k3_padded(zpad, W, b, d, x.shape[2])


def _m_no_residual(x, rm, rv, g, b_, eps, W, b, d):
    return oracle.prenorm_block(x, rm, rv, g, b_, eps, W, b, d) - R._f64(x)


def _m_no_bias(x, rm, rv, g, b_, eps, W, b, d):
    return oracle.prenorm_block(x, rm, rv, g, b_, eps, W, None, d)


def _m_eps_outside_sqrt(x, rm, rv, g, b_, eps, W, b, d):
    rv = R._f64(rv)
    rv_equiv = (np.sqrt(rv) + eps) ** 2 - eps          # makes sqrt(rv'+eps) = sqrt(rv)+eps
    return oracle.prenorm_block(x, rm, rv_equiv, g, b_, eps, W, b, d)


def _m_relu_missing(x, rm, rv, g, b_, eps, W, b, d):
    x = R._f64(x)
    norm = (x - R._f64(rm)[None, :, None]) / np.sqrt(R._f64(rv)[None, :, None] + eps)
    zfull = R._f64(g)[None, :, None] * norm + R._f64(b_)[None, :, None]
    return x + R.conv1d_k3_padded(R.zero_pad_time(zfull, d), W, b, d, x.shape[2])


def _m_off_by_one_tap(x, rm, rv, g, b_, eps, W, b, d):
    x = R._f64(x)
    z = R.bn_eval_relu(x, rm, rv, g, b_, eps)
    zpad = R.zero_pad_time(z, d + 1)                   # window shifted by one
    return x + R.conv1d_k3_padded(zpad, W, b, d, x.shape[2])


BLOCK_MUTANTS = [_m_tap_reversed, _m_w_transposed, _m_pad_before_bn, _m_no_residual,
                 _m_no_bias, _m_eps_outside_sqrt, _m_relu_missing, _m_off_by_one_tap]


def _g_unbiased(x, W, bias, gamma, beta, eps, G, padding=1, dilation=1):
    x = R._f64(x)
    T_out = R.conv_output_length(x.shape[2], padding, dilation)
    y = R.conv1d_k3_padded(R.zero_pad_time(x, padding), W, bias, dilation, T_out)
    N, C, T = y.shape
    yg = y.reshape(N, G, -1)
    m = yg.mean(axis=2, keepdims=True)
    v = yg.var(axis=2, ddof=1, keepdims=True)
    o = ((yg - m) / np.sqrt(v + eps)).reshape(N, C, T)
    return o * R._f64(gamma)[None, :, None] + R._f64(beta)[None, :, None]


def _g_interleaved_groups(x, W, bias, gamma, beta, eps, G, padding=1, dilation=1):
    x = R._f64(x)
    T_out = R.conv_output_length(x.shape[2], padding, dilation)
    y = R.conv1d_k3_padded(R.zero_pad_time(x, padding), W, bias, dilation, T_out)
    N, C, T = y.shape
    perm = np.argsort(np.arange(C) % G, kind="stable")     # channel c in group c % G
    inv = np.argsort(perm)
    o = R.group_norm(y[:, perm], G, None, None, eps)[:, inv]
    return o * R._f64(gamma)[None, :, None] + R._f64(beta)[None, :, None]


def _g_no_beta(x, W, bias, gamma, beta, eps, G, padding=1, dilation=1):
    return oracle.conv_groupnorm(x, W, bias, gamma, None, eps, G, padding, dilation)


def _g_no_padding(x, W, bias, gamma, beta, eps, G, padding=1, dilation=1):
    return oracle.conv_groupnorm(x, W, bias, gamma, beta, eps, G, padding + 1, dilation)[:, :, 1:-1]


def _g_stats_per_channel(x, W, bias, gamma, beta, eps, G, padding=1, dilation=1):
    C = np.asarray(W).shape[0]
    return oracle.conv_groupnorm(x, W, bias, gamma, beta, eps, C, padding, dilation)


def _g_beta_needs_gamma(x, W, bias, gamma, beta, eps, G, padding=1, dilation=1):
    # beta skipped whenever gamma is absent (the affine step only with gamma present)
    if gamma is None:
        beta = None
    return oracle.conv_groupnorm(x, W, bias, gamma, beta, eps, G, padding, dilation)


GN_MUTANTS = [_g_unbiased, _g_interleaved_groups, _g_no_beta, _g_no_padding, _g_stats_per_channel,
              _g_beta_needs_gamma]


def _t_unbiased_norm(x, rm, rv, g, b_, eps, mom, W, b, d):
    x64 = R._f64(x)
    N, C, L = x64.shape
    mean = x64.mean(axis=(0, 2))
    var = x64.var(axis=(0, 2), ddof=1)                      # wrong: unbiased for normalising
    out = oracle.prenorm_block(x64, mean, var, g, b_, eps, W, b, d)
    nrm, nrv = R.running_stats_update(rm, rv, mean, x64.var(axis=(0, 2)), N * L, mom)
    return out, nrm, nrv, mean, x64.var(axis=(0, 2))


def _t_biased_running(x, rm, rv, g, b_, eps, mom, W, b, d):
    out, nrm, _, mean, var = oracle.prenorm_block_train(x, rm, rv, g, b_, eps, mom, W, b, d)
    nrv = (1 - mom) * R._f64(rv) + mom * var                # wrong: no n/(n-1)
    return out, nrm, nrv, mean, var


def _t_stats_over_batch_only(x, rm, rv, g, b_, eps, mom, W, b, d):
    x64 = R._f64(x)
    N, C, L = x64.shape
    mean = x64.mean(axis=(0, 2))
    var = x64[:, :, :1].var(axis=(0, 2))                    # wrong: statistics of t=0 only
    out = oracle.prenorm_block(x64, mean, var, g, b_, eps, W, b, d)
    nrm, nrv = R.running_stats_update(rm, rv, mean, var, N * L, mom)
    return out, nrm, nrv, mean, var


def _t_momentum_swapped(x, rm, rv, g, b_, eps, mom, W, b, d):
    return oracle.prenorm_block_train(x, rm, rv, g, b_, eps, 1.0 - mom, W, b, d)


TRAIN_MUTANTS = [_t_unbiased_norm, _t_biased_running, _t_stats_over_batch_only,
                 _t_momentum_swapped]


def _e_residual_from_input(xn, W, b, residual, d):
    return oracle.relu_conv_residual(xn, W, b, xn, d)      # wrong: residual = conv input


def _e_no_relu(xn, W, b, residual, d):
    xn64 = R._f64(xn)
    y = R.conv1d_k3_padded(R.zero_pad_time(xn64, d), W, b, d, xn64.shape[2])   # wrong
    return R._f64(residual) + y


def _e_tap_reversed(xn, W, b, residual, d):
    return oracle.relu_conv_residual(xn, R._f64(W)[:, :, ::-1], b, residual, d)


def _e_bias_dropped(xn, W, b, residual, d):
    return oracle.relu_conv_residual(xn, W, None, residual, d)


EXT_MUTANTS = [_e_residual_from_input, _e_no_relu, _e_tap_reversed, _e_bias_dropped]


def _caught(pins, fn):
    failed = []
    for pin in pins:
        try:
            ok, msg = pin(fn)
        except Exception as e:  # a crash also counts as caught
            ok, msg = False, repr(e)
        if not ok:
            failed.append(pin.__name__)
    return failed


@pytest.mark.parametrize("mutant", BLOCK_MUTANTS, ids=lambda f: f.__name__)
def test_block_mutant_is_caught(mutant):
    assert _caught(BLOCK_PINS, mutant), f"no pin rejects {mutant.__name__}"


@pytest.mark.parametrize("mutant", EXT_MUTANTS, ids=lambda f: f.__name__)
def test_external_bn_mutant_is_caught(mutant):
    assert _caught(EXT_PINS, mutant), f"no pin rejects {mutant.__name__}"


@pytest.mark.parametrize("mutant", TRAIN_MUTANTS, ids=lambda f: f.__name__)
def test_train_mutant_is_caught(mutant):
    assert _caught(TRAIN_PINS, mutant), f"no pin rejects {mutant.__name__}"


@pytest.mark.parametrize("mutant", GN_MUTANTS, ids=lambda f: f.__name__)
def test_gn_mutant_is_caught(mutant):
    assert _caught(GN_PINS, mutant), f"no pin rejects {mutant.__name__}"
