"""Pins of the gradient oracle (oracle/backward.py) against what does not use autograd:

* central finite differences of the NumPy forward (oracle/nystrom.py) along random
  directions, per input (Q, K, V, w), for even and uneven segments and a padded batch;
* the m = n limit: with one token per segment and a converged pseudo-inverse the forward
  is exact softmax attention plus the conv, so the gradients are those of
  softmax(Q K^T / sqrt(d)) V (torch's fp64 scaled_dot_product_attention) plus the conv's;
* the closed form dw[h][k] = sum over (b, t, f) of dO[t, f] V[t + k - (W-1)/2, f];
* K-shift invariance: adding one vector to every key row leaves all three softmaxes
  unchanged (every logit row moves by a constant), so sum_t dK[t] = 0 per head.

Planted mistakes (paths cut from the differentiated forward) must each fail a pin.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import backward as bw


def _inputs(B, H, n, d, W, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, n, d)) * scale
    k = rng.standard_normal((B, H, n, d)) * scale
    v = rng.standard_normal((B, H, n, d))
    w = rng.uniform(-0.5, 0.5, size=(H, W))
    g = rng.standard_normal((B, H, n, d))
    return q, k, v, w, g


def _loss(q, k, v, w, g, m, iters, lengths=None):
    out, _ = oracle.nystrom_forward(q, k, v, w, m, iters, lengths=lengths)
    return float(np.sum(out * g))


def _fd_check(q, k, v, w, g, m, iters, lengths=None, seed=0, eps=1e-6, tol=2e-6):
    dq, dk, dv, dw = bw.nystrom_backward(q, k, v, w, g, m, iters, lengths=lengths)
    rng = np.random.default_rng(seed)
    worst = 0.0
    for name, grad in (("q", dq), ("k", dk), ("v", dv), ("w", dw)):
        x = {"q": q, "k": k, "v": v, "w": w}
        u = rng.standard_normal(x[name].shape)
        if lengths is not None and name != "w":  # padding rows are not inputs
            for b, L in enumerate(lengths):
                u[b, :, L:] = 0.0
        plus = dict(x, **{name: x[name] + eps * u})
        minus = dict(x, **{name: x[name] - eps * u})
        fd = (_loss(plus["q"], plus["k"], plus["v"], plus["w"], g, m, iters, lengths)
              - _loss(minus["q"], minus["k"], minus["v"], minus["w"], g, m, iters, lengths)) / (2 * eps)
        an = float(np.sum(grad * u))
        rel = abs(fd - an) / max(abs(fd), 1e-12)
        worst = max(worst, rel)
        assert rel < tol, (name, fd, an, rel)
    return worst


def test_finite_differences_even_segments():
    q, k, v, w, g = _inputs(1, 2, 40, 8, 5, seed=1)
    _fd_check(q, k, v, w, g, m=5, iters=6, seed=11)


def test_finite_differences_uneven_segments():
    q, k, v, w, g = _inputs(1, 1, 37, 8, 7, seed=2)
    _fd_check(q, k, v, w, g, m=6, iters=6, seed=12)


def test_finite_differences_padded_batch():
    q, k, v, w, g = _inputs(2, 1, 30, 8, 5, seed=3)
    _fd_check(q, k, v, w, g, m=4, iters=6, lengths=[30, 19], seed=13)
    dq, dk, dv, _ = bw.nystrom_backward(q, k, v, w, g, 4, 6, lengths=[30, 19])
    assert not dq[1, :, 19:].any() and not dk[1, :, 19:].any() and not dv[1, :, 19:].any()


def test_finite_differences_zero_iterations():
    q, k, v, w, g = _inputs(1, 1, 24, 8, 3, seed=4)
    _fd_check(q, k, v, w, g, m=4, iters=0, seed=14)


def test_m_equals_n_reduces_to_exact_attention_gradients():
    n, d, W = 12, 8, 5
    q, _, v, w, g = _inputs(1, 1, n, d, W, seed=5, scale=0.3)
    k = q.copy()  # diagonal-dominant kernel: well conditioned, the iteration converges
    dq, dk, dv, dw = bw.nystrom_backward(q, k, v, w, g, m=n, iters=40)
    qt, kt, vt = (torch.tensor(a[0, 0], requires_grad=True) for a in (q, k, v))
    att = torch.nn.functional.scaled_dot_product_attention(qt[None], kt[None], vt[None])[0]
    gq, gk, gv = torch.autograd.grad((att * torch.tensor(g[0, 0])).sum(), (qt, kt, vt))
    # the conv adds w-correlated copies of dO to dV: out[t] += w[k] v[t + k - half]
    half = (W - 1) // 2
    gconv = np.zeros((n, d))
    for kk in range(W):
        sh = kk - half
        for t in range(n):
            if 0 <= t + sh < n:
                gconv[t + sh] += w[0, kk] * g[0, 0, t]
    np.testing.assert_allclose(dq[0, 0], gq.numpy(), atol=1e-9)
    np.testing.assert_allclose(dk[0, 0], gk.numpy(), atol=1e-9)
    np.testing.assert_allclose(dv[0, 0], gv.numpy() + gconv, atol=1e-9)


def test_conv_weight_gradient_closed_form():
    q, k, v, w, g = _inputs(2, 2, 20, 4, 5, seed=6)
    lengths = [20, 13]
    _, _, _, dw = bw.nystrom_backward(q, k, v, w, g, 4, 6, lengths=lengths)
    W, half = 5, 2
    ref = np.zeros((2, W))
    for b, L in enumerate(lengths):
        for h in range(2):
            for kk in range(W):
                for f in range(4):
                    # correlation of dO with V shifted by kk - half (numpy.correlate, 'full')
                    full = np.correlate(v[b, h, :L, f], g[b, h, :L, f], mode="full")
                    ref[h, kk] += full[(L - 1) + (kk - half)]
    np.testing.assert_allclose(dw, ref, rtol=1e-12, atol=1e-12)


def test_key_shift_invariance():
    q, k, v, w, g = _inputs(2, 2, 33, 8, 5, seed=7)
    _, dk, _, _ = bw.nystrom_backward(q, k, v, w, g, 5, 6, lengths=[33, 21])
    for b, L in enumerate([33, 21]):
        for h in range(2):
            s = np.abs(dk[b, h, :L].sum(axis=0)).max()
            assert s < 1e-10 * np.abs(dk[b, h, :L]).sum(), s


# ------------------------------------------------------------------ planted mistakes
def _pinv_alpha_detached(a, iters):
    eye = torch.eye(a.shape[0], dtype=a.dtype)
    alpha = (1.0 / (a.abs().sum(dim=0).max() * a.abs().sum(dim=1).max())).detach()
    z = alpha * a.T
    for _ in range(iters):
        x = a @ z
        z = 0.25 * (z @ (13.0 * eye - x @ (15.0 * eye - x @ (7.0 * eye - x))))
    return z


def _pinv_z_detached(a, iters):
    return bw._ORIG_PINV(a.detach(), iters)


def _segment_means_detached(x, m):
    return bw._ORIG_SEGMEANS(x, m).detach()


def _conv_no_grad_to_v(v, w):
    return bw._ORIG_CONV(v.detach(), w)


def _conv_flipped(v, w):
    return bw._ORIG_CONV(v, torch.flip(w, dims=[0]))


MUTANTS = {
    "alpha detached": ("_pinv", _pinv_alpha_detached),
    "Z treated as constant": ("_pinv", _pinv_z_detached),
    "landmarks treated as constant": ("_segment_means", _segment_means_detached),
    "conv gives no dV": ("_conv", _conv_no_grad_to_v),
    "conv taps flipped": ("_conv", _conv_flipped),
}


def _pins_pass():
    try:
        q, k, v, w, g = _inputs(1, 1, 40, 8, 5, seed=1)
        _fd_check(q, k, v, w, g, m=5, iters=6, seed=11)
        test_conv_weight_gradient_closed_form()
        test_key_shift_invariance()
        test_m_equals_n_reduces_to_exact_attention_gradients()
    except AssertionError:
        return False
    return True


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistakes(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(bw, "_ORIG_PINV", bw._pinv, raising=False)
    monkeypatch.setattr(bw, "_ORIG_SEGMEANS", bw._segment_means, raising=False)
    monkeypatch.setattr(bw, "_ORIG_CONV", bw._conv, raising=False)
    monkeypatch.setattr(bw, attr, fn)
    assert not _pins_pass(), f"mutant '{name}' passes every pin"
