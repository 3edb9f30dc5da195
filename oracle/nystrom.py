"""fp64 CPU oracle for the Nystrom self-attention forward.

TEST INFRASTRUCTURE ONLY. Only the test suite, the package's smoke check and the
benchmark's CPU-baseline leg may import this module. The product path (the HIP library
and its Python binding) never calls it and shares no code with it.

Source of every step: the review page "Nystromformer: A Nystrom-Based Algorithm for
Approximating Self-Attention" (nubint.ai), section "Proposed method" (its six bullets,
cited below as M1..M6 in page order), plus its main-findings section for the O(n)
claims. The page prints no worked values for this computation, so the oracle is pinned
by mathematics instead (closed forms, limits, special cases, brute force; see
tests/test_oracle_pins.py).

Plain, slow, obviously correct: NumPy float64, one (batch, head) at a time, every step
in the order the page gives it, no blocking or fusion. Readings where the page is
silent (each one listed in the repository's design notes):

* softmax is row-wise over the last axis, no mask, no causality;
* the 1/sqrt(d) scale is applied inside all three softmaxes (M1, M3 show it; M2 omits
  it, read as shorthand);
* segments are m contiguous, equal-length blocks of tokens; n % m == 0 is required;
* the pseudo-inverse iteration (M5 names an iterative method and about six iterations,
  but gives no formula) is the third-order Newton-type scheme
  Z <- 1/4 Z (13I - X(15I - X(7I - X))), X = A Z, started from
  Z_0 = A^T / (||A||_1 ||A||_inf) computed per (batch, head) matrix;
* the skip connection (M6) is a depthwise convolution along the sequence with one
  odd-width filter per head shared over the d features, cross-correlation (no flip),
  zero "same" padding, no bias, added to the attention output.
"""
from __future__ import annotations

import numpy as np


def softmax_rows(x: np.ndarray) -> np.ndarray:
    """Row-wise softmax over the last axis, computed as exp(x - max)/sum."""
    x = np.asarray(x, dtype=np.float64)
    e = np.exp(x - x.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def segment_means(x: np.ndarray, m: int) -> np.ndarray:
    """M4: landmarks as segment means. x is (n, d); segment j is rows [j*l, (j+1)*l)
    with l = n/m; returns the (m, d) matrix of per-segment means."""
    n, d = x.shape
    if m < 1 or n % m != 0:
        raise ValueError("segment means need n % m == 0")
    l = n // m
    out = np.empty((m, d), dtype=np.float64)
    for j in range(m):
        out[j] = x[j * l:(j + 1) * l].astype(np.float64).sum(axis=0) / l
    return out


def pinv_scaling(a: np.ndarray) -> float:
    """alpha = 1 / (max column abs-sum * max row abs-sum) of the m x m kernel."""
    a = np.asarray(a, dtype=np.float64)
    col = np.abs(a).sum(axis=0).max()
    row = np.abs(a).sum(axis=1).max()
    return 1.0 / (col * row)


def iterative_pinv(a: np.ndarray, iters: int, return_all: bool = False):
    """M2/M5: approximate Moore-Penrose inverse of the m x m landmark kernel by a fixed
    number of Newton-type iterations (no SVD). Returns Z_iters (and, if asked, the list
    Z_0..Z_iters)."""
    a = np.asarray(a, dtype=np.float64)
    m = a.shape[0]
    eye = np.eye(m)
    z = pinv_scaling(a) * a.T
    seq = [z]
    for _ in range(iters):
        x = a @ z
        inner = 7.0 * eye - x
        inner = 15.0 * eye - x @ inner
        inner = 13.0 * eye - x @ inner
        z = 0.25 * (z @ inner)
        seq.append(z)
    return (z, seq) if return_all else z


def depthwise_conv_seq(v: np.ndarray, w: np.ndarray) -> np.ndarray:
    """M6 skip branch: out[t, :] = sum_k w[k] * v[t + k - (W-1)/2, :], with v = 0
    outside [0, n). v is (n, d), w is (W,) with W odd."""
    n, d = v.shape
    W = w.shape[0]
    if W % 2 != 1:
        raise ValueError("conv width must be odd")
    half = (W - 1) // 2
    out = np.zeros((n, d), dtype=np.float64)
    for k in range(W):
        shift = k - half
        lo = max(0, -shift)
        hi = min(n, n - shift)
        if hi > lo:
            out[lo:hi] += float(w[k]) * v[lo + shift:hi + shift]
    return out


def nystrom_head(q: np.ndarray, k: np.ndarray, v: np.ndarray, m: int, iters: int):
    """One (batch, head) of the Nystrom attention, without the conv skip.

    Returns every intermediate in a dict: q_land, k_land (m, d); a_s, z (m, m);
    f (n, m); b (m, n); w (m, d) = B V; y (m, d) = Z W; attn (n, d) = F Y.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    d = q.shape[1]
    s = 1.0 / np.sqrt(d)
    q_land = segment_means(q, m)                 # M4
    k_land = segment_means(k, m)                 # M4
    f = softmax_rows(s * (q @ k_land.T))         # M3, left factor  (n x m)
    a_s = softmax_rows(s * (q_land @ k_land.T))  # M2, landmark kernel (m x m)
    b = softmax_rows(s * (q_land @ k.T))         # M3, right factor (m x n)
    z = iterative_pinv(a_s, iters)               # M2, M5
    w = b @ v                                    # M6, right to left: B V first
    y = z @ w
    attn = f @ y
    return dict(q_land=q_land, k_land=k_land, a_s=a_s, z=z, f=f, b=b, w=w, y=y,
                attn=attn)


def nystrom_forward(q, k, v, conv_w, m: int, iters: int = 6, heads=None,
                    return_stages: bool = False):
    """Full forward over [B, H, n, d] inputs: attention part plus the depthwise-conv
    skip on V. ``conv_w`` is [H, W]. ``heads`` optionally restricts the computation
    to a list of (b, h) pairs (their outputs are returned in that order, stacked as
    [len(heads), n, d]); otherwise the result is [B, H, n, d].
    """
    q = np.asarray(q)
    B, H, n, d = q.shape
    pairs = [(b, h) for b in range(B) for h in range(H)] if heads is None else list(heads)
    outs, attns, stages = [], [], []
    for (b, h) in pairs:
        st = nystrom_head(q[b, h], k[b, h], v[b, h], m, iters)
        conv = depthwise_conv_seq(np.asarray(v[b, h], dtype=np.float64),
                                  np.asarray(conv_w[h], dtype=np.float64))
        outs.append(st["attn"] + conv)
        attns.append(st["attn"])
        if return_stages:
            stages.append(st)
    out = np.stack(outs)
    attn = np.stack(attns)
    if heads is None:
        out = out.reshape(B, H, n, d)
        attn = attn.reshape(B, H, n, d)
    if return_stages:
        return out, attn, stages
    return out, attn


def exact_attention_head(q, k, v) -> np.ndarray:
    """The quantity being approximated (M1): softmax(Q K^T / sqrt(d)) V, formed densely.
    Used only by the oracle's own pins on small n."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    s = 1.0 / np.sqrt(q.shape[1])
    return softmax_rows(s * (q @ k.T)) @ v
