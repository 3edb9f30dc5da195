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
* segments are m contiguous blocks of tokens: token t of a length-L sequence belongs to
  segment floor(t m / L), i.e. segment j is rows [ceil(j L / m), ceil((j+1) L / m)) of
  floor(L/m) or ceil(L/m) tokens (all equal when m divides L), with 1 <= m <= L;
* padding masks / ragged batches: batch element b has a valid length L_b (m <= L_b <= n).
  Rows [0, L_b) of its output are the forward of the unpadded length-L_b sequence
  (padding tokens are neither keys, values, landmark members nor conv inputs) and rows
  [L_b, n) are zero;
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


def segment_boundaries(n: int, m: int) -> list:
    """Start rows of the m contiguous segments of n tokens, plus n: segment j is rows
    [ceil(j n / m), ceil((j+1) n / m)) (l = n/m rows each when m divides n)."""
    if m < 1 or m > n:
        raise ValueError("segment means need 1 <= m <= n")
    return [(j * n + m - 1) // m for j in range(m + 1)]


def segment_means(x: np.ndarray, m: int) -> np.ndarray:
    """M4: landmarks as segment means. x is (n, d); returns the (m, d) matrix of the
    means of the m contiguous segments given by segment_boundaries."""
    n, d = x.shape
    bnd = segment_boundaries(n, m)
    out = np.empty((m, d), dtype=np.float64)
    for j in range(m):
        rows = x[bnd[j]:bnd[j + 1]].astype(np.float64)
        out[j] = rows.sum(axis=0) / rows.shape[0]
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
                    return_stages: bool = False, lengths=None):
    """Full forward over [B, H, n, d] inputs: attention part plus the depthwise-conv
    skip on V. ``conv_w`` is [H, W]. ``heads`` optionally restricts the computation
    to a list of (b, h) pairs (their outputs are returned in that order, stacked as
    [len(heads), n, d]); otherwise the result is [B, H, n, d]. ``lengths`` (B ints,
    default all n) are the valid lengths of a padded batch: each (b, h) is computed on
    its first lengths[b] tokens and the remaining output rows are zero.
    """
    q = np.asarray(q)
    B, H, n, d = q.shape
    lens = [n] * B if lengths is None else [int(x) for x in lengths]
    if len(lens) != B or any(not (m <= x <= n) for x in lens):
        raise ValueError("lengths must hold B values in [m, n]")
    pairs = [(b, h) for b in range(B) for h in range(H)] if heads is None else list(heads)
    outs, attns, stages = [], [], []
    for (b, h) in pairs:
        L = lens[b]
        st = nystrom_head(q[b, h, :L], k[b, h, :L], v[b, h, :L], m, iters)
        conv = depthwise_conv_seq(np.asarray(v[b, h, :L], dtype=np.float64),
                                  np.asarray(conv_w[h], dtype=np.float64))
        full = np.zeros((n, d))
        full[:L] = st["attn"] + conv
        attn = np.zeros((n, d))
        attn[:L] = st["attn"]
        outs.append(full)
        attns.append(attn)
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
    """The quantity being approximated (M1): softmax(Q K^T / sqrt(d)) V, formed densely
    (small n only). It is the expected value of the m = n reduction checks; pinned against
    torch's dense scaled-dot-product attention and pure-Python loops."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    s = 1.0 / np.sqrt(q.shape[1])
    return softmax_rows(s * (q @ k.T)) @ v
