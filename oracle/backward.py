"""fp64 CPU oracle of the gradients of the Nystrom attention forward.

TEST INFRASTRUCTURE ONLY (same rules as oracle/nystrom.py): only the test suite, the
package smoke check and the benchmark's CPU-baseline leg import it; the HIP library
shares no code with it.

What is computed. The pages train their models, so the forward's parameters and inputs
receive gradients, but no page writes a backward pass out: it is the derivative of the
forward (Nystromformer review page, "Proposed method", bullets M1..M6 as in
oracle/nystrom.py) and nothing else. Given an upstream gradient dO of the output, this
module returns dL/dQ, dL/dK, dL/dV and dL/dw for L = sum(O * dO).

How. The forward of oracle/nystrom.py is restated step by step with torch float64 CPU
tensors (segment means, the three row softmaxes, the pseudo-inverse scaling and
iteration, B V first, Z W, F Y, the depthwise conv skip) and differentiated by
torch.autograd, one (batch, head) at a time. Every path through the forward carries
gradient, including alpha = 1 / (max column sum * max row sum), which is differentiated
through its maxima (a subgradient at ties). Padding rows of a ragged batch are not part
of the forward, so their gradients are zero; dw sums over the batch.

Pins (tests/test_oracle_backward.py) do not use autograd: central finite differences of
the NumPy forward, exact-attention gradients in the m = n limit, a closed form for dw and
the K-shift invariance sum_t dK[t] = 0.
"""
from __future__ import annotations

import numpy as np
import torch

from .nystrom import segment_boundaries


def _segment_means(x: torch.Tensor, m: int) -> torch.Tensor:
    """M4 on a (n, d) tensor: means of the m contiguous segments."""
    bnd = segment_boundaries(x.shape[0], m)
    return torch.stack([x[bnd[j]:bnd[j + 1]].mean(dim=0) for j in range(m)])


def _pinv(a: torch.Tensor, iters: int) -> torch.Tensor:
    """M2/M5: Z_0 = A^T / (||A||_1 ||A||_inf), then Z <- 1/4 Z (13I - X(15I - X(7I - X)))
    with X = A Z, as in oracle.nystrom.iterative_pinv."""
    eye = torch.eye(a.shape[0], dtype=a.dtype)
    alpha = 1.0 / (a.abs().sum(dim=0).max() * a.abs().sum(dim=1).max())
    z = alpha * a.T
    for _ in range(iters):
        x = a @ z
        z = 0.25 * (z @ (13.0 * eye - x @ (15.0 * eye - x @ (7.0 * eye - x))))
    return z


def _conv(v: torch.Tensor, w: torch.Tensor) -> torch.Tensor:
    """M6 skip: out[t] = sum_k w[k] v[t + k - (W-1)/2], zero outside the sequence."""
    n = v.shape[0]
    half = (w.shape[0] - 1) // 2
    out = torch.zeros_like(v)
    for k in range(w.shape[0]):
        shift = k - half
        lo, hi = max(0, -shift), min(n, n - shift)
        if hi > lo:
            out[lo:hi] = out[lo:hi] + w[k] * v[lo + shift:hi + shift]
    return out


def head_forward(q, k, v, w, m: int, iters: int) -> torch.Tensor:
    """One (batch, head) of the forward: F (Z (B V)) + conv(V)."""
    s = 1.0 / np.sqrt(q.shape[1])
    q_land = _segment_means(q, m)
    k_land = _segment_means(k, m)
    f = torch.softmax(s * (q @ k_land.T), dim=-1)
    a_s = torch.softmax(s * (q_land @ k_land.T), dim=-1)
    b = torch.softmax(s * (q_land @ k.T), dim=-1)
    z = _pinv(a_s, iters)
    return f @ (z @ (b @ v)) + _conv(v, w)


def nystrom_backward(q, k, v, conv_w, dout, m: int, iters: int = 6, lengths=None,
                     heads=None):
    """Gradients of L = sum(O * dO) for inputs [B, H, n, d] and conv weights [H, W].

    Returns (dq, dk, dv, dw): dq, dk, dv as [B, H, n, d] (or, with ``heads`` a list of
    (b, h) pairs, stacked [len(heads), n, d] in that order), zero on padding rows; dw as
    [H, W], summed over the batch elements computed (all of them unless ``heads``)."""
    q = np.asarray(q)
    B, H, n, d = q.shape
    lens = [n] * B if lengths is None else [int(x) for x in lengths]
    if len(lens) != B or any(not (m <= x <= n) for x in lens):
        raise ValueError("lengths must hold B values in [m, n]")
    pairs = [(b, h) for b in range(B) for h in range(H)] if heads is None else list(heads)
    W = np.asarray(conv_w).shape[1]
    dq, dk, dv = (np.zeros((len(pairs), n, d)) for _ in range(3))
    dw = np.zeros((H, W))
    t64 = lambda a: torch.tensor(np.asarray(a, dtype=np.float64), requires_grad=True)
    for i, (b, h) in enumerate(pairs):
        L = lens[b]
        qt, kt, vt = t64(q[b, h, :L]), t64(np.asarray(k)[b, h, :L]), t64(np.asarray(v)[b, h, :L])
        wt = t64(np.asarray(conv_w)[h])
        out = head_forward(qt, kt, vt, wt, m, iters)
        g = torch.tensor(np.asarray(dout, dtype=np.float64)[b, h, :L])
        gq, gk, gv, gw = torch.autograd.grad((out * g).sum(), (qt, kt, vt, wt))
        dq[i, :L], dk[i, :L], dv[i, :L] = gq.numpy(), gk.numpy(), gv.numpy()
        dw[h] += gw.numpy()
    if heads is None:
        dq, dk, dv = (x.reshape(B, H, n, d) for x in (dq, dk, dv))
    return dq, dk, dv, dw
