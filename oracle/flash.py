"""fp64 CPU oracle of FLASH mixed-chunk attention.

TEST INFRASTRUCTURE ONLY (same rules as oracle/nystrom.py): only the test suite, the
package smoke check and the benchmark's CPU-baseline leg import it; the HIP library
shares no code with it.

Source: the review page "Transformer Quality in Linear Time" (nubint.ai), section
"Proposed method", third bullet: the sequence is split into non-overlapping chunks, a
local quadratic attention is applied inside each chunk, a global linear attention across
chunks (causal or not), and the two are combined. The page gives no formulas; the
readings taken here (each listed in the repository's design notes) are the plainest ones
the text supports:

* chunks: chunk g holds tokens [g c, min((g+1) c, n)) for a chunk size c (the last chunk
  may be shorter);
* local quadratic attention: scaled dot-product softmax attention restricted to the
  chunk, softmax(s Q_g K_g^T) V_g with s = 1/sqrt(d); causal: key t' <= query t;
* global linear attention: identity feature map, averaged over the keys it covers:
  s Q_t (sum over covered keys t' of K_t'^T V_t') / n_cov. Non-causal: every chunk of the
  sequence is covered; causal: only the chunks before the query's chunk (none for chunk
  0, whose global term is zero);
* combination: the sum of the two terms (the gate of the surrounding gated attention
  unit multiplies this sum and needs that layer's weights, so it is outside this core).

Plain, slow, obviously correct: NumPy float64, one (batch, head) and one chunk at a time.
"""
from __future__ import annotations

import numpy as np

from .nystrom import softmax_rows


def chunk_bounds(n: int, c: int) -> list:
    """[(start, end)] of the non-overlapping chunks of size c covering n tokens."""
    if c < 1:
        raise ValueError("chunk size must be >= 1")
    return [(s, min(s + c, n)) for s in range(0, n, c)]


def local_attention(q, k, v, causal: bool) -> np.ndarray:
    """Softmax attention inside one chunk (rows of q attend to rows of k, v)."""
    q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
    s = 1.0 / np.sqrt(q.shape[1])
    logits = s * (q @ k.T)
    if causal:
        logits = np.where(np.tril(np.ones(logits.shape, dtype=bool)), logits, -np.inf)
    return softmax_rows(logits) @ v


def chunk_state(k, v) -> np.ndarray:
    """sum over the chunk's tokens of K_t'^T V_t' (d x d)."""
    return np.asarray(k, dtype=np.float64).T @ np.asarray(v, dtype=np.float64)


def mixed_chunk_head(q, k, v, c: int, causal: bool) -> np.ndarray:
    """One (batch, head): local quadratic attention per chunk plus the global linear term."""
    q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
    n, d = q.shape
    s = 1.0 / np.sqrt(d)
    bnd = chunk_bounds(n, c)
    states = [chunk_state(k[a:b], v[a:b]) for a, b in bnd]
    out = np.zeros((n, d))
    for g, (a, b) in enumerate(bnd):
        out[a:b] = local_attention(q[a:b], k[a:b], v[a:b], causal)
        covered = range(g) if causal else range(len(bnd))
        n_cov = sum(bnd[j][1] - bnd[j][0] for j in covered)
        if n_cov > 0:
            state = sum(states[j] for j in covered)
            out[a:b] += s * (q[a:b] @ state) / n_cov
    return out


def mixed_chunk_attention(q, k, v, c: int, causal: bool = False, heads=None) -> np.ndarray:
    """[B, H, n, d] inputs -> [B, H, n, d] output (or, with ``heads`` a list of (b, h),
    the stacked heads in that order)."""
    q = np.asarray(q)
    B, H, n, d = q.shape
    pairs = [(b, h) for b in range(B) for h in range(H)] if heads is None else list(heads)
    out = np.stack([mixed_chunk_head(q[b, h], np.asarray(k)[b, h], np.asarray(v)[b, h], c,
                                     causal) for b, h in pairs])
    return out.reshape(B, H, n, d) if heads is None else out
