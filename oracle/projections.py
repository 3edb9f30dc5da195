"""fp64 CPU oracle of the projections around the Nystrom attention core.

TEST INFRASTRUCTURE ONLY (same rules as oracle/nystrom.py): only the test suite, the
package smoke check and the benchmark's CPU-baseline leg import it.

Source: the Fastformer review page, section "Proposed method" (the input embeddings are
turned into Q, K, V by three linear projections per attention head). Readings where the
pages are silent (listed in the design notes): no biases; the heads' outputs are
concatenated (head-major features) and mapped back to the model width by one linear
output projection; weights use the [out_features][in_features] layout.

Shapes: x [B, n, D] with D the model width; w_qkv [3 H d, D] (rows: Q heads 0..H-1,
then K heads, then V heads, d rows each); w_o [D, H d]; per-head tensors [B, H, n, d].
"""
from __future__ import annotations

import numpy as np

from .nystrom import nystrom_forward


def qkv_project(x: np.ndarray, w_qkv: np.ndarray, H: int, d: int):
    """Q, K, V [B, H, n, d]: for head h, Q_h = x W_q^h^T with W_q^h the d rows of w_qkv
    starting at h*d (then K at (H + h)*d, V at (2H + h)*d)."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w_qkv, dtype=np.float64)
    B, n, D = x.shape
    out = []
    for which in range(3):
        heads = []
        for h in range(H):
            rows = w[(which * H + h) * d:(which * H + h + 1) * d]   # [d, D]
            heads.append(x @ rows.T)                                # [B, n, d]
        out.append(np.stack(heads, axis=1))                         # [B, H, n, d]
    return tuple(out)


def out_project(o: np.ndarray, w_o: np.ndarray) -> np.ndarray:
    """y [B, n, D] = concat_h(o[:, h]) w_o^T, the concatenation taking head h's d
    features at columns h*d .. h*d + d - 1."""
    o = np.asarray(o, dtype=np.float64)
    B, H, n, d = o.shape
    cat = np.concatenate([o[:, h] for h in range(H)], axis=-1)     # [B, n, H d]
    return cat @ np.asarray(w_o, dtype=np.float64).T


def nystrom_layer(x, w_qkv, w_o, conv_w, H: int, d: int, m: int, iters: int = 6,
                  lengths=None, qkv_round=None):
    """Projections around the Nystrom core: y = out_project(nystrom(qkv_project(x))).
    ``qkv_round`` optionally maps the projected Q, K, V through a storage format (for
    example bf16 rounding) before the core, as a device path that stores them would."""
    q, k, v = qkv_project(x, w_qkv, H, d)
    if qkv_round is not None:
        q, k, v = qkv_round(q), qkv_round(k), qkv_round(v)
    out, _ = nystrom_forward(q, k, v, conv_w, m, iters, lengths=lengths)
    return out_project(out, w_o)
