"""Pins of the FLASH mixed-chunk oracle (oracle/flash.py) against independent routines:

* local part: with the global term removed, the output equals dense attention under a
  block-diagonal mask (torch's fp64 scaled_dot_product_attention with a boolean mask,
  causal inside each block when asked);
* global part: built per query from explicit sums of the outer products K_u^T V_u over
  the keys it covers (every key, or, causal, the keys of earlier chunks), divided by
  their number;
* one chunk (c >= n), non-causal: softmax attention of the whole sequence plus
  s Q (K^T V) / n;
* chunk size 1, causal: the local term is V itself (each token attends only to itself);
* brute force on tiny inputs: a pure-Python triple loop of the definition.

Planted mistakes must each fail a pin.
"""
import numpy as np
import pytest
import torch

from oracle import flash as fl


def _qkv(n, d, seed, H=1):
    rng = np.random.default_rng(seed)
    return tuple(rng.standard_normal((1, H, n, d)) for _ in range(3))


def _global_dense(q, k, v, c, causal):
    """Global term by dense products over explicit token masks."""
    n, d = q.shape
    s = 1.0 / np.sqrt(d)
    out = np.zeros((n, d))
    for t in range(n):
        g = t // c
        keys = [u for u in range(n) if (u // c < g if causal else True)]
        if keys:
            kv = sum(np.outer(k[u], v[u]) for u in keys)
            out[t] = s * (q[t] @ kv) / len(keys)
    return out


def _local_sdpa(q, k, v, c, causal):
    n = q.shape[0]
    idx = np.arange(n)
    mask = (idx[:, None] // c) == (idx[None, :] // c)
    if causal:
        mask &= idx[None, :] <= idx[:, None]
    t = lambda a: torch.tensor(a)[None]
    o = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v),
                                                         attn_mask=torch.tensor(mask)[None])
    return o[0].numpy()


@pytest.mark.parametrize("n,c,causal", [(48, 16, False), (50, 16, False), (48, 16, True),
                                        (37, 8, True), (64, 64, False)])
def test_local_plus_global_against_dense(n, c, causal):
    q, k, v = _qkv(n, 8, seed=n + c)
    got = fl.mixed_chunk_attention(q, k, v, c, causal)[0, 0]
    ref = _local_sdpa(q[0, 0], k[0, 0], v[0, 0], c, causal) + \
        _global_dense(q[0, 0], k[0, 0], v[0, 0], c, causal)
    np.testing.assert_allclose(got, ref, atol=1e-12, rtol=1e-10)


def test_single_chunk_is_full_attention_plus_mean_state():
    n, d = 40, 8
    q, k, v = _qkv(n, d, seed=3)
    got = fl.mixed_chunk_attention(q, k, v, c=64, causal=False)[0, 0]
    qq, kk, vv = q[0, 0], k[0, 0], v[0, 0]
    s = 1.0 / np.sqrt(d)
    lg = s * qq @ kk.T
    p = np.exp(lg - lg.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    ref = p @ vv + s * qq @ (kk.T @ vv) / n
    np.testing.assert_allclose(got, ref, atol=1e-12)


def test_chunk_size_one_causal_local_is_identity():
    n, d = 20, 4
    q, k, v = _qkv(n, d, seed=4)
    got = fl.mixed_chunk_attention(q, k, v, c=1, causal=True)[0, 0]
    glob = _global_dense(q[0, 0], k[0, 0], v[0, 0], 1, True)
    np.testing.assert_allclose(got - glob, v[0, 0], atol=1e-12)


def test_brute_force_tiny():
    n, d, c = 7, 3, 3
    q, k, v = _qkv(n, d, seed=5)
    qq, kk, vv = q[0, 0], k[0, 0], v[0, 0]
    s = 1.0 / np.sqrt(d)
    for causal in (False, True):
        ref = np.zeros((n, d))
        for t in range(n):
            g = t // c
            keys = [u for u in range(n) if u // c == g and (u <= t or not causal)]
            w = [np.exp(s * sum(qq[t][i] * kk[u][i] for i in range(d))) for u in keys]
            z = sum(w)
            for f in range(d):
                ref[t][f] = sum(wi * vv[u][f] for wi, u in zip(w, keys)) / z
            cov = [u for u in range(n) if (u // c < g if causal else True)]
            for f in range(d):
                acc = 0.0
                for u in cov:
                    acc += sum(qq[t][i] * kk[u][i] for i in range(d)) * vv[u][f]
                ref[t][f] += (s * acc / len(cov)) if cov else 0.0
        got = fl.mixed_chunk_attention(q, k, v, c, causal)[0, 0]
        np.testing.assert_allclose(got, ref, atol=1e-12)


# ------------------------------------------------------------------ planted mistakes
def _local_no_scale(q, k, v, causal):
    q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
    logits = q @ k.T
    if causal:
        logits = np.where(np.tril(np.ones(logits.shape, dtype=bool)), logits, -np.inf)
    return fl.softmax_rows(logits) @ v


def _local_anticausal(q, k, v, causal):
    q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
    logits = (q @ k.T) / np.sqrt(q.shape[1])
    if causal:
        logits = np.where(np.triu(np.ones(logits.shape, dtype=bool)), logits, -np.inf)
    return fl.softmax_rows(logits) @ v


def _state_transposed(k, v):
    return (np.asarray(k, dtype=np.float64).T @ np.asarray(v, dtype=np.float64)).T


MUTANTS = {
    "local softmax without 1/sqrt(d)": ("local_attention", _local_no_scale),
    "causal mask reversed": ("local_attention", _local_anticausal),
    "chunk state transposed": ("chunk_state", _state_transposed),
}


def _pins_pass():
    try:
        for args in [(48, 16, False), (48, 16, True), (37, 8, True)]:
            test_local_plus_global_against_dense(*args)
        test_single_chunk_is_full_attention_plus_mean_state()
        test_brute_force_tiny()
    except AssertionError:
        return False
    return True


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistakes(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(fl, attr, fn)
    assert not _pins_pass(), f"mutant '{name}' passes every pin"
