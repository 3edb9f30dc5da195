"""Pins for the projection oracle (oracle/projections.py) against brute force and closed
forms, plus planted mistakes that the pins must catch."""
import types

import numpy as np
import pytest

from oracle import nystrom as orc
from oracle import projections as prj


def _ns(**over):
    ns = types.SimpleNamespace(qkv_project=prj.qkv_project, out_project=prj.out_project)
    for k, v in over.items():
        setattr(ns, k, v)
    return ns


def pin_qkv_bruteforce(ns) -> float:
    """Every projected element as an explicit dot product over the model width."""
    rng = np.random.default_rng(41)
    B, n, D, H, d = 2, 5, 6, 2, 3
    x = rng.standard_normal((B, n, D))
    w = rng.standard_normal((3 * H * d, D))
    got = ns.qkv_project(x, w, H, d)
    worst = 0.0
    for which in range(3):
        for b in range(B):
            for h in range(H):
                for t in range(n):
                    for f in range(d):
                        row = (which * H + h) * d + f
                        acc = 0.0
                        for c in range(D):
                            acc += float(x[b, t, c]) * float(w[row, c])
                        worst = max(worst, abs(acc - got[which][b, h, t, f]))
    return worst


def pin_out_bruteforce(ns) -> float:
    rng = np.random.default_rng(43)
    B, H, n, d, D = 2, 3, 4, 2, 5
    o = rng.standard_normal((B, H, n, d))
    w = rng.standard_normal((D, H * d))
    got = ns.out_project(o, w)
    worst = 0.0
    for b in range(B):
        for t in range(n):
            for j in range(D):
                acc = 0.0
                for h in range(H):
                    for f in range(d):
                        acc += float(o[b, h, t, f]) * float(w[j, h * d + f])
                worst = max(worst, abs(acc - got[b, t, j]))
    return worst


def pin_identity_round_trip(ns) -> float:
    """D = H d and identity blocks: head h of Q/K/V is (1, 2, 3) x features h*d..h*d+d-1,
    and the output projection with the identity concatenates them back into x."""
    rng = np.random.default_rng(47)
    B, n, H, d = 2, 7, 3, 4
    D = H * d
    x = rng.standard_normal((B, n, D))
    eye = np.eye(D)
    q, k, v = ns.qkv_project(x, np.concatenate([eye, 2 * eye, 3 * eye]), H, d)
    worst = 0.0
    for h in range(H):
        sl = x[:, :, h * d:(h + 1) * d]
        worst = max(worst, np.abs(q[:, h] - sl).max(), np.abs(k[:, h] - 2 * sl).max(),
                    np.abs(v[:, h] - 3 * sl).max())
    worst = max(worst, np.abs(ns.out_project(v / 3.0, eye) - x).max())
    return worst


PINS = {"qkv_bruteforce": (pin_qkv_bruteforce, 1e-12),
        "out_bruteforce": (pin_out_bruteforce, 1e-12),
        "identity_round_trip": (pin_identity_round_trip, 1e-13)}


@pytest.mark.parametrize("name", sorted(PINS))
def test_projection_pin(name):
    fn, tol = PINS[name]
    err = fn(_ns())
    assert err <= tol, f"{name}: {err:.3e}"


def _qkv_transposed(x, w, H, d):
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    out = []
    for which in range(3):
        heads = []
        for h in range(H):
            rows = w[(which * H + h) * d:(which * H + h + 1) * d]
            heads.append(x[..., :d] @ rows[:, :d].T if x.shape[-1] != d else x @ rows)
        out.append(np.stack(heads, axis=1))
    return tuple(out)


def _qkv_head_interleaved(x, w, H, d):
    # rows taken as [head][which][d] instead of [which][head][d]
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    out = []
    for which in range(3):
        out.append(np.stack([x @ w[(h * 3 + which) * d:(h * 3 + which + 1) * d].T
                             for h in range(H)], axis=1))
    return tuple(out)


def _out_feature_major(o, w):
    # concatenation feature-major (f * H + h) instead of head-major
    o = np.asarray(o, dtype=np.float64)
    B, H, n, d = o.shape
    cat = np.transpose(o, (0, 2, 3, 1)).reshape(B, n, d * H)
    return cat @ np.asarray(w, dtype=np.float64).T


MUTANTS = {"qkv_transposed": dict(qkv_project=_qkv_transposed),
           "qkv_head_interleaved": dict(qkv_project=_qkv_head_interleaved),
           "out_feature_major": dict(out_project=_out_feature_major)}


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_projection_pins_catch_planted_mistakes(mutant):
    ns = _ns(**MUTANTS[mutant])
    failed = []
    for name, (fn, tol) in PINS.items():
        try:
            err = fn(ns)
        except Exception:
            err = np.inf
        if not (err <= tol):
            failed.append(name)
    assert failed, f"no pin catches {mutant}"


def test_layer_composition():
    """nystrom_layer is the composition of the pinned pieces (identity projections give
    the core on the head-split input, concatenated back)."""
    rng = np.random.default_rng(53)
    B, n, H, d, m = 1, 32, 2, 4, 8
    D = H * d
    x = rng.standard_normal((B, n, D))
    w = rng.standard_normal((H, 5)) * 0.2
    eye = np.eye(D)
    y = prj.nystrom_layer(x, np.concatenate([eye, eye, eye]), eye, w, H, d, m, 6)
    xs = np.stack([x[:, :, h * d:(h + 1) * d] for h in range(H)], axis=1)
    core, _ = orc.nystrom_forward(xs, xs, xs, w, m, 6)
    ref = np.concatenate([core[:, h] for h in range(H)], axis=-1)
    assert np.abs(y - ref).max() < 1e-12
