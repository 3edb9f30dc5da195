"""Helpers shared by the GPU tests: run the HIP path through the binding on seeded
inputs, and compare with the oracle. (Not a test module.)"""
from __future__ import annotations

import sys

import numpy as np


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev_tensor(x_dev: np.ndarray, dtype: str):
    import torch
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(x_dev).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(x_dev, dtype=np.float32))
    return t.to("cuda")


def upload(x):
    import torch
    cfg = x.cfg
    q, k, v = (dev_tensor(a, cfg.dtype) for a in (x.q_dev, x.k_dev, x.v_dev))
    w = torch.from_numpy(np.ascontiguousarray(x.w, dtype=np.float32)).to("cuda")
    return q, k, v, w


def make_taps(cfg):
    import torch
    BH, m, n, d = cfg.bh, cfg.m, cfg.n, cfg.d
    f = lambda *s: torch.empty(*s, dtype=torch.float32, device="cuda")
    return dict(q_land=f(BH, m, d), k_land=f(BH, m, d), a_s=f(BH, m, m), z=f(BH, m, m),
                w=f(BH, m, d), y=f(BH, m, d), attn=f(BH, n, d))


def run_hip(x, taps: bool = False, iters: int | None = None, att=None, lengths=None):
    """Forward on the GPU (``lengths``: valid length per batch element, or None).
    Returns (out fp64 [B,H,n,d], taps dict of fp64 arrays)."""
    import torch
    from efficient_transformer_attention_segment_amd import NystromAttention
    cfg = x.cfg
    it = cfg.pinv_iters if iters is None else iters
    own = att is None
    if own:
        att = NystromAttention(cfg.B, cfg.H, cfg.n, cfg.d, cfg.m, cfg.conv_width, it, cfg.dtype)
    q, k, v, w = upload(x)
    tp = make_taps(cfg) if taps else None
    out = att.forward(q, k, v, w, taps=tp, lengths=lengths)
    torch.cuda.synchronize()
    o = out.float().cpu().numpy().astype(np.float64)
    t = {key: val.cpu().numpy().astype(np.float64) for key, val in (tp or {}).items()}
    if own:
        att.close()
    return o, t


def tau_for(dtype: str) -> float:
    """Parity tolerance on max|GPU - oracle| relative to the oracle output's RMS:
    2e-3 for fp32 I/O, 2e-2 for bf16 I/O with fp32 accumulation."""
    return 2e-3 if dtype == "f32" else 2e-2


def rel_max_err(got, ref) -> float:
    rms = float(np.sqrt(np.mean(np.square(ref))))
    return float(np.max(np.abs(got - ref))) / rms if rms > 0 else float(np.max(np.abs(got - ref)))


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    """Spacing of bf16 numbers at |x| (8 significant bits)."""
    ax = np.maximum(np.abs(x), np.finfo(np.float32).tiny)
    return np.exp2(np.floor(np.log2(ax)) - 7.0)


def excess_over_rounding(got: np.ndarray, ref: np.ndarray, dtype: str) -> float:
    """max(|got - ref| - half an output ulp, 0) / rms(ref): the error a bf16 result has
    beyond the rounding of the exact value to its storage format (0 ulp for fp32)."""
    rms = float(np.sqrt(np.mean(np.square(ref))))
    err = np.abs(got - ref)
    if dtype == "bf16":
        err = np.maximum(err - 0.5 * bf16_ulp(np.maximum(np.abs(got), np.abs(ref))), 0.0)
    return float(err.max()) / rms
