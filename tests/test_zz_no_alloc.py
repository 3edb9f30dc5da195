"""The allocation-free forward (nys_attn_forward_noalloc) against the plan-based forward
(nys_attn_forward), through the C ABI: two calls in a row on the static scratch, the
second with a smaller problem (the scratch then holds the first call's data), each
compared with a fresh plan's output on the same inputs. Both paths run the same kernels
with the same launch geometry, so the outputs must agree bit for bit, which is stronger
than the parity bound (max |difference| <= 2e-2 RMS for bf16 I/O, 2e-3 for fp32), also
checked. A third call with m not a multiple of 32 exercises the clearing of the landmark
padding rows that the first calls left behind."""
import ctypes

import numpy as np
import pytest

from efficient_transformer_attention_segment_amd import inputs as gen
from hip_path import log, rel_max_err, run_hip, tau_for, upload

pytestmark = pytest.mark.gpu


def _noalloc(x):
    import torch
    from efficient_transformer_attention_segment_amd import _lib
    cfg = x.cfg
    q, k, v, w = upload(x)
    dt = torch.bfloat16 if cfg.dtype == gen.BF16 else torch.float32
    out = torch.full((cfg.B, cfg.H, cfg.n, cfg.d), float("nan"), dtype=dt, device="cuda")
    code = _lib.NYS_BF16 if cfg.dtype == gen.BF16 else _lib.NYS_F32
    stream = torch.cuda.current_stream().cuda_stream
    _lib.nys_attn_forward_noalloc(cfg.B, cfg.H, cfg.n, cfg.d, cfg.m, cfg.conv_width,
                                  cfg.pinv_iters, code, q.data_ptr(), k.data_ptr(),
                                  v.data_ptr(), w.data_ptr(), out.data_ptr(), stream)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64)


CALLS = [
    gen.CONFIGS["long"],                                     # the benchmark workload
    gen.CONFIGS["bert"].with_(B=4, H=3, seed=1102),          # smaller, second call
    gen.Config("pad", 2, 3, 600, 64, 40, seed=1103),         # m = 40: padded landmark rows
    gen.Config("f32", 1, 2, 512, 128, 96, dtype=gen.F32, seed=1104),
]


def test_noalloc_matches_plan_forward_on_consecutive_calls():
    for cfg in CALLS:
        log(f"[gpu] allocation-free forward vs plan forward: {cfg}")
        x = gen.make_inputs(cfg)
        got = _noalloc(x)
        ref, _ = run_hip(x)
        err = rel_max_err(got, ref)
        log(f"[gpu]   max |noalloc - plan| / rms = {err:.3e}, "
            f"identical: {np.array_equal(got, ref)}")
        assert np.isfinite(got).all()
        assert err <= tau_for(cfg.dtype)
        assert np.array_equal(got, ref)


def test_noalloc_rejects_oversized_workspace():
    """A shape whose workspace exceeds the static scratch fails with NYS_E_UNSUPPORTED and
    a message naming both sizes, before anything is launched."""
    from efficient_transformer_attention_segment_amd import _lib
    null = ctypes.c_void_p(16)
    st = _lib.lib().nys_attn_forward_noalloc(64, 16, 16384, 64, 256, 33, 6, _lib.NYS_BF16,
                                             null, null, null, null, null, None)
    assert st == _lib.NYS_E_UNSUPPORTED
    assert "static scratch" in _lib.nys_attn_last_error()
