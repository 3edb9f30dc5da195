"""The linear-cost claim of the Nystromformer review page ("Main findings": with m much
smaller than n, time and memory grow linearly in n) on this implementation: at fixed
B, H, d, m the forward's time at n = 16384 is 3.2 to 4.8 times its time at n = 4096, and
the plan's workspace grows at most linearly in n (it holds nothing of size n x n)."""
import numpy as np
import pytest

from hip_path import log

pytestmark = pytest.mark.gpu


def _forward_ms(B, H, n, d, m, reps=100):
    import torch
    from efficient_transformer_attention_segment_amd import NystromAttention
    g = torch.Generator(device="cuda").manual_seed(n)
    sets = [tuple(torch.randn((B, H, n, d), generator=g, device="cuda").to(torch.bfloat16)
                  for _ in range(3)) for _ in range(2)]
    w = torch.full((H, 33), 0.02, dtype=torch.float32, device="cuda")
    out = torch.empty((B, H, n, d), dtype=torch.bfloat16, device="cuda")
    att = NystromAttention(B, H, n, d, m)
    ws = att.workspace_bytes
    for i in range(reps):                      # warm-up, clocks up
        att.forward(*sets[i % 2], w, out=out)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record()
    for i in range(reps):
        att.forward(*sets[i % 2], w, out=out)
    ev[1].record()
    torch.cuda.synchronize()
    att.close()
    return ev[0].elapsed_time(ev[1]) / reps, ws


def test_time_and_workspace_linear_in_n():
    B, H, d, m = 16, 8, 64, 64
    t_small, ws_small = _forward_ms(B, H, 4096, d, m)
    t_large, ws_large = _forward_ms(B, H, 16384, d, m)
    ratio = t_large / t_small
    log(f"[gpu] n=4096: {t_small * 1e3:.1f} us, workspace {ws_small} B; n=16384: "
        f"{t_large * 1e3:.1f} us, workspace {ws_large} B; time ratio {ratio:.2f}")
    assert 3.2 <= ratio <= 4.8
    assert ws_large <= 4 * ws_small
    assert ws_large < B * H * 16384 * 16384 * 4 / 100   # far from any n x n buffer
