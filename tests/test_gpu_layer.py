"""GPU parity of the projections around the core (nys_proj_qkv, nys_proj_out) and of the
projected layer (projections + Nystrom forward) against the fp64 oracle in
oracle/projections.py, through the C ABI.

Criteria. A projection output is a bf16 rounding of an fp32-accumulated dot product of
exact bf16 inputs, so it must lie within half a bf16 ulp of the exact fp64 value plus
the fp32 accumulation error (bounded here by 1e-5 of the output RMS). The layer stores
Q, K, V and the attention output O in bf16 on the device, so its reference applies the
same storage rounding to the oracle's Q, K, V and O; the layer output y is bf16 as well,
and its own rounding alone (half an ulp of the largest |y|, about 2e-2 of the RMS on the
full-size workload, whose largest outputs reach 10 times the RMS) is not arithmetic
error. No page fixes a tolerance for the layer. The one used: the error beyond half a
bf16 ulp of y must stay <= 5e-3 RMS (LAYER_EXCESS; the full max-abs error and the
rounding floor are printed next to it). It is looser than the core's 2e-3 because the
core's own error in O (up to ~1e-3 of its RMS), and the bf16 rounding steps of O that this
error flips, pass through the output projection: measured 2.3e-3 at B=2, H=4, D=256.
"""
import numpy as np
import pytest

import oracle
from efficient_transformer_attention_segment_amd import inputs as gen
from hip_path import bf16_ulp, dev_tensor, excess_over_rounding, log, rel_max_err

pytestmark = pytest.mark.gpu

# (B, H, n, d, D): ragged token tiles (B n not a multiple of 128), feature tiles that
# end mid-tile (3 H d or D not multiples of 128), one k-slab (64) and many.
LAYER_EXCESS = 5e-3

PROJ_SHAPES = [
    (1, 1, 64, 64, 64),
    (2, 2, 100, 64, 128),
    (1, 6, 300, 32, 192),
    (3, 1, 129, 128, 256),
    (2, 4, 256, 64, 768),
    (1, 2, 200, 128, 448),
]


def _bf16_round(a):
    return gen.bf16_bits_to_f32(gen.f32_to_bf16_bits(a.astype(np.float32))).astype(np.float64)


def _within_rounding(got, ref, what):
    rms = float(np.sqrt(np.mean(np.square(ref))))
    excess = np.abs(got - ref) - 0.5 * bf16_ulp(ref)
    worst = float(excess.max()) / rms
    log(f"[gpu]   {what}: rel max err {rel_max_err(got, ref):.3e}, beyond rounding {worst:.3e}")
    assert worst <= 1e-5, what


def _proj_qkv(li):
    import torch
    from efficient_transformer_attention_segment_amd import nys_proj_qkv
    cfg = li.cfg
    x = dev_tensor(li.x_dev, "bf16")
    w = dev_tensor(li.w_qkv_dev, "bf16")
    q, k, v = (torch.full((cfg.B, cfg.H, cfg.n, cfg.d), float("nan"), dtype=torch.bfloat16,
                          device="cuda") for _ in range(3))
    nys_proj_qkv(x.data_ptr(), w.data_ptr(), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                 cfg.B, cfg.H, cfg.n, cfg.d, li.D, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return [t.float().cpu().numpy().astype(np.float64) for t in (q, k, v)]


def _proj_out(o_dev, w_o_dev, cfg, D):
    import torch
    from efficient_transformer_attention_segment_amd import nys_proj_out
    o = dev_tensor(o_dev, "bf16")
    w = dev_tensor(w_o_dev, "bf16")
    y = torch.full((cfg.B, cfg.n, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    nys_proj_out(o.data_ptr(), w.data_ptr(), y.data_ptr(), cfg.B, cfg.H, cfg.n, cfg.d, D,
                 torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return y.float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("shape", PROJ_SHAPES, ids=lambda s: "B%d_H%d_n%d_d%d_D%d" % s)
def test_qkv_projection(shape):
    B, H, n, d, D = shape
    cfg = gen.Config("proj", B, H, n, d, 8, seed=71 + sum(shape))
    log(f"[gpu] qkv projection {shape}")
    li = gen.make_layer_inputs(cfg, D)
    got = _proj_qkv(li)
    ref = oracle.qkv_project(li.x, li.w_qkv, H, d)
    for name, g, r in zip("qkv", got, ref):
        _within_rounding(g, r, name)


@pytest.mark.parametrize("shape", PROJ_SHAPES, ids=lambda s: "B%d_H%d_n%d_d%d_D%d" % s)
def test_out_projection(shape):
    B, H, n, d, D = shape
    cfg = gen.Config("proj", B, H, n, d, 8, seed=91 + sum(shape))
    log(f"[gpu] output projection {shape}")
    li = gen.make_layer_inputs(cfg, D)
    rng = np.random.default_rng(cfg.seed)
    o_dev = gen.f32_to_bf16_bits(rng.standard_normal((B, H, n, d), dtype=np.float32))
    o = gen.bf16_bits_to_f32(o_dev).astype(np.float64)
    got = _proj_out(o_dev, li.w_o_dev, cfg, D)
    _within_rounding(got, oracle.out_project(o, li.w_o), "y")


def _layer_ref(li, lengths=None, b=None):
    """Oracle layer output with the device's storage formats: Q, K, V and the attention
    output O rounded to bf16 before they are used again (batch element b, or all)."""
    cfg = li.cfg
    sl = slice(None) if b is None else slice(b, b + 1)
    q, k, v = (_bf16_round(t) for t in oracle.qkv_project(li.x[sl], li.w_qkv, cfg.H, cfg.d))
    lens = None if lengths is None else (lengths if b is None else [lengths[b]])
    o, _ = oracle.nystrom_forward(q, k, v, li.w, cfg.m, cfg.pinv_iters, lengths=lens)
    return oracle.out_project(_bf16_round(o), li.w_o)


def _layer_gpu(li, lengths=None, keep=None):
    import torch
    from efficient_transformer_attention_segment_amd import NystromLayer
    cfg = li.cfg
    layer = NystromLayer(cfg.B, cfg.H, cfg.n, cfg.d, cfg.m, li.D, cfg.conv_width,
                         cfg.pinv_iters)
    x = dev_tensor(li.x_dev, "bf16")
    wq = dev_tensor(li.w_qkv_dev, "bf16")
    wo = dev_tensor(li.w_o_dev, "bf16")
    w = torch.from_numpy(li.w).to("cuda")
    y = layer.forward(x, wq, wo, w, lengths=lengths)
    torch.cuda.synchronize()
    y = y[keep] if keep is not None else y
    out = y.float().cpu().numpy().astype(np.float64)
    layer.close()
    return out


LAYER_CASES = {
    "bert_like_small": (gen.Config("l1", 2, 4, 512, 64, 64, seed=81), 256, None),
    "uneven_D_wider": (gen.Config("l2", 1, 2, 1000, 64, 40, seed=82), 192, None),
    "ragged": (gen.Config("l3", 3, 2, 600, 64, 32, seed=83), 128, [600, 333, 64]),
    "d128": (gen.Config("l4", 1, 2, 512, 128, 64, seed=84), 256, None),
}


@pytest.mark.parametrize("name", sorted(LAYER_CASES))
def test_layer_parity(name):
    cfg, D, lengths = LAYER_CASES[name]
    log(f"[gpu] layer case {name}: {cfg} D={D} lengths={lengths}")
    li = gen.make_layer_inputs(cfg, D)
    got = _layer_gpu(li, lengths)
    ref = _layer_ref(li, lengths)
    lens = lengths or [cfg.n] * cfg.B
    # errors relative to the RMS over valid rows (padding rows are exact zeros, checked below)
    gv = np.concatenate([got[b, :L] for b, L in enumerate(lens)])
    rv = np.concatenate([ref[b, :L] for b, L in enumerate(lens)])
    err, ex = rel_max_err(gv, rv), excess_over_rounding(gv, rv, "bf16")
    pad = max(float(np.abs(got[b, L:]).max()) if L < cfg.n else 0.0 for b, L in enumerate(lens))
    log(f"[gpu]   rel max err {err:.3e}, beyond bf16 rounding {ex:.3e}, padding |y| {pad}")
    assert ex <= LAYER_EXCESS
    assert pad == 0.0


@pytest.mark.timeout(600)
def test_layer_full_size_every_element():
    """The long workload (B 16, H 8, n 4096, d 64, m 64) with model width 512 computed
    whole on the GPU; every batch element checked against the oracle in full, one at a
    time (errors relative to the RMS over the whole output)."""
    from hip_path import HeadStats
    cfg = gen.CONFIGS["long"]
    log(f"[gpu] layer at full size {cfg}, D=512, every batch element")
    li = gen.make_layer_inputs(cfg, 512)
    got = _layer_gpu(li)
    st, floor = HeadStats("bf16"), HeadStats("f32")
    for b in range(cfg.B):
        ref = _layer_ref(li, b=b)[0]
        st.add(got[b], ref)
        floor.add(_bf16_round(ref), ref)
    log(f"[gpu]   rel max err {st.rel:.3e} (bf16 rounding floor {floor.rel:.3e}), "
        f"beyond bf16 rounding {st.excess:.3e}")
    assert st.excess <= LAYER_EXCESS
