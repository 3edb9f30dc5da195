"""GPU parity of uneven segments (m not dividing the valid length) and padded (ragged)
batches against the fp64 oracle, through the C ABI (nys_attn_forward_varlen).

Reading checked (the page defines neither): token t of a length-L sequence belongs to
segment floor(t m / L); a batch element with valid length L_b gives the forward of its
unpadded length-L_b prefix on rows [0, L_b) and zeros on rows [L_b, n). The criteria are
those of test_gpu_parity.py on the valid rows (tau * rms over the valid rows, error
beyond bf16 storage rounding <= 2e-3 * rms, stage taps), plus exact zeros on padding
rows of the output and of the attention tap.
"""
import numpy as np
import pytest

import oracle
from efficient_transformer_attention_segment_amd import inputs as gen
from hip_path import excess_over_rounding, log, rel_max_err, run_hip, stage_tol, tau_for

pytestmark = pytest.mark.gpu


# (config, lengths or None)
CASES = {
    # m does not divide n; no padding
    "uneven_n1000_m64": (gen.Config("u1", 2, 2, 1000, 64, 64, seed=51), None),
    "uneven_n777_m40": (gen.Config("u2", 1, 2, 777, 64, 40, seed=52), None),
    "uneven_f32_n300_m16": (gen.Config("u3", 1, 2, 300, 32, 16, dtype=gen.F32, seed=53), None),
    "uneven_n1000_m96": (gen.Config("u4", 1, 2, 1000, 64, 96, seed=54), None),
    "uneven_n129_m128": (gen.Config("u5", 1, 2, 129, 64, 128, seed=55), None),
    # padded batches; 70 leaves most context chunks and output blocks of that element empty
    "ragged_b3_m64": (gen.Config("r1", 3, 2, 1024, 64, 64, seed=61), [1024, 987, 70]),
    "ragged_f32_m40": (gen.Config("r2", 2, 2, 600, 64, 40, dtype=gen.F32, seed=62), [600, 333]),
    "ragged_conv65": (gen.Config("r3", 2, 2, 512, 64, 64, conv_width=65, seed=63), [100, 512]),
    "ragged_d128_m128": (gen.Config("r4", 2, 1, 1024, 128, 128, seed=64), [1024, 300]),
    "ragged_m1": (gen.Config("r5", 4, 1, 100, 64, 1, seed=65), [1, 2, 50, 100]),
    "ragged_len_m_and_m_plus_1": (gen.Config("r6", 2, 2, 200, 64, 8, seed=66), [8, 9]),
    "ragged_m32_step128": (gen.Config("r7", 2, 2, 1000, 64, 32, seed=67), [999, 129]),
    # 8-wave output blocks (256-token steps): Kt read from L2 at d = 64, m = 256; and at
    # d = 128 with lengths that cut a step and a block
    "ragged_m256_8waves": (gen.Config("r8", 2, 1, 2048, 64, 256, seed=69), [2048, 700]),
    "ragged_d128_8waves": (gen.Config("r9", 2, 1, 2304, 128, 128, seed=70), [1500, 2303]),
    # fp32 I/O with m > 64 (online softmax over landmark tiles, fp32 staging)
    "ragged_f32_m128": (gen.Config("r10", 2, 2, 1024, 64, 128, dtype=gen.F32, seed=71),
                        [1024, 500]),
    "uneven_f32_n1000_m96": (gen.Config("r11", 1, 2, 1000, 32, 96, dtype=gen.F32, seed=72),
                             None),
}


def _check(cfg, x, lengths, heads=None, full_size=False):
    out, taps = run_hip(x, taps=heads is None, lengths=lengths)
    lens = [cfg.n] * cfg.B if lengths is None else list(lengths)
    pairs = heads or [(b, h) for b in range(cfg.B) for h in range(cfg.H)]
    ref, ref_attn, stages = oracle.nystrom_forward(
        x.q, x.k, x.v, x.w, cfg.m, cfg.pinv_iters, heads=pairs, return_stages=True,
        lengths=lengths)
    tau = tau_for(cfg.dtype)
    got = np.stack([out[b, h] for b, h in pairs])
    valid = [np.arange(cfg.n) < lens[b] for b, _ in pairs]
    gv = np.concatenate([g[v] for g, v in zip(got, valid)])
    rv = np.concatenate([r[v] for r, v in zip(ref, valid)])
    e_full = rel_max_err(gv, rv)
    e_ex = excess_over_rounding(gv, rv, cfg.dtype)
    pad_out = max((float(np.abs(g[~v]).max()) if (~v).any() else 0.0) for g, v in zip(got, valid))
    res = {"full": e_full, "beyond-rounding": e_ex, "padding |out|": pad_out}
    if taps:
        ga = np.stack([taps["attn"].reshape(cfg.B, cfg.H, cfg.n, cfg.d)[b, h] for b, h in pairs])
        res["attn"] = rel_max_err(np.concatenate([g[v] for g, v in zip(ga, valid)]),
                                  np.concatenate([r[v] for r, v in zip(ref_attn, valid)]))
        res["padding |attn|"] = max((float(np.abs(g[~v]).max()) if (~v).any() else 0.0)
                                    for g, v in zip(ga, valid))
        for key in stage_tol(cfg):
            res[key] = max(rel_max_err(taps[key][b * cfg.H + h], st[key])
                           for (b, h), st in zip(pairs, stages))
    log("[gpu]   " + "  ".join(f"{k} {v:.3e}" for k, v in res.items()))
    assert e_full <= tau and e_ex <= 2e-3
    assert pad_out == 0.0
    if taps:
        assert res["attn"] <= tau and res["padding |attn|"] == 0.0
        for key, tol in stage_tol(cfg, full_size).items():
            assert res[key] <= tol, (key, res[key])


@pytest.mark.parametrize("name", sorted(CASES))
def test_uneven_and_ragged_parity(name):
    cfg, lengths = CASES[name]
    log(f"[gpu] ragged/uneven case {name}: {cfg} lengths={lengths}")
    _check(cfg, gen.make_inputs(cfg), lengths)


@pytest.mark.timeout(600)
def test_ragged_full_workload_every_head():
    """The benchmark shape with seeded lengths in [n/2, n], in the launch configuration
    of the dense benchmark: every element of every head, with every stage tap."""
    cfg = gen.CONFIGS["long"]
    lengths = gen.ragged_lengths(cfg, seed=cfg.seed)
    log(f"[gpu] ragged full workload {cfg} lengths={lengths}")
    x = gen.make_inputs(cfg)
    _check(cfg, x, lengths, full_size=True)


def test_dense_lengths_match_plain_forward():
    """lengths = n everywhere gives bit-identical output to the plain forward."""
    cfg = gen.Config("eq", 2, 2, 512, 64, 64, seed=68)
    x = gen.make_inputs(cfg)
    a, _ = run_hip(x)
    b, _ = run_hip(x, lengths=[cfg.n] * cfg.B)
    assert np.array_equal(a, b)
