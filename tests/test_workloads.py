"""Seeded input generation: shapes, dtypes, determinism and the bias recipes."""
import math

import numpy as np
import torch

import oracle.moe_oracle as O
from workloads import PRESETS, generate, to_numpy
from workloads.configs import ORDER


def test_presets_match_the_listed_shapes():
    c = PRESETS
    assert [c[n].T for n in ORDER] == [256, 8192, 4096, 64, 8192]
    assert c["pages_worked_shape"].batch * c["pages_worked_shape"].seq == 8192
    assert (c["pages_worked_shape"].H, c["pages_worked_shape"].E, c["pages_worked_shape"].F) == (4096, 64, 16384)
    assert c["fine_grained_skewed"].k == 8 and c["fine_grained_skewed"].E == 256


def test_tiny_generation_is_deterministic_and_shaped():
    cfg = PRESETS["tiny_f32"]
    a = generate(cfg)
    b = generate(cfg)
    for key in ("x", "w_gate", "w_in", "w_up", "w_out"):
        assert torch.equal(a[key], b[key])
    assert a["x"].shape == (256, 128) and a["x"].dtype == torch.float32
    assert a["w_in"].shape == (8, 128, 256) and a["w_out"].shape == (8, 256, 128)
    assert a["bias"] is None
    # N(0, 1/fan_in) scale
    assert abs(a["w_in"].std().item() * math.sqrt(128) - 1) < 0.02
    assert abs(a["w_out"].std().item() * math.sqrt(256) - 1) < 0.02


def test_bf16_inputs_are_rounded_once():
    cfg = PRESETS["mixtral_style"].with_(T=16, H=64, F=128, E=4)
    a = generate(cfg)
    assert a["x"].dtype == torch.bfloat16 and a["w_gate"].dtype == torch.float32
    assert a["bias"].dtype == torch.float32
    assert abs(a["bias"].double().var().item() - 0.5) < 0.5    # 4 draws only: loose


def test_zipf_bias_recipe():
    cfg = PRESETS["fine_grained_skewed"]
    b = generate(cfg.with_(T=2, H=8, F=8), experts=False)["bias"].double().numpy()
    r = np.exp(-b / 1.1)
    assert np.allclose(np.sort(r), np.arange(1, 257), rtol=1e-5)


def test_tiny_oracle_runs_in_well_under_a_second():
    import time
    cfg = PRESETS["tiny_f32"]
    a = generate(cfg)
    w = (to_numpy(a["w_in"]), to_numpy(a["w_up"]), to_numpy(a["w_out"]))
    t0 = time.perf_counter()
    r = O.forward(to_numpy(a["x"]), to_numpy(a["w_gate"]), None, w, cfg.k, cfg.ffn)
    assert time.perf_counter() - t0 < 5.0
    assert int(r["counts"].sum()) == cfg.T * cfg.k
    assert r["out"].shape == (cfg.T, cfg.H)
