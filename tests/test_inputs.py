"""Seeded input recipes: determinism, distributions and bf16 rounding (CPU only)."""
import numpy as np
import pytest

import kla_inputs as KI


def test_bf16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10.0 ** rng.integers(-30, 30, 100000),
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3.4e38, 1e-40], np.float32)])
    x = x.astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(KI.bf16_bits(x), ref)
    r = KI.round_bf16(x)
    np.testing.assert_array_equal(r, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_ties_round_to_even():
    # 1 + 2^-8 sits exactly between 1 and 1 + 2^-7: ties go to the even mantissa (1.0)
    x = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8], np.float32)
    np.testing.assert_array_equal(KI.round_bf16(x), np.array([1.0, 1.0 + 2 ** -6], np.float32))


def test_forward_inputs_deterministic_and_shaped():
    a = KI.make_forward_inputs(0)
    b = KI.make_forward_inputs("tiny_f32")
    for name in ("q", "k", "v", "log_decay", "proc_noise", "val_prec"):
        np.testing.assert_array_equal(a[name], b[name])
    assert a["q"].shape == (1, 1, 256, 16) and a["v"].shape == (1, 1, 256, 16)
    assert a["dtype"] == "f32" and a["seed"] == 1000
    assert np.all(a["log_decay"] < 0) and np.all(a["proc_noise"] > 1e-3 - 1e-9)
    assert np.all(a["val_prec"] > 0)
    np.testing.assert_array_equal(a["lambda0"], 1.0)
    np.testing.assert_array_equal(a["M0"], 0.0)


def test_bf16_workload_values_are_bf16():
    x = KI.make_forward_inputs(1, B=1, H=2, T=64)
    for name in ("q", "k", "v", "log_decay", "proc_noise", "val_prec"):
        np.testing.assert_array_equal(KI.round_bf16(x[name]), x[name])


def test_distribution_moments():
    x = KI.make_forward_inputs(1, B=2, H=2, T=2048)
    assert abs(x["q"].var() * 64 - 1) < 0.02 and abs(x["v"].var() - 1) < 0.02
    sp = -x["log_decay"]
    assert abs(sp.mean() - 0.8066) < 0.02   # E softplus(N(0,1)) = 0.8066...


def test_spike_mask_fraction():
    w = KI.workload(2)
    x = KI.make_forward_inputs(w, B=2, H=3, T=2048)
    base = KI.make_forward_inputs(KI.Workload(99, "x", "forward", 2, 3, 2048, 64, 64, "bf16"),
                                  seed=w.seed)
    spiked = np.all(x["val_prec"] != base["val_prec"], axis=-1)
    assert abs(spiked.mean() - 0.05) < 0.006
    # a spike scales every d_k entry of the token's value precision
    np.testing.assert_array_equal(np.any(x["val_prec"] != base["val_prec"], axis=-1), spiked)


def test_precision_inputs():
    x = KI.make_precision_inputs(B=1, H=2, T=100, D=64)
    assert x["obs_prec"].dtype == np.float32 and np.all(x["obs_prec"] >= 0)
    assert np.all(x["proc_noise"] > 0)
    y = KI.make_precision_inputs(B=1, H=2, T=100, D=64)
    np.testing.assert_array_equal(x["log_decay"], y["log_decay"])
