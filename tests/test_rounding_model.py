"""Why the self-attention path misses G1's max bound at score std ~4: the
bf16 rounding of its MFMA operands (rotated and scaled q, rotated k, the
probabilities), modelled in numpy (tests/rounding_model.py), alone puts the
result that far from the fp64 oracle; at the workloads' spread (score std
0.25) and at the peaked test inputs (std ~2.25) it stays inside G1 and G2.

The GPU side of the argument (the kernel lands within rounding noise of the
model, tests/test_gpu_g3.py) needs a GPU; this file is CPU only.
"""
import numpy as np
import pytest

import oracle
import rounding_model as rm
from parity_util import MAX_ABS, MEAN_ABS, REL_RMS
from video_diffusion_transformer_wanattn_amd import seeded


def inputs(N, heads, seed, sigma):
    q, k = (seeded.normal_bf16((1, N, heads, 128), seed, s, sigma) for s in (1, 2))
    v = seeded.normal_bf16((1, N, heads, 128), seed, 3, 0.5)
    return q, k, v


def model_vs_oracle(grid, heads, seed, sigma):
    N = int(np.prod(grid))
    q, k, v = inputs(N, heads, seed, sigma)
    emu = rm.self_attention(q[0], k[0], v[0], grid).astype(np.float64)
    ref = oracle.self_rows(q, k, v, grid)[0]
    d = emu - ref
    return {"max_abs": float(np.max(np.abs(d))), "mean_abs": float(np.mean(np.abs(d))),
            "rel_rms": float(np.sqrt(np.mean(d * d)) / np.sqrt(np.mean(ref * ref)))}


def test_model_pins():
    # the model's pieces against closed forms: rotation at position 0 is the
    # identity, pair 0 at frame f turns by exactly f radians, and bf16 rounds
    # to nearest even
    x = seeded.normal_bf16((3, 128), 5, 1, 1.0)
    xf = seeded.bf16_bits_to_f32(x)
    np.testing.assert_array_equal(rm.rotate_fp32(x, np.zeros((3, 3), int), 1e4), xf)
    r = rm.rotate_fp32(x, np.array([[2, 0, 0]] * 3), 1e4)
    c, s = np.cos(2.0), np.sin(2.0)
    np.testing.assert_allclose(r[:, 0], xf[:, 0] * c - xf[:, 1] * s, rtol=1e-6, atol=1e-6)
    assert rm.bf16(np.float32(1.0 + 2 ** -8)) == 1.0          # tie to even
    assert rm.bf16(np.float32(1.0 + 3 * 2 ** -8)) == 1.0 + 2 ** -6


# The GPU test of the split tail at sigma 2 (tests/test_gpu_split.py) runs 40
# heads of 2000 tokens and compares heads 0 and 32..39 (the split heads on a
# 256-CU chip), where the kernel measured max |err| 0.0255 unsplit, 0.0242 split.
SIGMA2_HEADS = np.array([0] + list(range(32, 40)))


def sigma2_case():
    grid, N, heads = (5, 20, 20), 2000, 40
    q, k, v = inputs(N, heads, 913, 2.0)
    hs = SIGMA2_HEADS
    return grid, q[:, :, hs], k[:, :, hs], v[:, :, hs]


def test_bf16_operands_alone_miss_g1_max_at_score_std_4():
    grid, q, k, v = sigma2_case()
    ref = oracle.self_rows(q, k, v, grid)[0]
    emu = rm.self_attention(q[0], k[0], v[0], grid).astype(np.float64)
    d = emu - ref
    e = {"max_abs": float(np.max(np.abs(d))), "rel_rms": float(np.sqrt(np.mean(d * d) / np.mean(ref * ref)))}
    print("model vs oracle, sigma 2:", e)
    assert e["max_abs"] > MAX_ABS          # G1's max is missed by the arithmetic itself
    assert e["rel_rms"] <= REL_RMS
    # which rounding: the bf16 q' and k' operands alone miss it; the
    # probabilities' or the output's rounding alone stay well inside
    err = lambda *r: float(np.max(np.abs(rm.with_roundings(q, k, v, grid, *r) - ref)))
    qk, pp, oo = err(True, False, False), err(False, True, False), err(False, False, True)
    print(f"max |err| with only q'/k' rounded {qk:.4f}, only p {pp:.4f}, only o {oo:.4f}")
    assert qk > MAX_ABS and pp < 0.25 * MAX_ABS and oo < 0.5 * MAX_ABS


@pytest.mark.parametrize("sigma", [0.5, 1.5])
def test_bf16_operands_within_gates_at_test_spreads(sigma):
    e = model_vs_oracle((5, 20, 20), 2, 914, sigma)
    print(f"model vs oracle, sigma {sigma}:", e)
    assert e["max_abs"] <= MAX_ABS and e["mean_abs"] <= MEAN_ABS and e["rel_rms"] <= REL_RMS


def test_error_grows_with_score_spread():
    es = [model_vs_oracle((3, 10, 10), 2, 915, s)["rel_rms"] for s in (0.5, 1.0, 1.5, 2.0)]
    print("rel_rms by sigma 0.5 .. 2:", es)
    assert all(a < b for a, b in zip(es, es[1:]))
