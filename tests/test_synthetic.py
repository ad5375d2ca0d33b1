"""Seeded input generators: determinism, bf16 rounding, mask and row sample."""
import json
import os

import numpy as np
import torch

import synthetic as syn


def test_bf16_rne_matches_torch():
    rng = np.random.Generator(np.random.PCG64(5))
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10,
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3.4e38, -3.4e38,
                                  1e-40, np.inf, -np.inf], np.float32)])
    # ties: 1 + 2^-8 (even -> 1.0) and 1 + 3*2^-8 (even -> 1 + 2^-6)
    ours = syn.bf16_round(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(ours.view(np.uint32), ref.view(np.uint32))
    assert syn.bf16_round(np.array([1.00390625], np.float32))[0] == 1.0
    assert syn.bf16_round(np.array([1.01171875], np.float32))[0] == np.float32(1.015625)
    assert np.isnan(syn.bf16_round(np.array([np.nan], np.float32))[0])


def test_draws_are_seeded_and_ordered():
    a = syn.draw_qkvdo(1, 2, 16, 8, seed=3)
    b = syn.draw_qkvdo(1, 2, 16, 8, seed=3)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    rng = np.random.Generator(np.random.PCG64(3))
    q = rng.standard_normal((1, 2, 16, 8), dtype=np.float32)
    k = rng.standard_normal((1, 2, 16, 8), dtype=np.float32)
    assert np.array_equal(q, a[0]) and np.array_equal(k, a[1])
    c = syn.draw_qkvdo(1, 2, 16, 8, seed=3, qk_mult=2.0)
    assert np.array_equal(c[0], 2 * a[0]) and np.array_equal(c[2], a[2])


def test_config_shapes():
    assert syn.CONFIGS[3].B * syn.CONFIGS[3].H == 32 and syn.CONFIGS[3].N == 8192
    assert syn.CONFIGS[1].scale == np.float32(1 / 8)
    assert syn.CONFIGS[3].scale == float(np.float32(1 / np.sqrt(128)))
    q, k, v, do, mask = syn.config_inputs(syn.CONFIGS[1])
    assert q.shape == (1, 2, 128, 64) and mask is None
    assert np.array_equal(syn.bf16_round(q), q)


def test_block_mask_density_and_band():
    m = syn.block_mask(128)
    nb = 128
    I, J = np.meshgrid(np.arange(nb), np.arange(nb), indexing="ij")
    band = np.abs(I - J) <= 1
    assert np.all(m[band] == 1)
    assert band.sum() == 382
    assert int(m.sum()) == 382 + 1600
    assert abs(m.mean() - 1982 / 16384) < 1e-12
    assert np.array_equal(m, syn.block_mask(128))


def test_row_sample():
    rb, ri = syn.row_sample(8, 65536)
    assert rb.size == 256 and len(set(zip(rb.tolist(), ri.tolist()))) == 256
    assert rb.min() >= 0 and rb.max() < 8 and ri.min() >= 0 and ri.max() < 65536
    rb2, ri2 = syn.row_sample(8, 65536)
    assert np.array_equal(rb, rb2) and np.array_equal(ri, ri2)


def test_pages_dense_score_memory_figures():
    """The pages' worked figures for the dense score matrix (fp16, one head)
    follow from N^2 * 2 bytes; the GPU path must allocate none of it."""
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                    "dense_score_memory.json")))
    c8, c32 = g["cases"]
    assert abs(c8["N"] ** 2 - c8["stated_elements"]) / c8["stated_elements"] < 0.01
    assert c8["N"] ** 2 * c8["bytes_per_element"] == 128 * 2 ** 20
    assert c32["N"] ** 2 * c32["bytes_per_element"] == 2 * 2 ** 30


def test_e4m3_round_matches_torch():
    """The E4M3 quantizer of the FP8 inputs equals torch's float8_e4m3fn
    conversion (round to nearest even) on every value below the saturation
    point, decodes every finite code as torch does, and saturates at 448."""
    import torch
    rng = np.random.default_rng(11)
    x = np.concatenate([rng.standard_normal(50000).astype(np.float32) * s
                        for s in (1e-3, 3e-2, 1.0, 40.0, 400.0)])
    x = x[np.abs(x) <= 448]
    ours = syn.e4m3_round_bits(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)
    codes = np.arange(256, dtype=np.uint8)
    tv = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ok = np.isfinite(tv)
    assert np.array_equal(syn.e4m3_bits_to_f64(codes)[ok], tv[ok])
    assert syn.e4m3_bits_to_f64(syn.e4m3_round_bits(np.array([1e6, -1e6])))[0] == 448.0
    q8, s = syn.fp8_quantize(np.array([0.5, -3.0, 1.5], np.float32))
    assert s == np.float32(3.0 / 448) and abs(syn.e4m3_bits_to_f64(q8[1]) * s + 3.0) < 1e-6
