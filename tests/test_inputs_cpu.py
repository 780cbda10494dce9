"""The seeded synthetic inputs, on the CPU: every recipe's range and
distribution, determinism per seed, independence from the thread count, and
the five workloads' sizes (valid bytes and (N+1)-fold algorithmic bytes)."""

import numpy as np
import pytest
import torch

from cross_rank_collective_amd import workloads as W


def _bf16_to_f32(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32)


def test_draw_is_deterministic_per_seed():
    for recipe in ("uniform_pm1", "normal_1e-2", "int_pm2^20", "normal_sat"):
        a, b, c = W.draw(recipe, 4096, 11), W.draw(recipe, 4096, 11), W.draw(recipe, 4096, 12)
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), recipe
        assert not np.array_equal(a.view(np.uint8), c.view(np.uint8)), recipe


def test_uniform_pm1_is_f32_in_minus_one_to_one():
    v = W.draw("uniform_pm1", 200_000, 1)
    assert v.dtype == np.float32
    assert v.min() >= -1.0 and v.max() < 1.0
    assert abs(float(v.mean())) < 0.01 and abs(float(v.std()) - 1 / np.sqrt(3)) < 0.01


def test_normal_1e2_is_bf16_of_a_scaled_normal():
    bits = W.draw("normal_1e-2", 200_000, 2)
    assert bits.dtype == np.uint16
    v = _bf16_to_f32(bits)
    assert abs(float(v.mean())) < 3e-4 and abs(float(v.std()) / 1e-2 - 1) < 0.02
    # the bits are the round-to-nearest-even bf16 of the f32 draws
    rng = np.random.default_rng(2)
    ref = torch.from_numpy(rng.standard_normal(200_000, dtype=np.float32) * np.float32(1e-2))
    assert np.array_equal(bits, ref.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))


def test_int_pm2_20_range():
    v = W.draw("int_pm2^20", 200_000, 3)
    assert v.dtype == np.int32
    assert v.min() >= -(2 ** 20) and v.max() < 2 ** 20
    assert v.min() < -(2 ** 19) and v.max() > 2 ** 19


def test_normal_sat_has_one_percent_saturated_entries_of_both_signs():
    bits = W.draw("normal_sat", 1_000_000, 4)
    v = bits.view(np.float16).astype(np.float32)
    sat = np.abs(v) == 65504.0
    assert abs(sat.mean() - 0.01) < 0.001
    assert 0.4 < (v[sat] < 0).mean() < 0.6
    rest = v[~sat]
    assert np.isfinite(rest).all() and np.abs(rest).max() < 10
    assert abs(float(rest.std()) - 1) < 0.01


def test_sources_do_not_depend_on_the_thread_count():
    w = W.find("n4_f32_1024x1024_valid1000x1000")
    a, b = W.make_sources(w, threads=1), W.make_sources(w, threads=8)
    assert len(a) == w.nranks
    for r in range(w.nranks):
        assert a[r].size == w.rows * w.ld
        assert np.array_equal(a[r].view(np.uint8), b[r].view(np.uint8))
        assert np.array_equal(a[r].view(np.uint8),
                              W.draw(w.recipe, w.buffer_elems, w.seed_base + r).view(np.uint8))


@pytest.mark.parametrize("name,valid,alg", [
    ("n2_f32_16x16", 1024, 3072),
    ("n4_f32_1024x1024_valid1000x1000", 4_000_000, 20_000_000),
    ("n8_bf16_8192x8192", 134_217_728, 1_207_959_552),
    ("n16_i32_4096x4096", 67_108_864, 1_140_850_688),
    ("n8_f16_8192x12288_valid8191x12287", 201_285_634, 1_811_570_706),
])
def test_workload_sizes(name, valid, alg):
    w = W.find(name)
    assert w.valid_bytes == valid
    assert w.algorithmic_bytes == alg
    assert w.root == 0 and w.seed_base == 1000 * (list(W.WORKLOADS).index(name) + 1)
