"""Seeded input generator: published SplitMix64 vectors, draw definitions, RNE."""
from fractions import Fraction

import numpy as np
import pytest

import k3gen
from k3gen.workloads import DECODE, PREFILL, TINY, TOY, WORKLOADS


def test_splitmix64_published_vectors():
    # SplitMix64 reference outputs (Steele/Lea/Flood 2014; Vigna's splitmix64.c):
    # state 0 -> 0xe220a8397b1dcdaf, 0x6e789e6aa1b965f4, 0x06c45d188009454f
    assert [k3gen.at(0, i) for i in range(3)] == [
        0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]
    # state 1234567 -> the widely used test vector of the same generator
    assert [k3gen.at(1234567, i) for i in range(3)] == [
        6457827717110365317, 3203168211198807973, 9817491932198370423]


def test_key_derivation_is_nested_counter():
    s = 0x1234
    assert k3gen.key(s, 1, 2, 3) == k3gen.at(k3gen.at(k3gen.at(s, 1), 2), 3)


@pytest.mark.parametrize("start,n", [(0, 1), (0, 64), (3, 29), (13, 1000), (8, 8)])
def test_bytes_are_little_endian_words_and_offset_addressable(start, n):
    key = 0xABCDEF
    full = k3gen.host_bytes(key, start + n)
    part = k3gen.host_bytes(key, n, start)
    assert np.array_equal(full[start:], part)
    for j in range(start, start + n):
        assert full[j] == (k3gen.at(key, j // 8) >> (8 * (j % 8))) & 0xFF


def test_bytes_large_parallel_path_matches_scalar_definition():
    key = 77
    n = (1 << 20) + 13
    a = k3gen.host_bytes(key, n, 5)
    idx = np.array([0, 1, 7, 8, 9, 4095, n - 1])
    for i in idx:
        j = 5 + int(i)
        assert a[i] == (k3gen.at(key, j // 8) >> (8 * (j % 8))) & 0xFF


def test_e8m0_range_and_coverage():
    a = k3gen.host_e8m0(99, 200000, 120, 9)
    assert a.min() == 120 and a.max() == 128
    counts = np.bincount(a - 120, minlength=9)
    assert counts.min() > 200000 / 9 * 0.95
    for j in (0, 5, 199999):
        assert a[j] == 120 + (((k3gen.at(99, j) >> 32) * 9) >> 32)


def _rne_bf16_reference(v: float) -> int:
    """Exact rational RNE to bfloat16 (8-bit significand, emin -126)."""
    if v == 0:
        return 0x8000 if np.signbit(v) else 0
    sign = 0x8000 if v < 0 else 0
    a = Fraction(abs(v))
    e = 0
    while a >= 2:
        a /= 2
        e += 1
    while a < 1:
        a *= 2
        e -= 1
    if e < -126:  # subnormal: spacing 2^-133
        q = Fraction(abs(v)) / Fraction(1, 2 ** 133)
        n = round(q)  # Python round: ties to even
        return sign | n  # exponent field 0 (n may reach 128 -> min normal, still correct bits)
    q = a * 128
    n = round(q)
    if n == 256:
        n = 128
        e += 1
    if e > 127:
        return sign | 0x7F80
    return sign | ((e + 127) << 7) | (n - 128)


@pytest.mark.parametrize("v", [1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -8 + 2 ** -30, -2.5,
                               0.1, -0.02, 3.3895313892515355e38, 2.0 ** -130,
                               2.0 ** -126 * 1.5, 2.0 ** -133 * 0.5, 2.0 ** -133 * 1.5,
                               123456.789, -1e-10])
def test_f64_to_bf16_single_rne(v):
    assert k3gen.f64_to_bf16(v) == _rne_bf16_reference(v)


def test_f64_to_bf16_specials():
    assert k3gen.f64_to_bf16(float("inf")) == 0x7F80
    assert k3gen.f64_to_bf16(-float("inf")) == 0xFF80
    assert k3gen.f64_to_bf16(2.0 ** 128) == 0x7F80
    assert k3gen.f64_to_bf16(float("nan")) & 0x7FC0 == 0x7FC0
    assert k3gen.f64_to_bf16(-0.0) == 0x8000


def test_f64_to_bf16_random_against_rational_reference():
    rng = np.random.default_rng(5)
    for v in rng.standard_normal(300) * np.exp(rng.uniform(-20, 20, 300)):
        assert k3gen.f64_to_bf16(float(v)) == _rne_bf16_reference(float(v))


def test_normals_moments_and_definition():
    key = 4242
    z = np.array([k3gen.normal_f64(key, j) for j in range(20000)])
    assert abs(z.mean()) < 0.03 and abs(z.std() - 1) < 0.03
    b = k3gen.host_normal_bf16(key, 10, 0.0, 0.02)
    for j in range(10):
        assert b[j] == k3gen.f64_to_bf16(0.02 * z[j])


def test_zipf_bias_is_permutation_and_log_rank():
    ranks, bias = k3gen.zipf_bias(7, 896, 1.1)
    assert sorted(ranks.tolist()) == list(range(1, 897))
    assert np.array_equal(bias, (-1.1 * np.log(ranks.astype(np.float64))).astype(np.float32))


def test_workload_shapes_and_determinism():
    assert set(WORKLOADS) >= {"toy", "decode", "batched", "prefill", "stack8"}
    ex = TOY.expert_host(0, 3)
    assert ex["gate_q"].shape == (256, 256) and ex["gate_s"].shape == (256, 16)
    assert ex["down_q"].shape == (512, 128) and ex["down_s"].shape == (512, 8)
    ex2 = TOY.expert_host(0, 3)
    for n in ex:
        assert np.array_equal(ex[n], ex2[n])
    assert not np.array_equal(TOY.expert_host(0, 4)["gate_q"], ex["gate_q"])
    assert TOY.x_bf16().shape == (1, 512)
    assert PREFILL.bias(0).shape == (896,) and DECODE.bias(0) is None
    assert TINY.router_w(0).shape == (64, 8)
