"""Pins of the oracle's codebooks: the printed CQ2 header values, the printed
ternary level, and the textbook Gaussian Lloyd-Max quantisers (J. Max, 1960)."""
import importlib.util
import math
import os

import numpy as np
import pytest
from scipy import integrate, stats

import oracle
from conftest import GOLDEN, golden


def test_empirical_cq2_reproduces_printed_header_values():
    g = golden("cq2_printed.json")
    cb = oracle.lloyd_max_empirical(4, group=g["group"])
    assert cb.dtype == np.float32
    assert [float(v) for v in cb] == g["values"]  # bit for bit


def _cells(c):
    return np.concatenate([[-np.inf], (c[:-1] + c[1:]) / 2, [np.inf]])


def _mse(c):
    t = _cells(c)
    return sum(integrate.quad(lambda x, cj=cj: (x - cj) ** 2 * stats.norm.pdf(x), t[j], t[j + 1])[0]
               for j, cj in enumerate(c))


@pytest.mark.parametrize("L", [4, 8, 16])
def test_gaussian_lloyd_max_matches_max_1960_table(L):
    g = golden("max1960_gaussian.json")
    ref = g["levels"][str(L)]
    c = oracle.gaussian_lloyd_max(L)
    assert np.all(np.diff(c) > 0)
    assert np.allclose(c, -c[::-1], rtol=0, atol=1e-12)
    assert np.allclose(c[L // 2:], ref["outputs"], rtol=0, atol=g["tolerance"])
    assert abs(_mse(c) - ref["mse"]) / ref["mse"] < 2e-3


@pytest.mark.parametrize("L", [4, 8, 16])
def test_gaussian_lloyd_max_is_stationary(L):
    # centroid condition by numerical integration (not the closed form the oracle iterates)
    c = oracle.gaussian_lloyd_max(L)
    t = _cells(c)
    for j in range(L):
        mass = stats.norm.cdf(t[j + 1]) - stats.norm.cdf(t[j])
        mean = integrate.quad(lambda x: x * stats.norm.pdf(x), t[j], t[j + 1])[0] / mass
        assert abs(mean - c[j]) < 1e-8


def test_ternary_level_reproduces_printed_value():
    g = golden("ternary_level.json")
    a = oracle.ternary_level()
    assert round(a, 7) == g["level"]
    mean_above = integrate.quad(lambda x: x * stats.norm.pdf(x), a / 2, np.inf)[0] / stats.norm.sf(a / 2)
    assert abs(mean_above - a) < 1e-9
    m = golden("max1960_gaussian.json")
    assert abs(a - m["levels"]["3"]["outputs"][1]) < m["tolerance"]
    assert abs(_mse(np.array([-a, 0.0, a])) - m["levels"]["3"]["mse"]) < 2e-4


def test_ternary_fp32_codebook():
    a = oracle.ternary_level32()
    assert a == np.float32(golden("ternary_level.json")["level"] / math.sqrt(128))
    cb = oracle.codebook_for(5)
    assert cb.dtype == np.float32 and cb.tolist() == [-a, 0.0, a]


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_empirical_close_to_analytic_and_asymmetric(bits):
    L = 1 << bits
    emp = oracle.lloyd_max_empirical(L).astype(np.float64) * math.sqrt(128)
    ana = oracle.gaussian_lloyd_max(L)
    assert np.max(np.abs(emp - ana)) < 0.02 * np.max(np.abs(ana))
    # the pages warn the sample codebook is slightly asymmetric and must not be
    # replaced by symmetric centres
    assert not np.allclose(emp, -emp[::-1], rtol=0, atol=1e-6)
    if bits == 2:
        assert np.max(np.abs(emp / ana - 1)) < 5e-3


def test_golden_codebook_file_is_current():
    spec = importlib.util.spec_from_file_location("make_codebooks", os.path.join(GOLDEN, "make_codebooks.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    assert mod.build() == golden("codebooks.json")


def test_codebook_validation():
    with pytest.raises(ValueError):
        oracle.codebook_for(2, [0.1, 0.0, 0.2, 0.3])
    with pytest.raises(ValueError):
        oracle.codebook_for(2, [0.1, 0.2, 0.3])
    with pytest.raises(ValueError):
        oracle.codebook_for(5, [-1.0, 0.0, 1.0])
    with pytest.raises(ValueError):
        oracle.codebook_for(6, [0.0] * 64)
