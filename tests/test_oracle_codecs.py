"""Pins of the oracle's storage codecs against torch's CPU casts (library routines, round to nearest even)."""
import numpy as np
import pytest
import torch

from oracle import codecs


def test_bf16_matches_torch_cast_on_fp32_values():
    g = np.random.default_rng(1)
    x = np.concatenate([g.standard_normal(20000), g.standard_normal(2000) * 1e-30, g.standard_normal(2000) * 1e30])
    x32 = x.astype(np.float32)
    ref = torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = codecs.f64_to_bf16(x32.astype(np.float64))
    assert np.array_equal(got, ref)


def test_bf16_ties_go_to_even():
    # 1 + 2^-8 is exactly halfway between bf16 neighbours 1 and 1 + 2^-7 -> even (1.0)
    # 1 + 3*2^-8 is halfway between 1 + 2^-7 and 1 + 2^-6 -> even (1 + 2^-6)
    got = codecs.bf16_to_f64(codecs.f64_to_bf16(np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8)])))
    assert list(got) == [1.0, 1 + 2 ** -6, -1.0]


def test_bf16_roundtrip_is_exact():
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    vals = codecs.bf16_to_f64(bits)
    fin = np.isfinite(vals)
    assert np.array_equal(codecs.f64_to_bf16(vals[fin]).view(np.int16) & 0x7FFF,
                          bits[fin].view(np.int16) & 0x7FFF)


def test_e4m3_table_matches_torch():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    both_nan = np.isnan(ref) & np.isnan(codecs.E4M3_VALUES)
    assert np.array_equal(np.where(both_nan, 0, ref), np.where(both_nan, 0, codecs.E4M3_VALUES))
    assert codecs.E4M3_VALUES[0x7E] == 448.0 and codecs.E4M3_VALUES[0x01] == 2.0 ** -9
    assert np.isnan(codecs.E4M3_VALUES[0x7F]) and np.isnan(codecs.E4M3_VALUES[0xFF])


def test_e4m3_matches_torch_cast_in_range():
    g = np.random.default_rng(2)
    x = np.concatenate([g.uniform(-448, 448, 20000), g.standard_normal(20000), g.standard_normal(5000) * 2e-3])
    x32 = x.astype(np.float32)
    ref = torch.from_numpy(x32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = codecs.f64_to_e4m3(x32.astype(np.float64))
    assert np.array_equal(got, ref)


def test_e4m3_every_code_roundtrips():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    assert np.array_equal(codecs.f64_to_e4m3(codecs.E4M3_VALUES[codes]), codes)


def test_fp8_store_row_scale_rule():
    g = np.random.default_rng(3)
    y = g.standard_normal(512)
    codes, sc = codecs.store_row(y, codecs.FP8)
    amax = np.max(np.abs(codecs.f32(y)))
    assert sc == np.float32(amax / 448.0)
    k = int(np.argmax(np.abs(y)))
    assert codecs.E4M3_VALUES[codes[k]] == np.sign(y[k]) * 448.0
    deq = codecs.load_rows(codes[None], codecs.FP8, np.array([sc]))[0]
    # each element within half an e4m3 step (relative 2^-4) of its value, measured in scaled units
    step = np.maximum(np.ldexp(1.0, np.floor(np.log2(np.maximum(np.abs(y) / sc, 2.0 ** -6))).astype(int) - 3), 2.0 ** -9)
    assert np.all(np.abs(deq / sc - y / sc) <= 0.5 * step * (1 + 1e-6) + 1e-6)
    zc, zs = codecs.store_row(np.zeros(8), codecs.FP8)
    assert zs == 1.0 and not zc.any()
