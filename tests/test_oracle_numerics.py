"""Pins of the oracle's format decoders/encoders against library routines
(torch's and numpy's casts), over every bit pattern where that is small."""
import numpy as np
import pytest
import torch

from oracle import gemm as og
from oracle import numerics as on


def torch_decode(bits, dtype):
    t = torch.from_numpy(np.asarray(bits))
    if dtype == "bf16":
        return t.view(torch.bfloat16).double().numpy()
    if dtype == "f16":
        return t.view(torch.float16).double().numpy()
    if dtype == "e4m3":
        return t.view(torch.float8_e4m3fn).double().numpy()


def same(x, y):
    return np.array_equal(x, y, equal_nan=True) and np.array_equal(np.signbit(x), np.signbit(y))


@pytest.mark.parametrize("dtype,width", [("bf16", 16), ("f16", 16), ("e4m3", 8)])
def test_decode_every_pattern(dtype, width):
    bits = np.arange(1 << width, dtype=np.int64).astype(np.int16 if width == 16 else np.uint8)
    ref = torch_decode(bits, dtype)
    ubits = bits.view(np.uint16) if width == 16 else bits
    assert same(on.decode(ubits, dtype), ref)
    assert same(og.decode(ubits, dtype), ref)


def test_decode_f32():
    x = np.array([0.0, -0.0, 1.5, -3.25e-40, np.inf, 3.4e38], np.float32)
    assert same(on.decode(x, "f32"), x.astype(np.float64))
    assert same(og.decode(x, "f32"), x.astype(np.float64))


def edge_values():
    rng = np.random.default_rng(11)
    vals = [rng.standard_normal(20000) * s for s in (1e-3, 1.0, 100.0, 1e30)]
    # exact halfway points between neighbouring bf16 / fp16 / e4m3 values
    b = np.arange(0, 1 << 16, 7, dtype=np.int64).astype(np.uint16)
    bf = on.decode(b, "bf16")
    vals.append((bf[:-1] + bf[1:]) / 2)
    f = on.decode(np.arange(0, 1 << 15, 3).astype(np.uint16), "f16")
    vals.append((f[:-1] + f[1:]) / 2)
    e = on.decode(np.arange(0, 0x7F).astype(np.uint8), "e4m3")
    vals.append((e[:-1] + e[1:]) / 2)
    vals.append(np.array([0.0, -0.0, 1e-45, 6e-8, 2.0 ** -133, 2.0 ** -134, 65504.0, 65520.0,
                          448.0, 464.0, 2.0 ** -9, 2.0 ** -10, 3.0 * 2.0 ** -11]))
    v = np.concatenate(vals)
    v = np.concatenate([v, -v])
    return v[np.isfinite(v)].astype(np.float32)


def test_encode_bf16_matches_torch():
    x = edge_values()
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(on.encode(x.astype(np.float64), "bf16"), ref)


def test_encode_f16_matches_numpy():
    x = edge_values()
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(on.encode(x.astype(np.float64), "f16"), ref)


def test_encode_e4m3_matches_torch_in_range():
    x = edge_values()
    x = x[np.abs(x) <= 448.0]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(on.encode(x.astype(np.float64), "e4m3"), ref)


def test_e4m3_saturation_and_roundtrip():
    assert on.max_finite("e4m3") == 448.0
    assert on.encode(np.array([1000.0, -1e9]), "e4m3").tolist() == [0x7E, 0xFE]
    assert on.encode(np.array([1000.0]), "e4m3", saturate=False).tolist() == [0x7F]
    for dtype, width in (("bf16", 16), ("f16", 16), ("e4m3", 8)):
        bits = np.arange(1 << width).astype(np.uint16 if width == 16 else np.uint8)
        vals = on.decode(bits, dtype)
        ok = ~np.isnan(vals)
        assert np.array_equal(on.encode(vals[ok], dtype), bits[ok])
