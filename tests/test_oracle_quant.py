"""Pins of the oracle's FP8 codec, Hadamard rotation and quantiser (CPU only).

The oracle is pinned to library routines and closed forms, never to itself:
torch's float8_e4m3fn conversions, scipy's Sylvester Hadamard matrix, and the
format definition's landmark values ("MAX Pipeline 中的 DeepSeek-V3.2 架构实现解析",
配置体系: the indexer cache is float8_e4m3fn).
"""
import numpy as np
import pytest
import scipy.linalg
import torch

import oracle

pytestmark = pytest.mark.filterwarnings("ignore::DeprecationWarning")


def test_fp8_decode_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.fp8_decode(codes)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


def test_fp8_landmarks():
    dec = oracle.fp8_decode
    assert dec(0x7E) == 448.0            # max finite
    assert dec(0x01) == 2.0 ** -9        # smallest subnormal
    assert dec(0x08) == 2.0 ** -6        # smallest normal
    assert dec(0x38) == 1.0
    assert dec(0xB8) == -1.0
    # every finite value is an integer multiple of 2^-9 (basis of the exact dot products)
    v = oracle.fp8_decode(np.arange(256, dtype=np.uint8))
    v = v[~np.isnan(v)] * 512.0
    assert np.array_equal(v, np.round(v))


def _grid():
    # every code value, every midpoint between neighbours (ties) and a dense sweep
    vals = oracle.fp8_decode(np.arange(0x7F, dtype=np.uint8))
    mids = (vals[1:] + vals[:-1]) / 2
    sweep = np.linspace(0, 464, 20001)
    tiny = np.linspace(0, 2 ** -6, 2049)
    g = np.concatenate([vals, mids, sweep, tiny, np.nextafter(mids, 0), np.nextafter(mids, 1e9)])
    g = np.concatenate([g, -g]).astype(np.float32)
    return g[np.abs(g) <= 464.0]


def test_fp8_encode_matches_torch_rne():
    g = _grid()
    ours = oracle.fp8_encode(g)
    ref = torch.from_numpy(g).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_fp8_encode_saturates():
    # reading taken: saturate to +-448 beyond the finite range (torch gives NaN above 464)
    big = np.array([465.0, 1e4, 3e38, -500.0, np.inf, -np.inf], dtype=np.float32)
    assert list(oracle.fp8_encode(big)) == [0x7E, 0x7E, 0x7E, 0xFE, 0x7E, 0xFE]
    assert oracle.fp8_encode(np.array([np.nan], np.float32))[0] == 0x7F


@pytest.mark.parametrize("n", [2, 8, 64, 128])
def test_fwht_matches_sylvester_matrix(n):
    rng = np.random.default_rng(n)
    x = rng.standard_normal((5, n)).astype(np.float32)
    H = scipy.linalg.hadamard(n).astype(np.float64)
    ref = x.astype(np.float64) @ H.T
    got = oracle.fwht_f32(x).astype(np.float64)
    assert np.allclose(got, ref, rtol=1e-5, atol=1e-4 * np.sqrt(n))
    # H H^T = n I, applied to the identity
    eye = np.eye(n, dtype=np.float32)
    Hm = oracle.fwht_f32(eye).astype(np.float64)
    assert np.array_equal(Hm @ Hm.T, n * np.eye(n))


def test_quantize_roundtrip_and_scale_rule():
    rng = np.random.default_rng(7)
    for d in (64, 128):
        x = rng.standard_normal((200, d)).astype(np.float32)
        codes, scale = oracle.quantize(x)
        H = scipy.linalg.hadamard(d) / np.sqrt(d)
        y = x.astype(np.float64) @ H.T                 # orthonormal rotation (float64)
        deq = oracle.fp8_decode(codes) * scale[:, None].astype(np.float64)
        amax = np.abs(y).max(axis=1)
        assert np.allclose(scale, amax / 448.0, rtol=1e-6)
        # the amax element lands on the top code
        top = np.abs(oracle.fp8_decode(codes)).max(axis=1)
        assert np.all(top == 448.0)
        # e4m3 keeps 3 mantissa bits: relative error <= 2^-4 for normals, half a
        # subnormal step (scale * 2^-10) below the normal range; plus fp32 noise
        err = np.abs(deq - y)
        bound = np.maximum(np.abs(y) * 2.0 ** -4, scale[:, None] * 2.0 ** -10) + 1e-5 * amax[:, None]
        assert np.all(err <= bound)
        # rotation preserves dot products (before quantisation), up to fp32 rounding
        xr = oracle.fwht_f32(x).astype(np.float64) / np.sqrt(d)
        g1 = xr[:20] @ xr[20:40].T
        g0 = x[:20].astype(np.float64) @ x[20:40].T.astype(np.float64)
        assert np.allclose(g1, g0, rtol=1e-5, atol=1e-4)


def test_quantize_zero_vector_and_rejects_bad_dim():
    codes, scale = oracle.quantize(np.zeros((3, 128), np.float32))
    assert np.all(codes == 0) and np.all(scale == 1.0)
    with pytest.raises(ValueError):
        oracle.quantize(np.zeros((1, 96), np.float32))
