"""Pins of the float64 oracle of the short key convolution within blocks (CPU only).

The oracle is the definition written as a loop over tokens and taps.  It is pinned
against numpy.convolve (a library routine) applied to each block of each channel,
against closed forms (width 1, an impulse), and packed sequences against the batch
form of each sequence.
"""
import numpy as np
import pytest

import oracle


def conv_by_numpy(K, W, B):
    b, T, hkv, d = K.shape
    w = W.shape[2]
    out = np.zeros_like(K)
    for bi in range(b):
        for g in range(hkv):
            for c in range(d):
                for j0 in range(0, T, B):
                    x = K[bi, j0:j0 + B, g, c]
                    out[bi, j0:j0 + B, g, c] = np.convolve(x, W[g, c])[:x.size]
    return out


@pytest.mark.parametrize("b,T,hkv,d,B,w", [(2, 100, 2, 8, 16, 4), (1, 77, 1, 16, 32, 8),
                                           (1, 50, 3, 4, 16, 1), (1, 40, 2, 8, 48, 3)])
def test_conv_matches_numpy_convolve_per_block(b, T, hkv, d, B, w):
    r = np.random.default_rng(T + w)
    K = r.standard_normal((b, T, hkv, d))
    W = r.standard_normal((hkv, d, w))
    np.testing.assert_allclose(oracle.key_short_conv(K, W, B), conv_by_numpy(K, W, B),
                               rtol=0, atol=1e-12)


def test_conv_width_one_scales_each_channel():
    r = np.random.default_rng(1)
    K = r.standard_normal((1, 40, 2, 4))
    W = r.standard_normal((2, 4, 1))
    np.testing.assert_array_equal(oracle.key_short_conv(K, W, 16), K * W[None, None, :, :, 0])


def test_conv_impulse_stops_at_the_block_end():
    """A single 1 at token p gives the taps W[..., 0..] at p, p+1, ... up to the end of
    p's block, and nothing after it."""
    B, w = 16, 6
    K = np.zeros((1, 48, 1, 2))
    K[0, 13, 0, :] = 1.0                 # 3 tokens before the block end at 16
    W = np.arange(1, 2 * w + 1, dtype=np.float64).reshape(1, 2, w)
    out = oracle.key_short_conv(K, W, B)
    expect = np.zeros_like(K)
    for i in range(3):
        expect[0, 13 + i, 0, :] = W[0, :, i]
    np.testing.assert_array_equal(out, expect)


def test_conv_packed_is_per_sequence():
    r = np.random.default_rng(3)
    lengths = (20, 7, 33)
    cu = np.concatenate([[0], np.cumsum(lengths)])
    K = r.standard_normal((cu[-1], 2, 4))
    W = r.standard_normal((2, 4, 5))
    out = oracle.key_short_conv(K, W, 8, cu)
    for s in range(3):
        a, e = cu[s], cu[s + 1]
        np.testing.assert_allclose(out[a:e], conv_by_numpy(K[None, a:e], W, 8)[0], rtol=0,
                                   atol=1e-12)
