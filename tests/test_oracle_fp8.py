"""Pins for the fp8 oracle: the E4M3 codec against torch's float8_e4m3fn
conversion and the format's defining points, the block quantiser's scale rule
and error bound, and the Hadamard rotation's orthogonality and the invariance
of Q K^T under it."""
import os

import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import fp8 as F

HERE = os.path.dirname(os.path.abspath(__file__))
RNG = np.random.default_rng(99)


def torch_codes(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_decode_all_codes_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = F.e4m3_decode(codes)
    np.testing.assert_array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(got[ok], ref[ok])


def test_encode_matches_torch_on_random_and_grid_values():
    x = np.concatenate([
        RNG.standard_normal(20000).astype(np.float32) * 30,
        RNG.uniform(-448, 448, 20000).astype(np.float32),
        RNG.uniform(-0.02, 0.02, 20000).astype(np.float32),   # subnormal range
    ])
    grid = F.e4m3_decode(np.arange(256, dtype=np.uint8))
    grid = grid[np.isfinite(grid)]
    mids = ((grid[:-1] + grid[1:]) / 2)  # ties, exactly representable in fp32 here
    sg = np.sort(grid)
    ties = ((sg[:-1] + sg[1:]) / 2).astype(np.float32)
    x = np.concatenate([x, grid.astype(np.float32), ties]).astype(np.float32)
    x = np.clip(x, -448, 448)
    np.testing.assert_array_equal(F.e4m3_encode(x), torch_codes(x))
    del mids


def test_golden_points():
    with open(os.path.join(HERE, "golden", "e4m3_points.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            val, code = line.split()[:2]
            c = int(code, 16)
            assert int(F.e4m3_encode(np.float32(float(val)))) == c, line
            if float(val) != 0.0 and "tie" not in line:
                assert F.e4m3_decode(np.uint8(c)) == float(val), line


def test_encode_rejects_out_of_range():
    with pytest.raises(ValueError):
        F.e4m3_encode(np.float32(449.0))
    with pytest.raises(ValueError):
        F.e4m3_encode(np.float32(np.nan))


def test_block_quantize_scale_rule_and_bound():
    B, S, H, d = 2, 300, 3, 16       # 3 blocks, the last one ragged (44 rows)
    x = (RNG.standard_normal((B, S, H, d)) * RNG.uniform(0.1, 50, (1, 1, H, 1))).astype(np.float32)
    x[1, 128:256, 2] = 0.0           # an all-zero block
    codes, s = F.block_quantize(x)
    assert s.shape == (B, H, 3) and s.dtype == np.float32
    for b in range(B):
        for h in range(H):
            for j in range(3):
                blk = x[b, 128 * j:128 * (j + 1), h]
                amax = np.float32(np.abs(blk).max())
                if amax == 0:
                    assert s[b, h, j] == 1.0
                    assert np.all(codes[b, 128 * j:128 * (j + 1), h] == 0)
                    continue
                assert s[b, h, j] == np.float32(amax / np.float32(448.0))
                c = codes[b, 128 * j:128 * (j + 1), h]
                # the block's largest magnitude lands on +-448 (0x7e / 0xfe)
                assert (c & 0x7F).max() == 0x7E
    deq = F.dequantize(codes, s)
    rel = np.abs(deq - x) / np.maximum(np.abs(x), 1e-30)
    # normal range of the scaled value: relative error <= half a mantissa step (2^-4)
    big = np.abs(x) >= 2.0 ** -6 * np.transpose(s, (0, 2, 1)).repeat(128, axis=1)[:, :S, :, None]
    assert rel[big].max() <= 2.0 ** -4 + 1e-7
    # independence: changing one block leaves the others' codes unchanged
    x2 = x.copy()
    x2[0, :128, 0] *= 3
    c2, s2 = F.block_quantize(x2)
    np.testing.assert_array_equal(c2[0, 128:, 0], codes[0, 128:, 0])
    np.testing.assert_array_equal(c2[1], codes[1])


def test_hadamard_orthogonal():
    for n in (1, 2, 8, 128):
        h = F.hadamard_matrix(n)
        np.testing.assert_array_equal(h @ h.T, n * np.eye(n))
    signs = np.where(RNG.standard_normal(128) > 0, 1.0, -1.0)
    R = F.rotation(signs)
    np.testing.assert_allclose(R @ R.T, np.eye(128), atol=1e-15)
    with pytest.raises(ValueError):
        F.hadamard_matrix(6)


def test_rotation_leaves_attention_unchanged():
    B, S, H, d = 1, 40, 2, 128
    q, k, v = (RNG.standard_normal((B, S, H, d)) for _ in range(3))
    signs = np.where(RNG.standard_normal(d) > 0, 1.0, -1.0)
    O1, L1 = A.attention(q, k, v, d ** -0.5, True)
    O2, L2 = A.attention(F.rotate(q, signs), F.rotate(k, signs), v, d ** -0.5, True)
    np.testing.assert_allclose(O1, O2, atol=1e-12)
    np.testing.assert_allclose(L1, L2, atol=1e-12)


def test_rotation_spreads_outliers():
    # an outlier channel is spread evenly: |x R| for x = e_c is 1/sqrt(n) everywhere
    signs = np.where(RNG.standard_normal(128) > 0, 1.0, -1.0)
    e = np.zeros(128)
    e[17] = 20.0
    np.testing.assert_allclose(np.abs(F.rotate(e, signs)), 20.0 / np.sqrt(128), atol=1e-13)
