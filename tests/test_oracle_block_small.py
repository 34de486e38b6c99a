"""Pins of the oracle's square-block quantizer at b = 16 and b = 8 (Sec. 3
defines the square-block scheme for any b; Table 4 of "Stable FP4 Training
via Transposition-Invariant Block Quantization" compares b = 8, 16, 32, 64).

As for b = 64, the pins are facts the definition fixes:
- the truncation-free exponent is non-decreasing in the amax and a block's
  amax is the max of its four half-side sub-blocks' amaxes, so the byte of
  a 2b block is the max of its four b bytes (8 -> 16 -> 32);
- where a block's byte equals the byte of the block of twice the side that
  contains it, both use one scale and one random field per element, so the
  codes agree;
- square blocks: quantizing W^T gives the transpose of quantizing W;
- the grid covers the 32-padded planes, and blocks with no valid entry hold
  byte 0;
- hand-worked inputs: 16x16 block amaxes {6, 3, 0, 7} give bytes
  {127, 126, 0, 128}, and values that are on the E2M1 grid of their own 8x8
  block's scale come back exactly at b = 8 but not at b = 32, where a
  larger neighbour sets the scale (the reason smaller blocks keep more
  range)."""
import numpy as np
import pytest

from test_oracle_block64 import _input, unpack

SHAPES = [(100, 130), (64, 64), (65, 200), (33, 31), (8, 8)]


def _valid_max(sub_bytes, sub_side, r0, c0, rows, cols):
    """Max of the sub-block bytes whose blocks hold a valid entry."""
    best = 0
    for a in range(2):
        for b in range(2):
            if r0 + a * sub_side < rows and c0 + b * sub_side < cols:
                best = max(best, int(sub_bytes[a, b]))
    return best


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("bf16", [True, False])
@pytest.mark.parametrize("b", [8, 16])
def test_scale_of_2b_block_is_max_of_its_b_blocks(orc, shape, bf16, b):
    x = _input(shape, 12, bf16)
    r, c = shape
    _, _, sb = orc.quant2d_block(x, b, seed=1, stream=1)
    _, _, s2 = orc.quant2d_block(x, 2 * b, seed=1, stream=1)
    rp, cp = -(-r // 32) * 32, -(-c // 32) * 32
    assert sb.shape == (rp // b, cp // b)
    assert s2.shape == (-(-rp // (2 * b)), -(-cp // (2 * b)))
    for i in range(s2.shape[0]):
        for j in range(s2.shape[1]):
            want = _valid_max(sb[2 * i:2 * i + 2, 2 * j:2 * j + 2], b, 2 * b * i, 2 * b * j, r, c)
            assert s2[i, j] == want, (i, j)
    # blocks wholly in the padding hold byte 0
    for i in range(sb.shape[0]):
        for j in range(sb.shape[1]):
            if b * i >= r or b * j >= c:
                assert sb[i, j] == 0


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("b", [8, 16])
def test_codes_agree_where_scales_agree(orc, shape, mode, b):
    x = _input(shape, 13, bf16=True)
    r, c = shape
    rp, cp = -(-r // 32) * 32, -(-c // 32) * 32
    cb, tb, sb = orc.quant2d_block(x, b, mode, seed=7, stream=2)
    c2, t2, s2 = orc.quant2d_block(x, 2 * b, mode, seed=7, stream=2)
    a1, a2 = unpack(cb, rp, cp), unpack(c2, rp, cp)
    b1, b2 = unpack(tb, cp, rp), unpack(t2, cp, rp)
    same = 0
    for ti in range(rp // b):
        for tj in range(cp // b):
            if b * ti >= r or b * tj >= c:
                continue
            blk = (slice(b * ti, b * ti + b), slice(b * tj, b * tj + b))
            if sb[ti, tj] == s2[ti // 2, tj // 2]:
                same += 1
                assert np.array_equal(a1[blk], a2[blk]), (ti, tj)
                assert np.array_equal(b1[blk[1], blk[0]], b2[blk[1], blk[0]]), (ti, tj)
            else:
                assert sb[ti, tj] < s2[ti // 2, tj // 2]
    assert same > 0


@pytest.mark.parametrize("shape", [(100, 130), (48, 80), (33, 17)])
@pytest.mark.parametrize("b", [8, 16])
def test_transposition_invariance(orc, shape, b):
    x = _input(shape, 14, bf16=False)
    c, ct, s = orc.quant2d_block(x, b, seed=11, stream=5)
    cT, ctT, sT = orc.quant2d_block(np.ascontiguousarray(x.T), b, seed=11, stream=5)
    assert np.array_equal(cT, ct) and np.array_equal(ctT, c) and np.array_equal(sT, s.T)


def test_hand_worked_16x16_blocks(orc):
    """32x32 input, 16x16 block amaxes {6, 3, 0, 7}: bytes {127, 126, 0, 128};
    on-grid entries come back exactly for any seed; the lone 7 (v = 3.5 at
    S = 2) rounds to 3 or 4."""
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], dtype=np.float32)
    idx = (np.add.outer(np.arange(16) * 3, np.arange(16) * 5) % 8).astype(np.int64)
    idx[0, 0] = 7
    small = np.minimum(idx, 5)
    x = np.zeros((32, 32), dtype=np.float32)
    x[:16, :16] = grid[idx]                  # amax 6 -> S = 1
    x[:16, 16:] = -grid[small]               # amax 3 -> S = 1/2
    x[16:, 16:] = 2.0 * grid[small]          # on grid at S = 2 ...
    x[16 + 5, 16 + 9] = 7.0                  # ... one 7 -> amax 7, S = 2
    for seed in (0, 9):
        codes, _, scales = orc.quant2d_block(x, 16, seed=seed, stream=3)
        assert scales.tolist() == [[127, 126], [0, 128]]
        got = unpack(codes, 32, 32)
        assert np.array_equal(got[:16, :16], idx)
        assert np.array_equal(got[:16, 16:], 8 | np.searchsorted(grid, 2 * grid[small]))
        assert np.array_equal(got[16:, :16], np.zeros((16, 16), np.uint8))
        q = got[16:, 16:].copy()
        assert q[5, 9] in (5, 6)
        q[5, 9] = small[5, 9]
        assert np.array_equal(q, small)


def test_small_blocks_keep_range_large_blocks_flush(orc):
    """A 32x32 input whose sixteen 8x8 blocks each hold E2M1 grid values
    times their own power of two 2^e (e from -20 to 10): at b = 8 every
    value comes back exactly (RNE and SR alike); at b = 32 one scale, set by
    the largest block, cannot represent the smallest blocks' values."""
    rng = np.random.default_rng(5)
    grid = np.array([0.5, 1, 1.5, 2, 3, 4, 6], dtype=np.float64)
    x = np.zeros((32, 32))
    exps = rng.permutation(np.linspace(-20, 10, 16).astype(int))
    for t in range(16):
        i, j = divmod(t, 4)
        v = grid[rng.integers(0, 7, (8, 8))] * rng.choice([-1, 1], (8, 8))
        v[0, 0] = 6.0
        x[8 * i:8 * i + 8, 8 * j:8 * j + 8] = v * 2.0 ** exps[t]
    x32 = x.astype(np.float32)
    for mode in (0, 1):
        codes, _, scales = orc.quant2d_block(x32, 8, mode, seed=4, stream=2)
        assert np.array_equal(orc.dequant_fp4_blocks(codes, scales, 32, 32, 8, 8), x)
    codes, _, scales = orc.quant2d_block(x32, 32, 1, seed=4, stream=2)
    assert not np.array_equal(orc.dequant_fp4_blocks(codes, scales, 32, 32, 32, 32), x)
