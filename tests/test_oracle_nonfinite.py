"""Oracle pins for non-finite inputs (reading U9): every quantizer encodes nan_to_num of its input,
NaN as +0 and +-inf as +-M, M = 0x7F7F = (255/128) * 2^127 the largest finite bf16 -- the
substitution the FastVideo and SGLang pages apply before a weight's amax. Expected bytes are worked
by hand below from the format definitions, not taken from the oracle."""
import numpy as np

from oracle import formats as Fm
from oracle import mxfp4 as X4
from oracle import mxfp8 as X8
from oracle import nvfp4 as N

PINF, NINF, QNAN, SNAN, ONE = 0x7F80, 0xFF80, 0x7FC0, 0x7F81, 0x3F80


def _row(k, head):
    r = np.zeros((1, k), dtype=np.uint16)
    r[0, :len(head)] = head
    return r


def test_bf16_nan_to_num_codes():
    b = np.array([PINF, NINF, QNAN, SNAN, 0xFFC0, ONE, 0x8000, 0x7F7F], dtype=np.uint16)
    assert Fm.bf16_nan_to_num(b).tolist() == [0x7F7F, 0xFF7F, 0, 0, 0, ONE, 0x8000, 0x7F7F]


def test_nvfp4_block_with_inf_and_nan():
    # block [+inf, 1, NaN, -inf, 0 x 12] at g = 1 -> [M, 1, 0, -M, 0 ...]: amax M, s = fl32(M/6)
    # far above 448 -> S = 0x7E, r = fl32(1/448); M r saturates to code 7, -M r to 0xF, 1 * r =
    # 0.0022 < 0.25 rounds to code 0, NaN (now +0) is code 0. Bytes: (7 | 0 << 4), (0 | 0xF << 4).
    x = _row(16, [PINF, ONE, QNAN, NINF])
    packed, sf = N.quantize(x, np.float32(1.0), layout="linear")
    assert packed.tolist() == [[0x07, 0xF0, 0, 0, 0, 0, 0, 0]]
    assert sf.tolist() == [[0x7E]]
    # a block of NaNs only is an all-zero block: scale 0x00 and zero codes
    packed, sf = N.quantize(_row(16, [SNAN] * 16), np.float32(1.0), layout="linear")
    assert packed.tolist() == [[0] * 8] and sf.tolist() == [[0]]
    # the same substitution in the 128x4 layout (scale of row 0, column 0 at byte 0)
    packed, sf = N.quantize(x, np.float32(1.0))
    assert packed[0, :2].tolist() == [0x07, 0xF0] and sf[0] == 0x7E


def test_nvfp4_per_token_row_with_inf():
    # row [+inf, 1, NaN, 0 x 29] (K 32): row amax M, gsf = fl32(2688 / M) = fl32((896/85) 2^-120);
    # (896/85) 2^-120 = 1.3176... 2^-117 and its 23-bit mantissa field is 11053224.66 - 2^23 -> rounds
    # up to 0x28A8A9: bits 0x0528A8A9. Block 0: s = fl32(g fl32(M/6)) within an ulp of 448 -> 0x7E;
    # M r = M fl32(g/448) within ulps of 6 -> code 7; 1 r ~ 1.8e-38 -> 0; NaN -> 0. Block 1 is zero.
    x = _row(32, [PINF, ONE, QNAN])
    packed, sf, g = N.quantize_per_token(x, layout="linear")
    assert g.view(np.uint32).tolist() == [0x0528A8A9]
    assert packed.tolist() == [[0x07] + [0] * 15]
    assert sf.tolist() == [[0x7E, 0x00]]
    # a row of NaNs has amax 0: gsf 1 and all-zero bytes
    packed, sf, g = N.quantize_per_token(_row(32, [QNAN] * 32), layout="linear")
    assert g.tolist() == [1.0] and not packed.any() and not sf.any()


def test_mxfp8_block_with_inf_and_nan():
    # 32-block [+inf, 1, NaN, -inf, 0 ...] -> amax M = 1.9921875 * 2^127: floor(log2 M) = 127,
    # Es = 127 - 8 = 119, byte 246 (0xF6). M 2^-119 = 510 saturates to 448 (0x7E), -M to 0xFE;
    # 1 * 2^-119 is far below e4m3's smallest subnormal (2^-9): 0x00; NaN -> +0: 0x00.
    q, s = X8.quantize(_row(32, [PINF, ONE, QNAN, NINF]))
    assert q[0, :4].tolist() == [0x7E, 0x00, 0x00, 0xFE] and not q[0, 4:].any()
    assert s.tolist() == [[0xF6]]


def test_mxfp4_block_with_inf_and_nan():
    # Es = 127 - 2 = 125, byte 252 (0xFC); M 2^-125 = 7.97 saturates to 6 (code 7), -M to 0xF;
    # 1 * 2^-125 -> 0; NaN -> 0. Bytes (7 | 0 << 4), (0 | 0xF << 4).
    packed, s = X4.quantize(_row(32, [PINF, ONE, QNAN, NINF]), layout="linear")
    assert packed[0, :2].tolist() == [0x07, 0xF0] and not packed[0, 2:].any()
    assert s.tolist() == [[0xFC]]
