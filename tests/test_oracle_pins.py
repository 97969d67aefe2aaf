"""The CPU oracle against its pins (hand-worked blocks, closed forms,
invariants, library routines).  No GPU."""
import numpy as np
import pytest

import pins


@pytest.mark.parametrize("pin", pins.PINS, ids=[p.__name__ for p in pins.PINS])
def test_pin(orc, pin):
    pin(orc)


def test_half_to_float_exhaustive(orc):
    """All 65,536 binary16 patterns against numpy's binary16 -> float32."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = orc.half_to_float_array(bits)
    want = bits.view(np.float16).astype(np.float32)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), want[~nan].view(np.uint32))


def test_float_to_half_exhaustive(orc):
    """All 2^32 binary32 patterns, one biased exponent (2^23 patterns) of one
    sign at a time.  Exponents 102..142 (values that round to a finite
    nonzero binary16, or tie with the smallest one) are checked against
    numpy's float32 -> binary16 conversion (RNE).  Below that every value is
    a signed zero and above it a signed infinity, by the binary16 range
    (smallest subnormal 2^-24, largest finite 65504).  NaN must stay NaN
    (payloads are not part of the definition)."""
    half = 1 << 23
    base = np.arange(half, dtype=np.uint32)
    for start in range(0, 1 << 32, half):
        bits = base + np.uint32(start)
        vals = bits.view(np.float32)
        got = orc.float_to_half_array(vals)
        sign = np.uint16(0x8000 if start >= (1 << 31) else 0)
        e = (start >> 23) & 0xFF
        if e == 255:
            assert got[0] == (sign | 0x7C00), "infinity"
            g = got[1:]
            assert np.all(((g & 0x7C00) == 0x7C00) & ((g & 0x03FF) != 0)), "NaN must stay NaN"
            continue
        if e <= 101:
            assert np.all(got == sign), f"exponent {e}: must round to a signed zero"
        elif e >= 143:
            assert np.all(got == (sign | 0x7C00)), f"exponent {e}: must overflow to infinity"
        else:
            with np.errstate(over="ignore"):
                want = vals.astype(np.float16).view(np.uint16)
            bad = got != want
            assert not bad.any(), f"first mismatch at {int(bits[np.argmax(bad)]):#010x}"


def test_geometry(orc):
    assert [orc.block_size(t) for t in (1, 2, 8, 12, 13, 14, 10)] == [1, 32, 32, 256, 256, 256, 256]
    assert [orc.type_size(t) for t in (1, 2, 8, 12, 13, 14, 10)] == [2, 18, 34, 144, 176, 210, 84]
    assert orc.row_bytes(14, 4173) == 17 * 210
    assert orc.row_bytes(2, 128) == 4 * 18
    assert orc.block_size(3) == -1
