"""Host-side checks of the W2A8 boundary: mk_w2a8_pack writes the documented
bit layout (decoded here independently), rejects bad input, and the device
entry points reject bad sizes before touching a GPU."""

import ctypes

import numpy as np
import pytest

from persistent_megakernel_cu_amd import binding as mkb
from synth_inputs import make_w2a8_case


def unpack(packed: np.ndarray, cols: int) -> np.ndarray:
    """Codes from the layout stated in include/mk.h: column 16 w + 4 k + m of
    a row is code + 1 at bits 8 m + 2 k of word w."""
    rows = packed.shape[0]
    out = np.zeros((rows, cols), dtype=np.int8)
    for w in range(cols // 16):
        word = packed[:, w].astype(np.uint64)
        for k in range(4):
            for m in range(4):
                out[:, 16 * w + 4 * k + m] = ((word >> np.uint64(8 * m + 2 * k)) & np.uint64(3)).astype(np.int8) - 1
    return out


@pytest.mark.parametrize("rows,cols", [(1, 64), (7, 192), (33, 4096)])
def test_pack_layout(rows, cols):
    codes, _, _ = make_w2a8_case(rows, cols, master=3)
    packed = mkb.w2a8_pack(codes)
    assert packed.shape == (rows, cols // 16) and packed.dtype == np.uint32
    assert np.array_equal(unpack(packed, cols), codes)
    # no field holds the unused value 3
    p = packed.astype(np.uint64)
    assert not np.any(((p >> np.uint64(1)) & p & np.uint64(0x55555555)) != 0)


def test_pack_single_column_positions():
    # a lone +1 at column c lands at word c // 16, bits 8 (c % 4) + 2 ((c % 16) // 4), value 2
    for c in (0, 1, 3, 4, 5, 15, 16, 63):
        codes = np.zeros((1, 64), dtype=np.int8)
        codes[0, c] = 1
        packed = mkb.w2a8_pack(codes)
        w, k, m = c // 16, (c % 16) // 4, c % 4
        expect = np.full(4, 0x55555555, dtype=np.uint32)         # every other field holds code 0 + 1
        expect[w] = (expect[w] & ~np.uint32(3 << (8 * m + 2 * k))) | np.uint32(2 << (8 * m + 2 * k))
        assert np.array_equal(packed[0], expect), c


def test_pack_rejects_bad_input():
    with pytest.raises(mkb.MkError) as e:
        mkb.w2a8_pack(np.zeros((2, 96), dtype=np.int8))          # cols not a multiple of 64
    assert e.value.code == mkb.MK_E_INVAL
    bad = np.zeros((2, 64), dtype=np.int8)
    bad[1, 5] = 2
    with pytest.raises(mkb.MkError) as e:
        mkb.w2a8_pack(bad)
    assert e.value.code == mkb.MK_E_INVAL


def test_device_entry_points_reject_bad_sizes_without_a_gpu():
    L = mkb.lib()
    dummy = ctypes.c_void_p(16)
    assert L.mk_w2a8_quantize(dummy, 100, dummy, dummy, None) == mkb.MK_E_INVAL       # not a multiple of 64
    assert L.mk_w2a8_quantize(dummy, 16384 + 64, dummy, dummy, None) == mkb.MK_E_INVAL
    assert L.mk_w2a8_gemv(dummy, dummy, 4, 16448, dummy, dummy, dummy, None) == mkb.MK_E_INVAL
    assert L.mk_w2a8_gemv(dummy, dummy, -1, 64, dummy, dummy, dummy, None) == mkb.MK_E_INVAL
    assert L.mk_w2a8_gemv(ctypes.c_void_p(24), dummy, 4, 64, dummy, dummy, dummy, None) == mkb.MK_E_INVAL  # misaligned
    assert L.mk_w2a8_gemv(None, None, 0, 64, None, None, None, None) == mkb.MK_OK      # no rows: no-op
    assert L.mk_w2a8_linear(dummy, dummy, 4, 96, dummy, dummy, None) == mkb.MK_E_INVAL
    assert L.mk_w2a8_linear(dummy, dummy, 4, 64, ctypes.c_void_p(20), dummy, None) == mkb.MK_E_INVAL  # misaligned x
    assert L.mk_w2a8_linear(None, None, 0, 64, None, None, None) == mkb.MK_OK
