"""Pins of the oracle's MFMA 16x16x128 scale layout (an index map).

The hardware fact it encodes (measured with one-wave probes of the gfx950
scaled matrix instruction): for one 128-element K step, the scale byte of A
row r and 32-element block q comes from lane r + 16 q, byte ``opsel``.  The
checks below restate that from the lane's side -- what each lane must find
in its register for each of the four K steps a record covers -- and check
hand-worked offsets and that the map is a bijection onto the records.  The
GPU test that runs the instruction on quantizer output pins it to the
hardware."""
import numpy as np
import pytest

import oracle


def test_hand_worked_offsets():
    lds = 512                                # two records per row group (K = 1024)
    cases = {(0, 0): 0, (1, 0): 4, (15, 0): 60, (0, 1): 64, (0, 3): 192, (0, 4): 1, (0, 8): 2,
             (0, 12): 3, (0, 15): 195, (15, 15): 255, (0, 16): 256, (3, 17): 256 + 12 + 64,
             (16, 0): 512, (17, 5): 512 + 4 + 64 + 1, (40, 31): 2 * 512 + 256 + 4 * (8 + 48) + 3}
    for (r, kb), off in cases.items():
        assert oracle.mfma16_scale_offset(r, kb, lds) == off, (r, kb)


def test_each_record_is_a_permutation():
    offs = sorted(oracle.mfma16_scale_offset(r, kb, 256) for r in range(16) for kb in range(16))
    assert offs == list(range(256))


@pytest.mark.parametrize("rows,nblk", [(16, 16), (37, 40), (5, 3), (128, 224)])
def test_lane_view_of_the_layout(rows, nblk):
    rng = np.random.default_rng(rows + nblk)
    s = rng.integers(0, 256, (rows, nblk)).astype(np.uint8)
    lay = oracle.scales_to_mfma16(s, fill=0xEE)
    assert lay.shape == ((rows + 15) // 16, ((nblk + 15) // 16) * 256)
    for g in range(lay.shape[0]):
        for rec in range(lay.shape[1] // 256):
            dwords = lay[g, rec * 256:(rec + 1) * 256].reshape(64, 4)   # lane L, byte T
            for L in range(64):
                r, q = 16 * g + L % 16, L // 16
                for T in range(4):
                    kb = 16 * rec + 4 * T + q       # K step T of this record, block q of the step
                    want = s[r, kb] if (r < rows and kb < nblk) else 0xEE
                    assert dwords[L, T] == want, (g, rec, L, T)


def test_rejects_a_short_row_group_stride():
    with pytest.raises(ValueError):
        oracle.scales_to_mfma16(np.zeros((4, 20), np.uint8), lds_out=256)
