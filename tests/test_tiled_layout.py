"""The tiled-layout re-indexing used by the GPU tests, checked byte by byte
against positions picked by hand from the layout description (CPU only)."""
import numpy as np

from tiled_ref import tile_ref


def test_tile_ref_by_hand():
    """The re-indexing above against single hand-picked bytes of the layout."""
    rows, Kc = 24, 768  # 2 row blocks (rows 24..31 padding), 6 steps -> 8 padded steps, 2 groups
    vals = np.arange(rows * Kc // 2, dtype=np.int64).reshape(rows, Kc // 2).astype(np.uint8)
    meta = (np.arange(rows * Kc // 8, dtype=np.int64).reshape(rows, Kc // 8) * 7).astype(np.uint8)
    tv, tm = tile_ref(vals, meta)
    assert tv.size == 2 * 8 * 1024 and tm.size == 2 * 2 * 1024
    # block (b=1, s=5), lane l=37 (row 16+5, chunk 2), byte i=9
    b, s, l, i = 1, 5, 37, 9
    assert tv[(b * 8 + s) * 1024 + 16 * l + i] == vals[16 * b + l % 16, 64 * s + 16 * (l // 16) + i]
    # padding step and padding row are zero
    assert tv[(0 * 8 + 7) * 1024 + 16 * 3] == 0 and tv[(1 * 8 + 0) * 1024 + 16 * 15] == 0
    # metadata word of lane l=50 (row 2, chunk 3), step 4*1+1 = 5, byte 2
    gg, q, l, byte = 1, 1, 50, 2
    assert tm[(0 * 2 + gg) * 1024 + 16 * l + 4 * q + byte] == meta[l % 16, 16 * (4 * gg + q) + 4 * (l // 16) + byte]
    # step 6 (padding) of row 0
    assert tm[(0 * 2 + 1) * 1024 + 16 * 0 + 4 * 2] == 0x44


def test_tile_ref_bf16_by_hand():
    """BF16 values: same value bytes per step (64 K positions), 2-byte index words, 512-byte index blocks."""
    rows, Kc = 18, 512  # 2 row blocks, 8 steps of 64 K -> 2 groups
    vals = (np.arange(rows * Kc, dtype=np.int64).reshape(rows, Kc) % 251).astype(np.uint8)  # Kc/2 bf16 = Kc bytes
    meta = (np.arange(rows * Kc // 8, dtype=np.int64).reshape(rows, Kc // 8) * 5 % 256).astype(np.uint8)
    tv, tm = tile_ref(vals, meta, es=2)
    assert tv.size == 2 * 8 * 1024 and tm.size == 2 * 2 * 512
    b, s, l, i = 0, 6, 45, 3  # row 13, chunk 2
    assert tv[(b * 8 + s) * 1024 + 16 * l + i] == vals[16 * b + l % 16, 64 * s + 16 * (l // 16) + i]
    gg, q, l, byte = 1, 3, 17, 1  # row 1, chunk 1, step 7
    assert tm[(0 * 2 + gg) * 512 + 8 * l + 2 * q + byte] == meta[l % 16, 8 * (4 * gg + q) + 2 * (l // 16) + byte]
    # row 17 is real, row 18 is padding
    assert tm[(1 * 2 + 0) * 512 + 8 * 1] == meta[17, 0] and tm[(1 * 2 + 0) * 512 + 8 * 2] == 0x44
