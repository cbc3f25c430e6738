"""Expected bytes of the tiled sparse operand, re-indexed from the row-major
compressed operand as the layout description in include/ss.h states (test
plumbing; no arithmetic of the method)."""
import numpy as np


def tile_ref(vals: np.ndarray, meta: np.ndarray, es: int = 1):
    """Row-major compressed operand (uint8 views; vals [rows][Kc/2 * es] bytes, es = value bytes) ->
    expected tiled bytes."""
    rows = vals.shape[0]
    half = vals.shape[1] // es
    Kc = 2 * half
    ks = Kc * es // 128
    g = -(-ks // 4)
    rb = -(-rows // 16)
    wb = 4 // es  # index bytes per lane per step
    v = np.zeros((rb * 16, g * 4 * 64), np.uint8)
    v[:rows, : half * es] = vals
    m = np.full((rb * 16, g * 4 * 4 * wb), 0x44, np.uint8)
    m[:rows, : Kc // 8] = meta
    # values: [b][s][l] 16 bytes = v[16b + l%16][64s + 16(l/16) : +16]
    tv = v.reshape(rb, 16, g * 4, 4, 16).transpose(0, 2, 3, 1, 4).reshape(-1)
    # metadata: [b][gg][l][q] wb bytes = m[16b + l%16][4wb(4gg+q) + wb(l/16) : +wb]
    tm = m.reshape(rb, 16, g, 4, 4, wb).transpose(0, 2, 4, 1, 3, 5).reshape(-1)
    return tv, tm
