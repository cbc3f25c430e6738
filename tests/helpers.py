"""Shared test helpers: moving seeded numpy inputs to the GPU and results back."""
import numpy as np
import torch


def have_gpu() -> bool:
    return torch.cuda.is_available()


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def dev_f32(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def dev_u8(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.uint8)).cuda()


def dev_codes(codes: np.ndarray, q: str) -> torch.Tensor:
    """Oracle codes (int8 / E4M3 bytes / bf16 bits) as a device tensor of the matching dtype."""
    if q == "i8":
        return torch.from_numpy(np.ascontiguousarray(codes, dtype=np.int8)).cuda()
    if q == "fp8":
        return torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).cuda().view(torch.float8_e4m3fn)
    if q == "bf16":
        return dev_bf16(codes)
    raise ValueError(q)


def host(t: torch.Tensor) -> np.ndarray:
    """Raw host copy: int8 / uint8 bytes / uint16 bf16 bits / float32 / int32."""
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).cpu().numpy()
    return t.cpu().numpy()


def rel_fro(a: np.ndarray, b: np.ndarray) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    den = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (den if den > 0 else 1.0))


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def sum_abs_terms(sp_vals, sp_meta, dense_codes, Kc, ab, s_dense=None, s_sparse=None):
    """Sum over k of |a[r, k]| |b[c, k]|, times |s_dense[c]| |s_sparse[r]| when given: the magnitude sum that
    bounds the rounding of one output element (rows c of the dense operand x rows r of the sparse one), in
    float64 from the oracle's decoded codes."""
    import oracle
    dec = {"i8": lambda v: np.asarray(v, np.int8).astype(np.float64), "fp8": oracle.e4m3_decode,
           "bf16": lambda v: oracle.bf16_bits_to_f32(v).astype(np.float64)}[ab]
    a = np.abs(oracle.decompress24(dec(sp_vals)[:, : Kc // 2], sp_meta, Kc))
    b = np.abs(dec(dense_codes))[:, :Kc]
    t = b @ a.T
    if s_dense is not None:
        t = t * np.abs(np.asarray(s_dense, np.float64))[:, None]
    if s_sparse is not None:
        t = t * np.abs(np.asarray(s_sparse, np.float64))[None, :]
    return t


def assert_elementwise(got, exp, terms, out="bf16", c=4e-5):
    """|got - exp| <= c * sum|terms| + one rounding step of the output type, element by element. c = 4e-5
    covers the matrix core's FP8 / bf16 dot products, which keep about 16 bits relative to the sum of the
    magnitudes (measured up to 1.6e-5 on one 128-position group); the output's own rounding (bf16: up to
    one unit in the last place, 2^-7 relative; f32: 2^-23) may land the two sides one step apart. A wrong
    tile edge, a dropped step or a wrong scale moves whole terms and fails by orders of magnitude."""
    got = np.asarray(got, np.float64)
    exp = np.asarray(exp, np.float64)
    step = 2.0 ** -7 if out == "bf16" else 2.0 ** -23
    bound = c * terms + step * np.abs(exp) + 1e-30
    bad = np.abs(got - exp) > bound
    assert not bad.any(), (f"{int(bad.sum())} of {bad.size} elements outside c*sum|terms| + rounding; worst ratio "
                           f"{float(np.max(np.abs(got - exp) / bound)):.3g}")


def assert_product(got, exp, side, sp_vals, sp_meta, dense_codes, Kc, ab, sx, sw, out, tol=1e-2):
    """A sparse product against the oracle's: INT8 bit for bit; FP8 / bf16 within `tol` relative Frobenius
    error and element by element within assert_elementwise's bound (side "W": the sparse operand holds the
    N weight rows and the dense one the M tokens; side "X" the other way round)."""
    if ab == "i8":
        assert np.array_equal(got, exp), out
        return
    if out == "bf16":
        g, e = bf16_to_f64(got), bf16_to_f64(exp)
    else:
        g, e = np.asarray(got, np.float64), np.asarray(exp, np.float64)
    assert rel_fro(g, e) <= tol
    if side == "W":
        terms = sum_abs_terms(sp_vals, sp_meta, dense_codes, Kc, ab, sx, sw)
    else:
        terms = sum_abs_terms(sp_vals, sp_meta, dense_codes, Kc, ab, sw, sx).T
    assert_elementwise(g, e, terms, out=out)
