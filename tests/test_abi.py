"""The C ABI: the library loads, exports what include/ss.h declares, and rejects
bad arguments on the host before anything is enqueued (no GPU needed)."""
import ctypes
import os
import re

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "structured_sparse_quantized_amd", "libss.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libss.so not built")


def _declared():
    src = open(os.path.join(ROOT, "include", "ss.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(ss_[a-z0-9_]+)\s*\(", src)))


def test_every_declared_symbol_is_exported():
    import structured_sparse_quantized_amd as ss
    names = _declared()
    assert len(names) >= 10
    for name in names:
        assert hasattr(ss.lib, name), name
    assert set(names) == set(ss.EXPORTS)


def test_lifted_k_matches_oracle():
    import structured_sparse_quantized_amd as ss
    for n in range(2, 9):
        for K in (0, 1, 4, 7, 8, 12, 240, 250, 512, 3584, 4096, 14336, 18944):
            assert ss.lifted_k_logical(K, n) == oracle.lifted_k(K, n)
            assert ss.lifted_k(K, n) == oracle.lifted_k_alloc(K, n)
    assert ss.lifted_k(10, 1) == -1 and ss.lifted_k(10, 9) == -1 and ss.lifted_k(-1, 2) == -1


FAKE = ctypes.c_void_p(1 << 20)  # never dereferenced: validation fails first


def test_host_validation_statuses():
    import structured_sparse_quantized_amd as ss
    L = ss.lib
    # NULL input
    assert L.ss_prune24(None, ss.SS_F32, 4, 8, 8, ss.SS_I8, FAKE, 16, FAKE, 16, FAKE, None) == ss.SS_ERR_NULL
    assert b"NULL" in L.ss_last_error()
    # K not a multiple of 4
    assert L.ss_prune24(FAKE, ss.SS_F32, 4, 6, 8, ss.SS_I8, FAKE, 16, FAKE, 16, FAKE, None) == ss.SS_ERR_SHAPE
    # bad dtypes
    assert L.ss_prune24(FAKE, ss.SS_I8, 4, 8, 8, ss.SS_I8, FAKE, 256, FAKE, 32, FAKE, None) == ss.SS_ERR_DTYPE
    assert L.ss_quant_lift_act(FAKE, ss.SS_BF16, 4, 8, 8, 2, ss.SS_BF16, FAKE, 256, FAKE, None) == ss.SS_ERR_DTYPE
    # bad pattern
    assert L.ss_slide_decompose(FAKE, ss.SS_F32, 4, 8, 8, 1, ss.SS_I8, FAKE, 256, FAKE, 32, FAKE, None) == ss.SS_ERR_PATTERN
    assert L.ss_quant_lift_act(FAKE, ss.SS_BF16, 4, 8, 8, 9, ss.SS_I8, FAKE, 256, FAKE, None) == ss.SS_ERR_PATTERN
    # misaligned pointer and row stride
    odd = ctypes.c_void_p((1 << 20) + 4)
    assert L.ss_quant_lift_act(odd, ss.SS_BF16, 4, 8, 8, 2, ss.SS_I8, FAKE, 256, FAKE, None) == ss.SS_ERR_ALIGN
    assert L.ss_quant_lift_act(FAKE, ss.SS_BF16, 4, 12, 12, 2, ss.SS_I8, FAKE, 256, FAKE, None) == ss.SS_ERR_ALIGN
    # leading dimension smaller than the row
    assert L.ss_quant_lift_act(FAKE, ss.SS_BF16, 4, 16, 8, 2, ss.SS_I8, FAKE, 256, FAKE, None) == ss.SS_ERR_SHAPE
    # spgemm: Kc not aligned, I32 with fp8, missing scales, bad side
    args = (FAKE, 128, FAKE, 32, FAKE, 256, FAKE, FAKE)
    assert L.ss_spgemm(0, 4, 4, 100, ss.SS_I8, *args, ss.SS_I32, FAKE, 16, None) == ss.SS_ERR_SHAPE
    assert L.ss_spgemm(0, 4, 4, 256, ss.SS_FP8E4M3, *args, ss.SS_I32, FAKE, 16, None) == ss.SS_ERR_DTYPE
    assert L.ss_spgemm(0, 4, 4, 256, ss.SS_I8, FAKE, 128, FAKE, 32, FAKE, 256, None, FAKE, ss.SS_BF16, FAKE, 8,
                       None) == ss.SS_ERR_NULL
    assert L.ss_spgemm(5, 4, 4, 256, ss.SS_I8, *args, ss.SS_BF16, FAKE, 8, None) == ss.SS_ERR_SHAPE
    # BF16 output with a scale pointer
    assert L.ss_prune24_act(FAKE, ss.SS_BF16, 4, 8, 8, ss.SS_BF16, FAKE, 128, FAKE, 32, FAKE, None) == ss.SS_ERR_DTYPE
    # prune24_act needs BF16 activations
    assert L.ss_prune24_act(FAKE, ss.SS_F32, 4, 8, 8, ss.SS_BF16, FAKE, 128, FAKE, 32, None, None) == ss.SS_ERR_DTYPE


def test_empty_problems_are_ok_without_launch():
    import structured_sparse_quantized_amd as ss
    L = ss.lib
    assert L.ss_quant_lift_act(FAKE, ss.SS_BF16, 0, 64, 64, 4, ss.SS_I8, FAKE, 256, FAKE, None) == ss.SS_OK
    assert L.ss_prune24(FAKE, ss.SS_F32, 0, 64, 64, ss.SS_I8, FAKE, 128, FAKE, 32, FAKE, None) == ss.SS_OK
    assert L.ss_spgemm(0, 0, 16, 256, ss.SS_I8, FAKE, 128, FAKE, 32, FAKE, 256, FAKE, FAKE, ss.SS_BF16, FAKE, 16,
                       None) == ss.SS_OK
    assert L.ss_last_error() == b""


def _tiled_sizes(rows, Kc, es=1):
    # the sizes the tiled layout description in include/ss.h fixes
    ks4 = -(-(Kc * es // 128) // 4)
    rb = -(-rows // 16)
    return rb * ks4 * 4 * 1024, rb * ks4 * 256 * (4 // es)


def test_tiled_sizes():
    import structured_sparse_quantized_amd as ss
    for rows in (1, 15, 16, 17, 300, 4096, 28672):
        for Kc in (256, 512, 768, 1024, 6144, 61440):
            assert ss.tiled_bytes(rows, Kc, "i8") == _tiled_sizes(rows, Kc)
            assert ss.tiled_bytes(rows, Kc, "fp8") == _tiled_sizes(rows, Kc)
            assert ss.tiled_bytes(rows, Kc, "bf16") == _tiled_sizes(rows, Kc, 2)
    assert ss.tiled_bytes(0, 256) == (0, 0)
    assert ss.lib.ss_tiled_vals_bytes(4, 100, ss.SS_I8) == -1 and ss.lib.ss_tiled_meta_bytes(-1, 256, ss.SS_I8) == -1
    assert ss.lib.ss_tiled_vals_bytes(4, 256, ss.SS_F32) == -1


def test_tiled_validation_statuses():
    import structured_sparse_quantized_amd as ss
    L = ss.lib
    # pack: I8 / FP8 / BF16 values; other types are errors
    assert L.ss_pack_sparse(4, 256, ss.SS_F32, FAKE, 128, FAKE, 32, FAKE, FAKE, None) == ss.SS_ERR_DTYPE
    assert L.ss_pack_sparse(4, 256, ss.SS_BF16, FAKE, 100, FAKE, 32, FAKE, FAKE, None) == ss.SS_ERR_SHAPE
    assert L.ss_pack_sparse(4, 100, ss.SS_I8, FAKE, 128, FAKE, 32, FAKE, FAKE, None) == ss.SS_ERR_SHAPE
    assert L.ss_pack_sparse(4, 256, ss.SS_I8, FAKE, 100, FAKE, 32, FAKE, FAKE, None) == ss.SS_ERR_SHAPE
    assert L.ss_pack_sparse(4, 256, ss.SS_I8, FAKE, 128, FAKE, 32, None, FAKE, None) == ss.SS_ERR_NULL
    odd = ctypes.c_void_p((1 << 20) + 8)
    assert L.ss_pack_sparse(4, 256, ss.SS_I8, FAKE, 128, FAKE, 32, odd, FAKE, None) == ss.SS_ERR_ALIGN
    assert L.ss_pack_sparse(0, 256, ss.SS_I8, FAKE, 128, FAKE, 32, FAKE, FAKE, None) == ss.SS_OK
    # one-pass prune into the tiled layout
    P = L.ss_prune24_act_tiled
    assert P(FAKE, ss.SS_F32, 4, 8, 8, ss.SS_I8, FAKE, FAKE, FAKE, None) == ss.SS_ERR_DTYPE
    assert P(FAKE, ss.SS_BF16, 4, 6, 8, ss.SS_I8, FAKE, FAKE, FAKE, None) == ss.SS_ERR_SHAPE
    assert P(FAKE, ss.SS_BF16, 4, 8, 8, ss.SS_I8, FAKE, FAKE, None, None) == ss.SS_ERR_NULL
    assert P(FAKE, ss.SS_BF16, 4, 8, 8, ss.SS_BF16, FAKE, FAKE, FAKE, None) == ss.SS_ERR_DTYPE
    assert P(FAKE, ss.SS_BF16, 4, 8, 8, ss.SS_I8, None, FAKE, FAKE, None) == ss.SS_ERR_NULL
    assert P(FAKE, ss.SS_BF16, 0, 8, 8, ss.SS_I8, FAKE, FAKE, FAKE, None) == ss.SS_OK
    # one-pass weight preparation into the tiled layout
    S = L.ss_slide_decompose_tiled
    assert S(FAKE, ss.SS_F32, 4, 8, 8, 1, ss.SS_I8, FAKE, FAKE, FAKE, None) == ss.SS_ERR_PATTERN
    assert S(FAKE, ss.SS_F32, 4, 8, 8, 9, ss.SS_I8, FAKE, FAKE, FAKE, None) == ss.SS_ERR_PATTERN
    assert S(FAKE, ss.SS_I8, 4, 8, 8, 4, ss.SS_I8, FAKE, FAKE, FAKE, None) == ss.SS_ERR_DTYPE
    assert S(FAKE, ss.SS_F32, 4, 8, 8, 4, ss.SS_F32, FAKE, FAKE, FAKE, None) == ss.SS_ERR_DTYPE
    assert S(FAKE, ss.SS_F32, 4, 8, 8, 4, ss.SS_I8, FAKE, FAKE, None, None) == ss.SS_ERR_NULL
    assert S(FAKE, ss.SS_F32, 4, 8, 8, 4, ss.SS_BF16, FAKE, FAKE, FAKE, None) == ss.SS_ERR_DTYPE
    assert S(FAKE, ss.SS_F32, 4, 8, 8, 4, ss.SS_I8, None, FAKE, FAKE, None) == ss.SS_ERR_NULL
    assert S(FAKE, ss.SS_F32, 4, 8, 8, 4, ss.SS_I8, odd, FAKE, FAKE, None) == ss.SS_ERR_ALIGN
    assert S(FAKE, ss.SS_F32, 4, 8, 6, 4, ss.SS_I8, FAKE, FAKE, FAKE, None) == ss.SS_ERR_SHAPE
    assert S(None, ss.SS_F32, 4, 8, 8, 4, ss.SS_I8, FAKE, FAKE, FAKE, None) == ss.SS_ERR_NULL
    assert S(FAKE, ss.SS_F32, -1, 8, 8, 4, ss.SS_I8, FAKE, FAKE, FAKE, None) == ss.SS_ERR_SHAPE
    assert S(FAKE, ss.SS_F32, 0, 8, 8, 4, ss.SS_I8, FAKE, FAKE, FAKE, None) == ss.SS_OK
    assert S(FAKE, ss.SS_F32, 4, 0, 8, 4, ss.SS_I8, FAKE, FAKE, FAKE, None) == ss.SS_OK
    # workspace query and the split-K entry point
    Q = L.ss_spgemm_tiled_workspace_bytes
    assert Q(ss.SS_SPARSE_W, 64, 3584, 25344, ss.SS_I8) > 0          # few tokens, few row tiles
    assert Q(ss.SS_SPARSE_W, 16, 3584, 25344, ss.SS_I8) == 0         # row-block kernel, no workspace
    assert Q(ss.SS_SPARSE_W, 4096, 4096, 4096, ss.SS_I8) == 0        # prefill
    assert Q(ss.SS_SPARSE_X, 64, 3584, 4096, ss.SS_I8) == 0
    assert Q(ss.SS_SPARSE_W, 64, 3584, 100, ss.SS_I8) == -1
    assert Q(ss.SS_SPARSE_W, 64, 3584, 4096, ss.SS_F32) == -1
    assert Q(ss.SS_SPARSE_W, 0, 3584, 4096, ss.SS_I8) == 0
    need = Q(ss.SS_SPARSE_W, 64, 3584, 4096, ss.SS_I8)
    def gw(ws=FAKE, nb=need, M=64, N=3584, Kc=4096):
        return L.ss_spgemm_tiled_ws(0, M, N, Kc, ss.SS_I8, FAKE, FAKE, FAKE, Kc, FAKE, FAKE, ss.SS_BF16, FAKE, N,
                                    ws, nb, None)
    assert gw(ws=None) == ss.SS_ERR_NULL
    assert gw(nb=need - 16) == ss.SS_ERR_SHAPE
    assert gw(nb=-1) == ss.SS_ERR_SHAPE
    assert gw(ws=odd) == ss.SS_ERR_ALIGN
    assert gw(M=0) == ss.SS_OK
    # product
    def g(side=0, M=4, N=4, Kc=256, ab=ss.SS_I8, tv=FAKE, tm=FAKE, d=FAKE, ldd=256, sx=FAKE, sw=FAKE,
          y=ss.SS_BF16, Y=FAKE, ldy=8):
        return L.ss_spgemm_tiled(side, M, N, Kc, ab, tv, tm, d, ldd, sx, sw, y, Y, ldy, None)
    assert g(ab=ss.SS_F32) == ss.SS_ERR_DTYPE
    assert g(ab=ss.SS_BF16, y=ss.SS_I32) == ss.SS_ERR_DTYPE
    assert g(Kc=100) == ss.SS_ERR_SHAPE
    assert g(Kc=0) == ss.SS_ERR_SHAPE
    assert g(side=3) == ss.SS_ERR_SHAPE
    assert g(ab=ss.SS_FP8E4M3, y=ss.SS_I32) == ss.SS_ERR_DTYPE
    assert g(sx=None) == ss.SS_ERR_NULL
    assert g(tm=None) == ss.SS_ERR_NULL
    assert g(ldd=100) == ss.SS_ERR_SHAPE
    assert g(tv=odd) == ss.SS_ERR_ALIGN
    # dense operand beyond 32-bit byte offsets
    assert g(M=70000, ldd=65536, Kc=65536) == ss.SS_ERR_UNSUPPORTED
    assert g(M=0) == ss.SS_OK and g(N=0) == ss.SS_OK


def test_block_scaled_validation_statuses():
    import structured_sparse_quantized_amd as ss
    L = ss.lib
    odd = ctypes.c_void_p((1 << 20) + 8)
    P = L.ss_prune24_block
    assert P(FAKE, ss.SS_I8, 4, 8, 8, FAKE, FAKE, FAKE, None) == ss.SS_ERR_DTYPE
    assert P(FAKE, ss.SS_F32, 4, 6, 8, FAKE, FAKE, FAKE, None) == ss.SS_ERR_SHAPE
    assert P(FAKE, ss.SS_F32, 4, 8, 6, FAKE, FAKE, FAKE, None) == ss.SS_ERR_SHAPE
    assert P(FAKE, ss.SS_F32, 4, 8, 8, FAKE, FAKE, None, None) == ss.SS_ERR_NULL
    assert P(FAKE, ss.SS_F32, 4, 8, 8, None, FAKE, FAKE, None) == ss.SS_ERR_NULL
    assert P(FAKE, ss.SS_F32, 4, 8, 8, odd, FAKE, FAKE, None) == ss.SS_ERR_ALIGN
    assert P(None, ss.SS_F32, 4, 8, 8, FAKE, FAKE, FAKE, None) == ss.SS_ERR_NULL
    assert P(FAKE, ss.SS_F32, -1, 8, 8, FAKE, FAKE, FAKE, None) == ss.SS_ERR_SHAPE
    assert P(FAKE, ss.SS_F32, 0, 8, 8, FAKE, FAKE, FAKE, None) == ss.SS_OK
    Q = L.ss_quant_group_act
    assert Q(FAKE, ss.SS_I8, 4, 100, 104, FAKE, 256, FAKE, None) == ss.SS_ERR_DTYPE
    assert Q(FAKE, ss.SS_BF16, 4, 100, 104, FAKE, 100, FAKE, None) == ss.SS_ERR_SHAPE   # ldq < Kc = 256
    assert Q(FAKE, ss.SS_BF16, 4, 100, 100, FAKE, 256, FAKE, None) == ss.SS_ERR_ALIGN   # 200-byte rows
    assert Q(FAKE, ss.SS_BF16, 4, 100, 104, FAKE, 256, None, None) == ss.SS_ERR_NULL
    assert Q(FAKE, ss.SS_BF16, 4, 100, 104, None, 256, FAKE, None) == ss.SS_ERR_NULL
    assert Q(FAKE, ss.SS_BF16, 0, 100, 104, FAKE, 256, FAKE, None) == ss.SS_OK
    def g(M=4, N=4, Kc=256, tv=FAKE, tm=FAKE, d=FAKE, ldd=256, sx=FAKE, sw=FAKE, y=ss.SS_BF16, Y=FAKE, ldy=8):
        return L.ss_spgemm_tiled_block(M, N, Kc, tv, tm, d, ldd, sx, sw, y, Y, ldy, None)
    assert g(y=ss.SS_I32) == ss.SS_ERR_DTYPE and g(y=ss.SS_FP8E4M3) == ss.SS_ERR_DTYPE
    assert g(Kc=100) == ss.SS_ERR_SHAPE and g(Kc=0) == ss.SS_ERR_SHAPE and g(M=-1) == ss.SS_ERR_SHAPE
    assert g(sx=None) == ss.SS_ERR_NULL and g(sw=None) == ss.SS_ERR_NULL and g(tm=None) == ss.SS_ERR_NULL
    assert g(ldd=100) == ss.SS_ERR_SHAPE and g(tv=odd) == ss.SS_ERR_ALIGN and g(d=odd) == ss.SS_ERR_ALIGN
    assert g(M=70000, ldd=65536, Kc=65536) == ss.SS_ERR_UNSUPPORTED
    assert g(M=0) == ss.SS_OK and g(N=0) == ss.SS_OK


def test_fused_decode_validation_statuses():
    import structured_sparse_quantized_amd as ss
    L = ss.lib
    odd = ctypes.c_void_p((1 << 20) + 8)
    def f(X=FAKE, xdt=ss.SS_BF16, M=2, K=3584, ldx=3584, n=3, q=ss.SS_I8, tv=FAKE, tm=FAKE, sw=FAKE, N=4608,
          y=ss.SS_BF16, Y=FAKE, ldy=4608, sxo=None):
        return L.ss_quant_lift_spgemm_decode(X, xdt, M, K, ldx, n, q, tv, tm, sw, N, y, Y, ldy, sxo, None)
    assert f(n=1) == ss.SS_ERR_PATTERN and f(n=9) == ss.SS_ERR_PATTERN
    assert f(xdt=ss.SS_I8) == ss.SS_ERR_DTYPE and f(q=ss.SS_BF16) == ss.SS_ERR_DTYPE
    assert f(y=ss.SS_FP8E4M3) == ss.SS_ERR_DTYPE and f(q=ss.SS_FP8E4M3, y=ss.SS_I32) == ss.SS_ERR_DTYPE
    assert f(M=5) == ss.SS_ERR_UNSUPPORTED                       # more than four tokens
    assert f(M=4, K=20488, ldx=20488) == ss.SS_ERR_UNSUPPORTED    # bf16 row longer than the register share
    assert f(M=4, K=18944, ldx=18944, n=8) == ss.SS_ERR_UNSUPPORTED  # 4 x K' > 128 KB of LDS
    assert f(ldx=100) == ss.SS_ERR_SHAPE and f(X=None) == ss.SS_ERR_NULL and f(X=odd) == ss.SS_ERR_ALIGN
    assert f(tv=None) == ss.SS_ERR_NULL and f(tm=odd) == ss.SS_ERR_ALIGN and f(sw=None) == ss.SS_ERR_NULL
    assert f(K=0) == ss.SS_ERR_SHAPE and f(M=-1) == ss.SS_ERR_SHAPE
    assert f(M=0) == ss.SS_OK and f(N=0) == ss.SS_OK


def test_batched_validation_statuses():
    import structured_sparse_quantized_amd as ss
    L = ss.lib
    def b(batch=2, M=64, N=64, Kc=256, tvs=16384, tms=4096, ldd=256, ds=64 * 256, y=ss.SS_BF16, ldy=64, ys=64 * 64,
          side=ss.SS_SPARSE_X, ab=ss.SS_I8, sx=FAKE, sw=FAKE):
        return L.ss_spgemm_tiled_batched(side, batch, M, N, Kc, ab, FAKE, tvs, FAKE, tms, FAKE, ldd, ds, sx, 64, sw, 64,
                                         y, FAKE, ldy, ys, None)
    assert b(batch=-1) == ss.SS_ERR_SHAPE and b(batch=65536) == ss.SS_ERR_SHAPE
    assert b(tvs=8) == ss.SS_ERR_ALIGN and b(tms=4) == ss.SS_ERR_ALIGN and b(ds=8) == ss.SS_ERR_ALIGN
    assert b(ys=4) == ss.SS_ERR_ALIGN and b(tvs=-16) == ss.SS_ERR_SHAPE
    assert b(Kc=100) == ss.SS_ERR_SHAPE and b(ab=ss.SS_F32) == ss.SS_ERR_DTYPE and b(sx=None) == ss.SS_ERR_NULL
    assert b(batch=0) == ss.SS_OK and b(M=0) == ss.SS_OK


def test_binding_checks_tensor_sizes_before_the_call():
    """The C ABI sees pointers only; the binding compares every tensor with the region the call would touch
    and raises before anything is launched: too small -> SS_ERR_SHAPE, wrong dtype -> SS_ERR_DTYPE, a host
    tensor of the right size -> SS_ERR_UNSUPPORTED (the library runs on the GPU only)."""
    import torch
    import structured_sparse_quantized_amd as ss
    M, N, Kc = 20, 48, 512
    nv, nm = ss.tiled_bytes(N, Kc, "i8")
    u8 = lambda n: torch.zeros(n, dtype=torch.uint8)  # noqa: E731
    good = dict(tvals=u8(nv), tmeta=u8(nm), dense=torch.zeros((M, Kc), dtype=torch.int8),
                sx=torch.ones(M), sw=torch.ones(N), out=torch.zeros((M, N), dtype=torch.bfloat16))

    def call(**kw):
        a = dict(good, **kw)
        return ss.spgemm_tiled(ss.SS_SPARSE_W, M, N, Kc, a["tvals"], a["tmeta"], a["dense"], a["sx"], a["sw"], "bf16",
                               out=a["out"], workspace=False)

    def status(fn):
        with pytest.raises(ss.SSError) as e:
            fn()
        return e.value.status

    assert status(lambda: call(tvals=u8(nv - 1))) == ss.SS_ERR_SHAPE
    assert status(lambda: call(tmeta=u8(nm - 16))) == ss.SS_ERR_SHAPE
    assert status(lambda: call(dense=torch.zeros((M - 1, Kc), dtype=torch.int8))) == ss.SS_ERR_SHAPE
    assert status(lambda: call(dense=torch.zeros((M, Kc - 16), dtype=torch.int8))) == ss.SS_ERR_SHAPE
    assert status(lambda: call(sx=torch.ones(M - 1))) == ss.SS_ERR_SHAPE
    assert status(lambda: call(sw=torch.ones(N - 1))) == ss.SS_ERR_SHAPE
    assert status(lambda: call(out=torch.zeros((M, N - 1), dtype=torch.bfloat16))) == ss.SS_ERR_SHAPE
    assert status(lambda: call(out=torch.zeros((M, N), dtype=torch.float32))) == ss.SS_ERR_DTYPE
    assert status(lambda: call(sx=torch.ones(M, dtype=torch.float64))) == ss.SS_ERR_DTYPE
    assert status(lambda: call()) == ss.SS_ERR_UNSUPPORTED  # right sizes, host memory
    # the other entry points that take caller buffers
    X = torch.zeros((M, 100), dtype=torch.bfloat16)
    Kq = ss.lifted_k(100, 4)
    assert status(lambda: ss.quant_lift_act(X, 4, "i8", out=(torch.zeros((M, Kq - 16), dtype=torch.int8),
                                                                torch.ones(M)))) == ss.SS_ERR_SHAPE
    assert status(lambda: ss.quant_lift_act(X, 4, "i8", out=(torch.zeros((M, Kq), dtype=torch.int8),
                                                                torch.ones(M - 1)))) == ss.SS_ERR_SHAPE
    W = torch.zeros((N, 256))
    assert status(lambda: ss.slide_decompose_tiled(W, 2, "i8", out=(u8(nv // 2), u8(nm // 2), torch.ones(N)))) == \
        ss.SS_ERR_SHAPE
    assert status(lambda: ss.prune24(W, "i8", out=(torch.zeros((N, 100), dtype=torch.int8),
                                                   torch.zeros((N, 32), dtype=torch.uint8), torch.ones(N)))) == \
        ss.SS_ERR_SHAPE
    Xd = torch.zeros((4, 3584), dtype=torch.bfloat16)
    assert status(lambda: ss.quant_lift_spgemm_decode(Xd, 3, u8(16), u8(16), torch.ones(N), N)) == ss.SS_ERR_SHAPE
    B = 2
    assert status(lambda: ss.spgemm_tiled_batched(ss.SS_SPARSE_W, B, M, N, Kc, u8(nv), u8(2 * nm),
                                                  torch.zeros((B, M, Kc), dtype=torch.int8), None, None,
                                                  "i32")) == ss.SS_ERR_SHAPE
