"""GPU parity of the batched tiled product (ss_spgemm_tiled_batched) and of the online 2:4 operand roles of
attention it serves (deep reading of arXiv 2610.28947, introduction: either operand of a product can be the
2:4 one, pruned on the fly), one problem per head:

* S = Q K^T with Q pruned 2:4 along the head dimension (the reduction axis);
* O = P V with the attention probabilities P pruned 2:4 along the keys (V passed transposed, so the dense
  operand's rows run along the reduction).

Batched results equal one ss_spgemm_tiled call per problem bit for bit; the attention roles match the CPU
oracle (its 2:4 prune and product applied per head) within 1e-2 relative Frobenius error for bf16 and,
element by element, within 4e-5 sum|terms| plus one output rounding."""
import numpy as np
import pytest

import oracle
import synth
from helpers import (assert_elementwise, bf16_to_f64, dev_bf16, dev_codes, dev_f32, dev_u8, have_gpu, host, rel_fro,
                     sum_abs_terms)

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not have_gpu(), reason="needs a GPU")]


@pytest.fixture(scope="module")
def ss():
    import structured_sparse_quantized_amd as m
    return m


@pytest.mark.parametrize("q", ["i8", "fp8", "bf16"])
@pytest.mark.parametrize("side", ["X", "W"])
def test_batched_equals_single_calls(ss, side, q):
    import torch
    B, M, N, K = 3, 96, 208, 1024  # sparse rows a multiple of 16: the stacked tiled operand splits per problem
    sd = ss.SS_SPARSE_X if side == "X" else ss.SS_SPARSE_W
    rows_sp, rows_dn = (M, N) if side == "X" else (N, M)
    rng = np.random.default_rng(7)
    Xs = synth.f32_to_bf16_bits(rng.standard_normal((B * rows_sp, K)).astype(np.float32))
    tv, tm, ssc = ss.prune24_act_tiled(dev_bf16(Xs), q)
    if q == "bf16":
        dense = dev_bf16(synth.f32_to_bf16_bits(rng.standard_normal((B, rows_dn, K)).astype(np.float32) * 0.1))
        sxb = swb = None
    else:
        dq, dsc = ss.quant_lift_act(dev_f32(rng.standard_normal((B * rows_dn, K)).astype(np.float32)), 2, q)
        dense = dq.view(B, rows_dn, K)
        sp_scale, dn_scale = ssc.view(B, rows_sp), dsc.view(B, rows_dn)
        sxb, swb = (sp_scale, dn_scale) if side == "X" else (dn_scale, sp_scale)
    Yb = ss.spgemm_tiled_batched(sd, B, M, N, K, tv, tm, dense, sxb, swb, "f32")
    nv, nm = ss.tiled_bytes(rows_sp, K, q)
    for b in range(B):
        Y1 = ss.spgemm_tiled(sd, M, N, K, tv[b * nv:(b + 1) * nv], tm[b * nm:(b + 1) * nm], dense[b],
                             None if sxb is None else sxb[b], None if swb is None else swb[b], "f32", workspace=False)
        assert torch.equal(Yb[b], Y1), b


def _heads(seed, H, L, d):
    rng = np.random.default_rng(seed)
    q = synth.f32_to_bf16_bits(rng.standard_normal((H, L, d)).astype(np.float32))
    k = synth.f32_to_bf16_bits(rng.standard_normal((H, L, d)).astype(np.float32))
    v = synth.f32_to_bf16_bits(rng.standard_normal((H, L, d)).astype(np.float32))
    logits = rng.standard_normal((H, L, L)) * 2.0
    p = np.exp(logits - logits.max(axis=2, keepdims=True))
    p = synth.f32_to_bf16_bits((p / p.sum(axis=2, keepdims=True)).astype(np.float32))
    return q, k, v, p


@pytest.mark.parametrize("shape", [(2, 256, 128), (3, 512, 64), (4, 1024, 128)])
def test_qk_with_q_pruned_along_head_dim(ss, shape):
    H, L, d = shape
    q, k, _, _ = _heads(H + L + d, H, L, d)
    tv, tm, _ = ss.prune24_act_tiled(dev_bf16(q.reshape(H * L, d)), "bf16")
    Kc = ss.lifted_k(d, 2)
    kd = np.zeros((H, L, Kc), np.uint16)
    kd[:, :, :d] = k  # the dense operand spans Kc (zero past the head dimension)
    S = ss.spgemm_tiled_batched(ss.SS_SPARSE_X, H, L, L, Kc, tv, tm, dev_bf16(kd), None, None, "f32")
    got = host(S).astype(np.float64)
    for h in range(H):
        vals, meta, _ = oracle.prune24_act(q[h], "bf16")
        exp = oracle.spgemm_acc("X", vals, meta, kd[h], Kc, "bf16")
        assert rel_fro(got[h], exp) <= 1e-2
        assert_elementwise(got[h], exp, sum_abs_terms(vals, meta, kd[h], Kc, "bf16").T, out="f32")


@pytest.mark.parametrize("shape", [(2, 256, 128), (3, 512, 128), (2, 1000, 64)])
def test_pv_with_probabilities_pruned_along_keys(ss, shape):
    H, L, d = shape
    _, _, v, p = _heads(L + d, H, L, d)
    Kc = ss.lifted_k(L, 2)
    pw = np.zeros((H * L, -(-L // 8) * 8), np.uint16)  # rows padded to 16 bytes
    pw[:, :L] = p.reshape(H * L, L)
    M16 = -(-L // 16) * 16
    tv, tm, _ = ss.prune24_act_tiled(dev_bf16(pw)[:, :L], "bf16")
    vt = np.zeros((H, d, Kc), np.uint16)
    vt[:, :, :L] = v.transpose(0, 2, 1)  # V^T: rows along the keys
    if M16 == L:
        O = ss.spgemm_tiled_batched(ss.SS_SPARSE_X, H, L, d, Kc, tv, tm, dev_bf16(vt), None, None, "bf16")
        got = bf16_to_f64(host(O))
    else:  # rows per head not a multiple of 16: one tiled operand per head
        import torch
        outs = []
        for h in range(H):
            tvh, tmh, _ = ss.prune24_act_tiled(dev_bf16(pw[h * L:(h + 1) * L])[:, :L], "bf16")
            outs.append(ss.spgemm_tiled(ss.SS_SPARSE_X, L, d, Kc, tvh, tmh, dev_bf16(vt[h]), None, None, "bf16"))
        got = bf16_to_f64(host(torch.stack(outs)))
    for h in range(H):
        vals, meta, _ = oracle.prune24_act(p[h], "bf16")
        exp = oracle.spgemm("X", vals, meta, vt[h], Kc, "bf16", None, None, "bf16")
        assert rel_fro(got[h], bf16_to_f64(exp)) <= 1e-2
        assert_elementwise(got[h], bf16_to_f64(exp), sum_abs_terms(vals, meta, vt[h], Kc, "bf16").T, out="bf16")


@pytest.mark.parametrize("shape", [(2, 256, 128), (3, 512, 64), (2, 1000, 128)])
def test_qk_with_k_pruned_along_head_dim(ss, shape):
    """S = Q K^T with the keys pruned 2:4 along the head dimension: K is the sparse operand (side W of the
    batched product, one row per key), Q the dense one."""
    H, L, d = shape
    q, k, _, _ = _heads(3 * H + L + d, H, L, d)
    Kc = ss.lifted_k(d, 2)
    qd = np.zeros((H, L, Kc), np.uint16)
    qd[:, :, :d] = q
    got = []
    if L % 16 == 0:
        tv, tm, _ = ss.prune24_act_tiled(dev_bf16(k.reshape(H * L, d)), "bf16")
        S = ss.spgemm_tiled_batched(ss.SS_SPARSE_W, H, L, L, Kc, tv, tm, dev_bf16(qd), None, None, "f32")
        got = host(S).astype(np.float64)
    else:  # keys per head not a multiple of 16: one tiled operand per head
        for h in range(H):
            tv, tm, _ = ss.prune24_act_tiled(dev_bf16(k[h]), "bf16")
            got.append(host(ss.spgemm_tiled(ss.SS_SPARSE_W, L, L, Kc, tv, tm, dev_bf16(qd[h]), None, None, "f32")))
        got = np.stack(got).astype(np.float64)
    for h in range(H):
        vals, meta, _ = oracle.prune24_act(k[h], "bf16")
        exp = oracle.spgemm_acc("W", vals, meta, qd[h], Kc, "bf16")
        assert rel_fro(got[h], exp) <= 1e-2
        assert_elementwise(got[h], exp, sum_abs_terms(vals, meta, qd[h], Kc, "bf16"), out="f32")


@pytest.mark.parametrize("shape", [(2, 256, 128), (3, 512, 64), (2, 768, 128)])
def test_pv_with_v_pruned_along_keys(ss, shape):
    """O = P V with V pruned 2:4 along the keys (the reduction): V^T [d, L] is the sparse operand (side W,
    one row per head dimension), the probabilities P the dense one."""
    H, L, d = shape
    _, _, v, p = _heads(5 * L + d, H, L, d)
    Kc = ss.lifted_k(L, 2)
    vt = np.ascontiguousarray(v.transpose(0, 2, 1))  # [H, d, L]
    pd = np.zeros((H, L, Kc), np.uint16)
    pd[:, :, :L] = p
    tv, tm, _ = ss.prune24_act_tiled(dev_bf16(vt.reshape(H * d, L)), "bf16")
    O = ss.spgemm_tiled_batched(ss.SS_SPARSE_W, H, L, d, Kc, tv, tm, dev_bf16(pd), None, None, "bf16")
    got = bf16_to_f64(host(O))
    for h in range(H):
        vals, meta, _ = oracle.prune24_act(vt[h], "bf16")
        exp = oracle.spgemm("W", vals, meta, pd[h], Kc, "bf16", None, None, "bf16")
        assert rel_fro(got[h], bf16_to_f64(exp)) <= 1e-2
        assert_elementwise(got[h], bf16_to_f64(exp), sum_abs_terms(vals, meta, pd[h], Kc, "bf16"), out="bf16")
