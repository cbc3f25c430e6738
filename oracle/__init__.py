"""CPU oracle for the N:M structured-sparse, quantised linear layer.

TEST INFRASTRUCTURE ONLY. This package is a plain, slow, obviously correct
NumPy statement of what the sparse path computes, used to check the HIP
library. It shares no code with the HIP path and must never be used by it:
only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import it. Floating-point steps that the method fixes in float32 (scales,
products, rounding to int8/fp8/bf16) are done in float32 exactly as stated;
matrix products are done in float64, which is exact for the int8 and fp8
operands used here.

Sources (cited by page title and section throughout):

* "Deep reading of arXiv 2610.28947" (paper-daily.com, Chinese and English
  versions): 2:4 along the accumulate axis, bits accounting, energy removed.
* "SlideSparse: layout sparse boundary" (MSRA article on 66bd.net): the
  (2N-2):2N patterns, the sliding-window decomposition, activation lifting.
* SlideSparse blog (omica.com.cn): pattern table, flat window iteration.
* LLM Compressor "compression schemes" guide: per-channel weight scales,
  dynamic per-token activation scales, and the block-scaled FP8 scheme
  (128 x 128 weight blocks, per-token groups of 128).

Module map: ``prune`` (magnitude N:M masks, 2:4 compression, energy),
``slide`` (window decomposition, lift, K'), ``quant`` (per-row symmetric
INT8/FP8, the E4M3FN codec), ``gemm`` (sparse product and rescale epilogue),
``paths`` (the five library calls end to end), ``block`` (the block-scaled
FP8 prep and product), ``accounting`` (bits and closed forms).
"""
from .prune import (nm_keep_mask, prune_nm, compress24, decompress24, pack_meta, unpack_meta,
                    paired48_keep_mask, energy_removed)
from .slide import lifted_k, lifted_k_alloc, KALIGN, window_claims, slide_decompose_dense, lift
from .quant import (QMAX, quant_rows, e4m3_encode, e4m3_decode, e4m3_values, bf16_bits_to_f32,
                    f32_to_bf16_bits_rne)
from .gemm import spgemm_acc, epilogue, spgemm
from .paths import prune24, slide_decompose, quant_lift_act, prune24_act, dense_quant_rows
from .block import BLOCK, n_groups, quant_group_act, prune24_block, spgemm_block_f64, spgemm_block
from .accounting import bits_dense, bits_24, bits_slide, expansion, theoretical_speedup, density

__all__ = [n for n in dir() if not n.startswith("_")]
