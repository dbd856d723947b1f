"""CPU oracle for the three-segment INT2 decode path (TEST INFRASTRUCTURE).

This package is a plain, slow reference written from the pages that describe
OSCAR.  It exists only to check the HIP library.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it.  The product path (``bit_rotated_kv_attn_amd``) never imports,
calls or falls back to it.

It imports nothing but NumPy and shares no code, header, table or constant
generator with the HIP path.

Precision: every floating-point step runs in float64 on exactly widened
inputs (bf16, fp16 and fp32 all convert to float64 without rounding).  There
is one exception.  Where a floating-point value decides an integer (the INT2
code, and the fp16 scale/zero that fix the code grid), the oracle takes that
decision in float32, the precision of the kernel it checks.  The rotated value
is the float64 dot product rounded once to float32.

Page sources, cited by title and section:

* [GIST] gist.science, "OSCAR: Offline Spectral Covariance-Aware Rotation for
  2-bit KV Cache Quantization", technical summary: section 2.2A (offline
  rotation R = U . H_Had . P_br and per-layer clip thresholds) and section
  2.2B (hybrid-precision paged layout; a kernel that unpacks, dequantises,
  inverse-rotates and attends over INT2 history).
* [ZAKER] myzaker.com article on OSCAR: the paragraphs on the serving pipeline
  (three-segment token pool of a BF16 sink of 64 tokens, INT2 history and a
  BF16 recent window of 256 tokens; the oldest recent token is rotated,
  clipped, quantised and packed into history; 4 two-bit values per byte;
  decode runs an INT2 part with unpack and scale/zero-point dequantisation and
  a BF16 part, merged by an online softmax).
* [CSDN] aicoding.csdn.net explainer, section 3.1 "core idea": at inference,
  rotate by R, clip, quantise to INT2 and store; at attention time, load the
  INT2 values, inverse-rotate and run ordinary attention.

Parity status of each function is given in its docstring.  Every public
function is pinned by ``tests/test_oracle_*.py``.
"""
from .quant import (PAGE, quantize_rows_grouped, UNIFORM, LLOYD_MAX, LM_LEVELS, LM_THRESHOLDS, LM_UNIT, code_levels, bf16_to_f64,
                    f16_bits_to_f64, rotate_round_f32, quantize_group, quantize_group_lloyd_max,
                    pack_codes_row, unpack_codes_row, k_byte_offsets, v_byte_offsets,
                    quantize_pack_ref, read_history_codes, page_block_bytes)
from .attention import (attn_plain, attn_partial, merge_partials, dequant_history,
                        decode_attn_ref, bf16_paged_attn_ref)

__all__ = [
    "PAGE", "quantize_rows_grouped", "UNIFORM", "LLOYD_MAX", "LM_LEVELS", "LM_THRESHOLDS", "LM_UNIT", "code_levels",
    "bf16_to_f64", "f16_bits_to_f64", "rotate_round_f32", "quantize_group", "quantize_group_lloyd_max",
    "pack_codes_row", "unpack_codes_row", "k_byte_offsets", "v_byte_offsets",
    "quantize_pack_ref", "read_history_codes", "page_block_bytes",
    "attn_plain", "attn_partial", "merge_partials", "dequant_history", "decode_attn_ref",
    "bf16_paged_attn_ref",
]
