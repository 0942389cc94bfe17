"""CPU oracle -- test infrastructure only (tests, smoke check, CPU baseline).

The product path never imports this package.
"""
from .archead_oracle import (  # noqa: F401
    FORMAT, FORMAT_VERSION, MAGIC, layout, persistent_bytes, pack, unpack,
    bf16_bits_to_f64, f16_to_f64, dequant_R, dequant_rows, dequant_groups,
    w_hat, logits, row_argmax, top2_gap, row_stats, row_topk,
    quant_int8_rows, quant_int8_groups, quant_sc4, core_residual, quantize,
    damped_covariance, metric_transform, rsvd, metric_objective, fit, logit_error,
    ALT_FORMAT, ALT_PERM8, alt_persistent_bytes, pack_alt, unpack_alt, w_hat_alt, logits_alt,
    quant_group_int4,
)
