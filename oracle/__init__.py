"""CPU oracle for the group-wise INT4/INT2 quantizer and weight-only matmul.

TEST INFRASTRUCTURE: imported only by tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py.  Shares no code with the HIP library."""
from .gq_oracle import *  # noqa: F401,F403
from .gq_oracle import (FLAG_NONFINITE, FLAG_SCALE_OVERFLOW, GROUP_SIZE, Layout, Packed,
                        compare_linear, dequant, dequant_as, f64_to_bf16_bits, fake_quant, linear, linear_dx, kv_cache_pack, kv_decode_attention, pack,
                        quantize_groups, quantize_pack, quantize_unclamped_example, unpack, qmax,
                        bf16_bits_to_f64, block_fields)
