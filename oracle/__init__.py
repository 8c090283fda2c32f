"""CPU oracle (test infrastructure only; see the header of ternary_ref)."""
from .ternary_ref import (BLOCK, GROUP, FMT_TRIT5, FMT_SLOT2, FMT_BIT1, TRIT5_GROUP_BYTES,
                          hadamard, rotate, rotate_transpose, pack, unpack,
                          pack_trit5, unpack_trit5, pack_slot2, unpack_slot2,
                          pack_bit1, unpack_bit1, pack_bit1_loop,
                          pack_trit5_loop, pack_slot2_loop, packed_bytes,
                          trit5_group_bytes, dequant, matvec, matvec_packed, linear,
                          fold_weights, quantize_ternary, quantize_weights, round_bf16,
                          rel_l2, fp16_ulp)

__all__ = ["BLOCK", "GROUP", "FMT_TRIT5", "FMT_SLOT2", "FMT_BIT1", "TRIT5_GROUP_BYTES",
           "hadamard", "rotate", "rotate_transpose", "pack", "unpack", "pack_trit5",
           "unpack_trit5", "pack_slot2", "unpack_slot2", "pack_bit1", "unpack_bit1",
           "pack_bit1_loop", "pack_trit5_loop", "pack_slot2_loop",
           "packed_bytes", "trit5_group_bytes", "dequant", "matvec", "matvec_packed",
           "linear", "fold_weights", "quantize_ternary", "quantize_weights", "round_bf16",
           "rel_l2", "fp16_ulp"]
