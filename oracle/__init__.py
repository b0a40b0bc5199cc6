"""CPU float64 oracle for the Longformer band + global attention path.

TEST INFRASTRUCTURE: imported only by tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py.  The HIP library never uses it.
"""
from .longformer import (allowed_pairs, attention, encoder_layer, ffn_block, gelu,
                         global_partition, layer_projections, layernorm, mask_shift)

__all__ = ["allowed_pairs", "attention", "encoder_layer", "ffn_block", "gelu",
           "global_partition", "layer_projections", "layernorm", "mask_shift"]
