"""Oracle for paged decode: plain fp64 CPU reference.

TEST INFRASTRUCTURE: imported only by tests/, the smoke entry point and the benchmark's
CPU-baseline leg. The HIP library and its binding never import it.
"""
from .paged_attention import (copy_blocks, decode, decode_partials, gather, max_abs_err,
                              num_partitions, prefill, reduce_partials, to_f64, v_from_rows,
                              v_group, v_to_rows, write_cache)

__all__ = ["copy_blocks", "decode", "decode_partials", "gather", "max_abs_err",
           "num_partitions", "prefill", "reduce_partials", "to_f64", "v_from_rows", "v_group",
           "v_to_rows", "write_cache"]
