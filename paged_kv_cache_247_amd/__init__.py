"""PagedAttention decode for AMD Instinct MI355X (gfx950).

Hand-written HIP kernels behind the C ABI in include/pagedkv.h (libpagedkv.so), with a thin
ctypes binding. The seeded workload generators live in `workload`.
"""
from ._lib import (KERNELS, BlockManager, DeviceRegion, OutOfBlocks, PagedKVError, VmmPool,
                   auto_partition_size, copy_blocks, load, swap_blocks,
                   num_partitions, paged_attention, paged_attention_decode,
                   paged_attention_decode_grouped, paged_attention_decode_shared,
                   paged_attention_decode_static,
                   paged_attention_shared,
                   paged_attention_prefill, paged_attention_reduce, partition_workspace,
                   prefill_tile_tokens, probe_stream_read, probe_tile_gather,
                   reshape_and_cache, v_block_shape, v_cache_from_rows, v_cache_to_rows)

__all__ = ["KERNELS", "BlockManager", "DeviceRegion", "OutOfBlocks", "PagedKVError", "VmmPool",
           "auto_partition_size", "copy_blocks", "load", "swap_blocks",
           "num_partitions", "paged_attention", "paged_attention_decode",
           "paged_attention_decode_grouped", "paged_attention_decode_shared",
           "paged_attention_decode_static",
           "paged_attention_shared",
           "paged_attention_prefill", "paged_attention_reduce", "partition_workspace",
           "prefill_tile_tokens", "probe_stream_read", "probe_tile_gather",
           "reshape_and_cache", "v_block_shape", "v_cache_from_rows", "v_cache_to_rows"]
