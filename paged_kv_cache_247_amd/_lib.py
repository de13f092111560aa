"""ctypes binding of libpagedkv.so: argument marshalling only.

Every function here takes torch tensors that live on the GPU, checks their dtype, shape and
layout against the C header's contract, and passes raw device pointers, sizes and the current
HIP stream to the C ABI. All computation happens in the HIP kernels. A non-zero status raises
PagedKVError. If the library is not built, loading fails loudly: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

from . import contract as _contract

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libpagedkv.so")

PKV_F32, PKV_F16, PKV_BF16 = 0, 1, 2
KERNELS = {"auto": 0, "valu": 1, "mfma": 2}
_DTYPES = {torch.float32: PKV_F32, torch.float16: PKV_F16, torch.bfloat16: PKV_BF16}

PKV_DECODE_CACHED_KV = 1


class DecodeOptions(ctypes.Structure):
    """pkv_decode_options."""
    _fields_ = [("kernel", ctypes.c_int), ("flags", ctypes.c_uint32),
                ("new_key", ctypes.c_void_p), ("new_value", ctypes.c_void_p)]


# Exported symbols and their C prototypes (pagedkv.h).
_P, _I, _F, _Z = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
_OPT = ctypes.POINTER(DecodeOptions)
SIGNATURES = {
    "pkv_reshape_and_cache": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P]),
    "pkv_paged_attention_decode": (_I, [_P, _P, _P, _P, _P, _I, _P, _P, _I, _I, _I, _I, _I, _I,
                                        _I, _I, _F, _I, _I, _P, _P, _P, _P]),
    "pkv_paged_attention_decode_ex": (_I, [_OPT, _P, _P, _P, _P, _P, _I, _P, _P, _I, _I, _I,
                                           _I, _I, _I, _I, _I, _F, _I, _I, _P, _P, _P, _P]),
    "pkv_paged_attention_decode_shared": (_I, [_P, _P, _P, _P, _I, _P, _P, _I, _P, _I, _P, _P,
                                               _I, _I, _I, _I, _I, _I, _I, _F, _I, _I, _P, _P,
                                               _P, _P]),
    "pkv_paged_attention_decode_static": (_I, [_P, _P, _P, _P, _P, _I, _P, _P, _I, _I, _I, _I,
                                               _I, _I, _I, _I, _F, _I, _I, _P]),
    "pkv_paged_attention_decode_grouped": (_I, [_P, _P, _P, _P, _P, _I, _P, _P, _I, _I, _P, _P,
                                                _I, _I, _I, _I, _I, _I, _F, _I, _P]),
    "pkv_paged_attention_reduce": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P]),
    "pkv_copy_blocks": (_I, [_P, _P, _I, _P, _I, _I, _I, _I, _I, _I, _P]),
    "pkv_v_cache_from_rows": (_I, [_P, _P, _I, _I, _I, _I, _I, _P]),
    "pkv_v_cache_to_rows": (_I, [_P, _P, _I, _I, _I, _I, _I, _P]),
    "pkv_partition_workspace_bytes": (_Z, [_I, _I, _I, _I, _I]),
    "pkv_status_string": (ctypes.c_char_p, [_I]),
    "pkv_last_hip_error": (ctypes.c_int, []),
    "pkv_last_error_message": (ctypes.c_char_p, []),
    "pkv_abi_version": (ctypes.c_int, []),
    "pkv_paged_attention_prefill": (_I, [_P, _P, _P, _P, _P, _I, _P, _P, _I, _P, _I, _I, _I,
                                         _I, _I, _I, _I, _I, _F, _I, _P]),
    "pkv_prefill_tile_tokens": (_I, [_I, _I]),
    "pkv_bm_create": (_I, [_I, _I, _I, ctypes.POINTER(_P)]),
    "pkv_bm_destroy": (None, [_P]),
    "pkv_bm_free_blocks": (_I, [_P]),
    "pkv_bm_free_host_blocks": (_I, [_P]),
    "pkv_bm_add": (_I, [_P, ctypes.c_int64, _I]),
    "pkv_bm_fork": (_I, [_P, ctypes.c_int64, ctypes.c_int64]),
    "pkv_bm_append": (_I, [_P, ctypes.c_int64, ctypes.POINTER(ctypes.c_int64),
                           ctypes.POINTER(_I), ctypes.POINTER(_I)]),
    "pkv_bm_free": (_I, [_P, ctypes.c_int64]),
    "pkv_bm_num_tokens": (_I, [_P, ctypes.c_int64]),
    "pkv_bm_ref_count": (_I, [_P, _I]),
    "pkv_bm_tables": (_I, [_P, _P, _I, _I, _P, _P]),
    "pkv_bm_swap_out": (_I, [_P, ctypes.c_int64, _P, _I, ctypes.POINTER(_I)]),
    "pkv_bm_swap_in": (_I, [_P, ctypes.c_int64, _P, _I, ctypes.POINTER(_I)]),
    "pkv_swap_blocks": (_I, [_P, _P, _I, _P, _P, _I, _P, _I, _Z, _I, _P]),
    "pkv_vmm_pool_create": (_I, [_I, _I, _I, _I, _I, _I, _Z, ctypes.POINTER(_P)]),
    "pkv_vmm_pool_map": (_I, [_P, _I, _I]),
    "pkv_vmm_pool_unmap": (_I, [_P, _I]),
    "pkv_vmm_pool_copy": (_I, [_P, _I, _I, _P, _P, _I, _P]),
    "pkv_vmm_pool_destroy": (None, [_P]),
    "pkv_vmm_pool_k": (_P, [_P]),
    "pkv_vmm_pool_v": (_P, [_P]),
    "pkv_vmm_pool_blocks_per_seq": (_I, [_P]),
    "pkv_vmm_pool_page_bytes": (_Z, [_P]),
    "pkv_vmm_pool_mapped_bytes": (_Z, [_P]),
    "pkv_probe_stream_read": (_I, [_P, _Z, _I, _I, _P, _P]),
    "pkv_probe_tile_gather": (_I, [_P, _Z, _P, _I, _I, _I, _I, _P, _P]),
}


class PagedKVError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"status {status}: {message}")
        self.status = status
        self.message = message


def validating() -> bool:
    """PKV_VALIDATE=1: check the contents of tables, lengths, slots and copy pairs on the host
    before each call (a device-to-host copy per call; for debugging)."""
    return os.environ.get("PKV_VALIDATE", "0") not in ("", "0")


def _host(t):
    return None if t is None else t.detach().cpu().numpy()


def _contract_check(fn, *args, **kw):
    try:
        fn(*args, **kw)
    except _contract.ContractError as e:
        raise PagedKVError(1, f"caller contract: {e}") from None


_lib = None


def load(path: str | None = None) -> ctypes.CDLL:
    """Load the built library (once); raises if it is missing."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is not built: run `python -m paged_kv_cache_247_amd.build`")
    lib = ctypes.CDLL(p)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if lib.pkv_abi_version() != ABI_VERSION:
        raise RuntimeError(f"{p} implements ABI {lib.pkv_abi_version()}, this binding ABI "
                           f"{ABI_VERSION}: rebuild it (`python -m paged_kv_cache_247_amd.build`)")
    if path is None:
        _lib = lib
    return lib


class OutOfBlocks(PagedKVError):
    """PKV_ERR_NO_BLOCKS: the block manager has too few free blocks (nothing was changed)."""


PKV_ERR_HIP = 3
PKV_ERR_NO_BLOCKS = 4
ABI_VERSION = 6  # the argument lists in SIGNATURES
STATIC_WORKSPACE_BYTES = 80 << 20  # PKV_STATIC_WORKSPACE_BYTES


def _check(status: int):
    if status != 0:
        lib = load()
        cls = OutOfBlocks if status == PKV_ERR_NO_BLOCKS else PagedKVError
        raise cls(status, lib.pkv_last_error_message().decode())
    if os.environ.get("PKV_SYNC", "0") not in ("", "0") and torch.cuda.is_available():
        # Debugging: wait for the call's work so an asynchronous error is reported here, by
        # the call that caused it, rather than at some later synchronization.
        try:
            torch.cuda.synchronize()
        except RuntimeError as e:
            raise PagedKVError(PKV_ERR_HIP, f"after the call: {e}") from None


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t: torch.Tensor | None):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


class DeviceRegion:
    """A raw device buffer that the binding accepts wherever it takes a KV pool: a pointer, a
    shape, a dtype and a device, with no torch storage behind it. The virtual-memory pool hands
    these out because no torch operation may touch its unmapped parts."""
    is_cuda = True

    def __init__(self, ptr: int, shape, dtype: torch.dtype, device: torch.device):
        self._ptr = int(ptr)
        self.shape = tuple(int(x) for x in shape)
        self.dtype = dtype
        self.device = device

    def data_ptr(self) -> int:
        return self._ptr

    def dim(self) -> int:
        return len(self.shape)

    def is_contiguous(self) -> bool:
        return True


def _need(t: torch.Tensor, name: str, dtype=None, ndim=None, device=None):
    if not isinstance(t, (torch.Tensor, DeviceRegion)):
        raise TypeError(f"{name} must be a tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _dt(t: torch.Tensor) -> int:
    try:
        return _DTYPES[t.dtype]
    except KeyError:
        raise TypeError(f"unsupported dtype {t.dtype}") from None


def v_block_shape(num_kv_heads: int, head_dim: int, block_size: int) -> tuple:
    """Shape of one V block: column groups of VS = min(S, 32) positions, each a [D, VS] tile,
    stacked as [Hkv, (S / VS) D, VS] (for S <= 32 that is [Hkv, D, S])."""
    vs = min(block_size, 32)
    return (num_kv_heads, block_size // vs * head_dim, vs)


def reshape_and_cache(key, value, k_cache, v_cache, slot_mapping):
    """Write new K/V rows [T, Hkv, D] into their slots of the pools (pkv_reshape_and_cache)."""
    _need(k_cache, "k_cache", ndim=4)
    dt = k_cache.dtype
    N, Hkv, S, D = k_cache.shape
    _need(v_cache, "v_cache", dt, 4, k_cache.device)
    if tuple(v_cache.shape) != (N, *v_block_shape(Hkv, D, S)):
        raise ValueError(f"v_cache must be {(N, *v_block_shape(Hkv, D, S))}")
    _need(key, "key", dt, 3, k_cache.device)
    _need(value, "value", dt, 3, k_cache.device)
    T = key.shape[0]
    if tuple(key.shape) != (T, Hkv, D) or tuple(value.shape) != (T, Hkv, D):
        raise ValueError("key/value must be [T, Hkv, D]")
    _need(slot_mapping, "slot_mapping", torch.int64, 1, k_cache.device)
    if slot_mapping.shape[0] != T:
        raise ValueError("slot_mapping must have one slot per token")
    if validating():
        _contract_check(_contract.check_slots, _host(slot_mapping), S, N)
    _check(load().pkv_reshape_and_cache(_ptr(key), _ptr(value), _ptr(k_cache), _ptr(v_cache),
                                        _ptr(slot_mapping), T, Hkv, D, S, N, _dt(k_cache),
                                        _stream(k_cache)))


def num_partitions(max_context_len: int, partition_size: int) -> int:
    return -(-int(max_context_len) // int(partition_size)) if partition_size > 0 else 0


def partition_workspace(num_seqs, num_heads, head_dim, max_context_len, partition_size,
                        device):
    """fp32 (max_logits [B,H,NP], exp_sums [B,H,NP], tmp_out [B,H,NP,D]) carved from one buffer
    of pkv_partition_workspace_bytes bytes."""
    NP = num_partitions(max_context_len, partition_size)
    nbytes = load().pkv_partition_workspace_bytes(num_seqs, num_heads, head_dim,
                                                  max_context_len, partition_size)
    n = num_seqs * num_heads * NP
    assert nbytes == 4 * n * (head_dim + 2)
    buf = torch.empty(max(nbytes // 4, 1), dtype=torch.float32, device=device)
    # tmp_out first keeps it 16-byte aligned whatever n is.
    tmp_out = buf[:n * head_dim].view(num_seqs, num_heads, NP, head_dim)
    max_logits = buf[n * head_dim:n * (head_dim + 1)].view(num_seqs, num_heads, NP)
    exp_sums = buf[n * (head_dim + 1):n * (head_dim + 2)].view(num_seqs, num_heads, NP)
    return max_logits, exp_sums, tmp_out


def paged_attention_decode(out, q, k_cache, v_cache, block_tables, context_lens,
                           max_context_len, scale, partition_size=0, workspace=None,
                           kernel="auto", work_items=None, cached_kv=False, new_key=None,
                           new_value=None, max_blocks_per_seq=None):
    """pkv_paged_attention_decode_ex. Single pass writes `out`; with partition_size > 0 it
    writes only `workspace` = (max_logits, exp_sums, tmp_out). work_items: optional device int32
    list of units i * NP + p in dispatch order (largest first shortens the tail; see
    workload.Workload.work_items). cached_kv: ordinary
    cached K/V loads (for block tables that share blocks). new_key/new_value: optional
    [B, Hkv, D] newest-token rows, written to the cache and attended to in the same launch.
    block_tables=None selects the contiguous reservation (sequence i owns pool blocks
    i * max_blocks_per_seq onwards; max_blocks_per_seq is then required)."""
    _need(q, "q", ndim=3)
    dt = q.dtype
    B, H, D = q.shape
    _need(k_cache, "k_cache", dt, 4, q.device)
    N, Hkv, S, Dk = k_cache.shape
    if Dk != D:
        raise ValueError("head_dim of q and k_cache differ")
    _need(v_cache, "v_cache", dt, 4, q.device)
    if tuple(v_cache.shape) != (N, *v_block_shape(Hkv, D, S)):
        raise ValueError(f"v_cache must be {(N, *v_block_shape(Hkv, D, S))}")
    _need(context_lens, "context_lens", torch.int32, 1, q.device)
    if block_tables is None:  # contiguous reservation: max_blocks_per_seq blocks per sequence
        if max_blocks_per_seq is None:
            raise ValueError("max_blocks_per_seq is required without block tables")
        MB = int(max_blocks_per_seq)
    else:
        _need(block_tables, "block_tables", torch.int32, 2, q.device)
        MB = block_tables.shape[1]
        if block_tables.shape[0] != B:
            raise ValueError("block_tables must have one row per sequence")
    if context_lens.shape[0] != B:
        raise ValueError("context_lens must have one entry per sequence")
    if work_items is not None:
        _need(work_items, "work_items", torch.int32, 1, q.device)
    if (new_key is None) != (new_value is None):
        raise ValueError("new_key and new_value go together")
    if new_key is not None:
        for t, nm in ((new_key, "new_key"), (new_value, "new_value")):
            _need(t, nm, dt, 3, q.device)
            if tuple(t.shape) != (B, Hkv, D):
                raise ValueError(f"{nm} must be [B, Hkv, D]")
    ml = es = to = None
    if partition_size:
        if workspace is None:
            raise ValueError("split-context mode needs a workspace")
        ml, es, to = workspace
        NP = num_partitions(max_context_len, partition_size)
        for t, shp in ((ml, (B, H, NP)), (es, (B, H, NP)), (to, (B, H, NP, D))):
            _need(t, "workspace", torch.float32, len(shp), q.device)
            if tuple(t.shape) != shp:
                raise ValueError(f"workspace part must be {shp}, got {tuple(t.shape)}")
    else:
        _need(out, "out", dt, 3, q.device)
        if tuple(out.shape) != (B, H, D):
            raise ValueError("out must be [B, H, D]")
    if validating():
        _contract_check(_contract.check_decode, _host(block_tables), _host(context_lens),
                        int(max_context_len), S, N, MB, int(partition_size), _host(work_items),
                        new_key is not None)
    lib = load()
    opts = DecodeOptions(KERNELS[kernel], PKV_DECODE_CACHED_KV if cached_kv else 0,
                         None if new_key is None else new_key.data_ptr(),
                         None if new_value is None else new_value.data_ptr())
    _check(lib.pkv_paged_attention_decode_ex(
        ctypes.byref(opts), _ptr(out) if not partition_size else None, _ptr(q), _ptr(k_cache),
        _ptr(v_cache), _ptr(block_tables), MB, _ptr(context_lens), _ptr(work_items),
        0 if work_items is None else work_items.shape[0], int(max_context_len), B, H,
        Hkv, D, S, N, float(scale), _dt(q), int(partition_size), _ptr(ml), _ptr(es), _ptr(to),
        _stream(q)))


def paged_attention_decode_grouped(out, q, k_cache, v_cache, block_tables, context_lens, groups,
                                   shared_len, scale, new_key=None, new_value=None):
    """pkv_paged_attention_decode_grouped: every member of each group (groups: device int32
    [num_groups, 4], -1 pads) decoded in one pass per group -- the first shared_len positions,
    which the members' tables share, read once for all of them -- into `out` [B, H, D]; with
    new_key/new_value [B, Hkv, D] also each member's newest-position cache write."""
    _need(q, "q", ndim=3)
    dt = q.dtype
    B, H, D = q.shape
    _need(out, "out", dt, 3, q.device)
    if tuple(out.shape) != (B, H, D):
        raise ValueError("out must be [B, H, D]")
    _need(k_cache, "k_cache", dt, 4, q.device)
    N, Hkv, S, Dk = k_cache.shape
    if Dk != D:
        raise ValueError("head_dim of q and k_cache differ")
    _need(v_cache, "v_cache", dt, 4, q.device)
    if tuple(v_cache.shape) != (N, *v_block_shape(Hkv, D, S)):
        raise ValueError(f"v_cache must be {(N, *v_block_shape(Hkv, D, S))}")
    _need(block_tables, "block_tables", torch.int32, 2, q.device)
    _need(context_lens, "context_lens", torch.int32, 1, q.device)
    _need(groups, "groups", torch.int32, 2, q.device)
    if groups.shape[1] != 4 or block_tables.shape[0] != B or context_lens.shape[0] != B:
        raise ValueError("groups must be [num_groups, 4]; tables and lengths one row per sequence")
    if (new_key is None) != (new_value is None):
        raise ValueError("new_key and new_value go together")
    if new_key is not None:
        for t, nm in ((new_key, "new_key"), (new_value, "new_value")):
            _need(t, nm, dt, 3, q.device)
            if tuple(t.shape) != (B, Hkv, D):
                raise ValueError(f"{nm} must be {(B, Hkv, D)}")
    MB = block_tables.shape[1]
    if validating():
        _contract_check(_contract.check_whole_groups, _host(groups), _host(block_tables),
                        _host(context_lens), int(shared_len), S, N, H // Hkv,
                        fused_write=new_key is not None)
    _check(load().pkv_paged_attention_decode_grouped(
        _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), MB,
        _ptr(context_lens), _ptr(groups), groups.shape[0], int(shared_len), _ptr(new_key),
        _ptr(new_value), B, H, Hkv, D, S, N, float(scale), _dt(q), _stream(q)))


def paged_attention_decode_static(out, q, k_cache, v_cache, block_tables, context_lens,
                                  max_context_len, scale, partition_size, work_items=None):
    """pkv_paged_attention_decode_static: split-context decode and the merge into `out`, with
    the partition workspace in the library's static device array (nothing is allocated)."""
    _need(q, "q", ndim=3)
    dt = q.dtype
    B, H, D = q.shape
    _need(out, "out", dt, 3, q.device)
    if tuple(out.shape) != (B, H, D):
        raise ValueError("out must be [B, H, D]")
    _need(k_cache, "k_cache", dt, 4, q.device)
    N, Hkv, S, Dk = k_cache.shape
    if Dk != D:
        raise ValueError("head_dim of q and k_cache differ")
    _need(v_cache, "v_cache", dt, 4, q.device)
    if tuple(v_cache.shape) != (N, *v_block_shape(Hkv, D, S)):
        raise ValueError(f"v_cache must be {(N, *v_block_shape(Hkv, D, S))}")
    _need(block_tables, "block_tables", torch.int32, 2, q.device)
    _need(context_lens, "context_lens", torch.int32, 1, q.device)
    if block_tables.shape[0] != B or context_lens.shape[0] != B:
        raise ValueError("block_tables and context_lens need one row per sequence")
    if work_items is not None:
        _need(work_items, "work_items", torch.int32, 1, q.device)
    MB = block_tables.shape[1]
    if validating():
        _contract_check(_contract.check_decode, _host(block_tables), _host(context_lens),
                        int(max_context_len), S, N, MB, int(partition_size), _host(work_items),
                        False)
    _check(load().pkv_paged_attention_decode_static(
        _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), MB,
        _ptr(context_lens), _ptr(work_items), 0 if work_items is None else work_items.shape[0],
        int(max_context_len), B, H, Hkv, D, S, N, float(scale), _dt(q), int(partition_size),
        _stream(q)))


def paged_attention_decode_shared(q, k_cache, v_cache, block_tables, context_lens, groups,
                                  max_context_len, scale, partition_size, workspace,
                                  work_items=None, new_key=None, new_value=None):
    """pkv_paged_attention_decode_shared: partition 0 of every member of each group of
    sequences sharing its blocks (groups: device int32 [num_groups, 4], -1 pads), into
    `workspace` = (max_logits, exp_sums, tmp_out) as split-context decode would write it; in
    the same launch the units of `work_items` (device int32, units i * NP + p), with the fused
    newest-position write when new_key/new_value [B, Hkv, D] are given, as
    paged_attention_decode(..., work_items=work_items, cached_kv=True) would run them."""
    _need(q, "q", ndim=3)
    dt = q.dtype
    B, H, D = q.shape
    _need(k_cache, "k_cache", dt, 4, q.device)
    N, Hkv, S, Dk = k_cache.shape
    if Dk != D:
        raise ValueError("head_dim of q and k_cache differ")
    _need(v_cache, "v_cache", dt, 4, q.device)
    if tuple(v_cache.shape) != (N, *v_block_shape(Hkv, D, S)):
        raise ValueError(f"v_cache must be {(N, *v_block_shape(Hkv, D, S))}")
    _need(block_tables, "block_tables", torch.int32, 2, q.device)
    MB = block_tables.shape[1]
    _need(context_lens, "context_lens", torch.int32, 1, q.device)
    _need(groups, "groups", torch.int32, 2, q.device)
    if groups.shape[1] != 4 or block_tables.shape[0] != B or context_lens.shape[0] != B:
        raise ValueError("groups must be [num_groups, 4]; tables and lengths one row per sequence")
    ml, es, to = workspace
    NP = num_partitions(max_context_len, partition_size)
    for t, shp in ((ml, (B, H, NP)), (es, (B, H, NP)), (to, (B, H, NP, D))):
        _need(t, "workspace", torch.float32, len(shp), q.device)
        if tuple(t.shape) != shp:
            raise ValueError(f"workspace part must be {shp}, got {tuple(t.shape)}")
    if work_items is not None:
        _need(work_items, "work_items", torch.int32, 1, q.device)
    if (new_key is None) != (new_value is None):
        raise ValueError("new_key and new_value go together")
    if new_key is not None:
        if work_items is None:
            raise ValueError("new rows are written by the listed units: give work_items")
        for t, nm in ((new_key, "new_key"), (new_value, "new_value")):
            _need(t, nm, dt, 3, q.device)
            if tuple(t.shape) != (B, Hkv, D):
                raise ValueError(f"{nm} must be {(B, Hkv, D)}")
    if validating():
        listed = None if work_items is None else _host(work_items)
        if listed is not None:
            _contract_check(_contract.check_decode, _host(block_tables), _host(context_lens),
                            int(max_context_len), S, N, MB, int(partition_size), listed,
                            new_key is not None)
        _contract_check(_contract.check_groups, _host(groups), _host(block_tables),
                        _host(context_lens), int(partition_size), S, N, H // Hkv,
                        work_items=listed, num_partitions=NP, fused_write=new_key is not None)
    nw = 0 if work_items is None else work_items.shape[0]
    _check(load().pkv_paged_attention_decode_shared(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), MB, _ptr(context_lens),
        _ptr(groups), groups.shape[0], _ptr(work_items), nw, _ptr(new_key), _ptr(new_value),
        int(max_context_len), B, H, Hkv, D, S, N, float(scale), _dt(q), int(partition_size),
        _ptr(ml), _ptr(es), _ptr(to), _stream(q)))


def prefill_tile_tokens(num_heads: int, num_kv_heads: int) -> int:
    """Query tokens per prefill work unit (pkv_prefill_tile_tokens)."""
    return load().pkv_prefill_tile_tokens(num_heads, num_kv_heads)


def paged_attention_prefill(out, q, k_cache, v_cache, block_tables, context_lens, query_start,
                            max_query_len, scale, work_items=None):
    """pkv_paged_attention_prefill: causal attention of each sequence's new tokens (rows
    query_start[i] .. query_start[i + 1] - 1 of q [T, H, D], at the last Q_i positions of the
    sequence, already in the cache) over its paged cache; writes out [T, H, D]. work_items:
    optional device int32 list of units i * NT + t (tile t of prefill_tile_tokens tokens)."""
    _need(q, "q", ndim=3)
    dt = q.dtype
    T, H, D = q.shape
    _need(out, "out", dt, 3, q.device)
    if tuple(out.shape) != (T, H, D):
        raise ValueError("out must be shaped like q")
    _need(k_cache, "k_cache", dt, 4, q.device)
    N, Hkv, S, Dk = k_cache.shape
    if Dk != D:
        raise ValueError("head_dim of q and k_cache differ")
    _need(v_cache, "v_cache", dt, 4, q.device)
    if tuple(v_cache.shape) != (N, *v_block_shape(Hkv, D, S)):
        raise ValueError(f"v_cache must be {(N, *v_block_shape(Hkv, D, S))}")
    _need(block_tables, "block_tables", torch.int32, 2, q.device)
    B, MB = block_tables.shape
    _need(context_lens, "context_lens", torch.int32, 1, q.device)
    _need(query_start, "query_start", torch.int32, 1, q.device)
    if context_lens.shape[0] != B or query_start.shape[0] != B + 1:
        raise ValueError("context_lens [B] and query_start [B + 1] must match the tables")
    if work_items is not None:
        _need(work_items, "work_items", torch.int32, 1, q.device)
    if validating():
        _contract_check(_contract.check_prefill, _host(block_tables), _host(context_lens),
                        _host(query_start), int(max_query_len), S, N, T)
    _check(load().pkv_paged_attention_prefill(
        _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), MB,
        _ptr(context_lens), _ptr(query_start), int(max_query_len), _ptr(work_items),
        0 if work_items is None else work_items.shape[0], B, T, H, Hkv, D, S, N, float(scale),
        _dt(q), _stream(q)))


def paged_attention_reduce(out, workspace, context_lens, partition_size):
    """pkv_paged_attention_reduce: merge the partitions in `workspace` into `out`."""
    ml, es, to = workspace
    _need(out, "out", ndim=3)
    B, H, D = out.shape
    NP = ml.shape[2]
    for t, shp in ((ml, (B, H, NP)), (es, (B, H, NP)), (to, (B, H, NP, D))):
        _need(t, "workspace", torch.float32, len(shp), out.device)
        if tuple(t.shape) != shp:
            raise ValueError(f"workspace part must be {shp}")
    _need(context_lens, "context_lens", torch.int32, 1, out.device)
    _check(load().pkv_paged_attention_reduce(_ptr(out), _ptr(ml), _ptr(es), _ptr(to),
                                             _ptr(context_lens), B, H, D, int(partition_size),
                                             NP, _dt(out), _stream(out)))


def copy_blocks(k_caches, v_caches, block_mapping):
    """pkv_copy_blocks over every layer: block dst := block src for each (src, dst) row."""
    if len(k_caches) != len(v_caches) or not k_caches:
        raise ValueError("need matching non-empty lists of K and V pools")
    k0 = k_caches[0]
    _need(k0, "k_caches[0]", ndim=4)
    N, Hkv, S, D = k0.shape
    for k, v in zip(k_caches, v_caches):
        _need(k, "k_cache", k0.dtype, 4, k0.device)
        _need(v, "v_cache", k0.dtype, 4, k0.device)
        if tuple(k.shape) != (N, Hkv, S, D) or tuple(v.shape) != (N, *v_block_shape(Hkv, D, S)):
            raise ValueError("every layer's pools must have the same shape")
    _need(block_mapping, "block_mapping", torch.int64, 2, k0.device)
    if block_mapping.shape[1] != 2:
        raise ValueError("block_mapping must be [M, 2]")
    if validating():
        _contract_check(_contract.check_copy_pairs, _host(block_mapping), N)
    nl = len(k_caches)
    karr = (ctypes.c_void_p * nl)(*[k.data_ptr() for k in k_caches])
    varr = (ctypes.c_void_p * nl)(*[v.data_ptr() for v in v_caches])
    _check(load().pkv_copy_blocks(karr, varr, nl, _ptr(block_mapping), block_mapping.shape[0],
                                  Hkv, D, S, N, _dt(k0), _stream(k0)))


def _v_layout(name, src, dst, rows_src):
    rows, cols = (src, dst) if rows_src else (dst, src)
    _need(rows, "v_rows", ndim=4)
    N, Hkv, S, D = rows.shape
    _need(cols, "v_cache", rows.dtype, 4, rows.device)
    if tuple(cols.shape) != (N, *v_block_shape(Hkv, D, S)):
        raise ValueError(f"v_cache must be {(N, *v_block_shape(Hkv, D, S))} for v_rows "
                         f"{tuple(rows.shape)}, got {tuple(cols.shape)}")
    _check(getattr(load(), name)(_ptr(src), _ptr(dst), N, Hkv, D, S, _dt(rows), _stream(rows)))


def v_cache_from_rows(v_rows, v_cache):
    """pkv_v_cache_from_rows: fill the column-group V pool [N, Hkv, (S/VS) D, VS] from a pool of
    token rows [N, Hkv, S, D]. v_cache may view the same memory as v_rows (in place)."""
    _v_layout("pkv_v_cache_from_rows", v_rows, v_cache, True)


def v_cache_to_rows(v_cache, v_rows):
    """pkv_v_cache_to_rows: the inverse of v_cache_from_rows (in place allowed as well)."""
    _v_layout("pkv_v_cache_to_rows", v_cache, v_rows, False)


AUTO_PARTITION_TOKENS = 2048       # matrix-core decode (16-bit, query groups of 4 or more)
AUTO_PARTITION_TOKENS_VALU = 768   # vector-ALU decode (fp32, or groups of 1-2)


def auto_partition_size(num_seqs: int, num_kv_heads: int, block_size: int,
                        device=None, num_cus: int | None = None, group: int = 4,
                        dtype: str = "bf16") -> int:
    """Host policy for split-context decode: single pass (0) when the single-pass grid fills two
    rounds of the GPU's workgroup slots, else partitions, so that a few long sequences do not
    leave most CUs idle behind them and the last round stays even. The kernel family is the one
    the library picks for `group` (query heads per kv head) and `dtype`:
    * matrix cores (16-bit, group >= 4): a workgroup per (sequence, kv head), two per CU; else
      2048-token partitions. Measured on the GQA shape at equal total tokens: 128 sequences
      single pass 188 us; 64 sequences 195.5 -> 190.3 us and 32 sequences 218.7 -> 187.3 us with
      2048-token partitions (merge included).
    * vector ALUs (fp32, or group < 4): a workgroup per (sequence, two kv heads when their count
      is even), three per CU; else 768-token partitions. Measured on the MHA batch (64
      sequences, 32 heads, contexts up to 2048: 1.33 rounds): step 185.9 us single pass, 183.4
      us in 768-token partitions with the merge (512: 184.4, 1024: 186.0)."""
    if num_cus is None:
        num_cus = torch.cuda.get_device_properties(device if device is not None else
                                                   torch.cuda.current_device()).multi_processor_count
    mfma = dtype != "f32" and group >= 4
    if mfma:
        workgroups, per_cu, tokens = num_seqs * num_kv_heads, 2, AUTO_PARTITION_TOKENS
    else:
        hpw = 2 if num_kv_heads % 2 == 0 else 1
        workgroups, per_cu, tokens = num_seqs * (num_kv_heads // hpw), 3, AUTO_PARTITION_TOKENS_VALU
    if workgroups >= 2 * per_cu * num_cus:
        return 0
    return max(block_size, tokens // block_size * block_size)


def paged_attention(out, q, k_cache, v_cache, block_tables, context_lens, max_context_len,
                    scale, partition_size=0, workspace=None, kernel="auto", work_items=None,
                    cached_kv=False, new_key=None, new_value=None, max_blocks_per_seq=None):
    """The whole decode: single pass, or partitions then their merge, on the current stream.
    partition_size="auto" applies auto_partition_size (a work list, if given, must have been
    built for the size it picks)."""
    if partition_size == "auto":
        partition_size = auto_partition_size(
            q.shape[0], k_cache.shape[1], k_cache.shape[2], q.device,
            group=q.shape[1] // k_cache.shape[1],
            dtype={torch.float32: "f32", torch.float16: "f16"}.get(q.dtype, "bf16"))
    kw = dict(kernel=kernel, work_items=work_items, cached_kv=cached_kv, new_key=new_key,
              new_value=new_value, max_blocks_per_seq=max_blocks_per_seq)
    if partition_size:
        B, H, D = q.shape
        if workspace is None:
            workspace = partition_workspace(B, H, D, max_context_len, partition_size, q.device)
        paged_attention_decode(None, q, k_cache, v_cache, block_tables, context_lens,
                               max_context_len, scale, partition_size, workspace, **kw)
        paged_attention_reduce(out, workspace, context_lens, partition_size)
    else:
        paged_attention_decode(out, q, k_cache, v_cache, block_tables, context_lens,
                               max_context_len, scale, 0, None, **kw)
    return out


def paged_attention_shared(out, q, k_cache, v_cache, block_tables, context_lens,
                           max_context_len, scale, groups, work_items, partition_size,
                           workspace=None, new_key=None, new_value=None):
    """A decode step over shared prefix blocks (see sharing.plan, which gives groups,
    work_items and partition_size): one launch runs partition 0 of the grouped sequences in
    one pass per group beside every other unit of split-context decode (with the fused
    newest-token write, if rows are given), then the merge; on the current stream."""
    B, H, D = q.shape
    if workspace is None:
        workspace = partition_workspace(B, H, D, max_context_len, partition_size, q.device)
    paged_attention_decode_shared(q, k_cache, v_cache, block_tables, context_lens, groups,
                                  max_context_len, scale, partition_size, workspace,
                                  work_items=work_items, new_key=new_key, new_value=new_value)
    paged_attention_reduce(out, workspace, context_lens, partition_size)
    return out


class VmmPool:
    """pkv_vmm_pool_*: K and V regions kept virtually contiguous per sequence (the contiguous
    layout that decode reads without block tables) and backed by physical pages on demand.
    `k` and `v` are DeviceRegions over the whole reservation; map a sequence's positions before
    any GPU work touches them. Decode on the pool: paged_attention_decode(..., pool.k, pool.v,
    None, ..., max_blocks_per_seq=pool.blocks_per_seq)."""

    def __init__(self, num_seqs: int, max_context_len: int, num_kv_heads: int, head_dim: int,
                 block_size: int, dtype: torch.dtype, page_bytes: int = 0):
        lib = load()
        h = ctypes.c_void_p()
        _check(lib.pkv_vmm_pool_create(num_seqs, max_context_len, num_kv_heads, head_dim,
                                       block_size, _DTYPES[dtype], page_bytes, ctypes.byref(h)))
        self._h = h
        self.num_seqs = num_seqs
        self.blocks_per_seq = lib.pkv_vmm_pool_blocks_per_seq(h)
        self.page_bytes = lib.pkv_vmm_pool_page_bytes(h)
        self.block_shape = (num_kv_heads, block_size, head_dim)
        dev = torch.device("cuda", torch.cuda.current_device())
        N = num_seqs * self.blocks_per_seq
        self.k = DeviceRegion(lib.pkv_vmm_pool_k(h), (N, num_kv_heads, block_size, head_dim),
                              dtype, dev)
        self.v = DeviceRegion(lib.pkv_vmm_pool_v(h),
                              (N, *v_block_shape(num_kv_heads, head_dim, block_size)), dtype, dev)

    @property
    def mapped_bytes(self) -> int:
        return load().pkv_vmm_pool_mapped_bytes(self._h)

    def map(self, seq: int, num_positions: int):
        _check(load().pkv_vmm_pool_map(self._h, seq, num_positions))

    def unmap(self, seq: int):
        _check(load().pkv_vmm_pool_unmap(self._h, seq))

    def write(self, seq: int, k_blocks: torch.Tensor, v_blocks: torch.Tensor):
        """Copy blocks [0, n) of sequence seq in from device tensors [n, Hkv, S, D] and
        [n, *v_block_shape] (on the current stream)."""
        self._copy(seq, k_blocks, v_blocks, 1)

    def read(self, seq: int, num_blocks: int):
        """Blocks [0, num_blocks) of sequence seq, copied out into new tensors."""
        Hkv, S, D = self.block_shape
        k = torch.empty((num_blocks, Hkv, S, D), dtype=self.k.dtype, device=self.k.device)
        v = torch.empty((num_blocks, *v_block_shape(Hkv, D, S)), dtype=self.k.dtype,
                        device=self.k.device)
        self._copy(seq, k, v, 0)
        return k, v

    def _copy(self, seq, k, v, to_pool):
        Hkv, S, D = self.block_shape
        n = k.shape[0]
        _need(k, "k", self.k.dtype, 4, self.k.device)
        _need(v, "v", self.k.dtype, 4, self.k.device)
        if tuple(k.shape) != (n, Hkv, S, D) or tuple(v.shape) != (n, *v_block_shape(Hkv, D, S)):
            raise ValueError("blocks must be [n, Hkv, S, D] and [n, *v_block_shape]")
        _check(load().pkv_vmm_pool_copy(self._h, seq, n, _ptr(k), _ptr(v), to_pool, _stream(k)))

    def close(self):
        if self._h:
            torch.cuda.synchronize()
            load().pkv_vmm_pool_destroy(self._h)
            self._h = None

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()


class BlockManager:
    """pkv_bm_*: reference-counted physical blocks of a device pool and a host pool, per-sequence
    block lists, fork (sharing), copy-on-write on append, swap out/in. Host bookkeeping only:
    the copies it asks for are the caller's (copy_blocks, swap_blocks)."""

    def __init__(self, num_blocks: int, num_host_blocks: int, block_size: int):
        h = ctypes.c_void_p()
        _check(load().pkv_bm_create(num_blocks, num_host_blocks, block_size, ctypes.byref(h)))
        self._h = h
        self.num_blocks, self.num_host_blocks, self.block_size = num_blocks, num_host_blocks, block_size

    def __del__(self):
        if getattr(self, "_h", None):
            load().pkv_bm_destroy(self._h)
            self._h = None

    @property
    def free_blocks(self) -> int:
        return load().pkv_bm_free_blocks(self._h)

    @property
    def free_host_blocks(self) -> int:
        return load().pkv_bm_free_host_blocks(self._h)

    def add(self, seq: int, num_tokens: int):
        _check(load().pkv_bm_add(self._h, seq, num_tokens))

    def fork(self, parent: int, child: int):
        _check(load().pkv_bm_fork(self._h, parent, child))

    def append(self, seq: int):
        """Slot of seq's next token, and the (src, dst) block copy it needs first (or None)."""
        slot, src, dst = ctypes.c_int64(), ctypes.c_int32(), ctypes.c_int32()
        _check(load().pkv_bm_append(self._h, seq, ctypes.byref(slot), ctypes.byref(src),
                                    ctypes.byref(dst)))
        return slot.value, (None if src.value < 0 else (src.value, dst.value))

    def free(self, seq: int):
        _check(load().pkv_bm_free(self._h, seq))

    def num_tokens(self, seq: int) -> int:
        return load().pkv_bm_num_tokens(self._h, seq)

    def ref_count(self, block: int) -> int:
        return load().pkv_bm_ref_count(self._h, block)

    def tables(self, seqs, max_blocks: int):
        """(int32 [n, max_blocks] block tables, int32 [n] token counts) of the sequences."""
        import numpy as np
        ids = np.ascontiguousarray(seqs, dtype=np.int64)
        t = np.empty((len(ids), max_blocks), dtype=np.int32)
        lens = np.empty(len(ids), dtype=np.int32)
        _check(load().pkv_bm_tables(self._h, ids.ctypes.data, len(ids), max_blocks,
                                    t.ctypes.data, lens.ctypes.data))
        return t, lens

    def _swap(self, fn, seq, max_pairs):
        import numpy as np
        pairs = np.empty((max(max_pairs, 1), 2), dtype=np.int32)
        n = ctypes.c_int32()
        _check(fn(self._h, seq, pairs.ctypes.data, max_pairs, ctypes.byref(n)))
        return pairs[:n.value].copy()

    def swap_out(self, seq: int, max_pairs: int = 1 << 16):
        """(device block, host block) pairs to copy out; seq now lives in host blocks."""
        return self._swap(load().pkv_bm_swap_out, seq, max_pairs)

    def swap_in(self, seq: int, max_pairs: int = 1 << 16):
        """(host block, device block) pairs to copy in; seq lives on the device again."""
        return self._swap(load().pkv_bm_swap_in, seq, max_pairs)


def swap_blocks(src_k, src_v, dst_k, dst_v, pairs, to_device: bool):
    """pkv_swap_blocks: copy whole blocks (pairs int32 [M, 2] of (src, dst)) between a device
    pool and a host pool, on the current stream. The host pools are pinned CPU tensors shaped
    like the device pools."""
    import numpy as np
    dev = dst_k if to_device else src_k
    if len({t.dtype for t in (src_k, src_v, dst_k, dst_v)}) != 1:
        raise TypeError("the pools must share one dtype")
    for t, nm in ((src_k, "src_k"), (src_v, "src_v"), (dst_k, "dst_k"), (dst_v, "dst_v")):
        if not t.is_contiguous():
            raise ValueError(f"{nm} must be contiguous")
        on_device = nm.startswith("dst") == bool(to_device)
        if on_device and not t.is_cuda:
            raise ValueError(f"{nm} is the device pool: it must be on the GPU")
        if not on_device and (t.is_cuda or not t.is_pinned()):
            raise ValueError(f"{nm} is the host pool: it must be pinned CPU memory")
    if src_k.shape[1:] != dst_k.shape[1:] or src_v.shape[1:] != dst_v.shape[1:]:
        raise ValueError("pools of different block shapes")
    pairs = np.ascontiguousarray(pairs, dtype=np.int32).reshape(-1, 2)
    block_bytes = src_k[0].numel() * src_k.element_size()
    _check(load().pkv_swap_blocks(_ptr(src_k), _ptr(src_v), src_k.shape[0], _ptr(dst_k),
                                  _ptr(dst_v), dst_k.shape[0], pairs.ctypes.data, len(pairs),
                                  block_bytes, 1 if to_device else 0, _stream(dev)))


def probe_stream_read(buf: torch.Tensor, sink: torch.Tensor, nontemporal: bool = True,
                      workgroups: int = 2048):
    """pkv_probe_stream_read over all of buf (a contiguous device tensor whose size in bytes is
    a multiple of 32 KiB). sink: a device int32 tensor of at least one element."""
    _need(buf, "buf")
    _need(sink, "sink", torch.int32, 1, buf.device)
    nbytes = buf.numel() * buf.element_size()
    _check(load().pkv_probe_stream_read(_ptr(buf), nbytes, int(bool(nontemporal)),
                                        int(workgroups), _ptr(sink), _stream(buf)))


def probe_tile_gather(buf: torch.Tensor, offsets: torch.Tensor, tile_bytes: int,
                      sink: torch.Tensor, nontemporal: bool = True, workgroups: int = 2048):
    """pkv_probe_tile_gather: read the tiles of tile_bytes at the byte offsets (device int64
    [n]) into buf, in list order."""
    _need(buf, "buf")
    _need(offsets, "offsets", torch.int64, 1, buf.device)
    _need(sink, "sink", torch.int32, 1, buf.device)
    nbytes = buf.numel() * buf.element_size()
    _check(load().pkv_probe_tile_gather(_ptr(buf), nbytes, _ptr(offsets), offsets.shape[0],
                                        int(tile_bytes), int(bool(nontemporal)),
                                        int(workgroups), _ptr(sink), _stream(buf)))
