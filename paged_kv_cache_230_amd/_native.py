"""ctypes declarations for libpagedkv.so (the C ABI in include/pagedkv.h).

The library must have been built in-tree (``paged_kv_cache_230_amd.build``).
There is no fallback: importing this module without the library raises.
"""
from __future__ import annotations

import ctypes as C
import os

# torch must be loaded first: its HIP runtime (SONAME libamdhip64.so.7) then
# satisfies this library's dependency, so the process holds a single HIP
# runtime.  Loading the library first would map ROCm's copy and torch would
# map a second one, and device allocations and launches from the two do not
# mix.
import torch  # noqa: F401

HERE = os.path.dirname(os.path.abspath(__file__))
# PKV_LIB_PATH loads another build of the library instead of the in-tree one
# (the tests use it for a host-only sanitizer build of the block manager).
LIB_PATH = os.environ.get("PKV_LIB_PATH") or os.path.join(HERE, "libpagedkv.so")

PKV_OK = 0
PKV_ERR_INVALID_ARG = -1
PKV_ERR_OUT_OF_BLOCKS = -2
PKV_ERR_UNKNOWN_SEQ = -3
PKV_ERR_DEVICE = -4
PKV_ERR_UNSUPPORTED = -5
PKV_ERR_CAPACITY = -6
PKV_F32 = 0
PKV_BF16 = 1

# Flags of the device status word (pkv_device_status).
PKV_DEV_BAD_BLOCK_ID = 1
PKV_DEV_BAD_LENGTH = 2
PKV_DEV_BAD_SLOT = 4
PKV_DEV_BAD_PAIR = 8
PKV_DEV_BAD_RECORD = 16
PKV_DEV_BAD_QUERY_START = 32
PKV_DECODE_SHARED_BLOCKS = 1  # decode flag: several sequences read the same blocks

STATUS_NAMES = {
    PKV_ERR_INVALID_ARG: "INVALID_ARG",
    PKV_ERR_OUT_OF_BLOCKS: "OUT_OF_BLOCKS",
    PKV_ERR_UNKNOWN_SEQ: "UNKNOWN_SEQ",
    PKV_ERR_DEVICE: "DEVICE",
    PKV_ERR_UNSUPPORTED: "UNSUPPORTED",
    PKV_ERR_CAPACITY: "CAPACITY",
}


class PKVError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"pagedkv error {STATUS_NAMES.get(code, code)}: {msg}")
        self.code = code


if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python -m paged_kv_cache_230_amd.build` "
        "(the HIP library is required; there is no CPU fallback)"
    )

lib = C.CDLL(LIB_PATH)

_i32, _i64, _sz, _f32, _vp = C.c_int32, C.c_int64, C.c_size_t, C.c_float, C.c_void_p
_u32 = C.c_uint32
_pi32 = C.POINTER(C.c_int32)
_pi64 = C.POINTER(C.c_int64)
_u64 = C.c_uint64
_pu8 = C.POINTER(C.c_uint8)

_SIGS = {
    "pkv_last_error": (C.c_char_p, []),
    "pkv_version": (_i32, []),
    "pkv_device_status": (_i32, [_vp, _i32, _pi32]),
    "pkv_stream_read": (_i32, [_vp, _sz, _vp, _i32, _vp]),
    "pkv_mfma_rate": (_i32, [_vp, _i32, _i32, _vp]),
    "pkv_tile_read": (_i32, [_vp, _sz, _sz, _vp, _i64, _vp, _i32, _vp]),
    "paged_kv_append": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _vp]),
    "paged_kv_copy_blocks": (_i32, [_vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _vp]),
    "paged_attention_decode": (
        _i32,
        [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _f32, _i32, _vp, _sz, _i32,
         _u32, _vp],
    ),
    "paged_attention_decode_append": (
        _i32,
        [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _f32, _i32, _vp,
         _sz, _i32, _u32, _vp],
    ),
    "paged_attention_decode_append_noalloc": (
        _i32,
        [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _f32, _i32, _i32,
         _u32, _vp],
    ),
    "paged_attention_workgroups_per_head": (_i32, [_i32, _i32, _i32, _i32, _i32, _i32, _i32]),
    "paged_attention_segment_cost": (_i32, [_i32]),
    "paged_attention_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32, _i32]),
    "paged_attention_prefill": (
        _i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _f32, _i32,
               _vp]),
    "pkv_bm_create": (_i32, [_i32, _i32, _pi32, C.POINTER(_vp)]),
    "pkv_bm_destroy": (None, [_vp]),
    "pkv_bm_add_seq": (_i32, [_vp, _i64]),
    "pkv_bm_fork": (_i32, [_vp, _i64, _i64, _i32]),
    "pkv_bm_append_slots": (_i32, [_vp, _pi64, _i32, _pi32, _pi32, _pi32, _i32, _pi32, _pi32, _i32, _pi32]),
    "pkv_bm_free_seq": (_i32, [_vp, _i64]),
    "pkv_bm_block_tables": (_i32, [_vp, _pi64, _i32, _i32, _pi32, _pi32]),
    "pkv_bm_num_free": (_i32, [_vp]),
    "pkv_bm_refcount": (_i32, [_vp, _i32]),
    "pkv_bm_num_shared": (_i32, [_vp]),
    "pkv_bm_seq_len": (_i32, [_vp, _i64]),
    "pkv_bm_num_seqs": (_i32, [_vp]),
    "pkv_bm_free_stack": (_i32, [_vp, _pi32, _i32]),
    "pkv_bm_stage_step": (
        _i32, [_vp, _pi64, _i32, _pi32, _vp, _i32, _vp, _i32, _vp, _vp, _vp, _i32, _i32, _pi32, _pi32, _vp]),
    "pkv_bm_stage_capacity": (_i32, [_i32, _i32]),
    "pkv_block_digest": (_i32, [_pu8, _u64, _pi32, _i32, _pu8]),
    "paged_kv_swap_blocks": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _vp]),
    "pkv_bm_add_host_pool": (_i32, [_vp, _i32]),
    "pkv_bm_swap_out": (_i32, [_vp, _i64, _pi32, _i32, _pi32]),
    "pkv_bm_swap_in": (_i32, [_vp, _i64, _pi32, _i32, _pi32]),
    "pkv_bm_num_free_host": (_i32, [_vp]),
    "pkv_bm_is_swapped": (_i32, [_vp, _i64]),
    "pkv_radix_create": (_i32, [_vp, C.POINTER(_vp)]),
    "pkv_radix_destroy": (None, [_vp]),
    "pkv_radix_match": (_i32, [_vp, _pi32, _i32]),
    "pkv_radix_admit": (_i32, [_vp, _i64, _pi32, _i32, _pi32]),
    "pkv_radix_insert": (_i32, [_vp, _i64, _pi32, _i32, _pi32]),
    "pkv_radix_release": (_i32, [_vp, _i64]),
    "pkv_radix_evict": (_i32, [_vp, _i32, _pi32]),
    "pkv_radix_num_nodes": (_i32, [_vp]),
    "pkv_radix_nodes": (_i32, [_vp, _pi64, _pi32, _pi32, _pi32, _pi64, _i32]),
    "pkv_bm_add_seq_cached": (_i32, [_vp, _i64, _pi32, _i32, _u64, _pi32]),
    "pkv_bm_match_prefix": (_i32, [_vp, _pi32, _i32, _u64]),
    "pkv_bm_num_cached": (_i32, [_vp]),
    "pkv_bm_evictable": (_i32, [_vp, _pi32, _i32]),
    "pkv_bm_cached_digest": (_i32, [_vp, _i32, _pu8]),
}

for _name, (_res, _args) in _SIGS.items():
    _fn = getattr(lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args

EXPORTED = tuple(_SIGS)


def last_error() -> str:
    return lib.pkv_last_error().decode("utf-8", "replace")


def check(code: int) -> int:
    if code < 0:
        raise PKVError(code, last_error())
    return code
