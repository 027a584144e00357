"""Thin Python binding of libkvz.so (ctypes).

Argument marshalling only: every step of the path runs in the HIP library.  Functions carry the
C names; tensors are passed as device pointers (torch supplies device memory and the current
HIP stream).  If libkvz.so has not been built this module raises at import time - there is no
fallback of any kind.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvz.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with decode_attention_kvz_amd/build.py "
                      "(or __graft_entry__.build()) before using the binding")

_lib = ctypes.CDLL(LIB_PATH)

KVZ_OK = 0
KVZ_EINVAL = -1
KVZ_EUNSUPPORTED = -2
KVZ_EHIP = -4
KVZ_ESTATE = -5
KVZ_RAW_TAG = 0xFF
KVZ_OFF_NONE = 0xFFFFFFFF
KVZ_KIND_K = 0
KVZ_KIND_V = 1
KVZ_ENC_FORCE_RAW = 1
KVZ_ENC_SIMULATE_GIVE_UP = 2
KVZ_WS_BAD_COUNTER = 1
KVZ_PART_ALL, KVZ_PART_LOAD, KVZ_PART_LOAD_RESTORE = 0, 1, 2
GRANULE = 256
KVZ_FP8_E4M3 = 0
KVZ_FP8_E5M2 = 1
FP8_GRANULE = 128

EXPORTED = [
    "kvz_version", "kvz_last_error", "kvz_device_check", "kvz_pool_state_bytes", "kvz_pool_init",
    "kvz_pool_destroy", "kvz_slot_alloc", "kvz_slot_free", "kvz_encode_pages", "kvz_complete_pages",
    "kvz_decode_block",
    "kvz_attn_workspace_bytes", "kvz_decode_attention", "kvz_bf16_pack_pages",
    "kvz_bf16_decode_attention", "kvz_pool_stats", "kvz_stream_read", "kvz_decompress_pages",
    "kvz_pool_capacity", "kvz_gaac_calibrate", "kvz_gaac_encode_pages", "kvz_gaac_decompress_pages",
    "kvz_gaac_decode_attention", "kvz_fp8_pool_state_bytes", "kvz_fp8_pool_init",
    "kvz_fp8_calibrate", "kvz_fp8_encode_pages", "kvz_fp8_decompress_pages", "kvz_fp8_pack_pages",
    "kvz_fp8_decode_attention", "kvz_fp8_raw_decode_attention", "kvz_decode_attention_noalloc",
    "kvz_attn_workspace_status", "kvz_decode_attention_part", "kvz_bf16_decode_attention_part",
]


class KvzError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"kvz error {code}: {msg}")
        self.code = code


class PoolStats(ctypes.Structure):
    _fields_ = [("capacity_granules", ctypes.c_uint64), ("frontier_granules", ctypes.c_uint64),
                ("free_runs", ctypes.c_uint64 * 5), ("live_runs", ctypes.c_uint64),
                ("live_granules", ctypes.c_uint64), ("live_raw_blocks", ctypes.c_uint64),
                ("enospc", ctypes.c_uint64), ("bad_frees", ctypes.c_uint64),
                ("encoder_halted", ctypes.c_uint64)]


class Capacity(ctypes.Structure):
    _fields_ = [("free_granules", ctypes.c_uint64), ("guaranteed_groups", ctypes.c_uint64),
                ("guaranteed_pages", ctypes.c_uint64), ("guaranteed_tokens", ctypes.c_uint64),
                ("expected_group_granules", ctypes.c_double), ("expected_pages", ctypes.c_uint64),
                ("expected_tokens", ctypes.c_uint64)]


class AttnArgs(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("out", ctypes.c_void_p), ("arena", ctypes.c_void_p),
                ("arena_bytes", ctypes.c_uint64), ("meta", ctypes.c_void_p),
                ("n_phys_pages", ctypes.c_int32), ("block_table", ctypes.c_void_p),
                ("seq_lens", ctypes.c_void_p), ("n_comp_pages", ctypes.c_void_p),
                ("tail", ctypes.c_void_p), ("batch", ctypes.c_int32),
                ("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("max_pages", ctypes.c_int32), ("splits", ctypes.c_int32),
                ("sm_scale", ctypes.c_float), ("workspace", ctypes.c_void_p),
                ("workspace_bytes", ctypes.c_uint64)]


class Bf16AttnArgs(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("out", ctypes.c_void_p), ("pages", ctypes.c_void_p),
                ("n_phys_pages", ctypes.c_int32), ("block_table", ctypes.c_void_p),
                ("seq_lens", ctypes.c_void_p),
                ("n_comp_pages", ctypes.c_void_p), ("tail", ctypes.c_void_p),
                ("batch", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("max_pages", ctypes.c_int32),
                ("splits", ctypes.c_int32), ("sm_scale", ctypes.c_float),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_uint64)]


class Fp8AttnArgs(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("out", ctypes.c_void_p), ("arena", ctypes.c_void_p),
                ("arena_bytes", ctypes.c_uint64), ("meta", ctypes.c_void_p),
                ("bases", ctypes.c_void_p), ("pages", ctypes.c_void_p),
                ("n_phys_pages", ctypes.c_int32), ("block_table", ctypes.c_void_p),
                ("seq_lens", ctypes.c_void_p), ("n_comp_pages", ctypes.c_void_p),
                ("tail", ctypes.c_void_p), ("batch", ctypes.c_int32),
                ("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("max_pages", ctypes.c_int32), ("splits", ctypes.c_int32),
                ("format", ctypes.c_uint32), ("sm_scale", ctypes.c_float),
                ("k_scale", ctypes.c_float), ("v_scale", ctypes.c_float),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_uint64)]


# kvz_encode_item / kvz_block_ref as numpy record layouts (device arrays are built from these)
ENCODE_ITEM_DTYPE = np.dtype([("src", "<u8"), ("dst", "<u8"), ("src_stride", "<u4"),
                              ("kind", "<u4")])
BLOCK_REF_DTYPE = np.dtype([("meta", "<u8"), ("block", "<u4"), ("kind", "<u4")])
GAAC_ITEM_DTYPE = np.dtype([("src", "<u8"), ("dst", "<u8"), ("src_stride", "<u4"),
                            ("kind", "<u4"), ("bases", "<u8")])
FP8_ITEM_DTYPE = GAAC_ITEM_DTYPE          # kvz_fp8_item: the same fields (src points to bytes)

_vp = ctypes.c_void_p
_sig = {
    "kvz_version": ([], ctypes.c_int),
    "kvz_last_error": ([], ctypes.c_char_p),
    "kvz_device_check": ([ctypes.c_int], ctypes.c_int),
    "kvz_pool_state_bytes": ([ctypes.c_uint64, ctypes.POINTER(ctypes.c_uint64)], ctypes.c_int),
    "kvz_pool_init": ([ctypes.POINTER(_vp), _vp, ctypes.c_uint64, _vp, ctypes.c_uint64, _vp],
                      ctypes.c_int),
    "kvz_pool_destroy": ([_vp], ctypes.c_int),
    "kvz_slot_alloc": ([_vp, _vp, _vp, ctypes.c_int32, _vp], ctypes.c_int),
    "kvz_slot_free": ([_vp, _vp, ctypes.c_int32, _vp], ctypes.c_int),
    "kvz_encode_pages": ([_vp, _vp, ctypes.c_int32, ctypes.c_uint32, _vp], ctypes.c_int),
    "kvz_complete_pages": ([_vp, _vp, ctypes.c_int32, _vp, ctypes.c_int32, ctypes.c_uint32, _vp],
                           ctypes.c_int),
    "kvz_decode_block": ([_vp, ctypes.c_uint64, _vp, ctypes.c_int32, _vp, _vp], ctypes.c_int),
    "kvz_attn_workspace_bytes": ([ctypes.c_int32] * 5 + [ctypes.POINTER(ctypes.c_uint64)],
                                 ctypes.c_int),
    "kvz_decode_attention": ([ctypes.POINTER(AttnArgs), _vp], ctypes.c_int),
    "kvz_bf16_pack_pages": ([_vp, _vp, ctypes.c_int64, ctypes.c_int32, _vp], ctypes.c_int),
    "kvz_bf16_decode_attention": ([ctypes.POINTER(Bf16AttnArgs), _vp], ctypes.c_int),
    "kvz_pool_stats": ([_vp, ctypes.POINTER(PoolStats), _vp], ctypes.c_int),
    "kvz_stream_read": ([_vp, ctypes.c_uint64, _vp, ctypes.c_int32, _vp], ctypes.c_int),
    "kvz_gaac_calibrate": ([_vp, ctypes.c_int32, _vp, _vp, _vp], ctypes.c_int),
    "kvz_gaac_decode_attention": ([ctypes.POINTER(AttnArgs), _vp, _vp], ctypes.c_int),
    "kvz_gaac_encode_pages": ([_vp, _vp, ctypes.c_int32, ctypes.c_uint32, _vp], ctypes.c_int),
    "kvz_gaac_decompress_pages": ([_vp, ctypes.c_uint64, _vp, _vp, ctypes.c_int64, ctypes.c_int32,
                                   _vp, _vp], ctypes.c_int),
    "kvz_pool_capacity": ([ctypes.POINTER(PoolStats), ctypes.c_int32, ctypes.c_int32,
                           ctypes.POINTER(Capacity)], ctypes.c_int),
    "kvz_decompress_pages": ([_vp, ctypes.c_uint64, _vp, ctypes.c_int64, ctypes.c_int32, _vp, _vp],
                             ctypes.c_int),
    "kvz_fp8_pool_state_bytes": ([ctypes.c_uint64, ctypes.POINTER(ctypes.c_uint64)], ctypes.c_int),
    "kvz_fp8_pool_init": ([ctypes.POINTER(_vp), _vp, ctypes.c_uint64, _vp, ctypes.c_uint64, _vp],
                          ctypes.c_int),
    "kvz_fp8_calibrate": ([_vp, ctypes.c_int32, ctypes.c_uint32, _vp, _vp, _vp], ctypes.c_int),
    "kvz_fp8_encode_pages": ([_vp, _vp, ctypes.c_int32, ctypes.c_uint32, ctypes.c_uint32, _vp],
                             ctypes.c_int),
    "kvz_fp8_decompress_pages": ([_vp, ctypes.c_uint64, _vp, _vp, ctypes.c_int64, ctypes.c_int32,
                                  ctypes.c_uint32, _vp, _vp], ctypes.c_int),
    "kvz_fp8_pack_pages": ([_vp, _vp, ctypes.c_int64, ctypes.c_int32, _vp], ctypes.c_int),
    "kvz_fp8_decode_attention": ([ctypes.POINTER(Fp8AttnArgs), _vp], ctypes.c_int),
    "kvz_fp8_raw_decode_attention": ([ctypes.POINTER(Fp8AttnArgs), _vp], ctypes.c_int),
    "kvz_decode_attention_noalloc": ([ctypes.POINTER(AttnArgs), _vp], ctypes.c_int),
    "kvz_attn_workspace_status": ([_vp, ctypes.POINTER(ctypes.c_uint32), _vp], ctypes.c_int),
    "kvz_decode_attention_part": ([ctypes.POINTER(AttnArgs), ctypes.c_int32, _vp], ctypes.c_int),
    "kvz_bf16_decode_attention_part": ([ctypes.POINTER(Bf16AttnArgs), ctypes.c_int32, _vp], ctypes.c_int),
}
for _name, (_args, _ret) in _sig.items():
    _f = getattr(_lib, _name)
    _f.argtypes = _args
    _f.restype = _ret


def _check(rc):
    if rc != KVZ_OK:
        raise KvzError(rc, _lib.kvz_last_error().decode(errors="replace"))


def _ptr(t):
    """Device pointer of a tensor (None -> NULL)."""
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _nbytes(t) -> int:
    return t.numel() * t.element_size()


def _dev(name, t, dtype=None, shape=None, min_bytes=None):
    """A device-memory argument: a contiguous GPU tensor, of `dtype` and `shape` when given
    (None entries match any size), holding at least `min_bytes`.  The library cannot tell a
    host pointer or a short buffer from a good one, so these are checked before the call."""
    if t is None:
        raise ValueError(f"{name} is required")
    if not getattr(t, "is_cuda", False):
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None:
        if t.dim() != len(shape) or any(w is not None and int(g) != int(w)
                                        for g, w in zip(t.shape, shape)):
            raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if min_bytes is not None and _nbytes(t) < min_bytes:
        raise ValueError(f"{name} holds {_nbytes(t)} bytes, needs at least {min_bytes}")
    return t


def _torch():
    import torch
    return torch


def _stream(stream=None):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


# ---------------------------------------------------------------------------------------------
def kvz_version() -> int:
    return _lib.kvz_version()


def kvz_last_error() -> str:
    return _lib.kvz_last_error().decode(errors="replace")


def kvz_device_check(device: int = 0) -> None:
    _check(_lib.kvz_device_check(device))


def kvz_pool_state_bytes(arena_bytes: int) -> int:
    out = ctypes.c_uint64()
    _check(_lib.kvz_pool_state_bytes(arena_bytes, ctypes.byref(out)))
    return out.value


def kvz_pool_init(arena, state, stream=None):
    """arena, state: uint8 device tensors.  Returns the opaque pool handle."""
    _dev("arena", arena)
    _dev("state", state)
    h = ctypes.c_void_p()
    _check(_lib.kvz_pool_init(ctypes.byref(h), _ptr(arena), arena.numel() * arena.element_size(),
                              _ptr(state), state.numel() * state.element_size(), _stream(stream)))
    return h


def kvz_pool_destroy(pool) -> None:
    _check(_lib.kvz_pool_destroy(pool))


def kvz_slot_alloc(pool, tags, off, stream=None) -> None:
    """tags: uint8 [n, 4] device; off: int32/uint32 [n] device (receives offsets)."""
    n = tags.shape[0]
    _dev("tags", tags, min_bytes=4 * n)
    _dev("off", off, min_bytes=4 * n)
    _check(_lib.kvz_slot_alloc(pool, _ptr(tags), _ptr(off), n, _stream(stream)))


def kvz_slot_free(pool, meta_ptrs, stream=None) -> None:
    """meta_ptrs: int64 [n] device tensor of device pointers to kvz_group_meta."""
    _dev("meta_ptrs", meta_ptrs, dtype=_torch().int64)
    _check(_lib.kvz_slot_free(pool, _ptr(meta_ptrs), meta_ptrs.shape[0], _stream(stream)))


def kvz_encode_pages(pool, items, n: int, flags: int = 0, stream=None) -> None:
    """items: device tensor holding n kvz_encode_item records (ENCODE_ITEM_DTYPE)."""
    _dev("items", items, min_bytes=n * ENCODE_ITEM_DTYPE.itemsize)
    _check(_lib.kvz_encode_pages(pool, _ptr(items), n, flags, _stream(stream)))


def kvz_complete_pages(pool, meta_ptrs, items, n: int, flags: int = 0, stream=None) -> None:
    """kvz_slot_free(meta_ptrs) then kvz_encode_pages(items, n) in one call: meta_ptrs is an
    int64 [n_free] device tensor of device pointers to kvz_group_meta (or None)."""
    n_free = 0
    if meta_ptrs is not None:
        _dev("meta_ptrs", meta_ptrs, dtype=_torch().int64)
        n_free = meta_ptrs.shape[0]
    if n:
        _dev("items", items, min_bytes=n * ENCODE_ITEM_DTYPE.itemsize)
    _check(_lib.kvz_complete_pages(pool, _ptr(meta_ptrs) if n_free else None, n_free,
                                   _ptr(items) if n else None, n, flags, _stream(stream)))


def kvz_decode_block(arena, refs, n: int, out, stream=None) -> None:
    """refs: device tensor of n kvz_block_ref records; out: int16/uint16 [n, 16, 32] device."""
    _dev("arena", arena)
    _dev("refs", refs, min_bytes=n * BLOCK_REF_DTYPE.itemsize)
    _dev("out", out, min_bytes=n * 16 * 32 * 2)
    _check(_lib.kvz_decode_block(_ptr(arena), arena.numel() * arena.element_size(), _ptr(refs),
                                 n, _ptr(out), _stream(stream)))


def kvz_attn_workspace_bytes(batch, num_q_heads, num_kv_heads, max_pages, splits=0) -> int:
    out = ctypes.c_uint64()
    _check(_lib.kvz_attn_workspace_bytes(batch, num_q_heads, num_kv_heads, max_pages, splits,
                                         ctypes.byref(out)))
    return out.value


def kvz_attn_workspace_status(workspace=None, stream=None) -> int:
    """The sticky KVZ_WS_* flags of an attention workspace (None: the allocation-free call's
    scratch on the current device); synchronizes the stream."""
    if workspace is not None:
        _dev("workspace", workspace)
    flags = ctypes.c_uint32()
    _check(_lib.kvz_attn_workspace_status(None if workspace is None else workspace.data_ptr(),
                                          ctypes.byref(flags), _stream(stream)))
    return flags.value


def _check_attn_common(q, out, block_table, seq_lens, n_comp_pages, workspace, hkv,
                       tail=None, tail_dtype=None, tail_bytes_per_value=2, allow_no_workspace=False):
    """The arguments every decode-attention call shares: q [B,Hq,128] bf16, out [B,Hq,128] fp32,
    block_table [B,max_pages] int32, seq_lens / n_comp_pages [B] int32, the tail page
    [B,2,Hkv,16,128] (or None) and the workspace."""
    torch = _torch()
    _dev("q", q, dtype=torch.bfloat16, shape=(None, None, 128))
    bsz, hq = q.shape[0], q.shape[1]
    _dev("out", out, dtype=torch.float32, shape=(bsz, hq, 128))
    _dev("block_table", block_table, dtype=torch.int32, shape=(bsz, None))
    _dev("seq_lens", seq_lens, dtype=torch.int32, shape=(bsz,))
    _dev("n_comp_pages", n_comp_pages, dtype=torch.int32, shape=(bsz,))
    if workspace is not None or not allow_no_workspace:
        _dev("workspace", workspace)
    if tail is not None:
        _dev("tail", tail, dtype=tail_dtype, min_bytes=bsz * 2 * hkv * 16 * 128 * tail_bytes_per_value)


def _check_meta(meta):
    """Per-layer metadata [n_phys_pages, Hkv, ...]: 16 bytes (the K and V group records) per
    (physical page, KV head)."""
    _dev("meta", meta)
    if meta.dim() < 2 or _nbytes(meta) != meta.shape[0] * meta.shape[1] * 16:
        raise ValueError("meta must be [n_phys_pages, Hkv, ...] with 16 bytes per (page, KV head)")


def _attn_args(q, out, arena, meta, block_table, seq_lens, n_comp_pages, tail, sm_scale,
               workspace, splits):
    _check_meta(meta)
    _dev("arena", arena)
    _check_attn_common(q, out, block_table, seq_lens, n_comp_pages, workspace, meta.shape[1],
                       tail=tail, tail_dtype=_torch().bfloat16)
    bsz, hq, hd = q.shape
    return AttnArgs(q=q.data_ptr(), out=out.data_ptr(), arena=arena.data_ptr(),
                 arena_bytes=arena.numel() * arena.element_size(), meta=meta.data_ptr(),
                 n_phys_pages=meta.shape[0], block_table=block_table.data_ptr(), seq_lens=seq_lens.data_ptr(),
                 n_comp_pages=n_comp_pages.data_ptr(),
                 tail=None if tail is None else tail.data_ptr(), batch=bsz, num_q_heads=hq,
                 num_kv_heads=meta.shape[1], head_dim=hd, page_size=16,
                 max_pages=block_table.shape[1], splits=splits, sm_scale=sm_scale,
                 workspace=workspace.data_ptr(),
                 workspace_bytes=workspace.numel() * workspace.element_size())


def kvz_decode_attention(q, out, arena, meta, block_table, seq_lens, n_comp_pages, tail,
                         sm_scale: float, workspace, splits: int = 0, stream=None) -> None:
    """q [B,Hq,128] bf16; out [B,Hq,128] fp32; meta [n_phys,Hkv,2,8] uint8 (or any 8-byte
    records); block_table [B,max_pages] int32; seq_lens, n_comp_pages [B] int32;
    tail [B,2,Hkv,16,128] bf16 or None; workspace uint8 device tensor."""
    a = _attn_args(q, out, arena, meta, block_table, seq_lens, n_comp_pages, tail, sm_scale,
                   workspace, splits)
    _check(_lib.kvz_decode_attention(ctypes.byref(a), _stream(stream)))


def kvz_decode_attention_part(q, out, arena, meta, block_table, seq_lens, n_comp_pages, tail,
                              sm_scale: float, workspace, part: int, splits: int = 0,
                              stream=None) -> None:
    """kvz_decode_attention restricted to a part of the kernel (KVZ_PART_*), for the time
    breakdown; the partial variants leave out and the workspace as they are."""
    a = _attn_args(q, out, arena, meta, block_table, seq_lens, n_comp_pages, tail, sm_scale,
                   workspace, splits)
    _check(_lib.kvz_decode_attention_part(ctypes.byref(a), part, _stream(stream)))


def kvz_decode_attention_noalloc(q, out, arena, meta, block_table, seq_lens, n_comp_pages, tail,
                                 sm_scale: float, splits: int = 0, stream=None) -> None:
    """kvz_decode_attention without a workspace: the library's device-resident scratch holds the
    partial results (no device memory is allocated).  Same arguments otherwise."""
    _check_meta(meta)
    _dev("arena", arena)
    _check_attn_common(q, out, block_table, seq_lens, n_comp_pages, None, meta.shape[1],
                       tail=tail, tail_dtype=_torch().bfloat16, allow_no_workspace=True)
    bsz, hq, hd = q.shape
    a = AttnArgs(q=q.data_ptr(), out=out.data_ptr(), arena=arena.data_ptr(),
                 arena_bytes=arena.numel() * arena.element_size(), meta=meta.data_ptr(),
                 n_phys_pages=meta.shape[0], block_table=block_table.data_ptr(),
                 seq_lens=seq_lens.data_ptr(), n_comp_pages=n_comp_pages.data_ptr(),
                 tail=None if tail is None else tail.data_ptr(), batch=bsz, num_q_heads=hq,
                 num_kv_heads=meta.shape[1], head_dim=hd, page_size=16,
                 max_pages=block_table.shape[1], splits=splits, sm_scale=sm_scale,
                 workspace=None, workspace_bytes=0)
    _check(_lib.kvz_decode_attention_noalloc(ctypes.byref(a), _stream(stream)))


def kvz_gaac_decode_attention(q, out, arena, meta, bases, block_table, seq_lens, n_comp_pages,
                              tail, sm_scale: float, workspace, splits: int = 0,
                              stream=None) -> None:
    """As kvz_decode_attention over group-adaptive tiles; bases [Hkv,2,2,128] uint8 device."""
    _check_meta(meta)
    _dev("bases", bases, min_bytes=meta.shape[1] * 512)
    a = _attn_args(q, out, arena, meta, block_table, seq_lens, n_comp_pages, tail, sm_scale,
                   workspace, splits)
    _check(_lib.kvz_gaac_decode_attention(ctypes.byref(a), _ptr(bases), _stream(stream)))


def kvz_bf16_pack_pages(src, dst, stream=None) -> None:
    """src [n_pages,2,Hkv,16,128] bf16 natural pages -> dst [n_pages,2,Hkv,4,1024] uint8."""
    _dev("src", src, dtype=_torch().bfloat16, shape=(None, 2, None, 16, 128))
    _dev("dst", dst, min_bytes=_nbytes(src))
    _check(_lib.kvz_bf16_pack_pages(_ptr(src), _ptr(dst), src.shape[0], src.shape[2],
                                    _stream(stream)))


def kvz_bf16_decode_attention(q, out, pages, block_table, seq_lens, n_comp_pages, tail,
                              sm_scale: float, workspace, num_kv_heads: int, splits: int = 0,
                              stream=None) -> None:
    """The BF16 baseline: pages [n_phys,2,Hkv,4,1024] uint8 (kvz_bf16_pack_pages)."""
    _dev("pages", pages, min_bytes=pages.shape[0] * 2 * num_kv_heads * 4096)
    _check_attn_common(q, out, block_table, seq_lens, n_comp_pages, workspace, num_kv_heads,
                       tail=tail, tail_dtype=_torch().bfloat16)
    bsz, hq, hd = q.shape
    a = Bf16AttnArgs(q=q.data_ptr(), out=out.data_ptr(), pages=pages.data_ptr(),
                     n_phys_pages=pages.shape[0], block_table=block_table.data_ptr(), seq_lens=seq_lens.data_ptr(),
                     n_comp_pages=n_comp_pages.data_ptr(),
                     tail=None if tail is None else tail.data_ptr(), batch=bsz, num_q_heads=hq,
                     num_kv_heads=num_kv_heads, head_dim=hd, page_size=16,
                     max_pages=block_table.shape[1], splits=splits, sm_scale=sm_scale,
                     workspace=workspace.data_ptr(),
                     workspace_bytes=workspace.numel() * workspace.element_size())
    _check(_lib.kvz_bf16_decode_attention(ctypes.byref(a), _stream(stream)))


def kvz_bf16_decode_attention_part(q, out, pages, block_table, seq_lens, n_comp_pages, tail,
                                   sm_scale: float, workspace, num_kv_heads: int, part: int,
                                   splits: int = 0, stream=None) -> None:
    """kvz_bf16_decode_attention restricted to a part of the kernel (KVZ_PART_ALL or
    KVZ_PART_LOAD), for the time breakdown."""
    _dev("pages", pages, min_bytes=pages.shape[0] * 2 * num_kv_heads * 4096)
    _check_attn_common(q, out, block_table, seq_lens, n_comp_pages, workspace, num_kv_heads,
                       tail=tail, tail_dtype=_torch().bfloat16)
    bsz, hq, hd = q.shape
    a = Bf16AttnArgs(q=q.data_ptr(), out=out.data_ptr(), pages=pages.data_ptr(),
                     n_phys_pages=pages.shape[0], block_table=block_table.data_ptr(), seq_lens=seq_lens.data_ptr(),
                     n_comp_pages=n_comp_pages.data_ptr(),
                     tail=None if tail is None else tail.data_ptr(), batch=bsz, num_q_heads=hq,
                     num_kv_heads=num_kv_heads, head_dim=hd, page_size=16,
                     max_pages=block_table.shape[1], splits=splits, sm_scale=sm_scale,
                     workspace=workspace.data_ptr(),
                     workspace_bytes=workspace.numel() * workspace.element_size())
    _check(_lib.kvz_bf16_decode_attention_part(ctypes.byref(a), part, _stream(stream)))


def kvz_pool_stats(pool, stream=None) -> dict:
    st = PoolStats()
    _check(_lib.kvz_pool_stats(pool, ctypes.byref(st), _stream(stream)))
    return {"capacity_granules": st.capacity_granules, "frontier_granules": st.frontier_granules,
            "free_runs": list(st.free_runs), "live_runs": st.live_runs,
            "live_granules": st.live_granules, "live_raw_blocks": st.live_raw_blocks,
            "enospc": st.enospc, "bad_frees": st.bad_frees, "encoder_halted": st.encoder_halted}


def kvz_decompress_pages(arena, meta, dst, stream=None) -> None:
    """meta: [n_pages, Hkv, 2, 8] uint8; dst: n_pages * 2 * Hkv * 4096 bytes."""
    _check_meta(meta)
    n_pages, hkv = meta.shape[0], meta.shape[1]
    _dev("arena", arena)
    _dev("dst", dst, min_bytes=n_pages * 2 * hkv * 4096)
    _check(_lib.kvz_decompress_pages(_ptr(arena), arena.numel() * arena.element_size(), _ptr(meta),
                                     n_pages, hkv, _ptr(dst), _stream(stream)))


def kvz_pool_capacity(stats: dict, num_layers: int, num_kv_heads: int) -> dict:
    """stats: a kvz_pool_stats result (dict); host arithmetic only."""
    st = PoolStats()
    for k in ("capacity_granules", "frontier_granules", "live_runs", "live_granules",
              "live_raw_blocks", "enospc", "bad_frees"):
        setattr(st, k, int(stats[k]))
    for k in range(5):
        st.free_runs[k] = int(stats["free_runs"][k])
    cap = Capacity()
    _check(_lib.kvz_pool_capacity(ctypes.byref(st), num_layers, num_kv_heads, ctypes.byref(cap)))
    return {name: getattr(cap, name) for name, _ in Capacity._fields_}


def kvz_gaac_calibrate(items, n: int, hist, bases, stream=None) -> None:
    """items: device kvz_encode_item records (pages of one (layer, K|V, KV head)); hist: device
    >= 128*256 uint32 scratch; bases: device uint8 [2, 128] out (b3, b4)."""
    _dev("items", items, min_bytes=n * ENCODE_ITEM_DTYPE.itemsize)
    _dev("hist", hist, min_bytes=128 * 256 * 4)
    _dev("bases", bases, min_bytes=256)
    _check(_lib.kvz_gaac_calibrate(_ptr(items), n, _ptr(hist), _ptr(bases), _stream(stream)))


def kvz_gaac_encode_pages(pool, items, n: int, flags: int = 0, stream=None) -> None:
    """items: device tensor holding n kvz_gaac_item records (GAAC_ITEM_DTYPE)."""
    _dev("items", items, min_bytes=n * GAAC_ITEM_DTYPE.itemsize)
    _check(_lib.kvz_gaac_encode_pages(pool, _ptr(items), n, flags, _stream(stream)))


def kvz_gaac_decompress_pages(arena, meta, bases, dst, stream=None) -> None:
    """meta: [n_pages, Hkv, 2, 8] uint8; bases: [Hkv, 2, 2, 128] uint8; dst: n_pages*2*Hkv*4096 B."""
    _check_meta(meta)
    n_pages, hkv = meta.shape[0], meta.shape[1]
    _dev("arena", arena)
    _dev("bases", bases, min_bytes=hkv * 512)
    _dev("dst", dst, min_bytes=n_pages * 2 * hkv * 4096)
    _check(_lib.kvz_gaac_decompress_pages(_ptr(arena), arena.numel() * arena.element_size(),
                                          _ptr(meta), _ptr(bases), n_pages, hkv, _ptr(dst),
                                          _stream(stream)))


def kvz_fp8_pool_state_bytes(arena_bytes: int) -> int:
    out = ctypes.c_uint64()
    _check(_lib.kvz_fp8_pool_state_bytes(arena_bytes, ctypes.byref(out)))
    return out.value


def kvz_fp8_pool_init(arena, state, stream=None):
    """A pool of FP8 tiles (128-byte granules).  arena, state: uint8 device tensors."""
    _dev("arena", arena)
    _dev("state", state)
    h = ctypes.c_void_p()
    _check(_lib.kvz_fp8_pool_init(ctypes.byref(h), _ptr(arena),
                                  arena.numel() * arena.element_size(), _ptr(state),
                                  state.numel() * state.element_size(), _stream(stream)))
    return h


def kvz_fp8_calibrate(items, n: int, fmt: int, hist, bases, stream=None) -> None:
    """items: device kvz_fp8_item records (pages of one (layer, K|V, KV head)); hist: device
    >= 128*32 uint32 scratch; bases: device uint8 [2, 128] out (b3, b4)."""
    _dev("items", items, min_bytes=n * FP8_ITEM_DTYPE.itemsize)
    _dev("hist", hist, min_bytes=128 * 32 * 4)
    _dev("bases", bases, min_bytes=256)
    _check(_lib.kvz_fp8_calibrate(_ptr(items), n, fmt, _ptr(hist), _ptr(bases), _stream(stream)))


def kvz_fp8_encode_pages(pool, items, n: int, fmt: int, flags: int = 0, stream=None) -> None:
    """items: device tensor holding n kvz_fp8_item records (FP8_ITEM_DTYPE)."""
    _dev("items", items, min_bytes=n * FP8_ITEM_DTYPE.itemsize)
    _check(_lib.kvz_fp8_encode_pages(pool, _ptr(items), n, fmt, flags, _stream(stream)))


def kvz_fp8_decompress_pages(arena, meta, bases, fmt: int, dst, stream=None) -> None:
    """meta: [n_pages, Hkv, 2, 8] uint8; bases: [Hkv, 2, 2, 128] uint8; dst: n_pages*2*Hkv*2048 B."""
    _check_meta(meta)
    n_pages, hkv = meta.shape[0], meta.shape[1]
    _dev("arena", arena)
    _dev("bases", bases, min_bytes=hkv * 512)
    _dev("dst", dst, min_bytes=n_pages * 2 * hkv * 2048)
    _check(_lib.kvz_fp8_decompress_pages(_ptr(arena), arena.numel() * arena.element_size(),
                                         _ptr(meta), _ptr(bases), n_pages, hkv, fmt, _ptr(dst),
                                         _stream(stream)))


def kvz_fp8_pack_pages(src, dst, stream=None) -> None:
    """src [n_pages,2,Hkv,16,128] uint8 natural FP8 pages -> dst [n_pages,2,Hkv,2048] uint8."""
    _dev("src", src, dtype=_torch().uint8, shape=(None, 2, None, 16, 128))
    _dev("dst", dst, min_bytes=_nbytes(src))
    _check(_lib.kvz_fp8_pack_pages(_ptr(src), _ptr(dst), src.shape[0], src.shape[2],
                                   _stream(stream)))


def _fp8_args(q, out, fmt, block_table, seq_lens, n_comp_pages, tail, sm_scale, k_scale, v_scale,
              workspace, splits, num_kv_heads, n_phys, arena=None, meta=None, bases=None,
              pages=None):
    _check_attn_common(q, out, block_table, seq_lens, n_comp_pages, workspace, num_kv_heads,
                       tail=tail, tail_dtype=_torch().uint8, tail_bytes_per_value=1)
    bsz, hq, hd = q.shape
    return Fp8AttnArgs(
        q=q.data_ptr(), out=out.data_ptr(), arena=None if arena is None else arena.data_ptr(),
        arena_bytes=0 if arena is None else arena.numel() * arena.element_size(),
        meta=None if meta is None else meta.data_ptr(),
        bases=None if bases is None else bases.data_ptr(),
        pages=None if pages is None else pages.data_ptr(), n_phys_pages=n_phys,
        block_table=block_table.data_ptr(), seq_lens=seq_lens.data_ptr(),
        n_comp_pages=n_comp_pages.data_ptr(), tail=None if tail is None else tail.data_ptr(),
        batch=bsz, num_q_heads=hq, num_kv_heads=num_kv_heads, head_dim=hd, page_size=16,
        max_pages=block_table.shape[1], splits=splits, format=fmt, sm_scale=sm_scale,
        k_scale=k_scale, v_scale=v_scale, workspace=workspace.data_ptr(),
        workspace_bytes=workspace.numel() * workspace.element_size())


def kvz_fp8_decode_attention(q, out, fmt: int, arena, meta, bases, block_table, seq_lens,
                             n_comp_pages, tail, sm_scale: float, k_scale: float, v_scale: float,
                             workspace, splits: int = 0, stream=None) -> None:
    """Fused attention over FP8 tiles.  meta [n_phys,Hkv,2,8] uint8; bases [Hkv,2,2,128] uint8;
    tail [B,2,Hkv,16,128] uint8 (FP8) or None."""
    _check_meta(meta)
    _dev("arena", arena)
    _dev("bases", bases, min_bytes=meta.shape[1] * 512)
    a = _fp8_args(q, out, fmt, block_table, seq_lens, n_comp_pages, tail, sm_scale, k_scale,
                  v_scale, workspace, splits, meta.shape[1], meta.shape[0], arena=arena,
                  meta=meta, bases=bases)
    _check(_lib.kvz_fp8_decode_attention(ctypes.byref(a), _stream(stream)))


def kvz_fp8_raw_decode_attention(q, out, fmt: int, pages, block_table, seq_lens, n_comp_pages,
                                 tail, sm_scale: float, k_scale: float, v_scale: float,
                                 workspace, num_kv_heads: int, splits: int = 0,
                                 stream=None) -> None:
    """The FP8 baseline: pages [n_phys,2,Hkv,2048] uint8 (kvz_fp8_pack_pages)."""
    _dev("pages", pages, min_bytes=pages.shape[0] * 2 * num_kv_heads * 2048)
    a = _fp8_args(q, out, fmt, block_table, seq_lens, n_comp_pages, tail, sm_scale, k_scale,
                  v_scale, workspace, splits, num_kv_heads, pages.shape[0], pages=pages)
    _check(_lib.kvz_fp8_raw_decode_attention(ctypes.byref(a), _stream(stream)))


def kvz_stream_read(buf, sink, workgroups: int = 0, stream=None) -> None:
    _dev("buf", buf)
    _dev("sink", sink)
    _check(_lib.kvz_stream_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink),
                                workgroups, _stream(stream)))


# ---------------------------------------------------------------------------------------------
# record builders (host side marshalling of the C structs)
# ---------------------------------------------------------------------------------------------
def encode_items(src_ptrs, dst_ptrs, src_stride, kinds) -> np.ndarray:
    """kvz_encode_item records as a uint8 array (copy it to the device before the call)."""
    n = len(src_ptrs)
    rec = np.zeros(n, dtype=ENCODE_ITEM_DTYPE)
    rec["src"] = np.asarray(src_ptrs, dtype=np.uint64)
    rec["dst"] = np.asarray(dst_ptrs, dtype=np.uint64)
    rec["src_stride"] = src_stride
    rec["kind"] = np.asarray(kinds, dtype=np.uint32)
    return rec.view(np.uint8)


def gaac_items(src_ptrs, dst_ptrs, src_stride, kinds, bases_ptrs) -> np.ndarray:
    """kvz_gaac_item records as a uint8 array (copy it to the device before the call)."""
    n = len(src_ptrs)
    rec = np.zeros(n, dtype=GAAC_ITEM_DTYPE)
    rec["src"] = np.asarray(src_ptrs, dtype=np.uint64)
    rec["dst"] = np.asarray(dst_ptrs, dtype=np.uint64)
    rec["src_stride"] = src_stride
    rec["kind"] = np.asarray(kinds, dtype=np.uint32)
    rec["bases"] = np.asarray(bases_ptrs, dtype=np.uint64)
    return rec.view(np.uint8)


def block_refs(meta_ptrs, blocks, kinds) -> np.ndarray:
    n = len(meta_ptrs)
    rec = np.zeros(n, dtype=BLOCK_REF_DTYPE)
    rec["meta"] = np.asarray(meta_ptrs, dtype=np.uint64)
    rec["block"] = np.asarray(blocks, dtype=np.uint32)
    rec["kind"] = np.asarray(kinds, dtype=np.uint32)
    return rec.view(np.uint8)
