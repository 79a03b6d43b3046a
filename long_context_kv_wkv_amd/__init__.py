"""Python binding of the MI355X Compressor library (libcompressor.so).

Argument marshalling only: torch tensors are checked for device, dtype and
contiguity and passed to the C ABI of include/compressor.h as raw device
pointers, together with the current HIP stream.  Every step of the operator
runs in the library's HIP kernels; if the library is not built, every call
raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcompressor.so")

CMP_OK = 0
STATUS = {0: "CMP_OK", 1: "CMP_ERR_NULLPTR", 2: "CMP_ERR_INVALID", 3: "CMP_ERR_UNSUPPORTED",
          4: "CMP_ERR_WORKSPACE", 5: "CMP_ERR_OUT_ROWS", 6: "CMP_ERR_HIP"}
DEVERR_TABLE, DEVERR_START_POS, DEVERR_SEQLEN, DEVERR_OUT_ROWS, DEVERR_SLOT = 1, 2, 4, 8, 16

EXPORTS = ("compressor_prefill_workspace_size", "compressor_decode_workspace_size",
           "compressor_pack_weights", "compressor_state_init", "compressor_state_reset",
           "compressor_prefill", "compressor_decode", "compressor_last_device_error",
           "compressor_status_str", "compressor_timing_enable", "compressor_timing_query",
           "compressor_epilog", "compressor_set_prefill_tile_rows", "nsa_compress_with_cache",
           "compressor_decode_noalloc")
NSA_BF16, NSA_F16 = 0, 1
NSA_LAYOUT_PAGED, NSA_LAYOUT_TND = 0, 1
NSA_DEVERR_SLOT, NSA_DEVERR_TABLE, NSA_DEVERR_SEQLEN = 1, 2, 4


class CompressorError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {STATUS.get(status, status)}")
        self.status = status


class Shape(ctypes.Structure):
    _fields_ = [("ratio", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("hidden", ctypes.c_int32), ("rope_head_dim", ctypes.c_int32),
                ("rotate", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("num_blocks", ctypes.c_int32), ("table_stride", ctypes.c_int32)]

    @property
    def coff(self) -> int:
        return 2 if self.ratio == 4 else 1


class Args(ctypes.Structure):
    _fields_ = [("x", ctypes.c_void_p), ("T", ctypes.c_int32), ("batch", ctypes.c_int32),
                ("cu_seqlens", ctypes.c_void_p), ("seqused", ctypes.c_void_p),
                ("start_pos", ctypes.c_void_p), ("kv_state", ctypes.c_void_p),
                ("score_state", ctypes.c_void_p), ("kv_block_table", ctypes.c_void_p),
                ("state_block_table", ctypes.c_void_p), ("w_packed", ctypes.c_void_p),
                ("ape", ctypes.c_void_p), ("norm_weight", ctypes.c_void_p),
                ("hadamard", ctypes.c_void_p), ("sin", ctypes.c_void_p), ("cos", ctypes.c_void_p),
                ("out", ctypes.c_void_p), ("out_rows", ctypes.c_int32),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t)]


class NsaShape(ctypes.Structure):
    _fields_ = [("head_num", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("compress_block_size", ctypes.c_int32), ("compress_stride", ctypes.c_int32),
                ("page_block_size", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("layout", ctypes.c_int32)]


class NsaArgs(ctypes.Structure):
    _fields_ = [("input", ctypes.c_void_p), ("weight", ctypes.c_void_p),
                ("slot_mapping", ctypes.c_void_p), ("act_seq_len", ctypes.c_void_p),
                ("block_table", ctypes.c_void_p), ("batch", ctypes.c_int32),
                ("table_stride", ctypes.c_int32), ("num_blocks", ctypes.c_int32),
                ("T", ctypes.c_int64), ("output_cache", ctypes.c_void_p),
                ("result_len", ctypes.c_int64), ("device_error", ctypes.c_void_p)]


_lib = None


def library():
    """Load libcompressor.so (built in-tree); raise if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"HIP library not built: {LIB_PATH} (run __graft_entry__.build())")
        lib = ctypes.CDLL(LIB_PATH)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        sp, ap = ctypes.POINTER(Shape), ctypes.POINTER(Args)
        sig = {
            "compressor_prefill_workspace_size": (sp, i32, i32, i32, ctypes.POINTER(sz)),
            "compressor_decode_workspace_size": (sp, i32, i32, ctypes.POINTER(sz)),
            "compressor_pack_weights": (sp, vp, vp, vp, vp),
            "compressor_state_init": (sp, vp, vp, vp),
            "compressor_state_reset": (sp, vp, vp, vp, vp, vp, i32, i32, vp, vp),
            "compressor_prefill": (sp, ap, vp),
            "compressor_decode": (sp, ap, vp),
            "compressor_decode_noalloc": (sp, ap, vp, vp),
            "compressor_last_device_error": (vp, vp, ctypes.POINTER(i32)),
            "compressor_timing_enable": (i32,),
            "compressor_set_prefill_tile_rows": (i32,),
            "compressor_timing_query": (ctypes.c_char_p, ctypes.POINTER(i32),
                                        ctypes.POINTER(ctypes.c_double)),
            "compressor_epilog": (vp, i32, i32, vp, vp, vp, ctypes.c_int64, vp, vp),
            "nsa_compress_with_cache": (ctypes.POINTER(NsaShape), ctypes.POINTER(NsaArgs), vp),
        }
        for name, argt in sig.items():
            fn = getattr(lib, name)
            fn.argtypes = list(argt)
            fn.restype = ctypes.c_int
        lib.compressor_status_str.argtypes = [ctypes.c_int]
        lib.compressor_status_str.restype = ctypes.c_char_p
        _lib = lib
    return _lib


def _check(fn: str, status: int):
    if status != CMP_OK:
        raise CompressorError(fn, status)


# --------------------------------------------------------------------------
# marshalling helpers
# --------------------------------------------------------------------------
def _dev(t: Optional[torch.Tensor], dtype, name: str):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def make_shape(ratio: int, head_dim: int, hidden: int, rotate: bool, block_size: int,
               num_blocks: int, table_stride: int, rope_head_dim: int = 64) -> Shape:
    return Shape(ratio, head_dim, hidden, rope_head_dim, int(bool(rotate)), block_size,
                 num_blocks, table_stride)


def compressor_prefill_workspace_size(shape: Shape, T: int, batch: int, out_rows: int) -> int:
    n = ctypes.c_size_t(0)
    _check("compressor_prefill_workspace_size",
           library().compressor_prefill_workspace_size(ctypes.byref(shape), T, batch, out_rows,
                                                        ctypes.byref(n)))
    return n.value


def compressor_decode_workspace_size(shape: Shape, batch: int, out_rows: int) -> int:
    n = ctypes.c_size_t(0)
    _check("compressor_decode_workspace_size",
           library().compressor_decode_workspace_size(ctypes.byref(shape), batch, out_rows,
                                                      ctypes.byref(n)))
    return n.value


def compressor_pack_weights(shape: Shape, wkv: torch.Tensor, wgate: torch.Tensor,
                            w_packed: torch.Tensor, stream=None) -> None:
    bf = torch.bfloat16
    _check("compressor_pack_weights", library().compressor_pack_weights(
        ctypes.byref(shape), _dev(wkv, bf, "wkv"), _dev(wgate, bf, "wgate"),
        _dev(w_packed, bf, "w_packed"), _stream(stream)))


def compressor_state_init(shape: Shape, kv_state: torch.Tensor, score_state: torch.Tensor,
                          stream=None) -> None:
    f = torch.float32
    _check("compressor_state_init", library().compressor_state_init(
        ctypes.byref(shape), _dev(kv_state, f, "kv_state"), _dev(score_state, f, "score_state"),
        _stream(stream)))


def compressor_state_reset(shape: Shape, kv_state, score_state, kv_block_table,
                           state_block_table, rows: torch.Tensor, device_error=None,
                           stream=None) -> None:
    """Refill with kv 0 / score -inf every ring block that table rows `rows`
    name; device_error (int32 [1], optional) receives CMP_DEVERR_TABLE for
    a row or table entry out of range (skipped)."""
    f, i = torch.float32, torch.int32
    _check("compressor_state_reset", library().compressor_state_reset(
        ctypes.byref(shape), _dev(kv_state, f, "kv_state"), _dev(score_state, f, "score_state"),
        _dev(kv_block_table, i, "kv_block_table"), _dev(state_block_table, i, "state_block_table"),
        _dev(rows, i, "rows"), int(rows.numel()), int(state_block_table.shape[0]),
        _dev(device_error, i, "device_error"), _stream(stream)))


def check_sizes(shape: Shape, *, x, batch, kv_state, score_state, state_block_table, w_packed,
                ape, norm_weight, sin, cos, out, cu_seqlens=None, seqused=None, start_pos=None,
                kv_block_table=None, hadamard=None, **_) -> None:
    """Raise ValueError unless every tensor has the size the C ABI reads or
    writes for `shape` (the library sees plain pointers and cannot check)."""
    r, D, H, coff = shape.ratio, shape.head_dim, shape.hidden, shape.coff
    B = int(batch)
    T = int(x.shape[0])
    out_rows = int(out.shape[0])

    def need(t, dims, name):
        if t is not None and tuple(t.shape) != tuple(dims):
            raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(dims)}")

    need(x, (T, H), "x")
    need(w_packed, (2 * coff * D, H), "w_packed")
    need(ape, (r, coff * D), "ape")
    need(norm_weight, (D,), "norm_weight")
    need(out, (out_rows, D), "out")
    if out_rows > 0:
        need(sin, (out_rows, shape.rope_head_dim), "sin")
        need(cos, (out_rows, shape.rope_head_dim), "cos")
    if shape.rotate:
        if hadamard is None:
            raise ValueError("hadamard is required when rotate is set")
        need(hadamard, (D, D), "hadamard")
    pool = (shape.num_blocks, shape.block_size, coff * D)
    need(kv_state, pool, "kv_state")
    need(score_state, pool, "score_state")
    for name, tab in (("state_block_table", state_block_table), ("kv_block_table", kv_block_table)):
        if tab is not None and (tab.dim() != 2 or tab.shape[0] < B or
                                tab.shape[1] != shape.table_stride):
            raise ValueError(f"{name}: shape {tuple(tab.shape)}, expected "
                             f"[>= {B}, {shape.table_stride}]")
    need(cu_seqlens, (B + 1,), "cu_seqlens")
    need(seqused, (B,), "seqused")
    need(start_pos, (B,), "start_pos")


def make_args(*, x, batch, kv_state, score_state, state_block_table, w_packed, ape, norm_weight,
              sin, cos, out, workspace, cu_seqlens=None, seqused=None, start_pos=None,
              kv_block_table=None, hadamard=None, shape: Optional[Shape] = None) -> Args:
    """Marshal the tensors of one call; with `shape`, their sizes are checked
    against it first (check_sizes)."""
    if shape is not None:
        check_sizes(shape, x=x, batch=batch, kv_state=kv_state, score_state=score_state,
                    state_block_table=state_block_table, w_packed=w_packed, ape=ape,
                    norm_weight=norm_weight, sin=sin, cos=cos, out=out, cu_seqlens=cu_seqlens,
                    seqused=seqused, start_pos=start_pos, kv_block_table=kv_block_table,
                    hadamard=hadamard)
    bf, f, i = torch.bfloat16, torch.float32, torch.int32
    if workspace is not None and workspace.dtype != torch.uint8:
        raise ValueError("workspace must be a uint8 tensor")
    return Args(
        x=_dev(x, bf, "x"), T=int(x.shape[0]), batch=int(batch),
        cu_seqlens=_dev(cu_seqlens, i, "cu_seqlens"), seqused=_dev(seqused, i, "seqused"),
        start_pos=_dev(start_pos, i, "start_pos"), kv_state=_dev(kv_state, f, "kv_state"),
        score_state=_dev(score_state, f, "score_state"),
        kv_block_table=_dev(kv_block_table, i, "kv_block_table"),
        state_block_table=_dev(state_block_table, i, "state_block_table"),
        w_packed=_dev(w_packed, bf, "w_packed"), ape=_dev(ape, f, "ape"),
        norm_weight=_dev(norm_weight, bf, "norm_weight"), hadamard=_dev(hadamard, bf, "hadamard"),
        sin=_dev(sin, bf, "sin"), cos=_dev(cos, bf, "cos"), out=_dev(out, bf, "out"),
        out_rows=int(out.shape[0]), workspace=_dev(workspace, torch.uint8, "workspace"),
        workspace_bytes=0 if workspace is None else int(workspace.numel()))


def compressor_prefill(shape: Shape, args: Args, stream=None) -> None:
    _check("compressor_prefill",
           library().compressor_prefill(ctypes.byref(shape), ctypes.byref(args), _stream(stream)))


def compressor_decode(shape: Shape, args: Args, stream=None) -> None:
    _check("compressor_decode",
           library().compressor_decode(ctypes.byref(shape), ctypes.byref(args), _stream(stream)))


def compressor_decode_noalloc(shape: Shape, args: Args, device_error: torch.Tensor = None,
                              stream=None) -> None:
    """compressor_decode in the library's per-device scratch: args.workspace
    is ignored; device_error (int32 [1], optional) receives the call's
    device error bits (the caller clears it)."""
    _check("compressor_decode_noalloc", library().compressor_decode_noalloc(
        ctypes.byref(shape), ctypes.byref(args), _dev(device_error, torch.int32, "device_error"),
        _stream(stream)))


def compressor_last_device_error(workspace: torch.Tensor, stream=None) -> int:
    code = ctypes.c_int32(0)
    _check("compressor_last_device_error", library().compressor_last_device_error(
        _dev(workspace, torch.uint8, "workspace"), _stream(stream), ctypes.byref(code)))
    return code.value


def compressor_status_str(status: int) -> str:
    return library().compressor_status_str(status).decode()


def compressor_set_prefill_tile_rows(rows: int) -> None:
    """Prefill projection tile height for later calls: 0 = automatic (256,
    or 128 for calls too short to fill the device), 128 or 256 = forced."""
    _check("compressor_set_prefill_tile_rows", library().compressor_set_prefill_tile_rows(int(rows)))


def compressor_timing_enable(on) -> None:
    """True / 1: time every launch; 2: only the projection GEMM; False / 0: stop."""
    mode = 1 if on is True else int(on)
    _check("compressor_timing_enable", library().compressor_timing_enable(mode))


def compressor_timing_query(kernel: str):
    """(launches, total milliseconds) of `kernel` since timing was enabled."""
    n = ctypes.c_int32(0)
    ms = ctypes.c_double(0.0)
    _check("compressor_timing_query", library().compressor_timing_query(
        kernel.encode(), ctypes.byref(n), ctypes.byref(ms)))
    return n.value, ms.value


def compressor_epilog(rows: torch.Tensor, slot_mapping: torch.Tensor, cache: torch.Tensor,
                      cache_scale: torch.Tensor, device_error: torch.Tensor = None,
                      stream=None) -> None:
    """rows bf16 [n, D]; slot_mapping int32 [n] (-1: no slot); cache uint8
    [num_slots, D] (E4M3 codes) and cache_scale fp32 [num_slots, D / 128],
    both updated in place; device_error an int32 [1] word the kernel ORs
    DEVERR_SLOT into."""
    n, d = rows.shape
    if slot_mapping.numel() != n or cache.dim() != 2 or cache.shape[1] != d:
        raise ValueError("compressor_epilog: shapes of rows, slot_mapping and cache disagree")
    if cache_scale.shape != (cache.shape[0], d // 128):
        raise ValueError("compressor_epilog: cache_scale must be [num_slots, D / 128]")
    _check("compressor_epilog", library().compressor_epilog(
        _dev(rows, torch.bfloat16, "rows"), n, d, _dev(slot_mapping, torch.int32, "slot_mapping"),
        _dev(cache, torch.uint8, "cache"), _dev(cache_scale, torch.float32, "cache_scale"),
        int(cache.shape[0]), _dev(device_error, torch.int32, "device_error"), _stream(stream)))


# --------------------------------------------------------------------------
# NSA KV compression (include/nsa_compress.h)
# --------------------------------------------------------------------------
def make_nsa_shape(head_num: int, head_dim: int, compress_block_size: int, compress_stride: int,
                   page_block_size: int, dtype: int, layout: int) -> NsaShape:
    return NsaShape(head_num, head_dim, compress_block_size, compress_stride, page_block_size,
                    dtype, layout)


def nsa_compress_with_cache(shape: NsaShape, *, input: torch.Tensor, weight: torch.Tensor,
                            slot_mapping: torch.Tensor, act_seq_len: torch.Tensor,
                            output_cache: torch.Tensor, block_table: torch.Tensor = None,
                            device_error: torch.Tensor = None, stream=None) -> None:
    """input / weight / output_cache: bf16 or fp16 tensors (their codes);
    slot_mapping int32 [B]; act_seq_len int64 [B]; block_table int32
    [B, stride] for the paged layout; device_error an int32 [1] word the
    kernel ORs NSA_DEVERR_* bits into."""
    dt = torch.float16 if shape.dtype == NSA_F16 else torch.bfloat16
    paged = shape.layout == NSA_LAYOUT_PAGED
    N, D, cbs = shape.head_num, shape.head_dim, shape.compress_block_size
    B = int(slot_mapping.numel())
    # sizes the kernel reads or writes (it sees plain pointers)
    tok = (shape.page_block_size, N, D) if paged else (N, D)
    if tuple(input.shape[1:]) != tok:
        raise ValueError(f"input: shape {tuple(input.shape)}, expected [*, {', '.join(map(str, tok))}]")
    if tuple(weight.shape) != (cbs, N):
        raise ValueError(f"weight: shape {tuple(weight.shape)}, expected ({cbs}, {N})")
    if tuple(output_cache.shape[1:]) != (N, D):
        raise ValueError(f"output_cache: shape {tuple(output_cache.shape)}, expected [*, {N}, {D}]")
    if act_seq_len.numel() != B:
        raise ValueError("act_seq_len and slot_mapping must both have one entry per batch")
    if paged and (block_table is None or block_table.dim() != 2 or block_table.shape[0] != B):
        raise ValueError("block_table must be [batch, table_stride] for the paged layout")
    args = NsaArgs(_dev(input, dt, "input"), _dev(weight, dt, "weight"),
                   _dev(slot_mapping, torch.int32, "slot_mapping"),
                   _dev(act_seq_len, torch.int64, "act_seq_len"),
                   _dev(block_table, torch.int32, "block_table") if paged else None,
                   int(slot_mapping.numel()),
                   int(block_table.shape[1]) if paged else 0,
                   int(input.shape[0]) if paged else 0,
                   0 if paged else int(input.shape[0]),
                   _dev(output_cache, dt, "output_cache"), int(output_cache.shape[0]),
                   _dev(device_error, torch.int32, "device_error"))
    _check("nsa_compress_with_cache",
           library().nsa_compress_with_cache(ctypes.byref(shape), ctypes.byref(args),
                                             _stream(stream)))
