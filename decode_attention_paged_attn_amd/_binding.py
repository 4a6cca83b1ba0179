"""ctypes binding of ``include/paged_attn.h``.

Argument marshalling only: tensors are checked for dtype, device, shape and
layout, then their device pointers go to the C ABI together with torch's
current HIP stream.  Output and workspace buffers are allocated with torch
when the caller does not pass them.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libpagedattn.so"
_lock = threading.Lock()
_lib = None

HEAD_DIM = 128
BLOCK_SIZE = 16

_c_int = ctypes.c_int
_c_i64 = ctypes.c_int64
_c_size = ctypes.c_size_t
_c_float = ctypes.c_float
_vp = ctypes.c_void_p

class PdaLayout(ctypes.Structure):
    """pda_layout of include/paged_attn.h."""
    _fields_ = [("header_offset", ctypes.c_size_t), ("lse_offset", ctypes.c_size_t),
                ("o_offset", ctypes.c_size_t), ("total_bytes", ctypes.c_size_t),
                ("n_runs", ctypes.c_int), ("n_slots", ctypes.c_int),
                ("unit_tokens", ctypes.c_int)]


# name -> (restype, argtypes); mirrors include/paged_attn.h
_SIGNATURES = {
    "pda_workspace_size": (_c_int, [_c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
                                    ctypes.POINTER(_c_size)]),
    "paged_decode_attn_workspace_size": (_c_int, [_c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
                                                  ctypes.POINTER(_c_size)]),
    "pda_workspace_layout": (_c_int, [_c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
                                      _c_int, ctypes.POINTER(PdaLayout)]),
    "paged_decode_attn": (_c_int, [_vp, _vp, _vp, _vp, _vp, _c_i64, _vp, _c_int, _c_int, _c_int,
                                   _c_int, _c_int, _c_i64, _c_int, _c_float, _c_int, _vp, _vp,
                                   _c_size, _vp]),
    "paged_decode_attn_noalloc": (_c_int, [_vp, _vp, _vp, _vp, _vp, _c_i64, _vp, _c_int, _c_int,
                                           _c_int, _c_int, _c_int, _c_i64, _c_int, _c_float,
                                           _c_int, _vp, _vp]),
    "paged_decode_attn_partial": (_c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _c_i64, _vp, _c_int,
                                           _c_int, _c_int, _c_int, _c_int, _c_i64, _c_int,
                                           _c_float, _c_int, _vp, _c_size, _vp]),
    "paged_decode_attn_fp8": (_c_int, [_vp, _vp, _vp, _vp, _vp, _c_i64, _vp, _c_int, _c_int,
                                       _c_int, _c_int, _c_int, _c_i64, _c_int, _c_float,
                                       _c_float, _c_float, _c_int, _vp, _vp, _c_size, _vp]),
    "paged_decode_attn_partial_fp8": (_c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _c_i64, _vp, _c_int,
                                               _c_int, _c_int, _c_int, _c_int, _c_i64, _c_int,
                                               _c_float, _c_float, _c_float, _c_int, _vp, _c_size,
                                               _vp]),
    "merge_partials": (_c_int, [_vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _vp]),
    "paged_kv_append": (_c_int, [_vp, _vp, _vp, _vp, _vp, _c_i64, _vp, _c_int, _c_int, _c_int,
                                 _c_int, _c_i64, _c_int, _vp]),
    "pda_multi_query_workspace_size": (_c_int, [_c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
                                                _c_int, _c_int, ctypes.POINTER(_c_size)]),
    "paged_multi_query_attn": (_c_int, [_vp, _vp, _vp, _vp, _c_int, _vp, _vp, _vp, _c_i64, _vp,
                                        _c_int, _c_int, _c_int, _c_int, _c_int, _c_i64, _c_int,
                                        _c_float, _c_int, _c_int, _vp, _c_size, _vp]),
    "paged_multi_query_attn_partial": (_c_int, [_vp, _vp, _vp, _vp, _c_int, _vp, _vp, _vp, _c_i64,
                                                _vp, _c_int, _c_int, _c_int, _c_int, _c_int,
                                                _c_i64, _c_int, _c_float, _c_int, _c_int, _vp,
                                                _c_size, _vp]),
    "paged_multi_query_attn_fp8": (_c_int, [_vp, _vp, _vp, _vp, _c_int, _vp, _vp, _vp, _c_i64,
                                            _vp, _c_int, _c_int, _c_int, _c_int, _c_int, _c_i64,
                                            _c_int, _c_float, _c_float, _c_float, _c_int, _c_int,
                                            _vp, _c_size, _vp]),
    "paged_multi_query_attn_partial_fp8": (_c_int, [_vp, _vp, _vp, _vp, _c_int, _vp, _vp, _vp,
                                                    _c_i64, _vp, _c_int, _c_int, _c_int, _c_int,
                                                    _c_int, _c_i64, _c_int, _c_float, _c_float,
                                                    _c_float, _c_int, _c_int, _vp, _c_size, _vp]),
    "paged_kv_append_fp8": (_c_int, [_vp, _vp, _vp, _vp, _vp, _c_i64, _vp, _c_int, _c_int, _c_int,
                                     _c_int, _c_i64, _c_int, _c_float, _c_float, _vp]),
    "paged_decode_attn_append": (_c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _c_i64, _vp, _c_int,
                                          _c_int, _c_int, _c_int, _c_int, _c_i64, _c_int,
                                          _c_float, _c_int, _vp, _vp, _c_size, _vp]),
    "paged_decode_attn_append_fp8": (_c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _c_i64, _vp,
                                              _c_int, _c_int, _c_int, _c_int, _c_int, _c_i64,
                                              _c_int, _c_float, _c_float, _c_float, _c_int, _vp,
                                              _vp, _c_size, _vp]),
    "pda_stream_read": (_c_int, [_vp, _c_size, _vp, _c_int, _vp]),
    "pda_lds_probe": (_c_int, [_c_int, _vp, _c_int, _c_int, _vp]),
    "pda_last_error": (ctypes.c_char_p, []),
    "pda_version": (ctypes.c_char_p, []),
}

STATUS = {0: "PDA_OK", 1: "PDA_EINVAL", 2: "PDA_EUNSUPPORTED", 3: "PDA_EHIP"}


class PdaError(RuntimeError):
    """A non-zero status from the C ABI, with the library's message."""

    def __init__(self, code, message):
        super().__init__(f"{STATUS.get(code, code)}: {message}")
        self.code = code


def library_path():
    return os.environ.get("PDA_LIBRARY", os.path.join(_HERE, _LIB_NAME))


def load_library():
    """Load ``libpagedattn.so`` (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is None:
            path = library_path()
            if not os.path.exists(path):
                raise RuntimeError(
                    f"{path} is missing: build the HIP library first "
                    "(python -m decode_attention_paged_attn_amd.build_lib)")
            lib = ctypes.CDLL(path)
            for name, (res, args) in _SIGNATURES.items():
                fn = getattr(lib, name)
                fn.restype = res
                fn.argtypes = args
            _lib = lib
        return _lib


def _check(rc):
    if rc != 0:
        msg = load_library().pda_last_error().decode(errors="replace")
        raise PdaError(rc, msg)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


_ws_cache = {}


def workspace_size(B, Hq, Hkv, max_blocks_per_seq, partition_tokens=0, D=HEAD_DIM,
                   block_size=BLOCK_SIZE, device=None):
    """Bytes of workspace for this call shape on the current (or given) device."""
    dev = torch.cuda.current_device() if device is None and torch.cuda.is_available() else device
    key = (B, Hq, Hkv, max_blocks_per_seq, partition_tokens, D, block_size, dev)
    n = _ws_cache.get(key)
    if n is None:
        c = _c_size(0)
        _check(load_library().pda_workspace_size(B, Hq, Hkv, D, block_size, max_blocks_per_seq,
                                                 partition_tokens, ctypes.byref(c)))
        n = _ws_cache[key] = int(c.value)
    return n


def decode_workspace_size(B, Hq, max_blocks_per_seq, partition_tokens=0, D=HEAD_DIM,
                          block_size=BLOCK_SIZE):
    """Bytes of decode workspace for any supported KV-head count of Hq query heads
    (paged_decode_attn_workspace_size), on the current device."""
    c = _c_size(0)
    _check(load_library().paged_decode_attn_workspace_size(B, Hq, D, block_size,
                                                           max_blocks_per_seq, partition_tokens,
                                                           ctypes.byref(c)))
    return int(c.value)


def workspace_layout(B, Hq, Hkv, max_blocks_per_seq, partition_tokens=0, D=HEAD_DIM,
                     block_size=BLOCK_SIZE, kv_fp8=False):
    """The workspace layout as a dict (see pda_workspace_layout in the header)."""
    lay = PdaLayout()
    _check(load_library().pda_workspace_layout(B, Hq, Hkv, D, block_size, max_blocks_per_seq,
                                               partition_tokens, int(bool(kv_fp8)),
                                               ctypes.byref(lay)))
    return {name: int(getattr(lay, name)) for name, _ in PdaLayout._fields_}


FP8_DTYPES = (torch.uint8, torch.float8_e4m3fn)


def is_fp8_cache(k_cache):
    """True for a cache of FP8 E4M3 codes (uint8 or float8_e4m3fn storage)."""
    return k_cache.dtype in FP8_DTYPES


def _check_buffer(t, dtype, shape, dev, what):
    """A caller-given output: dtype, shape, contiguity and device, before any launch."""
    if (t.dtype != dtype or tuple(t.shape) != tuple(shape) or not t.is_contiguous()
            or t.device != dev):
        raise ValueError(f"{what} must be contiguous {dtype} {list(shape)} on {dev}")


def _workspace(workspace, nbytes, dev):
    """The caller's workspace (checked), or a new one of nbytes."""
    if workspace is None:
        return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    if workspace.device != dev or not workspace.is_contiguous():
        raise ValueError(f"workspace must be a contiguous buffer on {dev}")
    if workspace.numel() * workspace.element_size() < nbytes:
        raise ValueError(f"workspace needs {nbytes} bytes")
    return workspace


def _check_inputs(q, k_cache, v_cache, block_table, context_lens):
    if q.dtype != torch.float16:
        raise TypeError("q must be float16")
    if not (k_cache.dtype == v_cache.dtype and
            (k_cache.dtype == torch.float16 or k_cache.dtype in FP8_DTYPES)):
        raise TypeError("k_cache and v_cache must both be float16, or both FP8 E4M3 codes "
                        "(uint8 or float8_e4m3fn)")
    if block_table.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise TypeError("block_table and context_lens must be int32")
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a GPU")
    for t in (k_cache, v_cache, block_table, context_lens):
        if t.device != dev:
            raise ValueError("all tensors must be on the same device")
    if q.dim() != 3 or k_cache.dim() != 4 or k_cache.shape != v_cache.shape:
        raise ValueError("q is [B, Hq, D]; k_cache and v_cache are [num_blocks, bs, Hkv, D]")
    if not (q.is_contiguous() and k_cache.is_contiguous() and v_cache.is_contiguous()
            and context_lens.is_contiguous()):
        raise ValueError("q, k_cache, v_cache and context_lens must be contiguous")
    B = q.shape[0]
    if block_table.dim() != 2 or block_table.shape[0] != B or context_lens.shape != (B,):
        raise ValueError("block_table is [B, width] and context_lens is [B]")
    if block_table.stride(1) != 1:
        raise ValueError("block_table rows must be contiguous (stride(1) == 1)")
    if q.shape[2] != k_cache.shape[3]:
        raise ValueError("head dims of q and the caches differ")
    return dev


def _run(partial, q, k_cache, v_cache, block_table, context_lens, scale, out, lse, need_lse,
         partition_tokens, workspace, max_blocks_per_seq, k_scale=None, v_scale=None):
    dev = _check_inputs(q, k_cache, v_cache, block_table, context_lens)
    B, Hq, D = q.shape
    num_blocks, bs, Hkv, _ = k_cache.shape
    width = block_table.shape[1]
    mb = width if max_blocks_per_seq is None else int(max_blocks_per_seq)
    if mb > width:
        raise ValueError("max_blocks_per_seq exceeds the block table width")
    bt_stride = block_table.stride(0) if B > 0 else max(mb, 1)
    workspace = _workspace(workspace,
                           workspace_size(B, Hq, Hkv, mb, partition_tokens, D, bs, dev.index), dev)
    out_dtype = torch.float32 if partial else torch.float16
    if out is None:
        out = torch.empty((B, Hq, D), dtype=out_dtype, device=dev)
    _check_buffer(out, out_dtype, (B, Hq, D), dev, "the output")
    if lse is None and need_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    if lse is not None:
        _check_buffer(lse, torch.float32, (B, Hq), dev, "lse")
    lib = load_library()
    ws_n = workspace.numel() * workspace.element_size()
    if is_fp8_cache(k_cache):
        if k_scale is None or v_scale is None:
            raise ValueError("an FP8 cache needs k_scale and v_scale")
        args = (_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table), bt_stride,
                _ptr(context_lens), B, Hq, Hkv, D, bs, num_blocks, mb, float(scale),
                float(k_scale), float(v_scale), int(partition_tokens))
        if partial:
            rc = lib.paged_decode_attn_partial_fp8(_ptr(out), _ptr(lse), *args, _ptr(workspace),
                                                   ws_n, _stream(dev))
        else:
            rc = lib.paged_decode_attn_fp8(_ptr(out), *args, _ptr(lse), _ptr(workspace), ws_n,
                                           _stream(dev))
    else:
        args = (_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table), bt_stride,
                _ptr(context_lens), B, Hq, Hkv, D, bs, num_blocks, mb, float(scale),
                int(partition_tokens))
        if partial:
            rc = lib.paged_decode_attn_partial(_ptr(out), _ptr(lse), *args, _ptr(workspace), ws_n,
                                               _stream(dev))
        else:
            rc = lib.paged_decode_attn(_ptr(out), *args, _ptr(lse), _ptr(workspace), ws_n,
                                       _stream(dev))
    _check(rc)
    return out, lse


def paged_decode_attn(q, k_cache, v_cache, block_table, context_lens, scale, out=None,
                      lse_out=None, return_lse=False, partition_tokens=0, workspace=None,
                      max_blocks_per_seq=None, k_scale=None, v_scale=None):
    """Decode attention over a paged KV cache; see include/paged_attn.h.

    fp16 caches, or FP8 E4M3 caches (uint8 / float8_e4m3fn) with per-tensor
    ``k_scale`` and ``v_scale``.  Returns ``out`` (fp16 [B, Hq, D]), or
    ``(out, lse)`` when ``return_lse`` or ``lse_out`` is given.
    """
    out, lse = _run(False, q, k_cache, v_cache, block_table, context_lens, scale, out,
                    lse_out, return_lse, partition_tokens, workspace, max_blocks_per_seq,
                    k_scale, v_scale)
    return (out, lse) if (return_lse or lse_out is not None) else out


def paged_decode_attn_noalloc(q, k_cache, v_cache, block_table, context_lens, scale, out,
                              lse_out=None, partition_tokens=0, max_blocks_per_seq=None):
    """paged_decode_attn with the library's fixed device scratch as its workspace
    (paged_decode_attn_noalloc in include/paged_attn.h): fp16 caches; ``out``
    (fp16 [B, Hq, D]) and the optional ``lse_out`` (fp32 [B, Hq]) are the
    caller's, so nothing is allocated here or in the library.  Calls that may
    overlap on one GPU share its scratch and must be ordered by the caller."""
    dev = _check_inputs(q, k_cache, v_cache, block_table, context_lens)
    if is_fp8_cache(k_cache):
        raise TypeError("paged_decode_attn_noalloc takes fp16 caches")
    B, Hq, D = q.shape
    num_blocks, bs, Hkv, _ = k_cache.shape
    width = block_table.shape[1]
    mb = width if max_blocks_per_seq is None else int(max_blocks_per_seq)
    if mb > width:
        raise ValueError("max_blocks_per_seq exceeds the block table width")
    bt_stride = block_table.stride(0) if B > 0 else max(mb, 1)
    _check_buffer(out, torch.float16, (B, Hq, D), dev, "the output")
    if lse_out is not None:
        _check_buffer(lse_out, torch.float32, (B, Hq), dev, "lse")
    _check(load_library().paged_decode_attn_noalloc(
        _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table), bt_stride,
        _ptr(context_lens), B, Hq, Hkv, D, bs, num_blocks, mb, float(scale),
        int(partition_tokens), _ptr(lse_out), _stream(dev)))
    return (out, lse_out) if lse_out is not None else out


def paged_decode_attn_partial(q, k_cache, v_cache, block_table, context_lens, scale, o=None,
                              lse=None, partition_tokens=0, workspace=None,
                              max_blocks_per_seq=None, k_scale=None, v_scale=None):
    """Normalised partial (o fp32 [B, Hq, D], lse fp32 [B, Hq]) of a token range."""
    return _run(True, q, k_cache, v_cache, block_table, context_lens, scale, o, lse, True,
                partition_tokens, workspace, max_blocks_per_seq, k_scale, v_scale)


def stream_read(buf, sink, nontemporal=True):
    """Diagnostic: enqueue a read of all of ``buf`` (a contiguous GPU tensor of a
    multiple of 16 bytes) with the attention kernels' load forms; ``sink`` is a
    one-element int32 GPU tensor that is not written in practice."""
    if buf.device.type != "cuda" or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous GPU tensor")
    if sink.device != buf.device or sink.numel() < 1 or sink.element_size() != 4:
        raise ValueError("sink is one 4-byte element on buf's GPU")
    _check(load_library().pda_stream_read(_ptr(buf), buf.numel() * buf.element_size(),
                                          _ptr(sink), int(bool(nontemporal)),
                                          _stream(buf.device)))


def lds_probe(form, out, iters):
    """Diagnostic: enqueue ``out.numel() // 256`` work-groups of the LDS read
    probe of ``form`` (0 ds_read_b128, 1 ds_read_b64, 2 ds_read_b64_tr_b16,
    3 ds_read_b32) for ``iters`` passes; ``out`` is a contiguous int32 GPU
    tensor of 256 per work-group, filled with each thread's sum."""
    if out.device.type != "cuda" or not out.is_contiguous() or out.element_size() != 4:
        raise ValueError("out must be a contiguous 4-byte GPU tensor")
    if out.numel() % 256:
        raise ValueError("out holds 256 values per work-group")
    _check(load_library().pda_lds_probe(int(form), _ptr(out), out.numel() // 256, int(iters),
                                        _stream(out.device)))


def merge_partials(o_parts, lse_parts, out=None, lse_out=None, return_lse=True):
    """Log-sum-exp merge of R partials: o_parts [R, B, Hq, D], lse_parts [R, B, Hq]."""
    if o_parts.dtype != torch.float32 or lse_parts.dtype != torch.float32:
        raise TypeError("partials must be float32")
    if o_parts.dim() != 4 or lse_parts.shape != o_parts.shape[:3]:
        raise ValueError("o_parts is [R, B, Hq, D] and lse_parts [R, B, Hq]")
    if not (o_parts.is_contiguous() and lse_parts.is_contiguous()):
        raise ValueError("partials must be contiguous")
    if o_parts.device.type != "cuda" or lse_parts.device != o_parts.device:
        raise ValueError("partials must be on one GPU")
    R, B, Hq, D = o_parts.shape
    dev = o_parts.device
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float16, device=dev)
    _check_buffer(out, torch.float16, (B, Hq, D), dev, "out")
    if lse_out is None and return_lse:
        lse_out = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    if lse_out is not None:
        _check_buffer(lse_out, torch.float32, (B, Hq), dev, "lse_out")
    _check(load_library().merge_partials(_ptr(out), _ptr(lse_out), _ptr(o_parts),
                                         _ptr(lse_parts), R, B, Hq, D, _stream(dev)))
    return (out, lse_out) if return_lse else out


def paged_decode_attn_append(q, k_new, v_new, k_cache, v_cache, block_table, context_lens,
                             scale, out=None, lse_out=None, return_lse=False, partition_tokens=0,
                             workspace=None, max_blocks_per_seq=None, k_scale=None, v_scale=None):
    """paged_kv_append then paged_decode_attn in one launch.

    Writes k_new / v_new (fp16 [B, Hkv, D]) into slot context_lens[b] - 1
    (quantised with ``k_scale`` / ``v_scale`` for an FP8 cache) and attends over
    context_lens[b] tokens; the caches and results are bit for bit those of the
    two calls.  Returns ``out`` or ``(out, lse)``.
    """
    dev = _check_inputs(q, k_cache, v_cache, block_table, context_lens)
    fp8 = is_fp8_cache(k_cache)
    if fp8 and (k_scale is None or v_scale is None):
        raise ValueError("an FP8 cache needs k_scale and v_scale")
    B, Hq, D = q.shape
    num_blocks, bs, Hkv, _ = k_cache.shape
    for t in (k_new, v_new):
        _check_buffer(t, torch.float16, (B, Hkv, D), dev, "k_new and v_new")
    width = block_table.shape[1]
    mb = width if max_blocks_per_seq is None else int(max_blocks_per_seq)
    if mb > width:
        raise ValueError("max_blocks_per_seq exceeds the block table width")
    bt_stride = block_table.stride(0) if B > 0 else max(mb, 1)
    workspace = _workspace(workspace,
                           workspace_size(B, Hq, Hkv, mb, partition_tokens, D, bs, dev.index), dev)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float16, device=dev)
    _check_buffer(out, torch.float16, (B, Hq, D), dev, "the output")
    lse = lse_out
    if lse is None and return_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    if lse is not None:
        _check_buffer(lse, torch.float32, (B, Hq), dev, "lse")
    head = (_ptr(out), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
            _ptr(block_table), bt_stride, _ptr(context_lens), B, Hq, Hkv, D, bs, num_blocks, mb,
            float(scale))
    tail = (int(partition_tokens), _ptr(lse), _ptr(workspace),
            workspace.numel() * workspace.element_size(), _stream(dev))
    lib = load_library()
    if fp8:
        _check(lib.paged_decode_attn_append_fp8(*head, float(k_scale), float(v_scale), *tail))
    else:
        _check(lib.paged_decode_attn_append(*head, *tail))
    return (out, lse) if (return_lse or lse_out is not None) else out


def paged_kv_append(k_cache, v_cache, k_new, v_new, block_table, context_lens,
                    max_blocks_per_seq=None, k_scale=None, v_scale=None):
    """Write token ctx_b - 1 of every sequence (k_new, v_new: fp16 [B, Hkv, D]) in place.

    fp16 caches take the rows as they are; FP8 E4M3 caches (uint8 /
    float8_e4m3fn) store their codes quantised with ``k_scale`` / ``v_scale``.
    """
    dev = _check_inputs(k_new, k_cache, v_cache, block_table, context_lens)
    B = k_new.shape[0]
    num_blocks, bs, Hkv, D = k_cache.shape
    for t in (k_new, v_new):
        _check_buffer(t, torch.float16, (B, Hkv, D), dev, "k_new and v_new")
    width = block_table.shape[1]
    mb = width if max_blocks_per_seq is None else int(max_blocks_per_seq)
    if mb > width:
        raise ValueError("max_blocks_per_seq exceeds the block table width")
    bt_stride = block_table.stride(0) if B > 0 else max(mb, 1)
    args = (_ptr(k_cache), _ptr(v_cache), _ptr(k_new), _ptr(v_new), _ptr(block_table), bt_stride,
            _ptr(context_lens), B, Hkv, D, bs, num_blocks, mb)
    lib = load_library()
    if is_fp8_cache(k_cache):
        if k_scale is None or v_scale is None:
            raise ValueError("an FP8 cache needs k_scale and v_scale")
        _check(lib.paged_kv_append_fp8(*args, float(k_scale), float(v_scale), _stream(dev)))
    else:
        _check(lib.paged_kv_append(*args, _stream(dev)))


# --- several query tokens per sequence, and cascade attention ------------------

_mq_ws_cache = {}


def multi_query_workspace_size(S, num_queries, Hq, Hkv, max_blocks_per_seq, partition_tokens=0,
                               D=HEAD_DIM, block_size=BLOCK_SIZE, device=None):
    """Bytes of workspace for a multi-query call of this shape."""
    dev = torch.cuda.current_device() if device is None and torch.cuda.is_available() else device
    key = (S, num_queries, Hq, Hkv, max_blocks_per_seq, partition_tokens, D, block_size, dev)
    n = _mq_ws_cache.get(key)
    if n is None:
        c = _c_size(0)
        _check(load_library().pda_multi_query_workspace_size(
            S, num_queries, Hq, Hkv, D, block_size, max_blocks_per_seq, partition_tokens,
            ctypes.byref(c)))
        n = _mq_ws_cache[key] = int(c.value)
    return n


def _run_mq(partial, q, k_cache, v_cache, block_table, context_lens, query_start, scale, causal,
            out, lse, need_lse, partition_tokens, workspace, max_blocks_per_seq, k_scale=None,
            v_scale=None):
    if q.dtype != torch.float16:
        raise TypeError("q must be float16")
    if not (k_cache.dtype == v_cache.dtype and
            (k_cache.dtype == torch.float16 or k_cache.dtype in FP8_DTYPES)):
        raise TypeError("k_cache and v_cache must both be float16, or both FP8 E4M3 codes "
                        "(uint8 or float8_e4m3fn)")
    if (block_table.dtype != torch.int32 or context_lens.dtype != torch.int32
            or query_start.dtype != torch.int32):
        raise TypeError("block_table, context_lens and query_start must be int32")
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a GPU")
    for t in (k_cache, v_cache, block_table, context_lens, query_start):
        if t.device != dev:
            raise ValueError("all tensors must be on the same device")
    if q.dim() != 3 or k_cache.dim() != 4 or k_cache.shape != v_cache.shape:
        raise ValueError("q is [T, Hq, D]; k_cache and v_cache are [num_blocks, bs, Hkv, D]")
    if not all(t.is_contiguous() for t in (q, k_cache, v_cache, context_lens, query_start)):
        raise ValueError("q, k_cache, v_cache, context_lens and query_start must be contiguous")
    S = context_lens.shape[0]
    if (context_lens.dim() != 1 or block_table.dim() != 2 or block_table.shape[0] != S
            or query_start.shape != (S + 1,)):
        raise ValueError("block_table is [S, width], context_lens [S] and query_start [S + 1]")
    if block_table.stride(1) != 1:
        raise ValueError("block_table rows must be contiguous (stride(1) == 1)")
    T, Hq, D = q.shape
    num_blocks, bs, Hkv, _ = k_cache.shape
    width = block_table.shape[1]
    mb = width if max_blocks_per_seq is None else int(max_blocks_per_seq)
    if mb > width:
        raise ValueError("max_blocks_per_seq exceeds the block table width")
    bt_stride = block_table.stride(0) if S > 0 else max(mb, 1)
    workspace = _workspace(
        workspace, multi_query_workspace_size(S, T, Hq, Hkv, mb, partition_tokens, D, bs,
                                              dev.index), dev)
    out_dtype = torch.float32 if partial else torch.float16
    if out is None:
        out = torch.empty((T, Hq, D), dtype=out_dtype, device=dev)
    _check_buffer(out, out_dtype, (T, Hq, D), dev, "the output")
    if lse is None and need_lse:
        lse = torch.empty((T, Hq), dtype=torch.float32, device=dev)
    if lse is not None:
        _check_buffer(lse, torch.float32, (T, Hq), dev, "lse")
    lib = load_library()
    head = (_ptr(out), _ptr(lse), _ptr(q), _ptr(query_start), T, _ptr(k_cache), _ptr(v_cache),
            _ptr(block_table), bt_stride, _ptr(context_lens), S, Hq, Hkv, D, bs, num_blocks, mb,
            float(scale))
    tail = (int(bool(causal)), int(partition_tokens), _ptr(workspace),
            workspace.numel() * workspace.element_size(), _stream(dev))
    if is_fp8_cache(k_cache):
        if k_scale is None or v_scale is None:
            raise ValueError("an FP8 cache needs k_scale and v_scale")
        fn = (lib.paged_multi_query_attn_partial_fp8 if partial
              else lib.paged_multi_query_attn_fp8)
        _check(fn(*head, float(k_scale), float(v_scale), *tail))
    else:
        fn = lib.paged_multi_query_attn_partial if partial else lib.paged_multi_query_attn
        _check(fn(*head, *tail))
    return out, lse


def paged_multi_query_attn(q, k_cache, v_cache, block_table, context_lens, query_start, scale,
                           causal=True, out=None, lse_out=None, return_lse=False,
                           partition_tokens=0, workspace=None, max_blocks_per_seq=None,
                           k_scale=None, v_scale=None):
    """Several query tokens per sequence over a paged KV cache; see include/paged_attn.h.

    q fp16 [T, Hq, D] with the queries of sequence s in rows
    query_start[s] .. query_start[s+1]-1 (the last tokens of the sequence).
    fp16 caches, or FP8 E4M3 caches with per-tensor ``k_scale`` and ``v_scale``.
    Returns ``out`` (fp16 [T, Hq, D]) or ``(out, lse)``.
    """
    out, lse = _run_mq(False, q, k_cache, v_cache, block_table, context_lens, query_start, scale,
                       causal, out, lse_out, return_lse, partition_tokens, workspace,
                       max_blocks_per_seq, k_scale, v_scale)
    return (out, lse) if (return_lse or lse_out is not None) else out


def paged_multi_query_attn_partial(q, k_cache, v_cache, block_table, context_lens, query_start,
                                   scale, causal=True, o=None, lse=None, partition_tokens=0,
                                   workspace=None, max_blocks_per_seq=None, k_scale=None,
                                   v_scale=None):
    """Normalised partial (o fp32 [T, Hq, D], lse fp32 [T, Hq]) of multi-query attention."""
    return _run_mq(True, q, k_cache, v_cache, block_table, context_lens, query_start, scale,
                   causal, o, lse, True, partition_tokens, workspace, max_blocks_per_seq, k_scale,
                   v_scale)


def cascade_decode_attn(q, k_cache, v_cache, prefix_table, prefix_lens, group_start,
                        suffix_table, suffix_lens, scale, out=None, lse_out=None,
                        return_lse=False, partials=None, k_scale=None, v_scale=None):
    """Decode attention of B requests whose contexts are a shared prefix then a suffix.

    Requests group_start[r] .. group_start[r+1]-1 share prefix r (prefix_table
    row r, prefix_lens[r] tokens); request b continues with suffix_lens[b]
    tokens of suffix_table row b.  Three library calls: the prefix pass with
    every request of a group as a query of its prefix (no mask), the suffix
    pass, and the log-sum-exp merge of the two partials.  ``partials`` may
    pass preallocated (o fp32 [2, B, Hq, D], lse fp32 [2, B, Hq]).  FP8 caches take
    ``k_scale`` and ``v_scale`` as the other calls do.
    """
    B, Hq, D = q.shape
    if partials is None:
        o_parts = torch.empty((2, B, Hq, D), dtype=torch.float32, device=q.device)
        l_parts = torch.empty((2, B, Hq), dtype=torch.float32, device=q.device)
    else:
        o_parts, l_parts = partials
    paged_multi_query_attn_partial(q, k_cache, v_cache, prefix_table, prefix_lens, group_start,
                                   scale, causal=False, o=o_parts[0], lse=l_parts[0],
                                   k_scale=k_scale, v_scale=v_scale)
    paged_decode_attn_partial(q, k_cache, v_cache, suffix_table, suffix_lens, scale,
                              o=o_parts[1], lse=l_parts[1], k_scale=k_scale, v_scale=v_scale)
    res = merge_partials(o_parts, l_parts, out=out, lse_out=lse_out,
                         return_lse=return_lse or lse_out is not None)
    return res
