"""Block-sparse flash-attention forward for AMD Instinct MI355X (gfx950).

A thin ctypes binding over libbsattn.so (C ABI in include/bsattn.h).  Every step of
the computation runs in the library's HIP kernels; this module only checks
tensor properties, allocates outputs and workspace through torch, and passes raw
device pointers and torch's current HIP stream.  If libbsattn.so is missing the
calls raise: there is no fallback path.

    out, lse = fwd(q, k, v, block_mask, block_q, block_k, scale)

q, k, v: [B, H, S, D] CUDA (HIP) tensors, bf16 or fp32, contiguous.
block_mask: [B, H, S/block_q, S/block_k] uint8 or bool on the same device.
Returns out (dtype of q, [B, H, S, D]) and lse (fp32, [B, H, S]).
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libbsattn.so")

BSATTN_F32, BSATTN_BF16 = 0, 1
STATUS = {0: "BSATTN_OK", 1: "BSATTN_ERR_NULL", 2: "BSATTN_ERR_SHAPE",
          3: "BSATTN_ERR_UNSUPPORTED", 4: "BSATTN_ERR_ALIGN", 5: "BSATTN_ERR_WORKSPACE",
          6: "BSATTN_ERR_SCALE", 7: "BSATTN_ERR_ALIAS", 8: "BSATTN_ERR_HIP", 9: "BSATTN_ERR_IO"}


class BsattnError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(msg)
        self.status = status


class TileConfig(ctypes.Structure):
    _fields_ = [("tile_q", ctypes.c_int), ("tile_k", ctypes.c_int),
                ("waves", ctypes.c_int), ("stages", ctypes.c_int)]

    def as_tuple(self):
        return (self.tile_q, self.tile_k, self.waves, self.stages)

    def __repr__(self):
        return "TileConfig(tile_q=%d, tile_k=%d, waves=%d, stages=%d)" % self.as_tuple()


class TuneResult(ctypes.Structure):
    _fields_ = [("id", ctypes.c_int), ("cfg", TileConfig), ("t_mean_s", ctypes.c_double),
                ("t_std_s", ctypes.c_double), ("t_min_s", ctypes.c_double)]


_lib = None


def library():
    """Load libbsattn.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libbsattn.so is not built (%s); run "
                           "`python -m block_sparse_flash_mask_amd.build`" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    p, i32, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    szp = ctypes.POINTER(ctypes.c_size_t)
    cfgp = ctypes.POINTER(TileConfig)
    i32p = ctypes.POINTER(ctypes.c_int)
    sig = {
        "bsattn_version": ([], i32),
        "bsattn_status_string": ([i32], ctypes.c_char_p),
        "bsattn_last_hip_error": ([], i32),
        "bsattn_compact_workspace_size": ([i32, i32, i32, i32, szp], i32),
        "bsattn_compact_mask": ([p, i32, i32, i32, i32, p, p, p, sz, p], i32),
        "bsattn_workspace_size": ([i32, i32, i32, i32, i32, szp], i32),
        "bsattn_fwd": ([p, p, p, p, p, p, i32, i32, i32, i32, i32, i32, f32, i32, p, sz, p], i32),
        "bsattn_fwd_config": ([p, p, p, p, p, p, i32, i32, i32, i32, i32, i32, f32, i32, p, sz,
                               cfgp, p], i32),
        "bsattn_plan": ([p, i32, i32, i32, i32, i32, p, sz, p], i32),
        "bsattn_fwd_noalloc": ([p, p, p, p, p, p, i32, i32, i32, i32, i32, i32, f32, i32, cfgp, p], i32),
        "bsattn_noalloc_max_bytes": ([], sz),
        "bsattn_fwd_planned": ([p, p, p, p, p, i32, i32, i32, i32, i32, i32, f32, i32, p, sz,
                                cfgp, p], i32),
        "bsattn_fwd_compacted": ([p, p, p, p, p, sz, p, p, i32, i32, i32, i32, i32, i32, f32, i32,
                                  cfgp, p], i32),
        "bsattn_list_configs": ([i32, i32, i32, i32, cfgp, i32, i32p], i32),
        "bsattn_autotune": ([p, p, p, p, p, p, i32, i32, i32, i32, i32, i32, f32, i32, p, sz,
                             i32, i32, cfgp, ctypes.POINTER(TuneResult), i32, i32p,
                             ctypes.c_char_p, p], i32),
        "bsattn_plan_elem": ([p, p, i32, i32, i32, i32, i32, i32, p, sz, p], i32),
        "bsattn_fwd_planned_elem": ([p, p, p, p, p, i32, i32, i32, i32, i32, i32, f32, i32, p,
                                     i32, p, sz, cfgp, p], i32),
        "bsattn_fwd_elem": ([p, p, p, p, p, p, i32, p, p, i32, i32, i32, i32, i32, i32, f32, i32,
                             p, sz, cfgp, p], i32),
        "bsattn_list_configs_elem": ([i32, i32, i32, i32, cfgp, i32, i32p], i32),
        "bsattn_fp8_workspace_size": ([i32, i32, i32, i32, i32, i32, szp], i32),
        "bsattn_fwd_fp8": ([p, p, p, p, p, p, i32, i32, i32, i32, i32, i32, f32, p, sz, p], i32),
        "bsattn_fwd_fp8_planned": ([p, p, p, p, p, i32, i32, i32, i32, i32, i32, f32, p, sz, p], i32),
        "bsattn_fwd_fp8_elem": ([p, p, p, p, p, p, i32, p, p, i32, i32, i32, i32, i32, i32, f32, p, sz, p],
                                i32),
        "bsattn_fwd_fp8_planned_elem": ([p, p, p, p, p, i32, i32, i32, i32, i32, i32, f32, p, i32, p, sz, p],
                                        i32),
        "bsattn_bwd_workspace_size": ([i32, i32, i32, i32, i32, szp], i32),
        "bsattn_bwd": ([p, p, p, p, p, p, p, i32, i32, i32, i32, i32, i32, f32, i32, p, p, p, i32, p, sz,
                        p], i32),
        "bsattn_bwd_elem": ([p, p, p, p, p, p, p, p, p, i32, i32, i32, i32, i32, i32, i32, f32, i32, p, p, p,
                             i32, p, sz, p], i32),
        "bsattn_bwd_planned_elem": ([p, p, p, p, p, p, p, p, p, i32, i32, i32, i32, i32, i32, i32, f32, i32, p,
                                     p, p, i32, i32, p, sz, p], i32),
        "bsattn_bwd_plan": ([p, i32, i32, i32, i32, i32, p, sz, p], i32),
        "bsattn_bwd_planned": ([p, p, p, p, p, p, i32, i32, i32, i32, i32, i32, f32, i32, p, p, p, i32, i32,
                                p, sz, p], i32),
        "bsattn_ragged_dot_workspace_size": ([i32, i32, szp], i32),
        "bsattn_ragged_dot": ([p, p, p, p, i32, i32, i32, i32, i32, i32, p, sz, p], i32),
        "bsattn_ragged_plan": ([p, i32, i32, p, sz, p], i32),
        "bsattn_ragged_dot_planned": ([p, p, p, i32, i32, i32, i32, i32, i32, p, sz, p], i32),
        "bsattn_load_tune_cache": ([ctypes.c_char_p], i32),
        "bsattn_tune_lookup": ([i32, i32, i32, i32, i32, i32, i32, ctypes.c_longlong, cfgp], i32),
        "bsattn_clear_tune_cache": ([], None),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def _check(rc):
    if rc != 0:
        lib = library()
        msg = lib.bsattn_status_string(rc).decode()
        if rc == 8:
            msg += " (hipError %d)" % lib.bsattn_last_hip_error()
        raise BsattnError(rc, msg)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _check_tensor(t, name, device, dtypes=None, shape=None, min_bytes=None):
    """Refuse (ValueError / TypeError) a tensor argument that the library could
    not use safely: not a torch tensor, not on `device` (a GPU), not contiguous,
    of another dtype, another shape, or smaller than min_bytes.  Runs before any
    library call, so a refused argument never reaches the device."""
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch tensor" % name)
    if t.device != device:
        raise ValueError("%s must be on %s (it is on %s)" % (name, device, t.device))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtypes is not None and t.dtype not in dtypes:
        raise TypeError("%s must have dtype %s (it has %s)"
                        % (name, " or ".join(str(d) for d in dtypes), t.dtype))
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s (it has %s)" % (name, tuple(shape), tuple(t.shape)))
    if min_bytes is not None and t.numel() * t.element_size() < min_bytes:
        raise ValueError("%s too small: need %d bytes, have %d"
                         % (name, min_bytes, t.numel() * t.element_size()))
    return t


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _keep_alive(stream, *tensors):
    """Tensors this binding allocated and hands to a launch on `stream`: if that
    is not torch's current stream, tell torch's allocator the memory is in use
    there, so it is not reused before the launch has run."""
    if stream is None:
        return
    if not isinstance(stream, torch.cuda.Stream):
        stream = torch.cuda.ExternalStream(int(stream))
    if stream == torch.cuda.current_stream():
        return
    for t in tensors:
        if t is not None:
            t.record_stream(stream)


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return BSATTN_BF16
    if t.dtype == torch.float32:
        return BSATTN_F32
    raise TypeError("q/k/v must be bfloat16 or float32, got %s" % t.dtype)


def _cfg(config):
    if config is None:
        return None
    if isinstance(config, TileConfig):
        return ctypes.byref(config)
    return ctypes.byref(TileConfig(*config))


def default_scale(D):
    """1/sqrt(D) rounded to fp32."""
    return float(torch.tensor(1.0 / math.sqrt(D), dtype=torch.float32))


def _check_inputs(q, k, v):
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor):
            raise TypeError("%s must be a torch tensor" % name)
        if not t.is_cuda:
            raise ValueError("%s must be a GPU tensor" % name)
        if not t.is_contiguous():
            raise ValueError("%s must be contiguous [B, H, S, D]" % name)
        if t.dim() != 4:
            raise ValueError("%s must be 4-D [B, H, S, D]" % name)
    if q.shape != k.shape or q.shape != v.shape:
        raise ValueError("q, k, v must have one shape")
    if not (q.device == k.device == v.device):
        raise ValueError("q, k, v must be on one device")
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k, v must have one dtype")
    return tuple(q.shape)


def _mask_u8(block_mask, device=None, shape=None, name="block_mask"):
    """A uint8 (or bool, viewed as uint8) mask; with device/shape given, also on
    that device with that shape."""
    if not isinstance(block_mask, torch.Tensor):
        raise TypeError("%s must be a torch tensor" % name)
    if block_mask.dtype == torch.bool:
        block_mask = block_mask.view(torch.uint8)
    if block_mask.dtype != torch.uint8:
        raise TypeError("%s must be uint8 or bool" % name)
    if device is None:
        if not block_mask.is_cuda:
            raise ValueError("%s must be a GPU tensor" % name)
        device = block_mask.device
    return _check_tensor(block_mask, name, device, shape=shape)


def _outputs(q, out, lse, out_dtype=None):
    """out [B, H, S, D] (dtype of q unless out_dtype) and lse [B, H, S] fp32 on
    q's device: allocated when None, else checked."""
    B, H, S, D = q.shape
    od = out_dtype or q.dtype
    if out is None:
        out = torch.empty(q.shape, dtype=od, device=q.device)
    else:
        _check_tensor(out, "out", q.device, (od,), (B, H, S, D))
    if lse is None:
        lse = torch.empty((B, H, S), dtype=torch.float32, device=q.device)
    else:
        _check_tensor(lse, "lse", q.device, (torch.float32,), (B, H, S))
    return out, lse


def workspace_size(B, H, S, block_q, block_k):
    n = ctypes.c_size_t(0)
    _check(library().bsattn_workspace_size(B, H, S, block_q, block_k, ctypes.byref(n)))
    return n.value


def compact_workspace_size(B, H, n_q, n_k):
    n = ctypes.c_size_t(0)
    _check(library().bsattn_compact_workspace_size(B, H, n_q, n_k, ctypes.byref(n)))
    return n.value


def _workspace(nbytes, device, workspace, name="workspace"):
    if workspace is None:
        return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)
    return _check_tensor(workspace, name, device, min_bytes=nbytes)


def _mask_shape(q_shape, block_q, block_k):
    B, H, S, _ = q_shape
    if block_q <= 0 or block_k <= 0 or S % block_q or S % block_k:
        raise ValueError("S = %d must be a multiple of block_q = %d and block_k = %d" % (S, block_q, block_k))
    return (B, H, S // block_q, S // block_k)


def fwd(q, k, v, block_mask, block_q, block_k, scale=None, *, out=None, lse=None,
        workspace=None, config=None, stream=None):
    """Block-sparse attention forward; returns (out, lse)."""
    B, H, S, D = _check_inputs(q, k, v)
    block_mask = _mask_u8(block_mask, q.device, _mask_shape(q.shape, block_q, block_k))
    if scale is None:
        scale = default_scale(D)
    out, lse = _outputs(q, out, lse)
    ws = _workspace(workspace_size(B, H, S, block_q, block_k), q.device, workspace)
    _keep_alive(stream, out, lse, ws)
    lib = library()
    rc = lib.bsattn_fwd_config(_ptr(q), _ptr(k), _ptr(v), _ptr(block_mask), _ptr(out), _ptr(lse),
                               B, H, S, D, block_q, block_k, float(scale), _dtype_code(q),
                               _ptr(ws), ws.numel() * ws.element_size(), _cfg(config),
                               _stream(stream))
    _check(rc)
    return out, lse


def fwd_noalloc(q, k, v, block_mask, block_q, block_k, scale, out, lse, *, config=None, stream=None):
    """bsattn_fwd_noalloc: the forward with its plan in the library's fixed
    device array (no allocation by the library; the caller passes out and lse).
    Calls that overlap on one GPU race on that array."""
    B, H, S, D = _check_inputs(q, k, v)
    block_mask = _mask_u8(block_mask, q.device, _mask_shape(q.shape, block_q, block_k))
    _check_tensor(out, "out", q.device, (q.dtype,), q.shape)
    _check_tensor(lse, "lse", q.device, (torch.float32,), q.shape[:3])
    rc = library().bsattn_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(block_mask), _ptr(out), _ptr(lse),
                                      B, H, S, D, block_q, block_k, float(scale), _dtype_code(q), _cfg(config),
                                      _stream(stream))
    _check(rc)
    return out, lse


def noalloc_max_bytes():
    return library().bsattn_noalloc_max_bytes()


def plan(block_mask, S, block_q, block_k, *, workspace=None, stream=None):
    """The mask-dependent step of fwd() on its own: per-row key-block lists and
    the dispatch order, written into a workspace tensor (returned).  The plan
    depends only on the mask and (B, H, S, block_q, block_k): one plan serves
    every fwd_planned() call that shares the mask."""
    block_mask = _mask_u8(block_mask)
    if block_mask.dim() != 4:
        raise ValueError("block_mask must be [B, H, S/block_q, S/block_k]")
    B, H, n_q, n_k = block_mask.shape
    if (n_q * block_q, n_k * block_k) != (S, S):
        raise ValueError("block_mask must be [B, H, S/block_q, S/block_k]")
    ws = _workspace(workspace_size(B, H, S, block_q, block_k), block_mask.device, workspace)
    _keep_alive(stream, ws)
    rc = library().bsattn_plan(_ptr(block_mask), B, H, S, block_q, block_k, _ptr(ws),
                               ws.numel() * ws.element_size(), _stream(stream))
    _check(rc)
    return ws


def fwd_planned(q, k, v, plan_ws, block_q, block_k, scale=None, *, out=None, lse=None,
                config=None, stream=None):
    """The attention kernel alone on a plan from plan(); returns (out, lse)."""
    B, H, S, D = _check_inputs(q, k, v)
    _mask_shape(q.shape, block_q, block_k)
    _workspace(workspace_size(B, H, S, block_q, block_k), q.device, plan_ws, "plan_ws")
    if scale is None:
        scale = default_scale(D)
    out, lse = _outputs(q, out, lse)
    _keep_alive(stream, out, lse)
    rc = library().bsattn_fwd_planned(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, S,
                                      D, block_q, block_k, float(scale), _dtype_code(q),
                                      _ptr(plan_ws), plan_ws.numel() * plan_ws.element_size(),
                                      _cfg(config), _stream(stream))
    _check(rc)
    return out, lse


def compact_mask(block_mask, *, row_ptr=None, col_idx=None, workspace=None, stream=None):
    """CSR lists of active key blocks per mask row.  Returns (row_ptr [R+1],
    col_idx [R*n_k] int32, of which the first row_ptr[-1] entries are valid)."""
    block_mask = _mask_u8(block_mask)
    if block_mask.dim() != 4:
        raise ValueError("block_mask must be [B, H, n_q, n_k]")
    B, H, n_q, n_k = block_mask.shape
    R = B * H * n_q
    dev = block_mask.device
    if row_ptr is None:
        row_ptr = torch.empty(R + 1, dtype=torch.int32, device=dev)
    else:
        _check_tensor(row_ptr, "row_ptr", dev, (torch.int32,), (R + 1,))
    if col_idx is None:
        col_idx = torch.empty(max(R * n_k, 1), dtype=torch.int32, device=dev)
    else:
        _check_tensor(col_idx, "col_idx", dev, (torch.int32,), min_bytes=4 * R * n_k)
    ws = _workspace(compact_workspace_size(B, H, n_q, n_k), dev, workspace)
    _keep_alive(stream, row_ptr, col_idx, ws)
    rc = library().bsattn_compact_mask(_ptr(block_mask), B, H, n_q, n_k, _ptr(row_ptr),
                                       _ptr(col_idx), _ptr(ws), ws.numel() * ws.element_size(),
                                       _stream(stream))
    _check(rc)
    return row_ptr, col_idx


def fwd_compacted(q, k, v, row_ptr, col_idx, block_q, block_k, scale=None, *, out=None,
                  lse=None, config=None, stream=None):
    """The attention kernel alone on CSR lists from compact_mask()."""
    B, H, S, D = _check_inputs(q, k, v)
    _mask_shape(q.shape, block_q, block_k)
    _check_tensor(row_ptr, "row_ptr", q.device, (torch.int32,), (B * H * (S // block_q) + 1,))
    _check_tensor(col_idx, "col_idx", q.device, (torch.int32,))
    if scale is None:
        scale = default_scale(D)
    out, lse = _outputs(q, out, lse)
    _keep_alive(stream, out, lse)
    rc = library().bsattn_fwd_compacted(_ptr(q), _ptr(k), _ptr(v), _ptr(row_ptr), _ptr(col_idx),
                                        col_idx.numel(), _ptr(out), _ptr(lse), B, H, S, D, block_q,
                                        block_k, float(scale), _dtype_code(q), _cfg(config),
                                        _stream(stream))
    _check(rc)
    return out, lse


def _elem_tensors(block_states, partial_index, partial_bits, device=None, shape=None):
    """Check the element-mask tensors (see bsattn.h): uint8 states, int32 tile
    index per block, int32/uint32 bit tiles [n_tiles, block_q, block_k / 32];
    all on `device` (default: that of block_states, a GPU)."""
    for name, t in (("block_states", block_states), ("partial_index", partial_index),
                    ("partial_bits", partial_bits)):
        if not isinstance(t, torch.Tensor):
            raise TypeError("%s must be a torch tensor" % name)
    if device is None:
        if not block_states.is_cuda:
            raise ValueError("block_states must be a GPU tensor")
        device = block_states.device
    if block_states.dim() != 4:
        raise ValueError("block_states must be [B, H, S/block_q, S/block_k]")
    _check_tensor(block_states, "block_states", device, (torch.uint8,), shape)
    _check_tensor(partial_index, "partial_index", device, (torch.int32,), block_states.shape)
    _check_tensor(partial_bits, "partial_bits", device, (torch.int32, torch.uint32))
    if partial_bits.dim() != 3:
        raise ValueError("partial_bits must be [n_tiles, block_q, block_k / 32]")
    return partial_bits.shape[0]


def _check_bits(partial_bits, block_q, block_k):
    if tuple(partial_bits.shape[1:]) != (block_q, block_k // 32):
        raise ValueError("partial_bits must be [n_tiles, block_q, block_k / 32] = [n, %d, %d]"
                         % (block_q, block_k // 32))


def plan_elem(block_states, partial_index, partial_bits, S, block_q, block_k, *, workspace=None,
              stream=None):
    """Plan of an element-level mask (bsattn_plan_elem); returns the workspace."""
    n_tiles = _elem_tensors(block_states, partial_index, partial_bits)
    _check_bits(partial_bits, block_q, block_k)
    B, H, n_q, n_k = block_states.shape
    if (n_q * block_q, n_k * block_k) != (S, S):
        raise ValueError("block_states must be [B, H, S/block_q, S/block_k]")
    ws = _workspace(workspace_size(B, H, S, block_q, block_k), block_states.device, workspace)
    _keep_alive(stream, ws)
    rc = library().bsattn_plan_elem(_ptr(block_states), _ptr(partial_index), n_tiles, B, H, S,
                                    block_q, block_k, _ptr(ws), ws.numel() * ws.element_size(),
                                    _stream(stream))
    _check(rc)
    return ws


def fwd_planned_elem(q, k, v, partial_bits, plan_ws, block_q, block_k, scale=None, *, out=None,
                     lse=None, config=None, stream=None):
    """The attention kernel alone on a plan from plan_elem(); returns (out, lse)."""
    B, H, S, D = _check_inputs(q, k, v)
    _mask_shape(q.shape, block_q, block_k)
    _check_tensor(partial_bits, "partial_bits", q.device, (torch.int32, torch.uint32))
    if partial_bits.dim() != 3:
        raise ValueError("partial_bits must be [n_tiles, block_q, block_k / 32]")
    _check_bits(partial_bits, block_q, block_k)
    _workspace(workspace_size(B, H, S, block_q, block_k), q.device, plan_ws, "plan_ws")
    if scale is None:
        scale = default_scale(D)
    out, lse = _outputs(q, out, lse)
    _keep_alive(stream, out, lse)
    rc = library().bsattn_fwd_planned_elem(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H,
                                           S, D, block_q, block_k, float(scale), _dtype_code(q),
                                           _ptr(partial_bits), partial_bits.shape[0],
                                           _ptr(plan_ws), plan_ws.numel() * plan_ws.element_size(),
                                           _cfg(config), _stream(stream))
    _check(rc)
    return out, lse


def fwd_elem(q, k, v, block_states, partial_index, partial_bits, block_q, block_k, scale=None, *,
             out=None, lse=None, workspace=None, config=None, stream=None):
    """Forward pass with an element-level mask (bsattn_fwd_elem); returns (out, lse)."""
    B, H, S, D = _check_inputs(q, k, v)
    n_tiles = _elem_tensors(block_states, partial_index, partial_bits, q.device,
                            _mask_shape(q.shape, block_q, block_k))
    _check_bits(partial_bits, block_q, block_k)
    if scale is None:
        scale = default_scale(D)
    out, lse = _outputs(q, out, lse)
    ws = _workspace(workspace_size(B, H, S, block_q, block_k), q.device, workspace)
    _keep_alive(stream, out, lse, ws)
    rc = library().bsattn_fwd_elem(_ptr(q), _ptr(k), _ptr(v), _ptr(block_states),
                                   _ptr(partial_index), _ptr(partial_bits), n_tiles, _ptr(out),
                                   _ptr(lse), B, H, S, D, block_q, block_k, float(scale),
                                   _dtype_code(q), _ptr(ws), ws.numel() * ws.element_size(),
                                   _cfg(config), _stream(stream))
    _check(rc)
    return out, lse


def list_configs_elem(dtype, D, block_q, block_k):
    """Tile configs built for element-level masks."""
    code = _dtype_code(torch.empty(0, dtype=dtype))
    n = ctypes.c_int(0)
    lib = library()
    _check(lib.bsattn_list_configs_elem(code, D, block_q, block_k, None, 0, ctypes.byref(n)))
    arr = (TileConfig * max(n.value, 1))()
    _check(lib.bsattn_list_configs_elem(code, D, block_q, block_k, arr, n.value, ctypes.byref(n)))
    return [arr[i] for i in range(n.value)]


def _ragged_operands(lhs, rhs):
    for name, t in (("lhs", lhs), ("rhs", rhs)):
        if not isinstance(t, torch.Tensor):
            raise TypeError("%s must be a torch tensor" % name)
        if not t.is_cuda:
            raise ValueError("%s must be a GPU tensor" % name)
    if lhs.dtype != torch.bfloat16 or rhs.dtype != torch.bfloat16:
        raise TypeError("lhs and rhs must be bfloat16")
    if lhs.dim() != 2 or rhs.dim() != 3 or rhs.shape[1] != lhs.shape[1]:
        raise ValueError("shapes: lhs [M, K], rhs [G, K, N]")
    _check_tensor(lhs, "lhs", lhs.device)
    _check_tensor(rhs, "rhs", lhs.device)
    M, K = lhs.shape
    G, _, N = rhs.shape
    return M, K, N, G


def _ragged_out(lhs, M, N, out, out_dtype):
    if out is None:
        return torch.empty((M, N), dtype=out_dtype or torch.bfloat16, device=lhs.device)
    return _check_tensor(out, "out", lhs.device, (torch.bfloat16, torch.float32), (M, N))


def ragged_dot(lhs, rhs, group_sizes, *, out=None, out_dtype=None, workspace=None, stream=None):
    """Ragged dot (bsattn_ragged_dot): lhs [M, K] bf16, rhs [G, K, N] bf16,
    group_sizes [G] int32 on the device.  Returns out [M, N] (bf16, or out_dtype)."""
    M, K, N, G = _ragged_operands(lhs, rhs)
    _check_tensor(group_sizes, "group_sizes", lhs.device, (torch.int32,), (G,))
    out = _ragged_out(lhs, M, N, out, out_dtype)
    code = _dtype_code(out)
    n = ctypes.c_size_t(0)
    lib = library()
    _check(lib.bsattn_ragged_dot_workspace_size(M, G, ctypes.byref(n)))
    ws = _workspace(n.value, lhs.device, workspace)
    _keep_alive(stream, out, ws)
    rc = lib.bsattn_ragged_dot(_ptr(lhs), _ptr(rhs), _ptr(group_sizes), _ptr(out), M, K, N, G,
                               _dtype_code(lhs), code, _ptr(ws), ws.numel() * ws.element_size(),
                               _stream(stream))
    _check(rc)
    return out


def ragged_plan(group_sizes, M, *, workspace=None, stream=None):
    """The work plan of a ragged dot (bsattn_ragged_plan); returns the workspace."""
    if not isinstance(group_sizes, torch.Tensor) or not group_sizes.is_cuda:
        raise ValueError("group_sizes must be a GPU tensor")
    if group_sizes.dim() != 1:
        raise ValueError("group_sizes must be int32 [G]")
    _check_tensor(group_sizes, "group_sizes", group_sizes.device, (torch.int32,))
    G = group_sizes.shape[0]
    n = ctypes.c_size_t(0)
    lib = library()
    _check(lib.bsattn_ragged_dot_workspace_size(M, G, ctypes.byref(n)))
    ws = _workspace(n.value, group_sizes.device, workspace)
    _keep_alive(stream, ws)
    _check(lib.bsattn_ragged_plan(_ptr(group_sizes), M, G, _ptr(ws), ws.numel() * ws.element_size(),
                                  _stream(stream)))
    return ws


def ragged_dot_planned(lhs, rhs, plan_ws, *, out=None, out_dtype=None, stream=None):
    """The ragged-dot product alone on a plan from ragged_plan()."""
    M, K, N, G = _ragged_operands(lhs, rhs)
    n = ctypes.c_size_t(0)
    _check(library().bsattn_ragged_dot_workspace_size(M, G, ctypes.byref(n)))
    _workspace(n.value, lhs.device, plan_ws, "plan_ws")
    out = _ragged_out(lhs, M, N, out, out_dtype)
    _keep_alive(stream, out)
    rc = library().bsattn_ragged_dot_planned(_ptr(lhs), _ptr(rhs), _ptr(out), M, K, N, G,
                                             _dtype_code(lhs), _dtype_code(out), _ptr(plan_ws),
                                             plan_ws.numel() * plan_ws.element_size(),
                                             _stream(stream))
    _check(rc)
    return out


def fp8_workspace_size(B, H, S, D, block_q, block_k):
    n = ctypes.c_size_t(0)
    _check(library().bsattn_fp8_workspace_size(B, H, S, D, block_q, block_k, ctypes.byref(n)))
    return n.value


def fwd_fp8(q, k, v, block_mask, block_q, block_k, scale=None, *, out=None, lse=None, workspace=None,
            stream=None):
    """Forward with fp8 e4m3 q, k, v (torch.float8_e4m3fn), bf16 out (bsattn_fwd_fp8).
    Returns (out, lse)."""
    B, H, S, D = _check_inputs(q, k, v)
    if q.dtype != torch.float8_e4m3fn:
        raise TypeError("q, k, v must be torch.float8_e4m3fn")
    block_mask = _mask_u8(block_mask, q.device, _mask_shape(q.shape, block_q, block_k))
    if scale is None:
        scale = default_scale(D)
    out, lse = _outputs(q, out, lse, torch.bfloat16)
    ws = _workspace(fp8_workspace_size(B, H, S, D, block_q, block_k), q.device, workspace)
    _keep_alive(stream, out, lse, ws)
    _check(library().bsattn_fwd_fp8(_ptr(q), _ptr(k), _ptr(v), _ptr(block_mask), _ptr(out), _ptr(lse), B, H, S,
                                    D, block_q, block_k, float(scale), _ptr(ws), ws.numel() * ws.element_size(),
                                    _stream(stream)))
    return out, lse


def fwd_fp8_planned(q, k, v, fp8_ws, block_q, block_k, scale=None, *, out=None, lse=None, stream=None):
    """bsattn_fwd_fp8_planned on a workspace of fp8_workspace_size() bytes whose
    first part holds a plan written by plan(block_mask, ..., workspace=fp8_ws)."""
    B, H, S, D = _check_inputs(q, k, v)
    if q.dtype != torch.float8_e4m3fn:
        raise TypeError("q, k, v must be torch.float8_e4m3fn")
    _mask_shape(q.shape, block_q, block_k)
    _workspace(fp8_workspace_size(B, H, S, D, block_q, block_k), q.device, fp8_ws, "fp8_ws")
    if scale is None:
        scale = default_scale(D)
    out, lse = _outputs(q, out, lse, torch.bfloat16)
    _keep_alive(stream, out, lse)
    _check(library().bsattn_fwd_fp8_planned(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, S, D, block_q,
                                            block_k, float(scale), _ptr(fp8_ws),
                                            fp8_ws.numel() * fp8_ws.element_size(), _stream(stream)))
    return out, lse


def fwd_fp8_elem(q, k, v, block_states, partial_index, partial_bits, block_q, block_k, scale=None, *,
                 out=None, lse=None, workspace=None, stream=None):
    """Forward with fp8 e4m3 q, k, v and an element-level mask (bsattn_fwd_fp8_elem);
    bf16 out.  Returns (out, lse)."""
    B, H, S, D = _check_inputs(q, k, v)
    if q.dtype != torch.float8_e4m3fn:
        raise TypeError("q, k, v must be torch.float8_e4m3fn")
    n_tiles = _elem_tensors(block_states, partial_index, partial_bits, q.device,
                            _mask_shape(q.shape, block_q, block_k))
    _check_bits(partial_bits, block_q, block_k)
    if scale is None:
        scale = default_scale(D)
    out, lse = _outputs(q, out, lse, torch.bfloat16)
    ws = _workspace(fp8_workspace_size(B, H, S, D, block_q, block_k), q.device, workspace)
    _keep_alive(stream, out, lse, ws)
    _check(library().bsattn_fwd_fp8_elem(_ptr(q), _ptr(k), _ptr(v), _ptr(block_states), _ptr(partial_index),
                                         _ptr(partial_bits), n_tiles, _ptr(out), _ptr(lse), B, H, S, D,
                                         block_q, block_k, float(scale), _ptr(ws),
                                         ws.numel() * ws.element_size(), _stream(stream)))
    return out, lse


def fwd_fp8_planned_elem(q, k, v, partial_bits, fp8_ws, block_q, block_k, scale=None, *, out=None, lse=None,
                         stream=None):
    """bsattn_fwd_fp8_planned_elem on a workspace of fp8_workspace_size() bytes whose
    first part holds a plan written by plan_elem(..., workspace=fp8_ws)."""
    B, H, S, D = _check_inputs(q, k, v)
    if q.dtype != torch.float8_e4m3fn:
        raise TypeError("q, k, v must be torch.float8_e4m3fn")
    _mask_shape(q.shape, block_q, block_k)
    _check_tensor(partial_bits, "partial_bits", q.device, (torch.int32, torch.uint32))
    if partial_bits.dim() != 3:
        raise ValueError("partial_bits must be [n_tiles, block_q, block_k / 32]")
    _check_bits(partial_bits, block_q, block_k)
    _workspace(fp8_workspace_size(B, H, S, D, block_q, block_k), q.device, fp8_ws, "fp8_ws")
    if scale is None:
        scale = default_scale(D)
    out, lse = _outputs(q, out, lse, torch.bfloat16)
    _keep_alive(stream, out, lse)
    _check(library().bsattn_fwd_fp8_planned_elem(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, S, D,
                                                 block_q, block_k, float(scale), _ptr(partial_bits),
                                                 partial_bits.shape[0], _ptr(fp8_ws),
                                                 fp8_ws.numel() * fp8_ws.element_size(), _stream(stream)))
    return out, lse


def bwd_workspace_size(B, H, S, block_q, block_k):
    n = ctypes.c_size_t(0)
    _check(library().bsattn_bwd_workspace_size(B, H, S, block_q, block_k, ctypes.byref(n)))
    return n.value


def _bwd_tensors(q, out, lse, dout):
    """The forward's out [B,H,S,D] (dtype of q), lse [B,H,S] fp32 and the
    upstream gradient dout [B,H,S,D] (dtype of q), on q's device."""
    _check_tensor(out, "out", q.device, (q.dtype,), q.shape)
    _check_tensor(lse, "lse", q.device, (torch.float32,), q.shape[:3])
    _check_tensor(dout, "dout", q.device, (q.dtype,), q.shape)


def _grads(q, grad_dtype, dq, dk, dv):
    gd = grad_dtype or q.dtype
    if gd not in (torch.bfloat16, torch.float32):
        raise TypeError("gradients must be bfloat16 or float32")
    res = []
    for name, g in (("dq", dq), ("dk", dk), ("dv", dv)):
        if g is None:
            g = torch.empty(q.shape, dtype=gd, device=q.device)
        else:
            _check_tensor(g, name, q.device, (torch.bfloat16, torch.float32), q.shape)
        res.append(g)
    dq, dk, dv = res
    if not (dq.dtype == dk.dtype == dv.dtype):
        raise ValueError("dq, dk, dv must have one dtype")
    return dq, dk, dv


def bwd(q, k, v, out, lse, dout, block_mask, block_q, block_k, scale=None, *, grad_dtype=None,
        dq=None, dk=None, dv=None, workspace=None, stream=None):
    """Gradients of the forward (bsattn_bwd) for the upstream gradient dout, from
    the forward's out and lse.  Returns (dq, dk, dv) in grad_dtype (default: the
    input dtype; torch.float32 for fp32 gradients)."""
    B, H, S, D = _check_inputs(q, k, v)
    _bwd_tensors(q, out, lse, dout)
    block_mask = _mask_u8(block_mask, q.device, _mask_shape(q.shape, block_q, block_k))
    if scale is None:
        scale = default_scale(D)
    dq, dk, dv = _grads(q, grad_dtype, dq, dk, dv)
    ws = _workspace(bwd_workspace_size(B, H, S, block_q, block_k), q.device, workspace)
    _keep_alive(stream, dq, dk, dv, ws)
    rc = library().bsattn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(dout),
                              _ptr(block_mask), B, H, S, D, block_q, block_k, float(scale),
                              _dtype_code(q), _ptr(dq), _ptr(dk), _ptr(dv), _dtype_code(dq), _ptr(ws),
                              ws.numel() * ws.element_size(), _stream(stream))
    _check(rc)
    return dq, dk, dv


def bwd_elem(q, k, v, out, lse, dout, block_states, partial_index, partial_bits, block_q, block_k, scale=None, *,
             grad_dtype=None, dq=None, dk=None, dv=None, workspace=None, stream=None):
    """Gradients of the element-mask forward (fwd_elem) for the upstream gradient
    dout (bsattn_bwd_elem).  Returns (dq, dk, dv)."""
    B, H, S, D = _check_inputs(q, k, v)
    _bwd_tensors(q, out, lse, dout)
    n_tiles = _elem_tensors(block_states, partial_index, partial_bits, q.device,
                            _mask_shape(q.shape, block_q, block_k))
    _check_bits(partial_bits, block_q, block_k)
    if scale is None:
        scale = default_scale(D)
    dq, dk, dv = _grads(q, grad_dtype, dq, dk, dv)
    ws = _workspace(bwd_workspace_size(B, H, S, block_q, block_k), q.device, workspace)
    _keep_alive(stream, dq, dk, dv, ws)
    rc = library().bsattn_bwd_elem(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(dout), _ptr(block_states),
                                   _ptr(partial_index), _ptr(partial_bits), n_tiles, B, H, S, D, block_q,
                                   block_k, float(scale),
                                   _dtype_code(q), _ptr(dq), _ptr(dk), _ptr(dv), _dtype_code(dq), _ptr(ws),
                                   ws.numel() * ws.element_size(), _stream(stream))
    _check(rc)
    return dq, dk, dv


def bwd_planned_elem(q, k, v, out, lse, dout, block_states, partial_index, partial_bits, plan_ws, block_q,
                     block_k, scale=None, *, grad_dtype=None, dq=None, dk=None, dv=None, parts=7, stream=None):
    """The element-mask gradient kernels alone on a plan from bwd_plan(block_states)
    (bsattn_bwd_planned_elem); parts is an OR of BWD_PREP, BWD_DQ, BWD_DKDV."""
    B, H, S, D = _check_inputs(q, k, v)
    _bwd_tensors(q, out, lse, dout)
    n_tiles = _elem_tensors(block_states, partial_index, partial_bits, q.device,
                            _mask_shape(q.shape, block_q, block_k))
    _check_bits(partial_bits, block_q, block_k)
    _workspace(bwd_workspace_size(B, H, S, block_q, block_k), q.device, plan_ws, "plan_ws")
    if scale is None:
        scale = default_scale(D)
    dq, dk, dv = _grads(q, grad_dtype, dq, dk, dv)
    _keep_alive(stream, dq, dk, dv)
    rc = library().bsattn_bwd_planned_elem(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(dout),
                                           _ptr(block_states), _ptr(partial_index), _ptr(partial_bits), n_tiles,
                                           B, H, S, D, block_q, block_k, float(scale), _dtype_code(q), _ptr(dq),
                                           _ptr(dk), _ptr(dv), _dtype_code(dq), int(parts), _ptr(plan_ws),
                                           plan_ws.numel() * plan_ws.element_size(), _stream(stream))
    _check(rc)
    return dq, dk, dv


def bwd_plan(block_mask, S, block_q, block_k, *, workspace=None, stream=None):
    """The mask-dependent step of bwd() (bsattn_bwd_plan); returns the workspace."""
    block_mask = _mask_u8(block_mask)
    if block_mask.dim() != 4:
        raise ValueError("block_mask must be [B, H, S/block_q, S/block_k]")
    B, H, n_q, n_k = block_mask.shape
    if (n_q * block_q, n_k * block_k) != (S, S):
        raise ValueError("block_mask must be [B, H, S/block_q, S/block_k]")
    ws = _workspace(bwd_workspace_size(B, H, S, block_q, block_k), block_mask.device, workspace)
    _keep_alive(stream, ws)
    _check(library().bsattn_bwd_plan(_ptr(block_mask), B, H, S, block_q, block_k, _ptr(ws),
                                     ws.numel() * ws.element_size(), _stream(stream)))
    return ws


BWD_PREP, BWD_DQ, BWD_DKDV, BWD_ALL = 4, 1, 2, 7


def bwd_planned(q, k, v, out, lse, dout, plan_ws, block_q, block_k, scale=None, *, grad_dtype=None,
                dq=None, dk=None, dv=None, parts=BWD_ALL, stream=None):
    """The gradient kernels alone on a plan from bwd_plan() (bsattn_bwd_planned);
    parts is an OR of BWD_PREP, BWD_DQ, BWD_DKDV."""
    B, H, S, D = _check_inputs(q, k, v)
    _bwd_tensors(q, out, lse, dout)
    _mask_shape(q.shape, block_q, block_k)
    _workspace(bwd_workspace_size(B, H, S, block_q, block_k), q.device, plan_ws, "plan_ws")
    if scale is None:
        scale = default_scale(D)
    dq, dk, dv = _grads(q, grad_dtype, dq, dk, dv)
    _keep_alive(stream, dq, dk, dv)
    rc = library().bsattn_bwd_planned(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(dout), B, H,
                                      S, D, block_q, block_k, float(scale), _dtype_code(q), _ptr(dq),
                                      _ptr(dk), _ptr(dv), _dtype_code(dq), int(parts), _ptr(plan_ws),
                                      plan_ws.numel() * plan_ws.element_size(), _stream(stream))
    _check(rc)
    return dq, dk, dv


def list_configs(dtype, D, block_q, block_k):
    """Tile configs built for this shape, in the library's preference order."""
    code = _dtype_code(torch.empty(0, dtype=dtype))
    n = ctypes.c_int(0)
    lib = library()
    _check(lib.bsattn_list_configs(code, D, block_q, block_k, None, 0, ctypes.byref(n)))
    arr = (TileConfig * max(n.value, 1))()
    _check(lib.bsattn_list_configs(code, D, block_q, block_k, arr, n.value, ctypes.byref(n)))
    return [arr[i] for i in range(n.value)]


@dataclass
class TuneRow:
    id: int
    config: tuple
    t_mean_s: float
    t_std_s: float
    t_min_s: float


def autotune(q, k, v, block_mask, block_q, block_k, scale=None, *, warmup=3, iters=10,
             cache_path=None, stream=None):
    """Time every built tile config on these inputs; returns (best TileConfig,
    [TuneRow sorted by t_mean]).  The winner is cached in-process for bsattn_fwd
    (and merged into cache_path if given)."""
    B, H, S, D = _check_inputs(q, k, v)
    block_mask = _mask_u8(block_mask)
    if scale is None:
        scale = default_scale(D)
    out = torch.empty_like(q)
    lse = torch.empty((B, H, S), dtype=torch.float32, device=q.device)
    ws = _workspace(workspace_size(B, H, S, block_q, block_k), q.device, None)
    cap = 64
    res = (TuneResult * cap)()
    n = ctypes.c_int(0)
    best = TileConfig()
    path = cache_path.encode() if cache_path else None
    rc = library().bsattn_autotune(_ptr(q), _ptr(k), _ptr(v), _ptr(block_mask), _ptr(out),
                                   _ptr(lse), B, H, S, D, block_q, block_k, float(scale),
                                   _dtype_code(q), _ptr(ws), ws.numel() * ws.element_size(),
                                   warmup, iters, ctypes.byref(best), res, cap, ctypes.byref(n),
                                   path, _stream(stream))
    _check(rc)
    rows = [TuneRow(res[i].id, res[i].cfg.as_tuple(), res[i].t_mean_s, res[i].t_std_s,
                    res[i].t_min_s) for i in range(min(n.value, cap))]
    return best, rows


def tune_lookup(dtype, D, B, H, S, block_q, block_k, nnz=-1):
    """The cached tuned config for a mask of nnz active blocks on this shape
    (bsattn_tune_lookup; nnz < 0: the shape's densest tuned mask), or None."""
    cfg = TileConfig()
    code = _dtype_code(torch.empty(0, dtype=dtype))
    rc = library().bsattn_tune_lookup(code, D, B, H, S, block_q, block_k, int(nnz), ctypes.byref(cfg))
    if rc == 3:
        return None
    _check(rc)
    return cfg


def load_tune_cache(path):
    _check(library().bsattn_load_tune_cache(path.encode()))


def clear_tune_cache():
    library().bsattn_clear_tune_cache()


def version():
    v = library().bsattn_version()
    return (v >> 16, (v >> 8) & 0xFF, v & 0xFF)
