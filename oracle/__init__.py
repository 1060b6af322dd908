"""fp64 CPU oracle of block-sparse masked softmax attention (ctypes wrapper).

TEST INFRASTRUCTURE ONLY: the yardstick the HIP path is checked against.  Only the
test suite, the smoke check and the CPU-baseline leg of the benchmark may import
it; the product path never does.  It shares no code with the HIP library.

The arithmetic lives in ``oracle.c`` (plain C, fp64, OpenMP over rows); this module
only marshals numpy / torch CPU arrays into it.  What it computes, and the readings
of the pages it follows, are stated in the header of ``oracle.c``:
"Writing Pallas Kernels for JAX", section "Writing the Kernel Logic: Load, Compute,
Store" (masked scaled-dot-product softmax times V), and "Pallas-Triton kernels and
kernel auto-tuning", section "Flash Attention" (the tiled method is exact, so the
oracle is the plain operator).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

F32, BF16, F64, FP8 = 0, 1, 2, 3

_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc (-O2, OpenMP, no fast-math) into liboracle.so."""
    if not force and os.path.exists(_LIB):
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build()
    _lib = configure(ctypes.CDLL(_LIB))
    return _lib


def configure(lib):
    """Declare the C signatures on a loaded oracle library and return it."""
    p, i64, i32, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float
    lib.oracle_fwd.argtypes = [p, p, p, i32, p, i64, i64, i64, i64, i64, i64, f32, p, p, i32]
    lib.oracle_fwd.restype = i32
    lib.oracle_fwd_rows.argtypes = [p, p, p, i32, p, i64, i64, i64, i64, i64, i64, f32,
                                    p, i64, p, p, i32]
    lib.oracle_fwd_rows.restype = i32
    lib.oracle_fwd_elem.argtypes = [p, p, p, i32, p, p, p, i64, i64, i64, i64, i64, i64, i64,
                                    f32, p, p, i32]
    lib.oracle_fwd_elem.restype = i32
    lib.oracle_fwd_rows_elem.argtypes = [p, p, p, i32, p, p, p, i64, i64, i64, i64, i64, i64,
                                         i64, f32, p, i64, p, p, i32]
    lib.oracle_fwd_rows_elem.restype = i32
    lib.oracle_ragged_dot.argtypes = [p, p, i32, p, i64, i64, i64, i64, p, i32]
    lib.oracle_ragged_dot.restype = i32
    lib.oracle_bwd.argtypes = [p, p, p, p, i32, p, i64, i64, i64, i64, i64, i64, f32, p, p, p, i32]
    lib.oracle_bwd.restype = i32
    lib.oracle_bwd_sample.argtypes = [p, p, p, p, i32, p, i64, i64, i64, i64, i64, i64, f32,
                                      p, i64, p, p, i64, p, p, i32]
    lib.oracle_bwd_sample.restype = i32
    lib.oracle_bwd_elem.argtypes = [p, p, p, p, i32, p, p, p, i64, i64, i64, i64, i64, i64, i64, f32,
                                    p, p, p, i32]
    lib.oracle_bwd_elem.restype = i32
    lib.oracle_bwd_sample_elem.argtypes = [p, p, p, p, i32, p, p, p, i64, i64, i64, i64, i64, i64, i64,
                                           f32, p, i64, p, p, i64, p, p, i32]
    lib.oracle_bwd_sample_elem.restype = i32
    lib.oracle_probs.argtypes = [p, p, p, i32, p, i64, i64, i64, i64, i64, i64, f32, p]
    lib.oracle_probs.restype = i32
    lib.oracle_compact.argtypes = [p, i64, i64, p, p]
    lib.oracle_compact.restype = i64
    lib.oracle_max_threads.argtypes = []
    lib.oracle_max_threads.restype = i32
    return lib


def _as_raw(x):
    """Return (contiguous numpy array of raw element bits, dtype code).

    Accepts numpy float32/float64 arrays and torch CPU tensors of float32,
    float64 or bfloat16 (passed as their raw 16-bit patterns; the C code widens
    them exactly)."""
    try:
        import torch
    except ImportError:  # pragma: no cover
        torch = None
    if torch is not None and isinstance(x, torch.Tensor):
        if x.device.type != "cpu":
            raise ValueError("oracle inputs must live on the CPU")
        x = x.contiguous()
        if x.dtype == torch.bfloat16:
            return x.view(torch.int16).numpy(), BF16
        if x.dtype == torch.float8_e4m3fn:
            return x.view(torch.uint8).numpy(), FP8
        if x.dtype == torch.float32:
            return x.numpy(), F32
        if x.dtype == torch.float64:
            return x.numpy(), F64
        raise TypeError("unsupported tensor dtype %s" % x.dtype)
    x = np.ascontiguousarray(x)
    if x.dtype == np.float32:
        return x, F32
    if x.dtype == np.float64:
        return x, F64
    raise TypeError("unsupported array dtype %s" % x.dtype)


def _mask_u8(mask):
    try:
        import torch
        if isinstance(mask, torch.Tensor):
            mask = mask.contiguous().to(torch.uint8).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(mask) != 0, dtype=np.uint8)


def _shape(q, mask, block_q, block_k):
    B, H, S, D = q.shape
    n_q, n_k = S // block_q, S // block_k
    if tuple(mask.shape) != (B, H, n_q, n_k):
        raise ValueError("mask shape %s != %s" % (tuple(mask.shape), (B, H, n_q, n_k)))
    return B, H, S, D


def fwd(q, k, v, mask, block_q, block_k, scale, nthreads=0):
    """Full forward.  q, k, v: [B,H,S,D]; mask: [B,H,S/block_q,S/block_k].
    Returns (out float64 [B,H,S,D], lse float64 [B,H,S])."""
    lib = _load()
    qa, dt = _as_raw(q)
    ka, dt2 = _as_raw(k)
    va, dt3 = _as_raw(v)
    if not (dt == dt2 == dt3):
        raise TypeError("q, k, v must share a dtype")
    m = _mask_u8(mask)
    B, H, S, D = _shape(qa, m, block_q, block_k)
    out = np.empty((B, H, S, D), dtype=np.float64)
    lse = np.empty((B, H, S), dtype=np.float64)
    rc = lib.oracle_fwd(qa.ctypes.data, ka.ctypes.data, va.ctypes.data, dt, m.ctypes.data,
                        B, H, S, D, block_q, block_k, float(np.float32(scale)),
                        out.ctypes.data, lse.ctypes.data, int(nthreads))
    if rc:
        raise ValueError("oracle_fwd failed with code %d" % rc)
    return out, lse


def fwd_rows(q, k, v, mask, block_q, block_k, scale, rows, nthreads=0):
    """Selected rows: rows are flat indices (b*H + h)*S + s.
    Returns (out float64 [n, D], lse float64 [n])."""
    lib = _load()
    qa, dt = _as_raw(q)
    ka, _ = _as_raw(k)
    va, _ = _as_raw(v)
    m = _mask_u8(mask)
    B, H, S, D = _shape(qa, m, block_q, block_k)
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    n = rows.shape[0]
    out = np.empty((n, D), dtype=np.float64)
    lse = np.empty((n,), dtype=np.float64)
    rc = lib.oracle_fwd_rows(qa.ctypes.data, ka.ctypes.data, va.ctypes.data, dt, m.ctypes.data,
                             B, H, S, D, block_q, block_k, float(np.float32(scale)),
                             rows.ctypes.data, n, out.ctypes.data, lse.ctypes.data, int(nthreads))
    if rc:
        raise ValueError("oracle_fwd_rows failed with code %d" % rc)
    return out, lse


def _elem_args(states, pidx, pbits, B, H, n_q, n_k, block_q, block_k):
    """Raw block states (uint8, 0 empty / 1 full / else partial), tile index per
    block (int32) and bit tiles (uint32 [n_tiles, block_q, block_k / 32])."""
    try:
        import torch
        conv = lambda x: x.contiguous().numpy() if isinstance(x, torch.Tensor) else x
    except ImportError:  # pragma: no cover
        conv = lambda x: x
    st = np.ascontiguousarray(conv(states), dtype=np.uint8)
    pi = np.ascontiguousarray(conv(pidx), dtype=np.int32)
    pb = np.ascontiguousarray(conv(pbits))
    if pb.dtype != np.uint32:
        pb = pb.astype(np.int64).astype(np.uint32)
    if st.shape != (B, H, n_q, n_k) or pi.shape != (B, H, n_q, n_k):
        raise ValueError("states / pidx must be [B, H, S/block_q, S/block_k]")
    if pb.ndim != 3 or pb.shape[1:] != (block_q, block_k // 32):
        raise ValueError("pbits must be [n_tiles, block_q, block_k / 32]")
    if pb.shape[0] == 0:
        pb = np.zeros((1, block_q, block_k // 32), dtype=np.uint32)
        return st, pi, pb, 0
    return st, pi, pb, pb.shape[0]


def fwd_elem(q, k, v, states, pidx, pbits, block_q, block_k, scale, nthreads=0):
    """Full forward with an element-level mask (block states + bit tiles; see the
    header of oracle.c).  Returns (out float64 [B,H,S,D], lse float64 [B,H,S])."""
    lib = _load()
    qa, dt = _as_raw(q)
    ka, _ = _as_raw(k)
    va, _ = _as_raw(v)
    B, H, S, D = qa.shape
    st, pi, pb, nt = _elem_args(states, pidx, pbits, B, H, S // block_q, S // block_k,
                                block_q, block_k)
    out = np.empty((B, H, S, D), dtype=np.float64)
    lse = np.empty((B, H, S), dtype=np.float64)
    rc = lib.oracle_fwd_elem(qa.ctypes.data, ka.ctypes.data, va.ctypes.data, dt, st.ctypes.data,
                             pi.ctypes.data, pb.ctypes.data, nt, B, H, S, D, block_q, block_k,
                             float(np.float32(scale)), out.ctypes.data, lse.ctypes.data,
                             int(nthreads))
    if rc:
        raise ValueError("oracle_fwd_elem failed with code %d" % rc)
    return out, lse


def fwd_rows_elem(q, k, v, states, pidx, pbits, block_q, block_k, scale, rows, nthreads=0):
    """Selected rows (flat (b*H + h)*S + s) of fwd_elem: (out [n, D], lse [n])."""
    lib = _load()
    qa, dt = _as_raw(q)
    ka, _ = _as_raw(k)
    va, _ = _as_raw(v)
    B, H, S, D = qa.shape
    st, pi, pb, nt = _elem_args(states, pidx, pbits, B, H, S // block_q, S // block_k,
                                block_q, block_k)
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    n = rows.shape[0]
    out = np.empty((n, D), dtype=np.float64)
    lse = np.empty((n,), dtype=np.float64)
    rc = lib.oracle_fwd_rows_elem(qa.ctypes.data, ka.ctypes.data, va.ctypes.data, dt,
                                  st.ctypes.data, pi.ctypes.data, pb.ctypes.data, nt, B, H, S, D,
                                  block_q, block_k, float(np.float32(scale)), rows.ctypes.data, n,
                                  out.ctypes.data, lse.ctypes.data, int(nthreads))
    if rc:
        raise ValueError("oracle_fwd_rows_elem failed with code %d" % rc)
    return out, lse


def ragged_dot(lhs, rhs, group_sizes, nthreads=0):
    """Ragged dot ("Pallas-Triton kernels and kernel auto-tuning", section "Ragged
    Dot"): lhs [M, K], rhs [G, K, N], group_sizes [G] int.  Group g takes the
    next rows in order; a negative size counts as 0 and a group takes at most
    the rows that remain; rows after the last group's are 0.  Returns out
    float64 [M, N]."""
    lib = _load()
    la, dt = _as_raw(lhs)
    ra, dt2 = _as_raw(rhs)
    if dt != dt2:
        raise TypeError("lhs and rhs must share a dtype")
    try:
        import torch
        if isinstance(group_sizes, torch.Tensor):
            group_sizes = group_sizes.cpu().numpy()
    except ImportError:  # pragma: no cover
        pass
    gs = np.ascontiguousarray(np.asarray(group_sizes, dtype=np.int32))
    M, K = la.shape
    G, K2, N = ra.shape
    if K2 != K or gs.shape != (G,):
        raise ValueError("shapes: lhs [M,K], rhs [G,K,N], group_sizes [G]")
    out = np.empty((M, N), dtype=np.float64)
    rc = lib.oracle_ragged_dot(la.ctypes.data, ra.ctypes.data, dt, gs.ctypes.data, G, M, K, N,
                               out.ctypes.data, int(nthreads))
    if rc:
        raise ValueError("oracle_ragged_dot failed with code %d" % rc)
    return out


def _bwd_inputs(q, k, v, dout, mask, block_q, block_k):
    qa, dt = _as_raw(q)
    ka, dk_ = _as_raw(k)
    va, dv_ = _as_raw(v)
    oa, do_ = _as_raw(dout)
    if len({dt, dk_, dv_, do_}) != 1:
        raise TypeError("q, k, v and dout must share a dtype")
    if oa.shape != qa.shape:
        raise ValueError("dout shape %s != q shape %s" % (oa.shape, qa.shape))
    m = _mask_u8(mask)
    return qa, ka, va, oa, dt, m, _shape(qa, m, block_q, block_k)


def bwd(q, k, v, dout, mask, block_q, block_k, scale, nthreads=0):
    """Gradients of the forward for the upstream gradient dout (header of
    oracle.c, "Backward").  All arrays [B,H,S,D]; mask [B,H,S/block_q,S/block_k].
    Returns (dq, dk, dv), float64 [B,H,S,D]."""
    lib = _load()
    qa, ka, va, oa, dt, m, (B, H, S, D) = _bwd_inputs(q, k, v, dout, mask, block_q, block_k)
    dq = np.empty((B, H, S, D), dtype=np.float64)
    dk = np.empty_like(dq)
    dv = np.empty_like(dq)
    rc = lib.oracle_bwd(qa.ctypes.data, ka.ctypes.data, va.ctypes.data, oa.ctypes.data, dt,
                        m.ctypes.data, B, H, S, D, block_q, block_k, float(np.float32(scale)),
                        dq.ctypes.data, dk.ctypes.data, dv.ctypes.data, int(nthreads))
    if rc:
        raise ValueError("oracle_bwd failed with code %d" % rc)
    return dq, dk, dv


def bwd_sample(q, k, v, dout, mask, block_q, block_k, scale, q_rows, k_rows, nthreads=0):
    """dq of the flat query rows q_rows and dk, dv of the flat key rows k_rows
    (flat row = (b*H + h)*S + s).  Returns (dq [nq,D], dk [nk,D], dv [nk,D])."""
    lib = _load()
    qa, ka, va, oa, dt, m, (B, H, S, D) = _bwd_inputs(q, k, v, dout, mask, block_q, block_k)
    qr = np.ascontiguousarray(np.asarray(q_rows, dtype=np.int64))
    kr = np.ascontiguousarray(np.asarray(k_rows, dtype=np.int64))
    dq = np.empty((max(len(qr), 1), D), dtype=np.float64)
    dk = np.empty((max(len(kr), 1), D), dtype=np.float64)
    dv = np.empty_like(dk)
    rc = lib.oracle_bwd_sample(qa.ctypes.data, ka.ctypes.data, va.ctypes.data, oa.ctypes.data, dt,
                               m.ctypes.data, B, H, S, D, block_q, block_k,
                               float(np.float32(scale)), qr.ctypes.data, len(qr), dq.ctypes.data,
                               kr.ctypes.data, len(kr), dk.ctypes.data, dv.ctypes.data,
                               int(nthreads))
    if rc:
        raise ValueError("oracle_bwd_sample failed with code %d" % rc)
    return dq[:len(qr)], dk[:len(kr)], dv[:len(kr)]


def probs(q, k, v, mask, block_q, block_k, scale):
    """Dense softmax weights P [B,H,S,S] (zero where masked) for tiny shapes."""
    lib = _load()
    qa, dt = _as_raw(q)
    ka, _ = _as_raw(k)
    va, _ = _as_raw(v)
    m = _mask_u8(mask)
    B, H, S, D = _shape(qa, m, block_q, block_k)
    P = np.empty((B, H, S, S), dtype=np.float64)
    rc = lib.oracle_probs(qa.ctypes.data, ka.ctypes.data, va.ctypes.data, dt, m.ctypes.data,
                          B, H, S, D, block_q, block_k, float(np.float32(scale)), P.ctypes.data)
    if rc:
        raise ValueError("oracle_probs failed with code %d" % rc)
    return P


def compact(mask):
    """CSR compaction of a block mask [..., n_k] flattened to rows.
    Returns (row_ptr int32 [R+1], col_idx int32 [nnz])."""
    lib = _load()
    m = _mask_u8(mask)
    n_k = m.shape[-1]
    R = m.size // n_k
    row_ptr = np.empty(R + 1, dtype=np.int32)
    col_idx = np.empty(max(R * n_k, 1), dtype=np.int32)
    nnz = lib.oracle_compact(m.ctypes.data, R, n_k, row_ptr.ctypes.data, col_idx.ctypes.data)
    if nnz < 0:
        raise ValueError("oracle_compact failed")
    return row_ptr, col_idx[:nnz].copy()


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def bwd_elem(q, k, v, dout, states, pidx, pbits, block_q, block_k, scale, nthreads=0):
    """Gradients of the element-mask forward (fwd_elem) for the upstream gradient
    dout: the backward formulas over the kept (query, key) pairs.  Returns (dq,
    dk, dv), float64 [B,H,S,D]."""
    lib = _load()
    B, H, S, D = tuple(q.shape)
    qa, ka, va, oa, dt, _, _ = _bwd_inputs(q, k, v, dout, np.zeros((B, H, S // block_q, S // block_k),
                                                                     dtype=np.uint8), block_q, block_k)
    st, pi, pb, nt = _elem_args(states, pidx, pbits, B, H, S // block_q, S // block_k, block_q, block_k)
    dq = np.empty((B, H, S, D), dtype=np.float64)
    dk = np.empty_like(dq)
    dv = np.empty_like(dq)
    rc = lib.oracle_bwd_elem(qa.ctypes.data, ka.ctypes.data, va.ctypes.data, oa.ctypes.data, dt, st.ctypes.data,
                             pi.ctypes.data, pb.ctypes.data, nt, B, H, S, D, block_q, block_k,
                             float(np.float32(scale)), dq.ctypes.data, dk.ctypes.data, dv.ctypes.data,
                             int(nthreads))
    if rc:
        raise ValueError("oracle_bwd_elem failed with code %d" % rc)
    return dq, dk, dv


def bwd_sample_elem(q, k, v, dout, states, pidx, pbits, block_q, block_k, scale, q_rows, k_rows, nthreads=0):
    """bwd_sample for an element-level mask: dq of the flat query rows q_rows, dk
    and dv of the flat key rows k_rows."""
    lib = _load()
    B, H, S, D = tuple(q.shape)
    qa, ka, va, oa, dt, _, _ = _bwd_inputs(q, k, v, dout, np.zeros((B, H, S // block_q, S // block_k),
                                                                     dtype=np.uint8), block_q, block_k)
    st, pi, pb, nt = _elem_args(states, pidx, pbits, B, H, S // block_q, S // block_k, block_q, block_k)
    qr = np.ascontiguousarray(np.asarray(q_rows, dtype=np.int64))
    kr = np.ascontiguousarray(np.asarray(k_rows, dtype=np.int64))
    dq = np.empty((max(len(qr), 1), D), dtype=np.float64)
    dk = np.empty((max(len(kr), 1), D), dtype=np.float64)
    dv = np.empty_like(dk)
    rc = lib.oracle_bwd_sample_elem(qa.ctypes.data, ka.ctypes.data, va.ctypes.data, oa.ctypes.data, dt,
                                    st.ctypes.data, pi.ctypes.data, pb.ctypes.data, nt, B, H, S, D, block_q,
                                    block_k, float(np.float32(scale)), qr.ctypes.data, len(qr), dq.ctypes.data,
                                    kr.ctypes.data, len(kr), dk.ctypes.data, dv.ctypes.data, int(nthreads))
    if rc:
        raise ValueError("oracle_bwd_sample_elem failed with code %d" % rc)
    return dq[:len(qr)], dk[:len(kr)], dv[:len(kr)]
