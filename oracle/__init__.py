"""fp64 CPU oracle for the attention hot path — TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package. The product path (the HIP library and its binding) never does.

The arithmetic lives in ``oracle.c`` (plain loops, fp64, one definition per
operation); this module only builds it with gcc and marshals numpy arrays.
Every function here is pinned by the ``-m "not gpu"`` tests against
independent facts (brute force, library routines, closed forms, invariants,
printed numbers); see ``tests/test_oracle_pins.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
# A test may point the loader at another build of the same source (the
# mutation check of the pins does, with a planted mistake).
_LIB_OVERRIDE = os.environ.get("BGA_ORACLE_LIB")
_lib = None
GCC_FLAGS = ["-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-std=c11"]


def build(force: bool = True, src: str = _SRC, out: str = _LIB) -> str:
    """Compile oracle.c (or `src`) with gcc into liboracle.so next to it (or `out`)."""
    if force or not os.path.exists(out):
        tmp = out + ".tmp"
        subprocess.run(["gcc", *GCC_FLAGS, src, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, out)
    return out


def lib():
    global _lib
    if _lib is None:
        path = _LIB_OVERRIDE or _LIB
        if not _LIB_OVERRIDE and not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(path)
        P = ctypes.c_void_p
        i32, f64 = ctypes.c_int32, ctypes.c_double
        L.oracle_packed_prefill.argtypes = [P, P, P, P, i32, i32, i32, i32, f64, P, P, i32]
        L.oracle_shared_prefix_decode.argtypes = [P, P, P, P, P, i32, i32, i32, i32, i32, i32, i32, i32,
                                                  f64, P, P, i32]
        L.oracle_shared_prefix_decode_packed.argtypes = [P, P, P, P, P, P, i32, i32, i32, i32, i32, i32, i32,
                                                         f64, P, P, i32]
        L.oracle_last_token_gather.argtypes = [P, P, i32, ctypes.c_int64, P]
        L.oracle_suffix_reorder.argtypes = [P, P, P, P, P, P, P, i32, i32, i32, i32, i32, i32, i32, i32]
        L.oracle_beam_topk.argtypes = [P, P, i32, i32, i32, i32, i32, P, P, P, P, P, P, P, i32]
        L.oracle_beam_topk_given_lse.argtypes = [P, P, P, i32, i32, i32, i32, i32, P, P, P, P, P, P, P, i32]
        L.oracle_num_threads.argtypes = [i32]
        L.oracle_e4m3_encode.argtypes = [f64]
        L.oracle_e4m3_encode.restype = ctypes.c_uint8
        L.oracle_e4m3_encode_array.argtypes = [P, ctypes.c_int64, P]
        L.oracle_e4m3_encode_array.restype = i32
        L.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
        L.oracle_e4m3_decode.restype = f64
        L.oracle_swiglu_quant.argtypes = [P, i32, i32, P, P, P, P, i32]
        L.oracle_swiglu_quant.restype = i32
        for f in (L.oracle_packed_prefill, L.oracle_shared_prefix_decode, L.oracle_shared_prefix_decode_packed,
                  L.oracle_last_token_gather, L.oracle_suffix_reorder,
                  L.oracle_beam_topk, L.oracle_beam_topk_given_lse, L.oracle_num_threads):
            f.restype = i32
        _lib = L
    return _lib


def _bits(a) -> np.ndarray:
    """bf16 input as a contiguous uint16 array (accepts numpy uint16 or a torch bf16 tensor)."""
    if hasattr(a, "dtype") and str(a.dtype) == "torch.bfloat16":
        import torch
        a = a.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError("expected bf16 bits as uint16")
    return a


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def num_threads(requested: int = 0) -> int:
    return int(lib().oracle_num_threads(requested))


def packed_prefill(q, k, v, cu_seqlens, scale=None, nthreads: int = 0):
    """fp64 (out [T,Nq,D], lse [T,Nq]) of packed causal GQA prefill."""
    q, k, v = _bits(q), _bits(k), _bits(v)
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    t, nq, d = q.shape
    nkv = k.shape[1]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    out = np.zeros((t, nq, d), np.float64)
    lse = np.zeros((t, nq), np.float64)
    rc = lib().oracle_packed_prefill(_p(q), _p(k), _p(v), _p(cu), len(cu) - 1, nq, nkv, d, float(scale),
                                     _p(out), _p(lse), nthreads)
    if rc:
        raise ValueError(f"oracle_packed_prefill rejected its arguments ({rc})")
    return out, lse


def shared_prefix_decode(q, prefix_k, prefix_v, suffix_k, suffix_v, suffix_len, scale=None, nthreads: int = 0):
    """fp64 (out [R,W,Nq,D], lse [R,W,Nq]) of shared-prefix decode over [prefix; suffix[:suffix_len]]."""
    q, pk, pv = _bits(q), _bits(prefix_k), _bits(prefix_v)
    sk, sv = _bits(suffix_k), _bits(suffix_v)
    r, w, nq, d = q.shape
    lp, nkv = pk.shape[1], pk.shape[2]
    ls_cap = sk.shape[2]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    out = np.zeros((r, w, nq, d), np.float64)
    lse = np.zeros((r, w, nq), np.float64)
    rc = lib().oracle_shared_prefix_decode(_p(q), _p(pk), _p(pv), _p(sk), _p(sv), r, w, lp, suffix_len, ls_cap,
                                           nq, nkv, d, float(scale), _p(out), _p(lse), nthreads)
    if rc:
        raise ValueError(f"oracle_shared_prefix_decode rejected its arguments ({rc})")
    return out, lse


def shared_prefix_decode_packed(q, prefix_k, prefix_v, prefix_cu, suffix_k, suffix_v, suffix_len, scale=None,
                                nthreads: int = 0):
    """fp64 (out [R,W,Nq,D], lse [R,W,Nq]) of shared-prefix decode where request r's prompt is rows
    prefix_cu[r]..prefix_cu[r+1]-1 of the packed prompt K/V [T_p, Nkv, D]."""
    q, pk, pv = _bits(q), _bits(prefix_k), _bits(prefix_v)
    sk, sv = _bits(suffix_k), _bits(suffix_v)
    cu = np.ascontiguousarray(prefix_cu, dtype=np.int32)
    r, w, nq, d = q.shape
    nkv = pk.shape[1]
    ls_cap = sk.shape[2]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    out = np.zeros((r, w, nq, d), np.float64)
    lse = np.zeros((r, w, nq), np.float64)
    rc = lib().oracle_shared_prefix_decode_packed(_p(q), _p(pk), _p(pv), _p(cu), _p(sk), _p(sv), r, w, suffix_len,
                                                  ls_cap, nq, nkv, d, float(scale), _p(out), _p(lse), nthreads)
    if rc:
        raise ValueError(f"oracle_shared_prefix_decode_packed rejected its arguments ({rc})")
    return out, lse


def last_token_gather(src: np.ndarray, cu_seqlens) -> np.ndarray:
    """Row cu[i+1]-1 of src ([T, ...], any dtype) for every sequence i; zeros for empty sequences."""
    src = np.ascontiguousarray(src)
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    b = len(cu) - 1
    row_bytes = src[0].nbytes if src.shape[0] else int(np.prod(src.shape[1:])) * src.itemsize
    dst = np.empty((b,) + src.shape[1:], src.dtype)
    rc = lib().oracle_last_token_gather(_p(src), _p(cu), b, row_bytes, _p(dst))
    if rc:
        raise ValueError(f"oracle_last_token_gather rejected its arguments ({rc})")
    return dst


def suffix_reorder(src_k, src_v, parent, suffix_len, src_tokens=None, num_tokens=0):
    """Gathered copies (dst_k, dst_v[, dst_tokens]) ; positions >= suffix_len are left zero."""
    sk, sv = _bits(src_k), _bits(src_v)
    r, w, ls_cap, nkv, d = sk.shape
    par = np.ascontiguousarray(parent, dtype=np.int32)
    dk, dv = np.zeros_like(sk), np.zeros_like(sv)
    st = dt = None
    tok_cap = 0
    if src_tokens is not None:
        st = np.ascontiguousarray(src_tokens, dtype=np.int32)
        tok_cap = st.shape[2]
        dt = np.zeros_like(st)
    rc = lib().oracle_suffix_reorder(_p(sk), _p(sv), _p(dk), _p(dv), _p(par), _p(st), _p(dt), r, w, suffix_len,
                                     ls_cap, nkv, d, num_tokens, tok_cap)
    if rc:
        raise ValueError(f"oracle_suffix_reorder rejected its arguments ({rc})")
    return (dk, dv) if st is None else (dk, dv, dt)


def beam_topk(logits, cum, k_local, k_global, nthreads: int = 0, row_lse=None):
    """Two-stage selection. Returns a dict of numpy arrays:
    tokens/parents/scores [R,k_global], local_tokens/local_scores [R,W_in,k_local],
    row_lse (fp32) and row_lse64 [R,W_in]. With `row_lse` ([R,W_in] fp32) given,
    the rows' fp32 log-sum-exp is taken from it instead of computed."""
    x = _bits(logits)
    r, w_in, vocab = x.shape
    c = None if cum is None else np.ascontiguousarray(cum, dtype=np.float32)
    out = dict(
        tokens=np.zeros((r, k_global), np.int32), parents=np.zeros((r, k_global), np.int32),
        scores=np.zeros((r, k_global), np.float32),
        local_tokens=np.zeros((r, w_in, k_local), np.int32), local_scores=np.zeros((r, w_in, k_local), np.float32),
        row_lse=np.zeros((r, w_in), np.float32), row_lse64=np.zeros((r, w_in), np.float64),
    )
    if row_lse is None:
        rc = lib().oracle_beam_topk(_p(x), _p(c), r, w_in, vocab, k_local, k_global, _p(out["tokens"]),
                                    _p(out["parents"]), _p(out["scores"]), _p(out["local_tokens"]),
                                    _p(out["local_scores"]), _p(out["row_lse"]), _p(out["row_lse64"]), nthreads)
    else:
        given = np.ascontiguousarray(row_lse, dtype=np.float32).reshape(r, w_in)
        rc = lib().oracle_beam_topk_given_lse(_p(x), _p(c), _p(given), r, w_in, vocab, k_local, k_global,
                                              _p(out["tokens"]), _p(out["parents"]), _p(out["scores"]),
                                              _p(out["local_tokens"]), _p(out["local_scores"]), _p(out["row_lse"]),
                                              _p(out["row_lse64"]), nthreads)
    if rc:
        raise ValueError(f"oracle_beam_topk rejected its arguments ({rc})")
    return out


def e4m3_encode(x) -> np.ndarray:
    """OCP E4M3 codes (uint8) of float64 values: round to nearest even, saturating at 448."""
    x = np.ascontiguousarray(x, np.float64)
    out = np.zeros(x.shape, np.uint8)
    if lib().oracle_e4m3_encode_array(_p(x), x.size, _p(out)):
        raise ValueError("oracle_e4m3_encode_array rejected its arguments")
    return out


def e4m3_decode(codes) -> np.ndarray:
    c = np.asarray(codes, np.uint8)
    f = lib().oracle_e4m3_decode
    return np.array([f(int(v)) for v in c.ravel()], np.float64).reshape(c.shape)


def swiglu_quant(gate_up, nthreads: int = 0):
    """Fused SwiGLU requantisation of [T, 2I] bf16 (gate | up). Returns dict(codes uint8 [T, I],
    scale fp64 [T], h fp64 [T, I] (SiLU(gate) * up), x fp64 [T, I] (h / scale))."""
    g = _bits(gate_up)
    t, two_i = g.shape
    i = two_i // 2
    out = dict(codes=np.zeros((t, i), np.uint8), scale=np.zeros(t, np.float64), h=np.zeros((t, i), np.float64),
               x=np.zeros((t, i), np.float64))
    rc = lib().oracle_swiglu_quant(_p(g), t, i, _p(out["codes"]), _p(out["scale"]), _p(out["h"]), _p(out["x"]),
                                   nthreads)
    if rc:
        raise ValueError(f"oracle_swiglu_quant rejected its arguments ({rc})")
    return out
