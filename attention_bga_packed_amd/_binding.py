"""Thin ctypes binding of libbga.so (argument marshalling only).

Every call checks tensor dtypes, devices, contiguity and exact shapes (inputs
and caller-provided outputs alike), allocates missing outputs with torch on the
input's device, and forwards raw device pointers plus the current torch stream
to the C-ABI. All arithmetic happens in the HIP kernels; if the library is
missing, importing this module raises.

The library loaded is attention_bga_packed_amd/libbga.so, or the file named by
the environment variable BGA_LIBRARY (for instance libbga_debug.so, the build
that checks device-side preconditions).
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
RELEASE_LIB_PATH = os.path.join(_HERE, "libbga.so")
DEBUG_LIB_PATH = os.path.join(_HERE, "libbga_debug.so")
LIB_PATH = os.environ.get("BGA_LIBRARY") or RELEASE_LIB_PATH

STATUS_NAMES = {0: "BGA_OK", 1: "BGA_ERR_NULL", 2: "BGA_ERR_SHAPE", 3: "BGA_ERR_UNSUPPORTED",
                4: "BGA_ERR_ALIGN", 5: "BGA_ERR_WORKSPACE", 6: "BGA_ERR_ALIAS", 7: "BGA_ERR_HIP",
                8: "BGA_ERR_PRECONDITION"}

# Every symbol declared in include/bga.h.
EXPORTS = ("bga_packed_gqa_prefill", "bga_shared_prefix_decode", "bga_suffix_reorder",
           "bga_beam_topk_workspace_size", "bga_beam_topk", "bga_status_string", "bga_last_hip_error",
           "bga_version", "bga_debug_build", "bga_last_violations", "bga_beam_topk_noalloc",
           "bga_shared_prefix_decode_packed", "bga_last_token_gather", "bga_beam_advance", "bga_suffix_append",
           "bga_beam_finalize", "bga_swiglu_quant_e4m3")


class BgaError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str = ""):
        self.status = status
        super().__init__(f"{where}: {detail or STATUS_NAMES.get(status, status)}")


def load_library(path: str = LIB_PATH):
    """ctypes handle of a libbga build with every entry point's signature set."""
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m attention_bga_packed_amd.build`")
    L = ctypes.CDLL(path)
    P, i32, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    L.bga_packed_gqa_prefill.argtypes = [P, P, P, P, i32, i32, i32, i32, i32, i32, f32, P, P, P]
    L.bga_shared_prefix_decode.argtypes = [P, P, P, P, P, i32, i32, i32, i32, i32, i32, i32, i32, f32, P, P, P]
    L.bga_shared_prefix_decode_packed.argtypes = [P, P, P, P, i32, P, P, i32, i32, i32, i32, i32, i32, i32, f32, P,
                                                  P, P]
    L.bga_last_token_gather.argtypes = [P, P, i32, i32, ctypes.c_int64, P, P]
    L.bga_beam_advance.argtypes = [P, P, P, i32, i32, i32, i32, i32, P, P, i32, P, P, P, P, P, P, i32, P]
    L.bga_suffix_append.argtypes = [P, P, P, P, i32, i32, i32, i32, i32, i32, P]
    L.bga_swiglu_quant_e4m3.argtypes = [P, i32, i32, P, P, P]
    L.bga_beam_finalize.argtypes = [P, P, P, P, i32, P, P, i32, i32, i32, i32, P, P, P, P, P]
    L.bga_suffix_reorder.argtypes = [P, P, P, P, P, P, P, i32, i32, i32, i32, i32, i32, i32, i32, P]
    L.bga_beam_topk_workspace_size.argtypes = [i32, i32, i32, i32, i32]
    L.bga_beam_topk_workspace_size.restype = sz
    L.bga_beam_topk.argtypes = [P, P, i32, i32, i32, i32, i32, P, P, P, P, P, P, P, sz, P]
    L.bga_beam_topk_noalloc.argtypes = [P, P, i32, i32, i32, i32, i32, P, P, P, P, P, P, P]
    L.bga_status_string.argtypes = [i32]
    L.bga_status_string.restype = ctypes.c_char_p
    L.bga_last_hip_error.argtypes = []
    L.bga_version.argtypes = []
    L.bga_debug_build.argtypes = []
    L.bga_last_violations.argtypes = []
    L.bga_last_violations.restype = ctypes.c_uint32
    for f in (L.bga_packed_gqa_prefill, L.bga_shared_prefix_decode, L.bga_shared_prefix_decode_packed,
              L.bga_last_token_gather, L.bga_suffix_reorder, L.bga_beam_topk, L.bga_beam_advance,
              L.bga_suffix_append, L.bga_beam_finalize, L.bga_swiglu_quant_e4m3,
              L.bga_beam_topk_noalloc, L.bga_last_hip_error, L.bga_version, L.bga_debug_build):
        f.restype = i32
    return L


lib = load_library()


def _check(status: int, where: str):
    if status != 0:
        detail = lib.bga_status_string(status).decode()
        if status == 7:
            detail += f" (hipError {lib.bga_last_hip_error()})"
        if status == 8:
            detail += f" (violations 0x{lib.bga_last_violations():x})"
        raise BgaError(status, where, detail)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _need(t, name, dtype, device=None, ndim=None, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def packed_gqa_prefill(q, k, v, cu_seqlens, max_seqlen: int, softmax_scale=None, out=None, lse=None,
                       want_lse: bool = True):
    """Packed causal GQA prefill. q [T,Nq,D], k/v [T,Nkv,D] bf16; cu_seqlens int32 [B+1] on the GPU.
    Returns (out [T,Nq,D] bf16, lse [T,Nq] fp32 or None)."""
    _need(q, "q", torch.bfloat16, ndim=3)
    dev = q.device
    _need(k, "k", torch.bfloat16, dev, 3)
    _need(v, "v", torch.bfloat16, dev, 3)
    _need(cu_seqlens, "cu_seqlens", torch.int32, dev, 1)
    t, nq, d = q.shape
    nkv = k.shape[1]
    if k.shape != (t, nkv, d) or v.shape != k.shape:
        raise ValueError("k/v must be [T, Nkv, D] matching q")
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", torch.bfloat16, dev, shape=q.shape)
    if lse is None and want_lse:
        lse = torch.empty((t, nq), dtype=torch.float32, device=dev)
    if lse is not None:
        _need(lse, "lse", torch.float32, dev, shape=(t, nq))
    st = lib.bga_packed_gqa_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens), cu_seqlens.numel() - 1, t,
                                    int(max_seqlen), nq, nkv, d, float(softmax_scale), _ptr(out), _ptr(lse),
                                    _stream(q))
    _check(st, "bga_packed_gqa_prefill")
    return out, lse


def shared_prefix_decode(q, prefix_k, prefix_v, suffix_k, suffix_v, suffix_len: int, softmax_scale=None,
                         out=None, lse=None, want_lse: bool = True):
    """Shared-prefix beam decode. q [R,W,Nq,D]; prefix [R,Lp,Nkv,D]; suffix [R,W,Ls_cap,Nkv,D] (bf16).
    Returns (out [R,W,Nq,D] bf16, lse [R,W,Nq] fp32 or None)."""
    _need(q, "q", torch.bfloat16, ndim=4)
    dev = q.device
    _need(prefix_k, "prefix_k", torch.bfloat16, dev, 4)
    _need(prefix_v, "prefix_v", torch.bfloat16, dev, 4)
    _need(suffix_k, "suffix_k", torch.bfloat16, dev, 5)
    _need(suffix_v, "suffix_v", torch.bfloat16, dev, 5)
    r, w, nq, d = q.shape
    lp, nkv = prefix_k.shape[1], prefix_k.shape[2]
    ls_cap = suffix_k.shape[2]
    if prefix_k.shape != (r, lp, nkv, d) or prefix_v.shape != prefix_k.shape:
        raise ValueError("prefix K/V must be [R, Lp, Nkv, D]")
    if suffix_k.shape != (r, w, ls_cap, nkv, d) or suffix_v.shape != suffix_k.shape:
        raise ValueError("suffix K/V must be [R, W, Ls_cap, Nkv, D]")
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", torch.bfloat16, dev, shape=q.shape)
    if lse is None and want_lse:
        lse = torch.empty((r, w, nq), dtype=torch.float32, device=dev)
    if lse is not None:
        _need(lse, "lse", torch.float32, dev, shape=(r, w, nq))
    st = lib.bga_shared_prefix_decode(_ptr(q), _ptr(prefix_k), _ptr(prefix_v), _ptr(suffix_k), _ptr(suffix_v), r, w,
                                      lp, int(suffix_len), ls_cap, nq, nkv, d, float(softmax_scale), _ptr(out),
                                      _ptr(lse), _stream(q))
    _check(st, "bga_shared_prefix_decode")
    return out, lse


def shared_prefix_decode_packed(q, prefix_k, prefix_v, prefix_cu, suffix_k, suffix_v, suffix_len: int,
                                softmax_scale=None, out=None, lse=None, want_lse: bool = True):
    """Shared-prefix beam decode over prompts of their own lengths kept packed: q [R,W,Nq,D]; prefix [T_p,Nkv,D]
    with request r's prompt at rows prefix_cu[r]..prefix_cu[r+1]-1 (prefix_cu int32 [R+1] on the GPU);
    suffix [R,W,Ls_cap,Nkv,D] (bf16). Returns (out [R,W,Nq,D] bf16, lse [R,W,Nq] fp32 or None)."""
    _need(q, "q", torch.bfloat16, ndim=4)
    dev = q.device
    r, w, nq, d = q.shape
    _need(prefix_k, "prefix_k", torch.bfloat16, dev, 3)
    tp, nkv = prefix_k.shape[0], prefix_k.shape[1]
    if prefix_k.shape[2] != d:
        raise ValueError("prefix K/V must be [T_p, Nkv, D]")
    _need(prefix_v, "prefix_v", torch.bfloat16, dev, shape=prefix_k.shape)
    _need(prefix_cu, "prefix_cu", torch.int32, dev, shape=(r + 1,))
    _need(suffix_k, "suffix_k", torch.bfloat16, dev, 5)
    ls_cap = suffix_k.shape[2]
    if suffix_k.shape != (r, w, ls_cap, nkv, d):
        raise ValueError("suffix K/V must be [R, W, Ls_cap, Nkv, D]")
    _need(suffix_v, "suffix_v", torch.bfloat16, dev, shape=suffix_k.shape)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", torch.bfloat16, dev, shape=q.shape)
    if lse is None and want_lse:
        lse = torch.empty((r, w, nq), dtype=torch.float32, device=dev)
    if lse is not None:
        _need(lse, "lse", torch.float32, dev, shape=(r, w, nq))
    st = lib.bga_shared_prefix_decode_packed(_ptr(q), _ptr(prefix_k), _ptr(prefix_v), _ptr(prefix_cu), tp,
                                             _ptr(suffix_k), _ptr(suffix_v), r, w, int(suffix_len), ls_cap, nq, nkv,
                                             d, float(softmax_scale), _ptr(out), _ptr(lse), _stream(q))
    _check(st, "bga_shared_prefix_decode_packed")
    return out, lse


def last_token_gather(src, cu_seqlens, out=None):
    """Row cu[i+1]-1 of src [T, ...] for every sequence i (zeros for an empty one) -> [B, ...]."""
    if not isinstance(src, torch.Tensor) or not src.is_cuda or not src.is_contiguous() or src.dim() < 1:
        raise ValueError("src must be a contiguous GPU tensor [T, ...]")
    dev = src.device
    _need(cu_seqlens, "cu_seqlens", torch.int32, dev, 1)
    b = cu_seqlens.numel() - 1
    row_bytes = src.element_size() * (src[0].numel() if src.shape[0] else int(math.prod(src.shape[1:])))
    if out is None:
        out = torch.empty((b,) + tuple(src.shape[1:]), dtype=src.dtype, device=dev)
    _need(out, "out", src.dtype, dev, shape=(b,) + tuple(src.shape[1:]))
    st = lib.bga_last_token_gather(_ptr(src), _ptr(cu_seqlens), b, src.shape[0], int(row_bytes), _ptr(out),
                                   _stream(src))
    _check(st, "bga_last_token_gather")
    return out


def suffix_reorder(src_k, src_v, parent, suffix_len: int, dst_k=None, dst_v=None, src_tokens=None,
                   dst_tokens=None, num_tokens: int = 0):
    """Gather suffix K/V (and optionally token history) by parent index, out of place.
    src/dst [R,W,Ls_cap,Nkv,D] bf16; parent [R,W] int32; tokens [R,W,tok_cap] int32."""
    _need(src_k, "src_k", torch.bfloat16, ndim=5)
    dev = src_k.device
    r, w, ls_cap, nkv, d = src_k.shape
    _need(src_v, "src_v", torch.bfloat16, dev, shape=src_k.shape)
    _need(parent, "parent", torch.int32, dev, shape=(r, w))
    if dst_k is None:
        dst_k = torch.empty_like(src_k)
    if dst_v is None:
        dst_v = torch.empty_like(src_v)
    _need(dst_k, "dst_k", torch.bfloat16, dev, shape=src_k.shape)
    _need(dst_v, "dst_v", torch.bfloat16, dev, shape=src_k.shape)
    tok_cap = 0
    if src_tokens is None and dst_tokens is not None:
        raise ValueError("dst_tokens given without src_tokens")
    if src_tokens is not None:
        _need(src_tokens, "src_tokens", torch.int32, dev, 3)
        if src_tokens.shape[:2] != (r, w):
            raise ValueError(f"src_tokens must be [R, W, tok_cap] with R, W = {r}, {w}")
        tok_cap = src_tokens.shape[2]
        if dst_tokens is None:
            dst_tokens = torch.empty_like(src_tokens)
        _need(dst_tokens, "dst_tokens", torch.int32, dev, shape=src_tokens.shape)
    st = lib.bga_suffix_reorder(_ptr(src_k), _ptr(src_v), _ptr(dst_k), _ptr(dst_v), _ptr(parent), _ptr(src_tokens),
                                _ptr(dst_tokens), r, w, int(suffix_len), ls_cap, nkv, d, int(num_tokens), tok_cap,
                                _stream(src_k))
    _check(st, "bga_suffix_reorder")
    return (dst_k, dst_v) if src_tokens is None else (dst_k, dst_v, dst_tokens)


def beam_topk_workspace_size(num_requests, num_src_beams, vocab, k_local, k_global) -> int:
    return int(lib.bga_beam_topk_workspace_size(num_requests, num_src_beams, vocab, k_local, k_global))


def _topk_outputs(logits, cum_scores, k_local, k_global, want_local, want_lse, out):
    """Checked (and, where missing, allocated) output tensors of a beam top-K call."""
    _need(logits, "logits", torch.bfloat16, ndim=3)
    dev = logits.device
    r, w_in, vocab = logits.shape
    if cum_scores is not None:
        _need(cum_scores, "cum_scores", torch.float32, dev, shape=(r, w_in))
    res = out if out is not None else {}
    shapes = {"tokens": ((r, k_global), torch.int32), "parents": ((r, k_global), torch.int32),
              "scores": ((r, k_global), torch.float32)}
    if want_local or "local_tokens" in res or "local_scores" in res:
        shapes["local_tokens"] = ((r, w_in, k_local), torch.int32)
        shapes["local_scores"] = ((r, w_in, k_local), torch.float32)
    if want_lse or "row_lse" in res:
        shapes["row_lse"] = ((r, w_in), torch.float32)
    unknown = set(res) - set(shapes)
    if unknown:
        raise ValueError(f"unknown beam_topk outputs {sorted(unknown)}")
    for key, (shape, dtype) in shapes.items():
        if key not in res:
            res[key] = torch.empty(shape, dtype=dtype, device=dev)
        _need(res[key], key, dtype, dev, shape=shape)
    return res


def beam_topk(logits, cum_scores, k_local: int, k_global: int, workspace=None, want_local: bool = False,
              want_lse: bool = False, out=None):
    """Two-stage beam candidate selection. logits [R,W_in,V] bf16; cum_scores [R,W_in] fp32 or None.
    Returns dict(tokens, parents, scores[, local_tokens, local_scores][, row_lse])."""
    res = _topk_outputs(logits, cum_scores, k_local, k_global, want_local, want_lse, out)
    r, w_in, vocab = logits.shape
    need = beam_topk_workspace_size(r, w_in, vocab, k_local, k_global)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=logits.device)
    _need(workspace, "workspace", torch.uint8, logits.device, 1)
    st = lib.bga_beam_topk(_ptr(logits), _ptr(cum_scores), r, w_in, vocab, int(k_local), int(k_global),
                           _ptr(res["tokens"]), _ptr(res["parents"]), _ptr(res["scores"]),
                           _ptr(res.get("local_tokens")), _ptr(res.get("local_scores")), _ptr(res.get("row_lse")),
                           _ptr(workspace), workspace.numel(), _stream(logits))
    _check(st, "bga_beam_topk")
    return res


def beam_topk_noalloc(logits, cum_scores, k_local: int, k_global: int, out: dict, want_local: bool = False,
                      want_lse: bool = False):
    """bga_beam_topk_noalloc: beam_topk with the library's own per-device workspace. Every output tensor
    must be passed in `out` (tokens, parents, scores, and local_tokens/local_scores/row_lse when wanted):
    nothing is allocated on this path."""
    r, w_in, vocab = logits.shape
    keys = {"tokens", "parents", "scores"} | ({"local_tokens", "local_scores"} if want_local else set()) | \
        ({"row_lse"} if want_lse else set())
    missing = keys - set(out)
    if missing:
        raise ValueError(f"beam_topk_noalloc allocates nothing: pass {sorted(missing)} in out")
    res = _topk_outputs(logits, cum_scores, k_local, k_global, want_local, want_lse, out)
    st = lib.bga_beam_topk_noalloc(_ptr(logits), _ptr(cum_scores), r, w_in, vocab, int(k_local), int(k_global),
                                   _ptr(res["tokens"]), _ptr(res["parents"]), _ptr(res["scores"]),
                                   _ptr(res.get("local_tokens")), _ptr(res.get("local_scores")),
                                   _ptr(res.get("row_lse")), _stream(logits))
    _check(st, "bga_beam_topk_noalloc")
    return res


def beam_advance(cand_tokens, cand_parents, cand_scores, beam_width: int, stop_token: int, step: int, tokens_in,
                 tokens_out, parents_out, cum_out, pool: dict):
    """The 2W stop-token rule of one beam-search step (bga_beam_advance). cand_* [R, 2W] (best first);
    tokens_in [R, W_in, tok_cap], tokens_out [R, W, tok_cap] int32; parents_out [R, W] int32, cum_out [R, W] fp32;
    pool = dict(scores [R, P] fp32, lengths [R, P] int32, tokens [R, P, tok_cap] int32, count [R] int32)."""
    _need(cand_tokens, "cand_tokens", torch.int32, ndim=2)
    dev = cand_tokens.device
    r, k2 = cand_tokens.shape
    w = int(beam_width)
    if k2 != 2 * w:
        raise ValueError(f"expected 2W = {2 * w} candidates per request, got {k2}")
    _need(cand_parents, "cand_parents", torch.int32, dev, shape=(r, k2))
    _need(cand_scores, "cand_scores", torch.float32, dev, shape=(r, k2))
    _need(tokens_in, "tokens_in", torch.int32, dev, 3)
    w_in, tok_cap = tokens_in.shape[1], tokens_in.shape[2]
    if tokens_in.shape[0] != r:
        raise ValueError("tokens_in must be [R, W_in, tok_cap]")
    _need(tokens_out, "tokens_out", torch.int32, dev, shape=(r, w, tok_cap))
    _need(parents_out, "parents_out", torch.int32, dev, shape=(r, w))
    _need(cum_out, "cum_out", torch.float32, dev, shape=(r, w))
    p = pool["scores"].shape[1] if isinstance(pool.get("scores"), torch.Tensor) else 0
    _need(pool["scores"], "pool scores", torch.float32, dev, shape=(r, p))
    _need(pool["lengths"], "pool lengths", torch.int32, dev, shape=(r, p))
    _need(pool["tokens"], "pool tokens", torch.int32, dev, shape=(r, p, tok_cap))
    _need(pool["count"], "pool count", torch.int32, dev, shape=(r,))
    st = lib.bga_beam_advance(_ptr(cand_tokens), _ptr(cand_parents), _ptr(cand_scores), r, w_in, w, int(stop_token),
                              int(step), _ptr(tokens_in), _ptr(tokens_out), tok_cap, _ptr(parents_out), _ptr(cum_out),
                              _ptr(pool["scores"]), _ptr(pool["lengths"]), _ptr(pool["tokens"]), _ptr(pool["count"]),
                              p, _stream(cand_tokens))
    _check(st, "bga_beam_advance")


def suffix_append(new_k, new_v, suffix_k, suffix_v, pos: int):
    """new_k/new_v [R, W, Nkv, D] into suffix position pos of suffix_k/suffix_v [R, W, cap, Nkv, D] (bf16)."""
    _need(suffix_k, "suffix_k", torch.bfloat16, ndim=5)
    dev = suffix_k.device
    r, w, cap, nkv, d = suffix_k.shape
    _need(suffix_v, "suffix_v", torch.bfloat16, dev, shape=suffix_k.shape)
    _need(new_k, "new_k", torch.bfloat16, dev, shape=(r, w, nkv, d))
    _need(new_v, "new_v", torch.bfloat16, dev, shape=(r, w, nkv, d))
    st = lib.bga_suffix_append(_ptr(new_k), _ptr(new_v), _ptr(suffix_k), _ptr(suffix_v), r, w, int(pos), cap, nkv, d,
                               _stream(suffix_k))
    _check(st, "bga_suffix_append")


def beam_finalize(pool: dict, cum, tokens, length: int, out: dict | None = None):
    """Finished pool + last beams ranked by score, best first (bga_beam_finalize). Returns
    dict(scores [R, P+W], lengths [R, P+W], tokens [R, P+W, tok_cap], count [R])."""
    _need(cum, "cum", torch.float32, ndim=2)
    dev = cum.device
    r, w = cum.shape
    _need(tokens, "tokens", torch.int32, dev, 3)
    tok_cap = tokens.shape[2]
    if tokens.shape[:2] != (r, w):
        raise ValueError("tokens must be [R, W, tok_cap]")
    p = pool["scores"].shape[1]
    _need(pool["scores"], "pool scores", torch.float32, dev, shape=(r, p))
    _need(pool["lengths"], "pool lengths", torch.int32, dev, shape=(r, p))
    _need(pool["tokens"], "pool tokens", torch.int32, dev, shape=(r, p, tok_cap))
    _need(pool["count"], "pool count", torch.int32, dev, shape=(r,))
    out = {} if out is None else out
    shapes = {"scores": ((r, p + w), torch.float32), "lengths": ((r, p + w), torch.int32),
              "tokens": ((r, p + w, tok_cap), torch.int32), "count": ((r,), torch.int32)}
    for key, (shape, dtype) in shapes.items():
        if key not in out:
            out[key] = torch.empty(shape, dtype=dtype, device=dev)
        _need(out[key], key, dtype, dev, shape=shape)
    st = lib.bga_beam_finalize(_ptr(pool["scores"]), _ptr(pool["lengths"]), _ptr(pool["tokens"]), _ptr(pool["count"]),
                               p, _ptr(cum), _ptr(tokens), r, w, int(length), tok_cap, _ptr(out["scores"]),
                               _ptr(out["lengths"]), _ptr(out["tokens"]), _ptr(out["count"]), _stream(cum))
    _check(st, "bga_beam_finalize")
    return out


def swiglu_quant_e4m3(gate_up, codes=None, scale=None):
    """Fused SwiGLU + per-token E4M3 requantisation. gate_up [T, 2I] bf16 (gate | up).
    Returns (codes [T, I] uint8 E4M3, scale [T] fp32) with h ~= decode(code) * scale."""
    _need(gate_up, "gate_up", torch.bfloat16, ndim=2)
    dev = gate_up.device
    t, two_i = gate_up.shape
    if two_i % 2:
        raise ValueError("gate_up must be [T, 2I]")
    i = two_i // 2
    if codes is None:
        codes = torch.empty((t, i), dtype=torch.uint8, device=dev)
    _need(codes, "codes", torch.uint8, dev, shape=(t, i))
    if scale is None:
        scale = torch.empty((t,), dtype=torch.float32, device=dev)
    _need(scale, "scale", torch.float32, dev, shape=(t,))
    st = lib.bga_swiglu_quant_e4m3(_ptr(gate_up), t, i, _ptr(codes), _ptr(scale), _stream(gate_up))
    _check(st, "bga_swiglu_quant_e4m3")
    return codes, scale
