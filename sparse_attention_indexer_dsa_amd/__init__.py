"""Python binding of libdsa_index.so, the MI355X (gfx950) DSA lightning-indexer hot path.

Argument marshalling only: every step runs in the HIP kernels behind the C ABI declared
in ``include/dsa_index.h``. PyTorch supplies device memory and the current HIP stream.
There is no CPU fallback: if the library is missing, importing the binding's functions
raises.

Entry points (same names as the C ABI):

* ``preprocess``       - key LayerNorm -> RoPE (fp32) fused with quantisation to the
                         scoring operands (bf16, fp8 per-vector, mxfp8 per-32).
* ``kpool``            - KPool compression of keys into pooled keys.
* ``workspace_size``   - bytes of score workspace ``score_topk`` needs.
* ``score_topk``       - scores of all causal candidates, then the per-row top-k
                         (and pool expansion when kpool > 1).
* ``score``, ``topk``  - the two halves of ``score_topk`` (score rows into the
                         workspace; selection from it).

Status codes 1 (invalid argument) and 2 (unsupported) raise ``ValueError``; 3 (workspace
too small) and 4 (device error) raise ``RuntimeError``.
"""

import ctypes
import os

import torch

__all__ = ["preprocess", "kpool", "workspace_size", "score_topk", "score_topk_noalloc", "NOALLOC_SCRATCH_BYTES",
           "score", "score_fused", "topk", "forward",
           "forward_workspace_size", "selection_softmax", "sparse_attention", "bench_mfma", "bench_stream",
           "library_path", "load", "PRECISIONS", "DsaError"]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_NAME = "libdsa_index.so"
PRECISIONS = {"bf16": 0, "fp8": 1, "mxfp8": 2}
_DTYPES = {torch.bfloat16: 0, torch.float32: 1}

_lib = None


class DsaError(RuntimeError):
    pass


def library_path():
    return os.path.join(_HERE, LIB_NAME)


def load():
    """Load the in-tree HIP library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m sparse_attention_indexer_dsa_amd.build` "
                          "(there is no fallback path)")
    lib = ctypes.CDLL(path)
    vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    lib.dsa_index_preprocess.restype = i32
    lib.dsa_index_preprocess.argtypes = [vp, vp, i32, i32, i32, i32, i32, vp, i32, vp, vp, f32, vp, vp,
                                         i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp]
    lib.dsa_index_kpool.restype = i32
    lib.dsa_index_kpool.argtypes = [vp, i32, i32, i32, vp, i32, vp, vp, i32, i32, vp, vp, vp, vp]
    lib.dsa_index_workspace_size.restype = sz
    lib.dsa_index_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32, i32, i32]
    lib.dsa_index_score_topk.restype = i32
    lib.dsa_index_score_topk.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, vp, i32, i32, i32, vp,
                                         i32, i32, f32, i32, vp, vp, vp, vp, vp, sz, vp]
    lib.dsa_index_score_topk_noalloc.restype = i32
    lib.dsa_index_score_topk_noalloc.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, vp, i32, i32, i32,
                                                 vp, i32, i32, f32, i32, vp, vp, vp, vp, vp]
    lib.dsa_index_score.restype = i32
    lib.dsa_index_score.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, vp, i32, i32, i32, vp,
                                    f32, i32, vp, sz, vp]
    lib.dsa_index_topk.restype = i32
    lib.dsa_index_topk.argtypes = [vp, sz, i32, vp, i32, i32, i32, vp, i32, i32, vp, vp, vp, vp, vp]
    lib.dsa_index_forward_workspace_size.restype = sz
    lib.dsa_index_forward_workspace_size.argtypes = [i32, i32, i32, i32]
    lib.dsa_index_forward.restype = i32
    lib.dsa_index_forward.argtypes = [vp, vp, i32, vp, i32, i32, i32, i32, vp, i32, i32, vp, vp, f32, vp, vp,
                                      i32, i32, i32, i32, i32, f32, i32, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.dsa_index_selection_softmax.restype = i32
    lib.dsa_index_selection_softmax.argtypes = [vp, i32, i32, vp, vp]
    lib.dsa_index_sparse_attention.restype = i32
    lib.dsa_index_sparse_attention.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32, vp, vp, vp]
    lib.dsa_index_score_fused.restype = i32
    lib.dsa_index_score_fused.argtypes = [vp, i32, vp, vp, vp, i32, i32, i32, i32, i32, vp, i32, i32, vp, vp, i32,
                                          i32, i32, i32, f32, i32, vp, vp, vp, sz, vp]
    lib.dsa_bench_mfma.restype = i32
    lib.dsa_bench_mfma.argtypes = [i32, i32, i32, vp, vp]
    lib.dsa_bench_mfma_flops.restype = ctypes.c_double
    lib.dsa_bench_mfma_flops.argtypes = [i32, i32, i32]
    lib.dsa_bench_stream.restype = i32
    lib.dsa_bench_stream.argtypes = [vp, vp, sz, i32, vp]
    lib.dsa_last_error.restype = ctypes.c_char_p
    lib.dsa_last_error.argtypes = []
    _lib = lib
    return lib


def _check(status, what):
    if status == 0:
        return
    msg = load().dsa_last_error().decode(errors="replace")
    if status in (1, 2):
        raise ValueError(f"{what}: {msg}")
    raise DsaError(f"{what} (status {status}): {msg}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _prec(precision):
    if isinstance(precision, int):
        return precision
    if precision not in PRECISIONS:
        raise ValueError(f"unsupported DSA indexer scoring precision {precision!r}; expected bf16, fp8 or mxfp8")
    return PRECISIONS[precision]


def _need(t, name, dtypes=None, device=None):
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtypes is not None and t.dtype not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")


def _op_dtype(prec):
    return torch.bfloat16 if prec == 0 else torch.uint8


def preprocess(q=None, k=None, cu_seqlens=None, *, ln_gamma=None, ln_beta=None, ln_eps=1e-6,
               rope_cos=None, rope_sin=None, rope_dim=0, rope_interleaved=False, rope_fp32=False,
               precision="bf16", return_fp32=False, out=None):
    """Scoring operands of q [T,H,D] and/or k [S,D] (bf16 or fp32 inputs).

    Returns a dict with 'q_op', 'q_scale', 'k_op', 'k_scale' (and 'q_f32', 'k_f32' when
    ``return_fp32``). ``out`` may supply preallocated tensors under the same keys.
    """
    lib = load()
    prec = _prec(precision)
    src = q if q is not None else k
    if src is None:
        raise ValueError("q and k are both None")
    dev = src.device
    in_dtype = src.dtype
    if in_dtype not in _DTYPES:
        raise ValueError(f"inputs must be bf16 or fp32, got {in_dtype}")
    for name, t in (("q", q), ("k", k)):
        _need(t, name, (in_dtype,))
    _need(cu_seqlens, "cu_seqlens", (torch.int32,))
    if cu_seqlens is None:
        raise ValueError("cu_seqlens is required")
    for name, t in (("ln_gamma", ln_gamma), ("ln_beta", ln_beta), ("rope_cos", rope_cos), ("rope_sin", rope_sin)):
        _need(t, name, (torch.float32,))
    T, H, D = q.shape if q is not None else (0, 0, k.shape[1])
    S = k.shape[0] if k is not None else 0
    if q is None:
        H = 16
    out = dict(out or {})
    odt = _op_dtype(prec)
    nsb = {0: None, 1: 1, 2: D // 32}[prec]
    if q is not None:
        out.setdefault("q_op", torch.empty((T, H, D), dtype=odt, device=dev))
        if nsb is not None:
            out.setdefault("q_scale", torch.empty((T, H) if prec == 1 else (T, H, nsb), dtype=torch.uint8, device=dev))
        if return_fp32:
            out.setdefault("q_f32", torch.empty((T, H, D), dtype=torch.float32, device=dev))
    if k is not None:
        out.setdefault("k_op", torch.empty((S, D), dtype=odt, device=dev))
        if nsb is not None:
            out.setdefault("k_scale", torch.empty((S,) if prec == 1 else (S, nsb), dtype=torch.uint8, device=dev))
        if return_fp32:
            out.setdefault("k_f32", torch.empty((S, D), dtype=torch.float32, device=dev))
    max_pos = rope_cos.shape[0] if (rope_cos is not None and rope_dim) else 0
    st = lib.dsa_index_preprocess(
        _ptr(q), _ptr(k), _DTYPES[in_dtype], T, S, H, D, _ptr(cu_seqlens), cu_seqlens.numel() - 1,
        _ptr(ln_gamma), _ptr(ln_beta), float(ln_eps), _ptr(rope_cos), _ptr(rope_sin),
        int(rope_dim), int(max_pos), int(bool(rope_interleaved)), int(bool(rope_fp32)), prec,
        _ptr(out.get("q_op")), _ptr(out.get("q_scale")), _ptr(out.get("k_op")), _ptr(out.get("k_scale")),
        _ptr(out.get("q_f32")), _ptr(out.get("k_f32")), _stream(dev))
    _check(st, "dsa_index_preprocess")
    return out


def kpool(k, cu_seqlens, gate, slot_bias, kpool, *, precision="bf16", out=None):
    """Pooled keys of k [S,D]: returns (pooled_op [S//kpool, D], pooled_scale or None, cu_pools [B+1]).

    ``gate`` is bf16 [S] (torch.bfloat16, or int16/uint16 bit patterns); ``slot_bias``
    fp32 [kpool]. Only the first cu_pools[-1] rows of pooled_op are meaningful.
    """
    lib = load()
    prec = _prec(precision)
    if k.dtype not in _DTYPES:
        raise ValueError(f"k must be bf16 or fp32, got {k.dtype}")
    _need(k, "k")
    _need(cu_seqlens, "cu_seqlens", (torch.int32,))
    _need(gate, "gate", (torch.bfloat16, torch.int16, torch.uint16))
    _need(slot_bias, "slot_bias", (torch.float32,))
    S, D = k.shape
    dev = k.device
    out = dict(out or {})
    P = S // kpool
    pooled = out.get("pooled_op")
    if pooled is None:
        pooled = torch.empty((P, D), dtype=_op_dtype(prec), device=dev)
    scale = out.get("pooled_scale")
    if scale is None and prec != 0:
        scale = torch.empty((P,) if prec == 1 else (P, D // 32), dtype=torch.uint8, device=dev)
    cu_pools = out.get("cu_pools")
    if cu_pools is None:
        cu_pools = torch.empty(cu_seqlens.numel(), dtype=torch.int32, device=dev)
    st = lib.dsa_index_kpool(_ptr(k), _DTYPES[k.dtype], S, D, _ptr(cu_seqlens), cu_seqlens.numel() - 1,
                             _ptr(gate), _ptr(slot_bias), int(kpool), prec, _ptr(pooled), _ptr(scale),
                             _ptr(cu_pools), _stream(dev))
    _check(st, "dsa_index_kpool")
    return pooled, scale, cu_pools


def workspace_size(T, max_seqlen, topk, kpool=1, H=64, D=128, num_seqs=1, precision="bf16"):
    return int(load().dsa_index_workspace_size(int(T), int(H), int(D), int(num_seqs), int(max_seqlen),
                                               int(topk), int(kpool), _prec(precision)))


def score_topk(q_op, k_op, w, cu_seqlens, max_seqlen, topk, *, q_scale=None, k_scale=None,
               precision="bf16", sm_scale=1.0, kpool=1, cu_pools=None, kpool_tail=True,
               workspace=None, out=None):
    """Per-row top-k of the indexer scores.

    Returns a dict: 'indices' ([T,topk] global key rows, or [T, topk*kpool+kpool-1]
    expanded token indices when kpool > 1), 'scores' [T,topk], 'lengths' [T] and, when
    kpool > 1, 'pool_indices' [T,topk]. ``workspace`` (uint8, at least
    ``workspace_size(...)`` bytes) and ``out`` allow preallocated buffers.
    """
    lib = load()
    prec = _prec(precision)
    T, H, D = q_op.shape
    S = k_op.shape[0]
    dev = q_op.device
    for name, t in (("q_op", q_op), ("k_op", k_op), ("w", w), ("q_scale", q_scale), ("k_scale", k_scale),
                    ("cu_pools", cu_pools)):
        _need(t, name)
    _need(cu_seqlens, "cu_seqlens", (torch.int32,))
    if w.dtype not in _DTYPES:
        raise ValueError(f"w must be bf16 or fp32, got {w.dtype}")
    B = cu_seqlens.numel() - 1
    out = dict(out or {})
    width = topk if kpool == 1 else topk * kpool + kpool - 1
    out.setdefault("indices", torch.empty((T, width), dtype=torch.int32, device=dev))
    out.setdefault("scores", torch.empty((T, topk), dtype=torch.float32, device=dev))
    out.setdefault("lengths", torch.empty((T,), dtype=torch.int32, device=dev))
    if kpool > 1:
        out.setdefault("pool_indices", torch.empty((T, topk), dtype=torch.int32, device=dev))
    need = workspace_size(T, max_seqlen, topk, kpool, H, D, B, prec)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    st = lib.dsa_index_score_topk(
        _ptr(q_op), _ptr(q_scale), _ptr(k_op), _ptr(k_scale), _ptr(w), _DTYPES[w.dtype],
        T, S, H, D, _ptr(cu_seqlens), B, int(max_seqlen), int(kpool), _ptr(cu_pools), int(bool(kpool_tail)),
        int(topk), float(sm_scale), prec, _ptr(out["indices"]), _ptr(out["scores"]), _ptr(out["lengths"]),
        _ptr(out.get("pool_indices")), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(dev))
    _check(st, "dsa_index_score_topk")
    return out


# Bytes of the fixed device scratch score_topk_noalloc uses (DSA_NOALLOC_SCRATCH_BYTES).
NOALLOC_SCRATCH_BYTES = (128 << 20) + 4096


def score_topk_noalloc(q_op, k_op, w, cu_seqlens, max_seqlen, topk, *, out, q_scale=None, k_scale=None,
                       precision="bf16", sm_scale=1.0, kpool=1, cu_pools=None, kpool_tail=True):
    """``score_topk`` through dsa_index_score_topk_noalloc: no workspace; the score rows go to
    the library's fixed device scratch (NOALLOC_SCRATCH_BYTES per GPU, shared by every call
    on that GPU; calls that overlap on one GPU race). ``out`` must hold preallocated
    'indices', 'scores', 'lengths' (and 'pool_indices' or not, when kpool > 1), shaped as
    ``score_topk`` returns them; nothing is allocated here."""
    lib = load()
    prec = _prec(precision)
    T, H, D = q_op.shape
    S = k_op.shape[0]
    for name, t in (("q_op", q_op), ("k_op", k_op), ("w", w), ("q_scale", q_scale), ("k_scale", k_scale),
                    ("cu_pools", cu_pools)):
        _need(t, name)
    _need(cu_seqlens, "cu_seqlens", (torch.int32,))
    if w.dtype not in _DTYPES:
        raise ValueError(f"w must be bf16 or fp32, got {w.dtype}")
    width = topk if kpool == 1 else topk * kpool + kpool - 1
    for name, shape, dt in (("indices", (T, width), torch.int32), ("scores", (T, topk), torch.float32),
                            ("lengths", (T,), torch.int32)):
        t = out.get(name)
        if t is None or tuple(t.shape) != shape or t.dtype != dt:
            raise ValueError(f"out['{name}'] must be a preallocated {dt} tensor of shape {shape}")
        _need(t, name)
    pool = out.get("pool_indices") if kpool > 1 else None
    if pool is not None and (tuple(pool.shape) != (T, topk) or pool.dtype != torch.int32):
        raise ValueError(f"out['pool_indices'] must be an int32 tensor of shape {(T, topk)}")
    _need(pool, "pool_indices")
    st = lib.dsa_index_score_topk_noalloc(
        _ptr(q_op), _ptr(q_scale), _ptr(k_op), _ptr(k_scale), _ptr(w), _DTYPES[w.dtype],
        T, S, H, D, _ptr(cu_seqlens), cu_seqlens.numel() - 1, int(max_seqlen), int(kpool), _ptr(cu_pools),
        int(bool(kpool_tail)), int(topk), float(sm_scale), prec, _ptr(out["indices"]), _ptr(out["scores"]),
        _ptr(out["lengths"]), _ptr(pool), _stream(q_op.device))
    _check(st, "dsa_index_score_topk_noalloc")
    return out


def score_fused(q, k_op, w, cu_seqlens, max_seqlen, workspace, *, k_scale=None, rope_cos=None, rope_sin=None,
                rope_dim=0, rope_interleaved=False, rope_fp32=False, precision="bf16", sm_scale=1.0,
                out_operands=None):
    """Scores into ``workspace`` from raw queries q [T,H,D] (the query preprocessing runs inside
    the scoring kernel) and preprocessed keys. ``out_operands`` may hold 'q_op' / 'q_scale'
    tensors to receive the query operands the kernel built."""
    lib = load()
    prec = _prec(precision)
    T, H, D = q.shape
    S = k_op.shape[0]
    if q.dtype not in _DTYPES or w.dtype not in _DTYPES:
        raise ValueError("q and w must be bf16 or fp32")
    for name, t in (("q", q), ("k_op", k_op), ("w", w), ("k_scale", k_scale)):
        _need(t, name)
    _need(cu_seqlens, "cu_seqlens", (torch.int32,))
    ops = out_operands or {}
    max_pos = rope_cos.shape[0] if (rope_cos is not None and rope_dim) else 0
    st = lib.dsa_index_score_fused(
        _ptr(q), _DTYPES[q.dtype], _ptr(k_op), _ptr(k_scale), _ptr(w), _DTYPES[w.dtype], T, S, H, D,
        _ptr(cu_seqlens), cu_seqlens.numel() - 1, int(max_seqlen), _ptr(rope_cos), _ptr(rope_sin), int(rope_dim),
        int(max_pos), int(bool(rope_interleaved)), int(bool(rope_fp32)), float(sm_scale), prec,
        _ptr(ops.get("q_op")), _ptr(ops.get("q_scale")), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(q.device))
    _check(st, "dsa_index_score_fused")
    return workspace


def forward_workspace_size(T, D, max_seqlen, precision="bf16"):
    """Bytes of workspace `forward` needs."""
    return int(load().dsa_index_forward_workspace_size(int(T), int(D), int(max_seqlen), _prec(precision)))


def forward(q, k, w, cu_seqlens, max_seqlen, topk, *, ln_gamma=None, ln_beta=None, ln_eps=1e-6,
            rope_cos=None, rope_sin=None, rope_dim=0, rope_interleaved=False, rope_fp32=False,
            precision="bf16", sm_scale=1.0, return_operands=False, workspace=None, out=None):
    """The whole hot path in one call (kpool 1): key preprocessing, scoring with the query
    preprocessing done inside the scoring kernel, top-k.

    Returns a dict with 'indices' [T,topk], 'scores' [T,topk], 'lengths' [T] and, with
    ``return_operands``, the query operands the scoring kernel built ('q_op', 'q_scale').
    """
    lib = load()
    prec = _prec(precision)
    T, H, D = q.shape
    dev = q.device
    if q.dtype not in _DTYPES or k.dtype != q.dtype:
        raise ValueError(f"q and k must both be bf16 or both fp32, got {q.dtype} and {k.dtype}")
    if w.dtype not in _DTYPES:
        raise ValueError(f"w must be bf16 or fp32, got {w.dtype}")
    for name, t in (("q", q), ("k", k), ("w", w)):
        _need(t, name)
    _need(cu_seqlens, "cu_seqlens", (torch.int32,))
    for name, t in (("ln_gamma", ln_gamma), ("ln_beta", ln_beta), ("rope_cos", rope_cos), ("rope_sin", rope_sin)):
        _need(t, name, (torch.float32,))
    out = _alloc_outputs(out, T, topk, 1, dev)
    if return_operands:
        out.setdefault("q_op", torch.empty((T, H, D), dtype=_op_dtype(prec), device=dev))
        if prec != 0:
            out.setdefault("q_scale", torch.empty((T, H) if prec == 1 else (T, H, D // 32), dtype=torch.uint8,
                                                  device=dev))
    need = forward_workspace_size(T, D, max_seqlen, precision)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    max_pos = rope_cos.shape[0] if (rope_cos is not None and rope_dim) else 0
    st = lib.dsa_index_forward(
        _ptr(q), _ptr(k), _DTYPES[q.dtype], _ptr(w), _DTYPES[w.dtype], T, H, D, _ptr(cu_seqlens),
        cu_seqlens.numel() - 1, int(max_seqlen), _ptr(ln_gamma), _ptr(ln_beta), float(ln_eps), _ptr(rope_cos),
        _ptr(rope_sin), int(rope_dim), int(max_pos), int(bool(rope_interleaved)), int(bool(rope_fp32)), int(topk),
        float(sm_scale), prec, _ptr(out["indices"]), _ptr(out["scores"]), _ptr(out["lengths"]),
        _ptr(out.get("q_op")), _ptr(out.get("q_scale")), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(dev))
    _check(st, "dsa_index_forward")
    out["workspace"] = workspace
    return out


def _alloc_outputs(out, T, topk, kpool, dev):
    out = dict(out or {})
    width = topk if kpool == 1 else topk * kpool + kpool - 1
    out.setdefault("indices", torch.empty((T, width), dtype=torch.int32, device=dev))
    out.setdefault("scores", torch.empty((T, topk), dtype=torch.float32, device=dev))
    out.setdefault("lengths", torch.empty((T,), dtype=torch.int32, device=dev))
    if kpool > 1:
        out.setdefault("pool_indices", torch.empty((T, topk), dtype=torch.int32, device=dev))
    return out


def score(q_op, k_op, w, cu_seqlens, max_seqlen, workspace, *, q_scale=None, k_scale=None, precision="bf16",
          sm_scale=1.0, kpool=1, cu_pools=None):
    """Scores of every causal candidate into ``workspace`` (row t at t*stride, see the C header)."""
    lib = load()
    prec = _prec(precision)
    T, H, D = q_op.shape
    S = k_op.shape[0]
    for name, t in (("q_op", q_op), ("k_op", k_op), ("w", w), ("q_scale", q_scale), ("k_scale", k_scale),
                    ("cu_pools", cu_pools), ("workspace", workspace)):
        _need(t, name)
    _need(cu_seqlens, "cu_seqlens", (torch.int32,))
    if w.dtype not in _DTYPES:
        raise ValueError(f"w must be bf16 or fp32, got {w.dtype}")
    st = lib.dsa_index_score(
        _ptr(q_op), _ptr(q_scale), _ptr(k_op), _ptr(k_scale), _ptr(w), _DTYPES[w.dtype], T, S, H, D,
        _ptr(cu_seqlens), cu_seqlens.numel() - 1, int(max_seqlen), int(kpool), _ptr(cu_pools), float(sm_scale),
        prec, _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(q_op.device))
    _check(st, "dsa_index_score")
    return workspace


def topk(workspace, T, cu_seqlens, max_seqlen, topk, *, kpool=1, cu_pools=None, kpool_tail=True, out=None):
    """Per-row selection from the score rows ``score`` wrote; same outputs as ``score_topk``."""
    lib = load()
    _need(workspace, "workspace")
    _need(cu_seqlens, "cu_seqlens", (torch.int32,))
    _need(cu_pools, "cu_pools")
    out = _alloc_outputs(out, T, topk, kpool, workspace.device)
    st = lib.dsa_index_topk(
        _ptr(workspace), workspace.numel() * workspace.element_size(), int(T), _ptr(cu_seqlens),
        cu_seqlens.numel() - 1, int(max_seqlen), int(kpool), _ptr(cu_pools), int(bool(kpool_tail)), int(topk),
        _ptr(out["indices"]), _ptr(out["scores"]), _ptr(out["lengths"]), _ptr(out.get("pool_indices")),
        _stream(workspace.device))
    _check(st, "dsa_index_topk")
    return out


def selection_softmax(scores, *, out=None):
    """Softmax over each row of top-k scores ([T, topk] fp32, padding -inf): exp(s - max) / sum,
    padding 0, empty rows all zeros. ``out`` may be ``scores`` itself."""
    lib = load()
    _need(scores, "scores", (torch.float32,))
    if scores.dim() != 2:
        raise ValueError(f"scores must be [T, topk], got shape {tuple(scores.shape)}")
    if out is None:
        out = torch.empty_like(scores)
    _need(out, "out", (torch.float32,), device=scores.device)
    if out.shape != scores.shape:
        raise ValueError(f"out shape {tuple(out.shape)} differs from scores {tuple(scores.shape)}")
    T, k = scores.shape
    st = lib.dsa_index_selection_softmax(_ptr(scores), int(T), int(k), _ptr(out), _stream(scores.device))
    _check(st, "dsa_index_selection_softmax")
    return out


def sparse_attention(q, kv, indices, *, sm_scale, lengths=None, out=None, lse=None, return_lse=True):
    """Absorbed-MLA attention over the selected latent entries.

    q [T, H, 576] bf16, kv [S, 576] bf16, indices [T, topk] int32 (token indices, -1 empty),
    lengths [T] int32 or None. Returns out [T, H, 512] bf16 and, with ``return_lse``, the
    natural-log log-sum-exp [T, H] fp32."""
    lib = load()
    _need(q, "q", (torch.bfloat16,))
    _need(kv, "kv", (torch.bfloat16,), device=q.device)
    _need(indices, "indices", (torch.int32,), device=q.device)
    _need(lengths, "lengths", (torch.int32,), device=q.device)
    if q.dim() != 3 or kv.dim() != 2 or indices.dim() != 2:
        raise ValueError("q must be [T, H, dk], kv [S, dk] and indices [T, topk]")
    T, H, dk = q.shape
    S, dk2 = kv.shape
    if dk2 != dk or indices.shape[0] != T:
        raise ValueError(f"shapes do not agree: q {tuple(q.shape)}, kv {tuple(kv.shape)}, indices {tuple(indices.shape)}")
    if lengths is not None and tuple(lengths.shape) != (T,):
        raise ValueError(f"lengths must be [T], got {tuple(lengths.shape)}")
    dv = 512
    if out is None:
        out = torch.empty((T, H, dv), dtype=torch.bfloat16, device=q.device)
    _need(out, "out", (torch.bfloat16,), device=q.device)
    if tuple(out.shape) != (T, H, dv):
        raise ValueError(f"out must be [{T}, {H}, {dv}], got {tuple(out.shape)}")
    if return_lse and lse is None:
        lse = torch.empty((T, H), dtype=torch.float32, device=q.device)
    _need(lse, "lse", (torch.float32,), device=q.device)
    if lse is not None and tuple(lse.shape) != (T, H):
        raise ValueError(f"lse must be [{T}, {H}], got {tuple(lse.shape)}")
    st = lib.dsa_index_sparse_attention(_ptr(q), _ptr(kv), _ptr(indices), _ptr(lengths), int(T), int(H), int(S),
                                        int(indices.shape[1]), int(dk), int(dv), float(sm_scale), _ptr(out),
                                        _ptr(lse), _stream(q.device))
    _check(st, "dsa_index_sparse_attention")
    return (out, lse) if return_lse else out


def bench_mfma(precision, blocks, iters, out):
    """Compute-only MFMA stream (dsa_bench_mfma) on the current stream; `out` is a float32
    device tensor of blocks * 256 elements. Returns the flops of the call."""
    lib = load()
    prec = _prec(precision)
    _need(out, "out", (torch.float32,))
    if out.numel() < blocks * 256:
        raise ValueError(f"out holds {out.numel()} floats, needs {blocks * 256}")
    _check(lib.dsa_bench_mfma(prec, int(blocks), int(iters), _ptr(out), _stream(out.device)), "dsa_bench_mfma")
    return float(lib.dsa_bench_mfma_flops(prec, int(blocks), int(iters)))


def bench_stream(src, dst, copy):
    """HBM sweep over src (dsa_bench_stream) on the current stream: copy to dst, or read only.
    Returns the HBM bytes the call moves."""
    lib = load()
    _need(src, "src")
    _need(dst, "dst")
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() < (nbytes if copy else 16):
        raise ValueError("dst is smaller than src (copy) or than 16 bytes (read)")
    _check(lib.dsa_bench_stream(_ptr(src), _ptr(dst), nbytes, 1 if copy else 0, _stream(src.device)),
           "dsa_bench_stream")
    return 2 * nbytes if copy else nbytes
