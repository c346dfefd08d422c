"""ctypes binding over libssa.so: argument marshalling only.

Every step of the computation runs in the HIP kernels behind the C ABI in
``include/ssa.h``. PyTorch provides device memory (tensors) and the current
HIP stream. If the library is not built, every call raises; there is no
fallback path.
"""

from __future__ import annotations

import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# SSA_LIB may name another build of the same library (e.g. a tuning variant).
LIB_PATH = os.environ.get("SSA_LIB") or os.path.join(_HERE, "libssa.so")

SSA_OK = 0
SSA_ERR_INVALID_ARG = -1
SSA_ERR_UNSUPPORTED = -2
SSA_ERR_WORKSPACE = -3
SSA_ERR_HIP = -4
SSA_ERR_SCRATCH = -5
DECODE_SCRATCH_BYTES = 32 << 20
TILE_KEPT = 1
TILE_SKIPPED = 2

_lib = None

_p = ctypes.c_void_p
_i = ctypes.c_int
_f = ctypes.c_float
_sz = ctypes.c_size_t

_SIGNATURES = {
    "ssa_prefill": (_i, [_p, _p, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _i, _f, _i, _p, _p, _i, _p]),
    "ssa_prefill_nm": (_i, [_p, _p, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _i, _f, _i, _i, _i, _i, _i, _p]),
    "ssa_decode_workspace_size": (_sz, [_i, _i, _i, _i, _i, _i]),
    "ssa_decode": (_i, [_p, _p, _p, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _i, _f, _p, _sz, _p]),
    "ssa_decode_noalloc": (_i, [_p, _p, _p, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _i, _f, _p]),
    "ssa_block_mask_max_blocks": (_i, [_i, _i, _i, _i, _i]),
    "ssa_block_mask_workspace_size": (_sz, [_i, _i, _i, _i, _i]),
    "ssa_block_mask": (_i, [_p, _p, _i, _i, _i, _i, _i, _i, _i, _i, _i, _p, _p, _i, _p, _p, _sz, _p]),
    "ssa_block_mask_compressed_workspace_size": (_sz, [_i, _i, _i, _i, _i]),
    "ssa_block_mask_compressed": (_i, [_p, _p, _i, _i, _i, _i, _i, _i, _i, _i, _i, _i, _i, _p, _p, _i,
                                       _p, _p, _sz, _p]),
    "ssa_sparge_mask_workspace_size": (_sz, [_i, _i, _i, _i, _i]),
    "ssa_sparge_mask": (_i, [_p, _p, _i, _i, _i, _i, _i, _f, ctypes.c_double, _i, _i, _p, _p, _i, _p,
                             _p, _p, _sz, _p]),
    "ssa_vertical_slash_workspace_size": (_sz, [_i, _i, _i]),
    "ssa_vertical_slash_mask": (_i, [_p, _p, _i, _i, _i, _i, _i, _i, _i, _i, _i, _p, _p, _i, _p, _p,
                                     _p, _p, _p, _sz, _p]),
    "ssa_calibrate_workspace_size": (_sz, [_sz, ctypes.c_double]),
    "ssa_lambda_for_ratio": (_i, [_p, _sz, ctypes.c_double, ctypes.c_double, _p, _p, _sz, _p]),
    "ssa_lambda_from_scale_factor": (_f, [_f, _i]),
    "ssa_status_string": (ctypes.c_char_p, [_i]),
    "ssa_abi_version": (_i, []),
}


class SSAError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {status_string(status)} ({status})")


def lib() -> ctypes.CDLL:
    """Load libssa.so (once). Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m sparse_attention_long_skip_amd.build` "
                "or __graft_entry__.build()")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(l, name)
            fn.restype = res
            fn.argtypes = args
        _lib = l
    return _lib


def status_string(status: int) -> str:
    return lib().ssa_status_string(int(status)).decode()


def abi_version() -> int:
    return lib().ssa_abi_version()


def lambda_from_scale_factor(scale_factor: float, L: int) -> float:
    return float(lib().ssa_lambda_from_scale_factor(float(scale_factor), int(L)))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _need(t, name, dtype, ndim):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _check(fn, status):
    if status != SSA_OK:
        raise SSAError(fn, status)


def prefill(q, k, v, lam: float, Br: int = 128, Bc: int = 64, causal: bool = True,
            block_idx=None, block_cnt=None, lse: bool = True, stats: bool = False,
            margins: bool = False, out=None, stream=None, nm=None, dense_sink: int = 0,
            dense_recent: int = 0, counts: bool = False, skip_counts=None, lse_out=None) -> dict:
    """Skip-Softmax prefill (``ssa_prefill``; ``ssa_prefill_nm`` when ``nm`` =
    (N, M) asks for N:M sparse softmax). q [B,Hq,L,d], k/v [B,Hkv,L,d] bf16.
    Returns a dict: out, and lse / skip_counts / tile_state / tile_margin as
    requested (tile arrays are zero / NaN where not visited).

    ``stats`` asks for skip_counts and tile_state, ``margins`` for
    tile_margin; either selects the kernel instance that writes per-tile
    arrays. ``counts`` (or a caller-provided ``skip_counts`` tensor) asks for
    skip_counts alone, which the plain instance writes as well."""
    _need(q, "q", torch.bfloat16, 4)
    _need(k, "k", torch.bfloat16, 4)
    _need(v, "v", torch.bfloat16, 4)
    B, Hq, L, d = q.shape
    Hkv = k.shape[1]
    nQ, nK = math.ceil(L / Br), math.ceil(L / Bc)
    dev = q.device
    res = {}
    res["out"] = out if out is not None else torch.empty_like(q)
    if lse_out is not None:
        _need(lse_out, "lse_out", torch.float32, 3)
        res["lse"] = lse_out
    else:
        res["lse"] = torch.empty((B, Hq, L), dtype=torch.float32, device=dev) if lse else None
    if skip_counts is not None:
        _need(skip_counts, "skip_counts", torch.int32, 3)
        if tuple(skip_counts.shape) != (B, Hq, nQ):
            raise ValueError(f"skip_counts must be {(B, Hq, nQ)}, got {tuple(skip_counts.shape)}")
        res["skip_counts"] = skip_counts
    else:
        res["skip_counts"] = (torch.empty((B, Hq, nQ), dtype=torch.int32, device=dev)
                              if (stats or counts) else None)
    res["tile_state"] = torch.zeros((B, Hq, nQ, nK), dtype=torch.uint8, device=dev) if stats else None
    res["tile_margin"] = (torch.full((B, Hq, nQ, nK), float("nan"), dtype=torch.float32, device=dev)
                          if margins else None)
    max_blocks = 0
    if block_idx is not None:
        _need(block_idx, "block_idx", torch.int32, 4)
        _need(block_cnt, "block_cnt", torch.int32, 3)
        max_blocks = block_idx.shape[3]
    if nm is not None:
        if block_idx is not None:
            raise ValueError("N:M sparse softmax does not take a block list")
        st = lib().ssa_prefill_nm(
            _ptr(q), _ptr(k), _ptr(v), _ptr(res["out"]), _ptr(res["lse"]), _ptr(res["skip_counts"]),
            _ptr(res["tile_state"]), _ptr(res["tile_margin"]), B, Hq, Hkv, L, d, Br, Bc, float(lam),
            int(bool(causal)), int(nm[0]), int(nm[1]), int(dense_sink), int(dense_recent),
            _stream(stream))
        _check("ssa_prefill_nm", st)
        return res
    st = lib().ssa_prefill(
        _ptr(q), _ptr(k), _ptr(v), _ptr(res["out"]), _ptr(res["lse"]), _ptr(res["skip_counts"]),
        _ptr(res["tile_state"]), _ptr(res["tile_margin"]), B, Hq, Hkv, L, d, Br, Bc, float(lam),
        int(bool(causal)), _ptr(block_idx), _ptr(block_cnt), max_blocks, _stream(stream))
    _check("ssa_prefill", st)
    return res


def decode_workspace_size(B, Hq, S_max, d, Bc=64, split_tiles=32) -> int:
    return int(lib().ssa_decode_workspace_size(B, Hq, S_max, d, Bc, split_tiles))


def decode(q, k_cache, v_cache, seqlens, lam: float, split_tiles: int = 32, Bc: int = 64,
           workspace=None, lse: bool = True, stats: bool = False, margins: bool = False,
           out=None, stream=None, lse_out=None, skip_counts=None, counts: bool = False,
           noalloc: bool = False) -> dict:
    """Skip-Softmax split-K decode (``ssa_decode``). q [B,Hq,d]; caches
    [B,Hkv,S_max,d] bf16; seqlens [B] int32 (device). ``stats`` asks for
    skip_counts and tile_state, ``counts`` for skip_counts alone; ``lse_out``
    and ``skip_counts`` may be caller-provided tensors. ``noalloc`` calls
    ``ssa_decode_noalloc`` (the library's static scratch, no workspace)."""
    _need(q, "q", torch.bfloat16, 3)
    _need(k_cache, "k_cache", torch.bfloat16, 4)
    _need(v_cache, "v_cache", torch.bfloat16, 4)
    _need(seqlens, "seqlens", torch.int32, 1)
    B, Hq, d = q.shape
    _, Hkv, S_max, _ = k_cache.shape
    nT = math.ceil(S_max / Bc)
    nS = math.ceil(nT / split_tiles)
    dev = q.device
    if noalloc:
        if workspace is not None:
            raise ValueError("noalloc takes no workspace")
    elif workspace is None:
        need = decode_workspace_size(B, Hq, S_max, d, Bc, split_tiles)
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    res = {"workspace": workspace}
    res["out"] = out if out is not None else torch.empty_like(q)
    if lse_out is not None:
        _need(lse_out, "lse_out", torch.float32, 2)
        res["lse"] = lse_out
    else:
        res["lse"] = torch.empty((B, Hq), dtype=torch.float32, device=dev) if lse else None
    if skip_counts is not None:
        _need(skip_counts, "skip_counts", torch.int32, 3)
        if tuple(skip_counts.shape) != (B, Hkv, nS):
            raise ValueError(f"skip_counts must be {(B, Hkv, nS)}, got {tuple(skip_counts.shape)}")
        res["skip_counts"] = skip_counts
    else:
        res["skip_counts"] = (torch.empty((B, Hkv, nS), dtype=torch.int32, device=dev)
                              if (stats or counts) else None)
    res["tile_state"] = torch.zeros((B, Hkv, nT), dtype=torch.uint8, device=dev) if stats else None
    res["tile_margin"] = (torch.full((B, Hkv, nT), float("nan"), dtype=torch.float32, device=dev)
                          if margins else None)
    if noalloc:
        st = lib().ssa_decode_noalloc(
            _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seqlens), _ptr(res["out"]), _ptr(res["lse"]),
            _ptr(res["skip_counts"]), _ptr(res["tile_state"]), _ptr(res["tile_margin"]),
            B, Hq, Hkv, S_max, d, Bc, split_tiles, float(lam), _stream(stream))
        _check("ssa_decode_noalloc", st)
        return res
    st = lib().ssa_decode(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seqlens), _ptr(res["out"]), _ptr(res["lse"]),
        _ptr(res["skip_counts"]), _ptr(res["tile_state"]), _ptr(res["tile_margin"]),
        B, Hq, Hkv, S_max, d, Bc, split_tiles, float(lam), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream))
    _check("ssa_decode", st)
    return res


def block_mask_max_blocks(L, pool=64, topk=64, sink_blocks=1, window_tokens=1024) -> int:
    return int(lib().ssa_block_mask_max_blocks(L, pool, topk, sink_blocks, window_tokens))


def block_mask_workspace_size(B, H, L, d, pool=64) -> int:
    return int(lib().ssa_block_mask_workspace_size(B, H, L, d, pool))


def block_mask(q, k, pool: int = 64, topk: int = 64, sink_blocks: int = 1,
               window_tokens: int = 1024, scores: bool = False, workspace=None,
               stream=None, compress=None) -> dict:
    """Pooled-score block mask (``ssa_block_mask``). q, k [B,H,L,d] bf16.
    Returns block_idx [B,H,nB,max_blocks] int32 (ascending, -1 padded),
    block_cnt [B,H,nB] int32 and, if asked, the pooled scores. With
    ``compress=(kernel_size, stride)`` the key blocks are scored by
    overlapping compressed keys (``ssa_block_mask_compressed``)."""
    _need(q, "q", torch.bfloat16, 4)
    _need(k, "k", torch.bfloat16, 4)
    B, H, L, d = q.shape
    nB = math.ceil(L / pool)
    dev = q.device
    mb = block_mask_max_blocks(L, pool, topk, sink_blocks, window_tokens)
    if mb < 0:
        raise ValueError("invalid block-mask sizes")
    if compress is None:
        need = block_mask_workspace_size(B, H, L, d, pool)
    else:
        need = block_mask_compressed_workspace_size(B, H, L, d, pool)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    res = {
        "block_idx": torch.empty((B, H, nB, mb), dtype=torch.int32, device=dev),
        "block_cnt": torch.empty((B, H, nB), dtype=torch.int32, device=dev),
        "scores": torch.empty((B, H, nB, nB), dtype=torch.float32, device=dev) if scores else None,
        "workspace": workspace,
    }
    wsb = workspace.numel() * workspace.element_size()
    if compress is None:
        st = lib().ssa_block_mask(
            _ptr(q), _ptr(k), B, H, L, d, pool, topk, sink_blocks, window_tokens, 1,
            _ptr(res["block_idx"]), _ptr(res["block_cnt"]), mb, _ptr(res["scores"]),
            _ptr(workspace), wsb, _stream(stream))
        _check("ssa_block_mask", st)
    else:
        kernel_size, stride = compress
        st = lib().ssa_block_mask_compressed(
            _ptr(q), _ptr(k), B, H, L, d, pool, kernel_size, stride, topk, sink_blocks,
            window_tokens, 1, _ptr(res["block_idx"]), _ptr(res["block_cnt"]), mb,
            _ptr(res["scores"]), _ptr(workspace), wsb, _stream(stream))
        _check("ssa_block_mask_compressed", st)
    return res


def block_mask_compressed_workspace_size(B, H, L, d, pool=64) -> int:
    return int(lib().ssa_block_mask_compressed_workspace_size(B, H, L, d, pool))


TAU_MODES = {"mass": 0, "count": 1}


def sparge_mask_workspace_size(B, H, L, d, pool=64) -> int:
    return int(lib().ssa_sparge_mask_workspace_size(B, H, L, d, pool))


def sparge_mask(q, k, theta: float, tau: float, tau_mode: str = "mass", pool: int = 64,
                sim: bool = False, scores: bool = False, workspace=None, stream=None) -> dict:
    """SpargeAttn stage-one mask (``ssa_sparge_mask``). q, k [B,H,L,d] bf16.
    Returns block_idx [B,H,nB,nB] int32 (ascending, -1 padded), block_cnt
    [B,H,nB] int32 and, if asked, the block self-similarities [B,H,2,nB]
    and the pooled scores."""
    _need(q, "q", torch.bfloat16, 4)
    _need(k, "k", torch.bfloat16, 4)
    if tau_mode not in TAU_MODES:
        raise ValueError(f"tau_mode must be one of {sorted(TAU_MODES)}")
    B, H, L, d = q.shape
    nB = math.ceil(L / pool)
    dev = q.device
    need = sparge_mask_workspace_size(B, H, L, d, pool)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    res = {
        "block_idx": torch.empty((B, H, nB, nB), dtype=torch.int32, device=dev),
        "block_cnt": torch.empty((B, H, nB), dtype=torch.int32, device=dev),
        "sim": torch.empty((B, H, 2, nB), dtype=torch.float32, device=dev) if sim else None,
        "scores": torch.empty((B, H, nB, nB), dtype=torch.float32, device=dev) if scores else None,
        "workspace": workspace,
    }
    st = lib().ssa_sparge_mask(
        _ptr(q), _ptr(k), B, H, L, d, pool, float(theta), float(tau), TAU_MODES[tau_mode], 1,
        _ptr(res["block_idx"]), _ptr(res["block_cnt"]), nB, _ptr(res["sim"]), _ptr(res["scores"]),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream))
    _check("ssa_sparge_mask", st)
    return res


def vertical_slash_workspace_size(B, H, L) -> int:
    return int(lib().ssa_vertical_slash_workspace_size(B, H, L))


def vertical_slash_mask(q, k, n_vertical: int, n_slash: int, last_q: int = 64, pool: int = 64,
                        indices: bool = False, scores: bool = False, workspace=None,
                        stream=None) -> dict:
    """Vertical-slash block estimator (``ssa_vertical_slash_mask``). q, k
    [B,H,L,d] bf16. Returns block_idx [B,H,nB,nB] int32 (ascending, -1
    padded), block_cnt [B,H,nB] int32 and, if asked, the chosen vertical keys
    and slash offsets (``indices``) and the scores v, s (``scores``)."""
    _need(q, "q", torch.bfloat16, 4)
    _need(k, "k", torch.bfloat16, 4)
    B, H, L, d = q.shape
    nB = math.ceil(L / pool)
    dev = q.device
    need = vertical_slash_workspace_size(B, H, L)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    i32 = dict(dtype=torch.int32, device=dev)
    f32 = dict(dtype=torch.float32, device=dev)
    res = {
        "block_idx": torch.empty((B, H, nB, nB), **i32),
        "block_cnt": torch.empty((B, H, nB), **i32),
        "vertical": torch.empty((B, H, max(n_vertical, 1)), **i32) if indices else None,
        "slash": torch.empty((B, H, max(n_slash, 1)), **i32) if indices else None,
        "v": torch.empty((B, H, L), **f32) if scores else None,
        "s": torch.empty((B, H, L), **f32) if scores else None,
        "workspace": workspace,
    }
    st = lib().ssa_vertical_slash_mask(
        _ptr(q), _ptr(k), B, H, L, d, last_q, n_vertical, n_slash, pool, 1,
        _ptr(res["block_idx"]), _ptr(res["block_cnt"]), nB,
        _ptr(res["vertical"]) if n_vertical > 0 else None,
        _ptr(res["slash"]) if n_slash > 0 else None,
        _ptr(res["v"]), _ptr(res["s"]), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream))
    _check("ssa_vertical_slash_mask", st)
    return res


def calibrate_workspace_size(n_margins: int, window: float = 0.01) -> int:
    return int(lib().ssa_calibrate_workspace_size(int(n_margins), float(window)))


def lambda_for_ratio(margins, target: float, window: float = 0.01, workspace=None, result=None,
                     stream=None, sync: bool = True):
    """Device threshold calibration (``ssa_lambda_for_ratio``) over a fp32
    margin tensor (NaN = tile not visited). Returns (lambda, achieved ratio)
    as Python floats after synchronising the stream, or, with ``sync=False``,
    the device result tensor of 4 doubles (lambda, ratio, n, n below)."""
    if not isinstance(margins, torch.Tensor) or margins.dtype != torch.float32 or not margins.is_cuda:
        raise TypeError("margins must be a float32 device tensor")
    if not margins.is_contiguous():
        raise ValueError("margins must be contiguous")
    n = margins.numel()
    dev = margins.device
    need = calibrate_workspace_size(n, window)
    if need == 0:
        raise ValueError("invalid calibration sizes")
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    if result is None:
        result = torch.empty(4, dtype=torch.float64, device=dev)
    st = lib().ssa_lambda_for_ratio(
        _ptr(margins), n, float(target), float(window), _ptr(result), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream))
    _check("ssa_lambda_for_ratio", st)
    if not sync:
        return result
    r = result.cpu().tolist()
    if math.isnan(r[0]):
        raise RuntimeError("ssa_lambda_for_ratio: workspace bound exceeded")
    return float(r[0]), float(r[1])
