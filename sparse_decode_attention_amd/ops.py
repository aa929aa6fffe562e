"""ctypes binding of libspark.so over torch device tensors.

Argument marshalling only: every step of prefill pruning, statistics and
decode attention runs in the HIP kernels of libspark.so. Torch provides device
memory (outputs and workspaces are torch tensors) and the current HIP stream.
If the library is missing this module raises; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
import re
import threading

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libspark.so")
HEADER = os.path.join(os.path.dirname(_PKG), "include", "spark.h")

OK, EINVAL, EUNSUPPORTED, EALIGN, ENOSPACE, EHIP, ESCRATCH = 0, -1, -2, -3, -4, -5, -6
NOALLOC_SCRATCH_BYTES = 8 << 20
RECOVERY = {"mean_retained": 0, "zero": 1, "const": 2, "score_mean_pruned": 3, "gaussian": 4, "exponential": 5}
QAGG = {"l2": 0, "mean": 1}
DECODE_COUNTER_BYTES = 256 << 10

_lib = None
_lock = threading.Lock()

_vp, _i, _f, _sz, _u64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t, ctypes.c_uint64
_SIGS = {
    "spark_num_kept": (_i, [_i, _f]),
    "spark_strerror": (ctypes.c_char_p, [_i]),
    "spark_prefill_workspace_bytes": (_sz, [_i, _i, _i, _i]),
    "spark_decode_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i]),
    "spark_prefill_prune": (_i, [_vp, _vp, _i, _i, _i, _i, _i, _f, _i, _i, _i, _f,
                                 _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "spark_stats": (_i, [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _f, _i, _f, _vp, _vp, _vp, _sz, _vp]),
    "spark_decode_attn": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _f, _i, _vp, _vp, _sz, _vp]),
    "spark_decode_attn_sampled": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _u64, _i, _i, _i, _i, _i, _f, _f, _i,
                                       _vp, _vp, _sz, _vp]),
    "spark_prefill_prune_v": (_i, [_vp, _i, _i, _i, _i, _f, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "spark_num_kept_grouped": (_i, [_i, _i, ctypes.POINTER(ctypes.c_float)]),
    "spark_prefill_prune_topp": (_i, [_vp, _vp, _i, _i, _i, _i, _i, _f, _i, _i, _i, _f, _vp, _vp, _vp, _vp, _vp, _vp,
                                      _vp, _sz, _vp]),
    "spark_decode_attn_ragged": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _i, _vp, _vp, _sz, _vp]),
    "spark_prefill_prune_cap": (_i, [_vp, _vp, _i, _i, _i, _i, _i, _i, _f, _i, _i, _i, _f,
                                     _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "spark_append_token": (_i, [_vp, _vp, _vp, _i, _i, _i, _f, _i, _i, _vp, _vp, _vp, _vp]),
    "spark_decode_attn_cap": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _f, _f, _i, _vp, _vp, _sz, _vp]),
    "spark_prefill_prune_grouped": (_i, [_vp, _vp, _i, _i, _i, _i, _i, _i, ctypes.POINTER(ctypes.c_float), _i, _i,
                                         _i, _f, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "spark_decode_attn_kv": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _f, _f, _i,
                                  _vp, _vp, _sz, _vp]),
    "spark_num_kept_vblocks": (_i, [_i, _f]),
    "spark_vblock_mask_stride": (_sz, [_i]),
    "spark_prefill_prune_vblocks": (_i, [_vp, _i, _i, _i, _i, _f, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "spark_decode_attn_kvb": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _f, _f, _i,
                                   _vp, _vp, _sz, _vp]),
    "spark_decode_ws_init": (_i, [_vp, _sz, _vp]),
    "spark_decode_attn_noalloc": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _f, _i, _vp, _vp]),
    "spark_read_stream": (_i, [_vp, _sz, _vp, _i, _vp]),
    "spark_window_evict_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i]),
    "spark_window_evict": (_i, [_vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
}


class SparkError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {status} ({strerror(status)})")


def header_symbols() -> list[str]:
    """Entry points declared in include/spark.h."""
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char\*)\s+(spark_\w+)\s*\(", txt, re.M)))


def lib() -> ctypes.CDLL:
    """Load libspark.so (built by sparse_decode_attention_amd.build)."""
    global _lib
    if _lib is None:
        with _lock:
            if _lib is None:
                if not os.path.exists(LIB_PATH):
                    raise RuntimeError(f"{LIB_PATH} is missing: run `python -m sparse_decode_attention_amd.build`")
                l = ctypes.CDLL(LIB_PATH)
                for name, (res, args) in _SIGS.items():
                    fn = getattr(l, name)
                    fn.restype, fn.argtypes = res, args
                _lib = l
    return _lib


def strerror(status: int) -> str:
    return lib().spark_strerror(int(status)).decode()


def num_kept(D: int, lam: float) -> int:
    return int(lib().spark_num_kept(int(D), float(lam)))


def _floats(xs):
    return (ctypes.c_float * len(xs))(*[float(x) for x in xs])


def num_kept_grouped(D: int, ratios) -> int:
    """SparK-g: channels kept per token for equal groups pruned at `ratios`."""
    return int(lib().spark_num_kept_grouped(int(D), len(ratios), _floats(ratios)))


def _check(fn: str, status: int) -> None:
    if status != OK:
        raise SparkError(fn, status)


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(dev) -> int:
    return torch.cuda.current_stream(dev).cuda_stream


def _need(t: torch.Tensor, name: str, dtype, shape=None) -> None:
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous device tensor")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")


# workspaces are cached per (device, kind); decode workspaces are zeroed when
# allocated (the completion counters must start at zero and are left at zero)
_ws_cache: dict = {}


def workspace(dev, kind: str, nbytes: int) -> torch.Tensor:
    key = (str(dev), kind)
    ws = _ws_cache.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=dev)
        _ws_cache[key] = ws
    return ws


def prefill_prune(q_win: torch.Tensor, k: torch.Tensor, n_kv: int, lam: float, qagg: str = "l2",
                  recovery: str = "mean_retained", f_const: float = 0.01, out: dict | None = None) -> dict:
    """spark_prefill_prune: q_win bf16 [B][N_q][W][D], k bf16 [B][N_kv][S][D].

    Returns {"T", "k_packed", "mask", "chan_energy", "r", "cnt"} (new tensors
    unless `out` supplies them).
    """
    B, N_q, W, D = q_win.shape
    S = k.shape[2]
    _need(q_win, "q_win", torch.bfloat16)
    _need(k, "k", torch.bfloat16, (B, n_kv, S, D))
    T = num_kept(D, lam)
    if T < 0:
        raise SparkError("spark_num_kept", EINVAL)
    dev = k.device
    o = dict(out or {})
    o.setdefault("k_packed", torch.empty((B, n_kv, S, T), dtype=torch.bfloat16, device=dev))
    o.setdefault("mask", torch.empty((B, n_kv, S, (D + 31) // 32), dtype=torch.int32, device=dev))
    o.setdefault("chan_energy", torch.empty((B, n_kv, D), dtype=torch.float32, device=dev))
    o.setdefault("r", torch.empty((B, n_kv, D), dtype=torch.float32, device=dev))
    o.setdefault("cnt", torch.empty((B, n_kv, D), dtype=torch.int32, device=dev))
    nb = lib().spark_prefill_workspace_bytes(B, S, n_kv, D)
    ws = workspace(dev, "prefill", nb)
    st = lib().spark_prefill_prune(_ptr(q_win), _ptr(k), B, S, N_q, n_kv, D, float(lam), W,
                                   QAGG[qagg], RECOVERY[recovery], float(f_const),
                                   _ptr(o["k_packed"]) if T > 0 else None, _ptr(o["mask"]),
                                   _ptr(o["chan_energy"]), _ptr(o["r"]), _ptr(o["cnt"]),
                                   _ptr(ws), ws.numel(), _stream(dev))
    _check("spark_prefill_prune", st)
    o["T"] = T
    return o


def prefill_prune_grouped(q_win: torch.Tensor, k: torch.Tensor, n_kv: int, ratios, qagg: str = "l2",
                          recovery: str = "mean_retained", f_const: float = 0.01, out: dict | None = None) -> dict:
    """spark_prefill_prune_grouped (SparK-g). Same outputs as prefill_prune
    with T = num_kept_grouped(D, ratios); "lam" is the lambda to decode with."""
    B, N_q, W, D = q_win.shape
    S = k.shape[2]
    _need(q_win, "q_win", torch.bfloat16)
    _need(k, "k", torch.bfloat16, (B, n_kv, S, D))
    T = num_kept_grouped(D, ratios)
    if T < 0:
        raise SparkError("spark_num_kept_grouped", EINVAL)
    dev = k.device
    o = dict(out or {})
    o.setdefault("k_packed", torch.empty((B, n_kv, S, T), dtype=torch.bfloat16, device=dev))
    o.setdefault("mask", torch.empty((B, n_kv, S, (D + 31) // 32), dtype=torch.int32, device=dev))
    o.setdefault("chan_energy", torch.empty((B, n_kv, D), dtype=torch.float32, device=dev))
    o.setdefault("r", torch.empty((B, n_kv, D), dtype=torch.float32, device=dev))
    o.setdefault("cnt", torch.empty((B, n_kv, D), dtype=torch.int32, device=dev))
    ws = workspace(dev, "prefill", lib().spark_prefill_workspace_bytes(B, S, n_kv, D))
    st = lib().spark_prefill_prune_grouped(_ptr(q_win), _ptr(k), B, S, N_q, n_kv, D, len(ratios), _floats(ratios), W,
                                           QAGG[qagg], RECOVERY[recovery], float(f_const),
                                           _ptr(o["k_packed"]) if T > 0 else None, _ptr(o["mask"]),
                                           _ptr(o["chan_energy"]), _ptr(o["r"]), _ptr(o["cnt"]), _ptr(ws), ws.numel(),
                                           _stream(dev))
    _check("spark_prefill_prune_grouped", st)
    o["T"] = T
    o["lam"] = 1.0 - T / D
    return o


def prefill_prune_topp(q_win: torch.Tensor, k: torch.Tensor, n_kv: int, p: float = 0.99, qagg: str = "l2",
                       recovery: str = "mean_retained", f_const: float = 0.01, out: dict | None = None) -> dict:
    """spark_prefill_prune_topp (SparK-p): ragged packed rows.

    Returns {"k_packed" bf16 [B][N_kv][S*D] (each head's region), "row_off"
    int32 [B][N_kv][S+1], "mask", "chan_energy", "r", "cnt"}.
    """
    B, N_q, W, D = q_win.shape
    S = k.shape[2]
    _need(q_win, "q_win", torch.bfloat16)
    _need(k, "k", torch.bfloat16, (B, n_kv, S, D))
    dev = k.device
    o = dict(out or {})
    o.setdefault("k_packed", torch.empty((B, n_kv, S * D), dtype=torch.bfloat16, device=dev))
    o.setdefault("row_off", torch.empty((B, n_kv, S + 1), dtype=torch.int32, device=dev))
    o.setdefault("mask", torch.empty((B, n_kv, S, (D + 31) // 32), dtype=torch.int32, device=dev))
    o.setdefault("chan_energy", torch.empty((B, n_kv, D), dtype=torch.float32, device=dev))
    o.setdefault("r", torch.empty((B, n_kv, D), dtype=torch.float32, device=dev))
    o.setdefault("cnt", torch.empty((B, n_kv, D), dtype=torch.int32, device=dev))
    ws = workspace(dev, "prefill", lib().spark_prefill_workspace_bytes(B, S, n_kv, D))
    st = lib().spark_prefill_prune_topp(_ptr(q_win), _ptr(k), B, S, N_q, n_kv, D, float(p), W, QAGG[qagg],
                                        RECOVERY[recovery], float(f_const), _ptr(o["k_packed"]), _ptr(o["row_off"]),
                                        _ptr(o["mask"]), _ptr(o["chan_energy"]), _ptr(o["r"]), _ptr(o["cnt"]),
                                        _ptr(ws), ws.numel(), _stream(dev))
    _check("spark_prefill_prune_topp", st)
    return o


def decode_attn_ragged(q, k_packed, row_off, mask, v, r, scale: float = 0.0, splits: int = 0, out=None, ws=None):
    """spark_decode_attn_ragged: decode over a SparK-p cache."""
    B, N_q, D = q.shape
    n_kv, S = v.shape[1], v.shape[2]
    _need(q, "q", torch.bfloat16)
    _need(v, "v", torch.bfloat16, (B, n_kv, S, D))
    _need(row_off, "row_off", torch.int32, (B, n_kv, S + 1))
    _need(k_packed, "k_packed", torch.bfloat16, (B, n_kv, S * D))
    dev = q.device
    out = torch.empty((B, N_q, D), dtype=torch.float32, device=dev) if out is None else out
    if ws is None:
        ws = workspace(dev, "decode", decode_ws_bytes(B, S, N_q, n_kv, D, splits))
    st = lib().spark_decode_attn_ragged(_ptr(q), _ptr(k_packed), _ptr(row_off), _ptr(mask), _ptr(v), _ptr(r), B, S,
                                        N_q, n_kv, D, float(scale), int(splits), _ptr(out), _ptr(ws), ws.numel(),
                                        _stream(dev))
    _check("spark_decode_attn_ragged", st)
    return out


def stats(k_packed, mask, chan_energy, lam: float, recovery: str = "mean_retained", f_const: float = 0.01,
          k_dense=None, r=None, cnt=None):
    """spark_stats: recompute (r, cnt) from a stored pruned cache."""
    B, n_kv, S, nw = mask.shape
    D = chan_energy.shape[-1]
    dev = mask.device
    r = torch.empty((B, n_kv, D), dtype=torch.float32, device=dev) if r is None else r
    cnt = torch.empty((B, n_kv, D), dtype=torch.int32, device=dev) if cnt is None else cnt
    nb = lib().spark_prefill_workspace_bytes(B, S, n_kv, D)
    ws = workspace(dev, "prefill", nb)
    T = num_kept(D, lam)
    st = lib().spark_stats(_ptr(k_packed) if (k_packed is not None and T > 0) else None, _ptr(mask),
                           _ptr(chan_energy), _ptr(k_dense), B, S, n_kv, D, float(lam), RECOVERY[recovery],
                           float(f_const), _ptr(r), _ptr(cnt), _ptr(ws), ws.numel(), _stream(dev))
    _check("spark_stats", st)
    return r, cnt


def decode_ws_bytes(B, S, N_q, N_kv, D=128, splits=0) -> int:
    return int(lib().spark_decode_workspace_bytes(B, S, N_q, N_kv, D, splits))


def decode_attn(q, k_packed, mask, v, r, lam: float, scale: float = 0.0, splits: int = 0, out=None, ws=None):
    """spark_decode_attn: q bf16 [B][N_q][D] -> out fp32 [B][N_q][D]."""
    B, N_q, D = q.shape
    n_kv, S = v.shape[1], v.shape[2]
    _need(q, "q", torch.bfloat16)
    _need(v, "v", torch.bfloat16, (B, n_kv, S, D))
    dev = q.device
    out = torch.empty((B, N_q, D), dtype=torch.float32, device=dev) if out is None else out
    nb = decode_ws_bytes(B, S, N_q, n_kv, D, splits)
    if ws is None:
        ws = workspace(dev, "decode", nb)
    T = num_kept(D, lam)
    st = lib().spark_decode_attn(_ptr(q), _ptr(k_packed) if T > 0 else None, _ptr(mask), _ptr(v), _ptr(r),
                                 B, S, N_q, n_kv, D, float(lam), float(scale), int(splits), _ptr(out),
                                 _ptr(ws), ws.numel(), _stream(dev))
    _check("spark_decode_attn", st)
    return out


def decode_attn_noalloc(q, k_packed, mask, v, r, lam: float, scale: float = 0.0, splits: int = 0, out=None):
    """spark_decode_attn_noalloc: spark_decode_attn with the library's fixed
    per-device scratch instead of a workspace (no device allocation by the
    library; `out` is allocated here only when not given)."""
    B, N_q, D = q.shape
    n_kv, S = v.shape[1], v.shape[2]
    _need(q, "q", torch.bfloat16)
    _need(v, "v", torch.bfloat16, (B, n_kv, S, D))
    dev = q.device
    out = torch.empty((B, N_q, D), dtype=torch.float32, device=dev) if out is None else out
    T = num_kept(D, lam)
    st = lib().spark_decode_attn_noalloc(_ptr(q), _ptr(k_packed) if T > 0 else None, _ptr(mask), _ptr(v), _ptr(r),
                                         B, S, N_q, n_kv, D, float(lam), float(scale), int(splits), _ptr(out),
                                         _stream(dev))
    _check("spark_decode_attn_noalloc", st)
    return out


def decode_attn_sampled(q, k_packed, mask, v, chan_energy, r, recovery: str, seed: int, lam: float,
                        scale: float = 0.0, splits: int = 0, out=None, ws=None):
    """spark_decode_attn_sampled: decode with a sampled recovery F ("gaussian"
    or "exponential"); r holds (mu, sigma) from prefill_prune / stats of the
    same recovery, chan_energy the A_j."""
    B, N_q, D = q.shape
    n_kv, S = v.shape[1], v.shape[2]
    _need(q, "q", torch.bfloat16)
    _need(v, "v", torch.bfloat16, (B, n_kv, S, D))
    _need(chan_energy, "chan_energy", torch.float32, (B, n_kv, D))
    _need(r, "r", torch.float32, (B, n_kv, D))
    dev = q.device
    out = torch.empty((B, N_q, D), dtype=torch.float32, device=dev) if out is None else out
    nb = decode_ws_bytes(B, S, N_q, n_kv, D, splits)
    if ws is None:
        ws = workspace(dev, "decode", nb)
    T = num_kept(D, lam)
    st = lib().spark_decode_attn_sampled(_ptr(q), _ptr(k_packed) if T > 0 else None, _ptr(mask), _ptr(v),
                                         _ptr(chan_energy), _ptr(r), RECOVERY[recovery], int(seed) & (2**64 - 1),
                                         B, S, N_q, n_kv, D, float(lam), float(scale), int(splits), _ptr(out),
                                         _ptr(ws), ws.numel(), _stream(dev))
    _check("spark_decode_attn_sampled", st)
    return out


def prefill_prune_v(v: torch.Tensor, lam_v: float, out: dict | None = None) -> dict:
    """spark_prefill_prune_v: v bf16 [B][N_kv][S][D] -> {"T", "v_packed",
    "v_mask", "r_v", "cnt"} (new tensors unless `out` supplies them)."""
    B, n_kv, S, D = v.shape
    _need(v, "v", torch.bfloat16)
    T = num_kept(D, lam_v)
    if T < 0:
        raise SparkError("spark_num_kept", EINVAL)
    dev = v.device
    o = dict(out or {})
    o.setdefault("v_packed", torch.empty((B, n_kv, S, T), dtype=torch.bfloat16, device=dev))
    o.setdefault("v_mask", torch.empty((B, n_kv, S, (D + 31) // 32), dtype=torch.int32, device=dev))
    o.setdefault("r_v", torch.empty((B, n_kv, D), dtype=torch.float32, device=dev))
    o.setdefault("cnt", torch.empty((B, n_kv, D), dtype=torch.int32, device=dev))
    ws = workspace(dev, "prefill", lib().spark_prefill_workspace_bytes(B, S, n_kv, D))
    st = lib().spark_prefill_prune_v(_ptr(v), B, S, n_kv, D, float(lam_v), _ptr(o["v_packed"]) if T > 0 else None,
                                     _ptr(o["v_mask"]), _ptr(o["r_v"]), _ptr(o["cnt"]), _ptr(ws), ws.numel(),
                                     _stream(dev))
    _check("spark_prefill_prune_v", st)
    o["T"] = T
    return o


def decode_attn_kv(q, k_packed, k_mask, r, v_packed, v_mask, r_v, lam: float, lam_v: float, scale: float = 0.0,
                   splits: int = 0, out=None, ws=None):
    """spark_decode_attn_kv: decode over a cache with K and V channels pruned."""
    B, N_q, D = q.shape
    n_kv, S = v_mask.shape[1], v_mask.shape[2]
    _need(q, "q", torch.bfloat16)
    _need(v_mask, "v_mask", torch.int32, (B, n_kv, S, (D + 31) // 32))
    _need(r_v, "r_v", torch.float32, (B, n_kv, D))
    dev = q.device
    out = torch.empty((B, N_q, D), dtype=torch.float32, device=dev) if out is None else out
    if ws is None:
        ws = workspace(dev, "decode", decode_ws_bytes(B, S, N_q, n_kv, D, splits))
    T, Tv = num_kept(D, lam), num_kept(D, lam_v)
    st = lib().spark_decode_attn_kv(_ptr(q), _ptr(k_packed) if T > 0 else None, _ptr(k_mask), _ptr(r),
                                    _ptr(v_packed) if Tv > 0 else None, _ptr(v_mask), _ptr(r_v), B, S, N_q, n_kv, D,
                                    float(lam), float(lam_v), float(scale), int(splits), _ptr(out), _ptr(ws),
                                    ws.numel(), _stream(dev))
    _check("spark_decode_attn_kv", st)
    return out


VBLOCK = 8


def num_kept_vblocks(D: int, lam_v: float) -> int:
    """spark_num_kept_vblocks: V blocks of 8 channels kept per token."""
    return lib().spark_num_kept_vblocks(D, float(lam_v))


def vblock_mask_stride(S: int) -> int:
    """spark_vblock_mask_stride: block-mask entries per head (S rounded up to 64)."""
    return lib().spark_vblock_mask_stride(S)


def prefill_prune_vblocks(v: torch.Tensor, lam_v: float, out: dict | None = None) -> dict:
    """spark_prefill_prune_vblocks: v bf16 [B][N_kv][S][D] -> {"nb",
    "v_packed" [B][N_kv][S][8 nb], "v_bmask" int16 [B][N_kv][stride]
    (tile-interleaved), "r_v", "cnt"} (new tensors unless `out` supplies them)."""
    B, n_kv, S, D = v.shape
    _need(v, "v", torch.bfloat16)
    nb = num_kept_vblocks(D, lam_v)
    if nb < 0:
        raise SparkError("spark_num_kept_vblocks", EINVAL)
    dev = v.device
    o = dict(out or {})
    o.setdefault("v_packed", torch.empty((B, n_kv, S, VBLOCK * nb), dtype=torch.bfloat16, device=dev))
    o.setdefault("v_bmask", torch.empty((B, n_kv, vblock_mask_stride(S)), dtype=torch.int16, device=dev))
    o.setdefault("r_v", torch.empty((B, n_kv, D), dtype=torch.float32, device=dev))
    o.setdefault("cnt", torch.empty((B, n_kv, D), dtype=torch.int32, device=dev))
    ws = workspace(dev, "prefill", lib().spark_prefill_workspace_bytes(B, S, n_kv, D))
    st = lib().spark_prefill_prune_vblocks(_ptr(v), B, S, n_kv, D, float(lam_v),
                                           _ptr(o["v_packed"]) if nb > 0 else None, _ptr(o["v_bmask"]),
                                           _ptr(o["r_v"]), _ptr(o["cnt"]), _ptr(ws), ws.numel(), _stream(dev))
    _check("spark_prefill_prune_vblocks", st)
    o["nb"] = nb
    return o


def decode_attn_kvb(q, k_packed, k_mask, r, v_packed, v_bmask, r_v, lam: float, lam_v: float, scale: float = 0.0,
                    splits: int = 0, out=None, ws=None):
    """spark_decode_attn_kvb: decode over a cache with K channels pruned and V
    pruned in 8-channel blocks."""
    B, N_q, D = q.shape
    n_kv, S = k_mask.shape[1], k_mask.shape[2]
    _need(q, "q", torch.bfloat16)
    _need(v_bmask, "v_bmask", torch.int16, (B, n_kv, vblock_mask_stride(S)))
    _need(r_v, "r_v", torch.float32, (B, n_kv, D))
    dev = q.device
    out = torch.empty((B, N_q, D), dtype=torch.float32, device=dev) if out is None else out
    if ws is None:
        ws = workspace(dev, "decode", decode_ws_bytes(B, S, N_q, n_kv, D, splits))
    T, nb = num_kept(D, lam), num_kept_vblocks(D, lam_v)
    st = lib().spark_decode_attn_kvb(_ptr(q), _ptr(k_packed) if T > 0 else None, _ptr(k_mask), _ptr(r),
                                     _ptr(v_packed) if nb > 0 else None, _ptr(v_bmask), _ptr(r_v), B, S, N_q, n_kv,
                                     D, float(lam), float(lam_v), float(scale), int(splits), _ptr(out), _ptr(ws),
                                     ws.numel(), _stream(dev))
    _check("spark_decode_attn_kvb", st)
    return out


class GrowingCache:
    """A pruned KV cache with room for S_cap tokens per (b, KV head), filled by
    a prefill and grown one generated token at a time (spark_prefill_prune_cap,
    spark_append_token, spark_decode_attn_cap). Buffers are torch device
    tensors; every step runs in libspark."""

    def __init__(self, q_win, k, v, n_kv: int, lam: float, S_cap: int, qagg: str = "l2",
                 recovery: str = "mean_retained", f_const: float = 0.01):
        B, N_q, W, D = q_win.shape
        S = k.shape[2]
        _need(q_win, "q_win", torch.bfloat16)
        _need(k, "k", torch.bfloat16, (B, n_kv, S, D))
        _need(v, "v", torch.bfloat16, (B, n_kv, S, D))
        if S_cap < S:
            raise ValueError("S_cap < S")
        dev = k.device
        self.B, self.N_q, self.n_kv, self.D, self.lam, self.S_cap = B, N_q, n_kv, D, float(lam), int(S_cap)
        self.T = num_kept(D, lam)
        self.k_packed = torch.empty((B, n_kv, S_cap, self.T), dtype=torch.bfloat16, device=dev)
        self.mask = torch.zeros((B, n_kv, S_cap, (D + 31) // 32), dtype=torch.int32, device=dev)
        self.v = torch.zeros((B, n_kv, S_cap, D), dtype=torch.bfloat16, device=dev)
        self.v[:, :, :S].copy_(v)
        self.chan_energy = torch.empty((B, n_kv, D), dtype=torch.float32, device=dev)
        self.r = torch.empty((B, n_kv, D), dtype=torch.float32, device=dev)
        self.cnt = torch.empty((B, n_kv, D), dtype=torch.int32, device=dev)
        ws = workspace(dev, "prefill", lib().spark_prefill_workspace_bytes(B, S, n_kv, D))
        st = lib().spark_prefill_prune_cap(_ptr(q_win), _ptr(k), B, S, S_cap, N_q, n_kv, D, self.lam, W, QAGG[qagg],
                                           RECOVERY[recovery], float(f_const),
                                           _ptr(self.k_packed) if self.T > 0 else None, _ptr(self.mask),
                                           _ptr(self.chan_energy), _ptr(self.r), _ptr(self.cnt), _ptr(ws), ws.numel(),
                                           _stream(dev))
        _check("spark_prefill_prune_cap", st)
        self.S = S

    def append(self, k_new: torch.Tensor, v_new: torch.Tensor) -> None:
        """k_new, v_new bf16 [B][N_kv][D]: prune and append at row S."""
        _need(k_new, "k_new", torch.bfloat16, (self.B, self.n_kv, self.D))
        _need(v_new, "v_new", torch.bfloat16, (self.B, self.n_kv, self.D))
        if self.S >= self.S_cap:
            raise SparkError("spark_append_token", ENOSPACE)
        st = lib().spark_append_token(_ptr(k_new), _ptr(v_new), _ptr(self.chan_energy), self.B, self.n_kv, self.D,
                                      self.lam, self.S, self.S_cap, _ptr(self.k_packed) if self.T > 0 else None,
                                      _ptr(self.mask), _ptr(self.v), _stream(k_new.device))
        _check("spark_append_token", st)
        self.S += 1

    def decode(self, q: torch.Tensor, scale: float = 0.0, splits: int = 0, out=None, ws=None) -> torch.Tensor:
        """spark_decode_attn_cap over the S tokens held now."""
        _need(q, "q", torch.bfloat16, (self.B, self.N_q, self.D))
        dev = q.device
        out = torch.empty((self.B, self.N_q, self.D), dtype=torch.float32, device=dev) if out is None else out
        if ws is None:
            ws = workspace(dev, "decode", decode_ws_bytes(self.B, self.S_cap, self.N_q, self.n_kv, self.D, splits))
        st = lib().spark_decode_attn_cap(_ptr(q), _ptr(self.k_packed) if self.T > 0 else None, _ptr(self.mask),
                                         _ptr(self.v), _ptr(self.r), self.B, self.S, self.S_cap, self.N_q, self.n_kv,
                                         self.D, self.lam, float(scale), int(splits), _ptr(out), _ptr(ws), ws.numel(),
                                         _stream(dev))
        _check("spark_decode_attn_cap", st)
        return out


def decode_ws_init(ws: torch.Tensor) -> None:
    _check("spark_decode_ws_init", lib().spark_decode_ws_init(_ptr(ws), ws.numel(), _stream(ws.device)))


def read_stream(src: torch.Tensor, sink: torch.Tensor, blocks: int = 2048) -> None:
    """Diagnostic streaming read of `src` (measures the practical HBM read rate)."""
    _check("spark_read_stream", lib().spark_read_stream(_ptr(src), src.numel() * src.element_size(),
                                                        _ptr(sink), int(blocks), _stream(src.device)))


def window_evict(q_win: torch.Tensor, k: torch.Tensor, v: torch.Tensor | None, n_kv: int, keep: int,
                 gather: bool = True, scores: torch.Tensor | None = None) -> dict:
    """spark_window_evict: q_win bf16 [B][N_q][W][D], k/v bf16 [B][N_kv][S][D].

    Returns {"idx" int32 [B][N_kv][keep], "scores" fp32 [B][N_kv][S] (if
    requested or allocated here), "k", "v" bf16 [B][N_kv][keep][D] (gather)}.
    """
    B, N_q, W, D = q_win.shape
    S = k.shape[2]
    _need(q_win, "q_win", torch.bfloat16)
    _need(k, "k", torch.bfloat16, (B, n_kv, S, D))
    if gather:
        _need(v, "v", torch.bfloat16, (B, n_kv, S, D))
    dev = k.device
    idx = torch.empty((B, n_kv, keep), dtype=torch.int32, device=dev)
    o = {"idx": idx}
    if scores is None:
        scores = torch.empty((B, n_kv, S), dtype=torch.float32, device=dev)
    o["scores"] = scores
    if gather:
        o["k"] = torch.empty((B, n_kv, keep, D), dtype=torch.bfloat16, device=dev)
        o["v"] = torch.empty((B, n_kv, keep, D), dtype=torch.bfloat16, device=dev)
    nb = int(lib().spark_window_evict_workspace_bytes(B, S, N_q, n_kv, D, W))
    ws = workspace(dev, "evict", nb)
    st = lib().spark_window_evict(_ptr(q_win), _ptr(k), _ptr(v) if gather else None, B, S, N_q, n_kv, D, W, keep,
                                  _ptr(idx), _ptr(o.get("k")), _ptr(o.get("v")), _ptr(scores), _ptr(ws), ws.numel(),
                                  _stream(dev))
    _check("spark_window_evict", st)
    return o
