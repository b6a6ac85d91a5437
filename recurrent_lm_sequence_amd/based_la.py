"""Python binding of libbasedla.so (ctypes; argument marshalling only).

Every step of the method runs in the HIP kernels behind the C ABI declared in
include/based_la.h; PyTorch only provides device memory and the stream.
Importing this module fails loudly if the library has not been built.
"""
from __future__ import annotations

import ctypes
import os
import re

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libbasedla.so")
INCLUDE_DIR = os.path.join(os.path.dirname(_PKG), "include")
HEADER_PATH = os.path.join(INCLUDE_DIR, "based_la.h")

BLA_OK, BLA_ERR_INVALID, BLA_ERR_UNSUPPORTED, BLA_ERR_HIP = 0, 1, 2, 3
BLA_F32, BLA_BF16 = 0, 1

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python -m recurrent_lm_sequence_amd._build` "
        "(there is no fallback implementation)")

lib = ctypes.CDLL(LIB_PATH)

_i, _f, _p = ctypes.c_int, ctypes.c_float, ctypes.c_void_p
lib.bla_feature_dim.argtypes = [_i]
lib.bla_feature_dim.restype = _i
lib.bla_status_string.argtypes = [_i]
lib.bla_status_string.restype = ctypes.c_char_p
lib.based_prefill.argtypes = [_i, _i, _i, _i, _i, _i, _i, _f, _p, _p, _p, _p, _p, _p, _p, _p, _p]
lib.based_prefill.restype = _i
lib.jrt_prefix_prefill.argtypes = [_i, _i, _i, _i, _i, _i, _i, _i, _f, _p, _p, _p, _p, _p, _p,
                                   _p, _p, _p, _p, _p]
lib.jrt_prefix_prefill.restype = _i
lib.based_decode_step.argtypes = [_i, _i, _i, _i, _i, _i, _f, _p, _p, _p, _p, _p, _p, _p]
lib.based_decode_step.restype = _i
lib.bla_compact_dim.argtypes = [_i]
lib.bla_compact_dim.restype = _i
lib.based_prefill_compact.argtypes = lib.based_prefill.argtypes
lib.based_prefill_compact.restype = _i
lib.jrt_prefix_prefill_compact.argtypes = lib.jrt_prefix_prefill.argtypes
lib.jrt_prefix_prefill_compact.restype = _i
lib.based_decode_step_compact.argtypes = lib.based_decode_step.argtypes
lib.based_decode_step_compact.restype = _i
lib.jrt_prefix_prefill_ex.argtypes = [_i, _i, _i, _i, _i, _i, _i, _i, _f, _p, _p, _p, _p, _p, _p,
                                      _p, _p, _p, _p, _p, _i, _p]
lib.jrt_prefix_prefill_ex.restype = _i
BLA_STATE_FULL, BLA_STATE_COMPACT = 0, 1
lib.swa_prefill.argtypes = [_i, _i, _i, _i, _i, _i, _i, _i, _p, _p, _p, _p, _p, _p, _p]
lib.swa_prefill.restype = _i
lib.swa_decode_step.argtypes = [_i, _i, _i, _i, _i, _i, _i, _i, _p, _p, _p, _p, _p, _p, _p]
lib.swa_decode_step.restype = _i
lib.bla_probe_mfma_f16.argtypes = [_i, _i, _p, _p]
lib.bla_probe_mfma_f16.restype = _i
lib.bla_probe_copy.argtypes = [_p, _p, ctypes.c_longlong, _p]
lib.bla_probe_copy.restype = _i
lib.bla_probe_prefill_traffic.argtypes = [_i, _i, _p, _p, _p, _p, _p, _i, _p]
lib.bla_probe_prefill_traffic.restype = _i


class BlaError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)}")


def status_string(status: int) -> str:
    return lib.bla_status_string(int(status)).decode()


def feature_dim(d_feat: int) -> int:
    return int(lib.bla_feature_dim(int(d_feat)))


def compact_dim(d_feat: int) -> int:
    return int(lib.bla_compact_dim(int(d_feat)))


def declared_functions() -> list[str]:
    """Names of the functions declared in every header under include/."""
    names = []
    for fn in sorted(os.listdir(INCLUDE_DIR)):
        if not fn.endswith(".h"):
            continue
        with open(os.path.join(INCLUDE_DIR, fn)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names += re.findall(r"^[A-Za-z_][\w \*]*?\b([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M)
    return names


_DT = {torch.float32: BLA_F32, torch.bfloat16: BLA_BF16}


def _dt(t: torch.Tensor) -> int:
    if t.dtype not in _DT:
        raise TypeError(f"unsupported dtype {t.dtype}; use float32 or bfloat16")
    return _DT[t.dtype]


def _ptr(t):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(status: int, what: str):
    if status != BLA_OK:
        raise BlaError(status, what)


def _outputs(q, v, N, y, S_out, z_out, out_dtype, want_y, want_state, compact=False):
    B, H = q.shape[0], q.shape[1]
    D = compact_dim(q.shape[-1]) if compact else feature_dim(q.shape[-1])
    dv = v.shape[-1]
    dev = v.device
    if y is None and want_y:
        y = torch.empty((B, H, N, dv), dtype=out_dtype or torch.float32, device=dev)
    if want_state:
        if S_out is None:
            S_out = torch.empty((B, H, D, dv), dtype=torch.float32, device=dev)
        if z_out is None:
            z_out = torch.empty((B, H, D), dtype=torch.float32, device=dev)
    return y, S_out, z_out


def based_prefill(q, k, v, S0=None, z0=None, *, eps: float = 0.0, y=None, S_out=None,
                  z_out=None, out_dtype=None, want_y: bool = True, want_state: bool = True,
                  stream=None, compact: bool = False):
    """Causal prefill; returns (y, S_out, z_out) (entries None when not requested).
    compact=True: the state tensors use the compact layout (based_prefill_compact)."""
    B, H, N, d = q.shape
    dv = v.shape[-1]
    y, S_out, z_out = _outputs(q, v, N, y, S_out, z_out, out_dtype, want_y, want_state, compact)
    fn = lib.based_prefill_compact if compact else lib.based_prefill
    st = fn(B, H, N, d, dv, _dt(q), _dt(y) if y is not None else BLA_F32,
                           float(eps), _ptr(q), _ptr(k), _ptr(v), _ptr(S0), _ptr(z0), _ptr(y),
                           _ptr(S_out), _ptr(z_out), _stream(stream))
    _check(st, "based_prefill_compact" if compact else "based_prefill")
    return y, S_out, z_out


def jrt_prefix_prefill(q, k, v, k_e, v_e, S0=None, z0=None, *, eps: float = 0.0, y=None,
                       S_out=None, z_out=None, out_dtype=None, want_y: bool = True,
                       want_state: bool = True, stream=None, compact: bool = False,
                       prefix_len=None):
    """JRT-RNN prefix prefill; returns (y, S_out, z_out) with the merged state.
    compact=True: the state tensors use the compact layout (jrt_prefix_prefill_compact).
    prefix_len: int32 device tensor [B] of valid (left-padded) prefix lengths
    (jrt_prefix_prefill_ex), or None."""
    B, H, N, d = q.shape
    M = k_e.shape[2]
    dv = v.shape[-1]
    y, S_out, z_out = _outputs(q, v, N, y, S_out, z_out, out_dtype, want_y, want_state, compact)
    if prefix_len is not None:
        if prefix_len.dtype != torch.int32 or prefix_len.numel() != B:
            raise ValueError("prefix_len must be an int32 tensor with B entries")
        st = lib.jrt_prefix_prefill_ex(
            B, H, N, M, d, dv, _dt(q), _dt(y) if y is not None else BLA_F32, float(eps), _ptr(q),
            _ptr(k), _ptr(v), _ptr(k_e), _ptr(v_e), _ptr(prefix_len), _ptr(S0), _ptr(z0), _ptr(y),
            _ptr(S_out), _ptr(z_out), BLA_STATE_COMPACT if compact else BLA_STATE_FULL,
            _stream(stream))
        _check(st, "jrt_prefix_prefill_ex")
        return y, S_out, z_out
    fn = lib.jrt_prefix_prefill_compact if compact else lib.jrt_prefix_prefill
    st = fn(B, H, N, M, d, dv, _dt(q), _dt(y) if y is not None else BLA_F32,
                                float(eps), _ptr(q), _ptr(k), _ptr(v), _ptr(k_e), _ptr(v_e),
                                _ptr(S0), _ptr(z0), _ptr(y), _ptr(S_out), _ptr(z_out),
                                _stream(stream))
    _check(st, "jrt_prefix_prefill_compact" if compact else "jrt_prefix_prefill")
    return y, S_out, z_out


def based_decode_step(q, k, v, S, z, *, eps: float = 0.0, y=None, out_dtype=None, stream=None,
                      compact: bool = False):
    """One decode step; S and z are updated in place; returns y [B,H,d_v].
    compact=True: S, z use the compact layout (based_decode_step_compact)."""
    B, H, d = q.shape
    dv = v.shape[-1]
    if y is None:
        y = torch.empty((B, H, dv), dtype=out_dtype or torch.float32, device=v.device)
    fn = lib.based_decode_step_compact if compact else lib.based_decode_step
    st = fn(B, H, d, dv, _dt(q), _dt(y), float(eps), _ptr(q), _ptr(k),
                               _ptr(v), _ptr(S), _ptr(z), _ptr(y), _stream(stream))
    _check(st, "based_decode_step_compact" if compact else "based_decode_step")
    return y


def swa_prefill(q, k, v, window: int, *, y=None, out_dtype=None, want_cache: bool = False,
                k_cache=None, v_cache=None, stream=None):
    """Sliding-window softmax attention over [B,H,N,64] bf16 inputs; returns
    (y, k_cache, v_cache) (caches None unless requested)."""
    B, H, N, d = q.shape
    dv = v.shape[-1]
    if y is None:
        y = torch.empty((B, H, N, dv), dtype=out_dtype or torch.float32, device=v.device)
    if want_cache and k_cache is None:
        k_cache = torch.zeros((B, H, window, d), dtype=k.dtype, device=k.device)
        v_cache = torch.zeros((B, H, window, dv), dtype=v.dtype, device=v.device)
    st = lib.swa_prefill(B, H, N, d, dv, int(window), _dt(q), _dt(y), _ptr(q), _ptr(k), _ptr(v),
                         _ptr(y), _ptr(k_cache), _ptr(v_cache), _stream(stream))
    _check(st, "swa_prefill")
    return y, k_cache, v_cache


def swa_decode_step(q, k, v, k_cache, v_cache, pos: int, window: int, *, y=None, out_dtype=None,
                    stream=None):
    """One SWA decode step for the token at position pos (caches updated in place); returns y."""
    B, H, d = q.shape
    dv = v.shape[-1]
    if y is None:
        y = torch.empty((B, H, dv), dtype=out_dtype or torch.float32, device=v.device)
    st = lib.swa_decode_step(B, H, d, dv, int(window), int(pos), _dt(q), _dt(y), _ptr(q), _ptr(k),
                             _ptr(v), _ptr(k_cache), _ptr(v_cache), _ptr(y), _stream(stream))
    _check(st, "swa_decode_step")
    return y


def probe_mfma_f16(sink, blocks: int, iters: int, stream=None):
    """Matrix-core peak probe (include/based_la_probe.h); returns its FLOP count."""
    _check(lib.bla_probe_mfma_f16(int(blocks), int(iters), _ptr(sink), _stream(stream)),
           "bla_probe_mfma_f16")
    return blocks * 4 * iters * 8 * 16384


def probe_copy(src, dst, stream=None):
    """HBM streaming-copy probe; returns the bytes moved (read + write)."""
    nbytes = src.numel() * src.element_size()
    _check(lib.bla_probe_copy(_ptr(src), _ptr(dst), nbytes, _stream(stream)), "bla_probe_copy")
    return 2 * nbytes


def probe_prefill_traffic(q, k, v, y, sink, mode: int = 0, stream=None):
    """The prefill's HBM traffic with no arithmetic (include/based_la_probe.h);
    returns the bytes it moves (mode 0: reads + writes, 1: reads, 2: writes)."""
    B, H, N, _ = q.shape
    _check(lib.bla_probe_prefill_traffic(B * H, N, _ptr(q), _ptr(k), _ptr(v), _ptr(y), _ptr(sink), int(mode),
                                         _stream(stream)), "bla_probe_prefill_traffic")
    rd, wr = B * H * N * 192, B * H * N * 256
    return (rd + wr, rd, wr)[mode]
