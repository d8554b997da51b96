"""Python binding of libseed.so: argument marshalling only.

Every function here takes torch tensors that already live in device memory,
checks that their shapes agree, and passes raw pointers and sizes to the C
ABI declared in include/seed.h, on torch's current HIP stream.  All
arithmetic happens in the HIP kernels.  If the library has not been built
the first call raises; there is no fallback of any kind.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# SEED_LIBRARY names another build of the same C ABI (the tests' host-only
# sanitizer build); by default the in-tree libseed.so
LIB_PATH = os.environ.get("SEED_LIBRARY") or os.path.join(_PKG, "libseed.so")
HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "seed.h")

RULES = {"gdn": 0, "kda": 1, "mamba2": 2}
STATUS = {0: "SEED_OK", 1: "SEED_E_ARG", 2: "SEED_E_SHAPE", 3: "SEED_E_UNSUPPORTED",
          4: "SEED_E_FULL", 5: "SEED_E_DEVICE"}

_lib = None


class SeedError(RuntimeError):
    def __init__(self, fn: str, status: int, detail: str):
        super().__init__(f"{fn} failed: {STATUS.get(status, status)}: {detail}")
        self.fn = fn
        self.status = status
        self.detail = detail


def header_functions() -> list:
    """Names of the functions include/seed.h declares."""
    text = open(HEADER_PATH).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?[a-z_]+\s*\*?\s*([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M)


def lib() -> ctypes.CDLL:
    """Load libseed.so (once).  Raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m sink_rank_recurrent_amd.build` (no fallback exists)")
    L = ctypes.CDLL(LIB_PATH)
    i, p, f = ctypes.c_int, ctypes.c_void_p, ctypes.c_float
    L.seed_decode_step.argtypes = [i, i, i, i, i, i, i, p, p, p, p, p, p, p, i, p, p, p, p]
    L.seed_decode_step_lazy.argtypes = [i, i, i, i, i, i, i, p, p, p, p, p, p, p, p, i, p, p, p, p]
    L.seed_compress.argtypes = [i, i, i, i, i, i, i, p, p, p]
    L.seed_compress_lazy.argtypes = [i, i, i, i, i, i, i, i, p, p, p, p]
    L.seed_state_from_dense.argtypes = [i, i, i, i, i, i, p, p, p, p, p, p]
    L.dense_decode_step.argtypes = [i, i, i, i, i, p, p, p, p, i, p, p, p, p]
    u64, u32 = ctypes.c_uint64, ctypes.c_uint32
    L.seed_decode_step_h16.argtypes = [i, i, i, i, i, i, i, i, p, p, p, p, p, p, p, p, p, p, i, i,
                                       p, p, p, p]
    L.seed_compress_h16.argtypes = [i, i, i, i, i, i, i, i, p, p, p, p, p, i, i, u64, u32, p]
    L.seed_round_factors.argtypes = [i, i, i, i, i, p, p, p, p, i, i, u64, u32, p]
    L.seed_pack_states.argtypes = [i, i, i, i, i, i, i, i, p, p, p, p, p, p]
    L.seed_unpack_states.argtypes = [i, i, i, i, i, i, i, i, p, p, p, p, p, p]
    L.seed_state_stats.argtypes = [i, i, i, i, i, p, p, p, p, p, p]
    L.seed_decode_step_sched.argtypes = [i, i, i, i, i, i, i, i, i, p, p, p, p, p, p, p, p, p, p,
                                         p, p, i, p, p, p, p]
    L.seed_compress_sched.argtypes = [i, i, i, i, i, i, i, i, i, p, i, p, p, p, p, p, p, p]
    L.seed_stat_fields.argtypes = []
    L.seed_handoff_head_bytes.argtypes = [i, i, i, i]
    L.seed_handoff_head_bytes.restype = ctypes.c_size_t
    L.seed_stream_copy.argtypes = [p, p, ctypes.c_size_t, p]
    L.seed_join_states.argtypes = [i, i, i, i, i, i, i, i, i, p, p, p, p, p, p, p]
    L.seed_workspace_bytes.argtypes = [i, i, i, i, i, i]
    L.seed_workspace_bytes.restype = ctypes.c_size_t
    for fn in ("seed_decode_step", "seed_decode_step_lazy", "seed_compress", "seed_compress_lazy",
               "seed_state_from_dense", "dense_decode_step", "seed_decode_step_h16",
               "seed_compress_h16", "seed_round_factors", "seed_pack_states",
               "seed_unpack_states", "seed_state_stats", "seed_stat_fields",
               "seed_decode_step_sched", "seed_compress_sched", "seed_stream_copy",
               "seed_abi_version", "seed_join_states"):
        getattr(L, fn).restype = ctypes.c_int
    L.seed_status_string.argtypes = [i]
    L.seed_status_string.restype = ctypes.c_char_p
    L.seed_last_error.argtypes = []
    L.seed_last_error.restype = ctypes.c_char_p
    _lib = L
    return L


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise SeedError(fn, status, lib().seed_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(stream, device_index: int):
    """Handle of `stream`, else of torch's current stream on the tensors' device."""
    if stream is not None:
        return stream.cuda_stream
    if _raw_stream is not None:
        return _raw_stream(device_index)
    return torch.cuda.current_stream(device_index).cuda_stream


def _need(t: torch.Tensor, name: str, shape: tuple, dtypes) -> None:
    # one combined test on the hot path; the detailed message only on failure
    if (isinstance(t, torch.Tensor) and t.is_cuda and t.shape == shape and t.dtype in dtypes
            and t.is_contiguous()):
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be in device memory (got {t.device})")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    raise ValueError(f"{name} must be contiguous")


_F32 = (torch.float32,)
_IN = (torch.float32, torch.bfloat16)


def _in_dtype(q, k, v) -> int:
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k and v must share one dtype")
    return 1 if q.dtype == torch.bfloat16 else 0


def seed_decode_step(rule: str, a, U, V, vbar, q, k, v, g, beta, o, r: int, stream=None) -> None:
    """One decode step on the shallow states (see include/seed.h)."""
    B, H, cap, d_k = U.shape
    d_v = V.shape[-1]
    _need(a, "a", (B, H, d_k), _F32)
    _need(U, "U", (B, H, cap, d_k), _F32)
    _need(V, "V", (B, H, cap, d_v), _F32)
    _need(vbar, "vbar", (H, d_v), _F32)
    _need(q, "q", (B, H, d_k), _IN)
    _need(k, "k", (B, H, d_k), _IN)
    _need(v, "v", (B, H, d_v), _IN)
    _need(g, "g", (B, H, d_k) if rule == "kda" else (B, H), _F32)
    if beta is not None:
        _need(beta, "beta", (B, H), _F32)
    _need(o, "o", (B, H, d_v), _F32)
    st = lib().seed_decode_step(RULES[rule], B, H, d_k, d_v, cap, int(r), _ptr(a), _ptr(U),
                                _ptr(V), _ptr(vbar), _ptr(q), _ptr(k), _ptr(v), _in_dtype(q, k, v),
                                _ptr(g), _ptr(beta), _ptr(o), _stream(stream, U.device.index))
    _check("seed_decode_step", st)


def _gam_shape(rule: str, B: int, H: int, d_k: int) -> tuple:
    return (B, H, d_k) if rule == "kda" else (B, H)


def seed_decode_step_lazy(rule: str, a, U, V, gam, vbar, q, k, v, g, beta, o, r: int,
                          stream=None) -> None:
    """One decode step on lazily decayed shallow states (see include/seed.h)."""
    B, H, cap, d_k = U.shape
    d_v = V.shape[-1]
    _need(a, "a", (B, H, d_k), _F32)
    _need(U, "U", (B, H, cap, d_k), _F32)
    _need(V, "V", (B, H, cap, d_v), _F32)
    _need(gam, "gam", _gam_shape(rule, B, H, d_k), _F32)
    _need(vbar, "vbar", (H, d_v), _F32)
    _need(q, "q", (B, H, d_k), _IN)
    _need(k, "k", (B, H, d_k), _IN)
    _need(v, "v", (B, H, d_v), _IN)
    _need(g, "g", (B, H, d_k) if rule == "kda" else (B, H), _F32)
    if beta is not None:
        _need(beta, "beta", (B, H), _F32)
    _need(o, "o", (B, H, d_v), _F32)
    st = lib().seed_decode_step_lazy(RULES[rule], B, H, d_k, d_v, cap, int(r), _ptr(a), _ptr(U),
                                     _ptr(V), _ptr(gam), _ptr(vbar), _ptr(q), _ptr(k), _ptr(v),
                                     _in_dtype(q, k, v), _ptr(g), _ptr(beta), _ptr(o),
                                     _stream(stream, U.device.index))
    _check("seed_decode_step_lazy", st)


def seed_compress_lazy(rule: str, U, V, gam, r: int, R: int, stream=None) -> None:
    """Compress lazily decayed factors from r to R columns (see include/seed.h)."""
    B, H, cap, d_k = U.shape
    d_v = V.shape[-1]
    _need(U, "U", (B, H, cap, d_k), _F32)
    _need(V, "V", (B, H, cap, d_v), _F32)
    _need(gam, "gam", _gam_shape(rule, B, H, d_k), _F32)
    st = lib().seed_compress_lazy(RULES[rule], B, H, d_k, d_v, cap, int(r), int(R), _ptr(U),
                                  _ptr(V), _ptr(gam), _stream(stream, U.device.index))
    _check("seed_compress_lazy", st)


def seed_compress(U, V, r: int, R: int, stream=None) -> None:
    """Compress every unit's factors from r to R columns (see include/seed.h)."""
    B, H, cap, d_k = U.shape
    d_v = V.shape[-1]
    _need(U, "U", (B, H, cap, d_k), _F32)
    _need(V, "V", (B, H, cap, d_v), _F32)
    st = lib().seed_compress(B, H, d_k, d_v, cap, int(r), int(R), _ptr(U), _ptr(V),
                             _stream(stream, U.device.index))
    _check("seed_compress", st)


def seed_state_from_dense(S, vbar, a, U, V, R: int, stream=None) -> None:
    """Convert dense states to sink + rank-R factors (see include/seed.h)."""
    B, H, cap, d_k = U.shape
    d_v = V.shape[-1]
    _need(S, "S", (B, H, d_k, d_v), _F32)
    _need(vbar, "vbar", (H, d_v), _F32)
    _need(a, "a", (B, H, d_k), _F32)
    _need(U, "U", (B, H, cap, d_k), _F32)
    _need(V, "V", (B, H, cap, d_v), _F32)
    st = lib().seed_state_from_dense(B, H, d_k, d_v, cap, int(R), _ptr(S), _ptr(vbar), _ptr(a),
                                     _ptr(U), _ptr(V), _stream(stream, U.device.index))
    _check("seed_state_from_dense", st)


def dense_decode_step(rule: str, S, q, k, v, g, beta, o, stream=None) -> None:
    """Dense-state baseline step (see include/seed.h)."""
    B, H, d_k, d_v = S.shape
    _need(S, "S", (B, H, d_k, d_v), _F32)
    _need(q, "q", (B, H, d_k), _IN)
    _need(k, "k", (B, H, d_k), _IN)
    _need(v, "v", (B, H, d_v), _IN)
    _need(g, "g", (B, H, d_k) if rule == "kda" else (B, H), _F32)
    if beta is not None:
        _need(beta, "beta", (B, H), _F32)
    _need(o, "o", (B, H, d_v), _F32)
    st = lib().dense_decode_step(RULES[rule], B, H, d_k, d_v, _ptr(S), _ptr(q), _ptr(k), _ptr(v),
                                 _in_dtype(q, k, v), _ptr(g), _ptr(beta), _ptr(o),
                                 _stream(stream, S.device.index))
    _check("dense_decode_step", st)


def workspace_bytes(batch: int, heads: int, d_k: int, d_v: int, cap: int, R: int) -> int:
    """Device workspace the compressions and the conversion need (see
    include/seed.h); raises for a shape they reject."""
    n = int(lib().seed_workspace_bytes(batch, heads, d_k, d_v, cap, R))
    if n == ctypes.c_size_t(-1).value:
        raise ValueError(f"seed_workspace_bytes: shape rejected (batch={batch} heads={heads} "
                         f"d_k={d_k} d_v={d_v} cap={cap} R={R})")
    return n


def stream_copy(src, dst, stream=None) -> None:
    """Bandwidth probe (see include/seed.h): copy src into dst, two
    contiguous device tensors of the same byte size."""
    if not (src.is_cuda and dst.is_cuda):
        raise ValueError("stream_copy: tensors must be in device memory")
    if not (src.is_contiguous() and dst.is_contiguous()):
        raise ValueError("stream_copy: tensors must be contiguous")
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes:
        raise ValueError("stream_copy: src and dst differ in size")
    st = lib().seed_stream_copy(_ptr(src), _ptr(dst), nbytes, _stream(stream, src.device.index))
    _check("seed_stream_copy", st)


# 16-bit kept factors: the tensor dtype names the pattern format
_STORE = {torch.bfloat16: 1, torch.float16: 2}
_H16 = tuple(_STORE)
ROUNDING = {"nearest": 0, "stochastic": 1}


def _store_dtype(Uk, Vk) -> int:
    if Uk.dtype != Vk.dtype or Uk.dtype not in _STORE:
        raise ValueError("Uk and Vk must share one dtype, bfloat16 or float16")
    return _STORE[Uk.dtype]


def seed_decode_step_h16(rule: str, a, Uk, Vk, Uw, Vw, gam, vbar, q, k, v, g, beta, o, r: int,
                         stream=None) -> None:
    """One decode step on the 16-bit form (see include/seed.h)."""
    B, H, R, d_k = Uk.shape
    W, d_v = Uw.shape[2], Vk.shape[-1]
    _need(a, "a", (B, H, d_k), _F32)
    _need(Uk, "Uk", (B, H, R, d_k), _H16)
    _need(Vk, "Vk", (B, H, R, d_v), _H16)
    _need(Uw, "Uw", (B, H, W, d_k), _F32)
    _need(Vw, "Vw", (B, H, W, d_v), _F32)
    _need(gam, "gam", _gam_shape(rule, B, H, d_k), _F32)
    _need(vbar, "vbar", (H, d_v), _F32)
    _need(q, "q", (B, H, d_k), _IN)
    _need(k, "k", (B, H, d_k), _IN)
    _need(v, "v", (B, H, d_v), _IN)
    _need(g, "g", (B, H, d_k) if rule == "kda" else (B, H), _F32)
    if beta is not None:
        _need(beta, "beta", (B, H), _F32)
    _need(o, "o", (B, H, d_v), _F32)
    st = lib().seed_decode_step_h16(RULES[rule], B, H, d_k, d_v, R, W, int(r), _ptr(a), _ptr(Uk),
                                    _ptr(Vk), _ptr(Uw), _ptr(Vw), _ptr(gam), _ptr(vbar), _ptr(q),
                                    _ptr(k), _ptr(v), _in_dtype(q, k, v), _store_dtype(Uk, Vk),
                                    _ptr(g), _ptr(beta), _ptr(o), _stream(stream, Uk.device.index))
    _check("seed_decode_step_h16", st)


def seed_compress_h16(rule: str, Uk, Vk, Uw, Vw, gam, r: int, rounding: str = "nearest",
                      seed: int = 0, epoch: int = 0, stream=None) -> None:
    """Compress the 16-bit form from r to R columns, rounding into Uk, Vk
    (see include/seed.h)."""
    B, H, R, d_k = Uk.shape
    W, d_v = Uw.shape[2], Vk.shape[-1]
    _need(Uk, "Uk", (B, H, R, d_k), _H16)
    _need(Vk, "Vk", (B, H, R, d_v), _H16)
    _need(Uw, "Uw", (B, H, W, d_k), _F32)
    _need(Vw, "Vw", (B, H, W, d_v), _F32)
    _need(gam, "gam", _gam_shape(rule, B, H, d_k), _F32)
    st = lib().seed_compress_h16(RULES[rule], B, H, d_k, d_v, R, W, int(r), _ptr(Uk), _ptr(Vk),
                                 _ptr(Uw), _ptr(Vw), _ptr(gam), _store_dtype(Uk, Vk),
                                 ROUNDING[rounding], int(seed), int(epoch),
                                 _stream(stream, Uk.device.index))
    _check("seed_compress_h16", st)


def seed_round_factors(U, V, Uk, Vk, rounding: str = "nearest", seed: int = 0, epoch: int = 0,
                       stream=None) -> None:
    """Round fp32 rank-R factors into 16-bit kept columns (see include/seed.h)."""
    B, H, R, d_k = U.shape
    d_v = V.shape[-1]
    _need(U, "U", (B, H, R, d_k), _F32)
    _need(V, "V", (B, H, R, d_v), _F32)
    _need(Uk, "Uk", (B, H, R, d_k), _H16)
    _need(Vk, "Vk", (B, H, R, d_v), _H16)
    st = lib().seed_round_factors(B, H, d_k, d_v, R, _ptr(U), _ptr(V), _ptr(Uk), _ptr(Vk),
                                  _store_dtype(Uk, Vk), ROUNDING[rounding], int(seed), int(epoch),
                                  _stream(stream, U.device.index))
    _check("seed_round_factors", st)


def _bound_step(fn, name: str, head: tuple, tail_state: tuple, rule: str, B: int, H: int,
                d_k: int, d_v: int, o, extra_code: tuple = ()):
    """A decode-step call whose state arguments are fixed: `head` are the
    leading integer arguments before r, `tail_state` the state pointers that
    follow r.  Each call checks only the step inputs (one combined test, the
    detailed checks only on failure) and passes their pointers."""
    _need(o, "o", (B, H, d_v), _F32)
    sq = torch.Size((B, H, d_k))
    sv = torch.Size((B, H, d_v))
    sg = torch.Size((B, H, d_k) if rule == "kda" else (B, H))
    sb = torch.Size((B, H))
    op = o.data_ptr()
    dev = o.device.index
    mamba = rule == "mamba2"

    def step(q, k, v, g, beta, r: int, stream=None) -> None:
        dt = q.dtype
        if not (q.shape == sq and k.shape == sq and v.shape == sv and g.shape == sg
                and k.dtype is dt and v.dtype is dt and (dt is torch.bfloat16 or dt is torch.float32)
                and g.dtype is torch.float32 and q.is_cuda and k.is_cuda and v.is_cuda and g.is_cuda
                and q.is_contiguous() and k.is_contiguous() and v.is_contiguous()
                and g.is_contiguous()
                and (beta is None if mamba else (beta.shape == sb and beta.dtype is torch.float32
                                                 and beta.is_cuda and beta.is_contiguous()))):
            _need(q, "q", tuple(sq), _IN)
            _need(k, "k", tuple(sq), _IN)
            _need(v, "v", tuple(sv), _IN)
            _need(g, "g", tuple(sg), _F32)
            if beta is not None:
                _need(beta, "beta", tuple(sb), _F32)
            _in_dtype(q, k, v)
        st = fn(*head, int(r), *tail_state, q.data_ptr(), k.data_ptr(), v.data_ptr(),
                1 if dt is torch.bfloat16 else 0, *extra_code, g.data_ptr(),
                None if beta is None else beta.data_ptr(), op, _stream(stream, dev))
        if st != 0:
            _check(name, st)

    return step


_STORE_CODE = {torch.float32: 0, torch.bfloat16: 1, torch.float16: 2}


def handoff_head_bytes(d_k: int, d_v: int, R: int, store=torch.float32) -> int:
    """Bytes of one packed head (see include/seed.h)."""
    return int(lib().seed_handoff_head_bytes(d_k, d_v, R, _STORE_CODE[store]))


def _handoff_args(a, U, V, R, idx, buf, n_sel):
    B, H, cap, d_k = U.shape
    d_v = V.shape[-1]
    if U.dtype not in _STORE_CODE or V.dtype != U.dtype:
        raise ValueError("U and V must share one dtype: float32, bfloat16 or float16")
    _need(a, "a", (B, H, d_k), _F32)
    _need(U, "U", (B, H, cap, d_k), (U.dtype,))
    _need(V, "V", (B, H, cap, d_v), (U.dtype,))
    _need(idx, "indices", (n_sel,), (torch.int32,))
    nbytes = n_sel * H * handoff_head_bytes(d_k, d_v, R, U.dtype)
    _need(buf, "buf", (nbytes,), (torch.uint8,))
    return B, H, d_k, d_v, cap, _STORE_CODE[U.dtype]


def seed_pack_states(a, U, V, R: int, sel, buf, stream=None) -> None:
    """Pack requests `sel` (int32, device) of a state into `buf` (uint8,
    device, n_sel * heads * head bytes); see include/seed.h."""
    n_sel = sel.shape[0]
    B, H, d_k, d_v, cap, code = _handoff_args(a, U, V, R, sel, buf, n_sel)
    st = lib().seed_pack_states(B, H, d_k, d_v, cap, int(R), code, n_sel, _ptr(sel), _ptr(a),
                                _ptr(U), _ptr(V), _ptr(buf), _stream(stream, a.device.index))
    _check("seed_pack_states", st)


def seed_unpack_states(buf, a, U, V, R: int, slots, stream=None) -> None:
    """Write the packed requests of `buf` into batch slots `slots`; see
    include/seed.h."""
    n_sel = slots.shape[0]
    B, H, d_k, d_v, cap, code = _handoff_args(a, U, V, R, slots, buf, n_sel)
    st = lib().seed_unpack_states(B, H, d_k, d_v, cap, int(R), code, n_sel, _ptr(slots), _ptr(buf),
                                  _ptr(a), _ptr(U), _ptr(V), _stream(stream, a.device.index))
    _check("seed_unpack_states", st)


def seed_join_states(rule: str, buf, a, U, V, gam, R: int, r: int, slots, stream=None) -> None:
    """Write packed fp32 requests into batch slots `slots` of a batch that
    holds r columns, zeroing its columns R..r-1 and (gam given) setting
    its decay product to 1; see include/seed.h."""
    n_sel = slots.shape[0]
    B, H, cap, d_k = U.shape
    d_v = V.shape[-1]
    _need(a, "a", (B, H, d_k), _F32)
    _need(U, "U", (B, H, cap, d_k), _F32)
    _need(V, "V", (B, H, cap, d_v), _F32)
    _need(slots, "slots", (n_sel,), (torch.int32,))
    if gam is not None:
        _need(gam, "gam", _gam_shape(rule, B, H, d_k), _F32)
    _need(buf, "buf", (n_sel * H * handoff_head_bytes(d_k, d_v, R),), (torch.uint8,))
    st = lib().seed_join_states(RULES[rule], B, H, d_k, d_v, cap, int(R), int(r), n_sel,
                                _ptr(slots), _ptr(buf), _ptr(a), _ptr(U), _ptr(V), _ptr(gam),
                                _stream(stream, a.device.index))
    _check("seed_join_states", st)


STAT_FIELDS = ("e_state", "e_sink", "e_content", "sink_share", "top_share",
               "abs_cos_vstar_vbar", "rank90", "rank99", "beyond_R_share")


def seed_state_stats(S, vbar, R: int, rec, spec_S=None, spec_C=None, stream=None) -> None:
    """Statistics of dense states into rec [B, H, seed_stat_fields()] and,
    optionally, the sorted spectra [B, H, d_k] (see include/seed.h)."""
    B, H, d_k, d_v = S.shape
    nf = lib().seed_stat_fields()
    _need(S, "S", (B, H, d_k, d_v), _F32)
    _need(vbar, "vbar", (H, d_v), _F32)
    _need(rec, "rec", (B, H, nf), _F32)
    for name, t in (("spec_S", spec_S), ("spec_C", spec_C)):
        if t is not None:
            _need(t, name, (B, H, d_k), _F32)
    st = lib().seed_state_stats(B, H, d_k, d_v, int(R), _ptr(S), _ptr(vbar), _ptr(rec),
                                _ptr(spec_S), _ptr(spec_C), _stream(stream, S.device.index))
    _check("seed_state_stats", st)


def _first_window(W: int, first_window) -> int:
    fw = W if first_window is None else int(first_window)
    if not 1 <= fw <= W:
        raise ValueError(f"first_window must lie in 1 .. W = {W} (got {fw})")
    return fw


class ShallowState:
    """Device tensors of one layer's shallow states plus the column count r.

    a [B, H, d_k], U [B, H, R+W, d_k], V [B, H, R+W, d_v] (fp32, zeroed) and the
    shared vbar [H, d_v].  `step` advances r; `step_and_maybe_compress`
    compresses when r reaches `limit`: R + first_window for the first window
    after a conversion, R + W after that.  A first window shorter than W puts
    this layer's compressions on another phase than those of layers that
    start with a full one (the pages compress every W steps; at which step a
    layer's cycle starts is the engine's choice).
    """

    def __init__(self, rule: str, batch: int, heads: int, d_k: int, d_v: int, R: int, W: int,
                 vbar: torch.Tensor, device="cuda", lazy: bool = False, first_window=None):
        self.rule, self.R, self.W, self.lazy = rule, R, W, lazy
        self.first_window = _first_window(W, first_window)
        self.limit = R + W
        self.batch, self.heads, self.d_k, self.d_v = batch, heads, d_k, d_v
        f32 = torch.float32
        self.a = torch.zeros(batch, heads, d_k, device=device, dtype=f32)
        self.U = torch.zeros(batch, heads, R + W, d_k, device=device, dtype=f32)
        self.V = torch.zeros(batch, heads, R + W, d_v, device=device, dtype=f32)
        self.vbar = vbar.to(device=device, dtype=f32).contiguous()
        # lazy form: U = Diag(gam) U~, gam the decay product since the last compression
        self.gam = (torch.ones(_gam_shape(rule, batch, heads, d_k), device=device, dtype=f32)
                    if lazy else None)
        self.r = 0

    @property
    def cap(self) -> int:
        return self.R + self.W

    def from_dense(self, S: torch.Tensor, stream=None) -> None:
        seed_state_from_dense(S, self.vbar, self.a, self.U, self.V, self.R, stream)
        if self.lazy:
            self.gam.fill_(1.0)
        self.r = self.R
        self.limit = self.R + self.first_window

    def step(self, q, k, v, g, beta, o, stream=None) -> None:
        if self.lazy:
            seed_decode_step_lazy(self.rule, self.a, self.U, self.V, self.gam, self.vbar, q, k, v,
                                  g, beta, o, self.r, stream)
        else:
            seed_decode_step(self.rule, self.a, self.U, self.V, self.vbar, q, k, v, g, beta, o,
                             self.r, stream)
        self.r += 1

    def bind_step(self, o):
        """A fast form of `step` for a loop that writes read-outs to `o`:
        the state's tensors and o are checked once, each call checks only
        the step's inputs.  Call it as f(q, k, v, g, beta, r); it does not
        advance self.r.  Valid while the state's tensors are not replaced."""
        B, H, d_k, d_v = self.batch, self.heads, self.d_k, self.d_v
        head = (RULES[self.rule], B, H, d_k, d_v, self.cap)
        if self.lazy:
            tail = (self.a.data_ptr(), self.U.data_ptr(), self.V.data_ptr(),
                    self.gam.data_ptr(), self.vbar.data_ptr())
            return _bound_step(lib().seed_decode_step_lazy, "seed_decode_step_lazy", head, tail,
                               self.rule, B, H, d_k, d_v, o)
        tail = (self.a.data_ptr(), self.U.data_ptr(), self.V.data_ptr(), self.vbar.data_ptr())
        return _bound_step(lib().seed_decode_step, "seed_decode_step", head, tail, self.rule, B, H,
                           d_k, d_v, o)

    def launch_compress(self, r: int, stream=None) -> None:
        """The compression of r held columns to R, without touching the
        host bookkeeping (for a caller that plans r itself, e.g. a graph)."""
        if self.lazy:
            seed_compress_lazy(self.rule, self.U, self.V, self.gam, r, self.R, stream)
        else:
            seed_compress(self.U, self.V, r, self.R, stream)

    def compress(self, stream=None) -> None:
        self.launch_compress(self.r, stream)
        self.r = min(self.r, self.R)
        self.limit = self.cap

    def pack(self, sel, buf=None, stream=None) -> torch.Tensor:
        """Pack requests `sel` (int32 device tensor) right after a
        compression or conversion (r = R) into a handoff buffer."""
        if self.r != self.R:
            raise RuntimeError("pack needs a compressed state (r = R)")
        if buf is None:
            buf = torch.empty(sel.shape[0] * self.heads
                              * handoff_head_bytes(self.d_k, self.d_v, self.R),
                              dtype=torch.uint8, device=self.a.device)
        seed_pack_states(self.a, self.U, self.V, self.R, sel, buf, stream)
        return buf

    def unpack(self, buf, slots, stream=None) -> None:
        """Write packed requests into batch slots `slots`; the batch must be
        right after a compression (r = R), where gam is 1."""
        if self.r != self.R:
            raise RuntimeError("unpack needs the batch at r = R (aligned schedule)")
        seed_unpack_states(buf, self.a, self.U, self.V, self.R, slots, stream)

    def join(self, buf, slots, stream=None) -> None:
        """Requests packed in `buf` (fp32, seed_pack_states' layout) join the
        batch in slots `slots` mid-window: they hold r columns from now on
        (the ones beyond R zero) and compress with the batch."""
        if not self.R <= self.r < self.cap:
            raise RuntimeError("join needs R <= r < R + W (compress a full window first)")
        seed_join_states(self.rule, buf, self.a, self.U, self.V, self.gam, self.R, self.r, slots,
                         stream)

    def step_and_maybe_compress(self, q, k, v, g, beta, o, stream=None) -> bool:
        """One decode step; compress afterwards when the window is full."""
        self.step(q, k, v, g, beta, o, stream)
        if self.r >= self.limit:
            self.compress(stream)
            return True
        return False


class ShallowState16:
    """Device tensors of one layer's shallow states in the 16-bit form.

    a [B, H, d_k] fp32, kept factors Uk [B, H, R, d_k], Vk [B, H, R, d_v] as
    bfloat16 or float16 patterns, the window Uw [B, H, W, d_k], Vw [B, H, W,
    d_v] fp32, the decay product gam and the shared vbar [H, d_v].  r runs
    from R (right after a compression) to R + W.  Every rounding (from_dense
    and each compression) takes the next epoch of the generator.
    """

    def __init__(self, rule: str, batch: int, heads: int, d_k: int, d_v: int, R: int, W: int,
                 vbar: torch.Tensor, store=torch.float16, rounding: str = "nearest",
                 seed: int = 0, device="cuda", first_window=None):
        if store not in _STORE:
            raise ValueError("store must be torch.bfloat16 or torch.float16")
        self.rule, self.R, self.W, self.store = rule, R, W, store
        self.first_window = _first_window(W, first_window)
        self.limit = R + W
        self.rounding, self.seed, self.epoch = rounding, int(seed), 0
        self.batch, self.heads, self.d_k, self.d_v = batch, heads, d_k, d_v
        f32 = torch.float32
        self.a = torch.zeros(batch, heads, d_k, device=device, dtype=f32)
        self.Uk = torch.zeros(batch, heads, R, d_k, device=device, dtype=store)
        self.Vk = torch.zeros(batch, heads, R, d_v, device=device, dtype=store)
        self.Uw = torch.zeros(batch, heads, W, d_k, device=device, dtype=f32)
        self.Vw = torch.zeros(batch, heads, W, d_v, device=device, dtype=f32)
        self.vbar = vbar.to(device=device, dtype=f32).contiguous()
        self.gam = torch.ones(_gam_shape(rule, batch, heads, d_k), device=device, dtype=f32)
        self.r = R

    @property
    def cap(self) -> int:
        return self.R + self.W

    def from_dense(self, S: torch.Tensor, stream=None) -> None:
        """End-of-prefill compression into the 16-bit form (fp32 factors
        from seed_state_from_dense, then rounded)."""
        B, H, R = self.batch, self.heads, self.R
        U = torch.empty(B, H, R, self.d_k, device=self.a.device, dtype=torch.float32)
        V = torch.empty(B, H, R, self.d_v, device=self.a.device, dtype=torch.float32)
        seed_state_from_dense(S, self.vbar, self.a, U, V, R, stream)
        seed_round_factors(U, V, self.Uk, self.Vk, self.rounding, self.seed, self.epoch, stream)
        self.epoch += 1
        self.gam.fill_(1.0)
        self.r = R
        self.limit = R + self.first_window

    def step(self, q, k, v, g, beta, o, stream=None) -> None:
        seed_decode_step_h16(self.rule, self.a, self.Uk, self.Vk, self.Uw, self.Vw, self.gam,
                             self.vbar, q, k, v, g, beta, o, self.r, stream)
        self.r += 1

    def bind_step(self, o):
        """A fast form of `step` (see ShallowState.bind_step)."""
        B, H, d_k, d_v = self.batch, self.heads, self.d_k, self.d_v
        head = (RULES[self.rule], B, H, d_k, d_v, self.R, self.W)
        tail = (self.a.data_ptr(), self.Uk.data_ptr(), self.Vk.data_ptr(), self.Uw.data_ptr(),
                self.Vw.data_ptr(), self.gam.data_ptr(), self.vbar.data_ptr())
        return _bound_step(lib().seed_decode_step_h16, "seed_decode_step_h16", head, tail,
                           self.rule, B, H, d_k, d_v, o, (_STORE[self.store],))

    def launch_compress(self, r: int, stream=None) -> None:
        """The compression of r held columns into the kept columns with the
        next epoch's words, without touching r (see ShallowState)."""
        if r > self.R:
            seed_compress_h16(self.rule, self.Uk, self.Vk, self.Uw, self.Vw, self.gam, r,
                              self.rounding, self.seed, self.epoch, stream)
            self.epoch += 1

    def compress(self, stream=None) -> None:
        self.launch_compress(self.r, stream)
        self.r = self.R
        self.limit = self.cap

    def pack(self, sel, buf=None, stream=None) -> torch.Tensor:
        """Pack requests `sel` right after a compression (see ShallowState.pack)."""
        if self.r != self.R:
            raise RuntimeError("pack needs a compressed state (r = R)")
        if buf is None:
            buf = torch.empty(sel.shape[0] * self.heads
                              * handoff_head_bytes(self.d_k, self.d_v, self.R, self.store),
                              dtype=torch.uint8, device=self.a.device)
        seed_pack_states(self.a, self.Uk, self.Vk, self.R, sel, buf, stream)
        return buf

    def unpack(self, buf, slots, stream=None) -> None:
        """Write packed requests into batch slots (see ShallowState.unpack)."""
        if self.r != self.R:
            raise RuntimeError("unpack needs the batch at r = R (aligned schedule)")
        seed_unpack_states(buf, self.a, self.Uk, self.Vk, self.R, slots, stream)

    def step_and_maybe_compress(self, q, k, v, g, beta, o, stream=None) -> bool:
        """One decode step; compress afterwards when the window is full."""
        self.step(q, k, v, g, beta, o, stream)
        if self.r >= self.limit:
            self.compress(stream)
            return True
        return False


class ScheduledState:
    """Shallow states of requests that start at different times, each on its
    own compression schedule (see include/seed.h, seed_decode_step_sched).

    Device tensors: a, the kept buffers KU [2, B, H, R, d_k], KV, the window
    rings Uw [B, H, W + D, d_k], Vw, gam, gam_snap, t_start [B] (int32).
    `step` launches one decode step of every request on torch's current
    stream.  The snapshots of `batch_steps` consecutive steps (the requests
    whose windows those steps fill) are compressed by one launch, issued
    after the last of them; a snapshot must be compressed before its merge
    D steps later, so batch_steps <= max(D, 1), and the default, max(D, 1),
    amortises one launch over as many snapshots as the delay allows (fewer,
    larger launches measured faster than more, smaller ones).  With
    side_streams = 0 (the default) the launches run in order on the steps'
    stream; with side_streams > 0 they take that many side streams (default
    priority) in turn and overlap the steps, and the step that merges a
    compression first waits for it.  D = 0 makes every compression finish
    before the next step.
    """

    def __init__(self, rule: str, batch: int, heads: int, d_k: int, d_v: int, R: int, W: int,
                 D: int, vbar: torch.Tensor, t_start, device="cuda", batch_steps=None,
                 side_streams: int = 0):
        import numpy as np

        if not 0 <= D < W:
            raise ValueError("need 0 <= D < W")
        if side_streams < 0:
            raise ValueError("side_streams must be at least 0")
        if batch_steps is None:
            batch_steps = max(D, 1)
        if not 1 <= batch_steps <= max(D, 1):
            raise ValueError("batch_steps must lie in 1 .. max(D, 1)")
        self.rule, self.R, self.W, self.D = rule, R, W, D
        self.batch, self.heads, self.d_k, self.d_v = batch, heads, d_k, d_v
        f32 = torch.float32
        self.a = torch.zeros(batch, heads, d_k, device=device, dtype=f32)
        self.KU = torch.zeros(2, batch, heads, R, d_k, device=device, dtype=f32)
        self.KV = torch.zeros(2, batch, heads, R, d_v, device=device, dtype=f32)
        self.Uw = torch.zeros(batch, heads, W + D, d_k, device=device, dtype=f32)
        self.Vw = torch.zeros(batch, heads, W + D, d_v, device=device, dtype=f32)
        self.vbar = vbar.to(device=device, dtype=f32).contiguous()
        gshape = _gam_shape(rule, batch, heads, d_k)
        self.gam = torch.ones(gshape, device=device, dtype=f32)
        self.gam_snap = torch.ones(gshape, device=device, dtype=f32)
        ts = np.asarray(t_start, dtype=np.int64)
        if ts.shape != (batch,):
            raise ValueError("t_start needs one step per request")
        self.t_start_host = ts
        self.t_start = torch.tensor(ts, dtype=torch.int32, device=device)
        # the units of the requests whose windows fill at the same steps
        self.cohorts = []
        for p in range(W):
            reqs = np.nonzero(ts % W == p)[0]
            units = (reqs[:, None] * heads + np.arange(heads)[None, :]).reshape(-1)
            self.cohorts.append(torch.tensor(units, dtype=torch.int32, device=device)
                                if units.size else None)
        self.batch_steps = int(batch_steps)
        # no side stream: the compressions run in order on the steps' stream
        self.sides = [torch.cuda.Stream(device=device) for _ in range(side_streams)]
        self.pending = {}
        self.t = 0
        self._acc = []         # (snapshot step, phase) of the snapshots not yet launched
        self._lists = {}       # the unit list of each tuple of phases, made once
        self._launches = 0

    def from_dense(self, S: torch.Tensor, stream=None) -> None:
        """Every request's state from its dense state (kept buffer 0)."""
        U = torch.empty(self.batch, self.heads, self.R, self.d_k, device=self.a.device)
        V = torch.empty(self.batch, self.heads, self.R, self.d_v, device=self.a.device)
        seed_state_from_dense(S, self.vbar, self.a, U, V, self.R, stream)
        self.KU[0].copy_(U)
        self.KV[0].copy_(V)
        self.gam.fill_(1.0)
        self.gam_snap.fill_(1.0)

    def held_columns(self, b: int, t=None) -> int:
        """Columns request b holds before step t (default: the next step)."""
        A = (self.t if t is None else t) - int(self.t_start_host[b])
        if A < 0:
            return self.R
        c = 0 if A < self.W + self.D else (A - self.D) // self.W
        return self.R + A - c * self.W

    def step(self, q, k, v, g, beta, o, stream=None) -> None:
        B, H, d_k, d_v = self.batch, self.heads, self.d_k, self.d_v
        cur = torch.cuda.current_stream(self.a.device) if stream is None else stream
        ev = self.pending.pop(self.t, None)
        if ev is not None:
            cur.wait_event(ev)
        for name, t_, shape, dts in (("q", q, (B, H, d_k), _IN), ("k", k, (B, H, d_k), _IN),
                                     ("v", v, (B, H, d_v), _IN),
                                     ("g", g, (B, H, d_k) if self.rule == "kda" else (B, H), _F32),
                                     ("o", o, (B, H, d_v), _F32)):
            _need(t_, name, shape, dts)
        if beta is not None:
            _need(beta, "beta", (B, H), _F32)
        st = lib().seed_decode_step_sched(
            RULES[self.rule], B, H, d_k, d_v, self.R, self.W, self.D, self.t, _ptr(self.t_start),
            _ptr(self.a), _ptr(self.KU), _ptr(self.KV), _ptr(self.Uw), _ptr(self.Vw),
            _ptr(self.gam), _ptr(self.gam_snap), _ptr(self.vbar), _ptr(q), _ptr(k), _ptr(v),
            _in_dtype(q, k, v), _ptr(g), _ptr(beta), _ptr(o), cur.cuda_stream)
        _check("seed_decode_step_sched", st)
        self.t += 1
        p = self.t % self.W
        if self.cohorts[p] is not None:
            self._acc.append((self.t, p))
        if self._acc and self.t - self._acc[0][0] + 1 >= self.batch_steps:
            self._launch(cur)

    def _launch(self, cur) -> None:
        """One compression launch for the accumulated snapshots, on the next
        side stream, after everything enqueued on `cur` so far."""
        key = tuple(p for _, p in self._acc)
        lst = self._lists.get(key)
        if lst is None:
            # made on `cur`, so that every stream ordered after `cur` sees it
            with torch.cuda.stream(cur):
                lst = torch.cat([self.cohorts[p] for p in key])
            self._lists[key] = lst
        if self.sides:
            side = self.sides[self._launches % len(self.sides)]
            snap = torch.cuda.Event()
            snap.record(cur)
            side.wait_event(snap)
        else:
            side = cur
        self._launches += 1
        B, H, d_k, d_v = self.batch, self.heads, self.d_k, self.d_v
        st = lib().seed_compress_sched(
            RULES[self.rule], B, H, d_k, d_v, self.R, self.W, self.D, self.t,
            _ptr(self.t_start), lst.shape[0], _ptr(lst), _ptr(self.KU), _ptr(self.KV),
            _ptr(self.Uw), _ptr(self.Vw), _ptr(self.gam_snap), side.cuda_stream)
        _check("seed_compress_sched", st)
        if self.sides:
            done = torch.cuda.Event()
            done.record(side)
            for ts, _ in self._acc:
                self.pending[ts + self.D] = done
        self._acc = []

    def join(self, stream=None) -> None:
        """Launch the snapshots still waiting for their batch, then order
        `stream` (default: the current one) after every compression launched
        so far."""
        cur = torch.cuda.current_stream(self.a.device) if stream is None else stream
        if self._acc:
            self._launch(cur)
        for side in self.sides:
            cur.wait_stream(side)
