"""ctypes binding of liborca.so: the C entry points of include/orca.h under
the same names, with argument marshalling only.

Device buffers are passed as integers (device addresses) or as torch tensors
(their ``data_ptr()``); streams as ``torch.cuda.Stream`` / raw handles.  Every
status other than ORCA_OK raises ``OrcaError`` carrying the library's
message.  The shared library is loaded on first use; if it has not been built
yet it is built in-tree.  There is no other implementation to fall back to.
"""
from __future__ import annotations

import ctypes
import os
import re
from ctypes import (POINTER, Structure, byref, c_char_p, c_double, c_float, c_int32,
                    c_int64, c_size_t, c_void_p)
from typing import Iterable, List, Optional, Sequence

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
# ORCA_LIB names another build of the library (the sanitized host-only
# build); ORCA_HOST_ONLY=1 accepts one that has only the host entry points
LIB_PATH = os.environ.get("ORCA_LIB") or os.path.join(PKG, "liborca.so")
HOST_ONLY = os.environ.get("ORCA_HOST_ONLY") == "1"
HEADER = os.path.join(ROOT, "include", "orca.h")

ORCA_OK, ORCA_ERR_INVALID, ORCA_ERR_NOSPACE, ORCA_ERR_HIP, ORCA_ERR_UNSUPPORTED = range(5)
ORCA_F32, ORCA_BF16 = 0, 1
ORCA_INITIATION, ORCA_INCREMENT = 0, 1
ORCA_EPI_BIAS, ORCA_EPI_BIAS_GELU, ORCA_EPI_BIAS_RESID = 0, 1, 2
ORCA_POLICY_ITERATION, ORCA_POLICY_STATIC, ORCA_POLICY_CHUNKED = 0, 1, 2
ORCA_STEP_QKV, ORCA_STEP_ATTENTION, ORCA_STEP_OUT_PROJ, ORCA_STEP_FFN1, ORCA_STEP_FFN2 = range(5)

LAYER_KEYS = ("ln1_g", "ln1_b", "w_qkv", "b_qkv", "w_o", "b_o",
              "ln2_g", "ln2_b", "w_1", "b_1", "w_2", "b_2")


class OrcaError(RuntimeError):
    def __init__(self, status: int, where: str, msg: str):
        super().__init__(f"{where}: {_STATUS.get(status, status)}: {msg}")
        self.status = status


_STATUS = {0: "ORCA_OK", 1: "ORCA_ERR_INVALID", 2: "ORCA_ERR_NOSPACE", 3: "ORCA_ERR_HIP",
           4: "ORCA_ERR_UNSUPPORTED"}


class orca_req_desc(Structure):
    _fields_ = [("q_offset", c_int32), ("q_len", c_int32), ("kv_len", c_int32),
                ("phase", c_int32), ("kv_base", c_int64)]


class orca_model_desc(Structure):
    _fields_ = [("layers", c_int32), ("hidden", c_int32), ("heads", c_int32), ("ffn", c_int32),
                ("dtype", c_int32), ("ln_eps", c_float), ("kv_capacity", c_int64)]


class orca_layer_weights(Structure):
    _fields_ = [(k, c_void_p) for k in LAYER_KEYS]


_lib = None


def _declare(lib):
    V, I32, I64, S = c_void_p, c_int32, c_int64, c_size_t
    sig = {
        "orca_status_str": (c_char_p, [c_int32]),
        "orca_last_error": (c_char_p, []),
        "orca_kv_create": (c_int32, [I64, POINTER(V)]),
        "orca_kv_destroy": (None, [V]),
        "orca_kv_alloc": (c_int32, [V, I64, POINTER(I64)]),
        "orca_kv_free": (c_int32, [V, I64]),
        "orca_kv_used": (I64, [V]),
        "orca_kv_capacity": (I64, [V]),
        "orca_kv_reservation": (I64, [V, I64]),
        "orca_create": (c_int32, [POINTER(orca_model_desc), POINTER(orca_layer_weights), V, V,
                                  I32, I32, POINTER(V)]),
        "orca_destroy": (c_int32, [V]),
        "orca_workspace_bytes": (S, [V]),
        "orca_iteration": (c_int32, [V, POINTER(orca_req_desc), I32, V, V, V, S, V]),
        "orca_time_step": (c_int32, [V, I32]),
        "orca_step_times": (c_int32, [V, POINTER(c_float), I32]),
        "orca_op_layernorm": (c_int32, [I32, V, V, V, V, I32, I32, c_float, V]),
        "orca_op_linear_workspace_bytes": (S, [I32, I32, I32, I32]),
        "orca_op_linear_variant": (I32, [I32, I32, I32, I32]),
        "orca_op_prefill_keys": (I32, [I32, I32]),
        "orca_op_prefill_order": (I32, [POINTER(orca_req_desc), I32, I32, POINTER(I32),
                                        POINTER(I32), POINTER(I32), I32]),
        "orca_op_linear": (c_int32, [I32, I32, V, V, V, V, I32, I32, I32, V, S, V]),
        "orca_op_linear_noalloc": (c_int32, [I32, I32, V, V, V, V, I32, I32, I32, V]),
        "orca_op_qkv": (c_int32, [I32, V, V, V, V, V, V, I32, I32, I32, I64, V, S, V]),
        "orca_op_attention": (c_int32, [V, I32, POINTER(orca_req_desc), I32, V, V, V, S, V]),
        "orca_sched_create": (c_int32, [V, I32, I32, I32, POINTER(V)]),
        "orca_sched_destroy": (None, [V]),
        "orca_sched_submit": (c_int32, [V, I64, c_double, I32, I32, I32]),
        "orca_sched_step": (c_int32, [V, c_double, POINTER(orca_req_desc), POINTER(I64), I32,
                                      POINTER(I32)]),
        "orca_sched_cancel": (c_int32, [V, I64]),
        "orca_sched_idle": (I32, [V]),
        "orca_sched_next_arrival": (c_int32, [V, POINTER(c_double)]),
        "orca_sched_request_info": (c_int32, [V, I64, POINTER(I64), POINTER(I64), POINTER(I64)]),
        "orca_sched_used": (I64, [V]),
    }
    for name, (res, args) in sig.items():
        if HOST_ONLY and not hasattr(lib, name):
            continue
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args


def _stale() -> bool:
    """True when a source is newer than the built library."""
    built = os.path.getmtime(LIB_PATH)
    srcs = [os.path.join(PKG, "csrc", f) for f in os.listdir(os.path.join(PKG, "csrc"))]
    return any(os.path.getmtime(f) > built for f in srcs + [HEADER] if os.path.exists(f))


def load():
    """The loaded library.  If it has not been built yet it is built
    in-tree first; a build older than its sources is loaded with a warning
    (rebuild: python -m orca_selective_iteration_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            if os.environ.get("ORCA_LIB"):
                raise OSError(f"ORCA_LIB names a missing library: {LIB_PATH}")
            from .build import build
            build()
        elif not os.environ.get("ORCA_LIB") and _stale():
            import warnings
            warnings.warn(f"{LIB_PATH} is older than its sources; rebuild with "
                          f"python -m orca_selective_iteration_amd.build", stacklevel=2)
        lib = ctypes.CDLL(LIB_PATH)
        _declare(lib)
        _lib = lib
    return _lib


def header_functions() -> List[str]:
    """Names of the functions include/orca.h declares."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(orca_[a-z0-9_]+)\s*\(", text)))


def _check(st: int, where: str):
    if st != ORCA_OK:
        raise OrcaError(st, where, load().orca_last_error().decode())


def ptr(x) -> Optional[int]:
    """Device address of a tensor / int / None."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def stream_handle(stream) -> Optional[int]:
    if stream is None:
        return None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def req_array(reqs: Sequence) -> "ctypes.Array":
    """Descriptors from tuples (q_offset, q_len, kv_len, phase, kv_base) or
    orca_req_desc instances; an array this function built passes through
    (callers timing short launches marshal once)."""
    if isinstance(reqs, ctypes.Array) and reqs._type_ is orca_req_desc:
        return reqs
    arr = (orca_req_desc * max(len(reqs), 1))()
    for i, r in enumerate(reqs):
        arr[i] = r if isinstance(r, orca_req_desc) else orca_req_desc(*[int(v) for v in r])
    return arr


# ------------------------------------------------------------------ status

def orca_status_str(s: int) -> str:
    return load().orca_status_str(s).decode()


def orca_last_error() -> str:
    return load().orca_last_error().decode()


# -------------------------------------------------------------- K/V manager

def orca_kv_create(capacity: int) -> int:
    h = c_void_p()
    _check(load().orca_kv_create(capacity, byref(h)), "orca_kv_create")
    return h.value


def orca_kv_destroy(kv: int) -> None:
    load().orca_kv_destroy(kv)


def orca_kv_alloc(kv: int, n_tokens: int) -> int:
    base = c_int64()
    _check(load().orca_kv_alloc(kv, n_tokens, byref(base)), "orca_kv_alloc")
    return base.value


def orca_kv_free(kv: int, base: int) -> None:
    _check(load().orca_kv_free(kv, base), "orca_kv_free")


def orca_kv_used(kv: int) -> int:
    return load().orca_kv_used(kv)


def orca_kv_capacity(kv: int) -> int:
    return load().orca_kv_capacity(kv)


def orca_kv_reservation(kv: int, base: int) -> int:
    return load().orca_kv_reservation(kv, base)


# ------------------------------------------------------------------ engine

def orca_create(layers: int, hidden: int, heads: int, ffn: int, dtype: int, ln_eps: float,
                kv_capacity: int, weights: Sequence[dict], kv_pool, kv: Optional[int],
                max_rows: int, max_reqs: int) -> int:
    """weights: one dict per layer mapping LAYER_KEYS to tensors / addresses;
    kv_pool: [layers][heads][kv_capacity][2][d] (each slot's key row, then its
    value row)."""
    desc = orca_model_desc(layers, hidden, heads, ffn, dtype, ln_eps, kv_capacity)
    arr = (orca_layer_weights * layers)()
    for l, w in enumerate(weights):
        arr[l] = orca_layer_weights(*[ptr(w[k]) for k in LAYER_KEYS])
    h = c_void_p()
    _check(load().orca_create(byref(desc), arr, ptr(kv_pool), kv, max_rows, max_reqs,
                              byref(h)), "orca_create")
    return h.value


def orca_destroy(ctx: int) -> None:
    _check(load().orca_destroy(ctx), "orca_destroy")


def orca_workspace_bytes(ctx: int) -> int:
    return load().orca_workspace_bytes(ctx)


def orca_iteration(ctx: int, reqs: Sequence, x, y, workspace, ws_bytes: int,
                   stream=None) -> None:
    arr = req_array(reqs)
    _check(load().orca_iteration(ctx, arr, len(reqs), ptr(x), ptr(y), ptr(workspace), ws_bytes,
                                 stream_handle(stream)), "orca_iteration")


def orca_time_step(ctx: int, step: int) -> None:
    _check(load().orca_time_step(ctx, step), "orca_time_step")


def orca_step_times(ctx: int, layers: int) -> List[float]:
    ms = (c_float * max(layers, 1))()
    _check(load().orca_step_times(ctx, ms, layers), "orca_step_times")
    return [ms[i] for i in range(layers)]


def orca_op_layernorm(dtype: int, x, gamma, beta, out, rows: int, hidden: int, eps: float,
                      stream=None) -> None:
    _check(load().orca_op_layernorm(dtype, ptr(x), ptr(gamma), ptr(beta), ptr(out), rows,
                                    hidden, eps, stream_handle(stream)), "orca_op_layernorm")


def orca_op_linear_workspace_bytes(dtype: int, m: int, n: int, k: int) -> int:
    return int(load().orca_op_linear_workspace_bytes(dtype, m, n, k))


def orca_op_linear_variant(dtype: int, m: int, n: int, k: int) -> int:
    return int(load().orca_op_linear_variant(dtype, m, n, k))


def orca_op_prefill_keys(heads: int, tiles: int) -> int:
    return int(load().orca_op_prefill_keys(heads, tiles))


def orca_op_prefill_order(reqs, heads: int):
    """(req, q0, head) of each workgroup of the prefill launch, in launch
    order; raises OrcaError on arguments the library rejects."""
    arr = req_array(reqs)
    n = len(reqs)
    count = int(load().orca_op_prefill_order(arr, n, heads, None, None, None, 0))
    if count < 0:
        raise OrcaError(ORCA_ERR_INVALID, "orca_op_prefill_order", "invalid arguments")
    r, q, h = ((c_int32 * max(count, 1))() for _ in range(3))
    load().orca_op_prefill_order(arr, n, heads, r, q, h, count)
    return [(r[i], q[i], h[i]) for i in range(count)]


def orca_op_linear(dtype: int, epilogue: int, a, w, bias, out, m: int, n: int, k: int,
                   workspace=None, ws_bytes: int = 0, stream=None) -> None:
    _check(load().orca_op_linear(dtype, epilogue, ptr(a), ptr(w), ptr(bias), ptr(out), m, n, k,
                                 ptr(workspace), ws_bytes, stream_handle(stream)),
           "orca_op_linear")


ORCA_NOALLOC_SCRATCH_BYTES = 32 << 20


def orca_op_linear_noalloc(dtype: int, epilogue: int, a, w, bias, out, m: int, n: int, k: int,
                           stream=None) -> None:
    _check(load().orca_op_linear_noalloc(dtype, epilogue, ptr(a), ptr(w), ptr(bias), ptr(out),
                                         m, n, k, stream_handle(stream)),
           "orca_op_linear_noalloc")


def orca_op_qkv(dtype: int, a, w_qkv, b_qkv, q_out, kv_pool_l, row_dst, m: int,
                hidden: int, heads: int, kv_capacity: int, workspace=None, ws_bytes: int = 0,
                stream=None) -> None:
    """kv_pool_l: one layer's pool [heads][kv_capacity][2][d]."""
    _check(load().orca_op_qkv(dtype, ptr(a), ptr(w_qkv), ptr(b_qkv), ptr(q_out), ptr(kv_pool_l),
                              ptr(row_dst), m, hidden, heads, kv_capacity,
                              ptr(workspace), ws_bytes, stream_handle(stream)), "orca_op_qkv")


def orca_op_attention(ctx: int, layer: int, reqs: Sequence, q, o, workspace, ws_bytes: int,
                      stream=None) -> None:
    arr = req_array(reqs)
    _check(load().orca_op_attention(ctx, layer, arr, len(reqs), ptr(q), ptr(o), ptr(workspace),
                                    ws_bytes, stream_handle(stream)), "orca_op_attention")


# --------------------------------------------------------------- scheduler

def orca_sched_create(kv: int, max_batch: int, token_budget: int, policy: int) -> int:
    h = c_void_p()
    _check(load().orca_sched_create(kv, max_batch, token_budget, policy, byref(h)),
           "orca_sched_create")
    return h.value


def orca_sched_destroy(s: int) -> None:
    load().orca_sched_destroy(s)


def orca_sched_submit(s: int, rid: int, arrival: float, prompt_len: int, max_tokens: int,
                      out_len: int) -> None:
    _check(load().orca_sched_submit(s, rid, arrival, prompt_len, max_tokens, out_len),
           "orca_sched_submit")


def orca_sched_step(s: int, now: float, cap: int):
    """Returns (list of orca_req_desc, list of ids)."""
    out = (orca_req_desc * cap)()
    ids = (c_int64 * cap)()
    n = c_int32()
    _check(load().orca_sched_step(s, now, out, ids, cap, byref(n)), "orca_sched_step")
    return [out[i] for i in range(n.value)], [ids[i] for i in range(n.value)]


def orca_sched_cancel(s: int, rid: int) -> None:
    _check(load().orca_sched_cancel(s, rid), "orca_sched_cancel")


def orca_sched_idle(s: int) -> bool:
    return bool(load().orca_sched_idle(s))


def orca_sched_next_arrival(s: int) -> Optional[float]:
    t = c_double()
    st = load().orca_sched_next_arrival(s, byref(t))
    return t.value if st == ORCA_OK else None


def orca_sched_request_info(s: int, rid: int):
    a, f, r = c_int64(), c_int64(), c_int64()
    _check(load().orca_sched_request_info(s, rid, byref(a), byref(f), byref(r)),
           "orca_sched_request_info")
    return a.value, f.value, r.value


def orca_sched_used(s: int) -> int:
    return load().orca_sched_used(s)
