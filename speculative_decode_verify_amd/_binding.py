"""ctypes binding of the C ABI in include/verify_attn.h: argument marshalling only.

Tensors are torch tensors on the GPU; their device pointers, strides and the
current HIP stream are handed to the library, which launches every kernel.
There is no fallback: a missing library raises.
"""
import ctypes
import math
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "lib", "libverify_attn.so")

VA_MAX_ROWS = 16

STATUS = {0: "VA_OK", 1: "VA_ERR_INVALID", 2: "VA_ERR_UNSUPPORTED", 3: "VA_ERR_CAPACITY",
          4: "VA_ERR_WORKSPACE", 5: "VA_ERR_HIP"}
MASKS = {"causal": 0, "window": 1, "tree": 2}
KV_FORMATS = {"bf16": 0, "e4m3_wht_i8": 1}


class VAError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn}: {STATUS.get(status, status)} ({_lib().va_status_string(status).decode()})")


class va_problem(ctypes.Structure):
    _fields_ = [
        ("rows", ctypes.c_int32), ("live_rows", ctypes.c_int32),
        ("q_heads", ctypes.c_int32), ("kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("mask", ctypes.c_int32), ("kv_fmt", ctypes.c_int32),
        ("window", ctypes.c_int32), ("ring_slots", ctypes.c_int32),
        ("splits", ctypes.c_int32), ("num_cus", ctypes.c_int32),
        ("parent", ctypes.c_int32 * VA_MAX_ROWS),
        ("first_pos", ctypes.c_int64), ("prefix_len", ctypes.c_int64),
        ("kv_capacity", ctypes.c_int64), ("scale", ctypes.c_float), ("reserved", ctypes.c_int32),
    ]


class va_state(ctypes.Structure):
    _fields_ = [
        ("first_pos", ctypes.c_int64), ("prefix_len", ctypes.c_int64),
        ("live_rows", ctypes.c_int32), ("reserved", ctypes.c_int32),
        ("parent", ctypes.c_int32 * VA_MAX_ROWS),
    ]


class va_sample_params(ctypes.Structure):
    _fields_ = [
        ("rows", ctypes.c_int32), ("top_k", ctypes.c_int32), ("vocab", ctypes.c_int64),
        ("row_stride", ctypes.c_int64), ("temperature", ctypes.c_float), ("top_p", ctypes.c_float),
        ("seed", ctypes.c_uint64), ("first_position", ctypes.c_int64), ("purpose", ctypes.c_uint32),
        ("reserved", ctypes.c_int32),
    ]


class va_plan(ctypes.Structure):
    _fields_ = [("words", ctypes.c_uint64 * 256)]


class va_plan_info(ctypes.Structure):
    _fields_ = [
        ("splits", ctypes.c_int32), ("matrix_rows", ctypes.c_int32),
        ("lo", ctypes.c_int64), ("hi", ctypes.c_int64),
        ("chunk_lo", ctypes.c_int64), ("chunks", ctypes.c_int64),
        ("row_lo", ctypes.c_int64 * VA_MAX_ROWS), ("row_hi", ctypes.c_int64 * VA_MAX_ROWS),
        ("anc", ctypes.c_uint32 * VA_MAX_ROWS), ("workspace_bytes", ctypes.c_size_t),
        ("row_groups", ctypes.c_int32),
    ]


_LIB = None


def library_path():
    return _LIB_PATH


def trace_library_path():
    """The trace build (phase timestamps; include/verify_probe.h)."""
    return os.path.join(os.path.dirname(_LIB_PATH), "libverify_attn_trace.so")


def load_library():
    """Load libverify_attn.so (raises if it is missing)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is missing: build it with `python -m speculative_decode_verify_amd.build`")
    lib = ctypes.CDLL(_LIB_PATH)
    P, V, I32, I64, SZ = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    lib.verify_attn_plan.argtypes = [ctypes.POINTER(va_problem), ctypes.POINTER(va_plan), ctypes.POINTER(SZ)]
    lib.verify_attn_plan_query.argtypes = [ctypes.POINTER(va_plan), ctypes.POINTER(va_plan_info)]
    lib.verify_attn_plan_split_range.argtypes = [ctypes.POINTER(va_plan), I32, ctypes.POINTER(I64),
                                                 ctypes.POINTER(I64)]
    lib.verify_attn_split.argtypes = [ctypes.POINTER(va_plan), V, V, V, V, I64, I64, I64, V, SZ, V]
    lib.verify_attn_combine.argtypes = [ctypes.POINTER(va_plan), V, SZ, V, V, V, V]
    lib.verify_attn_split_state.argtypes = [ctypes.POINTER(va_plan), V, V, V, V, V, I64, I64, I64, V, SZ, V]
    lib.verify_attn_combine_state.argtypes = [ctypes.POINTER(va_plan), V, V, SZ, V, V, V, V]
    lib.verify_attn_noalloc.argtypes = [ctypes.POINTER(va_plan), V, V, V, V, I64, I64, I64, V, V, V, V]
    lib.verify_attn_split_append.argtypes = [ctypes.POINTER(va_plan), V, V, V, V, V, I64, I64, V, SZ, V]
    lib.verify_attn_split_append_state.argtypes = [ctypes.POINTER(va_plan), V, V, V, V, V, V, I64, I64, V, SZ, V]
    lib.swa_ring_write.argtypes = [V, V, I32, I64, I32, I32, V, V, I32, I64, I64, V]
    lib.verify_kv_write.argtypes = [V, V, I32, I64, I32, I32, I32, V, V, V, I64, I64, I32, I64, I64, V]
    SP = ctypes.POINTER(va_sample_params)
    lib.va_sample_workspace_bytes.argtypes = [SP]
    lib.va_sample_workspace_bytes.restype = SZ
    lib.va_sample.argtypes = [SP, V, V, V, V, V, V, SZ, V]
    lib.va_accept.argtypes = [V, V, V, V, I32, V, V, V, I32, V, I32, ctypes.c_uint64, I64, V, V, V]
    lib.va_sample_accept.argtypes = [SP, V, V, V, V, I32, V, V, V, V, V, V, V, V, SZ, V]
    lib.va_read_probe.argtypes = [V, SZ, V, V]
    lib.va_status_string.argtypes = [ctypes.c_int]
    lib.va_status_string.restype = ctypes.c_char_p
    for fn in ("verify_attn_plan", "verify_attn_plan_query", "verify_attn_plan_split_range",
               "verify_attn_split", "verify_attn_combine", "verify_attn_split_state", "verify_attn_split_append",
               "verify_attn_split_append_state",
               "verify_attn_combine_state", "verify_attn_noalloc", "swa_ring_write", "verify_kv_write", "va_sample", "va_accept",
               "va_sample_accept", "va_read_probe"):
        getattr(lib, fn).restype = ctypes.c_int
    _LIB = lib
    return lib


_lib = load_library


def _check(fn, status):
    if status != 0:
        raise VAError(fn, status)


def _default_cus():
    try:
        import torch
        if torch.cuda.is_available():
            return int(torch.cuda.get_device_properties(torch.cuda.current_device()).multi_processor_count)
    except Exception:
        pass
    return 256


class Plan:
    """A validated plan (host memory).  Keyword arguments mirror va_problem."""

    def __init__(self, rows, live_rows, q_heads, kv_heads, head_dim, mask="causal", kv_fmt="bf16",
                 first_pos=0, prefix_len=0, parent=None, window=0, ring_slots=0, kv_capacity=0,
                 scale=None, splits=0, num_cus=None):
        p = va_problem()
        p.rows, p.live_rows, p.q_heads, p.kv_heads, p.head_dim = rows, live_rows, q_heads, kv_heads, head_dim
        p.mask = MASKS[mask] if isinstance(mask, str) else int(mask)
        p.kv_fmt = KV_FORMATS[kv_fmt] if isinstance(kv_fmt, str) else int(kv_fmt)
        p.window, p.ring_slots, p.splits = window, ring_slots, splits
        p.num_cus = _default_cus() if num_cus is None else num_cus
        par = list(parent) if parent is not None else []
        if len(par) > VA_MAX_ROWS:
            raise ValueError("at most 16 tree nodes")
        for i in range(VA_MAX_ROWS):
            p.parent[i] = par[i] if i < len(par) else -1
        p.first_pos, p.prefix_len, p.kv_capacity = first_pos, prefix_len, kv_capacity
        p.scale = (1.0 / math.sqrt(head_dim)) if scale is None else scale
        p.reserved = 0
        self.problem = p
        self.plan = va_plan()
        ws = ctypes.c_size_t(0)
        _check("verify_attn_plan", _lib().verify_attn_plan(ctypes.byref(p), ctypes.byref(self.plan), ctypes.byref(ws)))
        self.workspace_bytes = ws.value
        self.info = verify_attn_plan_query(self)
        self.rows, self.live_rows, self.q_heads, self.kv_heads, self.head_dim = rows, live_rows, q_heads, kv_heads, head_dim
        self.kv_fmt = p.kv_fmt

    @property
    def splits(self):
        return self.info["splits"]


def verify_attn_plan(**kw):
    return Plan(**kw)


def verify_attn_plan_query(plan):
    info = va_plan_info()
    _check("verify_attn_plan_query", _lib().verify_attn_plan_query(ctypes.byref(plan.plan), ctypes.byref(info)))
    return {
        "splits": info.splits, "matrix_rows": info.matrix_rows, "lo": info.lo, "hi": info.hi,
        "chunk_lo": info.chunk_lo, "chunks": info.chunks, "row_lo": list(info.row_lo), "row_hi": list(info.row_hi),
        "anc": list(info.anc), "workspace_bytes": info.workspace_bytes, "row_groups": info.row_groups,
    }


def verify_attn_plan_split_range(plan, s):
    a, b = ctypes.c_int64(0), ctypes.c_int64(0)
    _check("verify_attn_plan_split_range",
           _lib().verify_attn_plan_split_range(ctypes.byref(plan.plan), s, ctypes.byref(a), ctypes.byref(b)))
    return a.value, b.value


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _require(t, name, dtypes, device=True):
    import torch
    if t is None:
        raise ValueError(f"{name} is required")
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype} not in {dtypes}")
    if device and t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor")


def workspace_for(plan, device=None):
    import torch
    n = (plan.workspace_bytes + 3) // 4
    return torch.empty(max(n, 1), dtype=torch.float32, device=device or "cuda")


def pack_state(first_pos=0, prefix_len=0, live_rows=0, parent=None):
    """The 88-byte va_state record as a CPU int64 tensor of 11 words (copy it
    into a device tensor of the same shape between graph replays)."""
    import torch
    st = va_state()
    st.first_pos, st.prefix_len, st.live_rows, st.reserved = first_pos, prefix_len, live_rows, 0
    par = list(parent) if parent is not None else []
    if len(par) > VA_MAX_ROWS:
        raise ValueError("at most 16 tree nodes")
    for i in range(VA_MAX_ROWS):
        st.parent[i] = par[i] if i < len(par) else -1
    t = torch.empty(ctypes.sizeof(va_state) // 8, dtype=torch.int64)
    ctypes.memmove(t.data_ptr(), ctypes.byref(st), ctypes.sizeof(va_state))
    return t


def _require_state(state):
    import torch
    _require(state, "state", (torch.int64,))
    if not state.is_contiguous() or state.numel() * 8 != ctypes.sizeof(va_state):
        raise ValueError("state must be a contiguous int64 tensor of 11 words (a packed va_state)")


def _split_args(plan, q, k, v, workspace, v_scale):
    """q [rows, Hq, D] bf16 contiguous; k, v [Hkv, slots, D] (bf16, or uint8/int8
    for the quantised format) with the last dimension contiguous; v_scale
    [Hkv, slots] float32 for the quantised format."""
    import torch
    _require(q, "q", (torch.bfloat16,))
    if not q.is_contiguous() or tuple(q.shape) != (plan.rows, plan.q_heads, plan.head_dim):
        raise ValueError(f"q must be contiguous [{plan.rows}, {plan.q_heads}, {plan.head_dim}]")
    if plan.kv_fmt == 0:
        _require(k, "k", (torch.bfloat16,))
        _require(v, "v", (torch.bfloat16,))
    else:
        _require(k, "k", (torch.uint8,))
        _require(v, "v", (torch.int8,))
        _require(v_scale, "v_scale", (torch.float32,))
        if v_scale.stride(1) != 1:
            raise ValueError("v_scale rows must be contiguous")
    if k.shape != v.shape or k.stride() != v.stride():
        raise ValueError("k and v must share shape and strides")
    if k.dim() != 3 or k.shape[0] != plan.kv_heads or k.shape[2] != plan.head_dim or k.stride(2) != 1:
        raise ValueError(f"k/v must be [{plan.kv_heads}, slots, {plan.head_dim}] with contiguous rows")
    # the kernel reads slots below the ring size, or below the plan's extent
    # end (a per-call state never reads past it)
    need = plan.problem.ring_slots or plan.info["hi"]
    if k.shape[1] < need or (v_scale is not None and (v_scale.dim() != 2 or v_scale.shape[1] < need)):
        raise ValueError(f"k/v (and v_scale) must hold at least {need} slots")
    _require(workspace, "workspace", (torch.float32,))
    return (_ptr(q), _ptr(k), _ptr(v), _ptr(v_scale), v_scale.stride(0) if v_scale is not None else 0,
            k.stride(0), k.stride(1), _ptr(workspace), workspace.numel() * 4)


def verify_attn_split(plan, q, k, v, workspace, v_scale=None, stream=None):
    """Partial attention of every split (shapes as in _split_args)."""
    _check("verify_attn_split", _lib().verify_attn_split(
        ctypes.byref(plan.plan), *_split_args(plan, q, k, v, workspace, v_scale), _stream(stream)))


def _append_rows(plan, k_new, v_new):
    import torch
    for t, n in ((k_new, "k_new"), (v_new, "v_new")):
        _require(t, n, (torch.bfloat16,))
    shape = (plan.rows, plan.kv_heads, plan.head_dim)
    if not (k_new.is_contiguous() and v_new.is_contiguous()) or tuple(k_new.shape) != shape or \
            tuple(v_new.shape) != shape:
        raise ValueError(f"k_new/v_new must be contiguous {list(shape)} bfloat16")


def verify_attn_split_append(plan, q, k_new, v_new, k, v, workspace, stream=None):
    """verify_attn_split that also stores the rows' own K/V (k_new, v_new
    [rows, Hkv, D] bf16 contiguous) into the cache k, v in the same launch."""
    _append_rows(plan, k_new, v_new)
    first = plan.problem.prefix_len if plan.problem.mask == MASKS["tree"] else plan.problem.first_pos
    if not plan.problem.ring_slots and k.shape[1] < first + plan.rows:
        raise ValueError(f"k/v must hold the {plan.rows} rows' slots from {first}")
    qp, kp, vp, _, _, hs, rs, wp, wb = _split_args(plan, q, k, v, workspace, None)
    _check("verify_attn_split_append", _lib().verify_attn_split_append(
        ctypes.byref(plan.plan), qp, _ptr(k_new), _ptr(v_new), kp, vp, hs, rs, wp, wb, _stream(stream)))


def verify_attn_split_append_state(plan, state, q, k_new, v_new, k, v, workspace, stream=None):
    """verify_attn_split_append with positions, live rows and tree read on the
    device from `state`; a linear cache must hold kv_capacity slots."""
    _require_state(state)
    _append_rows(plan, k_new, v_new)
    if not plan.problem.ring_slots and k.shape[1] < plan.problem.kv_capacity:
        raise ValueError(f"k/v must hold the plan's {plan.problem.kv_capacity} slots")
    qp, kp, vp, _, _, hs, rs, wp, wb = _split_args(plan, q, k, v, workspace, None)
    _check("verify_attn_split_append_state", _lib().verify_attn_split_append_state(
        ctypes.byref(plan.plan), _ptr(state), qp, _ptr(k_new), _ptr(v_new), kp, vp, hs, rs, wp, wb,
        _stream(stream)))


def verify_attn_split_state(plan, state, q, k, v, workspace, v_scale=None, stream=None):
    """verify_attn_split with positions, live rows and tree read on the device
    from `state` (a device copy of pack_state(...)) when the kernel runs."""
    _require_state(state)
    _check("verify_attn_split_state", _lib().verify_attn_split_state(
        ctypes.byref(plan.plan), _ptr(state), *_split_args(plan, q, k, v, workspace, v_scale), _stream(stream)))


def _combine_args(plan, workspace, out, lse, sink):
    """out [rows, Hq, D] float32 contiguous; lse [rows, Hq] float32 or None;
    sink [Hq] float32 or None."""
    import torch
    _require(workspace, "workspace", (torch.float32,))
    _require(out, "out", (torch.float32,))
    if not out.is_contiguous() or tuple(out.shape) != (plan.rows, plan.q_heads, plan.head_dim):
        raise ValueError("out must be contiguous [rows, Hq, D] float32")
    if lse is not None:
        _require(lse, "lse", (torch.float32,))
        if not lse.is_contiguous() or tuple(lse.shape) != (plan.rows, plan.q_heads):
            raise ValueError("lse must be contiguous [rows, Hq] float32")
    if sink is not None:
        _require(sink, "sink", (torch.float32,))
        if not sink.is_contiguous() or sink.numel() != plan.q_heads:
            raise ValueError("sink must be contiguous [Hq] float32")
    return _ptr(workspace), workspace.numel() * 4, _ptr(sink), _ptr(out), _ptr(lse)


def verify_attn_combine(plan, workspace, out, lse=None, sink=None, stream=None):
    """Merge the splits' partials into out (and lse); shapes as in _combine_args."""
    _check("verify_attn_combine", _lib().verify_attn_combine(
        ctypes.byref(plan.plan), *_combine_args(plan, workspace, out, lse, sink), _stream(stream)))


def verify_attn_noalloc(plan, q, k, v, out, lse=None, sink=None, v_scale=None, stream=None):
    """verify_attn_split + verify_attn_combine with the library's static
    per-GPU workspace (no allocation anywhere in the call); shapes as in
    _split_args and _combine_args."""
    import torch
    empty = torch.empty(0, dtype=torch.float32, device=q.device)   # placeholder: no workspace is passed
    qp, kp, vp, vsp, vss, khs, krs, _, _ = _split_args(plan, q, k, v, empty, v_scale)
    _, _, sp, op, lp = _combine_args(plan, empty, out, lse, sink)
    _check("verify_attn_noalloc", _lib().verify_attn_noalloc(
        ctypes.byref(plan.plan), qp, kp, vp, vsp, vss, khs, krs, sp, op, lp, _stream(stream)))


NOALLOC_WORKSPACE_BYTES = 16 << 20


def verify_attn_combine_state(plan, state, workspace, out, lse=None, sink=None, stream=None):
    """verify_attn_combine for a verify_attn_split_state call with the same state."""
    _require_state(state)
    _check("verify_attn_combine_state", _lib().verify_attn_combine_state(
        ctypes.byref(plan.plan), _ptr(state), *_combine_args(plan, workspace, out, lse, sink), _stream(stream)))


def swa_ring_write(k_new, v_new, first_pos, k_ring, v_ring, stream=None):
    """k_new, v_new [rows, Hkv, D] bf16 contiguous; k_ring, v_ring [Hkv, C, D] bf16."""
    import torch
    for t, n in ((k_new, "k_new"), (v_new, "v_new"), (k_ring, "k_ring"), (v_ring, "v_ring")):
        _require(t, n, (torch.bfloat16,))
    if not (k_new.is_contiguous() and v_new.is_contiguous()) or k_new.shape != v_new.shape:
        raise ValueError("k_new/v_new must be contiguous [rows, Hkv, D]")
    if k_ring.shape != v_ring.shape or k_ring.stride() != v_ring.stride() or k_ring.stride(2) != 1:
        raise ValueError("k_ring/v_ring must share shape and strides, rows contiguous")
    rows, hkv, d = k_new.shape
    if k_ring.shape[0] != hkv or k_ring.shape[2] != d:
        raise ValueError("ring shape does not match the new rows")
    _check("swa_ring_write", _lib().swa_ring_write(
        _ptr(k_new), _ptr(v_new), rows, first_pos, hkv, d, _ptr(k_ring), _ptr(v_ring), k_ring.shape[1],
        k_ring.stride(0), k_ring.stride(1), _stream(stream)))


def verify_kv_write(k_new, v_new, first_pos, k_cache, v_cache, v_scale=None, ring_slots=0, stream=None):
    """k_new, v_new [rows, Hkv, D] bf16 contiguous.  k_cache, v_cache
    [Hkv, slots, D]: bf16 (copied), or uint8 keys / int8 values (encoded,
    with v_scale [Hkv, slots] float32).  ring_slots = 0 writes slot
    first_pos + r of a linear cache, else (first_pos + r) mod ring_slots."""
    import torch
    _require(k_new, "k_new", (torch.bfloat16,))
    _require(v_new, "v_new", (torch.bfloat16,))
    if not (k_new.is_contiguous() and v_new.is_contiguous()) or k_new.shape != v_new.shape or k_new.dim() != 3:
        raise ValueError("k_new/v_new must be contiguous [rows, Hkv, D]")
    if k_cache.dtype == torch.bfloat16:
        fmt = 0
        _require(v_cache, "v_cache", (torch.bfloat16,))
    else:
        fmt = 1
        _require(k_cache, "k_cache", (torch.uint8,))
        _require(v_cache, "v_cache", (torch.int8,))
        _require(v_scale, "v_scale", (torch.float32,))
        if v_scale.dim() != 2 or v_scale.stride(1) != 1 or v_scale.shape[1] < k_cache.shape[1]:
            raise ValueError("v_scale must be [Hkv, slots] with contiguous rows")
    if k_cache.shape != v_cache.shape or k_cache.stride() != v_cache.stride() or k_cache.dim() != 3 \
            or k_cache.stride(2) != 1:
        raise ValueError("k_cache/v_cache must share shape and strides, rows contiguous")
    rows, hkv, d = k_new.shape
    if k_cache.shape[0] != hkv or k_cache.shape[2] != d:
        raise ValueError("cache shape does not match the new rows")
    _check("verify_kv_write", _lib().verify_kv_write(
        _ptr(k_new), _ptr(v_new), rows, first_pos, hkv, d, fmt, _ptr(k_cache), _ptr(v_cache), _ptr(v_scale),
        v_scale.stride(0) if v_scale is not None else 0, k_cache.shape[1], ring_slots,
        k_cache.stride(0), k_cache.stride(1), _stream(stream)))


def verify_attn(plan, q, k, v, sink=None, v_scale=None, workspace=None, out=None, lse=None, stream=None,
                state=None):
    """Split then combine on one stream; allocates what is not passed in.
    With `state` (device int64 [11]) the state entry points run instead."""
    import torch
    dev = q.device
    if workspace is None:
        workspace = workspace_for(plan, dev)
    if out is None:
        out = torch.empty((plan.rows, plan.q_heads, plan.head_dim), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((plan.rows, plan.q_heads), dtype=torch.float32, device=dev)
    if state is None:
        verify_attn_split(plan, q, k, v, workspace, v_scale=v_scale, stream=stream)
        verify_attn_combine(plan, workspace, out, lse=lse, sink=sink, stream=stream)
    else:
        verify_attn_split_state(plan, state, q, k, v, workspace, v_scale=v_scale, stream=stream)
        verify_attn_combine_state(plan, state, workspace, out, lse=lse, sink=sink, stream=stream)
    return out, lse


# ----------------------------------------------------------------------------- sampling and acceptance

PURPOSE_TARGET, PURPOSE_ACCEPT, PURPOSE_RESIDUAL = 0, 1, 2


def sample_params(rows, vocab, top_k=20, top_p=0.95, temperature=1.0, seed=0, first_position=0, purpose=0,
                  row_stride=None):
    p = va_sample_params()
    p.rows, p.top_k, p.vocab = rows, top_k, vocab
    p.row_stride = vocab if row_stride is None else row_stride
    p.temperature, p.top_p, p.seed = temperature, top_p, seed
    p.first_position, p.purpose, p.reserved = first_position, purpose, 0
    return p


def sample_workspace_bytes(params):
    return _lib().va_sample_workspace_bytes(ctypes.byref(params))


def sample_workspace_for(params, device=None):
    """A zero-filled workspace (its counters must start at zero; every call
    leaves them zero, so it can be reused)."""
    import torch
    return torch.zeros((sample_workspace_bytes(params) + 7) // 8, dtype=torch.int64, device=device or "cuda")


def _sample_call_args(logits, top_k, top_p, temperature, seed, first_position, purpose, workspace, out):
    import torch
    _require(logits, "logits", (torch.float32,))
    if logits.dim() != 2 or logits.stride(1) != 1:
        raise ValueError("logits must be [rows, vocab] with contiguous rows")
    rows, vocab = logits.shape
    p = sample_params(rows, vocab, top_k, top_p, temperature, seed, first_position, purpose, logits.stride(0))
    need = sample_workspace_bytes(p)
    if need == 0:
        raise VAError("va_sample_workspace_bytes", 1)
    dev = logits.device
    if workspace is None:
        workspace = torch.zeros((need + 7) // 8, dtype=torch.int64, device=dev)
    if out is None:
        out = dict(ids=torch.empty((rows, top_k), dtype=torch.int32, device=dev),
                   probs=torch.empty((rows, top_k), dtype=torch.float32, device=dev),
                   kept=torch.empty(rows, dtype=torch.int32, device=dev),
                   tokens=torch.empty(rows, dtype=torch.int32, device=dev))
    return p, workspace, out


def va_sample(logits, top_k=20, top_p=0.95, temperature=1.0, seed=0, first_position=0, purpose=PURPOSE_TARGET,
              workspace=None, out=None, stream=None):
    """Top-k / top-p sampling of every row of FP32 logits [rows, vocab].
    Returns dict(ids [rows, top_k], probs [rows, top_k], kept [rows], tokens [rows])."""
    p, ws, out = _sample_call_args(logits, top_k, top_p, temperature, seed, first_position, purpose, workspace, out)
    _check("va_sample", _lib().va_sample(
        ctypes.byref(p), _ptr(logits), _ptr(out["ids"]), _ptr(out["probs"]), _ptr(out["kept"]), _ptr(out["tokens"]),
        _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))
    return out


def _q_args(q_ids, q_probs, q_kept, drafts):
    if q_ids is None:
        return None, None, None, 1, None
    if q_ids.dim() != 2 or not q_ids.is_contiguous() or q_probs.shape != q_ids.shape or not q_probs.is_contiguous():
        raise ValueError("q_ids / q_probs must be contiguous [n - 1, q_stride]")
    return _ptr(q_ids), _ptr(q_probs), _ptr(q_kept), q_ids.shape[1], _ptr(drafts)


def va_accept(p_ids, p_probs, p_kept, p_tokens, q_ids, q_probs, q_kept, drafts, seed, first_position,
              accepted=None, out_tokens=None, stream=None):
    """Rejection acceptance of n - 1 drafts against n target rows (int32 / FP32
    device tensors as va_sample writes them).  Returns (accepted [1], out_tokens [n])."""
    import torch
    n = p_ids.shape[0]
    dev = p_ids.device
    if accepted is None:
        accepted = torch.empty(1, dtype=torch.int32, device=dev)
    if out_tokens is None:
        out_tokens = torch.empty(n, dtype=torch.int32, device=dev)
    qi, qp, qk, qs, dr = _q_args(q_ids, q_probs, q_kept, drafts)
    _check("va_accept", _lib().va_accept(
        _ptr(p_ids), _ptr(p_probs), _ptr(p_kept), _ptr(p_tokens), p_ids.shape[1], qi, qp, qk, qs, dr, n,
        seed, first_position, _ptr(accepted), _ptr(out_tokens), _stream(stream)))
    return accepted, out_tokens


def va_sample_accept(logits, q_ids, q_probs, q_kept, drafts, top_k=20, top_p=0.95, temperature=1.0, seed=0,
                     first_position=0, purpose=PURPOSE_TARGET, workspace=None, out=None, accepted=None,
                     out_tokens=None, stream=None):
    """va_sample of the n verification rows and the acceptance in one launch (the
    last row's merging workgroup runs the acceptance).
    Returns (dict as va_sample, accepted [1], out_tokens [n])."""
    import torch
    p, ws, out = _sample_call_args(logits, top_k, top_p, temperature, seed, first_position, purpose, workspace, out)
    dev = logits.device
    if accepted is None:
        accepted = torch.empty(1, dtype=torch.int32, device=dev)
    if out_tokens is None:
        out_tokens = torch.empty(p.rows, dtype=torch.int32, device=dev)
    qi, qp, qk, qs, dr = _q_args(q_ids, q_probs, q_kept, drafts)
    _check("va_sample_accept", _lib().va_sample_accept(
        ctypes.byref(p), _ptr(logits), qi, qp, qk, qs, dr, _ptr(out["ids"]), _ptr(out["probs"]), _ptr(out["kept"]),
        _ptr(out["tokens"]), _ptr(accepted), _ptr(out_tokens), _ptr(ws), ws.numel() * ws.element_size(),
        _stream(stream)))
    return out, accepted, out_tokens


def va_read_probe(src, nbytes, sink, stream=None):
    """Stream nbytes of the device tensor src (measurement only)."""
    if nbytes > src.numel() * src.element_size():
        raise ValueError("nbytes exceeds the tensor")
    _check("va_read_probe", _lib().va_read_probe(_ptr(src), nbytes, _ptr(sink), _stream(stream)))
