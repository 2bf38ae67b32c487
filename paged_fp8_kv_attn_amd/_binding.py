"""ctypes binding of libpagedattn.so: argument marshalling only.

Tensors are torch tensors on the GPU; the binding passes their data pointers
and the current HIP stream to the C ABI, which does all of the work.
"""

from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libpagedattn.so"

ATTN_DTYPE_F32 = 0
ATTN_DTYPE_BF16 = 1
_DTYPES = {torch.float32: ATTN_DTYPE_F32, torch.bfloat16: ATTN_DTYPE_BF16}

# names declared in include/pagedattn.h
_FUNCTIONS = [
    "attn_plan_create",
    "attn_paged_forward",
    "attn_plan_destroy",
    "attn_plan_get_info",
    "attn_plan_set_kernel_events",
    "attn_status_string",
    "attn_last_hip_error",
    "attn_debug_gather",
    "attn_debug_decode_fp8",
    "attn_debug_decode_int8",
    "attn_kv_append",
    "attn_debug_encode_fp8",
    "attn_mtp_accept_workspace_size",
    "attn_mtp_accept",
]


class AttnError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        text = status_string(status)
        if status == 4:
            text += f" (hipError {load_library().attn_last_hip_error()})"
        super().__init__(f"{what}: {text}")


class PlanDesc(ctypes.Structure):
    _fields_ = [
        ("num_seqs", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("num_pages", ctypes.c_int32),
        ("max_pages_per_seq", ctypes.c_int32),
        ("max_q_len", ctypes.c_int32),
        ("max_ctx_len", ctypes.c_int32),
        ("q_dtype", ctypes.c_int32),
        ("out_dtype", ctypes.c_int32),
        ("sm_scale", ctypes.c_float),
        ("num_kv_splits", ctypes.c_int32),
        ("kv_format", ctypes.c_int32),
        ("reserved", ctypes.c_int32 * 3),
    ]


class PlanInfo(ctypes.Structure):
    _fields_ = [
        ("col_tiles", ctypes.c_int32),
        ("dup_lo_columns", ctypes.c_int32),
        ("cols_per_block", ctypes.c_int32),
        ("col_blocks", ctypes.c_int32),
        ("waves_per_group", ctypes.c_int32),
        ("num_segments", ctypes.c_int32),
        ("grid_size", ctypes.c_int32),
        ("merge_grid_size", ctypes.c_int32),
        ("work_units", ctypes.c_int32),
        ("packed", ctypes.c_int32),
        ("shared_kv", ctypes.c_int32),
        ("resident_groups_per_cu", ctypes.c_int32),
        ("compute_units", ctypes.c_int32),
        ("workspace_bytes", ctypes.c_size_t),
    ]

    def as_dict(self):
        return {name: getattr(self, name) for name, _ in self._fields_}


_lib = None


def library_path() -> str:
    return os.path.join(_HERE, _LIB_NAME)


def load_library():
    """Load the in-tree HIP library; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m paged_fp8_kv_attn_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    lib.attn_plan_create.argtypes = [ctypes.POINTER(PlanDesc), ctypes.POINTER(vp)]
    lib.attn_plan_create.restype = i32
    lib.attn_paged_forward.argtypes = [vp] * 10
    lib.attn_paged_forward.restype = i32
    lib.attn_plan_destroy.argtypes = [vp]
    lib.attn_plan_destroy.restype = i32
    lib.attn_plan_get_info.argtypes = [vp, ctypes.POINTER(PlanInfo)]
    lib.attn_plan_get_info.restype = i32
    lib.attn_plan_set_kernel_events.argtypes = [vp, vp, vp]
    lib.attn_plan_set_kernel_events.restype = i32
    lib.attn_status_string.argtypes = [i32]
    lib.attn_status_string.restype = ctypes.c_char_p
    lib.attn_last_hip_error.argtypes = []
    lib.attn_last_hip_error.restype = ctypes.c_int
    lib.attn_debug_gather.argtypes = [vp] * 11
    lib.attn_debug_gather.restype = i32
    lib.attn_debug_decode_fp8.argtypes = [vp, vp, i64, vp]
    lib.attn_debug_decode_fp8.restype = i32
    lib.attn_debug_decode_int8.argtypes = [vp, vp, i64, vp]
    lib.attn_debug_decode_int8.restype = i32
    lib.attn_kv_append.argtypes = [vp, vp, vp, i32] + [vp] * 7
    lib.attn_kv_append.restype = i32
    lib.attn_debug_encode_fp8.argtypes = [vp, vp, i64, vp]
    lib.attn_debug_encode_fp8.restype = i32
    lib.attn_mtp_accept_workspace_size.argtypes = [i32, i32, i32]
    lib.attn_mtp_accept_workspace_size.restype = ctypes.c_size_t
    lib.attn_mtp_accept.argtypes = [vp, i32, vp, i32, i32, i32, vp, vp, vp, ctypes.c_size_t, vp, vp, vp]
    lib.attn_mtp_accept.restype = i32
    _lib = lib
    return lib


def exported_symbols() -> dict:
    lib = load_library()
    return {name: hasattr(lib, name) for name in _FUNCTIONS}


def status_string(status: int) -> str:
    return load_library().attn_status_string(int(status)).decode()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(status: int, what: str):
    if status != 0:
        raise AttnError(status, what)


def _dtype_code(dt) -> int:
    if isinstance(dt, int):
        return dt
    if isinstance(dt, str):
        return {"f32": ATTN_DTYPE_F32, "bf16": ATTN_DTYPE_BF16}[dt]
    return _DTYPES[dt]


class Plan:
    """A plan: static shape, chosen tiling, and its one-time workspace."""

    def __init__(self, *, num_seqs, num_q_heads, num_kv_heads, head_dim, num_pages, max_pages_per_seq,
                 max_q_len, max_ctx_len, q_dtype="bf16", out_dtype="bf16", sm_scale=0.0, num_kv_splits=0,
                 page_size=16, kv_format="e4m3", reserved=(0, 0, 0)):
        lib = load_library()
        d = PlanDesc()
        d.num_seqs = num_seqs
        d.num_q_heads = num_q_heads
        d.num_kv_heads = num_kv_heads
        d.head_dim = head_dim
        d.page_size = page_size
        d.num_pages = num_pages
        d.max_pages_per_seq = max_pages_per_seq
        d.max_q_len = max_q_len
        d.max_ctx_len = max_ctx_len
        d.q_dtype = _dtype_code(q_dtype)
        d.out_dtype = _dtype_code(out_dtype)
        d.sm_scale = float(sm_scale)
        d.num_kv_splits = num_kv_splits
        d.kv_format = {"e4m3": 0, "int8": 1}.get(kv_format, kv_format) if isinstance(kv_format, str) else kv_format
        for i, r in enumerate(reserved):
            d.reserved[i] = r
        self.desc = d
        self._h = ctypes.c_void_p()
        _check(lib.attn_plan_create(ctypes.byref(d), ctypes.byref(self._h)), "attn_plan_create")

    @property
    def handle(self):
        return self._h

    def info(self) -> dict:
        inf = PlanInfo()
        _check(load_library().attn_plan_get_info(self._h, ctypes.byref(inf)), "attn_plan_get_info")
        return inf.as_dict()

    def set_kernel_events(self, start=None, stop=None):
        """Record events `start`/`stop` (raw hipEvent_t handles as ints or
        c_void_p, or objects with a `cuda_event` handle) around the attention
        kernel of every later forward (None, None: stop recording)."""
        def ev(e):
            if e is None:
                return None
            if isinstance(e, ctypes.c_void_p):
                return e
            if isinstance(e, int):
                return ctypes.c_void_p(e)
            return ctypes.c_void_p(e.cuda_event)
        _check(load_library().attn_plan_set_kernel_events(self._h, ev(start), ev(stop)),
               "attn_plan_set_kernel_events")

    def forward(self, q, k_pages, v_pages, kv_scales, block_table, ctx_lens, q_lens, out, stream=None):
        st = load_library().attn_paged_forward(
            self._h, _ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(kv_scales), _ptr(block_table),
            _ptr(ctx_lens), _ptr(q_lens), _ptr(out), _stream(stream))
        _check(st, "attn_paged_forward")
        return out

    def kv_append(self, k_new, v_new, k_pages, v_pages, kv_scales, block_table, ctx_lens, q_lens, stream=None):
        """Quantise the new rows k_new/v_new ([sum Q][Hkv][D], bf16 or fp32)
        into the pools in place (attn_kv_append)."""
        if k_new.dtype != v_new.dtype:
            raise ValueError("k_new and v_new must have the same dtype")
        st = load_library().attn_kv_append(
            self._h, _ptr(k_new), _ptr(v_new), _dtype_code(k_new.dtype), _ptr(k_pages), _ptr(v_pages),
            _ptr(kv_scales), _ptr(block_table), _ptr(ctx_lens), _ptr(q_lens), _stream(stream))
        _check(st, "attn_kv_append")

    def close(self):
        if self._h:
            _check(load_library().attn_plan_destroy(self._h), "attn_plan_destroy")
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def debug_gather(plan: Plan, k_pages, v_pages, kv_scales, block_table, ctx_lens, k_out, v_out, scale_out,
                 page_out, stream=None):
    st = load_library().attn_debug_gather(plan.handle, _ptr(k_pages), _ptr(v_pages), _ptr(kv_scales),
                                          _ptr(block_table), _ptr(ctx_lens), _ptr(k_out), _ptr(v_out),
                                          _ptr(scale_out), _ptr(page_out), _stream(stream))
    _check(st, "attn_debug_gather")


def debug_decode_fp8(codes, out, stream=None):
    st = load_library().attn_debug_decode_fp8(_ptr(codes), _ptr(out), int(codes.numel()), _stream(stream))
    _check(st, "attn_debug_decode_fp8")
    return out


def debug_decode_int8(codes, out, stream=None):
    st = load_library().attn_debug_decode_int8(_ptr(codes), _ptr(out), int(codes.numel()), _stream(stream))
    _check(st, "attn_debug_decode_int8")
    return out


def debug_encode_fp8(values, out, stream=None):
    st = load_library().attn_debug_encode_fp8(_ptr(values), _ptr(out), int(values.numel()), _stream(stream))
    _check(st, "attn_debug_encode_fp8")
    return out


def mtp_accept_workspace_size(num_seqs: int, num_drafts: int, vocab: int) -> int:
    return int(load_library().attn_mtp_accept_workspace_size(num_seqs, num_drafts, vocab))


def mtp_accept(logits, drafts, target_tokens, num_accepted, workspace, kernel_events=None, stream=None):
    """Greedy acceptance (attn_mtp_accept): logits [B][K+1][V] bf16/fp32,
    drafts int32 [B][K]; fills target_tokens int32 [B][K+1] and
    num_accepted int32 [B].  workspace: a uint8 device tensor of at least
    mtp_accept_workspace_size(B, K, V) bytes."""
    B, K1, V = logits.shape
    ev = (None, None) if kernel_events is None else tuple(ctypes.c_void_p(e) if isinstance(e, int) else e
                                                        for e in kernel_events)
    st = load_library().attn_mtp_accept(
        _ptr(logits), _dtype_code(logits.dtype), _ptr(drafts), B, K1 - 1, V, _ptr(target_tokens),
        _ptr(num_accepted), _ptr(workspace), workspace.numel() * workspace.element_size(), ev[0], ev[1],
        _stream(stream))
    _check(st, "attn_mtp_accept")
