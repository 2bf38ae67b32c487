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
TIMELINE_WORDS = 64  # words per wave in a timeline row (ATTN_TIMELINE_WORDS)

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
    "attn_plan_set_merge_events",
    "attn_plan_set_timeline",
    "attn_status_string",
    "attn_last_hip_error",
    "attn_debug_gather",
    "attn_debug_decode_fp8",
    "attn_debug_decode_int8",
    "attn_debug_decode_int4",
    "attn_kv_append",
    "attn_debug_encode_fp8",
    "attn_mtp_accept_workspace_size",
    "attn_mtp_accept",
    "attn_calib_stream_read",
    "attn_paged_forward_static",
    "attn_static_scratch_bytes",
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
        ("kv_piece_len", ctypes.c_int32),
        ("reserved", ctypes.c_int32 * 2),
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
        ("wallclock_khz", ctypes.c_int32),
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
    lib.attn_plan_set_merge_events.argtypes = [vp, vp, vp]
    lib.attn_plan_set_merge_events.restype = i32
    lib.attn_plan_set_timeline.argtypes = [vp, vp, ctypes.c_size_t]
    lib.attn_plan_set_timeline.restype = i32
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
    lib.attn_debug_decode_int4.argtypes = [vp, vp, i64, vp]
    lib.attn_debug_decode_int4.restype = i32
    lib.attn_kv_append.argtypes = [vp, vp, vp, i32] + [vp] * 7
    lib.attn_kv_append.restype = i32
    lib.attn_debug_encode_fp8.argtypes = [vp, vp, i64, vp]
    lib.attn_debug_encode_fp8.restype = i32
    lib.attn_mtp_accept_workspace_size.argtypes = [i32, i32, i32]
    lib.attn_mtp_accept_workspace_size.restype = ctypes.c_size_t
    lib.attn_mtp_accept.argtypes = [vp, i32, vp, i32, i32, i32, vp, vp, vp, ctypes.c_size_t, vp, vp, vp]
    lib.attn_mtp_accept.restype = i32
    lib.attn_calib_stream_read.argtypes = [vp, i64, vp, i64, i32, i32, i32, vp, vp, vp, vp]
    lib.attn_calib_stream_read.restype = i32
    lib.attn_paged_forward_static.argtypes = [ctypes.POINTER(PlanDesc)] + [vp] * 9
    lib.attn_paged_forward_static.restype = i32
    lib.attn_static_scratch_bytes.argtypes = []
    lib.attn_static_scratch_bytes.restype = ctypes.c_size_t
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


def _event(e):
    """A hipEvent_t handle from None, an int, a c_void_p or an object with a
    `cuda_event` handle."""
    if e is None:
        return None
    if isinstance(e, ctypes.c_void_p):
        return e
    if isinstance(e, int):
        return ctypes.c_void_p(e)
    return ctypes.c_void_p(e.cuda_event)


def _check(status: int, what: str):
    if status != 0:
        raise AttnError(status, what)


def _dtype_code(dt) -> int:
    if isinstance(dt, int):
        return dt
    if isinstance(dt, str):
        return {"f32": ATTN_DTYPE_F32, "bf16": ATTN_DTYPE_BF16}[dt]
    return _DTYPES[dt]


_TORCH_OF = {ATTN_DTYPE_F32: torch.float32, ATTN_DTYPE_BF16: torch.bfloat16}
KV_FORMATS = {"e4m3": 0, "int8": 1, "int4": 2}


def _chunk_bytes(desc) -> int:
    """Bytes of one (page, kv head) chunk of a pool: 16 slots x D codes, two
    codes per byte for INT4."""
    return desc.page_size * desc.head_dim // (2 if desc.kv_format == 2 else 1)


def _want(t, name: str, device, dtypes, min_numel: int = 0, numel: int | None = None):
    """Raise ValueError unless tensor t is contiguous, on `device` (a
    torch.device; None: any GPU device), of one of `dtypes`, with at least
    min_numel (or exactly numel) elements.  Runs before any library call, so
    a bad tensor never reaches a kernel as a device pointer."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name}: expected a torch tensor, got {type(t).__name__}")
    if device is None:
        if t.device.type != "cuda":
            raise ValueError(f"{name}: expected a GPU tensor, got one on {t.device}")
    elif t.device != device:
        raise ValueError(f"{name}: expected a tensor on {device}, got one on {t.device}")
    if t.dtype not in dtypes:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {' or '.join(str(d) for d in dtypes)}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name}: {t.numel()} elements, expected {numel}")
    if t.numel() < min_numel:
        raise ValueError(f"{name}: {t.numel()} elements, expected at least {min_numel}")


def check_forward_tensors(desc: "PlanDesc", device, q, k_pages, v_pages, kv_scales, block_table, ctx_lens,
                          q_lens, out):
    """The checks Plan.forward makes before calling attn_paged_forward:
    device, dtype against the descriptor, contiguity and element counts
    (pools of P pages, scales [2][P][Hkv], a [B][max_pages_per_seq] block
    table, B lengths, q and out of equal row counts between B and
    B * max_q_len rows of Hq x D).  The sum of q_lens is device data and
    stays a precondition: it must not exceed q's rows."""
    d = desc
    row = d.num_q_heads * d.head_dim
    chunk = d.num_pages * d.num_kv_heads * _chunk_bytes(d)
    _want(q, "q", device, (_TORCH_OF[d.q_dtype],), min_numel=d.num_seqs * row)
    if q.numel() % row or q.numel() > d.num_seqs * d.max_q_len * row:
        raise ValueError(f"q: {q.numel()} elements is not a whole number of rows of Hq x D = {row} "
                         f"up to num_seqs * max_q_len = {d.num_seqs * d.max_q_len} rows")
    _want(k_pages, "k_pages", device, (torch.uint8,), min_numel=chunk)
    _want(v_pages, "v_pages", device, (torch.uint8,), min_numel=chunk)
    _want(kv_scales, "kv_scales", device, (torch.float32,), min_numel=2 * d.num_pages * d.num_kv_heads)
    _want(block_table, "block_table", device, (torch.int32,), min_numel=d.num_seqs * d.max_pages_per_seq)
    _want(ctx_lens, "ctx_lens", device, (torch.int32,), min_numel=d.num_seqs)
    _want(q_lens, "q_lens", device, (torch.int32,), min_numel=d.num_seqs)
    _want(out, "out", device, (_TORCH_OF[d.out_dtype],), numel=q.numel() // row * d.num_q_heads * d.head_dim)


def check_append_tensors(desc: "PlanDesc", device, k_new, v_new, k_pages, v_pages, kv_scales, block_table,
                         ctx_lens, q_lens):
    """The checks Plan.kv_append makes before calling attn_kv_append."""
    d = desc
    row = d.num_kv_heads * d.head_dim
    chunk = d.num_pages * d.num_kv_heads * _chunk_bytes(d)
    _want(k_new, "k_new", device, (torch.bfloat16, torch.float32), min_numel=d.num_seqs * row)
    _want(v_new, "v_new", device, (k_new.dtype,), numel=k_new.numel())
    if k_new.numel() % row or k_new.numel() > d.num_seqs * d.max_q_len * row:
        raise ValueError(f"k_new: {k_new.numel()} elements is not a whole number of rows of Hkv x D = {row} "
                         f"up to num_seqs * max_q_len = {d.num_seqs * d.max_q_len} rows")
    _want(k_pages, "k_pages", device, (torch.uint8,), min_numel=chunk)
    _want(v_pages, "v_pages", device, (torch.uint8,), min_numel=chunk)
    _want(kv_scales, "kv_scales", device, (torch.float32,), min_numel=2 * d.num_pages * d.num_kv_heads)
    _want(block_table, "block_table", device, (torch.int32,), min_numel=d.num_seqs * d.max_pages_per_seq)
    _want(ctx_lens, "ctx_lens", device, (torch.int32,), min_numel=d.num_seqs)
    _want(q_lens, "q_lens", device, (torch.int32,), min_numel=d.num_seqs)


def make_desc(*, num_seqs, num_q_heads, num_kv_heads, head_dim, num_pages, max_pages_per_seq, max_q_len,
              max_ctx_len, q_dtype="bf16", out_dtype="bf16", sm_scale=0.0, num_kv_splits=0, page_size=16,
              kv_format="e4m3", kv_piece_len=0, reserved=(0, 0)) -> PlanDesc:
    """A filled attn_plan_desc_t."""
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
    d.kv_format = KV_FORMATS.get(kv_format, kv_format) if isinstance(kv_format, str) else kv_format
    d.kv_piece_len = kv_piece_len
    for i, r in enumerate(reserved):
        d.reserved[i] = r
    return d


def forward_static(desc: PlanDesc, q, k_pages, v_pages, kv_scales, block_table, ctx_lens, q_lens, out,
                   stream=None):
    """attn_paged_forward_static: the forward of a plan for `desc`, with the
    split partials in the library's per-GPU scratch array (no allocation)."""
    _want(q, "q", None, (torch.bfloat16, torch.float32))
    check_forward_tensors(desc, q.device, q, k_pages, v_pages, kv_scales, block_table, ctx_lens, q_lens, out)
    st = load_library().attn_paged_forward_static(
        ctypes.byref(desc), _ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(kv_scales), _ptr(block_table),
        _ptr(ctx_lens), _ptr(q_lens), _ptr(out), _stream(stream))
    _check(st, "attn_paged_forward_static")
    return out


def static_scratch_bytes() -> int:
    return int(load_library().attn_static_scratch_bytes())


class Plan:
    """A plan: static shape, chosen tiling, and its one-time workspace."""

    def __init__(self, *, num_seqs, num_q_heads, num_kv_heads, head_dim, num_pages, max_pages_per_seq,
                 max_q_len, max_ctx_len, q_dtype="bf16", out_dtype="bf16", sm_scale=0.0, num_kv_splits=0,
                 page_size=16, kv_format="e4m3", kv_piece_len=0, reserved=(0, 0)):
        lib = load_library()
        d = make_desc(num_seqs=num_seqs, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads, head_dim=head_dim,
                      num_pages=num_pages, max_pages_per_seq=max_pages_per_seq, max_q_len=max_q_len,
                      max_ctx_len=max_ctx_len, q_dtype=q_dtype, out_dtype=out_dtype, sm_scale=sm_scale,
                      num_kv_splits=num_kv_splits, page_size=page_size, kv_format=kv_format,
                      kv_piece_len=kv_piece_len, reserved=reserved)
        self.desc = d
        self._h = ctypes.c_void_p()
        _check(lib.attn_plan_create(ctypes.byref(d), ctypes.byref(self._h)), "attn_plan_create")
        # the library created the plan on the current HIP device
        self.device = torch.device("cuda", torch.cuda.current_device())

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
        _check(load_library().attn_plan_set_kernel_events(self._h, _event(start), _event(stop)),
               "attn_plan_set_kernel_events")

    def set_merge_events(self, start=None, stop=None):
        """As set_kernel_events, for the merge kernel that follows a split
        forward (a forward without a merge records both at one point)."""
        _check(load_library().attn_plan_set_merge_events(self._h, _event(start), _event(stop)),
               "attn_plan_set_merge_events")

    def set_timeline(self, rows=None):
        """Have every later forward record its attention kernel's per-wave
        timeline into `rows`, an int64 tensor on the plan's device with at
        least grid_size * waves_per_group rows of TIMELINE_WORDS words
        (zeroed by the caller before each forward); None stops recording."""
        if rows is None:
            _check(load_library().attn_plan_set_timeline(self._h, None, 0), "attn_plan_set_timeline")
            self._timeline = None
            return
        inf = self.info()
        need = inf["grid_size"] * inf["waves_per_group"]
        _want(rows, "timeline rows", self.device, (torch.int64,), min_numel=need * TIMELINE_WORDS)
        _check(load_library().attn_plan_set_timeline(self._h, _ptr(rows), rows.numel() // TIMELINE_WORDS),
               "attn_plan_set_timeline")
        self._timeline = rows  # kept alive while the library holds its address

    def forward(self, q, k_pages, v_pages, kv_scales, block_table, ctx_lens, q_lens, out, stream=None):
        check_forward_tensors(self.desc, self.device, q, k_pages, v_pages, kv_scales, block_table, ctx_lens,
                              q_lens, out)
        st = load_library().attn_paged_forward(
            self._h, _ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(kv_scales), _ptr(block_table),
            _ptr(ctx_lens), _ptr(q_lens), _ptr(out), _stream(stream))
        _check(st, "attn_paged_forward")
        return out

    def kv_append(self, k_new, v_new, k_pages, v_pages, kv_scales, block_table, ctx_lens, q_lens, stream=None):
        """Quantise the new rows k_new/v_new ([sum Q][Hkv][D], bf16 or fp32)
        into the pools in place (attn_kv_append)."""
        check_append_tensors(self.desc, self.device, k_new, v_new, k_pages, v_pages, kv_scales, block_table,
                             ctx_lens, q_lens)
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
    d, dev = plan.desc, plan.device
    chunk = d.num_pages * d.num_kv_heads * _chunk_bytes(d)
    per_tok = d.num_seqs * d.num_kv_heads * d.max_ctx_len
    _want(k_pages, "k_pages", dev, (torch.uint8,), min_numel=chunk)
    _want(v_pages, "v_pages", dev, (torch.uint8,), min_numel=chunk)
    _want(kv_scales, "kv_scales", dev, (torch.float32,), min_numel=2 * d.num_pages * d.num_kv_heads)
    _want(block_table, "block_table", dev, (torch.int32,), min_numel=d.num_seqs * d.max_pages_per_seq)
    _want(ctx_lens, "ctx_lens", dev, (torch.int32,), min_numel=d.num_seqs)
    _want(k_out, "k_out", dev, (torch.uint8,), numel=per_tok * d.head_dim)
    _want(v_out, "v_out", dev, (torch.uint8,), numel=per_tok * d.head_dim)
    _want(scale_out, "scale_out", dev, (torch.float32,), numel=2 * per_tok)
    _want(page_out, "page_out", dev, (torch.int32,), numel=d.num_seqs * d.max_ctx_len)
    st = load_library().attn_debug_gather(plan.handle, _ptr(k_pages), _ptr(v_pages), _ptr(kv_scales),
                                          _ptr(block_table), _ptr(ctx_lens), _ptr(k_out), _ptr(v_out),
                                          _ptr(scale_out), _ptr(page_out), _stream(stream))
    _check(st, "attn_debug_gather")


def _check_codec(src, src_dtypes, out, out_dtypes):
    _want(src, "input", None, src_dtypes)
    _want(out, "out", src.device, out_dtypes, min_numel=src.numel())


def debug_decode_fp8(codes, out, stream=None):
    _check_codec(codes, (torch.uint8,), out, (torch.float32,))
    st = load_library().attn_debug_decode_fp8(_ptr(codes), _ptr(out), int(codes.numel()), _stream(stream))
    _check(st, "attn_debug_decode_fp8")
    return out


def debug_decode_int8(codes, out, stream=None):
    _check_codec(codes, (torch.uint8, torch.int8), out, (torch.float32,))
    st = load_library().attn_debug_decode_int8(_ptr(codes), _ptr(out), int(codes.numel()), _stream(stream))
    _check(st, "attn_debug_decode_int8")
    return out


def debug_decode_int4(codes, out, stream=None):
    """Two INT4 codes per byte of `codes` (low nibble first) -> 2n floats as
    the attention kernels widen them (attn_debug_decode_int4)."""
    _want(codes, "input", None, (torch.uint8,))
    _want(out, "out", codes.device, (torch.float32,), min_numel=2 * codes.numel())
    st = load_library().attn_debug_decode_int4(_ptr(codes), _ptr(out), int(codes.numel()), _stream(stream))
    _check(st, "attn_debug_decode_int4")
    return out


def debug_encode_fp8(values, out, stream=None):
    _check_codec(values, (torch.float32,), out, (torch.uint8,))
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
    _want(logits, "logits", None, (torch.bfloat16, torch.float32))
    if logits.dim() != 3:
        raise ValueError(f"logits: expected [B][K+1][vocab], got shape {tuple(logits.shape)}")
    B, K1, V = logits.shape
    dev = logits.device
    _want(drafts, "drafts", dev, (torch.int32,), numel=B * (K1 - 1))
    _want(target_tokens, "target_tokens", dev, (torch.int32,), numel=B * K1)
    _want(num_accepted, "num_accepted", dev, (torch.int32,), numel=B)
    _want(workspace, "workspace", dev, (torch.uint8,), min_numel=mtp_accept_workspace_size(B, K1 - 1, V))
    ev = (None, None) if kernel_events is None else tuple(ctypes.c_void_p(e) if isinstance(e, int) else e
                                                        for e in kernel_events)
    st = load_library().attn_mtp_accept(
        _ptr(logits), _dtype_code(logits.dtype), _ptr(drafts), B, K1 - 1, V, _ptr(target_tokens),
        _ptr(num_accepted), _ptr(workspace), workspace.numel() * workspace.element_size(), ev[0], ev[1],
        _stream(stream))
    _check(st, "attn_mtp_accept")


def calib_stream_read(pool, chunk_ids, chunk_bytes: int, waves: int, sink, kernel_events=None, stream=None,
                      access: int = 0):
    """Streaming-read calibration (attn_calib_stream_read): `waves` waves read
    the chunks chunk_ids (int32 device tensor) of chunk_bytes each from pool
    (uint8 device tensor) and write one XOR word per lane into sink (int32 or
    uint32 device tensor of at least waves * 64 elements)."""
    _want(pool, "pool", None, (torch.uint8,), min_numel=int(chunk_bytes))
    _want(chunk_ids, "chunk_ids", pool.device, (torch.int32,), min_numel=1)
    _want(sink, "sink", pool.device, (torch.int32,), min_numel=int(waves) * 64)
    ev = (None, None) if kernel_events is None else tuple(ctypes.c_void_p(e) if isinstance(e, int) else e
                                                        for e in kernel_events)
    st = load_library().attn_calib_stream_read(
        _ptr(pool), pool.numel() * pool.element_size(), _ptr(chunk_ids), int(chunk_ids.numel()), int(chunk_bytes),
        int(waves), int(access), _ptr(sink), ev[0], ev[1], _stream(stream))
    _check(st, "attn_calib_stream_read")
