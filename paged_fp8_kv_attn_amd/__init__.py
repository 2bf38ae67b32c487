"""MI355X (gfx950) paged FP8-KV attention.

The compute runs in the HIP library libpagedattn.so (C ABI in
include/pagedattn.h); this package only loads it and marshals arguments.
There is no CPU fallback: without the built library every call raises.
"""

from ._binding import (  # noqa: F401
    TIMELINE_WORDS,
    AttnError,
    Plan,
    PlanInfo,
    calib_stream_read,
    debug_decode_fp8,
    debug_decode_int4,
    debug_decode_int8,
    debug_encode_fp8,
    debug_gather,
    exported_symbols,
    forward_static,
    library_path,
    load_library,
    make_desc,
    mtp_accept,
    mtp_accept_workspace_size,
    static_scratch_bytes,
    status_string,
)
