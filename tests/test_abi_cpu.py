"""The C ABI without a GPU: the library loads, exports every function the
header declares, names every status, and rejects bad descriptors and
arguments before touching the device."""

import os
import re

import pytest

import paged_fp8_kv_attn_amd as pa
from paged_fp8_kv_attn_amd import _binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pagedattn.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = pa.load_library()
    names = _declared()
    assert names, "header declares nothing?"
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing
    assert set(names) == set(_binding._FUNCTIONS)


def test_status_strings():
    for code, prefix in [(0, "ATTN_OK"), (1, "ATTN_ERR_INVALID_ARGUMENT"), (2, "ATTN_ERR_UNSUPPORTED"),
                         (3, "ATTN_ERR_OUT_OF_MEMORY"), (4, "ATTN_ERR_HIP")]:
        assert pa.status_string(code).startswith(prefix)
    assert "unknown" in pa.status_string(99)


GOOD = dict(num_seqs=2, num_q_heads=8, num_kv_heads=2, head_dim=128, num_pages=10, max_pages_per_seq=4,
            max_q_len=1, max_ctx_len=64)


@pytest.mark.parametrize("change,status", [
    (dict(num_q_heads=6, num_kv_heads=4), 1),
    (dict(num_seqs=0), 1),
    (dict(num_kv_heads=0), 1),
    (dict(max_q_len=0), 1),
    (dict(max_ctx_len=0), 1),
    (dict(max_q_len=8, max_ctx_len=4), 1),
    (dict(max_pages_per_seq=3), 1),
    (dict(num_pages=0), 1),
    (dict(num_kv_splits=-1), 1),
    (dict(sm_scale=float("nan")), 1),
    (dict(sm_scale=-1.0), 1),
    (dict(q_dtype=7), 1),
    (dict(reserved=(0, 1)), 1),
    (dict(kv_piece_len=-32), 1),
    (dict(kv_piece_len=48), 1),
    (dict(kv_piece_len=96), 1),
    (dict(kv_piece_len=512, num_kv_splits=2), 1),
    (dict(kv_format=3), 1),
    (dict(kv_format="int4", head_dim=64), 2),
    (dict(kv_format="int4", q_dtype="f32"), 2),
    (dict(kv_format="int8", q_dtype="f32"), 2),
    (dict(kv_format="int8", out_dtype="f32"), 2),
    (dict(head_dim=96), 2),
    (dict(head_dim=256), 2),
    (dict(page_size=32, max_pages_per_seq=2), 2),
])
def test_bad_descriptor_rejected_before_device_work(change, status):
    kw = dict(GOOD)
    kw.update(change)
    with pytest.raises(pa.AttnError) as e:
        pa.Plan(**kw)
    assert e.value.status == status


def test_null_arguments_rejected():
    lib = pa.load_library()
    assert lib.attn_plan_create(None, None) == 1
    assert lib.attn_paged_forward(*([None] * 10)) == 1
    assert lib.attn_plan_get_info(None, None) == 1
    assert lib.attn_debug_gather(*([None] * 11)) == 1
    assert lib.attn_plan_destroy(None) == 0
    assert lib.attn_debug_decode_fp8(None, None, -1, None) == 1
    assert lib.attn_debug_decode_fp8(None, None, 0, None) == 0
    assert lib.attn_debug_decode_fp8(None, None, 5, None) == 1
    assert lib.attn_debug_decode_int8(None, None, -1, None) == 1
    assert lib.attn_debug_decode_int8(None, None, 0, None) == 0
    assert lib.attn_debug_decode_int8(None, None, 5, None) == 1
    assert lib.attn_kv_append(None, None, None, 1, *([None] * 7)) == 1
    assert lib.attn_debug_encode_fp8(None, None, -1, None) == 1
    assert lib.attn_debug_encode_fp8(None, None, 0, None) == 0
    assert lib.attn_debug_encode_fp8(None, None, 3, None) == 1
    assert lib.attn_mtp_accept(None, 1, None, 1, 4, 64, None, None, None, 0, None, None, None) == 1
    assert lib.attn_mtp_accept_workspace_size(0, 4, 64) == 0
    assert lib.attn_mtp_accept_workspace_size(128, 4, 151936) > 0


@pytest.mark.parametrize("chunk_bytes,waves,access", [
    (1024, 64, 1),      # half-line access needs 2 KB rows of 16 x 128 bytes
    (2048, 64, 2),      # no such access pattern
    (3072, 64, 0),      # not a power of two
    (512, 64, 0),       # below one 1 KB line
    (2048, 0, 0),       # no waves
])
def test_calibration_arguments_rejected(chunk_bytes, waves, access):
    import ctypes as c
    lib = pa.load_library()
    fake = c.c_void_p(1 << 20)  # aligned, non-null, never dereferenced: rejected first
    assert lib.attn_calib_stream_read(fake, 1 << 30, fake, 16, chunk_bytes, waves, access, fake,
                                      None, None, None) == 1
