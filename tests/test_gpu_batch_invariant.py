"""Fixed pieces (the plan's kv_piece_len): parity with the fp64 oracle on
every kernel family, and a sequence's output rows bit-identical whatever its
batch-mates, the batch size and max_ctx_len of the plan, and its place in
the batch and in the page pool."""

import numpy as np
import pytest

import oracle
from synth import custom_workload, make_workload
from tests.gpu_helpers import check_contract, log, plan_for, run_gpu

pytestmark = pytest.mark.gpu


def _oracle(w, kv_format):
    return oracle.paged_attention(w.q, w.k_pages, w.v_pages, w.kv_scales, w.block_table, w.ctx_lens, w.q_lens,
                                  num_kv_heads=w.num_kv_heads, sm_scale=w.sm_scale, kv_format=kv_format)


def _run(w, piece, kv_format):
    plan = plan_for(w, kv_piece_len=piece, kv_format=kv_format)
    info = plan.info()
    got = run_gpu(w, plan=plan)
    plan.close()
    return got, info


PARITY = {
    # name: (workload, keys per piece, kv format)
    "decode": (lambda: make_workload("llama3_8b_decode", batch=6, ctx_range=(1, 2500)), 256, "e4m3"),
    "decode_one_chunk": (lambda: custom_workload([1] * 4, [1, 31, 32, 700], num_q_heads=32, num_kv_heads=8,
                                                 seed=401), 32, "e4m3"),
    "mqa": (lambda: make_workload("mqa_decode", batch=5, ctx_range=(256, 4000)), 512, "e4m3"),
    "mtp": (lambda: make_workload("mtp_verify", batch=9, ctx_range=(128, 900)), 128, "e4m3"),
    "prefill": (lambda: make_workload("prefill_chunk", batch=3, ctx_range=(0, 600), q_len=96), 256, "e4m3"),
    "single_tile_d64": (lambda: custom_workload([1, 2, 1], [900, 64, 2000], num_q_heads=16, num_kv_heads=2,
                                                head_dim=64, seed=402), 512, "e4m3"),
    "decode_int8": (lambda: make_workload("llama3_8b_decode", batch=4, ctx_range=(300, 2000), kv_format="int8"),
                    512, "int8"),
    "mtp_int4": (lambda: make_workload("mtp_verify", batch=6, ctx_range=(128, 900), kv_format="int4"), 256,
                 "int4"),
    # full size: 32 sequences x 8 kv heads of up to 8192 keys, 1024-key pieces
    "decode_full": (lambda: make_workload("llama3_8b_decode", keep_logical=False), 1024, "e4m3"),
    "mqa_full": (lambda: make_workload("mqa_decode", keep_logical=False), 2048, "e4m3"),
}


@pytest.mark.parametrize("case", sorted(PARITY))
def test_fixed_pieces_parity(case):
    make, piece, fmt = PARITY[case]
    w = make()
    log(f"fixed pieces parity: {case} piece={piece} B={w.num_seqs} Hq={w.num_q_heads} Hkv={w.num_kv_heads} "
        f"D={w.head_dim} ctx=[{w.ctx_lens.min()},{w.ctx_lens.max()}] fmt={fmt}")
    got, info = _run(w, piece, fmt)
    assert not info["packed"] or info["work_units"] >= 1
    check_contract(got, _oracle(w, fmt), w.out_dtype, what=f"fixed pieces {case}")


def _rows(w, b):
    r0 = int(np.sum(w.q_lens[:b]))
    return slice(r0, r0 + int(w.q_lens[b]))


def _transplant(src, b_src, dst, b_dst):
    """Give sequence b_dst of dst the queries and the page contents of
    sequence b_src of src (same lengths), in dst's own physical pages."""
    assert src.ctx_lens[b_src] == dst.ctx_lens[b_dst] and src.q_lens[b_src] == dst.q_lens[b_dst]
    dst.q[_rows(dst, b_dst)] = src.q[_rows(src, b_src)]
    for j in range(-(-int(src.ctx_lens[b_src]) // 16)):
        ps, pd = int(src.block_table[b_src, j]), int(dst.block_table[b_dst, j])
        dst.k_pages[pd] = src.k_pages[ps]
        dst.v_pages[pd] = src.v_pages[ps]
        dst.kv_scales[:, pd] = src.kv_scales[:, ps]


INVARIANT = {
    # name: (heads q/kv, head_dim, q_len, lengths of batch A (sequence 1 is the
    #        one compared), lengths of batch B (sequence 3 gets it), piece, format)
    "packed_decode": (32, 8, 128, 1, [900, 1234, 40, 3000], [70, 5000, 2, 1234, 800, 16, 4096], 256, "e4m3"),
    "tile_mqa": (64, 1, 128, 1, [2000, 3333, 300], [5000, 16, 700, 3333, 90, 1200, 64, 4100, 2], 512, "e4m3"),
    "tile_mtp": (40, 8, 128, 5, [300, 701, 50], [900, 20, 400, 701] + [333] * 60, 128, "e4m3"),
    # A: every segment one piece, so the units take whole segments longest
    # first; B: a longer sequence, so the units walk the pieces
    "tile_mtp_whole": (40, 8, 128, 5, [300, 701, 400], [900, 20, 5000, 701], 1024, "e4m3"),
    "prefill": (32, 8, 128, 96, [200, 480], [600, 96, 300, 480, 150], 256, "e4m3"),
    "packed_decode_int8": (32, 8, 128, 1, [900, 1234, 40], [5000, 2, 66, 1234, 700], 512, "int8"),
}


@pytest.mark.parametrize("case", sorted(INVARIANT))
def test_rows_do_not_depend_on_the_batch(case):
    hq, hkv, d, ql, la, lb, piece, fmt = INVARIANT[case]
    a = custom_workload([ql] * len(la), la, num_q_heads=hq, num_kv_heads=hkv, head_dim=d, seed=410,
                        kv_format=fmt, name=f"inv_a_{case}")
    b = custom_workload([ql] * len(lb), lb, num_q_heads=hq, num_kv_heads=hkv, head_dim=d, seed=411,
                        kv_format=fmt, name=f"inv_b_{case}")
    _transplant(a, 1, b, 3)
    log(f"batch invariance: {case} piece={piece} A={la} B={lb} fmt={fmt}")
    got_a, info_a = _run(a, piece, fmt)
    got_b, info_b = _run(b, piece, fmt)
    log(f"  units A={info_a['work_units']} B={info_b['work_units']}")
    # the compared rows match the oracle in both batches and are bit-identical
    check_contract(got_a, _oracle(a, fmt), a.out_dtype, what=f"invariance A {case}")
    check_contract(got_b, _oracle(b, fmt), b.out_dtype, what=f"invariance B {case}")
    assert np.array_equal(got_a[_rows(a, 1)], got_b[_rows(b, 3)]), case


def test_full_size_decode_rows_in_another_batch():
    # a sequence of the 32-sequence decode batch (up to 8192 keys), moved into
    # a batch of three with other lengths, keeps its rows bit for bit
    a = make_workload("llama3_8b_decode", keep_logical=False)
    j = int(np.argmax(a.ctx_lens))
    b = custom_workload([1] * 4, [100, 3000, 7, int(a.ctx_lens[j])], num_q_heads=a.num_q_heads,
                        num_kv_heads=a.num_kv_heads, head_dim=a.head_dim, seed=412, keep_logical=False,
                        name="inv_full_b")
    _transplant(a, j, b, 3)
    log(f"batch invariance, full size: sequence {j} of {a.num_seqs} (ctx {int(a.ctx_lens[j])}) piece=1024")
    got_a, _ = _run(a, 1024, "e4m3")
    got_b, _ = _run(b, 1024, "e4m3")
    check_contract(got_b, _oracle(b, "e4m3"), b.out_dtype, what="invariance, full size B")
    assert np.array_equal(got_a[_rows(a, j)], got_b[_rows(b, 3)])
