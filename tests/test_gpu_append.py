"""GPU parity of the paged FP8 KV append (attn_kv_append) with the oracle,
through the C ABI: the whole K and V pools and every scale must come back
bit for bit (untouched pages, poisoned tails and NaN scales included)."""

import numpy as np
import pytest
import torch

import oracle.kv_append as ka
from oracle import e4m3
from paged_fp8_kv_attn_amd import Plan, debug_encode_fp8
from synth import append as sa
from tests.gpu_helpers import log

pytestmark = pytest.mark.gpu


def _probe_values():
    vals = e4m3.decode(np.arange(0x7F, dtype=np.uint8))
    mids = (vals[:-1] + vals[1:]) / 2
    f = np.float32
    ys = [vals, mids, np.nextafter(mids.astype(f), f(0)), np.nextafter(mids.astype(f), f(1000)),
          np.array([0.0, 2.0 ** -10, 2.0 ** -11, 3 * 2.0 ** -11, 2.0 ** -30, 1e-38, 447.99, 448.0, 448.01, 464.0,
                    464.01, 500.0, 1e6, 3e38])]
    rng = np.random.default_rng(11)
    ys.append(np.exp(rng.uniform(np.log(2.0 ** -14), np.log(600.0), 100000)))
    y = np.concatenate([np.asarray(a, dtype=np.float64) for a in ys]).astype(np.float32)
    return np.concatenate([y, -y, np.array([-0.0], dtype=np.float32)])


def test_encode_bit_exact():
    y = _probe_values()
    log(f"encode: {y.size} values")
    x = torch.from_numpy(y).cuda()
    out = torch.empty(y.size, dtype=torch.uint8, device="cuda")
    debug_encode_fp8(x, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    want = ka.encode(y)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, f"{bad.size} mismatches, e.g. {[(float(y[i]), int(got[i]), int(want[i])) for i in bad[:8]]}"


def _plan_for(c):
    return Plan(num_seqs=c.num_seqs, num_q_heads=c.num_kv_heads, num_kv_heads=c.num_kv_heads, head_dim=c.head_dim,
                num_pages=c.num_pages, max_pages_per_seq=c.max_pages_per_seq, max_q_len=c.max_q_len,
                max_ctx_len=c.max_ctx_len, kv_format=c.kv_format)


def _append_parity(c):
    log(f"append: {c.name} seed={c.seed} B={c.num_seqs} Hkv={c.num_kv_heads} D={c.head_dim} dtype={c.new_dtype} "
        f"kv={c.kv_format} "
        f"q=[{c.q_lens.min()},{c.q_lens.max()}] ctx=[{c.ctx_lens.min()},{c.ctx_lens.max()}]")
    dev = "cuda"
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)  # noqa: E731
    k, v, s = t(c.k_pages), t(c.v_pages), t(c.kv_scales)
    plan = _plan_for(c)
    plan.kv_append(c.k_new.to(dev).contiguous(), c.v_new.to(dev).contiguous(), k, v, s, t(c.block_table),
                   t(c.ctx_lens), t(c.q_lens))
    torch.cuda.synchronize()
    plan.close()
    ok, ov, os_ = ka.kv_append(c.k_new, c.v_new, c.k_pages, c.v_pages, c.kv_scales, c.block_table, c.ctx_lens,
                               c.q_lens, kv_format=c.kv_format)
    gk, gv, gs = k.cpu().numpy(), v.cpu().numpy(), s.cpu().numpy()
    nk = int((gk != ok).sum())
    nv = int((gv != ov).sum())
    ns = int((gs.view(np.uint32) != os_.view(np.uint32)).sum())
    assert nk == 0 and nv == 0 and ns == 0, f"{c.name}: K bytes off {nk}, V bytes off {nv}, scales off {ns}"


CASES = [
    # (q_lens, ctx_lens, Hkv, D, new_dtype, sigmas)
    ([3], [20], 1, 64, "f32", (4.0,)),
    ([1, 2], [17, 16], 2, 64, "bf16", (1.0,)),
    ([5, 1], [5, 33], 1, 128, "f32", (0.25,)),
    ([18], [40], 1, 64, "bf16", (2.0, 0.5)),
    ([1, 1, 1, 1], [1, 16, 17, 300], 8, 128, "bf16", (1.0, 3.0)),
    ([5, 5, 5], [5, 133, 700], 8, 128, "bf16", (0.5, 2.0)),  # MTP-shaped appends
    ([64, 33, 16], [64, 40, 1000], 2, 128, "f32", (1.0, 8.0)),
    ([16], [16], 1, 64, "f32", (0.0,)),  # all-zero rows: scale 1
    ([16, 5], [16, 5], 1, 64, "f32", (1e-30,)),  # page scales below 2^-90: plain IEEE division
    ([16, 9], [16, 9], 1, 128, "f32", (1e30,)),  # page scales above 2^90
]


@pytest.mark.parametrize("idx", range(len(CASES)))
def test_append_cases(idx):
    ql, cl, hkv, d, dt, sig = CASES[idx]
    _append_parity(sa.append_case(ql, cl, num_kv_heads=hkv, head_dim=d, new_dtype=dt, seed=60 + idx,
                                  new_sigmas=sig, name=f"append_edge{idx}"))


def test_append_decode_full():
    _append_parity(sa.make_append_case("append_decode"))


def test_append_prefill_reduced():
    _append_parity(sa.make_append_case("append_prefill", batch=3, ctx_range=(0, 700), q_len=96))


def test_append_prefill_full():
    _append_parity(sa.make_append_case("append_prefill"))


@pytest.mark.parametrize("idx", range(len(CASES)))
def test_append_cases_int8(idx):
    ql, cl, hkv, d, dt, sig = CASES[idx]
    _append_parity(sa.append_case(ql, cl, num_kv_heads=hkv, head_dim=d, new_dtype=dt, seed=90 + idx,
                                  new_sigmas=sig, name=f"append_int8_edge{idx}", kv_format="int8"))


@pytest.mark.parametrize("kv_format", ["e4m3", "int8"])
def test_append_quotients_at_rounding_midpoints(kv_format):
    # fresh pages whose values, divided by the page scale, land on (and one
    # or two fp32 ulps beside) every rounding midpoint of the format, so that
    # any quotient not rounded exactly as IEEE fp32 division changes a byte
    rng = np.random.default_rng(7 if kv_format == "e4m3" else 8)
    qmax = 448.0 if kv_format == "e4m3" else 127.0
    if kv_format == "e4m3":
        vals = e4m3.decode(np.arange(0x7F, dtype=np.uint8))
        mids = (vals[:-1] + vals[1:]) / 2
    else:
        mids = np.arange(-127, 127) + 0.5
    B, D, S = 12, 128, 16
    c = sa.append_case([S] * B, [S] * B, num_kv_heads=1, head_dim=D, new_dtype="f32", seed=70, kv_format=kv_format,
                       name=f"append_midpoints_{kv_format}")
    f32 = np.float32
    for which, tens in ((0, c.k_new), (1, c.v_new)):
        x = np.empty((B * S, 1, D), dtype=f32)
        for b in range(B):
            s0 = f32(np.exp(rng.uniform(np.log(1e-3), np.log(50.0))))
            xmax = f32(s0 * f32(qmax))
            scale = f32(xmax / f32(qmax))  # the scale the append will compute
            m = rng.choice(mids, size=S * D)
            m = m * rng.choice([-1.0, 1.0], size=m.size) if kv_format == "e4m3" else m
            q = np.nextafter(m.astype(f32), np.where(rng.random(m.size) < 0.5, f32(-1e9), f32(1e9)))
            q = np.where(rng.random(m.size) < 0.4, m.astype(f32), q)
            vals_b = (q.astype(np.float64) * np.float64(scale)).astype(f32)
            vals_b = np.clip(vals_b, -xmax, xmax)
            vals_b[0] = xmax
            x[b * S:(b + 1) * S, 0, :] = vals_b.reshape(S, D)
        tens.copy_(torch.from_numpy(x))
    _append_parity(c)
