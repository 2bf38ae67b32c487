"""The balanced chunk schedule that the attention kernels walk, written out
on the CPU and checked against what the merge relies on (CPU only).

The kernels give unit w of W the positions [floor(wT/W), floor((w+1)T/W))
of the concatenated segment counts, a segment counting its chunks plus a
start cost; position v of a segment is its chunk v - start_cost.  Every
real chunk must be covered exactly once, every (segment, unit) piece must
have its own partial slot (segment + w), the unit holding a segment's start
must record its first slot and the number of pieces, and a segment held by
one unit is written whole."""

import itertools
import random

import pytest


def _wg_of_chunk(g, T, W):
    return ((g + 1) * W + T - 1) // T - 1


def _walk(real, w_max, min_chunks, start_cost):
    sched = [n + start_cost if n > 0 else 0 for n in real]
    T = sum(sched)
    W = max(1, min(w_max, T // min_chunks))
    starts = [0] + list(itertools.accumulate(sched))
    pieces = {s: [] for s in range(len(real))}
    merge = {}
    for w in range(W):
        lo, hi = w * T // W, (w + 1) * T // W
        if lo >= hi:
            continue
        s = next(i for i in range(len(real)) if sched[i] > 0 and starts[i] <= lo < starts[i] + sched[i])
        r, cur = lo - starts[s], lo
        while True:
            n = sched[s]
            take = min(n - r, hi - cur)
            whole = r == 0 and take == n
            pieces[s].append((w, max(r - start_cost, 0), max(r + take - start_cost, 0), whole))
            if r == 0:
                merge[s] = (s + w, 1 if whole else _wg_of_chunk(cur + n - 1, T, W) - w + 1)
            cur += take
            if cur >= hi:
                break
            r = 0
            s += 1
            while sched[s] == 0:
                s += 1
    return pieces, merge


def _check(real, w_max, min_chunks, start_cost):
    if sum(real) == 0:
        return
    pieces, merge = _walk(real, w_max, min_chunks, start_cost)
    slots = set()
    for s, n in enumerate(real):
        ps = pieces[s]
        if n == 0:
            assert not ps
            continue
        cover = [0] * n
        for w, cb, ce, _ in ps:
            assert 0 <= cb <= ce <= n
            for c in range(cb, ce):
                cover[c] += 1
            assert s + w not in slots
            slots.add(s + w)
        assert cover == [1] * n, (real, s, ps)
        first, count = merge[s]
        assert first == s + ps[0][0] and count == len(ps)
        assert [p[0] for p in ps] == list(range(ps[0][0], ps[0][0] + count))
        if count == 1:
            assert ps[0][3] and ps[0][1:3] == (0, n)
        else:
            assert not any(p[3] for p in ps)
        assert any(ce > cb for _, cb, ce, _ in ps)  # some unit reads the segment


@pytest.mark.parametrize("start_cost", [0, 1, 2, 3])
def test_schedule_random_mixes(start_cost):
    rng = random.Random(100 + start_cost)
    for _ in range(600):
        real = [rng.choice([0, rng.randint(1, 3), rng.randint(1, 200)]) for _ in range(rng.randint(1, 40))]
        _check(real, rng.choice([1, 2, 7, 64, 1024]), rng.choice([1, 2, 8]), start_cost)


def test_schedule_decode_shapes():
    # 32 sequences x 8 kv heads: aligned lengths, alternating lengths, one long one
    for real in ([72] * 256, [70] * 8 + [74] * 8, [1] * 255 + [4000]):
        for sc in (0, 1):
            _check(real * (256 // len(real)) if len(real) < 256 else real, 1024, 8, sc)


def test_empty_start_piece_is_possible_and_covered():
    # with a start cost a unit can hold only a segment's start position: its
    # piece has no chunks (the kernel writes an empty partial for it)
    found = False
    rng = random.Random(7)
    for _ in range(300):
        real = [rng.randint(1, 30) for _ in range(rng.randint(2, 12))]
        pieces, _ = _walk(real, 64, 1, 1)
        if any(cb == ce for ps in pieces.values() for _, cb, ce, _ in ps):
            found = True
            _check(real, 64, 1, 1)
    assert found


# ---- fixed pieces (kv_piece_len > 0) -----------------------------------------
# A segment of n chunks counts ceil(n / C) positions, position k being its
# chunks [kC, min((k+1)C, n)); unit w of W = min(units, positions) runs each
# position in [floor(wT/W), floor((w+1)T/W)) on its own, into the partial
# slot of its global position, and the unit holding a segment's position 0
# records (that slot, the segment's piece count).

def _walk_fixed(real, w_max, C):
    cnt = [-(-n // C) for n in real]
    T = sum(cnt)
    W = max(1, min(w_max, T))
    starts = [0] + list(itertools.accumulate(cnt))
    pieces = {s: [] for s in range(len(real))}
    merge = {}
    for w in range(W):
        lo, hi = w * T // W, (w + 1) * T // W
        if lo >= hi:
            continue
        s = next(i for i in range(len(real)) if cnt[i] > 0 and starts[i] <= lo < starts[i] + cnt[i])
        r, cur = lo - starts[s], lo
        while True:
            n = cnt[s]
            pieces[s].append((w, r * C, min(r * C + C, real[s]), n == 1, cur))
            if r == 0:
                merge[s] = (cur, n)
            cur += 1
            if cur >= hi:
                break
            r += 1
            if r < n:
                continue
            r = 0
            s += 1
            while cnt[s] == 0:
                s += 1
    return pieces, merge


def _check_fixed(real, w_max, C):
    if sum(real) == 0:
        return
    pieces, merge = _walk_fixed(real, w_max, C)
    slot_bound = len(real) * -(-max(real) // C)  # the plan's slots for this many segments
    slots = set()
    for s, n in enumerate(real):
        ps = pieces[s]
        if n == 0:
            assert not ps and s not in merge
            continue
        # cut points of the segment alone, whatever the other segments and W
        assert [(cb, ce) for _, cb, ce, _, _ in ps] == [(k * C, min(k * C + C, n)) for k in range(-(-n // C))]
        for *_, slot in ps:
            assert 0 <= slot < slot_bound and slot not in slots
            slots.add(slot)
        first, count = merge[s]
        assert count == len(ps) and [p[4] for p in ps] == list(range(first, first + count))
        assert all(p[3] == (count == 1) for p in ps)


@pytest.mark.parametrize("C", [1, 2, 16, 64])
def test_fixed_pieces_random_mixes(C):
    rng = random.Random(300 + C)
    for _ in range(400):
        real = [rng.choice([0, rng.randint(1, 3), rng.randint(1, 300)]) for _ in range(rng.randint(1, 40))]
        _check_fixed(real, rng.choice([1, 2, 7, 64, 1024]), C)


def test_fixed_pieces_do_not_depend_on_batch_mates():
    # the same segment among different batch-mates and unit counts is cut
    # at the same chunks and merged from the same number of pieces
    rng = random.Random(11)
    target = 157
    for _ in range(200):
        mates = [rng.randint(0, 400) for _ in range(rng.randint(0, 30))]
        at = rng.randint(0, len(mates))
        real = mates[:at] + [target] + mates[at:]
        pieces, merge = _walk_fixed(real, rng.choice([1, 5, 256, 2048]), 16)
        assert [(cb, ce) for _, cb, ce, _, _ in pieces[at]] == [(k * 16, min(k * 16 + 16, target)) for k in range(10)]
        assert merge[at][1] == 10


# ---- whole-segment schedule of the shared-KV tile kernel --------------------
# When the segments (one column block each) are at least 3/4 of the units W
# and at most W, and the longest holds at most twice the mean chunks, unit w
# takes kv head w % H of the sequence ranked w // H (most chunks first, ties
# by index) whole.  The kernel ranks the sequences two per lane: lane i holds
# sequences i and 64 + i and counts, over j < 64, the sequences that sort
# before each of its own.

def _kernel_ranks(n):
    """Ranks as the kernel computes them: 8 classes of equal width of the
    chunk count up to the longest, the longest class first, sequence index
    within a class (sequences past len(n) hold 0 chunks and no rank)."""
    mx = max(n) if n else 0
    cls = [(x * 8) // (mx + 1) for x in n]
    order = sorted(range(len(n)), key=lambda i: (-cls[i], i))
    rk = [0] * len(n)
    for r, i in enumerate(order):
        rk[i] = r
    return rk + [0] * (128 - len(n))


def _whole_decision(n, H, W):
    S = len(n) * H
    if len(n) > 128 or S > W or 4 * S < 3 * W:
        return False
    return max(n) * len(n) <= 2 * sum(n)


def _whole_units(n, H, W):
    """The piece of each unit as the kernel builds it: (sequence, kv head,
    first chunk, end chunk), or None for units past the segments."""
    B = len(n)
    rk = _kernel_ranks(n)[:B]
    out = []
    for w in range(W):
        if w >= B * H:
            out.append(None)
            continue
        r, h = divmod(w, H)
        b = rk.index(r)
        out.append((b, h, 0, n[b]))
    return out


def test_kernel_ranks_order_by_length_class():
    rng = random.Random(11)
    for _ in range(300):
        B = rng.randint(1, 128)
        n = [rng.choice([rng.randint(0, 3), rng.randint(1, 40), 7]) for _ in range(B)]
        rk = _kernel_ranks(n)[:B]
        assert sorted(rk) == list(range(B))
        by_rank = [n[i] for i in sorted(range(B), key=lambda i: rk[i])]
        # a sequence ranked after another is shorter, or in the same class
        mx = max(n)
        width = (mx + 1) / 8
        for a, b in zip(by_rank, by_rank[1:]):
            assert b <= a or b - a < width
        # exact order where the classes separate the lengths: all distinct classes
        if len(set((x * 8) // (mx + 1) for x in n)) == B:
            assert by_rank == sorted(n, reverse=True)


def test_whole_segment_units_cover_each_segment_once():
    rng = random.Random(200)
    seen = 0
    for _ in range(300):
        H = rng.choice([1, 2, 8])
        B = rng.randint(1, 128)
        W = rng.choice([B * H, B * H + rng.randint(0, B * H // 3), 1024])
        lo_n = rng.randint(1, 20)
        n = [rng.choice([0, rng.randint(lo_n, 2 * lo_n)]) if rng.random() < 0.05 else rng.randint(lo_n, 2 * lo_n)
             for _ in range(B)]
        if not _whole_decision(n, H, W):
            continue
        seen += 1
        units = _whole_units(n, H, W)
        got = sorted(u for u in units if u is not None and u[3] > u[2])
        assert got == [(b, h, 0, n[b]) for b in range(B) for h in range(H) if n[b] > 0]
        # longest class first: unit numbers rise as the classes shorten
        mx = max(n)
        cls = [(u[3] * 8) // (mx + 1) for u in units if u is not None]
        assert cls == sorted(cls, reverse=True)
    assert seen > 50


def test_whole_decision_on_the_named_shapes():
    rng = random.Random(5)
    # MTP verification: 128 sequences x 8 kv heads, 5 new tokens, 128-1152 keys
    n = [(rng.randint(128, 1152) + 31) // 32 for _ in range(128)]
    assert _whole_decision(n, 8, 1024)
    # one long sequence among short ones stays with the balanced split
    assert not _whole_decision([4] * 127 + [400], 8, 1024)
    # fewer segments than three quarters of the units (MQA decode, 64 x 1)
    assert not _whole_decision([100] * 64, 1, 512)
