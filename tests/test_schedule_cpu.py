"""Work-order arithmetic of the kernels, replayed on the CPU.

The decode and prefill kernels each turn a work-group index into a work unit with integer
steps that every work-group repeats on its own (decode: rank the sequences by length, take the
unit of its rank, mirror every second lap when the grid is resident; prefill: count the query
tiles above a key, search the key of its rank -- 64 probes a round, one per lane, with up to 16
prefill sequences, else bisection -- and resolve ties by sequence; packed step: interleave the
two roles within each residue class of the work-group index mod 8).  The GPU parity
tests show that every output row gets computed; these tests replay the same integer steps in
Python on many random batches and check the properties the order is meant to have: the grid maps
onto the units one to one, in the intended order, and the host's grid bound covers every unit.
"""
import numpy as np
import pytest


# ---------------------------------------------------------------- decode: longest first, snake
def decode_unit(j, lens, hkv, snake, resident=None, q_counts=None):
    """(sequence, KV head) of work-group j = z * hkv + x, as the decode kernel computes it: in a
    packed batch (q_counts given) the sequences that are not 1-token rows rank last, and the
    snake order applies when the taking-part units fit the resident work-groups."""
    n = len(lens)
    key = [(-1 if q_counts is not None and q_counts[t] != 1 else lens[t]) for t in range(n)]
    order = [0] * n
    for t in range(n):
        r = sum(1 for u in range(n) if key[u] > key[t] or (key[u] == key[t] and u < t))
        order[r] = t
    total = (n - sum(1 for k in key if k < 0)) * hkv
    if resident is None:
        resident = n * hkv
    if snake > 0 and total <= resident and j < total:
        lap, pos = divmod(j, snake)
        lap_len = min(snake, total - lap * snake)
        if lap & 1:
            j = lap * snake + (lap_len - 1 - pos)
    return order[j // hkv], j % hkv


@pytest.mark.parametrize("seed", range(12))
def test_decode_order_is_a_bijection_longest_first(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 70))
    hkv = int(rng.choice([1, 2, 3, 8]))
    lens = rng.integers(0, 40, size=n).tolist()  # many ties
    for snake in (0, 7, 16, 256):
        units = [decode_unit(j, lens, hkv, snake) for j in range(n * hkv)]
        assert sorted(units) == [(s, g) for s in range(n) for g in range(hkv)]
        if snake == 0:  # dispatch order: lengths never increase, ties by sequence index
            keys = [(-lens[s], s) for s, _ in units]
            assert keys == sorted(keys)
        else:  # each lap holds the same units as the plain order's lap (mirrored on odd laps)
            plain = [decode_unit(j, lens, hkv, 0) for j in range(n * hkv)]
            for lap0 in range(0, n * hkv, snake):
                assert sorted(units[lap0:lap0 + snake]) == sorted(plain[lap0:lap0 + snake])


@pytest.mark.parametrize("seed", range(12))
def test_packed_decode_rows_rank_first_and_keep_the_snake(seed):
    # a packed batch: only the 1-token rows take part; the others rank last, and the snake
    # order holds when the 1-token rows' units fit the resident grid, however many others there are
    rng = np.random.default_rng(1000 + seed)
    n = int(rng.integers(2, 60))
    hkv = int(rng.choice([1, 2, 8]))
    lens = rng.integers(1, 400, size=n).tolist()
    q = rng.choice([0, 1, 1, 1, 5, 40], size=n).tolist()
    active = sum(1 for x in q if x == 1)
    for snake, resident in ((16, active * hkv), (16, active * hkv - 1), (5, 10 ** 6)):
        units = [decode_unit(j, lens, hkv, snake, resident, q) for j in range(n * hkv)]
        assert sorted(units) == [(s, g) for s in range(n) for g in range(hkv)]
        head = units[:active * hkv]  # the 1-token rows' units come first
        assert all(q[s] == 1 for s, _ in head) and all(q[s] != 1 for s, _ in units[active * hkv:])
        plain = sorted(head, key=lambda u: (-lens[u[0]], u[0], u[1]))
        if resident >= active * hkv:  # snake: each lap of the plain order, odd laps mirrored
            for lap0 in range(0, active * hkv, snake):
                lap = plain[lap0:lap0 + snake]
                want = lap[::-1] if (lap0 // snake) & 1 else lap
                assert [lens[s] for s, _ in head[lap0:lap0 + snake]] == [lens[s] for s, _ in want]
        else:  # too many to be resident: plain longest-first order
            assert [lens[s] for s, _ in head] == [lens[s] for s, _ in plain]


# ---------------------------------------------------------------- prefill: rank -> unit
def prefill_schedule(cu_q, context_lens, tokw):
    """Unit (sequence, query tile) of every rank, or None for a spare work-group, as the prefill
    kernel computes it; and the host's bound on the number of ranks."""
    nseq = len(context_lens)
    q = np.diff(cu_q)
    comp = [(int(context_lens[s] - q[s]), int(q[s]), s) for s in range(nseq) if q[s] >= 2]

    def count_gt(k):
        c = 0
        for base, nn, _ in comp:
            x = k - base
            t = (nn + tokw - 1) // tokw
            c += t if x < 0 else (0 if x >= nn else t - x // tokw)
        return c

    total_q = int(cu_q[-1])
    chunks = min(nseq, total_q // 2)
    tiles_per_seq = (int(q.max()) + tokw - 1) // tokw if nseq else 0
    bound = min((total_q + chunks * (tokw - 1)) // tokw, tiles_per_seq * nseq)

    out = []
    for pair in range(bound):
        if not comp:
            out.append(None)
            continue
        klo = min(b + 1 for b, _, _ in comp)
        khi = max(b + nn for b, nn, _ in comp)
        if pair >= count_gt(klo - 1):
            out.append(None)
            continue
        if len(comp) <= 16:
            while klo < khi:  # lane l probes klo + ceil(span * l / 64); the true lanes are a prefix
                span = khi - klo + 1
                probes = [klo + (span * lane + 63) // 64 for lane in range(64)]
                true = [c <= khi and count_gt(c - 1) > pair for c in probes]
                h = max(lane for lane in range(64) if true[lane])
                assert all(true[:h + 1]) and not any(true[h + 1:])
                klo, khi = probes[h], (khi if h == 63 else probes[h + 1] - 1)
        else:
            while klo < khi:
                mid = klo + (khi - klo + 1) // 2
                if count_gt(mid - 1) > pair:
                    klo = mid
                else:
                    khi = mid - 1
        rank_in_key = pair - count_gt(klo)
        seen = 0
        unit = None
        for base, nn, s in comp:
            x = klo - base
            has = x == nn or (tokw <= x < nn and x % tokw == 0)
            if has:
                if seen == rank_in_key:
                    tt = (nn + tokw - 1) // tokw - 1 if x == nn else x // tokw - 1
                    unit = (s, tt, klo)
                    break
                seen += 1
        out.append(unit)
    return out, bound


def _random_packed(rng):
    nseq = int(rng.integers(1, 40))
    q = np.where(rng.random(nseq) < 0.5, 1, rng.integers(2, 300, size=nseq))
    q[rng.random(nseq) < 0.2] = 0  # sequences with no row this step
    cached = rng.integers(0, 500, size=nseq)
    cached[rng.random(nseq) < 0.3] = 0
    lens = cached + q
    # ties on purpose: equal chunks at equal offsets
    if nseq >= 4:
        q[1], lens[1] = q[0], lens[0]
        q[3], lens[3] = q[2], lens[2]
    cu = np.concatenate([[0], np.cumsum(q)]).astype(np.int64)
    return cu, lens.astype(np.int64)


@pytest.mark.parametrize("G", [1, 2, 4, 8, 16])
@pytest.mark.parametrize("seed", range(8))
def test_prefill_order_is_a_bijection_in_descending_key(G, seed):
    rng = np.random.default_rng(100 * G + seed)
    cu, lens = _random_packed(rng)
    tokw = 128 // G
    got, bound = prefill_schedule(cu, lens, tokw)
    q = np.diff(cu)
    want = {(s, t) for s in range(len(lens)) if q[s] >= 2 for t in range((q[s] + tokw - 1) // tokw)}
    units = [u for u in got if u is not None]
    assert sorted((s, t) for s, t, _ in units) == sorted(want)  # every unit once, none twice
    assert len(want) <= bound  # the host's grid bound covers every unit
    n_units = len(units)
    assert all(u is not None for u in got[:n_units]) and all(u is None for u in got[n_units:])  # spares last
    keys = [k for _, _, k in units]
    assert keys == sorted(keys, reverse=True)  # longest (most keys seen) first
    for s, t, k in units:  # the key is the keys seen by the tile's last row
        base = int(lens[s] - q[s])
        assert k == base + min(int(q[s]), (t + 1) * tokw)


@pytest.mark.parametrize("seed", range(4))
def test_prefill_order_over_wide_key_ranges(seed):
    # contexts far apart (tens of thousands of keys) and few chunks: the lane-probe search takes
    # several rounds
    rng = np.random.default_rng(500 + seed)
    nseq = int(rng.integers(2, 10))
    q = rng.integers(2, 700, size=nseq)
    lens = rng.integers(0, 60000, size=nseq) + q
    cu = np.concatenate([[0], np.cumsum(q)]).astype(np.int64)
    got, _ = prefill_schedule(cu, lens, 32)
    keys = [k for u in got if u is not None for k in [u[2]]]
    assert keys == sorted(keys, reverse=True)
    assert sorted((s, t) for s, t, _ in (u for u in got if u is not None)) == sorted(
        (s, t) for s in range(nseq) for t in range((q[s] + 31) // 32))


# ---------------------------------------------------------------- packed step: roles per XCD class
def packed_positions(n_pre, n_dec):
    """(role, rank) of every position of the packed-step grid, or None for a spare position: the
    roles are interleaved evenly within each residue class of the position mod 8, and class x takes
    the ranks x, x + 8, ... of both lists."""
    grid = 8 * ((n_pre + 7) // 8 + (n_dec + 7) // 8)
    out = []
    for b in range(grid):
        x, q = b % 8, b // 8
        npx = (n_pre - x + 7) // 8 if n_pre > x else 0
        ndx = (n_dec - x + 7) // 8 if n_dec > x else 0
        if q >= npx + ndx:
            out.append(None)
            continue
        before, upto = q * npx // (npx + ndx), (q + 1) * npx // (npx + ndx)
        role, idx = (1, before) if upto > before else (0, q - before)
        out.append((role, idx * 8 + x))
    return out


@pytest.mark.parametrize("seed", range(6))
def test_packed_roles_cover_both_lists_on_their_xcd(seed):
    rng = np.random.default_rng(900 + seed)
    for _ in range(50):
        n_pre, n_dec = int(rng.integers(0, 2000)), int(rng.integers(0, 2000))
        pos = packed_positions(n_pre, n_dec)
        taken = [p for p in pos if p is not None]
        assert sorted(r for role, r in taken if role == 1) == list(range(n_pre))
        assert sorted(r for role, r in taken if role == 0) == list(range(n_dec))
        assert all(p is None or p[1] % 8 == b % 8 for b, p in enumerate(pos))  # rank's class = XCD
        for x in range(8):  # within a class both lists keep their order (longest first)
            cls = [p for p in pos[x::8] if p is not None]
            for role in (0, 1):
                ranks = [r for ro, r in cls if ro == role]
                assert ranks == sorted(ranks)
