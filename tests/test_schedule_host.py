"""The balanced schedule of the prefill, checked on the host (no GPU).

For a fixed-length batch whose chains do not fill whole rounds of the compute
units, the prefill lays the chains' chunks end to end and cuts them into equal
runs, one workgroup per run and round; a chain cut between two runs hands its
state over.  kda_balanced_schedule returns the workgroups' items exactly as the
kernel computes them (the same function of the workgroup index), and the
planner's decision whether the schedule pays is made from those same items.
These tests check that item list against an independent enumeration of the
definition, its invariants (every chunk of every chain once, in order; a chain's
second part waits on the workgroup holding its first part, dispatched earlier),
and the planner's decision against a re-simulation of its cost model.
"""
import heapq
import itertools

import pytest

import gated_delta_rule_10_amd as kda

C_TOK = 64


def expected_runs(C, n, U):
    """Runs of the definition: the C n chunks laid end to end (chain-major), cut
    into runs of L = ceil(C n / U) chunks.  Each run's items, in the order the
    kernel takes them: the head of a chain the next run finishes (if any), the
    whole chains, the tail of a chain the previous run began (if any)."""
    total = C * n
    L = -(-total // U)
    runs = []
    for s in range(0, total, L):
        e = min(s + L, total)
        pieces = []  # (chain, c0, c1) in chunk order
        pos = s
        while pos < e:
            c, off = divmod(pos, n)
            end = min(e, (c + 1) * n)
            pieces.append((c, off, end - c * n))
            pos = end
        items = []
        head = [p for p in pieces if p[1] == 0 and p[2] < n]
        tail = [p for p in pieces if p[1] > 0]
        whole = [p for p in pieces if p[1] == 0 and p[2] == n]
        if head:
            items.append((*head[0], 1))
        items += [(*p, 0) for p in whole]
        if tail:
            items.append((*tail[0], 2))
        runs.append(items)
    return L, runs


def pays(C, n, U, runs):
    """The planner's cost model: workgroup i goes to accelerator complex i mod 8
    and there to the first free unit; an item costs its chunks plus one."""
    W = len(runs)
    L = -(-(C * n) // U)
    K = L // n + 2
    if W > 4096 or K > 64 or C * n >= 1 << 30:
        return False
    rounds = max(len(r) for r in runs)
    cost = [None] * (rounds * W)
    for w, items in enumerate(runs):
        for k, it in enumerate(items):
            cost[k * W + w] = it[2] - it[1]
    xcd = 8 if U % 8 == 0 else 1
    finish = 0
    for x in range(xcd):
        free = [0] * (U // xcd)
        for i in range(x, rounds * W, xcd):
            if cost[i] is None:
                continue
            t = heapq.heappop(free) + cost[i] + 1
            heapq.heappush(free, t)
            finish = max(finish, t)
    whole = -(-C // U) * (n + 1)
    return 10 * finish <= 9 * whole


def applies(C, n, U):
    return C > U and C % U != 0 and n >= 2


CASES = [
    (4, 8192, 96, 256),    # 384 chains of 128 chunks: the 4 x 8,192 x 96 batch
    (3, 1000, 96, 256),    # ragged last chunk
    (1, 65536, 300, 256),
    (5, 4096, 64, 256),
    (2, 640, 9, 16),
    (7, 130, 3, 8),
    (3, 64 * 5, 5, 6),     # units not a multiple of 8
    (1, 8192, 257, 256),
    (2, 100, 200, 256),
    (6, 2048, 50, 64),
]


@pytest.mark.parametrize("N,T,H,U", CASES)
def test_schedule_matches_definition(N, T, H, U):
    C, n = N * H, -(-T // C_TOK)
    got = kda.balanced_schedule(N, T, H, U)
    if not applies(C, n, U):
        assert got is None
        return
    L, runs = expected_runs(C, n, U)
    use = pays(C, n, U, runs)
    assert (got is not None) == use, f"planner decision differs from its cost model ({C}, {n}, {U})"
    if got is None:
        return
    W = len(runs)
    rounds = max(len(r) for r in runs)
    assert len(got) == W * rounds
    for w, items in enumerate(runs):
        for k in range(rounds):
            b = k * W + w
            chain, c0, c1, role, wait = got[b]
            if k >= len(items):
                assert chain == -1, f"workgroup {b} should be empty"
                continue
            ec, e0, e1, erole = items[k]
            assert (chain, c0, c1, role) == (ec, e0, e1, erole), f"workgroup {b}"
            assert wait == (w - 1 if role == 2 else -1)


@pytest.mark.parametrize("N,T,H,U", CASES)
def test_schedule_invariants(N, T, H, U):
    got = kda.balanced_schedule(N, T, H, U)
    if got is None:
        return
    C, n = N * H, -(-T // C_TOK)
    pieces = {}
    for b, (chain, c0, c1, role, wait) in enumerate(got):
        if chain < 0:
            continue
        assert 0 <= chain < C and 0 <= c0 < c1 <= n
        pieces.setdefault(chain, []).append((c0, c1, role, wait, b))
    assert sorted(pieces) == list(range(C)), "every chain has work"
    for chain, ps in pieces.items():
        ps.sort()
        assert ps[0][0] == 0 and ps[-1][1] == n
        for a, b in zip(ps, ps[1:]):
            assert a[1] == b[0], f"chain {chain}: chunks skipped or repeated"
        if len(ps) == 1:
            assert ps[0][2] == 0
            continue
        assert len(ps) == 2, "a chain is cut at most once"
        head, tail = ps
        assert head[2] == 1 and tail[2] == 2
        assert tail[3] == head[4], "the tail waits on the workgroup holding the head"
        assert head[4] < tail[4], "the head is dispatched before the tail"
        # the head never waits: it is its run's first item
        assert head[3] == -1


def test_schedule_rejects_bad_sizes():
    lib = kda.library()
    import ctypes
    n = ctypes.c_int64(-1)
    for args in [(0, 64, 1, 256), (1, -1, 1, 256), (1, 64, 0, 256), (1, 64, 1, 0)]:
        assert lib.kda_balanced_schedule(*args, None, 0, ctypes.byref(n)) == 1
    assert lib.kda_balanced_schedule(1, 64, 1, 256, None, 0, None) == 1
    # capacity below the count with items given
    assert lib.kda_balanced_schedule(4, 8192, 96, 256, None, 0, ctypes.byref(n)) == 0
    assert n.value == 512
    buf = (ctypes.c_int32 * 10)()
    assert lib.kda_balanced_schedule(4, 8192, 96, 256, buf, 2, ctypes.byref(n)) == 1
    assert n.value == 512


def test_handoff_poll_limit_setting():
    old = kda.handoff_poll_limit()
    assert old == 1 << 22
    try:
        kda.set_handoff_poll_limit(0)
        assert kda.handoff_poll_limit() == 0
        with pytest.raises(kda.KDAError):
            kda.set_handoff_poll_limit(-1)
        assert kda.handoff_poll_limit() == 0
    finally:
        kda.set_handoff_poll_limit(old)


@pytest.mark.parametrize("U", [8, 16, 64, 256])
def test_schedule_decisions_sweep(U):
    """The planner's decision agrees with the cost model over a sweep of batch
    shapes, and every accepted schedule matches the definition."""
    for H, T in itertools.product((1, 3, 7, 9, 33, 96), (64, 130, 640, 2048)):
        for N in (1, 2, 3):
            C, n = N * H, -(-T // C_TOK)
            got = kda.balanced_schedule(N, T, H, U)
            if not applies(C, n, U):
                assert got is None
                continue
            L, runs = expected_runs(C, n, U)
            assert (got is not None) == pays(C, n, U, runs), (N, T, H, U)
            if got is not None:
                W = len(runs)
                flat = {k * W + w: it for w, items in enumerate(runs)
                        for k, it in enumerate(items)}
                for b, g in enumerate(got):
                    if b in flat:
                        assert g[:4] == flat[b]
                    else:
                        assert g[0] == -1
