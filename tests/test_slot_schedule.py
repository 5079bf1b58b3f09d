"""The in-place decode's pass schedule (splitzip_slot_schedule, host code of
the C-ABI library; no GPU).

The slot holds the payload in page 1's layout ("splitzip_codec.py -- SplitZip
codec adapter for diffusers-dynamic-offloader", assemble_payload) and
receives the 2n decoded bytes over it.  From the schedule the library
returns, these tests rebuild what every pass reads from the slot and writes
to it under the kernels' rules, byte by byte, and check that

* no pass reads a slot byte that an earlier pass has overwritten,
* no tile writes a byte that another tile of the same pass reads from the
  slot (pass 1's copies to the stash included),
* the tiles' outputs cover [0, 2n) exactly once,
* the tensor's last pass holds at least one tile (it applies escape streams
  not marked ascending),

for many sizes, payload lengths and pass counts; and that the bisection the
library uses agrees with the recursive definition of a tile's pass."""
import random

import numpy as np
import pytest

from lossless_bf16_tensor_splitzip_amd import _abi

T = 8192


def a4(v):
    return (v + 3) & ~3


def geom(n):
    N = -(-n // T)
    P = -(-n // 2)
    S0 = a4(P)
    C0 = a4(S0 + n)
    return N, P, S0, C0


def tile_len(n, t):
    return min(T, n - t * T)


def assignment(n, comp, passes):
    """Per tile: pass, pk from the stash, sm from the stash (kernel rules)."""
    used, t_min, lo, hi = _abi.splitzip_slot_schedule(n, passes)
    N, P, S0, C0 = geom(n)
    assert t_min == min(N, -(-C0 // (2 * T)))
    assert lo[2] == 0 and hi[2] == t_min
    for k in range(2, used):
        assert lo[k] <= lo[k + 1] <= hi[k + 1] <= hi[k], (n, passes, lo, hi)
    t_split = min(N, -(-comp // (2 * T)))
    assert t_split >= t_min
    p = np.zeros(N, np.int64)
    pk_st = np.zeros(N, bool)
    sm_st = np.zeros(N, bool)
    for t in range(N):
        if t >= t_split:
            p[t] = 1
        elif t >= t_min:
            p[t], pk_st[t], sm_st[t] = used, True, True
        else:
            k = max(k for k in range(2, used + 1) if lo[k] <= t < hi[k])
            p[t], pk_st[t], sm_st[t] = k, True, k == used
    return used, t_min, p, pk_st, sm_st


def simulate(n, comp, passes, g=1):
    """Byte-level check of one schedule; g = granule (every boundary a multiple of it)."""
    used, t_min, p, pk_st, sm_st = assignment(n, comp, passes)
    N, P, S0, C0 = geom(n)
    size = max(2 * n, comp)
    assert size % g == 0
    written = np.zeros(size // g, bool)
    cover = np.zeros(size // g, np.int32)

    def rng(a, b):
        assert a % g == 0 and b % g == 0, (a, b, g)
        return slice(a // g, b // g)

    for k in range(1, used + 1):
        reader = np.full(size // g, -1, np.int64)   # -1 none, -2 several
        def read(a, b, who):
            if b <= a:
                return
            s = rng(a, b)
            assert not written[s].any(), ("read after overwrite", n, comp, passes, k, who)
            r = reader[s]
            reader[s] = np.where(r == -1, who, np.where(r == who, who, -2))
        tiles = np.nonzero(p == k)[0]
        for t in tiles:
            L = tile_len(n, t)
            if not pk_st[t]:
                read(t * T // 2, (t * T + L + 1) // 2, t)
            if not sm_st[t]:
                read(S0 + t * T, S0 + t * T + L, t)
            if k == 1:
                read(C0, comp, t)   # its escapes, found in the slot
        if k == 1:   # the copies to the stash
            for t in range(N):
                L = tile_len(n, t)
                if pk_st[t]:
                    read(t * T // 2, (t * T + L + 1) // 2, -3)
                if sm_st[t]:
                    read(S0 + t * T, S0 + t * T + L, -3)
            read(C0, comp, -3)
        for t in tiles:
            s = rng(2 * t * T, 2 * t * T + 2 * tile_len(n, t))
            r = reader[s]
            assert ((r == -1) | (r == t)).all(), ("same-pass overwrite", n, comp, passes, k, t)
            cover[s] += 1
        for t in tiles:
            written[rng(2 * t * T, 2 * t * T + 2 * tile_len(n, t))] = True
    assert (cover[: 2 * n // g] == 1).all()
    assert (cover[2 * n // g:] == 0).all()
    if n:
        assert (p[:t_min] == used).any(), "the last pass holds a tile below t_min"
    return used, p, pk_st, sm_st


def comps(n):
    """Payload lengths: no escapes, a few, 0.1 %, about the most that fits in
    2n bytes, and one longer than 2n (a slot larger than the output)."""
    return sorted({_abi.splitzip_payload_size(n, e) for e in (0, 7, n // 1000, n // 14, n // 3)})


SMALL = [1, 2, 3, 5, 8, 100, 8191, 8192, 8193, 16383, 16384, 16385, 3 * 8192 + 5, 5 * 8192,
         7 * 8192 + 1, 100003, 1000003]


@pytest.mark.parametrize("n", SMALL)
def test_schedule_is_hazard_free_small(n):
    for passes in range(2, 9):
        for comp in comps(n):
            simulate(n, comp, passes)


def test_schedule_is_hazard_free_kv_layer():
    n = 4194304
    for passes in (2, 3, 4, 6, 8):
        for comp in comps(n):
            simulate(n, comp, passes)


def test_schedule_is_hazard_free_random_sizes():
    rnd = random.Random(20261202)
    for _ in range(16):
        n = rnd.randint(1, 1 << 21)
        passes = rnd.randint(2, 8)
        for comp in comps(n):
            simulate(n, comp, passes)


@pytest.mark.parametrize("n", [1 << 25, 37748736])
def test_schedule_is_hazard_free_full_sizes(n):
    # every boundary is a multiple of 4 here (n % 8 == 0, payload lengths
    # rounded down to a whole escape count whose length is a multiple of 4)
    for passes in (2, 4, 8):
        for e in (0, 3000, n // 1000 // 4 * 4):
            comp = _abi.splitzip_payload_size(n, e)
            if comp % 4:
                continue
            simulate(n, comp, passes, g=4)


def direct_pass(n, passes):
    """Pass of every tile below t_min from the recursive definition (all readers)."""
    N, P, S0, C0 = geom(n)
    t_min = min(N, -(-C0 // (2 * T)))
    depth = {}

    def readers(w):
        o0, o1 = 2 * w * T, 2 * w * T + 2 * tile_len(n, w)
        return [t for t in range(max(0, (o0 - S0) // T - 1), min(t_min, (o1 - S0) // T + 2))
                if S0 + t * T < o1 and S0 + t * T + tile_len(n, t) > o0]

    def dep(w):
        if w not in depth:
            r = readers(w)
            if w in r:
                depth[w] = 10 ** 9
            else:
                depth[w] = 1 + max((dep(t) for t in r), default=-1)
        return depth[w]

    order = sorted(range(t_min), key=lambda w: -abs(w - S0 // T))   # outermost first
    for w in order:
        dep(w)
    return [min(passes, 2 + depth[w]) for w in range(t_min)]


@pytest.mark.parametrize("n", [8192 * 5, 100003, 1000003, 4194304, (1 << 23) + 4, 1 << 25])
def test_bisection_matches_definition(n):
    for passes in range(3, 9):
        used, t_min, lo, hi = _abi.splitzip_slot_schedule(n, passes)
        want = direct_pass(n, passes)
        if used != passes:   # fallback: every tile in pass 2
            assert max(want, default=2) < passes
            continue
        got = [max(k for k in range(2, used + 1) if lo[k] <= w < hi[k]) for w in range(t_min)]
        assert got == want


def test_stash_traffic_falls_with_passes():
    """Bytes moved per algorithmic byte (3.5 per element) on a 2^25-element
    tensor with 0.1 % escapes: 1.65x with every overlapping tile stashed,
    about 1.32x with four passes."""
    n = 1 << 25
    comp = _abi.splitzip_payload_size(n, 33000)
    ratios = {}
    for passes in (2, 3, 4, 5, 8):
        used, t_min, p, pk_st, sm_st = assignment(n, comp, passes)
        N, P, S0, C0 = geom(n)
        lens = np.array([tile_len(n, t) for t in range(N)])
        pk = (lens + 1) // 2
        extra = 2 * (pk * pk_st).sum() + 2 * (lens * sm_st).sum() + 2 * (comp - C0)
        ratios[passes] = (3.5 * n + extra) / (3.5 * n)
    assert 1.64 < ratios[2] < 1.66
    assert 1.31 < ratios[4] < 1.34
    assert ratios[2] > ratios[3] > ratios[4] > ratios[5] > ratios[8]


def test_schedule_argument_errors():
    assert _abi.splitzip_slot_schedule(100, 1) is None
    assert _abi.splitzip_slot_schedule(100, 9) is None
    assert _abi.splitzip_slot_schedule((1 << 36) + 1, 4) is None
    assert _abi.splitzip_slot_schedule(0, 4)[1] == 0


@pytest.mark.parametrize("mistake", ["lo3+1", "lo3-1", "hi3+1", "hi3-1", "loK+1", "hiK-1",
                                     "last pass reads sm from the slot"])
def test_checker_catches_planted_schedule_mistakes(mistake, monkeypatch):
    """The byte-level check fails for a schedule with one range bound moved
    by a tile, or with the last pass's sm bytes left in the slot."""
    n = 1 << 22
    comp = _abi.splitzip_payload_size(n, 4000)
    orig = _abi.splitzip_slot_schedule
    if mistake.startswith(("lo", "hi")):
        def planted(n_, passes):
            used, t_min, lo, hi = orig(n_, passes)
            arr = lo if mistake.startswith("lo") else hi
            k = used if mistake[2] == "K" else 3
            arr[k] += 1 if mistake.endswith("+1") else -1
            return used, t_min, lo, hi
        monkeypatch.setattr(_abi, "splitzip_slot_schedule", planted)
    else:
        orig_assign = assignment

        def planted_assignment(n_, comp_, passes):
            used, t_min, p, pk_st, sm_st = orig_assign(n_, comp_, passes)
            sm_st = sm_st & ~((p == used) & (np.arange(len(p)) < t_min))
            return used, t_min, p, pk_st, sm_st
        monkeypatch.setitem(globals(), "assignment", planted_assignment)
    with pytest.raises(AssertionError):
        simulate(n, comp, 4)
