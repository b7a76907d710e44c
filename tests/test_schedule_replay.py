"""CPU replay of the attention kernels' tile schedules (attn_kernels.hip,
FusedAttn): every LDS buffer access, register hand-off and tile load of one
workgroup, restated in Python from the kernel's constants and loop bounds, and
checked for the hazards a wrong bound would cause on the GPU:

  * an LDS read of tile t must find tile t in its buffer slot, written in an
    earlier barrier interval, and no wave may write that slot in the interval
    of the read (read-after-overwrite);
  * a tile is committed from the registers that loaded that same tile;
  * a clamped tile load has no negative clamped row (tile * 64 <= NK - 1: the
    row offsets are unsigned), an unclamped one lies wholly inside the keys,
    and no load reaches outside [t_lo, n_tiles);
  * the unmasked (steady) softmax and score tiles lie wholly below every row
    of the block;
  * both wave groups of the two-group schedule pass the same number of
    barriers, and every tile of the range is scored and multiplied once;
  * cached launches read the index-map entries of the next K and V tiles one
    step ahead: every pipelined tile load must find the entries of that very
    tile in hand (read in the prologue or by the load of the tile before).

Schedules (constants as in the kernel): plain (2 buffers, K staged 2 tiles and
V 1 tile ahead, one barrier per tile), PAIR (4 buffers, 3 and 2 ahead, one
barrier per two tiles), PP (two wave groups one phase apart, 3 buffers), each
over key-tile counts 0..80 of plain and cached (prefix) blocks, and split-K
ranges (kMinSplitTiles = 4) for split counts 1..8 at every split index.
"""

import itertools
import math

import pytest

BN = 64
K_MIN_SPLIT_TILES = 4

SCHEDULES = {
    # name: (buffers, K ahead, V ahead, pair steps, two groups)
    "plain": (2, 2, 1, False, False),
    "pair": (4, 3, 2, True, False),
    "pp": (3, None, None, False, True),
}


class Replay:
    def __init__(self, sched, kshift, S, q0, bmp, n_split=1, split=0, ahead_skew=0):
        self.sched = sched
        self.ahead_skew = ahead_skew  # tests only: a wrong first read-ahead tile
        self.bufs, self.KA, self.VA, self.pair, self.pp = SCHEDULES[sched]
        self.NK = kshift + S
        self.n_all = math.ceil((kshift + min(q0 + bmp, S)) / BN)
        self.n_full = min((kshift + q0) // BN, self.n_all)
        self.t_lo, self.n_tiles = 0, self.n_all
        self.split = n_split > 1
        if self.split:
            eff = max(1, min(n_split, self.n_all // K_MIN_SPLIT_TILES))
            per = -(-self.n_all // eff)
            self.t_lo = min(split * per, self.n_all)
            self.n_tiles = min(self.t_lo + per, self.n_all)
        self.events = []  # (epoch, group, op, buf, slot, tile)
        self.loads = []   # (tile, clamped)
        self.full = []    # tiles scored / softmaxed without a mask
        self.barriers = {}
        self.scored = {}  # group -> tiles read from the K buffers by Q.K^T
        self.multiplied = {}
        self.ahead = {}   # (group, "K"/"V") -> tile whose map entries are held

    # --- map entries read ahead (cached launches)
    def _read_ahead(self, g, kind, t):
        self.ahead[(g, kind)] = t

    def _pipelined_load(self, g, kind, t, clamped):
        held = self.ahead.get((g, kind))
        assert held == t, f"{self.sched}: {kind} load of tile {t} with the map entries of tile {held}"
        self._load(t, clamped)
        self._read_ahead(g, kind, t + 1)

    def slot(self, t):
        if self.pp:
            return (t - self.t_lo) % 3
        if self.pair:
            return (t - self.t_lo) & 3
        return t & 1

    def run(self):
        if self.t_lo >= self.n_tiles:
            return self  # empty split: returns before any load or barrier
        if self.pp:
            for g in (0, 1):
                self._pp_group(g)
        else:
            self._plain(0)
        return self

    # --- the kernel's primitives
    def _load(self, t, clamped):
        self.loads.append((t, clamped))

    def _rw(self, e, g, op, buf, t):
        self.events.append((e, g, op, buf, self.slot(t), t))

    # --- run(): plain and PAIR
    def _plain(self, g):
        KA, VA, t_lo, n = self.KA, self.VA, self.t_lo, self.n_tiles
        e = 0
        k1, v1, k2 = t_lo + 1 < n, self.pair and t_lo + 1 < n, self.pair and t_lo + 2 < n
        self._load(t_lo, True)
        self._load(t_lo, True)
        for t, on in ((t_lo + 1, k1), (t_lo + 1, v1), (t_lo + 2, k2)):
            if on:
                self._load(t, True)
        self._read_ahead(g, "K", t_lo + KA + self.ahead_skew)
        self._read_ahead(g, "V", t_lo + VA)
        self._rw(e, g, "w", "K", t_lo)
        self._rw(e, g, "w", "V", t_lo)
        if k1:
            self._rw(e, g, "w", "K", t_lo + 1)
        if v1:
            self._rw(e, g, "w", "V", t_lo + 1)
        if k2:
            self._rw(e, g, "w", "K", t_lo + 2)
        e += 1
        self._rw(e, g, "r", "K", t_lo)
        self.scored.setdefault(g, []).append(t_lo)
        e += 1
        t_steady = min(self.n_full, n) if self.split else self.n_full

        def step(t, steady, bar):
            nonlocal e
            ld_k = steady or t + KA < n
            ld_v = steady or t + VA < n
            if ld_k:
                self._pipelined_load(g, "K", t + KA, not steady)
            if ld_v:
                self._pipelined_load(g, "V", t + VA, not steady)
            if steady:
                self.full.append(t)
            if steady or t + 1 < n:
                self._rw(e, g, "r", "K", t + 1)
                self.scored[g].append(t + 1)
                if steady:
                    self.full.append(t + 1)
            self._rw(e, g, "r", "V", t)
            self.multiplied.setdefault(g, []).append(t)
            if ld_k:
                self._rw(e, g, "w", "K", t + KA)
            if ld_v:
                self._rw(e, g, "w", "V", t + VA)
            if not self.pair or bar:
                e += 1

        t = t_lo
        while t + KA + 1 < t_steady:
            step(t, True, False)
            step(t + 1, True, True)
            t += 2
        while t < n:
            two = t + 1 < n
            step(t, False, not two)
            if two:
                step(t + 1, False, True)
            t += 2
        self.barriers[g] = e

    # --- run_pp(): group 0 leads, group 1 lags one phase
    def _pp_group(self, g):
        t_lo, n = self.t_lo, self.n_tiles
        e = 0
        regs = {"K": None, "V": None}
        self._load(t_lo, True)
        self._load(t_lo, True)
        if t_lo + 1 < n:
            self._load(t_lo + 1, True)
            self._load(t_lo + 1, True)
            regs["V"] = t_lo + 1
        if t_lo + 2 < n:
            self._load(t_lo + 2, True)
            regs["K"] = t_lo + 2
        self._read_ahead(g, "K", t_lo + 3 + self.ahead_skew)
        self._read_ahead(g, "V", t_lo + 2)
        self._rw(e, g, "w", "K", t_lo)
        self._rw(e, g, "w", "V", t_lo)
        if t_lo + 1 < n:
            self._rw(e, g, "w", "K", t_lo + 1)
        e += 1
        self._rw(e, g, "r", "K", t_lo)
        self.scored.setdefault(g, []).append(t_lo)
        if g == 1:
            e += 1
        t_steady = min(self.n_full, n) if self.split else self.n_full

        def vector(t, steady):
            if steady or t + 2 < n:
                assert regs["K"] == t + 2, ("K registers", regs["K"], t + 2)
                self._rw(e, g, "w", "K", t + 2)
            if steady or t + 1 < n:
                assert regs["V"] == t + 1, ("V registers", regs["V"], t + 1)
                self._rw(e, g, "w", "V", t + 1)
            if steady or t + 3 < n:
                self._pipelined_load(g, "K", t + 3, not steady)
                regs["K"] = t + 3
            if steady or t + 2 < n:
                self._pipelined_load(g, "V", t + 2, not steady)
                regs["V"] = t + 2
            if steady:
                self.full.append(t)

        def matrix(t, steady):
            self._rw(e, g, "r", "V", t)
            self.multiplied.setdefault(g, []).append(t)
            if steady or t + 1 < n:
                self._rw(e, g, "r", "K", t + 1)
                self.scored[g].append(t + 1)
                if steady:
                    self.full.append(t + 1)

        t = t_lo
        while t + 3 < t_steady:
            vector(t, True)
            e += 1
            matrix(t, True)
            e += 1
            t += 1
        while t < n:
            vector(t, False)
            e += 1
            matrix(t, False)
            e += 1
            t += 1
        if g == 0:
            e += 1
        self.barriers[g] = e

    # --- checks
    def check(self):
        n, t_lo = self.n_tiles, self.t_lo
        what = f"{self.sched} NK={self.NK} n_all={self.n_all} n_full={self.n_full} range=[{t_lo},{n})"
        for t, clamped in self.loads:
            assert t_lo <= t < n, f"{what}: load of tile {t} outside the range"
            if clamped:
                assert t * BN <= self.NK - 1, f"{what}: negative clamped row in tile {t}"
            else:
                assert (t + 1) * BN <= self.NK, f"{what}: unclamped tile {t} reaches past the last key"
        for t in self.full:
            assert t < self.n_full, f"{what}: tile {t} taken unmasked"
        if self.t_lo >= self.n_tiles:
            assert not self.events and not self.loads
            return
        assert len(set(self.barriers.values())) == 1, f"{what}: barrier counts {self.barriers}"
        for g in self.scored:
            assert sorted(self.scored[g]) == list(range(t_lo, n)), f"{what}: scored {self.scored[g]}"
            assert sorted(self.multiplied[g]) == list(range(t_lo, n)), f"{what}: multiplied {self.multiplied[g]}"
        # LDS: per (buffer, slot), the tile last written before each read's
        # interval is the tile read, and nothing is written in that interval.
        by_slot = {}
        for ev in self.events:
            by_slot.setdefault((ev[3], ev[4]), []).append(ev)
        for key, evs in by_slot.items():
            writes = [(e, t) for e, g, op, b, s, t in evs if op == "w"]
            for e, g, op, b, s, t in evs:
                if op != "r":
                    continue
                before = [(we, wt) for we, wt in writes if we < e]
                assert before, f"{what}: read of {b}{t} at {e} before any write"
                last = max(before)[1]
                assert last == t, f"{what}: read of {b}{t} at interval {e} finds tile {last}"
                same = [wt for we, wt in writes if we == e]
                assert not same, f"{what}: {b} slot {s} written ({same}) in the interval of a read of {t}"
            for (e1, t1), (e2, t2) in itertools.combinations(writes, 2):
                assert e1 != e2 or t1 == t2, f"{what}: two tiles written to {key} in one interval"


def _blocks(bmp, s_values, prefixes):
    for kshift in prefixes:
        for S in s_values:
            for qb in range(-(-S // bmp)):
                yield kshift, S, qb * bmp


S_VALUES = [1, 63, 64, 65, 200, 256, 511, 1000, 2048, 4096, 5000]
PREFIXES = [0, 1, 64, 700, 2047] + list(range(3, 5120, 97))


@pytest.mark.parametrize("sched", list(SCHEDULES))
def test_plain_and_cached_blocks(sched):
    bmp = 256 if sched != "plain" else 128
    counts = set()
    for kshift, S, q0 in _blocks(bmp, S_VALUES, PREFIXES):
        r = Replay(sched, kshift, S, q0, bmp).run()
        r.check()
        counts.add(r.n_all)
    assert set(range(1, 81)) <= counts, sorted(set(range(1, 81)) - counts)


@pytest.mark.parametrize("sched", ["plain", "pp", "pair"])
def test_split_ranges(sched):
    """Split-K runs the plain schedule (four-wave), PP (head_dim 128) and PAIR (eight-wave, 64 and 96)."""
    bmp = 128 if sched == "plain" else 256
    seen = set()
    for n_all in range(0, 81):
        for n_split in range(1, 9):
            for split in range(n_split):
                # a chunk of S tokens after a prefix: choose the prefix so the block has n_all tiles
                S = 100
                kshift = max(0, n_all * BN - S)
                r = Replay(sched, kshift, S, 0, bmp, n_split=n_split, split=split)
                if r.n_all != n_all:
                    continue
                r.run().check()
                seen.add((n_all, n_split, split))
    assert len({a for a, _, _ in seen}) >= 75


def test_replay_detects_a_wrong_bound():
    """A schedule with one buffer too few must fail the replay (the check is not vacuous)."""
    saved = SCHEDULES["pair"]
    SCHEDULES["pair"] = (4, 4, 2, True, False)  # K staged 4 ahead into 4 buffers
    try:
        with pytest.raises(AssertionError):
            for kshift, S, q0 in _blocks(256, [1000], [0]):
                Replay("pair", kshift, S, q0, 256).run().check()
    finally:
        SCHEDULES["pair"] = saved
    saved = SCHEDULES["plain"]
    try:
        SCHEDULES["plain"] = (2, 3, 1, False, False)
        with pytest.raises(AssertionError):
            Replay("plain", 0, 1000, 768, 128).run().check()
    finally:
        SCHEDULES["plain"] = saved
    for sched in SCHEDULES:  # a first read-ahead one tile off
        with pytest.raises(AssertionError):
            for kshift, S, q0 in _blocks(256, [1000], [0]):
                Replay(sched, kshift, S, q0, 256, ahead_skew=-1).run().check()


def test_replay_constants_match_the_kernel_source():
    """The replay's schedule table restates the kernel's constants; a change to
    either one alone must fail here (the replay would otherwise keep checking
    a schedule the kernel no longer runs)."""
    import pathlib
    import re
    src = (pathlib.Path(__file__).resolve().parents[1] / "rope_causal_attention_amd" / "csrc" /
           "attn_kernels.hip").read_text()

    def ternary(name):
        m = re.search(r"static constexpr int " + name + r" = (.+?);", src)
        assert m, name
        return m.group(1).replace(" ", "")

    assert ternary("kBufs") == "PP?3:(PAIR?4:2)"
    assert ternary("KA") == "PAIR?3:2"
    assert ternary("VA") == "PAIR?2:1"
    m = re.search(r"constexpr int kMinSplitTiles = (\d+);", src)
    assert m and int(m.group(1)) == K_MIN_SPLIT_TILES
    # the table: (buffers, K ahead, V ahead) of each schedule, from the same expressions
    pp, pair, plain = SCHEDULES["pp"], SCHEDULES["pair"], SCHEDULES["plain"]
    assert (plain[0], plain[1], plain[2]) == (2, 2, 1)
    assert (pair[0], pair[1], pair[2]) == (4, 3, 2)
    assert pp[0] == 3
    # the two-group schedule's look-ahead is spelled out in its phases: K(t+3), V(t+2)
    assert "next_k<!STEADY>(t + 3)" in src and "next_v<!STEADY>(t + 2)" in src
