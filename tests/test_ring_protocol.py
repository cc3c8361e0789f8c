"""A CPU model of the decoder's per-wave word ring (the bookkeeping of the
streaming kernels, restated step by step) run against random consumption
patterns, checking the properties the kernels rely on:
  * every word a renormalising lane reads sits in the ring slot it reads,
    and was issued before the last wait for the ring's loads;
  * every LDS read, including the don't-care reads of lanes that do not
    renormalise, stays inside the wave's 1,024-word ring;
  * a refill never overwrites a word that is still to be read;
  * with consistent input the words consumed equal the chunk's words; with
    corrupt input (more words consumed than exist) reads still stay inside.
Ring: word i at index i mod 768, the unit at index 0 mirrored at 768.."""
import numpy as np

UNIT, SPAN, BLOCK = 256, 768, 256
WORDS = SPAN + UNIT
LEAD = SPAN - UNIT


class Ring:
    def __init__(self, nw):
        self.nw = nw
        self.slot = np.full(WORDS, -1, np.int64)      # stream word held by each slot
        self.slot_issue = np.full(WORDS, -1, np.int64)  # fill number that wrote it
        self.fills = 0
        self.waited = 0                              # fills known landed
        self.pos, self.base = 0, 0                   # ring-relative position
        self.issued = 0
        while self.issued < nw and self.issued < LEAD:
            self.fill()
        self.waited = self.fills                     # vmcnt(0) at chunk start
        self.landed = self.issued
        self.horizon()

    def consumed(self):
        return self.base + self.pos

    def fill(self):
        at = self.issued % SPAN
        for dest in ([at, SPAN] if at == 0 else [at]):
            for k in range(UNIT):
                w = self.issued + k
                if w >= (self.nw + 7) // 8 * 8:
                    continue                          # lanes past the region do not load
                old = self.slot[dest + k]
                # overwriting a word still to be read would be a bug
                assert old < self.consumed() or old < 0 or old == w, (old, self.consumed())
                self.slot[dest + k] = w
                self.slot_issue[dest + k] = self.fills
        self.fills += 1
        self.issued += UNIT

    def horizon(self):
        a = 2**32 - 1 if self.landed >= self.nw else self.landed - BLOCK
        b = 2**32 - 1 if self.issued >= self.nw else self.issued - LEAD
        h = min(a, b) - self.base
        assert h >= 0
        self.hpos = min(h, SPAN - 1)

    def service(self):
        if self.pos >= SPAN:
            self.pos -= SPAN
            self.base += SPAN
        p = self.consumed()
        need_to = min(p + BLOCK, self.nw)
        if self.landed < need_to:
            self.waited = self.fills                 # vmcnt(1): all loads but the store
            self.landed = self.issued
        while self.issued < self.nw and self.issued < p + LEAD:
            self.fill()
        self.horizon()

    def step(self, need, valid=True):
        """One wave step: need[j] says lane j renormalises."""
        prefix = np.cumsum(need) - need
        for j in range(64):
            idx = self.pos + prefix[j]
            assert 0 <= idx < WORDS, idx                # inside the ring
            if need[j] and valid:
                want = self.consumed() + prefix[j]
                assert self.slot[idx] == want, (idx, self.slot[idx], want)
                assert self.slot_issue[idx] < self.waited  # landed
        self.pos += int(need.sum())


def run(nw, rng, rate, corrupt=False):
    r = Ring(nw)
    blocks = 0
    while r.consumed() < nw or (corrupt and blocks < 400):
        if r.pos > r.hpos:
            r.service()
        for _ in range(4):
            left = nw - r.consumed()
            if left <= 0 and not corrupt:
                break
            need = rng.random(64) < rate
            if not corrupt and need.sum() > left:
                need[np.flatnonzero(need)[left:]] = False
            r.step(need, valid=r.consumed() + need.sum() <= nw)
        blocks += 1
        if blocks > 100000:
            raise AssertionError("no progress")
    if not corrupt:
        assert r.consumed() == nw


def test_ring_protocol_holds_for_random_streams():
    rng = np.random.default_rng(17)
    for nw in [0, 1, 7, 8, 255, 256, 257, 511, 512, 513, 767, 768, 769, 1023, 1024, 1025,
               2000, 4096, 9000, 32768]:
        for rate in (0.02, 0.2, 0.6, 1.0):
            run(nw, rng, rate)


def test_ring_reads_stay_inside_on_corrupt_streams():
    rng = np.random.default_rng(18)
    for nw in [0, 100, 700, 3000]:
        run(nw, rng, 1.0, corrupt=True)
