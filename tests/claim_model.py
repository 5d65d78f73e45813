"""Step-by-step model of chunk-claim protocols for a persistent decode grid
(test infrastructure: host-side models only, nothing here runs on a GPU).

Each wave is a Python generator that yields one atomic operation at a time
on a shared 64-bit word and receives the value the operation returned, so a
scheduler chooses the interleaving. Operations:

    ("add", n)            fetch-and-add, returns the old value
    ("cas", expect, new)  compare-and-swap, returns the old value

Protocols:

* ``epoch_fetch_cas_claim`` -- a chunk counter tagged with the call's epoch in
  its high 32 bits, so that no reset is needed between calls. A wave
  fetch-adds 1; if the old value carries this call's epoch, its low word is
  the claimed chunk. Otherwise the word is stale (left by an earlier call) and
  the wave tries to install (epoch, 1) with a compare-and-swap that expects
  exactly old + 1, claiming chunk 0; when that fails it starts over, with a new
  fetch-add. Every retry's fetch-add moves the word, which makes the
  expectation of every other wave's pending compare-and-swap wrong, so waves
  can keep failing each other indefinitely (a livelock), and the stale low
  word keeps counting up and eventually carries into the epoch field.

* ``local_counter_claim`` -- the protocol the decode stream uses: the chunk
  counter lives in the work-group's LDS, is zeroed when the work-group starts
  (before its waves begin), and a claim is one fetch-add. Claims are distinct
  and increasing, a wave stops at its first claim past the chunk count, and
  every wave ends after at most chunks + 1 operations, under any schedule.
"""

MASK32 = (1 << 32) - 1
MASK64 = (1 << 64) - 1


def epoch_fetch_cas_claim(epoch):
    """Claim one chunk index; returns it (the generator's return value)."""
    while True:
        old = yield ("add", 1)
        if (old >> 32) == epoch:
            return old & MASK32
        expect = (old + 1) & MASK64
        prev = yield ("cas", expect, (epoch << 32) | 1)
        if prev == expect:
            return 0


def local_counter_claim():
    old = yield ("add", 1)
    return old


class Word:
    def __init__(self, value):
        self.value = value & MASK64
        self.ops = 0

    def apply(self, op):
        self.ops += 1
        old = self.value
        if op[0] == "add":
            self.value = (old + op[1]) & MASK64
        elif op[0] == "cas":
            if old == op[1]:
                self.value = op[2] & MASK64
        else:
            raise ValueError(op)
        return old


class Wave:
    """A wave that claims chunks with ``claim`` until a claim reaches
    ``chunks``; records the chunks it got."""

    def __init__(self, claim, chunks):
        self.claim = claim
        self.chunks = chunks
        self.got = []
        self.done = False
        self._gen = None
        self._pending = None
        self._start()

    def _start(self):
        self._gen = self.claim()
        self._pending = next(self._gen)

    def pending(self):
        return self._pending

    def step(self, word):
        """Apply this wave's pending operation; returns True when it finished."""
        result = word.apply(self._pending)
        try:
            self._pending = self._gen.send(result)
        except StopIteration as stop:
            idx = stop.value
            if idx >= self.chunks:
                self.done = True
                return True
            self.got.append(idx)
            self._start()
        return False


def run(waves, word, schedule, max_ops):
    """Drive ``waves`` by ``schedule`` (an iterator of wave indices; finished
    waves are skipped) for at most ``max_ops`` operations. Returns True when
    every wave finished."""
    for i in schedule:
        if word.ops >= max_ops:
            return False
        if all(w.done for w in waves):
            return True
        w = waves[i]
        if not w.done:
            w.step(word)
    return all(w.done for w in waves)


def staggered_schedule(n_waves):
    """A fair schedule: one opening operation per wave, then every wave gets
    two operations per turn, in turn (0, 1, 0, 0, 1, 1, 0, 0, ... for two
    waves). Each wave's compare-and-swap then always follows another wave's
    fetch-add."""
    yield from range(n_waves)
    while True:
        for i in range(n_waves):
            yield i
            yield i


def random_schedule(n_waves, rng):
    while True:
        yield int(rng.integers(0, n_waves))


def latency_schedule(n_waves, rng, lat_lo, lat_hi):
    """Memory applies one operation per tick, oldest ready wave first; a wave
    is ready again lat_lo..lat_hi ticks after its operation was applied (its
    round trip), so between a wave's two operations about that many operations
    of other waves are applied. Waves start at random times within one round
    trip."""
    ready = [int(rng.integers(0, lat_hi + 1)) for _ in range(n_waves)]
    t = 0
    while True:
        i = min(range(n_waves), key=lambda k: (ready[k], k))
        t = max(t, ready[i]) + 1
        ready[i] = t + int(rng.integers(lat_lo, lat_hi + 1))
        yield i

