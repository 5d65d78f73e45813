"""Host-side models of chunk-claim protocols (tests/claim_model.py).

The epoch-tagged fetch-add / compare-and-swap claim that an earlier
dynamic-chunk variant of the decode stream used never finished on the GPU.
Modelled step by step, it livelocks under a fair schedule: every retry's
fetch-add invalidates the other waves' pending compare-and-swap, no wave ever
installs the epoch, and the stale low word counts up until it carries into the
epoch field. Under random schedules its chance to finish falls as waves are
added. The work-group-local counter the decode stream uses instead (zeroed
before the work-group's waves start, one fetch-add per claim) hands out every
chunk exactly once and ends after chunks + waves operations under any
schedule, checked exhaustively for small cases."""

import itertools

import numpy as np

from tests import claim_model as cm


def _waves(claim, n, chunks):
    return [cm.Wave(claim, chunks) for _ in range(n)]


def test_epoch_claim_livelocks_under_a_fair_schedule():
    for n in (2, 3, 8):
        stale = (7 << 32) | 5                      # an earlier call's epoch 7
        word = cm.Word(stale)
        waves = _waves(lambda: cm.epoch_fetch_cas_claim(9), n, chunks=4)
        finished = cm.run(waves, word, cm.staggered_schedule(n), max_ops=20000)
        assert not finished
        assert all(w.got == [] for w in waves), "no wave may claim anything"
        assert word.value >> 32 == 7, "the epoch is never installed"
        assert (word.value & cm.MASK32) > 5000, "the stale low word keeps counting up"


def test_epoch_claim_low_word_carries_into_the_epoch_field():
    word = cm.Word((7 << 32) | (cm.MASK32 - 3))
    waves = _waves(lambda: cm.epoch_fetch_cas_claim(9), 2, chunks=4)
    cm.run(waves, word, cm.staggered_schedule(2), max_ops=100)
    assert word.value >> 32 == 8, "the carry moved the epoch field to 8"


def test_epoch_claim_stops_finishing_when_round_trips_are_long():
    """With a round trip of a few operations (one or two waves) the protocol
    finishes; with dozens of waves whose round trips span tens of other
    operations, as on a GPU, it practically never does."""
    rng = np.random.default_rng(0)

    def rate(n, lo, hi, trials=30):
        ok = 0
        for _ in range(trials):
            word = cm.Word((3 << 32) | 11)
            waves = _waves(lambda: cm.epoch_fetch_cas_claim(4), n, chunks=2 * n)
            ok += cm.run(waves, word, cm.latency_schedule(n, rng, lo, hi), max_ops=200 * n)
        return ok / trials

    assert rate(2, 0, 1) == 1.0
    assert rate(64, 20, 40) == 0.0


def test_local_counter_claims_every_chunk_once_under_every_schedule():
    """Exhaustive over all interleavings for 2 and 3 waves."""
    for n, chunks in ((2, 3), (3, 2)):
        total = chunks + n                          # each wave's last claim fails
        for order in itertools.product(range(n), repeat=total):
            word = cm.Word(0)
            waves = _waves(cm.local_counter_claim, n, chunks)
            cm.run(waves, word, iter(order), max_ops=total)
            if not all(w.done for w in waves):
                continue                            # the order starved a wave: not complete
            got = sorted(c for w in waves for c in w.got)
            assert got == list(range(chunks))
            assert word.ops == total
            for w in waves:
                assert w.got == sorted(w.got), "a wave's claims increase"


def test_local_counter_ends_under_adversarial_and_random_schedules():
    rng = np.random.default_rng(1)
    for n, chunks in ((8, 40), (12, 7), (8, 0)):
        for sched in (cm.staggered_schedule(n), cm.random_schedule(n, rng)):
            word = cm.Word(0)
            waves = _waves(cm.local_counter_claim, n, chunks)
            assert cm.run(waves, word, sched, max_ops=10 * (chunks + n) + 100)
            got = sorted(c for w in waves for c in w.got)
            assert got == list(range(chunks))
            assert word.ops == chunks + n
