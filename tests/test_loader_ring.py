"""Model of the MQA kernel's loader ring (decode_mqa.hip), checked on the CPU.

The loaders keep S phases in flight in registers: phase i (K tile i/2 for
even i, V^T tile i/2 for odd i) lives in stage i % S.  Start-up loads phases
0 .. S-1 from the first ceil(S/2) tiles; after phase 0 is published, stage 0
is refilled with phase S, clamped to the last phase of the same K/V parity
when the split is shorter.  Step q publishes phase q+1 and refills its stage
with phase q+1+S while that is in range.  The rules below are the kernel's;
the test checks that every phase of a split is published exactly once, in
order, from a stage that holds that phase, and that every block-id index
stays inside its array, for every phase count the ring may be built with.
"""

import pytest


def run_ring(stages, ntiles):
    nphase = 2 * ntiles
    first_tiles = (stages + 1) // 2
    ring = [None] * stages
    published = []

    def store(ph, st):
        if ph >= nphase:
            return
        assert ring[st] == ph, f"stage {st} holds phase {ring[st]}, publishing {ph}"
        published.append(ph)

    def load_cached(ph, st):
        assert 0 <= ph // 2 < ntiles, f"block-id index {ph // 2} outside {ntiles} tiles"
        ring[st] = ph

    for ph in range(stages):
        assert ph // 2 < first_tiles
        ring[ph] = ph
    store(0, 0)
    load_cached(min(stages, nphase - 2 + (stages & 1)), 0)

    def step(i, q, more):
        st = (i + 1) % stages
        store(q + 1, st)
        if more:
            load_cached(q + 1 + stages, st)

    q = 0
    while q + 2 * stages < nphase:
        for i in range(stages):
            step(i, q + i, True)
        q += stages
    while q < nphase:
        for i in range(stages):
            if q + i < nphase:
                step(i, q + i, q + i + 1 + stages < nphase)
        q += stages
    return published


@pytest.mark.parametrize("stages", [2, 3, 4, 5, 6, 7, 8])
def test_every_phase_published_once_in_order(stages):
    for ntiles in range(1, 80):
        assert run_ring(stages, ntiles) == list(range(2 * ntiles))


def test_clamp_without_parity_fails_for_odd_counts():
    """The parity term of the clamp matters: clamping to the last K phase
    would publish a K copy as the V phase of a three-phase ring's last tile."""
    nphase, stages = 4, 3
    assert min(stages, nphase - 2) % 2 != stages % 2
    assert min(stages, nphase - 2 + (stages & 1)) % 2 == stages % 2
