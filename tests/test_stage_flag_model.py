"""Model check of the stage-flag hand-off (the FusedMerge layout: one full and
one empty arrive counter per ring stage), run on the CPU.

Each wave of a workgroup is a straight-line program of the actions the kernel's
flag form performs (issue a stage's loads, arrive on full, wait for full, read,
release, wait for empty), over several tiles with a workgroup barrier between
them. Every interleaving of the waves is explored. The check: no deadlock, no
wave reads a stage before every loading wave's data of that use is in, and no
wave overwrites a stage before every wave has released its previous use. A
protocol with a wrong count or a missing wait must be caught, which pins the
checker itself.

This is a model written from the description of the protocol, not the device
code: the device code's counts are what the GPU tests exercise.
"""
from __future__ import annotations

import itertools

import pytest

STAGES = 2


def wave_program(wave, tiles, waves, protocol):
    """Action list of one wave. `tiles` is a list of (nk, loaders): k-tiles of the
    tile and how many waves (the first `loaders`) load its stages."""
    unit = waves
    uses = [0] * STAGES
    prog = []
    for t, (nk, loaders) in enumerate(tiles):
        loads = wave < loaders
        share = unit // loaders
        use = lambda kt: uses[kt % STAGES] + kt // STAGES  # noqa: E731
        if nk > 0:
            if loads:
                prog.append(("issue", kt_stage(0), use(0)))
                prog.append(("arrive_full", kt_stage(0), share))
            prog.append(("wait_full", kt_stage(0), unit * (use(0) + 1) + protocol.get("full_slack", 0)))
            if nk > 1 and loads:
                prog.append(("issue", kt_stage(1), use(1)))
            prog.append(("read", kt_stage(0), use(0)))
            for kt in range(nk):
                prog.append(("read", kt_stage(kt), use(kt)))
                if not protocol.get("no_release"):
                    prog.append(("release", kt_stage(kt), 1))
                if kt + 1 < nk:
                    if loads:
                        prog.append(("arrive_full", kt_stage(kt + 1), share))
                    prog.append(("wait_full", kt_stage(kt + 1), unit * (use(kt + 1) + 1)))
                    if kt + 2 < nk and loads:
                        if not protocol.get("no_empty_wait"):
                            prog.append(("wait_empty", kt_stage(kt), unit * (use(kt) + 1)))
                        prog.append(("issue", kt_stage(kt + 2), use(kt + 2)))
                    prog.append(("read", kt_stage(kt + 1), use(kt + 1)))
        uses[0] += (nk + 1) // 2
        uses[1] += nk // 2
        prog.append(("barrier", t, 0))
    return prog


def kt_stage(kt):
    return kt % STAGES


def check(tiles_for_wave, waves, protocol=None):
    """Explore every interleaving; return the first problem found, or None."""
    protocol = protocol or {}
    progs = [wave_program(w, tiles_for_wave, waves, protocol) for w in range(waves)]
    seen = set()
    stack = [tuple([0] * waves)]
    while stack:
        pcs = stack.pop()
        if pcs in seen:
            continue
        seen.add(pcs)
        # counter values and stage contents follow from the executed prefixes
        full = [0] * STAGES
        empty = [0] * STAGES
        written = {}  # (stage, use) -> waves that issued it
        for w, pc in enumerate(pcs):
            for (op, s, x) in progs[w][:pc]:
                if op == "arrive_full":
                    full[s] += x
                elif op == "release":
                    empty[s] += x
                elif op == "issue":
                    written.setdefault((s, x), set()).add(w)
        moved = False
        for w, pc in enumerate(pcs):
            if pc == len(progs[w]):
                continue
            op, s, x = progs[w][pc]
            if op == "wait_full" and full[s] < x:
                continue
            if op == "wait_empty" and empty[s] < x:
                continue
            if op == "barrier" and any(
                    p2 < len(progs[w2]) and progs[w2][p2] != ("barrier", s, 0) for w2, p2 in enumerate(pcs)):
                continue
            if op == "read":
                loaders = {w2 for w2 in range(waves) for (o, s2, u) in progs[w2] if o == "issue" and (s2, u) == (s, x)}
                if written.get((s, x), set()) != loaders:
                    return f"wave {w} reads stage {s} use {x} before all its loads are in"
                if any(u > x for (s2, u) in written if s2 == s):
                    return f"wave {w} reads stage {s} use {x} after it was overwritten"
            if op == "issue" and x > 0:
                # every wave must have released the previous use of the stage
                need = waves * x
                if empty[s] < need:
                    return f"wave {w} overwrites stage {s} (use {x}) before every wave released use {x - 1}"
            nxt = list(pcs)
            if op == "barrier":
                nxt = [p2 + 1 if p2 < len(progs[w2]) and progs[w2][p2] == ("barrier", s, 0) else p2
                       for w2, p2 in enumerate(pcs)]
            else:
                nxt[w] += 1
            stack.append(tuple(nxt))
            moved = True
        if not moved and any(pc < len(progs[w]) for w, pc in enumerate(pcs)):
            return f"deadlock at {pcs}"
    return None


CASES = [
    # (waves, tiles as (k-tiles, loading waves))
    (2, [(1, 2), (3, 2)]),
    (2, [(4, 1), (2, 2)]),
    (4, [(3, 2), (2, 4), (1, 2)]),
    (4, [(4, 4), (4, 2)]),
    (3, [(2, 3), (5, 3)]),
]


@pytest.mark.parametrize("waves,tiles", CASES)
def test_protocol_is_safe_and_live(waves, tiles):
    assert check(tiles, waves) is None


@pytest.mark.parametrize("mutation,fragment", [
    ({"no_empty_wait": True}, "overwrites"),
    ({"no_release": True}, "deadlock"),
    ({"full_slack": 1}, "deadlock"),
])
def test_broken_protocols_are_caught(mutation, fragment):
    problems = [check(tiles, waves, mutation) for waves, tiles in CASES]
    assert any(p is not None and fragment in p for p in problems), problems


def test_every_use_adds_the_same_count():
    # both full (split over the loading waves) and empty (one per wave) grow
    # by exactly `waves` per use of a stage, whatever the number of loaders
    for waves, tiles in CASES:
        for (nk, loaders) in tiles:
            assert waves % loaders == 0
            assert loaders * (waves // loaders) == waves
    for waves, loaders in itertools.product([2, 4, 8], [1, 2, 4, 8]):
        if loaders <= waves and waves % loaders == 0:
            assert loaders * (waves // loaders) == waves
