"""A CPU model of the window-slot kernel's hand-over protocol (host logic, no GPU).

The kernel gives each channel kSlots = 3 waves; slot k takes windows k, k + 3, k + 6, ... and at
its step s works on position q = s - k D (pair np = q mod Ns of its r-th window, r = q div Ns).
Before reading the carried states of a pair (a window w > 0) it waits until the wave of the
previous slot has published s - D + 1 completed steps (slot 0: s - Ns + 2 D + 1, from the last
slot of the round before); it reads the pair's carried word, later writes the pair's end state
into the same word, and publishes s + 1 at the end of the step.

The model runs the three waves as interleaved state machines, choosing at random which runnable
wave moves next (so also orders far from the kernel's usual lockstep), and checks what the
kernel's comments claim: every read of a carried word sees the value written by the window just
before (never an older or a newer one), no wave ever waits for a step that can no longer come
(the walk always completes), and the number of steps the launch computes covers every window.
"""
import random

import pytest

KSLOTS = 3


def launch_params(N, L, W=1024):
    """Steps per window (two states a step), skew, windows and steps per slot, as launched."""
    ns = (N + 1) // 2
    skew = max(1, ns // 3)
    nwin = (L + W - 1) // W
    steps = 0
    for k in range(min(KSLOTS, nwin)):
        windows = (nwin - k + KSLOTS - 1) // KSLOTS
        steps = max(steps, windows * ns + k * skew)
    return ns, skew, nwin, steps


def simulate(N, L, seed, bias=None, fewer_steps=0, early=0):
    """Run the protocol with random interleavings (`bias`: a slot favoured 9 times in 10;
    `early`: a wait that accepts a published count that many steps short, a planted error)."""
    ns, skew, nwin, nsteps = launch_params(N, L)
    nsteps -= fewer_steps
    rng = random.Random(seed)
    prog = [0] * KSLOTS                 # steps each slot has published
    word = {}                           # pair -> (window that wrote it)
    seen = {}                           # (window, pair) -> window whose end state it read
    done_pairs = set()
    # per wave: current step and phase (0 wait/read, 1 write, 2 publish)
    state = [[0, 0] for _ in range(KSLOTS)]

    def position(k, s):
        q = s - k * skew
        if q < 0:
            return None
        r, np = divmod(q, ns)
        w = r * KSLOTS + k
        return (w, np) if w < nwin else None

    def runnable(k):
        s, ph = state[k]
        if s >= nsteps:
            return False
        if ph != 0:
            return True
        pos = position(k, s)
        if pos is None or pos[0] == 0:
            return True
        src = s - skew if k else s - ns + (KSLOTS - 1) * skew
        return prog[(k + KSLOTS - 1) % KSLOTS] >= src + 1 - early

    while True:
        ready = [k for k in range(KSLOTS) if runnable(k)]
        if not ready:
            break
        k = ready[0] if bias is not None and bias in ready and rng.random() < 0.9 else rng.choice(ready)
        s, ph = state[k]
        pos = position(k, s)
        if ph == 0:
            if pos is not None:
                w, np = pos
                # the carried word: the previous window's end state (or the initial state)
                seen[(w, np)] = word.get(np, -1) if w > 0 else -1
            state[k][1] = 1
        elif ph == 1:
            if pos is not None:
                w, np = pos
                word[np] = w
                done_pairs.add((w, np))
            state[k][1] = 2
        else:
            prog[k] = s + 1
            state[k] = [s + 1, 0]
    return ns, skew, nwin, nsteps, state, seen, done_pairs


@pytest.mark.parametrize("N,L", [(5, 3 * 1024), (6, 4096 + 8), (16, 5 * 1024 + 264), (16, 40 * 1024 + 8),
                                 (17, 6 * 1024 + 8), (64, 3 * 1024 + 1000), (128, 4 * 1024), (33, 7 * 1024)])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_every_window_reads_the_window_before(N, L, seed):
    ns, skew, nwin, nsteps, state, seen, done = simulate(N, L, seed, bias=seed % KSLOTS if seed else None)
    assert 1 <= skew <= (ns - 1) // 2
    # the walk completed: every wave ran all its steps, and every (window, pair) was computed
    assert all(s == nsteps for s, _ in state), state
    assert done == {(w, np) for w in range(nwin) for np in range(ns)}
    # each pair of window w > 0 read exactly window w - 1's end state; window 0 the initial one
    for (w, np), src in seen.items():
        assert src == w - 1, (w, np, src)


def test_launch_steps_are_tight():
    """The launch's step count is the least that computes every window: one step fewer leaves
    the last window's last pair undone."""
    for N in (5, 16, 128):
        for L in (3 * 1024, 4 * 1024 + 8, 10 * 1024):
            ns, skew, nwin, nsteps, state, seen, done = simulate(N, L, 0, fewer_steps=1)
            assert len(done) == nwin * ns - 1, (N, L)


def test_a_broken_wait_is_caught():
    """The model has teeth: with a wait that accepts the previous slot's count one step short,
    some window reads a stale carried word."""
    stale = 0
    for seed in range(20):
        _, _, _, _, _, seen, _ = simulate(16, 12 * 1024, seed, early=1)
        stale += sum(src != w - 1 for (w, _), src in seen.items())
    assert stale > 0
