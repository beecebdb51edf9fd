"""Host model of the ring pipeline's task schedule (no GPU).

One launch of the ring kernel holds three kinds of task: row copies of the
next minibatch, UP tiles of the current one and DOWN tiles of the previous
one.  Its workgroups take them as the kernel does:
  * with mover workgroups, workgroup b < movers takes the copies b,
    b + movers, ...;
  * the other tasks are cut into eight runs, run x holding the x-th eighth of
    the UP tiles, then of the DOWN tiles, then (without movers) of the
    copies; a workgroup on XCD b % 8 takes positions of run b % 8 from that
    run's counter, then of the next runs in turn, until all eight are
    exhausted;
  * every workgroup, once done, adds one to a finish counter; the one that
    brings it to the workgroup count sets all nine counters back to zero.
This model replays that protocol with the 256 workgroups interleaved in a
seeded random order at every counter access, and checks what the kernel
relies on: every task runs exactly once, a run hands out its longest tasks
first, every workgroup ends, and the counters are zero for the next launch.
A counter that is not zeroed, a run cut that drops or repeats a task, or a
finish test that fires early fails one of these.
"""
import random

import pytest

G = 256          # workgroups of a ring launch (one per CU)
NCTR = 9         # eight run counters and the finish counter


def _cut(n, x):
    return (n * x) >> 3


def _plan(n_cp, n_up, n_dn, movers):
    """Per run x, the task indices in the order the run hands them out
    (task index: copies [0, n_cp), UP [n_cp, n_cp + n_up), DOWN after)."""
    n_rcp = 0 if movers else n_cp
    runs = []
    for x in range(8):
        up = [n_cp + t for t in range(_cut(n_up, x), _cut(n_up, x + 1))]
        dn = [n_cp + n_up + t for t in range(_cut(n_dn, x), _cut(n_dn, x + 1))]
        cp = list(range(_cut(n_rcp, x), _cut(n_rcp, x + 1)))
        runs.append(up + dn + cp)
    return runs


def _launch(n_cp, n_up, n_dn, movers, ctr, rng):
    """One launch: returns the multiset of executed tasks; mutates ctr."""
    runs = _plan(n_cp, n_up, n_dn, movers)
    done = []
    # each workgroup is a generator that yields before every counter access
    def wg(b):
        if b < movers:
            for t in range(b, n_cp, movers):
                done.append(t)
        else:
            x = b % 8
            for _ in range(8):
                while True:
                    yield
                    v = ctr[x]
                    ctr[x] += 1
                    if v >= len(runs[x]):
                        break
                    done.append(runs[x][v])
                x = (x + 1) % 8
        yield
        fin = ctr[8]
        ctr[8] += 1
        if fin == G - 1:
            for i in range(NCTR):
                ctr[i] = 0
    live = {b: wg(b) for b in range(G)}
    steps = 0
    while live:
        b = rng.choice(list(live))
        try:
            next(live[b])
        except StopIteration:
            del live[b]
        steps += 1
        assert steps < 10 * (G + n_cp + n_up + n_dn) * 9, "a workgroup never ends"
    return done


@pytest.mark.parametrize("seed", range(6))
def test_every_task_once_and_counters_left_zero(seed):
    rng = random.Random(seed)
    ctr = [0] * NCTR
    # several launches in a row on the same counters, as one chain of the
    # pipeline uses them: minibatch shapes of the training routing (R = 512 ..
    # 2048: tens to hundreds of tasks) and edge cases (no task of a kind, fewer
    # tasks than runs, one workgroup left for the tiles)
    shapes = [(32, 72, 64, 0), (64, 120, 96, 0), (128, 216, 160, 0), (0, 0, 0, 0), (1, 0, 0, 0),
              (0, 3, 0, 0), (5, 7, 2, 0), (64, 120, 96, 32), (64, 120, 96, 255), (3, 1, 1, 8), (0, 200, 0, 1)]
    for n_cp, n_up, n_dn, movers in shapes + [tuple(rng.randrange(0, 300) for _ in range(3)) + (0,)]:
        done = _launch(n_cp, n_up, n_dn, movers, ctr, rng)
        assert sorted(done) == list(range(n_cp + n_up + n_dn)), (n_cp, n_up, n_dn, movers)
        assert ctr == [0] * NCTR, "counters not zero for the next launch"


def test_runs_hand_out_longest_tasks_first():
    for n_cp, n_up, n_dn in [(64, 120, 96), (7, 9, 30), (100, 3, 5)]:
        for run in _plan(n_cp, n_up, n_dn, 0):
            kinds = [0 if t >= n_cp and t < n_cp + n_up else 1 if t >= n_cp + n_up else 2 for t in run]
            assert kinds == sorted(kinds), "a run hands out UP tiles, then DOWN tiles, then copies"


def test_a_stale_counter_is_caught():
    """The model's checks are not vacuous: a launch that starts from a
    counter left non-zero loses tasks."""
    rng = random.Random(3)
    ctr = [0] * NCTR
    ctr[2] = 1
    done = _launch(64, 120, 96, 0, ctr, rng)
    assert sorted(done) != list(range(64 + 120 + 96))
