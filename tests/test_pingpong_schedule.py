"""Host model of the ping-pong kernel's load schedule (gemm_kernel_pingpong.h):
the order of its loads, load waits, fragment reads and barriers, per wave
group, for the split-load schedule (group 0 loads A of tile t+1, group 1 B of
tile t+2; A in two LDS stages, B in three) and the one-loader schedule
(group 0 loads both operands of tile t+1 into two stages).  The checker
replays the events and asserts the two hazards the barriers and waits exist
for: no read of a tile before its loads have been waited for by the loading
group and a barrier has followed; no load into a stage before every read of
the tile that held it has been followed by a barrier.  It also rejects the
schedules one small change away from the kernel's (B in two stages, a missing
wait, loads one tile further ahead, group 0's wait moved past the barrier that
ends its compute phase), so the checks have teeth.

A group is four waves, and each loads a quarter of its tile; a wave's wait
covers its own loads only, while its fragment reads take every quarter.  So a
read is safe only after a barrier that follows the loading waves' waits, even
in the loading group: the checker counts a load as visible from the epoch
after its wait, never in the same epoch."""
import itertools

import pytest

# events: ("load", op, tile, stage), ("wait", keep) -- all but the `keep`
# most recent loads of this group are complete --, ("read", op, tile, stage),
# ("barrier",)


def split_schedule(KT, b_stages=3, b_ahead=2, group1_waits=True, g0_wait_after_barrier=False):
    """The split-load schedule as the kernel runs it; the keyword arguments
    plant the mistakes the tests expect to be caught (g0_wait_after_barrier:
    group 0 waits for A of tile t+1 at the start of M(t+1), just before its
    own first read, instead of before the barrier that ends C(t))."""
    a_st = lambda t: t % 2
    b_st = lambda t: t % b_stages
    g = {0: [], 1: []}
    # prologue: each group loads its operand of tiles 0 and 1, waits for tile 0
    for grp, op, st in ((0, "A", a_st), (1, "B", b_st)):
        for t in range(min(2, KT)):
            g[grp].append(("load", op, t, st(t)))
        g[grp].append(("wait", 1 if KT > 1 else 0))
        g[grp].append(("barrier",))                           # b = 0
    g[1].append(("barrier",))                                 # b = 1: group 1 starts one phase late
    for kt in range(KT):
        for grp in (0, 1):
            ev = g[grp]
            if grp == 0 and kt >= 1 and g0_wait_after_barrier:
                ev.append(("wait", 0))
            ev += [("read", "A", kt, a_st(kt)), ("read", "B", kt, b_st(kt))]
            if grp == 0 and kt >= 1 and kt + 1 < KT:
                ev.append(("load", "A", kt + 1, a_st(kt + 1)))
            loaded = grp == 1 and kt + b_ahead < KT
            if loaded:
                ev.append(("load", "B", kt + b_ahead, b_st(kt + b_ahead)))
            if grp == 1 and group1_waits:
                ev.append(("wait", 1 if loaded else 0))
            ev.append(("barrier",))                           # end of M(kt)
            if grp == 0:
                if not g0_wait_after_barrier:
                    ev.append(("wait", 0))                    # A of tile kt+1 landed
                ev.append(("barrier",))                       # end of C(kt)
            elif kt + 1 < KT:
                ev.append(("barrier",))
    return g


def one_loader_schedule(KT, stages=2):
    st = lambda t: t % stages
    g = {0: [], 1: []}
    for t in range(min(2, KT)):
        g[0] += [("load", "A", t, st(t)), ("load", "B", t, st(t))]
    g[0].append(("wait", 1 if KT > 1 else 0))
    g[0].append(("barrier",))
    g[1].append(("barrier",))
    g[1].append(("barrier",))
    for kt in range(KT):
        for grp in (0, 1):
            ev = g[grp]
            ev += [("read", "A", kt, st(kt)), ("read", "B", kt, st(kt))]
            if grp == 0 and kt >= 1 and kt + 1 < KT:
                ev += [("load", "A", kt + 1, st(kt + 1)), ("load", "B", kt + 1, st(kt + 1))]
            ev.append(("barrier",))
            if grp == 0:
                ev.append(("wait", 0))
                ev.append(("barrier",))
            elif kt + 1 < KT:
                ev.append(("barrier",))
    return g


def check(g, KT):
    """Replay a schedule; returns the list of hazards found (empty if none).

    Each group's events are numbered by barrier epoch (barriers passed so
    far); across groups only the epochs order events.  A wait makes a load
    'landed' in the epoch it runs in; another wave sees it from the next
    epoch on (after a barrier)."""
    nb = {grp: sum(1 for e in ev if e[0] == "barrier") for grp, ev in g.items()}
    problems = []
    if len(set(nb.values())) != 1:
        problems.append(f"barrier counts differ: {nb}")
    landed = {}        # (op, tile) -> epoch in which its loading group waited for it
    reads = {}         # (op, tile) -> list of epochs of its reads
    # the groups' events by epoch, replayed epoch by epoch
    per_epoch = {grp: [] for grp in g}
    for grp, ev in g.items():
        epoch, loads = 0, []
        for e in ev:
            if e[0] == "barrier":
                epoch += 1
                continue
            per_epoch[grp].append((epoch, e))
            if e[0] == "load":
                loads.append((e[1], e[2]))
            elif e[0] == "wait":
                done = loads if e[1] == 0 else loads[:-e[1]]
                for key in done:
                    landed.setdefault(key, epoch)
    for grp, evs in per_epoch.items():
        for epoch, e in evs:
            if e[0] == "read":
                key = (e[1], e[2])
                reads.setdefault(key, []).append(epoch)
                if key not in landed or landed[key] >= epoch:
                    problems.append(f"group {grp} reads {key} in epoch {epoch} before it has landed "
                                    f"(landed in {landed.get(key)})")
    for grp, evs in per_epoch.items():
        for epoch, e in evs:
            if e[0] == "load":
                op, t, st = e[1], e[2], e[3]
                old = [tt for tt in range(t) if (op, tt) in reads and _stage(g, op, tt) == st]
                for tt in old:
                    late = [r for r in reads[(op, tt)] if r >= epoch]
                    if late:
                        problems.append(f"group {grp} loads {op}{t} into stage {st} in epoch {epoch} "
                                        f"while {op}{tt} is still read there (epochs {late})")
    for op, t in itertools.product("AB", range(KT)):
        if (op, t) not in reads:
            problems.append(f"{op}{t} never read")
    return problems


def _stage(g, op, t):
    for ev in g.values():
        for e in ev:
            if e[0] in ("load", "read") and e[1] == op and e[2] == t:
                return e[3]
    return None


@pytest.mark.parametrize("KT", range(1, 9))
def test_split_load_schedule_is_hazard_free(KT):
    assert check(split_schedule(KT), KT) == []


@pytest.mark.parametrize("KT", range(1, 9))
def test_one_loader_schedule_is_hazard_free(KT):
    assert check(one_loader_schedule(KT), KT) == []


def test_split_loads_need_a_third_b_stage():
    probs = check(split_schedule(6, b_stages=2), 6)
    assert any("still read there" in p for p in probs), probs


def test_group1_must_wait_for_its_loads():
    probs = check(split_schedule(6, group1_waits=False), 6)
    assert any("before it has landed" in p for p in probs), probs


def test_b_loads_three_tiles_ahead_overwrite_a_live_stage():
    probs = check(split_schedule(7, b_ahead=3), 7)
    assert any("still read there" in p for p in probs), probs


def test_group0_wait_must_precede_the_barrier_before_its_own_reads():
    """Moving group 0's wait off its compute phase, to just before its own
    reads, leaves the other waves' quarters of the tile unsynchronised."""
    probs = check(split_schedule(6, g0_wait_after_barrier=True), 6)
    assert any(p.startswith("group 0 reads ('A', 1)") for p in probs), probs


def test_one_loader_with_one_stage_is_rejected():
    probs = check(one_loader_schedule(5, stages=1), 5)
    assert probs, "a single stage must conflict"
