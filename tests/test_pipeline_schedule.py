"""Host model of the fused kernels' LDS staging schedules.

The fused forward kernels stream K and V tiles into rings of LDS stages with
direct global-to-LDS copies that every wave of a workgroup shares.  A stage
may be read only after the copy that fills it has completed in every wave and
the workgroup has synchronised (a wait for the copies, then a barrier), and
it may be refilled only after a barrier that follows every read of its
previous tile.  All waves run the same program, so both rules can be checked
on the program order alone: the events below are the ones the kernels issue,
iteration by iteration, in the order the kernels issue them (copies at the
top of an iteration, the LDS reads of its products, the wait and barrier at
its bottom).

A wait may leave the newest copies in flight (the vector-memory counter
counts down in issue order): (WAIT, keep) completes every copy but the last
`keep`.  Every copy must also be complete before the workgroup ends.

Each schedule is checked for every tile count from 1 to 64, and a schedule
with one barrier too few must fail the same check.
"""
import pytest

COPY, READ, WAIT, BARRIER = "copy", "read", "wait", "barrier"


def fused16_events(nt, stages=4, k_ahead=3, v_ahead=1, barrier_every=2, keep=0):
    """fa_fwd_16_kernel: K tile t lives in K stage t % stages and is copied in
    iteration t - k_ahead; V tile t in V stage t % stages, copied in iteration
    t - v_ahead.  Iteration j reads V_{j-1} (P V of the previous tile) and
    K_{j+1} (scores of the next); it closes with a wait and a barrier when
    (j + 1) % barrier_every == 0 (after every odd iteration for 2).  The last
    iteration reads V_{j-1}, waits and synchronises, then reads V_j.  The
    waits of iteration 0 and of the loop leave the `keep` newest copies in
    flight; the prologue's and the last iteration's wait for every copy.
    fa_fwd_16_stream_kernel (queries shorter than one tile) runs v_ahead=2,
    barrier_every=1, keep=3: V two tiles ahead, and across each barrier the
    iteration's K and V copies and the previous iteration's V copy stay in
    flight."""
    ev = []

    def copy(buf, t):
        ev.append((COPY, buf, t % stages, t))

    def read(buf, t):
        ev.append((READ, buf, t % stages, t))

    def sync(k=0):
        ev.extend([(WAIT, k), (BARRIER,)])

    # prologue: K_0 .. K_{k_ahead-1} and V_0 .. V_{v_ahead-1}, then scores_0
    for t in range(k_ahead):
        copy("K", t)
    for t in range(v_ahead):
        copy("V", t)
    sync()
    read("K", 0)
    if nt == 1:
        sync()
        read("V", 0)
        return ev
    # iteration 0: copies K_{k_ahead}, V_{v_ahead}; scores_1; bottom
    copy("K", k_ahead)
    copy("V", v_ahead)
    read("K", 1)
    sync(keep)
    for j in range(1, nt - 1):
        copy("K", j + k_ahead)
        copy("V", j + v_ahead)
        read("V", j - 1)
        read("K", j + 1)
        if (j + 1) % barrier_every == 0:
            sync(keep)
    j = nt - 1
    read("V", j - 1)
    sync()
    read("V", j)
    return ev


def fp8_events(nt, drop_refill_barrier=False):
    """fa_fwd_fp8_kernel: two K and two V stages.  The prologue copies K_0 and
    K_1, waits and synchronises, computes scores_0 from K stage 0 and
    synchronises again (K stage 0 is refilled in iteration 0).  Iteration j
    (stage parity P = j % 2) copies K_{j+2} into K stage P and V_j into V
    stage P, reads V_{j-1} and K_{j+1}, then waits and synchronises.  The
    last iteration copies V_j, reads V_{j-1}, waits and synchronises, then
    reads V_j."""
    ev = []

    def copy(buf, t):
        ev.append((COPY, buf, t % 2, t))

    def read(buf, t):
        ev.append((READ, buf, t % 2, t))

    def sync():
        ev.extend([(WAIT, 0), (BARRIER,)])

    copy("K", 0)
    copy("K", 1)
    sync()
    read("K", 0)
    if not drop_refill_barrier:
        ev.append((BARRIER,))
    if nt == 1:
        copy("V", 0)
        sync()
        read("V", 0)
        return ev
    # iteration 0
    copy("K", 2)
    copy("V", 0)
    read("K", 1)
    sync()
    for j in range(1, nt - 1):
        copy("K", j + 2)
        copy("V", j)
        read("V", j - 1)
        read("K", j + 1)
        sync()
    j = nt - 1
    copy("V", j)
    read("V", j - 1)
    sync()
    read("V", j)
    return ev


def hazards(ev):
    """Violations of the staging rules in one program order."""
    bad = []
    # per stage: tile of the last copy, whether a wait and then a barrier
    # followed it, whether a barrier followed the last read
    last_copy = {}
    copy_seq = {}           # stage -> issue number of its last copy
    copy_ready = {}
    read_since_barrier = {}
    waited = set()          # stages whose copy a wait has covered
    issued = 0              # copies issued so far
    done = 0                # copies known complete (issue numbers below it)
    for i, e in enumerate(ev):
        kind = e[0]
        if kind == COPY:
            _, buf, st, t = e
            if read_since_barrier.get((buf, st)):
                bad.append(f"event {i}: copy of {buf}{t} into stage {st} before a barrier "
                           f"after the stage's last read")
            last_copy[(buf, st)] = t
            copy_seq[(buf, st)] = issued
            issued += 1
            copy_ready[(buf, st)] = False
            waited.discard((buf, st))
        elif kind == READ:
            _, buf, st, t = e
            if last_copy.get((buf, st)) != t:
                bad.append(f"event {i}: read of {buf}{t} from stage {st}, which holds "
                           f"{buf}{last_copy.get((buf, st))}")
            elif not copy_ready[(buf, st)]:
                bad.append(f"event {i}: read of {buf}{t} before a wait and a barrier "
                           f"after its copy")
            read_since_barrier[(buf, st)] = True
        elif kind == WAIT:
            done = max(done, issued - e[1])
            waited.update(key for key, seq in copy_seq.items() if seq < done)
        elif kind == BARRIER:
            for key in waited:
                copy_ready[key] = True
            waited.clear()
            for key in read_since_barrier:
                read_since_barrier[key] = False
    if done < issued:
        bad.append(f"{issued - done} copies still in flight when the workgroup ends")
    return bad


@pytest.mark.parametrize("nt", range(1, 65))
def test_fused16_rings_are_hazard_free(nt):
    assert hazards(fused16_events(nt)) == []


@pytest.mark.parametrize("nt", range(1, 65))
def test_stream_schedule_is_hazard_free(nt):
    assert hazards(fused16_events(nt, v_ahead=2, barrier_every=1, keep=3)) == []


def test_stream_schedule_limits():
    # V three ahead would refill the stage of the V tile the same iteration
    # reads; four copies in flight would leave K_{j+2} unfinished when
    # iteration j+1 reads it; a barrier every other iteration lets a copy
    # land in a stage read since the last barrier
    assert hazards(fused16_events(12, v_ahead=3, barrier_every=1, keep=3))
    assert any("before a wait" in h
               for h in hazards(fused16_events(12, v_ahead=2, barrier_every=1, keep=4)))
    assert hazards(fused16_events(12, v_ahead=2, barrier_every=2, keep=3))


@pytest.mark.parametrize("nt", range(1, 65))
def test_fp8_double_buffer_is_hazard_free(nt):
    assert hazards(fp8_events(nt)) == []


def test_a_barrier_too_few_is_caught():
    # one barrier per three tiles with the same four stages: a K copy lands
    # in a stage whose previous tile may still be read
    assert any("before a barrier" in h for h in hazards(fused16_events(12, barrier_every=3)))
    # three stages with copies three ahead: a stage is refilled while its
    # tile is still to be read
    assert hazards(fused16_events(12, stages=3))
    # the FP8 prologue without the barrier after scores_0: K stage 0 is
    # refilled in iteration 0 while other waves may still read K_0
    assert any("K2 into stage 0" in h for h in hazards(fp8_events(8, drop_refill_barrier=True)))


def test_the_copy_wait_is_required():
    # the same fused schedule with the waits removed: a read follows a
    # barrier but the copy may still be in flight
    ev = [e for e in fused16_events(10) if e[0] != WAIT]
    assert any("before a wait" in h for h in hazards(ev))
    # the last wait leaving copies in flight ends the workgroup with them
    ev = fused16_events(10)
    last_wait = max(i for i, e in enumerate(ev) if e[0] == WAIT)
    ev[last_wait] = (WAIT, 1)
    assert any("in flight" in h for h in hazards(ev))
