"""A host-side model of the LDS hand-off protocols of the tile loops.

The split-KV decode kernel and the bf16 prefill kernel stream tiles through
LDS slots with direct-to-LDS copies, read fragments with counted waits, and
synchronise the waves of a workgroup with barriers.  The decode's tile
barrier does not drain LDS operations: the next step's first fragment reads
stay in flight across it, and a barrier alone does not wait for a wave's
own LDS writes or copies.  Whether such a schedule is free of races is a
property of the order of issues, waits and barriers alone, so it is checked
here on a model:

* every wave of a workgroup runs the same program;
* a copy or an LDS write produces version v of a resource (a ring slot, a
  buffer); a read consumes version v; versions of one resource are ordered;
* an operation is issued at its position and completes at the first wait
  that covers it (copies: a vmcnt wait; reads and writes: an lgkmcnt wait,
  also the one a draining barrier starts with);
* a barrier orders, across waves, only what each wave completed before it;
* a private operation touches rows that only its own wave reads or writes
  (the decode's staging rows); two private operations of one wave are
  ordered by program order once the first has completed.

Rules, for every pair of operations on one resource (other waves included):
  visibility -- the producer of the version a read consumes completes
                before a barrier that precedes the read's issue;
  overwrite  -- a read completes before a barrier that precedes the issue
                of a producer of a later version;
  order      -- a producer completes before a barrier that precedes the
                issue of the producer of the next version.
The schedules below restate the kernels' loops: ring slots, how many tiles
are in flight, where copies and fragment reads are issued, which waits and
barriers end each step.  Schedules that break the rules in plausible ways
are shown to be caught.
"""

import pytest


class Wave:
    """The program of one wave, in program order."""

    def __init__(self):
        self.ops = []       # dicts: kind, res, ver, tag, private
        self.pending = []   # issued, not yet completed op indices
        self.done = {}      # op index -> position of the wait that completes it
        self.barriers = []  # positions of barriers

    def _add(self, **op):
        self.ops.append(op)
        return len(self.ops) - 1

    def copy(self, res, ver):
        i = self._add(kind="copy", res=res, ver=ver, tag=None, private=False)
        self.pending.append(i)
        return i

    def write(self, res, ver, private=False):
        i = self._add(kind="write", res=res, ver=ver, tag=None, private=private)
        self.pending.append(i)
        return i

    def read(self, res, ver, tag=None, private=False):
        i = self._add(kind="read", res=res, ver=ver, tag=tag, private=private)
        self.pending.append(i)
        return i

    def wait(self, pred):
        """A wait that completes every pending operation for which pred holds."""
        pos = self._add(kind="wait", res=None, ver=None, tag=None, private=False)
        keep = []
        for i in self.pending:
            (self.done.__setitem__(i, pos) if pred(self.ops[i]) else keep.append(i))
        self.pending = keep

    def wait_vm(self, pred=lambda op: True):
        self.wait(lambda op: op["kind"] == "copy" and pred(op))

    def wait_lgkm(self, pred=lambda op: True):
        self.wait(lambda op: op["kind"] in ("read", "write") and pred(op))

    def wait_op(self, i):
        self.wait(lambda op: op is self.ops[i])

    def barrier(self, drain_lds):
        if drain_lds:  # s_waitcnt lgkmcnt(0); s_barrier
            self.wait_lgkm()
        self.barriers.append(self._add(kind="barrier", res=None, ver=None, tag=None, private=False))

    def end(self):
        self.wait(lambda op: True)


def _first_barrier_at_or_after(w, pos):
    return next((b for b, p in enumerate(w.barriers) if p >= pos), len(w.barriers) + 1)


def _last_barrier_before(w, pos):
    return max((b for b, p in enumerate(w.barriers) if p < pos), default=-1)


def _ordered(w, first, second):
    """first completes before second is issued in every wave that matters."""
    a, b = w.ops[first], w.ops[second]
    if a["private"] and b["private"]:
        return w.done[first] < second
    return _first_barrier_at_or_after(w, w.done[first]) <= _last_barrier_before(w, second)


def check(w):
    """Rule violations of a wave program run by every wave of a workgroup."""
    issues = set()
    prods, reads = {}, []
    for i, op in enumerate(w.ops):
        if op["kind"] in ("copy", "write"):
            prods.setdefault(op["res"], []).append(i)
        elif op["kind"] == "read":
            reads.append(i)
    for r in reads:
        ro = w.ops[r]
        for p in prods.get(ro["res"], []):
            po = w.ops[p]
            if po["ver"] == ro["ver"] and not _ordered(w, p, r):
                issues.add(("visibility", ro["res"], ro["ver"], ro["tag"]))
            elif po["ver"] > ro["ver"] and not _ordered(w, r, p):
                issues.add(("overwrite", ro["res"], ro["ver"], ro["tag"]))
    for res, lst in prods.items():
        lst = sorted(lst, key=lambda i: w.ops[i]["ver"])
        for p0, p1 in zip(lst, lst[1:]):
            if w.ops[p1]["ver"] > w.ops[p0]["ver"] and not _ordered(w, p0, p1):
                issues.add(("order", res, w.ops[p0]["ver"], w.ops[p1]["ver"]))
    return sorted(issues, key=repr)


# ---------------------------------------------------------------------------
# Kept schedules
# ---------------------------------------------------------------------------
def decode_split_kernel(pieces, nbuf=4, ahead=2, epilogue_vm_wait=True, trailing_barrier=True):
    """mla_split_kernel: the in-kernel plan, then pieces of pieces[k] tiles.

    Versions of a ring slot are (piece, phase, tile): phase 0 the plan
    scan's scratch at the start of the ring, 1 the tiles, 2 the epilogue's
    staging rows.  In a piece, tile j sits in slot j % nbuf; `ahead` tiles
    are copied first; the top of step j (j < T) waits until this wave's
    copies of tile j have landed (younger copies stay in flight) and passes
    the non-draining tile barrier; step j reads tile j as keys and tile j-1
    as values (the first value fragments of the step were read at the end
    of step j-1, across the barrier), copies tile j + ahead (a tile past the
    end writes zeros into its slot: the copy counts stay fixed), and ends by
    reading the first value fragments of tile j for step j+1.  A last
    value-only step (no barrier, no copies) follows.  The epilogue waits for
    every copy and passes a draining barrier, writes each wave's normalised
    rows into its own staging rows over the ring, reads them back for whole-
    row global stores, and ends with a draining barrier before the next
    piece copies into the ring.
    """
    w = Wave()
    slot = lambda j: ("ring", j % nbuf)
    # The plan scan's reduction scratch and per-part minimum at the start of
    # the ring, ended by a draining barrier before the first tile copy.
    w.write(slot(0), (-1, 0, 0))
    w.barrier(drain_lds=True)
    w.read(slot(0), (-1, 0, 0), "plan scratch")
    w.barrier(drain_lds=True)
    for k, T in enumerate(pieces):
        tile = lambda j: (k, 1, j)
        for j in range(ahead):
            w.copy(slot(j), tile(j))
        pre = None
        for j in range(T):
            w.wait_vm(lambda op, j=j: op["ver"] <= tile(j))  # dec_wait_tile<ahead - 1>
            w.barrier(drain_lds=False)                      # dec_barrier
            if pre is not None:
                w.wait_op(pre)                              # prefetched value fragments used
            if j >= 1:
                w.read(slot(j - 1), tile(j - 1), "values")
            w.read(slot(j), tile(j), "keys")
            w.copy(slot(j + ahead), tile(j + ahead))
            w.wait_lgkm(lambda op: op["tag"] in ("values", "keys"))
            pre = w.read(slot(j), tile(j), "values, first groups")
        w.wait_op(pre)
        w.read(slot(T - 1), tile(T - 1), "values, last step")
        w.wait_lgkm()
        if epilogue_vm_wait:
            w.wait_vm()                                     # wait_vmcnt<0>
        w.barrier(drain_lds=True)                           # lds_barrier
        for s in range(nbuf):
            w.write(("ring", s), (k, 2, 0), private=True)
        w.wait_lgkm()
        for s in range(nbuf):
            w.read(("ring", s), (k, 2, 0), "staging", private=True)
        w.wait_lgkm()
        if trailing_barrier:
            w.barrier(drain_lds=True)
    w.end()
    return w


def prefill_bf16_kernel(T, epilogue_barrier=True):
    """attn_fwd_bf16_kernel: K and V of tile j in buffer j % 2.  Tile 0 is
    copied before the loop; step j waits for every copy of this wave and
    passes a draining barrier, reads K of tile j while it copies tile j+1
    into the other buffer (one K or V copy per score k-step; a tile past
    the end copies zeros), reads V of tile j, and ends with a draining
    barrier.  The epilogue waits for the last step's copies, passes a
    draining barrier, writes the wave's output rows into its own staging
    rows over both buffers and reads them back for whole-row stores."""
    w = Wave()
    for kv in ("K", "V"):
        w.copy((kv, 0), 0)
    for j in range(T):
        w.wait_vm()
        w.barrier(drain_lds=True)
        w.read(("K", j % 2), j, "scores")
        for kv in ("K", "V"):
            w.copy((kv, (j + 1) % 2), j + 1)
        w.wait_lgkm()
        w.read(("V", j % 2), j, "values")
        w.wait_lgkm()
        w.barrier(drain_lds=True)
    w.wait_vm()
    if epilogue_barrier:
        w.barrier(drain_lds=True)
    out = T + 1  # a version after every tile copy, including the empty tile T
    for b in range(2):
        for kv in ("K", "V"):
            w.write((kv, b), out, private=True)
    w.wait_lgkm()
    for b in range(2):
        for kv in ("K", "V"):
            w.read((kv, b), out, "staging", private=True)
    w.wait_lgkm()
    w.end()
    return w


# ---------------------------------------------------------------------------
# A decode step that exchanges P through LDS (scores split by heads, values
# by dims): each wave writes the probabilities (and rescale factors) of its
# heads for tile j into an LDS buffer double-buffered by tile parity, and
# every wave reads all of them for the value product of tile j in step j+1.
# One non-draining barrier per tile, a ring of nbuf tiles.
# ---------------------------------------------------------------------------
def decode_p_exchange(T, nbuf=3, ahead=1, wait_p_writes=True, prefetch_p=False):
    w = Wave()
    slot = lambda j: ("ring", j % nbuf)
    pbuf = lambda j: ("P", j % 2)
    for j in range(ahead):
        w.copy(slot(j), j)
    pre = None
    for j in range(T):
        w.wait_vm(lambda op, j=j: op["ver"] <= j)
        w.barrier(drain_lds=False)
        if pre is not None:
            w.wait_op(pre)
        if j >= 1:
            w.read(slot(j - 1), j - 1, "values")
            w.read(pbuf(j - 1), j - 1, "P")
        w.read(slot(j), j, "keys")
        w.copy(slot(j + ahead), j + ahead)
        w.wait_lgkm(lambda op: op["kind"] == "read")
        w.write(pbuf(j), j)
        if wait_p_writes:
            w.wait_lgkm(lambda op: op["kind"] == "write")
        pre = w.read(pbuf(j), j, "P, read ahead") if prefetch_p else None
    w.end()
    return w


# ---------------------------------------------------------------------------
@pytest.mark.parametrize("pieces", [[1], [2], [3], [4], [9], [1, 1], [3, 1, 5], [2, 7, 2]])
def test_decode_split_kernel_protocol_is_race_free(pieces):
    assert check(decode_split_kernel(pieces)) == []


@pytest.mark.parametrize("T", [1, 2, 3, 8])
def test_prefill_bf16_protocol_is_race_free(T):
    assert check(prefill_bf16_kernel(T)) == []


def test_prefill_epilogue_without_its_barrier_races_other_waves_copies():
    # A wave that has waited only for its own copies may stage its rows over
    # a buffer into which another wave's last (empty-tile) copies still land.
    issues = check(prefill_bf16_kernel(3, epilogue_barrier=False))
    assert any(i[0] == "order" and i[3] == 4 for i in issues), issues


def test_decode_three_slot_ring_with_two_tiles_in_flight_overwrites_the_values_tile():
    # Keys of tile j, values of tile j-1 and two tiles in flight take four
    # slots; with three, the copy of tile j+2 lands in tile j-1's slot while
    # step j still reads it as values.
    issues = check(decode_split_kernel([6], nbuf=3, ahead=2))
    assert any(i[0] == "overwrite" and i[3] == "values" for i in issues), issues


def test_decode_epilogue_without_the_copy_wait_races_the_empty_tiles():
    # The copies of the (empty) tiles past a piece's end may still land in
    # the ring when the staging rows are written.
    issues = check(decode_split_kernel([3], epilogue_vm_wait=False))
    assert any(i[0] == "order" and i[2][1] == 1 and i[3][1] == 2 for i in issues), issues


def test_decode_without_the_trailing_barrier_races_the_next_piece():
    # Another wave's copies for the next piece overwrite staging rows that
    # this wave may still be reading.
    issues = check(decode_split_kernel([2, 2], trailing_barrier=False))
    assert any(i[0] == "overwrite" and i[3] == "staging" for i in issues), issues


def test_p_exchange_needs_its_writes_waited_before_the_non_draining_barrier():
    # s_barrier does not wait for LDS writes in flight; the barrier that
    # keeps prefetched reads in flight therefore also lets a slow wave's P
    # writes land after a fast wave has read them.
    assert check(decode_p_exchange(6, wait_p_writes=True)) == []
    issues = check(decode_p_exchange(6, wait_p_writes=False))
    assert any(i[0] == "visibility" and i[1][0] == "P" for i in issues), issues


def test_p_exchange_read_ahead_across_the_barrier_reads_unwritten_p():
    # Reading P of tile j at the end of step j (for step j+1), the way the
    # value fragments are read ahead, reads the other waves' P before the
    # barrier that publishes it.
    issues = check(decode_p_exchange(6, prefetch_p=True))
    assert any(i[0] == "visibility" and i[3] == "P, read ahead" for i in issues), issues


def test_model_flags_a_read_of_a_tile_whose_copies_were_not_waited():
    w = Wave()
    w.copy(("ring", 0), 0)
    w.barrier(drain_lds=False)
    w.read(("ring", 0), 0, "keys")
    w.end()
    assert check(w) == [("visibility", ("ring", 0), 0, "keys")]


def test_model_lets_a_wave_reread_its_own_private_rows_without_a_barrier():
    w = Wave()
    w.write(("ring", 0), 0, private=True)
    w.wait_lgkm()
    w.read(("ring", 0), 0, "own rows", private=True)
    w.end()
    assert check(w) == []
    w = Wave()
    w.write(("ring", 0), 0)
    w.wait_lgkm()
    w.read(("ring", 0), 0, "other waves' rows")
    w.end()
    assert check(w) == [("visibility", ("ring", 0), 0, "other waves' rows")]
