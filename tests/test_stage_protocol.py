"""CPU replay of the stage protocol of the 512-row FC1 kernel
(prefill_fc1_512_kernel with its pipelined K loop, csrc/prefill.hip).

The kernel's per-wave sequence of stage requests (LDS DMAs), epilogue
stores, waits and workgroup barriers is transcribed here step by step from
the kernel (pb_issue_first, pb_k_loop, pb_barrier, pb_half0/pb_half1, the
item loop and the wait before exit), for waves with and without token rows
in the group, over several items and K step counts, and replayed under the
hardware's rules: a wave's vector memory operations complete in the order
issued, `s_waitcnt vmcnt(N)` returns once at most the N newest are
outstanding, `lgkmcnt(0)` once the wave's LDS reads are done, and a barrier
releases every wave once all have reached it.  The checks:

* a stage is read only after every wave's requests for it are complete;
* no request writes a buffer before every wave's reads of the stage it held
  are complete (requests past the item's last stage write zeros, so they
  count);
* every wave takes the same barriers;
* nothing is outstanding when the workgroup leaves;
* every request lands inside the ring of three stages.

A planted mistake (a wait one request too short, the next item's stages
requested before the item's last barrier, no wait before exit) must fail.
"""

import itertools

import pytest

K_DMAS = 8           # requests per wave per stage
STAGES = 3
STAGE_BYTES = 53760
RING_BYTES = STAGES * STAGE_BYTES


class Wave:
    def __init__(self):
        self.ops = []          # vector memory ops in issue order: ("dma", stage_uid, buffer) or ("store",)
        self.events = []       # program order: ("issue", op index) / ("wait", N, lgkm) / ("barrier",) / ("read", stage_uid, buffer)

    def dma(self, uid, buf, lds_off=0):
        assert 0 <= buf < STAGES and 0 <= buf * STAGE_BYTES + lds_off < RING_BYTES
        for _ in range(K_DMAS):
            self.ops.append(("dma", uid, buf))
            self.events.append(("issue", len(self.ops) - 1))

    def stores(self, n):
        for _ in range(n):
            self.ops.append(("store",))
            self.events.append(("issue", len(self.ops) - 1))

    def wait(self, n, lgkm=True):
        self.events.append(("wait", n, lgkm))

    def barrier(self):
        self.events.append(("barrier",))

    def read(self, uid, buf):
        self.events.append(("read", uid, buf))


def transcribe(items, wave_active, mistake=None):
    """The per-wave programs of one workgroup that runs `items` (a list of
    K step counts, one per item; every item of a launch has the same count,
    but a workgroup may have any number of items), wave w active in item i
    when wave_active[i][w].  Mirrors prefill_fc1_512_kernel."""
    n_waves = len(wave_active[0])
    waves = [Wave() for _ in range(n_waves)]
    uid = itertools.count()
    # stage uids per item (same on every wave): uid[i][s]
    uids = [[next(uid) for _ in range(max(steps, 1) + 2)] for steps in items]

    def issue_first(w, i):
        steps = items[i]
        for s in range(3):   # pb_issue_first: stages 0..2, live or past the end
            w.dma(uids[i][s] if s < steps else ("past", i, s), s)

    for wi, w in enumerate(waves):
        if items:
            # before the loop: lds_barrier (an LDS-read wait only), then the
            # first item's first three stages
            w.wait(10**9, True)
            w.barrier()
            issue_first(w, 0)
        for i, steps in enumerate(items):
            active = wave_active[i][wi]
            # pb_k_loop prologue: certify stage 0
            w.wait(2 * K_DMAS if mistake != "short_prologue" else 2 * K_DMAS + 1)
            w.barrier()
            if active:
                w.read(uids[i][0], 0)       # weight tiles, token tiles 0, 1
            bc = 0
            for j in range(steps - 1):
                if active:
                    w.read(uids[i][j], bc)  # half0: token tiles 2, 3 of stage j
                w.wait(K_DMAS if mistake != "short_wait" else K_DMAS + 1)   # pb_barrier
                w.barrier()
                bn = (bc + 1) % 3
                live = j + 3 < steps
                st = uids[i][j + 3] if live else ("past", i, j + 3)
                if active:
                    w.read(uids[i][j + 1], bn)   # token tiles 0, 1 of stage j + 1
                    w.dma(st, bc)                # xs + the seven of pb_half1, between ...
                    w.read(uids[i][j + 1], bn)   # ... the weight refills from stage j + 1
                else:
                    w.dma(st, bc)
                bc = bn
            if active:
                w.read(uids[i][steps - 1], bc)   # the last step's half0
            # after the loop: lds_barrier, the next item's first stages, then the epilogue
            if mistake == "early_next":
                if i + 1 < len(items):
                    issue_first(w, i + 1)
                w.wait(10**9, True)
                w.barrier()
            else:
                w.wait(10**9, True)
                w.barrier()
                if i + 1 < len(items):
                    issue_first(w, i + 1)
            w.stores(4 if active else 0)
        if mistake != "no_exit_wait":
            w.wait(0, False)   # s_waitcnt vmcnt(0) before exit
    return waves


def replay(waves):
    """Walk every wave's program, numbering the barrier intervals (interval
    k lies between barrier k and barrier k + 1; every barrier of this kernel
    is preceded by an LDS-read wait, so a read is complete by the end of its
    interval); returns a list of violations."""
    bad = []
    n = len(waves)
    writes, reads = [], []               # (wave, interval, op index, uid, buffer) / (wave, interval, uid, buffer)
    certified = [[] for _ in range(n)]   # certified[w][k]: ops [0, c) of wave w complete at barrier k
    outstanding = []
    for w, wave in enumerate(waves):
        interval, issued, done = 0, 0, 0
        for e in wave.events:
            if e[0] == "issue":
                op = wave.ops[e[1]]
                if op[0] == "dma":
                    writes.append((w, interval, e[1], op[1], op[2]))
                issued += 1
            elif e[0] == "wait":
                done = max(done, issued - min(e[1], issued))
            elif e[0] == "barrier":
                certified[w].append(done)
                interval += 1
            elif e[0] == "read":
                reads.append((w, interval, e[1], e[2]))
        outstanding.append(issued - done)
    counts = {len(c) for c in certified}
    if len(counts) != 1:
        bad.append(f"waves take different numbers of barriers: {[len(c) for c in certified]}")
        return bad
    for w in range(n):
        if outstanding[w]:
            bad.append(f"wave {w} leaves with {outstanding[w]} requests possibly outstanding")
    # (a) a stage is read only once every wave's requests for it are certified
    by_stage = {}
    for (w, iv, k, uid, b) in writes:
        by_stage.setdefault((uid, b), []).append((w, k))
    for (r, iv, uid, b) in reads:
        if (uid, b) not in by_stage:
            bad.append(f"wave {r} reads stage {uid} in buffer {b}, which no request fills")
            continue
        if iv == 0:
            bad.append(f"wave {r} reads stage {uid} before any barrier")
            continue
        for (v, k) in by_stage[(uid, b)]:
            if k >= certified[v][iv - 1]:
                bad.append(f"wave {r} reads stage {uid} in buffer {b} in interval {iv} before wave {v}'s "
                           f"request {k} is certified")
                break
    # (b) no request writes a buffer's next occupant until every read of its
    # current one is complete: each read's interval precedes each such write's
    for b in range(STAGES):
        first = {}
        for (w, iv, k, uid, bb) in writes:
            if bb == b:
                first[uid] = min(first.get(uid, iv), iv)
        order = sorted(first, key=lambda u: first[u])
        rank = {u: i for i, u in enumerate(order)}
        for (r, ir, x, bb) in reads:
            if bb != b:
                continue
            for (w, iw, k, y, b2) in writes:
                if b2 == b and rank[y] > rank[x] and iw <= ir:
                    bad.append(f"wave {w} writes stage {y} into buffer {b} in interval {iw} while wave {r} "
                               f"reads stage {x} there in interval {ir}")
                    break
    return bad


def _run(items, active, mistake=None):
    return replay(transcribe(items, active, mistake))


CASES = []
for steps in (1, 2, 3, 4, 5, 6, 7, 28):
    for n_items in (1, 2, 3):
        for pattern in ("all", "half", "alternate"):
            CASES.append((steps, n_items, pattern))


def _active(n_items, pattern, n_waves=8):
    if pattern == "all":
        return [[True] * n_waves for _ in range(n_items)]
    if pattern == "half":   # waves with wm = 1 (waves 4..7) have no token rows
        return [[w < 4 for w in range(n_waves)] for _ in range(n_items)]
    return [[(w < 4) or (i % 2 == 0) for w in range(n_waves)] for i in range(n_items)]


@pytest.mark.parametrize("steps,n_items,pattern", CASES)
def test_pipelined_fc1_protocol(steps, n_items, pattern):
    bad = _run([steps] * n_items, _active(n_items, pattern))
    assert bad == [], bad[:5]


@pytest.mark.parametrize("mistake", ["short_wait", "short_prologue", "early_next", "no_exit_wait"])
def test_planted_protocol_mistakes_are_caught(mistake):
    found = False
    for steps in (2, 3, 5, 28):
        for n_items in (1, 2):
            if _run([steps] * n_items, _active(n_items, "all"), mistake):
                found = True
    assert found, mistake
