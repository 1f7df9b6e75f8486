"""Pure-Python model of the synchronisation protocols of the two single-launch
MoE layer kernels (test infrastructure, CPU only).

The model executes the kernels' control protocol, not their arithmetic: the
grid's blocks and each block's waves are generators that yield at every point
where the real wave issues a memory operation another wave can observe, and a
seeded random scheduler interleaves them.  Every wait is bounded exactly as in
the kernels (a poll budget after which PQ_ERR_TIMEOUT is recorded and the wave
goes on), so a run always ends; a protocol that deadlocks shows up as a run
whose waits time out although every block was resident.

Barrier kernel (one token):
  * block b owns the units [split(U, G, b), split(U, G, b+1)); its waves take
    them one at a time from the block's LDS counter and publish each unit's h
    (a non-zero word: h is stored bit-inverted into a region that is zero
    between calls);
  * once every wave of the block is done with its units (block barrier: the
    staged h overwrites x), each wave waits until every h word of its share
    is non-zero (it polls the values themselves); the block then runs its
    down rows;
  * each block counts itself out; the last one clears h and the exit
    counter.

Stream kernel (three tokens or more):
  * gate_up unit k of block b is entry b + k*G of the expert-major list;
    waves claim k from the block's LDS counter and publish each unit's h;
  * a wave out of gate_up units leaves the block's LDS busy count, then claims
    staging items (union entry, pair) from a second LDS counter; the stager
    polls the pair's h (every unit of that entry, whichever block owns it)
    and counts the entry staged; with aliased LDS, an item whose staging slot
    (its index in union order) is hsplit or later overlays the x codes, and
    its stager first waits until no wave of the block is still in gate_up;
  * then it claims down units (entry, row pair), two consecutive ones per claim,
    from a third counter and, before consuming one, waits until its entry is
    fully staged;
  * the last block to exit clears h and the exit counter.
"""
from __future__ import annotations

import random


def split_start(n: int, p: int, i: int) -> int:
    """First index of part i when n items are dealt to p parts as evenly as
    possible (the first n % p parts get one more) -- the kernels' rule."""
    q, r = divmod(n, p)
    return i * q + min(i, r)



class Grid:
    """Shared state of one launch: global memory words and the error word.
    ``nh`` counts the non-zero h words (what a poll over all of h sees)."""

    def __init__(self, G: int):
        self.G = G
        self.error = 0
        self.mem = {}
        self.nh = 0

    def get(self, k, default=0):
        return self.mem.get(k, default)

    def put(self, k, v):
        if isinstance(k, tuple) and k[0] == "h":
            self.nh += (v != 0) - (self.mem.get(k, 0) != 0)
        self.mem[k] = v

    def record_timeout(self):
        if self.error == 0:
            self.error = -7


def wait_until(cond, grid: Grid, limit: int):
    """A bounded poll: yields once per poll; after `limit` failed polls records
    PQ_ERR_TIMEOUT and returns False (the wave goes on)."""
    for _ in range(limit + 1):
        if cond():
            return True
        yield
    grid.record_timeout()
    return False


# ---------------------------------------------------------------------------
# barrier kernel
# ---------------------------------------------------------------------------

def barrier_block(grid: Grid, b: int, W: int, U: int, limit: int, log: dict, clear_h: bool = True):
    """The waves of block b, as a list of generators.  clear_h=False models a
    last block that leaves h set (a mistake: the next call would read the
    previous call's h as its own before it is written)."""
    lds = {"next": 0}
    start, end = split_start(U, grid.G, b), split_start(U, grid.G, b + 1)
    nrows = end - start
    waves_done = {"gate_up": 0, "staged": 0, "exit": 0}

    def wave(w):
        # gate_up: claim units from the block's LDS counter, publish each h
        while True:
            c = lds["next"]
            lds["next"] += 1
            yield
            if c >= nrows:
                break
            u = start + c
            grid.put(("h", u), 1)
            log["h_written"][u] = log["h_written"].get(u, 0) + 1
            log["n_written"] += 1
            yield
        # block barrier (the staged h overwrites x in LDS), then staging: poll
        # until every h word of the call is non-zero (bounded)
        waves_done["gate_up"] += 1
        yield from wait_until(lambda: waves_done["gate_up"] == W, grid, 10 ** 9)
        ok = yield from wait_until(lambda: grid.nh >= U, grid, limit)
        if ok and log["n_written"] != U:           # what it read must be this call's h
            log["early_release"].append((b, U - log["n_written"]))
        # block barrier after staging, then down rows (no cross-block waits)
        waves_done["staged"] += 1
        yield from wait_until(lambda: waves_done["staged"] == W, grid, 10 ** 9)
        yield
        waves_done["exit"] += 1
        yield from wait_until(lambda: waves_done["exit"] == W, grid, 10 ** 9)
        if w == 0:
            old = grid.get("exit_count")
            grid.put("exit_count", old + 1)
            yield
            if old == grid.G - 1:                     # the last block clears what the call used
                grid.put("exit_count", 0)
                if clear_h:
                    for u0 in range(0, U, 1024 * 8):  # the block's threads clear 8 words each per store
                        for u in range(u0, min(u0 + 1024 * 8, U)):
                            grid.put(("h", u), 0)
                        yield
                log["cleared_by"].append(b)

    return [wave(w) for w in range(W)]


# ---------------------------------------------------------------------------
# stream kernel
# ---------------------------------------------------------------------------

DN_CLAIM = 2     # down units (row pairs) per claim in the stream kernel


def stream_block(grid: Grid, b: int, W: int, nU: int, I: int, unp: list, alias: bool, limit: int, log: dict,
                 hsplit: int = 0, room: int | None = None):
    """Waves of block b of the stream kernel.  nU union entries of I h-rows
    each; unp[u] pairs routed to entry u; the block's down rows are one row
    per entry here (the row count changes nothing in the protocol).  With
    alias, the LDS holds `room` staging slots apart from the x codes; the
    later slots overlay the x codes that gate_up reads.  The kernel makes the
    stagers of slots hsplit and later wait for the end of gate_up (its plan
    sets hsplit = room; a different value models a wrong plan)."""
    room = hsplit if room is None else room
    G = grid.G
    total = nU * I
    items = [(u, t) for u in range(nU) for t in range(unp[u])]
    lds = {"next": 0, "iclaim": 0, "dnext": 0, "gu_busy": W, "staged": [0] * nU}
    exits = {"n": 0}

    def wave(w):
        # gate_up units b + k*G
        while True:
            k = lds["next"]
            lds["next"] += 1
            yield
            v = b + k * G
            if v >= total:
                break
            grid.put(("h", v), 1)                      # the unit's h, stored for every pair of its entry
            log["h_written"][v] = log["h_written"].get(v, 0) + 1
            yield
        lds["gu_busy"] -= 1
        yield
        # staging: items in union order
        while True:
            j = lds["iclaim"]
            lds["iclaim"] += 1
            yield
            if j >= len(items):
                break
            u, t = items[j]
            if alias and j >= hsplit:
                yield from wait_until(lambda: lds["gu_busy"] == 0, grid, limit)
            ok = yield from wait_until(lambda: all(grid.get(("h", u * I + i)) for i in range(I)), grid, limit)
            if lds["gu_busy"] > 0:                     # the slot's codes are written now
                if alias and j >= room:
                    log["x_clobbered"].append((b, j))
                else:
                    log["staged_during_gate_up"] += 1
            if ok:
                log["staged"].append((b, u, t))
            lds["staged"][u] += 1
            yield
        # down units: one per entry, claimed kDnClaim at a time; each consumed
        # once its entry is staged
        done_claims = False
        while not done_claims:
            c = lds["dnext"]
            lds["dnext"] += 1
            yield
            for d in range(DN_CLAIM * c, DN_CLAIM * c + DN_CLAIM):
                if d >= nU:
                    done_claims = True
                    break
                ok = yield from wait_until(lambda: lds["staged"][d] >= unp[d], grid, limit)
                if ok and not all(grid.get(("h", d * I + i)) for i in range(I)):
                    log["early_release"].append((b, d))
                yield
        exits["n"] += 1
        yield from wait_until(lambda: exits["n"] == W, grid, 10 ** 9)
        if w == 0:
            old = grid.get("exit_count")
            grid.put("exit_count", old + 1)
            yield
            if old == G - 1:
                for v in range(total):
                    grid.put(("h", v), 0)
                grid.put("exit_count", 0)
                log["cleared_by"].append(b)

    return [wave(w) for w in range(W)]


# ---------------------------------------------------------------------------
# scheduler
# ---------------------------------------------------------------------------

def run(kernel: str, G: int, W: int = 4, *, U: int = 12, nU: int = 3, I: int = 4, unp=None, alias=False,
        hsplit: int = 0, room: int | None = None, limit: int = 10 ** 6, seed: int = 0,
        late_block: int | None = None,
        max_steps: int = 10 ** 8, grid: Grid | None = None, clear_h: bool = True):
    """Run one launch of the model; returns (grid, log, steps).

    late_block: that block is not resident until every other block has ended
    (a concurrent kernel holds its CU) -- the kernels' bounded waits must then
    end the run with PQ_ERR_TIMEOUT instead of hanging.
    grid: the global memory left by a previous launch (calls in a row on one
    workspace); a fresh, zeroed one by default."""
    rng = random.Random(seed)
    grid = grid if grid is not None else Grid(G)
    log = {"h_written": {}, "n_written": 0, "early_release": [], "staged": [], "cleared_by": [],
           "x_clobbered": [], "staged_during_gate_up": 0}
    blocks = []
    for b in range(G):
        if kernel == "barrier":
            blocks.append(barrier_block(grid, b, W, U, limit, log, clear_h))
        else:
            blocks.append(stream_block(grid, b, W, nU, I, unp or [1] * nU, alias, limit, log, hsplit, room))
    live = [(b, g) for b, ws in enumerate(blocks) for g in ws if b != late_block]
    steps = 0
    while live:
        i = rng.randrange(len(live))
        try:
            next(live[i][1])
        except StopIteration:
            live[i] = live[-1]
            live.pop()
        steps += 1
        if steps > max_steps:
            raise RuntimeError("model did not end within the step bound")
        if not live and late_block is not None:
            live = [(late_block, g) for g in blocks[late_block]]
            late_block = None
    return grid, log, steps


# ---------------------------------------------------------------------------
# SIMT model of a work claim inside a loop (the lane-0 claim mistake)
# ---------------------------------------------------------------------------

def simt_claim_loop(claim_form: str, n_items: int, lanes_exit_early: bool, max_iter: int = 1000):
    """A 64-lane wave runs `while (claim() < n_items) work;` where the claim is
    either 'all_lanes' (every active lane adds 1 to an LDS counter, the claim
    is the first active lane's old value / 64) or 'lane0_branch' (only lane 0
    adds 1, inside an `if (lane == 0)` branch, and the claim is read back from
    the first active lane).  With lanes_exit_early, the compiler's divergent
    form of the loop has retired lane 0 from the exec mask (the loop keeps
    running for the other lanes), which is what the kernels' hang came from.
    Returns the list of claims the wave made, or None if it never left the
    loop within max_iter iterations."""
    counter = 0
    exec_mask = [True] * 64
    if lanes_exit_early:
        exec_mask[0] = False
    reg = [0] * 64
    claims = []
    for _ in range(max_iter):
        active = [l for l in range(64) if exec_mask[l]]
        if claim_form == "all_lanes":
            if len(active) != 64:
                raise AssertionError("wave_claim requires a fully active wave")
            old = counter
            for l in active:
                reg[l] = counter
                counter += 1
            c = reg[active[0]] // 64
            assert c == old // 64
        else:
            for l in active:
                if l == 0:
                    reg[l] = counter
                    counter += 1
            c = reg[active[0]]
        if c >= n_items:
            return claims
        claims.append(c)
    return None
