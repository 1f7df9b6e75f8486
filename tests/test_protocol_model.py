"""CPU checks of the layer kernels' synchronisation protocols on the model in
``protocol_model`` (claim, publish, release, staging and clearing), for grid
sizes 1 to 4096: every run ends, every unit is computed exactly once, nothing
reads h before every unit it needs has been published, and the workspace
words return to zero; a block that is not resident makes the bounded waits
end with PQ_ERR_TIMEOUT rather than hang; and the lane-0 claim inside a
divergent loop never leaves its loop, while the all-lane claim does."""
import pytest

import protocol_model as pm

LARGE_GRIDS = [100, 255, 256, 257, 1000, 1024, 2048, 4095, 4096]


def _clean_barrier(grid, log, U):
    assert grid.error == 0, "a bounded wait timed out although every block was resident"
    assert not log["early_release"], log["early_release"][:4]
    assert sorted(log["h_written"]) == list(range(U)) and set(log["h_written"].values()) == {1}
    assert len(log["cleared_by"]) == 1
    assert all(v == 0 for v in grid.mem.values()), "workspace words left non-zero"


def _clean_stream(grid, log, nU, I, unp, G):
    assert grid.error == 0
    assert not log["early_release"]
    assert sorted(log["h_written"]) == list(range(nU * I)) and set(log["h_written"].values()) == {1}
    assert len(log["staged"]) == G * sum(unp), "every block stages every pair once"
    assert len(log["cleared_by"]) == 1
    assert all(v == 0 for v in grid.mem.values())
    assert not log["x_clobbered"], "h codes written over x while a wave still read x"


def test_every_grid_size_covers_every_unit_once():
    """For every grid size 1..4096, the barrier kernel's block shares tile the
    units exactly, and the stream kernel's unit numbering b + k*G reaches every
    unit exactly once (the structural half of deadlock freedom: no unit is
    left unowned, so every wait on a published h ends)."""
    for U in (1, 7, 64, 8 * 2048):
        for G in range(1, 4097):
            assert pm.split_start(U, G, 0) == 0 and pm.split_start(U, G, G) == U
            if G <= 300 or G % 97 == 0:
                sizes = [pm.split_start(U, G, b + 1) - pm.split_start(U, G, b) for b in range(G)]
                assert min(sizes) >= 0 and max(sizes) - min(sizes) <= 1
    for total in (5, 64, 300):
        for G in range(1, 4097, 13):
            owners = sorted(b + k * G for b in range(G) for k in range((total - b + G - 1) // G) if b < total)
            assert owners == list(range(total))


@pytest.mark.parametrize("G", list(range(1, 33)))
def test_barrier_protocol_small_grids(G):
    for seed in range(3):
        for U in (1, 12, 40):
            grid, log, _ = pm.run("barrier", G, W=4, U=U, seed=seed)
            _clean_barrier(grid, log, U)


@pytest.mark.parametrize("G", LARGE_GRIDS)
def test_barrier_protocol_large_grids(G):
    U = 3 * G // 2 + 5                       # blocks with one and with two units, none without
    grid, log, _ = pm.run("barrier", G, W=2, U=U, seed=G)
    _clean_barrier(grid, log, U)
    grid, log, _ = pm.run("barrier", G, W=2, U=G // 3 + 1, seed=G + 1)   # most blocks own no unit
    _clean_barrier(grid, log, G // 3 + 1)


@pytest.mark.parametrize("G", list(range(1, 25)))
@pytest.mark.parametrize("alias", [False, True])
def test_stream_protocol_small_grids(G, alias):
    for seed in range(2):
        unp = [1, 3, 2]
        grid, log, _ = pm.run("stream", G, W=4, nU=3, I=4, unp=unp, alias=alias, seed=seed)
        _clean_stream(grid, log, 3, 4, unp, G)


@pytest.mark.parametrize("G", [1, 2, 3, 7, 16, 64])
@pytest.mark.parametrize("hsplit", [1, 3, 5])
def test_stream_protocol_partial_alias(G, hsplit):
    """Aliased LDS with the first hsplit staging slots outside the x codes:
    those are staged while waves of the block still stream gate_up (in some
    interleaving), the later ones only once every wave is past it, and no run
    writes h codes over x early, deadlocks or leaves the workspace dirty."""
    unp = [2, 1, 3]
    early = 0
    for seed in range(4):
        grid, log, _ = pm.run("stream", G, W=4, nU=3, I=4, unp=unp, alias=True, hsplit=hsplit, seed=seed)
        _clean_stream(grid, log, 3, 4, unp, G)
        early += log["staged_during_gate_up"]
    assert early > 0, "no slot before the split was staged during gate_up"


def test_stream_protocol_model_catches_an_unguarded_slot():
    """A plan whose split lies past the slots that really fit apart from x (so
    stagers of slots over the x codes skip the wait) shows up as h written
    over x while a wave still streams gate_up."""
    unp = [2, 1, 3]
    clobbered = 0
    for seed in range(8):
        _, log, _ = pm.run("stream", 3, W=4, nU=3, I=4, unp=unp, alias=True, hsplit=6, room=1, seed=seed)
        clobbered += len(log["x_clobbered"])
    assert clobbered > 0, "the model failed to show the unguarded slot"


@pytest.mark.parametrize("G", [100, 256, 1000, 4096])
def test_stream_protocol_large_grids(G):
    unp = [2, 1]
    grid, log, _ = pm.run("stream", G, W=2, nU=2, I=3, unp=unp, alias=True, seed=G)
    _clean_stream(grid, log, 2, 3, unp, G)


def test_calls_in_a_row_release_only_after_h_is_written():
    """Two calls on one workspace: the h words the first call wrote are cleared
    by its last block, so the second call's blocks wait for its own h.  A last
    block that leaves h set (the mistake this guards against) lets the second
    call read h before it is written."""
    for G in (1, 5, 64):
        grid, log, _ = pm.run("barrier", G, W=3, U=20, seed=1)
        _clean_barrier(grid, log, 20)
        grid, log, _ = pm.run("barrier", G, W=3, U=20, seed=2, grid=grid)
        _clean_barrier(grid, log, 20)
    grid, _, _ = pm.run("barrier", 16, W=3, U=40, seed=3, clear_h=False)
    _, log, _ = pm.run("barrier", 16, W=3, U=40, seed=4, grid=grid, clear_h=False)
    assert log["early_release"], "the model failed to show the stale-h mistake"


@pytest.mark.parametrize("kernel", ["barrier", "stream"])
def test_non_resident_block_times_out_instead_of_hanging(kernel):
    """One block starts only after all the others have ended (a concurrent
    kernel held its CU): the waits that depend on it give up after their poll
    budget, PQ_ERR_TIMEOUT is recorded, the launch ends, and the workspace
    words are back at zero for the next call."""
    G = 12
    kw = dict(U=30) if kernel == "barrier" else dict(nU=2, I=24, unp=[1, 2], alias=True)
    grid, log, _ = pm.run(kernel, G, W=3, limit=50, seed=7, late_block=G - 1, **kw)
    assert grid.error == -7
    assert len(log["cleared_by"]) == 1 and log["cleared_by"][0] == G - 1
    assert all(v == 0 for v in grid.mem.values())


def test_lane0_claim_in_divergent_loop_never_ends():
    """The claim made by lane 0 inside an `if (lane == 0)` branch is read back
    from the first active lane.  While the loop is uniform this works; once the
    compiler's divergent form of the loop has taken lane 0 out of the exec
    mask, no lane adds to the counter, the first active lane's register never
    changes, and the wave claims item 0 forever.  The all-lane claim (every
    lane adds 1, the claim is the first lane's old value / 64) has no lane
    branch to diverge on and claims 0, 1, 2, ... then ends."""
    assert pm.simt_claim_loop("lane0_branch", 5, lanes_exit_early=False) == [0, 1, 2, 3, 4]
    assert pm.simt_claim_loop("lane0_branch", 5, lanes_exit_early=True) is None
    assert pm.simt_claim_loop("all_lanes", 5, lanes_exit_early=False) == [0, 1, 2, 3, 4]
    with pytest.raises(AssertionError):
        pm.simt_claim_loop("all_lanes", 5, lanes_exit_early=True)
