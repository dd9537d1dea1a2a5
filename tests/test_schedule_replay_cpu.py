"""CPU replay of the persistent kernel's stream-K bookkeeping.

The tile kernel (gemm_persistent) gives virtual workgroup v < sk_grid the MAC
iterations [floor(v T / G), floor((v+1) T / G)) of the T = sk_tiles * ipt
stream-K iterations, G = sk_grid; a tile cut between workgroups is finished
by the contributor that counts the tile's last expected arrival, where the
expectation is (owner of the tile's last iteration) - (owner of its first).
This replays that arithmetic in exact integers for schedules the library
decides (gemm_plan_describe: host-only, no device) and checks that every
stream-K tile is covered exactly once, receives exactly the expected
arrivals, and that the finisher reads exactly the partial slots that were
written. The data-parallel remainder must cover the other tiles once.
"""
import itertools

import pytest

import dense_gemm_epilogue_02_amd as g

S, T = g.Schedule, g.Tile


def sk_owner(x, T_, G):
    # ceil((x + 1) G / T) - 1, the kernel's owner of iteration x
    return ((x + 1) * G + T_ - 1) // T_ - 1


def replay(total, ipt, grid, sk_tiles, sk_grid):
    """Returns a list of problems found (empty when the schedule is sound)."""
    errs = []
    T_ = sk_tiles * ipt
    G = sk_grid
    covered = {}          # tile -> list of (k0, k1)
    arrivals = {}         # tile -> list of slot ids written
    if sk_tiles > 0:
        if not (1 <= G <= grid and G <= T_):
            return [f"sk_grid {G} outside [1, min(grid {grid}, T {T_})]"]
        for v in range(G):
            it, end = v * T_ // G, (v + 1) * T_ // G
            first_tile = it // ipt
            while it < end:
                t = it // ipt
                t0 = t * ipt
                k0, k1 = it - t0, min(end, t0 + ipt) - t0
                covered.setdefault(t, []).append((k0, k1))
                if not (k0 == 0 and k1 == ipt):
                    arrivals.setdefault(t, []).append(2 * v + (0 if t == first_tile else 1))
                it = t0 + k1
    for t in range(sk_tiles):
        segs = sorted(covered.get(t, []))
        pos = 0
        for a, b in segs:
            if a != pos or b <= a:
                errs.append(f"tile {t}: segments {segs} do not tile [0, {ipt})")
                break
            pos = b
        else:
            if pos != ipt:
                errs.append(f"tile {t}: segments {segs} stop at {pos} of {ipt}")
        if t in arrivals:
            t0 = t * ipt
            v0, v1 = sk_owner(t0, T_, G), sk_owner(t0 + ipt - 1, T_, G)
            if len(arrivals[t]) != v1 - v0 + 1:
                errs.append(f"tile {t}: {len(arrivals[t])} arrivals, finisher expects {v1 - v0 + 1}")
            # the slots the finisher sums, in contributor order
            want = []
            for u in range(v0, v1 + 1):
                ft = (u * T_ // G) // ipt
                want.append(2 * u + (0 if t == ft else 1))
            if sorted(want) != sorted(arrivals[t]):
                errs.append(f"tile {t}: finisher reads slots {want}, written {arrivals[t]}")
    dp = {}
    for v in range(grid):
        for t in range(sk_tiles + v, total, grid):
            dp[t] = dp.get(t, 0) + 1
    for t in range(sk_tiles, total):
        if dp.get(t, 0) != 1:
            errs.append(f"data-parallel tile {t} run {dp.get(t, 0)} times")
    return errs


def test_replay_catches_the_empty_range_case():
    # 16 stream-K tiles of 4 k-tiles over 256 workgroups: with G = grid most
    # workgroups own empty ranges and no tile ever sees its last arrival
    assert replay(total=16 * 17, ipt=4, grid=256, sk_tiles=16, sk_grid=256)
    assert not replay(total=16 * 17, ipt=4, grid=256, sk_tiles=16, sk_grid=64)


@pytest.mark.parametrize("M,N,K", [(4096, 4352, 256), (3072, 3200, 256), (4096, 10240, 8192),
                                   (4352, 4352, 512), (2304, 2560, 192)])
def test_auto_hybrid_shapes_replay_clean(M, N, K):
    p = g.Plan("bf16", la="row", lb="col", lc="row")
    try:
        d = p.describe(M, N, K)
        assert d["kernel"] == "tile"
        assert not replay(d["tiles"], d["ipt"], d["grid"], d["sk_tiles"], d["sk_grid"]), d
        if d["schedule"] == "hybrid":
            assert d["sk_grid"] <= d["sk_iters"]
    finally:
        p.close()


def test_forced_schedules_replay_clean_over_many_shapes():
    plans = {lb: g.Plan("bf16", la="row", lb=lb, lc="row") for lb in ("col", "row")}
    f8 = g.Plan("f8e4m3", la="row", lb="col", lc="row")
    f32 = g.Plan("f32", la="row", lb="row", lc="row")
    checked = 0
    try:
        shapes = [(m, n, k) for m, n, k in itertools.product(
            (32, 200, 512, 1000, 2304, 4096), (128, 700, 2560, 4352), (64, 256, 1000, 4096))]
        for (M, N, K), (plan, sched, grid, cus) in itertools.product(
                shapes, itertools.product(list(plans.values()) + [f8, f32],
                                          (S.AUTO, S.STREAM_K, S.HYBRID),
                                          (0, 16, 100, 256), (256, 80, 304))):
            plan.set_config(sched, T.AUTO, grid)
            d = plan.describe(M, N, K, num_cus=cus)
            if d["kernel"] != "tile" or d["split"]:
                continue
            errs = replay(d["tiles"], d["ipt"], d["grid"], d["sk_tiles"], d["sk_grid"])
            assert not errs, (M, N, K, sched, grid, cus, d, errs[:3])
            checked += 1
    finally:
        for p in list(plans.values()) + [f8, f32]:
            p.close()
    assert checked > 1000


# ---- the grouped launches' tile queues ---------------------------------------
#
# With a queue, workgroup v (virtual id) runs tile v first; every later tile
# comes from a claim on its XCD's queue (blockIdx & 7 when the grid is a
# multiple of 8 and the XCD remap is on, else one queue). Claim c of queue x
# is tile grid + ((c // chunk) * nq + x) * chunk + c % chunk (chunk = 16 with
# eight queues, grid with one);
# a claim past the last tile ends the workgroup. The replay interleaves the
# workgroups' claims in an arbitrary order (a seeded shuffle of who claims
# next) and checks that every tile runs exactly once and that each queue's
# claims run out only after all of its tiles were handed out.

def queue_replay(total, grid, remap, order_seed):
    import random
    nq = 8 if remap and grid % 8 == 0 else 1
    chunk = 16 if nq == 8 else grid
    claims = [0] * nq
    ran = {}
    rng = random.Random(order_seed)
    live = list(range(grid))           # blockIdx values still claiming
    for w in live:
        v = (w & 7) * (grid >> 3) + (w >> 3) if nq == 8 else w
        ran[v] = ran.get(v, 0) + 1     # the first tile, no claim
    claimed_total = 0
    while live:
        w = rng.choice(live)
        x = (w & 7) if nq == 8 else 0
        c = claims[x]
        claims[x] += 1
        claimed_total += 1
        t = grid + ((c // chunk) * nq + x) * chunk + c % chunk
        if t >= total:
            live.remove(w)
            continue
        ran[t] = ran.get(t, 0) + 1
    return ran, claimed_total, nq


@pytest.mark.parametrize("remap", [0, 1])
def test_tile_queue_runs_every_tile_once(remap):
    for total, grid in [(1, 1), (7, 7), (8, 8), (9, 8), (512, 512), (513, 512), (5011, 512),
                        (5011, 256), (1000, 24), (777, 40), (4096, 512), (130, 16)]:
        grid = min(grid, total)
        for seed in range(3):
            ran, claimed, nq = queue_replay(total, grid, remap, seed)
            assert sorted(ran) == list(range(total)), (total, grid, remap)
            assert all(n == 1 for n in ran.values()), (total, grid, remap)
            # one claim per tile run (the first tiles need none, and every
            # workgroup makes one claim that comes back past the end)
            assert claimed == total, (total, grid, claimed)
