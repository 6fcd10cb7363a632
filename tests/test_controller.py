"""CPU simulation of the on-GPU controller rule (the same C++ function the fused
kernel runs, exported as mk_controller_eval).

The pages fix the controller's intent, not its formula: it reads progress counters
and publishes a target number of communication blocks (Figure 2 caption, the
thelatestinai.com page), and for GEMM+AllReduce the target shifts toward
communication as computation nears completion (Figure 7a). These tests check that
behaviour and the rule's own guarantees (bounds, hysteresis, seeding, and that
waiting reducers do not look slow). Output bits never depend on the controller.
"""
import pytest

import tile_gemm_all_amd as mk

G = 256


def ev(T, c, r, bc, br, seed, cur):
    return mk.controller_eval(G, T, c, r, bc, br, seed, cur)


def test_bounds_and_drain():
    for seed in (0.0, 0.01, 0.5, 0.99, 1.0):
        t = ev(100, 0, 0, 0, 0, seed, 128)
        assert 1 <= t <= G - 1
    assert ev(100, 100, 10, 1000, 1000, 0.5, 40) == G  # no compute left: everyone reduces


def test_seed_used_until_rates_exist():
    assert ev(1000, 0, 0, 0, 0, 0.91, 1) == round(0.91 * G)
    assert ev(1000, 10, 0, 500, 0, 0.25, 1) == round(0.25 * G)


def test_equal_remaining_work_splits_evenly():
    # rates: compute 1 tile per 100 ticks, reduce 1 tile per 100 ticks; same remaining
    assert ev(1000, 100, 100, 100 * 100, 100 * 100, 0.9, 10) == G // 2


def test_hysteresis():
    cur = 128
    assert ev(1000, 100, 100, 10000, 10100, 0.5, cur) == cur  # tiny change ignored
    assert ev(1000, 100, 100, 10000, 30000, 0.5, cur) != cur  # large change applied


def simulate(T, t_c, t_r, period=8, seed=0.5, static=None, waits=False):
    """Discrete-event model: G workgroups, compute tiles take t_c, reduce tiles t_r
    (WG-time). Reducers may only reduce published tiles. Returns (makespan, trace)."""
    import heapq
    target = static if static is not None else max(1, min(G - 1, round(seed * G)))
    time = 0.0
    computed = reduced = claimed_c = claimed_r = 0
    busy_c = busy_r = 0.0
    published = []  # heap of publish times of computed tiles (by tile index)
    pub_time = {}
    events = []  # (time, wg, kind, tile)
    idle = list(range(G))
    trace = []
    completions = 0
    while reduced < T:
        # assign idle workgroups
        still = []
        for wg in idle:
            reducer = wg < target
            if not reducer and claimed_c < T:
                heapq.heappush(events, (time + t_c, wg, "c", claimed_c))
                claimed_c += 1
            elif claimed_r < T and claimed_r in pub_time:
                t = claimed_r
                claimed_r += 1
                heapq.heappush(events, (time + t_r, wg, "r", t))
            elif claimed_c >= T and claimed_r < T and claimed_r not in pub_time:
                still.append(wg)  # drain: wait for publication
            else:
                still.append(wg)
        idle = still
        if not events:
            break
        time, wg, kind, tile = heapq.heappop(events)
        if kind == "c":
            computed += 1
            busy_c += t_c
            pub_time[tile] = time
        else:
            reduced += 1
            busy_r += t_r
        completions += 1
        idle.append(wg)
        if static is None and completions % period == 0:
            target = mk.controller_eval(G, T, computed, reduced, int(busy_c), int(busy_r), seed,
                                        target)
            trace.append((time, computed, reduced, target))
    return time, trace


def test_target_rises_toward_reduce_as_compute_finishes():
    # Figure 7a: near the end of the GEMM the target moves toward communication
    _, trace = simulate(T=2048, t_c=100.0, t_r=30.0, seed=0.2)
    early = [t for (_, c, _, t) in trace if c < 1024]
    late = [t for (_, c, _, t) in trace if c >= 2040]
    assert early and late
    assert max(late) > sum(early) / len(early)
    assert trace[-1][3] == G


def test_hbm_bound_shape_gets_many_reducers_compute_bound_few():
    _, tr_hbm = simulate(T=2048, t_c=10.0, t_r=100.0, seed=0.91)
    _, tr_mfma = simulate(T=1024, t_c=100.0, t_r=15.0, seed=0.28)
    mid_hbm = [t for (_, c, _, t) in tr_hbm if 200 < c < 1800]
    mid_mfma = [t for (_, c, _, t) in tr_mfma if 100 < c < 900]
    assert min(mid_hbm) > G * 0.75
    assert max(mid_mfma) < G * 0.3


def test_adaptive_close_to_best_static():
    T, t_c, t_r = 1024, 100.0, 20.0
    best = min(simulate(T, t_c, t_r, static=n)[0] for n in range(4, 96, 4))
    adaptive, _ = simulate(T, t_c, t_r, seed=0.5)
    assert adaptive <= 1.25 * best


def test_waiting_does_not_count_as_reduce_time():
    # Same completed work; the controller only sees busy time. If waits were counted
    # the reduce rate would look 10x slower and the target would jump up.
    a = ev(1000, 200, 100, 200 * 100, 100 * 20, 0.5, 64)
    b = ev(1000, 200, 100, 200 * 100, 100 * 200, 0.5, 64)
    assert a < b


def test_cap_limits_reducers_while_compute_remains():
    # HBM-bound: the rate rule alone would hand almost everything to reducers
    free = ev(2048, 500, 400, 500 * 30, 400 * 90, 0.9, 128)
    capped = mk.controller_eval(G, 2048, 500, 400, 500 * 30, 400 * 90, 0.9, 128, 64)
    assert free > 64
    assert capped == 64
    # once every tile is computed, the cap no longer applies
    assert mk.controller_eval(G, 2048, 2048, 1900, 1, 1, 0.9, 64, 64) == G


def test_tiles_reduced_in_place_are_compute_work():
    # Half the tiles reduced in place by their compute workgroup: less work is left
    # for reducers, so the target drops; once every handed-over tile is reduced the
    # reducers are told to compute.
    all_handed = mk.controller_eval(G, 1024, 300, 200, 300 * 50, 200 * 60, 0.5, 128)
    half_handed = mk.controller_eval(G, 1024, 300, 200, 300 * 50, 200 * 60, 0.5, 128, T_r=512)
    assert half_handed < all_handed
    assert mk.controller_eval(G, 1024, 700, 512, 700 * 50, 512 * 60, 0.5, 128, T_r=512) == 1
    # T_r = T is the rule without in-place tiles
    assert (mk.controller_eval(G, 1024, 300, 200, 300 * 50, 200 * 60, 0.5, 128, T_r=1024)
            == all_handed)


def test_zero_cap_keeps_every_workgroup_computing():
    # cap 0: no dedicated reducers while GEMM tiles remain, everyone at the end
    assert mk.controller_eval(G, 1024, 300, 0, 0, 0, 0.4, 0, cap=0) == 0
    assert mk.controller_eval(G, 1024, 300, 200, 300 * 50, 200 * 60, 0.9, 5, cap=0) == 0
    assert mk.controller_eval(G, 1024, 1024, 200, 1, 1, 0.9, 0, cap=0) == G
