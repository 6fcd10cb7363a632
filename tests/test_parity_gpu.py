"""GPU parity: libmk.so's fused kernel and two-kernel baseline against the CPU oracle.

Operation: C = A*B + sum of the P-1 peer partials (GEMM + AllReduce row of Table 3,
thelatestinai.com page). Bars:
  - integer-valued inputs: bit-exact against the oracle;
  - Gaussian inputs: tests/compare.py's rule (literal 2e-3*rms(C) bound for fp32 C;
    that bound plus half a bfloat16 ulp for bf16 C);
  - the output is bitwise identical for every reducer count, for the adaptive
    controller, for every reduce schedule (tiles reduced in place, handed over,
    peers summed early) and for the baseline (all reduce in the same order),
    except that a tile computed as two k-halves (MK_OPT_KSPLIT) sums the halves'
    fp32 partials: such calls agree among themselves, and the baseline is matched
    with the split off.
Full-size workloads are checked on sampled rows (first, last and one random row of
every 256-row band), with the oracle evaluating those rows only.
"""
import math

import numpy as np
import pytest
import torch

import mk_inputs
import oracle
from tests.compare import check_exact, check_tolerance

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import tile_gemm_all_amd as mk
else:  # collected on CPU-only machines, never run there
    mk = None

DEV = "cuda"
TORCH_DT = {"bf16": torch.bfloat16, "f32": torch.float32}


def announce(msg):
    print(f"\n[case] {msg}", flush=True)


def oracle_rows(A, B, peers, c_dtype, rows=None):
    Ab = mk_inputs.bits(A if rows is None else A[torch.as_tensor(rows, device=A.device)])
    Bb = mk_inputs.bits(B)
    if peers is None or peers.numel() == 0:
        Pb = None
    elif rows is None:
        Pb = mk_inputs.bits(peers)
    else:
        Pb = mk_inputs.bits(peers[:, torch.as_tensor(rows, device=peers.device), :])
    return oracle.gemm_ar(Ab, Bb, Pb, c_dtype)


def new_c(M, N, c_dtype):
    # poison: NaN bit patterns everywhere, so an unwritten element cannot pass
    C = torch.empty((M, N), dtype=TORCH_DT[c_dtype], device=DEV)
    if c_dtype == "bf16":
        C.view(torch.int16).fill_(0x7FC1)
    else:
        C.view(torch.int32).fill_(0x7FC00001)
    return C


def run(A, B, peers, c_dtype, mode):
    M, N = A.shape[0], B.shape[1]
    C = new_c(M, N, c_dtype)
    if mode == "baseline":
        mk.gemm_then_reduce_baseline(A, B, peers, C)
    else:
        mk.gemm_ar_local(A, B, peers, C, n_reduce_wg=None if mode == "adaptive" else int(mode))
    mk.stream_status()
    return C


def c_bits(C, rows=None):
    if rows is not None:
        C = C[torch.as_tensor(rows, device=C.device)]
    return mk_inputs.bits(C)


def sample_rows(M, band=256, seed=0):
    rng = np.random.default_rng(seed)
    rows = set()
    for m0 in range(0, M, band):
        m1 = min(M, m0 + band)
        rows.update({m0, m1 - 1, int(rng.integers(m0, m1))})
    return sorted(rows)


MODES = ["adaptive", "0", "3", "baseline"]

SMALL = [  # M, N, K, n_peers, peer dtype, c dtype
    (256, 512, 512, 3, "f32", "f32"),
    (300, 264, 200, 3, "bf16", "bf16"),      # ragged in M, N and K
    (130, 136, 72, 15, "bf16", "bf16"),
    (1, 8, 8, 0, "bf16", "bf16"),
    (64, 64, 0, 2, "bf16", "f32"),           # K == 0: C is the peer sum
    (257, 520, 264, 7, "f32", "bf16"),
    (520, 776, 1032, 1, "bf16", "f32"),
    (200, 136, 96, 5, "bf16", "bf16"),       # peer counts without a compile-time ring
    (130, 264, 104, 9, "f32", "f32"),
    (72, 64, 48, 64, "bf16", "bf16"),        # most peers
]


@pytest.fixture(params=[(-1, -1, 0, 0), (0, 0, 0, 0), (0, 1, 0, 2), (0, 0, 1, 0), (-2, 0, 0, 0),
                        (-1, -1, 0, 4), (-1, -1, 0, 5)],
                ids=["auto", "handover-all", "handover-all-early", "handover-all-agent-scope",
                     "dynamic", "wave-specialised", "wave-specialised-128"])
def inplace_policy(request):
    """Runs a test under the default policies (in place and early reduce automatic),
    with every tile handed to reducers through its flag (the role-split path), the
    same with reducers that sum a unit's peers before its tile is finished (early
    reduce; with 128x128 tiles, since 64x64 tiles are always reduced in place),
    every tile handed over under agent-scope release/acquire flags
    (MK_OPT_FLAG_SCOPE=1), with each tile reduced in place or published when its
    GEMM ends by the free streaming slots (dynamic hand-over, -2), and under the
    wave-specialised schedule (MK_OPT_TILE_SHAPE=4 and 5: four waves of each
    workgroup compute a 64x256 or 128x128 tile while two reduce the one before;
    peer counts without a compile-time ring, or a call with telemetry, fall back to
    the automatic choice). Yields the in-place option."""
    inplace, early, scope, shape = request.param
    old = (mk.get_option(mk.OPT_INPLACE), mk.get_option(mk.OPT_EARLY),
           mk.get_option(mk.OPT_FLAG_SCOPE), mk.get_option(mk.OPT_TILE_SHAPE))
    mk.set_option(mk.OPT_INPLACE, inplace)
    mk.set_option(mk.OPT_EARLY, early)
    mk.set_option(mk.OPT_FLAG_SCOPE, scope)
    mk.set_option(mk.OPT_TILE_SHAPE, shape)
    yield inplace
    mk.set_option(mk.OPT_INPLACE, old[0])
    mk.set_option(mk.OPT_EARLY, old[1])
    mk.set_option(mk.OPT_FLAG_SCOPE, old[2])
    mk.set_option(mk.OPT_TILE_SHAPE, old[3])


@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "x".join(map(str, s[:4])) + f"-{s[4]}-{s[5]}")
@pytest.mark.parametrize("mode", MODES)
def test_small_integer_bit_exact(shape, mode, inplace_policy):
    M, N, K, npeer, pdt, cdt = shape
    announce(f"integer {shape} {mode}")
    A, B, peers = mk_inputs.make_inputs(M, N, K, npeer, pdt, "integer", 7, device="cpu")
    _, want = oracle_rows(A, B, peers, cdt)
    C = run(A.to(DEV), B.to(DEV), peers.to(DEV), cdt, mode)
    check_exact(c_bits(C), want, f"{shape} {mode}")


@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "x".join(map(str, s[:4])) + f"-{s[4]}-{s[5]}")
@pytest.mark.parametrize("mode", ["adaptive", "baseline"])
def test_small_gaussian_tolerance(shape, mode):
    M, N, K, npeer, pdt, cdt = shape
    announce(f"gaussian {shape} {mode}")
    A, B, peers = mk_inputs.make_inputs(M, N, K, npeer, pdt, "gaussian", 11, device="cpu")
    C64, _ = oracle_rows(A, B, peers, cdt)
    C = run(A.to(DEV), B.to(DEV), peers.to(DEV), cdt, mode)
    check_tolerance(c_bits(C), C64, cdt, f"{shape} {mode}")


def test_empty_shapes_are_no_ops():
    announce("empty shapes")
    A = torch.zeros((0, 64), dtype=torch.bfloat16, device=DEV)
    B = torch.zeros((64, 32), dtype=torch.bfloat16, device=DEV)
    C = torch.zeros((0, 32), dtype=torch.bfloat16, device=DEV)
    mk.gemm_ar_local(A, B, None, C)
    mk.gemm_then_reduce_baseline(A, B, None, C)
    A = torch.zeros((16, 64), dtype=torch.bfloat16, device=DEV)
    B = torch.zeros((64, 0), dtype=torch.bfloat16, device=DEV)
    C = torch.zeros((16, 0), dtype=torch.float32, device=DEV)
    mk.gemm_ar_local(A, B, None, C)
    mk.stream_status()


@pytest.mark.parametrize("w", mk_inputs.WORKLOADS, ids=lambda w: w.name)
@pytest.mark.parametrize("variant", ["integer", "gaussian", "zeropeer"])
def test_workload_parity(w, variant):
    """Every workload at full size, fused (adaptive) and baseline; sampled rows."""
    announce(f"workload {w.name} {variant}")
    A, B, peers = mk_inputs.workload_inputs(w, variant, device=DEV)
    rows = None if w.M * w.N <= 1 << 20 else sample_rows(w.M, seed=w.index)
    C64, want = oracle_rows(A, B, peers, w.c_dtype, rows)
    rms = float(np.sqrt(np.mean(C64 * C64)))
    for mode in ("adaptive", "baseline"):
        C = run(A, B, peers, w.c_dtype, mode)
        got = c_bits(C, rows)
        if variant == "integer":
            check_exact(got, want, f"{w.name} {mode}")
        else:
            check_tolerance(got, C64, w.c_dtype, f"{w.name} {variant} {mode}", rms_ref=rms)
        del C
    if variant == "gaussian" and w.c_dtype == "bf16":
        # fp32 output of the same inputs meets the literal bound
        C64f, _ = oracle_rows(A, B, peers, "f32", rows)
        C = run(A, B, peers, "f32", "adaptive")
        check_tolerance(c_bits(C, rows), C64f, "f32", f"{w.name} f32 output", rms_ref=rms)
    del A, B, peers
    torch.cuda.empty_cache()


@pytest.mark.parametrize("ksplit", [-1, 1], ids=["ksplit-auto", "ksplit-off"])
def test_bitwise_invariance_across_reducer_counts(inplace_policy, ksplit):
    """Every reducer count gives the bits of the adaptive call; with the k-split off
    (one k-loop per tile) those are also the baseline's bits. (With early reduce this
    shape's tiles are split in two k-halves by default, whose fp32 sum rounds
    differently from one k-loop.)"""
    announce(f"invariance across reducer counts, k-split {ksplit}")
    M, N, K, npeer = 1024, 2048, 576, 7
    A, B, peers = mk_inputs.make_inputs(M, N, K, npeer, "bf16", "gaussian", 21, device=DEV)
    old = mk.get_option(mk.OPT_KSPLIT)
    mk.set_option(mk.OPT_KSPLIT, ksplit)
    try:
        G = mk.fused_grid(A, B, peers, new_c(M, N, "bf16"))
        ref = c_bits(run(A, B, peers, "bf16", "adaptive"))
        if ksplit == 1:
            check_exact(ref, c_bits(run(A, B, peers, "bf16", "baseline")), "adaptive vs baseline")
        for mode in ["0", "1", "4", "16", "64", str(G - 1)]:
            check_exact(c_bits(run(A, B, peers, "bf16", mode)), ref, f"mode {mode}")
    finally:
        mk.set_option(mk.OPT_KSPLIT, old)


INPLACE_SHAPES = [
    # M, N, K, n_peers, peer dtype, C dtype: 128x128 tiles with a ragged edge, 256x256
    # tiles (>= 256 of them), fp32 peers and C
    (300, 264, 200, 3, "bf16", "bf16"),
    (1024, 2048, 576, 7, "bf16", "bf16"),
    (4096, 4096, 256, 1, "bf16", "bf16"),
    (4096, 4096, 256, 3, "f32", "bf16"),
    (1024, 1024, 320, 4, "f32", "f32"),
]


@pytest.mark.parametrize("shape", INPLACE_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_inplace_reduce_matches_published(shape):
    """Tiles reduced in place (partial staged through LDS) give the same bits as tiles
    handed to reducers, and integer inputs stay exact against the oracle."""
    M, N, K, npeer, pdt, cdt = shape
    announce(f"in-place reduce {shape}")
    A, B, peers = mk_inputs.make_inputs(M, N, K, npeer, pdt, "integer", 61, device="cpu")
    rows = sample_rows(M)
    _, want = oracle_rows(A, B, peers, cdt, rows)
    A, B, peers = A.to(DEV), B.to(DEV), peers.to(DEV)
    old = mk.get_option(mk.OPT_INPLACE), mk.get_option(mk.OPT_EARLY)
    try:
        outs = {}
        for inplace in (-1, 0, 1 << 20):
            mk.set_option(mk.OPT_INPLACE, inplace)
            for early in (0, 1):
                mk.set_option(mk.OPT_EARLY, early)
                for nr in (None, 0, 8):
                    C = new_c(M, N, cdt)
                    mk.gemm_ar_local(A, B, peers, C, n_reduce_wg=nr)
                    mk.stream_status()
                    outs[(inplace, early, nr)] = (c_bits(C), c_bits(C, rows))
    finally:
        mk.set_option(mk.OPT_INPLACE, old[0])
        mk.set_option(mk.OPT_EARLY, old[1])
    ref = outs[(0, 0, None)][0]
    for key, (got, got_rows) in outs.items():
        check_exact(got, ref, f"in-place {key}")
        check_exact(got_rows, want, f"in-place {key} against the oracle")


TILE256_SHAPES = [  # M, N, K, n_peers, peer dtype, C dtype; ragged against 256 x 256 x 64
    (300, 264, 200, 3, "bf16", "bf16"),      # ragged M, N and K (K: three k-tiles and a tail)
    (520, 776, 1032, 1, "bf16", "f32"),      # K = 16 k-tiles and 8 columns
    (257, 520, 576, 7, "f32", "bf16"),       # k-halves of 288: a half ends inside a k-tile
    (512, 512, 640, 15, "bf16", "bf16"),     # whole tiles, k-halves of 320
]


@pytest.mark.parametrize("shape", TILE256_SHAPES, ids=lambda s: "x".join(map(str, s[:4])))
def test_256_tiles_on_ragged_shapes(shape):
    """The 256 x 256 tile (64-deep k-tiles, two LDS stages) on shapes ragged in M, N
    and K: integer inputs stay exact against the oracle under the default policy,
    with every tile handed over, with early reduce, with early reduce and k-halves,
    and in the two-kernel baseline."""
    M, N, K, npeer, pdt, cdt = shape
    announce(f"256 tiles {shape}")
    A, B, peers = mk_inputs.make_inputs(M, N, K, npeer, pdt, "integer", 71, device="cpu")
    _, want = oracle_rows(A, B, peers, cdt)
    A, B, peers = A.to(DEV), B.to(DEV), peers.to(DEV)
    opts = (mk.OPT_TILE_SHAPE, mk.OPT_INPLACE, mk.OPT_EARLY, mk.OPT_KSPLIT)
    old = [mk.get_option(o) for o in opts]
    try:
        mk.set_option(mk.OPT_TILE_SHAPE, 1)
        for inplace, early, ks in ((-1, -1, -1), (0, 0, 1), (0, 1, 1), (0, 1, 2)):
            if ks == 2 and K % 64 != 0:
                continue
            mk.set_option(mk.OPT_INPLACE, inplace)
            mk.set_option(mk.OPT_EARLY, early)
            mk.set_option(mk.OPT_KSPLIT, ks)
            for mode in ("adaptive", "0", "baseline"):
                C = run(A, B, peers, cdt, mode)
                check_exact(c_bits(C), want, f"{shape} inplace {inplace} early {early} ksplit {ks} {mode}")
    finally:
        for o, v in zip(opts, old):
            mk.set_option(o, v)


def test_back_to_back_alternating_inputs(inplace_policy):
    """Reducers must never read a partial before its flag: alternate two input sets so
    that any early read would pick up the other set's partial."""
    announce("alternating inputs")
    M, N, K, npeer = 768, 1024, 320, 3
    sets = []
    for s in (31, 32):
        A, B, peers = mk_inputs.make_inputs(M, N, K, npeer, "bf16", "integer", s, device="cpu")
        _, want = oracle_rows(A, B, peers, "bf16")
        sets.append((A.to(DEV), B.to(DEV), peers.to(DEV), want))
    C = new_c(M, N, "bf16")
    G = mk.fused_grid(sets[0][0], sets[0][1], sets[0][2], C)
    for i in range(60):
        A, B, peers, want = sets[i % 2]
        nr = [None, 0, G - 1, 8, min(200, G - 2)][i % 5]
        mk.gemm_ar_local(A, B, peers, C, n_reduce_wg=nr)
        if i % 2 == 1 or i > 50:
            mk.stream_status()
            check_exact(c_bits(C), want, f"call {i} reducers {nr}")
    mk.stream_status()


@pytest.mark.parametrize("early", [0, 1])
def test_withheld_flag_times_out_and_recovers(early):
    """Failure injection from the host: one tile's flag is never published; reducers
    give up after a short wait, the kernel exits normally, and the error is reported."""
    announce(f"withheld flag, early reduce {early}")
    M, N, K, npeer = 512, 512, 128, 2
    A, B, peers = mk_inputs.make_inputs(M, N, K, npeer, "bf16", "integer", 41, device="cpu")
    _, want = oracle_rows(A, B, peers, "bf16")
    A, B, peers = A.to(DEV), B.to(DEV), peers.to(DEV)
    C = new_c(M, N, "bf16")
    old = mk.get_option(mk.OPT_SPIN_TIMEOUT_US)
    old_inplace = mk.get_option(mk.OPT_INPLACE)
    old_early = mk.get_option(mk.OPT_EARLY)
    try:
        mk.set_option(mk.OPT_SPIN_TIMEOUT_US, 20000)
        mk.set_option(mk.OPT_INPLACE, 0)  # every tile handed over through its flag
        mk.set_option(mk.OPT_EARLY, early)
        mk.set_option(mk.OPT_WITHHOLD_TILE, 0)
        mk.gemm_ar_local(A, B, peers, C, n_reduce_wg=4)
        with pytest.raises(mk.MkError) as ei:
            mk.stream_status()
        assert ei.value.status == mk.MK_ERR_TIMEOUT
    finally:
        mk.set_option(mk.OPT_WITHHOLD_TILE, -1)
        mk.set_option(mk.OPT_SPIN_TIMEOUT_US, old)
        mk.set_option(mk.OPT_INPLACE, old_inplace)
        mk.set_option(mk.OPT_EARLY, old_early)
    mk.stream_status()  # error word was cleared
    mk.gemm_ar_local(A, B, peers, C)
    mk.stream_status()
    check_exact(c_bits(C), want, "after recovery")
    mk.workspace_reset()
    C2 = new_c(M, N, "bf16")
    mk.gemm_ar_local(A, B, peers, C2)
    mk.stream_status()
    check_exact(c_bits(C2), want, "after workspace reset")


def test_telemetry_and_controller_trace(inplace_policy):
    announce(f"telemetry, in-place policy {inplace_policy}")
    w = mk_inputs.BY_NAME["mlp"]
    A, B, peers = mk_inputs.workload_inputs(w, "gaussian", device=DEV)
    C = new_c(w.M, w.N, "bf16")
    tel = mk.new_telemetry()
    mk.gemm_ar_local(A, B, peers, C, telemetry=tel)
    mk.stream_status()
    # the call traced is checked too: bitwise the baseline, and sampled rows within
    # the tolerance rule against the oracle
    rows = sample_rows(w.M, seed=w.index)
    check_exact(c_bits(C), c_bits(run(A, B, peers, "bf16", "baseline")), "traced call vs baseline")
    C64, _ = oracle_rows(A, B, peers, "bf16", rows)
    check_tolerance(c_bits(C, rows), C64, "bf16", "traced call vs oracle")
    t = mk.read_telemetry(tel)
    G = mk.fused_grid(A, B, peers, C)
    assert t.tiles in ((w.M // 256) * (w.N // 256), (w.M // 128) * (w.N // 128))
    assert t.grid == G
    assert t.n_xcd == 8
    # with tiles reduced in place the derived cap keeps every workgroup computing
    # (target 0) while GEMM tiles remain; with every tile handed over, at least one
    # workgroup reduces
    lo = 0 if inplace_policy == -1 else 1
    assert lo <= t.initial_target <= G - 1
    assert lo <= t.final_target <= G
    assert 0 < t.n_trace <= mk.MK_TRACE_CAP
    assert t.t_end > t.t_start
    assert t.busy_compute > 0
    # every tile reduced in place counts as compute work; tiles handed over (or
    # reduced in place under dynamic hand-over) count as reduce work
    assert t.busy_reduce > 0 or inplace_policy == -1
    targets = [t.trace[i].target for i in range(t.n_trace)]
    computed = [t.trace[i].computed for i in range(t.n_trace)]
    assert all(a <= b for a, b in zip(computed, computed[1:]))
    assert all(lo <= x <= G for x in targets)
    # once every tile is computed the controller hands all workgroups to the reduce
    assert all(t.trace[i].target == G for i in range(t.n_trace) if computed[i] == t.tiles)
    # flag-overhead timers: every tile handed over is published once and each of its
    # reduce units (64-row slabs) acquires once; tiles reduced in place use no flag
    rsplit = 4 if t.tiles == (w.M // 256) * (w.N // 256) else 2
    if inplace_policy == -1:
        assert t.published == 0 and t.acquired == 0
        assert t.publish_ticks == 0 and t.acquire_ticks == 0
    elif inplace_policy == 0:
        assert t.published == t.tiles and t.acquired == t.tiles * rsplit
        assert t.publish_ticks > 0
    else:
        assert 0 <= t.published <= t.tiles and 0 <= t.acquired <= t.tiles * rsplit
    # an acquire ends after its poll, within the call
    assert t.acquire_ticks <= t.wait_reduce


@pytest.mark.parametrize("name", ["mlp", "attn"])
@pytest.mark.parametrize("variant", ["integer", "gaussian"])
def test_role_split_at_full_size(name, variant):
    """The role-split path at full size: every tile handed to reducers through its
    flag (MK_OPT_INPLACE=0), so that reducers wait on flags, hold units, compute when
    nothing is ready and follow the controller over several rounds of tiles (mlp: two
    rounds of 256 tiles on 256 workgroups; attn: eight). Adaptive, 0 and 64 reducers,
    and adaptive under agent-scope flags: sampled rows against the oracle (bit-exact on
    integer inputs, the tolerance rule on Gaussian ones), every element bitwise
    against the two-kernel baseline."""
    w = mk_inputs.BY_NAME[name]
    A, B, peers = mk_inputs.workload_inputs(w, variant, device=DEV)
    rows = sample_rows(w.M, seed=w.index)
    C64, want = oracle_rows(A, B, peers, w.c_dtype, rows)
    rms = float(np.sqrt(np.mean(C64 * C64)))
    ref = c_bits(run(A, B, peers, w.c_dtype, "baseline"))
    opts = (mk.OPT_INPLACE, mk.OPT_FLAG_SCOPE)
    old = [mk.get_option(o) for o in opts]
    try:
        mk.set_option(mk.OPT_INPLACE, 0)
        for scope, mode, policy in ((0, "adaptive", 0), (0, "0", 0), (0, "64", 0),
                                    (1, "adaptive", 0), (0, "adaptive", -2), (0, "64", -2)):
            announce(f"role split {name} {variant} reducers {mode} flag scope {scope} "
                     f"policy {policy}")
            mk.set_option(mk.OPT_FLAG_SCOPE, scope)
            mk.set_option(mk.OPT_INPLACE, policy)
            C = run(A, B, peers, w.c_dtype, mode)
            check_exact(c_bits(C), ref, f"{name} {mode} scope {scope} vs baseline")
            got = c_bits(C, rows)
            if variant == "integer":
                check_exact(got, want, f"{name} {mode} scope {scope} vs oracle")
            else:
                check_tolerance(got, C64, w.c_dtype, f"{name} {mode} scope {scope}", rms_ref=rms)
            del C
    finally:
        for o, v in zip(opts, old):
            mk.set_option(o, v)
    del A, B, peers
    torch.cuda.empty_cache()


def test_early_reduce_grid_and_parity_on_a_decode_shard():
    """With 128x128 tiles, a shard whose tiles and reduce units fit one round of
    workgroups gets early reduce automatically: one workgroup per tile plus one per
    64-row reduce unit. The result is the same bits as with early reduce off and as
    the baseline."""
    announce("early reduce on a decode-sized shard")
    M, N, K, npeer = 128, 2048, 448, 15
    A, B, peers = mk_inputs.make_inputs(M, N, K, npeer, "bf16", "integer", 71, device="cpu")
    _, want = oracle_rows(A, B, peers, "bf16")
    A, B, peers = A.to(DEV), B.to(DEV), peers.to(DEV)
    C = new_c(M, N, "bf16")
    tiles = (M // 128) * (N // 128)
    old = mk.get_option(mk.OPT_EARLY), mk.get_option(mk.OPT_TILE_SHAPE)
    try:
        mk.set_option(mk.OPT_TILE_SHAPE, 2)
        assert mk.fused_grid(A, B, peers, C) == tiles * 3  # 128x128 tiles, 2 units each
        mk.set_option(mk.OPT_EARLY, 0)
        assert mk.fused_grid(A, B, peers, C) == tiles * 2
        off = c_bits(run(A, B, peers, "bf16", "adaptive"))
        mk.set_option(mk.OPT_EARLY, old[0])
        for mode in ["adaptive", "0", str(tiles * 2), "baseline"]:
            got = c_bits(run(A, B, peers, "bf16", mode))
            check_exact(got, want, f"early reduce {mode}")
            check_exact(got, off, f"early reduce {mode} against early off")
    finally:
        mk.set_option(mk.OPT_EARLY, old[0])
        mk.set_option(mk.OPT_TILE_SHAPE, old[1])


@pytest.mark.parametrize("shape", [(128, 8192, 1792, 15, "bf16", "bf16"),
                                   (256, 512, 512, 3, "f32", "f32"),
                                   (200, 4104, 136, 7, "bf16", "f32"),
                                   (64, 64, 64, 1, "bf16", "bf16")],
                         ids=lambda s: "x".join(map(str, s[:4])))
def test_few_tile_shapes_take_64_tiles_in_place(shape):
    """Shapes with fewer 128x128 tiles than compute units take 64x64 tiles, each
    computed and reduced in place by one workgroup (the grid is one workgroup per
    tile): integer inputs bit-exact against the oracle, and bitwise equal to the
    baseline, to 128x128 tiles with early reduce and k-halves (exact on integers),
    and to the same call with telemetry (which takes the persistent loop)."""
    M, N, K, npeer, pdt, cdt = shape
    announce(f"64x64 tiles in place {shape}")
    A, B, peers = mk_inputs.make_inputs(M, N, K, npeer, pdt, "integer", 91, device="cpu")
    rows = sample_rows(M)
    _, want = oracle_rows(A, B, peers, cdt, rows)
    A, B, peers = A.to(DEV), B.to(DEV), peers.to(DEV)
    C = new_c(M, N, cdt)
    tiles = ((M + 63) // 64) * ((N + 63) // 64)
    assert mk.fused_grid(A, B, peers, C) == min(max(tiles, 8), 2 * mk.num_workgroups())
    ref = c_bits(run(A, B, peers, cdt, "adaptive"))
    check_exact(ref[rows], want, "64x64 tiles against the oracle")
    check_exact(c_bits(run(A, B, peers, cdt, "baseline")), ref, "baseline")
    tel = mk.new_telemetry()
    C2 = new_c(M, N, cdt)
    mk.gemm_ar_local(A, B, peers, C2, telemetry=tel)
    mk.stream_status()
    check_exact(c_bits(C2), ref, "with telemetry (persistent loop)")
    assert mk.read_telemetry(tel).tiles == tiles
    old = mk.get_option(mk.OPT_TILE_SHAPE)
    try:
        mk.set_option(mk.OPT_TILE_SHAPE, 2)
        check_exact(c_bits(run(A, B, peers, cdt, "adaptive")), ref, "128x128 tiles")
    finally:
        mk.set_option(mk.OPT_TILE_SHAPE, old)


WS_SHAPES = [  # several rounds per workgroup, ragged edges, every ring peer count
    (2100, 2056, 136, 15, "bf16", "bf16"),
    (2176, 2048, 64, 8, "f32", "f32"),
    (1000, 1032, 1000, 1, "bf16", "bf16"),
    (4224, 4096, 40, 4, "bf16", "f32"),
    (4160, 2312, 104, 7, "f32", "bf16"),
    (1088, 4160, 96, 2, "bf16", "bf16"),
    (2112, 2304, 72, 3, "f32", "f32"),
]


@pytest.mark.parametrize("tile", [4, 5], ids=["64x256", "128x128"])
@pytest.mark.parametrize("shape", WS_SHAPES, ids=lambda s: "x".join(map(str, s[:4])) + f"-{s[4]}")
def test_wave_specialised_schedule(shape, tile):
    """The wave-specialised kernel (MK_OPT_TILE_SHAPE=4: 64x256 tiles, 5: 128x128) on
    shapes where each of the 256 workgroups runs several rounds (the GEMM of one
    tile while the tile before is reduced from LDS): integer inputs bit-exact against the oracle on
    sampled rows and bitwise equal to the two-kernel baseline and to the default
    schedule over the whole output, twice in a row (the LDS hand-over starts clean
    in every call); Gaussian inputs within tolerance."""
    M, N, K, npeer, pdt, cdt = shape
    announce(f"wave-specialised {shape} tile option {tile}")
    rows = sample_rows(M, band=128, seed=M)
    A, B, peers = mk_inputs.make_inputs(M, N, K, npeer, pdt, "integer", 17, device="cpu")
    _, want = oracle_rows(A, B, peers, cdt, rows)
    A, B, peers = A.to(DEV), B.to(DEV), peers.to(DEV)
    ref = c_bits(run(A, B, peers, cdt, "baseline"))
    check_exact(ref[rows], want, "baseline against the oracle")
    check_exact(c_bits(run(A, B, peers, cdt, "adaptive")), ref, "default schedule")
    old = mk.get_option(mk.OPT_TILE_SHAPE)
    try:
        mk.set_option(mk.OPT_TILE_SHAPE, tile)
        for rep in range(2):
            check_exact(c_bits(run(A, B, peers, cdt, "adaptive")), ref, f"wave-specialised {rep}")
        A, B, peers = mk_inputs.make_inputs(M, N, K, npeer, pdt, "gaussian", 18, device="cpu")
        C64, _ = oracle_rows(A, B, peers, cdt, rows)
        A, B, peers = A.to(DEV), B.to(DEV), peers.to(DEV)
        got = c_bits(run(A, B, peers, cdt, "adaptive"), rows)
        check_tolerance(got, C64, cdt, "wave-specialised gaussian",
                        rms_ref=float(np.sqrt(np.mean(C64 * C64))))
    finally:
        mk.set_option(mk.OPT_TILE_SHAPE, old)


STATIC_SHAPES = [  # M, N, K, n_peers, peer dtype, C dtype: more 256x256 tiles than workgroups
    (4608, 4096, 2176, 7, "bf16", "bf16"),   # 288 tiles: 256 workgroups, a second round for 32
    (4600, 4104, 2120, 3, "bf16", "f32"),    # ragged M, N and K
    (4608, 4096, 1024, 15, "bf16", "bf16"),  # 15 peers
    (4608, 4096, 1024, 7, "f32", "bf16"),    # float32 peers
    (8448, 8192, 64, 1, "bf16", "bf16"),     # 1056 tiles (five rounds), one k-tile
]


@pytest.mark.parametrize("shape", STATIC_SHAPES, ids=lambda s: "x".join(map(str, s[:4])) + f"-{s[4]}")
def test_inplace_kernel_matches_claim_queues(shape):
    """256x256 tiles all reduced in place with more tiles than workgroups: the
    in-place kernel (each XCD's tiles dealt to its workgroups in a fixed order)
    with eight waves where they fit (MK_OPT_STATIC_TILES=2, the default) and with
    four (1), and the persistent kernel's per-XCD claim queues (0). Integer inputs bit-exact against the oracle on sampled rows and
    bitwise equal to the two-kernel baseline over the whole output, twice in a
    row; the baseline itself with its GEMM on the 256x256 tile of eight waves
    (option 2) and of four (1, 0) gives the same bits. Gaussian inputs within
    tolerance."""
    M, N, K, npeer, pdt, cdt = shape
    announce(f"in-place kernel {shape}")
    rows = sample_rows(M, band=256, seed=M + K)
    A, B, peers = mk_inputs.make_inputs(M, N, K, npeer, pdt, "integer", 27, device="cpu")
    _, want = oracle_rows(A, B, peers, cdt, rows)
    A, B, peers = A.to(DEV), B.to(DEV), peers.to(DEV)
    ref = c_bits(run(A, B, peers, cdt, "baseline"))
    check_exact(ref[rows], want, "baseline against the oracle")
    opts = (mk.OPT_TILE_SHAPE, mk.OPT_STATIC_TILES)
    old = [mk.get_option(o) for o in opts]
    try:
        mk.set_option(mk.OPT_TILE_SHAPE, 1)
        for static in (2, 1, 0, 2):
            mk.set_option(mk.OPT_STATIC_TILES, static)
            for rep in range(2):
                check_exact(c_bits(run(A, B, peers, cdt, "adaptive")), ref, f"static tiles {static} call {rep}")
            check_exact(c_bits(run(A, B, peers, cdt, "baseline")), ref,
                        f"baseline, 256x256 GEMM tiles, static tiles {static}")
        A, B, peers = mk_inputs.make_inputs(M, N, K, npeer, pdt, "gaussian", 28, device="cpu")
        C64, _ = oracle_rows(A, B, peers, cdt, rows)
        A, B, peers = A.to(DEV), B.to(DEV), peers.to(DEV)
        got = c_bits(run(A, B, peers, cdt, "adaptive"), rows)
        check_tolerance(got, C64, cdt, "in-place kernel gaussian",
                        rms_ref=float(np.sqrt(np.mean(C64 * C64))))
    finally:
        for o, v in zip(opts, old):
            mk.set_option(o, v)


ZERO_PEER_CASES = [  # M, N, K, C dtype, MK_OPT_TILE_SHAPE: no peers (C = round(A*B)), every in-place path
    (4608, 4096, 256, "bf16", 1),   # 288 tiles of 256x256: the in-place kernel
    (4608, 4096, 256, "f32", 0),    # automatic
    (2100, 2056, 136, "bf16", 4),   # wave-specialised, 64x256 (rounded partial streamed from LDS)
    (2100, 2056, 136, "f32", 5),    # wave-specialised, 128x128
    (1000, 1032, 1000, "bf16", 2),  # 128x128 tiles in place
    (300, 264, 200, "f32", 3),      # 64x64 tiles, one per workgroup
]


@pytest.mark.parametrize("case", ZERO_PEER_CASES, ids=lambda c: "x".join(map(str, c)))
def test_zero_peers_reduced_in_place(case):
    """A call with no peers (one GPU: C = round(A*B)) reduces its tiles in place
    like any other peer count: integer inputs bit-exact against the oracle on
    sampled rows and bitwise equal to the two-kernel baseline, twice in a row."""
    M, N, K, cdt, shape = case
    announce(f"zero peers {case}")
    rows = sample_rows(M, band=256, seed=M + N)
    A, B, peers = mk_inputs.make_inputs(M, N, K, 0, "bf16", "integer", 37, device="cpu")
    _, want = oracle_rows(A, B, None, cdt, rows)
    A, B = A.to(DEV), B.to(DEV)
    ref = c_bits(run(A, B, None, cdt, "baseline"))
    check_exact(ref[rows], want, "baseline against the oracle")
    old = mk.get_option(mk.OPT_TILE_SHAPE)
    try:
        mk.set_option(mk.OPT_TILE_SHAPE, shape)
        for rep in range(2):
            check_exact(c_bits(run(A, B, None, cdt, "adaptive")), ref, f"tile option {shape} call {rep}")
    finally:
        mk.set_option(mk.OPT_TILE_SHAPE, old)


def test_automatic_schedule_per_workload():
    """The automatic choice on MI355X (256 CUs): few-tile shapes take 64x64 tiles
    in place, stream-dominated ones the wave-specialised kernel (64x256 tiles for
    attn, 128x128 for mlp), the compute-bound shard 256x256 tiles in place; an
    explicit schedule option or a forced shape is honoured."""
    want = {"tiny": 3, "decode": 3, "mlp": 5, "attn": 4, "large": 1}
    for w in mk_inputs.WORKLOADS:
        A = torch.empty((w.M, w.K), dtype=torch.bfloat16, device=DEV)
        B = torch.empty((w.K, w.N), dtype=torch.bfloat16, device=DEV)
        peers = torch.empty((w.n_peers, w.M, w.N), dtype=TORCH_DT[w.peer_dtype], device=DEV)
        C = torch.empty((w.M, w.N), dtype=TORCH_DT[w.c_dtype], device=DEV)
        assert mk.fused_schedule(A, B, peers, C) == want[w.name], w.name
        if w.name == "attn":
            old = mk.get_option(mk.OPT_INPLACE), mk.get_option(mk.OPT_TILE_SHAPE)
            try:
                mk.set_option(mk.OPT_INPLACE, 0)  # an explicit schedule keeps the role split
                assert mk.fused_schedule(A, B, peers, C) == 1
                mk.set_option(mk.OPT_INPLACE, -1)
                mk.set_option(mk.OPT_TILE_SHAPE, 2)
                assert mk.fused_schedule(A, B, peers, C) == 2
            finally:
                mk.set_option(mk.OPT_INPLACE, old[0])
                mk.set_option(mk.OPT_TILE_SHAPE, old[1])
        del A, B, peers, C


TWO_STREAM_SHAPES = [
    # M, N, K, n_peers, peer dtype, C dtype: one tile row, ragged rows, 256x256 tiles
    (256, 512, 512, 3, "f32", "f32"),
    (300, 264, 200, 3, "bf16", "bf16"),
    (1000, 776, 264, 7, "bf16", "f32"),
    (2304, 2048, 512, 15, "bf16", "bf16"),
    (130, 136, 72, 0, "bf16", "bf16"),
]


@pytest.mark.parametrize("shape", TWO_STREAM_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_two_stream_schedule_matches_baseline(shape):
    """The stream-overlap schedule (per-chunk GEMM kernels, per-chunk reduces on a
    second stream) gives the baseline's bits for every chunk count, and integer
    inputs stay exact against the oracle."""
    M, N, K, npeer, pdt, cdt = shape
    announce(f"two-stream schedule {shape}")
    A, B, peers = mk_inputs.make_inputs(M, N, K, npeer, pdt, "integer", 81, device="cpu")
    rows = sample_rows(M)
    _, want = oracle_rows(A, B, peers, cdt, rows)
    A, B, peers = A.to(DEV), B.to(DEV), peers.to(DEV)
    ref = c_bits(run(A, B, peers, cdt, "baseline"))
    for chunks in (0, 1, 2, 3, 64):
        C = new_c(M, N, cdt)
        mk.gemm_ar_two_stream(A, B, peers, C, n_chunks=chunks)
        mk.stream_status()
        check_exact(c_bits(C), ref, f"{chunks} chunks against the baseline")
        check_exact(c_bits(C, rows), want, f"{chunks} chunks against the oracle")


@pytest.mark.parametrize("shape", TWO_STREAM_SHAPES[1:4], ids=lambda s: "x".join(map(str, s)))
def test_two_stream_cu_masked_matches_baseline(shape):
    """The two-stream schedule on CU-masked streams (MK_OPT_STREAM_CU_SPLIT: the
    GEMM and reduce kernels on disjoint sets of compute units) gives the baseline's
    bits for several splits, switched between calls and back to unmasked streams;
    integer inputs stay exact against the oracle. A split that does not fit the
    device is refused at the call."""
    M, N, K, npeer, pdt, cdt = shape
    announce(f"two-stream CU-masked {shape}")
    A, B, peers = mk_inputs.make_inputs(M, N, K, npeer, pdt, "integer", 83, device="cpu")
    rows = sample_rows(M)
    _, want = oracle_rows(A, B, peers, cdt, rows)
    A, B, peers = A.to(DEV), B.to(DEV), peers.to(DEV)
    ref = c_bits(run(A, B, peers, cdt, "baseline"))
    cus = mk.num_workgroups()  # resident 256x256 workgroups: one per compute unit
    old = mk.get_option(mk.OPT_STREAM_CU_SPLIT)
    try:
        for split in (cus // 4, cus // 2, 3 * cus // 4, cus // 4, 0):
            mk.set_option(mk.OPT_STREAM_CU_SPLIT, split)
            for chunks in (0, 3):
                C = new_c(M, N, cdt)
                mk.gemm_ar_two_stream(A, B, peers, C, n_chunks=chunks)
                mk.stream_status()
                check_exact(c_bits(C), ref, f"split {split}, {chunks} chunks against the baseline")
                check_exact(c_bits(C, rows), want, f"split {split}, {chunks} chunks against the oracle")
        for bad in (cus // 4 + 8, cus):
            mk.set_option(mk.OPT_STREAM_CU_SPLIT, bad)
            C = new_c(M, N, cdt)
            with pytest.raises(mk.MkError):
                mk.gemm_ar_two_stream(A, B, peers, C)
    finally:
        mk.set_option(mk.OPT_STREAM_CU_SPLIT, old)
    mk.stream_status()


def test_two_stream_then_fused_on_one_stream():
    """The two schedules share the stream's partial buffer: back-to-back calls with
    alternating inputs must each see only their own partials."""
    announce("two-stream and fused calls alternating")
    M, N, K, npeer = 768, 1024, 320, 3
    sets = []
    for s in (91, 92):
        A, B, peers = mk_inputs.make_inputs(M, N, K, npeer, "bf16", "integer", s, device="cpu")
        _, want = oracle_rows(A, B, peers, "bf16")
        sets.append((A.to(DEV), B.to(DEV), peers.to(DEV), want))
    outs = [new_c(M, N, "bf16") for _ in range(4)]
    for i in range(4):
        A, B, peers, _ = sets[i % 2]
        if i < 2:
            mk.gemm_ar_two_stream(A, B, peers, outs[i], n_chunks=3)
        else:
            mk.gemm_ar_local(A, B, peers, outs[i])
    mk.stream_status()
    for i in range(4):
        check_exact(c_bits(outs[i]), sets[i % 2][3], f"call {i}")


RS_CASES = [
    # M, N, K, n_peers, peer dtype, C dtype, owned rows [o0, o1)
    (520, 776, 264, 3, "bf16", "bf16", 128, 256),   # whole 128-row tiles
    (520, 776, 264, 3, "bf16", "bf16", 100, 300),   # owned rows cut through tiles
    (300, 264, 200, 15, "bf16", "f32", 0, 19),      # first rows, ragged everything
    (300, 264, 200, 7, "f32", "bf16", 281, 300),    # last rows
    (256, 512, 512, 1, "f32", "f32", 0, 256),       # every row owned: nothing published
    (256, 512, 512, 2, "bf16", "bf16", 77, 77),     # nothing owned: everything published
    (130, 136, 72, 0, "bf16", "bf16", 64, 130),     # no peers
    (1024, 2048, 576, 15, "bf16", "bf16", 192, 448),  # 256x256 tiles
    (300, 264, 200, 5, "bf16", "bf16", 10, 150),     # a peer count without a compile-time ring
]


def rs_poisoned(M, N, own, pdt, cdt):
    C = new_c(own, N, cdt)
    send = new_c(M, N, pdt)
    return C, send


@pytest.mark.parametrize("case", RS_CASES, ids=lambda c: "x".join(map(str, c)))
def test_reduce_scatter_share(case):
    """One GPU's share of GEMM+ReduceScatter: owned rows reduced, other rows published
    in the peer type. Integer inputs: bit-exact against the oracle, for the fused
    kernel and the baseline; rows of send that this GPU owns are left untouched."""
    M, N, K, npeer, pdt, cdt, o0, o1 = case
    announce(f"reduce-scatter share {case}")
    own = o1 - o0
    A, B, peers = mk_inputs.make_inputs(M, N, K, npeer, pdt, "integer", 101, device="cpu")
    peers = peers[:, o0:o1].contiguous()
    (owned, _, c_want), (other, _, s_want) = oracle.gemm_rs(
        mk_inputs.bits(A), mk_inputs.bits(B), mk_inputs.bits(peers) if npeer else None, o0, o1,
        cdt, pdt)
    A, B, peers = A.to(DEV), B.to(DEV), peers.to(DEV)
    outs = []
    runs = [(f"fused, reducers {nr}", lambda C, send, nr=nr: mk.gemm_rs_local(
        A, B, peers, C, send, o0, o1, n_reduce_wg=nr)) for nr in (None, 0, 4)]
    runs.append(("baseline", lambda C, send: mk.gemm_rs_baseline(A, B, peers, C, send, o0, o1)))
    for name, fn in runs:
        C, send = rs_poisoned(M, N, own, pdt, cdt)
        fn(C, send)
        mk.stream_status()
        cb, sb = c_bits(C), c_bits(send)
        check_exact(cb, c_want, f"{name} owned rows")
        check_exact(sb[other], s_want, f"{name} published rows")
        poison = 0x7FC1 if pdt == "bf16" else 0x7FC00001
        assert np.all(sb[o0:o1].view(np.uint16 if pdt == "bf16" else np.uint32) == poison)
        outs.append((cb, sb))
    for cb, sb in outs[:-1]:
        check_exact(cb, outs[-1][0], "fused against baseline, owned rows")
        check_exact(sb, outs[-1][1], "fused against baseline, send")


def test_reduce_scatter_share_gaussian_full_size():
    """The mlp workload's GEMM (4096x8192x1792, bf16 peers and C) as a ReduceScatter
    share of a 16-GPU group that owns rows [768, 1024): sampled rows against the oracle
    (tolerance rule for C, the same rule in the peer type for send), bitwise against
    the baseline."""
    w = mk_inputs.BY_NAME["mlp"]
    announce("reduce-scatter share, mlp size")
    A, B, peers_all = mk_inputs.workload_inputs(w, "gaussian", device=DEV)
    o0, o1 = 768, 1024
    peers = peers_all[:, o0:o1].contiguous()
    del peers_all
    rows = sample_rows(w.M)
    (owned, c64, _), (other, s64, _) = oracle.gemm_rs(
        mk_inputs.bits(A.cpu()), mk_inputs.bits(B.cpu()), mk_inputs.bits(peers.cpu()), o0, o1,
        "bf16", "bf16", rows=rows)
    outs = []
    for fn in (mk.gemm_rs_local, mk.gemm_rs_baseline):
        C, send = rs_poisoned(w.M, w.N, o1 - o0, "bf16", "bf16")
        fn(A, B, peers, C, send, o0, o1)
        mk.stream_status()
        cb, sb = c_bits(C), c_bits(send)
        check_tolerance(cb[owned - o0], c64, "bf16", f"{fn.__name__} owned rows")
        check_tolerance(sb[other], s64, "bf16", f"{fn.__name__} published rows")
        outs.append((cb, sb))
    check_exact(outs[0][0], outs[1][0], "fused against baseline, owned rows")
    check_exact(outs[0][1], outs[1][1], "fused against baseline, send")


AG_CASES = [
    # Ms (rows per GPU), P, N, K, rank, C dtype
    (128, 4, 264, 200, 1, "bf16"),     # ragged N, partial k-tile
    (256, 3, 512, 512, 0, "f32"),
    (128, 1, 136, 64, 0, "bf16"),      # no peers: the gather is a copy
    (128, 16, 256, 72, 15, "bf16"),    # last rank, many bands
    (384, 2, 136, 1040, 1, "f32"),
    (128, 5, 8, 8, 2, "bf16"),         # the smallest N and K
    (256, 4, 2048, 576, 3, "bf16"),
    (128, 3, 64, 0, 1, "bf16"),        # K = 0: nothing to gather, C = 0
    (128, 2, 0, 64, 0, "f32"),         # N = 0: the gather alone
]


def ag_poisoned(M, N, K, cdt):
    A_full = torch.empty((M, K), dtype=torch.bfloat16, device=DEV)
    A_full.view(torch.int16).fill_(0x7FC1)
    return A_full, new_c(M, N, cdt)


@pytest.mark.parametrize("shape_opt", [0, 1], ids=["auto-tiles", "256-tiles"])
@pytest.mark.parametrize("case", AG_CASES, ids=lambda c: "x".join(map(str, c)))
def test_allgather_share(case, shape_opt):
    """One GPU's share of AllGather+GEMM ("AllGather + GEMM (TP)" row of Table 3).
    Integer inputs: the gathered matrix and C bit-exact against the oracle, for the
    fused kernel with the default, no and the most landing workgroups, and for the
    baseline."""
    Ms, P, N, K, rank, cdt = case
    if shape_opt == 1 and Ms % 256 != 0:
        pytest.skip("256-row bands need Ms a multiple of 256")
    announce(f"allgather share {case} tile option {shape_opt}")
    shards, B = mk_inputs.make_ag_inputs(Ms, P, N, K, "integer", 201, device="cpu")
    A_local, peers_A = mk_inputs.shard_split(shards, rank)
    f_want, _, c_want = oracle.gemm_ag(mk_inputs.bits(A_local), mk_inputs.bits(peers_A), rank,
                                       mk_inputs.bits(B), cdt)
    A_local, peers_A, B = A_local.to(DEV), peers_A.to(DEV), B.to(DEV)
    old = mk.get_option(mk.OPT_TILE_SHAPE)
    mk.set_option(mk.OPT_TILE_SHAPE, shape_opt)
    try:
        A_full, C = ag_poisoned(P * Ms, N, K, cdt)
        G = mk.ag_grid(A_local, peers_A, A_full, B, C)
        runs = [(f"fused, landing {nc}", lambda F, C, nc=nc: mk.gemm_ag_local(
            A_local, peers_A, F, B, C, rank, n_comm_wg=nc)) for nc in (None, 0, G - 1)]
        runs.append(("baseline", lambda F, C: mk.gemm_ag_baseline(A_local, peers_A, F, B, C,
                                                                   rank)))
        for name, fn in runs:
            A_full, C = ag_poisoned(P * Ms, N, K, cdt)
            fn(A_full, C)
            mk.stream_status()
            check_exact(mk_inputs.bits(A_full), f_want, f"{name} gathered matrix")
            check_exact(c_bits(C), c_want, f"{name} C")
    finally:
        mk.set_option(mk.OPT_TILE_SHAPE, old)


def test_allgather_share_gaussian_and_alternating_ranks():
    """Gaussian inputs within the tolerance rule; then calls that alternate the rank
    (and so which bands are local and which XCD lands each band) on the same
    buffers, each checked bitwise against the baseline of the same rank."""
    Ms, P, N, K = 256, 6, 776, 520
    announce(f"allgather share gaussian {Ms}x{P}x{N}x{K}")
    shards, B = mk_inputs.make_ag_inputs(Ms, P, N, K, "gaussian", 202, device="cpu")
    Bd = B.to(DEV)
    A_full, C = ag_poisoned(P * Ms, N, K, "bf16")
    A_ref, C_ref = ag_poisoned(P * Ms, N, K, "bf16")
    for i, rank in enumerate([2, 5, 0, 2, 3]):
        A_local, peers_A = mk_inputs.shard_split(shards, rank)
        if i == 0:
            _, c64, _ = oracle.gemm_ag(mk_inputs.bits(A_local), mk_inputs.bits(peers_A), rank,
                                       mk_inputs.bits(B), "bf16")
        A_local, peers_A = A_local.to(DEV), peers_A.to(DEV)
        mk.gemm_ag_local(A_local, peers_A, A_full, Bd, C, rank)
        mk.gemm_ag_baseline(A_local, peers_A, A_ref, Bd, C_ref, rank)
        mk.stream_status()
        if i == 0:
            check_tolerance(c_bits(C), c64, "bf16", "fused gaussian")
        check_exact(mk_inputs.bits(A_full), mk_inputs.bits(shards.reshape(P * Ms, K)),
                    f"gathered matrix, rank {rank}")
        check_exact(c_bits(C), c_bits(C_ref), f"fused against baseline, rank {rank}")


def test_allgather_share_full_size():
    """The ag_up workload (16 GPUs x 256 rows, K=8192, N=3584, bf16): sampled rows of C
    against the oracle (tolerance rule), the gathered matrix and C bitwise against the
    baseline."""
    w = mk_inputs.AG_BY_NAME["ag_up"]
    rank = 5
    announce(f"allgather share, {w.name} size")
    shards, B = mk_inputs.make_ag_inputs(w.Ms, w.P, w.N, w.K, "gaussian", 1000 * w.index,
                                         device=DEV)
    A_local, peers_A = mk_inputs.shard_split(shards, rank)
    rows = sample_rows(w.M)
    _, c64, _ = oracle.gemm_ag(mk_inputs.bits(A_local), mk_inputs.bits(peers_A), rank,
                               mk_inputs.bits(B), "bf16", rows=rows)
    outs = []
    for fn in (mk.gemm_ag_local, mk.gemm_ag_baseline):
        A_full, C = ag_poisoned(w.M, w.N, w.K, "bf16")
        fn(A_local, peers_A, A_full, B, C, rank)
        mk.stream_status()
        cb = c_bits(C)
        check_tolerance(cb[rows], c64, "bf16", f"{fn.__name__} sampled rows")
        outs.append((mk_inputs.bits(A_full), cb))
    check_exact(outs[0][0], mk_inputs.bits(shards.reshape(w.M, w.K)), "gathered matrix")
    check_exact(outs[0][0], outs[1][0], "fused against baseline, gathered matrix")
    check_exact(outs[0][1], outs[1][1], "fused against baseline, C")


@pytest.mark.parametrize("variant", ["integer", "gaussian"])
def test_ksplit_on_a_decode_shard(variant):
    """Early-reduce shards with K a multiple of 64 and at least 512 compute each tile
    as two k-halves (MK_OPT_KSPLIT automatic): the grid holds two workgroups per tile
    plus one per reduce unit. Integer inputs: bit-exact against the oracle with the
    split on and off and for the baseline. Gaussian inputs: within the tolerance rule
    (the sum of the two halves' fp32 partials rounds differently from one k-loop)."""
    announce(f"k-split on a decode shard, {variant}")
    M, N, K, npeer = 128, 2048, 1792, 15
    A, B, peers = mk_inputs.make_inputs(M, N, K, npeer, "bf16", variant, 73, device="cpu")
    C64, want = oracle_rows(A, B, peers, "bf16")
    A, B, peers = A.to(DEV), B.to(DEV), peers.to(DEV)
    tiles = (M // 128) * (N // 128)
    old = mk.get_option(mk.OPT_KSPLIT), mk.get_option(mk.OPT_TILE_SHAPE)
    try:
        mk.set_option(mk.OPT_TILE_SHAPE, 2)  # early reduce and k-halves are for 128x128 tiles
        outs = {}
        for ks, grid in ((-1, tiles * 4), (2, tiles * 4), (1, tiles * 3)):
            mk.set_option(mk.OPT_KSPLIT, ks)
            assert mk.fused_grid(A, B, peers, new_c(M, N, "bf16")) == grid, ks
            for mode in ("adaptive", "0"):
                outs[(ks, mode)] = c_bits(run(A, B, peers, "bf16", mode))
        outs["baseline"] = c_bits(run(A, B, peers, "bf16", "baseline"))
    finally:
        mk.set_option(mk.OPT_KSPLIT, old[0])
        mk.set_option(mk.OPT_TILE_SHAPE, old[1])
    for key, got in outs.items():
        if variant == "integer":
            check_exact(got, want, f"k-split {key}")
        else:
            check_tolerance(got, C64, "bf16", f"k-split {key}")
    check_exact(outs[(-1, "adaptive")], outs[(2, "0")], "split calls agree bitwise")
    check_exact(outs[(1, "adaptive")], outs["baseline"], "unsplit call against the baseline")


def test_concurrent_calls_on_two_streams():
    """Two fused calls (and an AllGather share) in flight at once on two streams,
    each with its own workspace and each sized for the whole GPU: every wait is on
    work claimed by a running workgroup, so neither can stall the other; integer
    inputs stay bit-exact."""
    announce("concurrent calls on two streams")
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    cases = []
    for seed, (M, N, K, npeer) in ((41, (1024, 2048, 576, 7)), (42, (768, 1024, 1792, 15))):
        A, B, peers = mk_inputs.make_inputs(M, N, K, npeer, "bf16", "integer", seed, device="cpu")
        _, want = oracle_rows(A, B, peers, "bf16")
        cases.append((A.to(DEV), B.to(DEV), peers.to(DEV), want, new_c(M, N, "bf16")))
    shards, Bag = mk_inputs.make_ag_inputs(256, 4, 1024, 512, "integer", 43, device="cpu")
    A_loc, peers_A = mk_inputs.shard_split(shards, 2)
    f_want, _, c_want = oracle.gemm_ag(mk_inputs.bits(A_loc), mk_inputs.bits(peers_A), 2,
                                       mk_inputs.bits(Bag), "bf16")
    A_loc, peers_A, Bag = A_loc.to(DEV), peers_A.to(DEV), Bag.to(DEV)
    A_full, C_ag = ag_poisoned(1024, 1024, 512, "bf16")
    torch.cuda.synchronize()
    for rep in range(5):
        (A1, B1, P1, _, C1), (A2, B2, P2, _, C2) = cases
        with torch.cuda.stream(s1):
            mk.gemm_ar_local(A1, B1, P1, C1, stream=s1)
            mk.gemm_ag_local(A_loc, peers_A, A_full, Bag, C_ag, 2, stream=s1)
        with torch.cuda.stream(s2):
            mk.gemm_ar_local(A2, B2, P2, C2, stream=s2)
        mk.stream_status(s1)
        mk.stream_status(s2)
        for i, (_, _, _, want, C) in enumerate(cases):
            check_exact(c_bits(C), want, f"stream call {i}, repetition {rep}")
        check_exact(mk_inputs.bits(A_full), f_want, f"gathered matrix, repetition {rep}")
        check_exact(c_bits(C_ag), c_want, f"AllGather C, repetition {rep}")
