"""The C ABI library loads, exports every function include/mk.h declares, and
rejects bad arguments before touching the GPU (runs without a GPU)."""
import ctypes
import os
import re

import pytest

import tile_gemm_all_amd as mk

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    text = open(os.path.join(ROOT, "include", "mk.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mk_[a-z_]+)\s*\(", text)))


def test_header_declares_the_binding_exports():
    assert declared_functions() == sorted(mk.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(mk.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert mk.library().mk_version() == 1


def test_status_strings():
    assert mk.status_string(0) == "MK_OK"
    assert mk.status_string(4) == "MK_ERR_TIMEOUT"
    assert mk.status_string(99) == "MK_ERR_UNKNOWN"


A16 = 0x10000  # fake, 16-byte aligned addresses: validation never dereferences them
B16 = 0x20000000
P16 = 0x40000000
C16 = 0x80000000


def call(A=A16, B=B16, peers=P16, n_peers=3, C=C16, M=64, N=64, K=64, pdt=0, cdt=0, nr=-1):
    return mk.library().mk_gemm_ar_local(A, B, peers, n_peers, C, M, N, K, pdt, cdt, None, nr,
                                         None)


def noalloc(A=A16, B=B16, peers=P16, n_peers=3, C=C16, M=64, N=64, K=64, pdt=0, cdt=0, nr=-1):
    return mk.library().mk_gemm_ar_local_noalloc(A, B, peers, n_peers, C, M, N, K, pdt, cdt, None,
                                                 nr, None)


def base(A=A16, B=B16, peers=P16, n_peers=3, C=C16, M=64, N=64, K=64, pdt=0, cdt=0):
    return mk.library().mk_gemm_then_reduce_baseline(A, B, peers, n_peers, C, M, N, K, pdt, cdt,
                                                     None)


def two(A=A16, B=B16, peers=P16, n_peers=3, C=C16, M=64, N=64, K=64, pdt=0, cdt=0, chunks=0):
    return mk.library().mk_gemm_ar_two_stream(A, B, peers, n_peers, C, M, N, K, pdt, cdt, None,
                                              chunks)


@pytest.mark.parametrize("kw,status", [
    (dict(A=None), mk.MK_ERR_INVALID_ARG),
    (dict(B=None), mk.MK_ERR_INVALID_ARG),
    (dict(C=None), mk.MK_ERR_INVALID_ARG),
    (dict(peers=None), mk.MK_ERR_INVALID_ARG),
    (dict(A=A16 + 2), mk.MK_ERR_INVALID_ARG),
    (dict(C=C16 + 8), mk.MK_ERR_INVALID_ARG),
    (dict(M=-1), mk.MK_ERR_INVALID_ARG),
    (dict(K=-8), mk.MK_ERR_INVALID_ARG),
    (dict(n_peers=-1), mk.MK_ERR_INVALID_ARG),
    (dict(n_peers=65), mk.MK_ERR_INVALID_ARG),
    (dict(pdt=2), mk.MK_ERR_INVALID_ARG),
    (dict(cdt=-1), mk.MK_ERR_INVALID_ARG),
    (dict(N=60), mk.MK_ERR_UNSUPPORTED),
    (dict(K=12), mk.MK_ERR_UNSUPPORTED),
    (dict(C=A16), mk.MK_ERR_INVALID_ARG),               # C aliases A
    (dict(C=P16 + 64 * 64 * 2), mk.MK_ERR_INVALID_ARG),  # C inside peer 1
    (dict(M=1 << 41), mk.MK_ERR_UNSUPPORTED),
    (dict(M=1, N=(1 << 22) + 8, C=C16 + (1 << 30)), mk.MK_ERR_UNSUPPORTED),  # N beyond 2^22
])
def test_validation_rejects(kw, status):
    assert call(**kw) == status, mk.last_error()
    assert noalloc(**kw) == status, mk.last_error()
    assert base(**kw) == status, mk.last_error()
    assert two(**kw) == status, mk.last_error()
    assert mk.last_error()


def test_chunk_count_outside_range_is_rejected():
    assert two(chunks=-1) == mk.MK_ERR_INVALID_ARG
    assert two(chunks=mk.MK_MAX_CHUNKS + 1) == mk.MK_ERR_INVALID_ARG


def test_reducer_count_below_adaptive_is_rejected():
    assert call(nr=-2) == mk.MK_ERR_INVALID_ARG
    assert noalloc(nr=-2) == mk.MK_ERR_INVALID_ARG


def test_peers_may_be_null_without_peers_and_inputs_without_size():
    # valid arguments reach the device query; without a GPU that is the first failure
    st = call(peers=None, n_peers=0)
    assert st in (mk.MK_OK, mk.MK_ERR_NO_DEVICE, mk.MK_ERR_HIP), mk.last_error()
    st = call(A=None, B=None, K=0)
    assert st in (mk.MK_OK, mk.MK_ERR_NO_DEVICE, mk.MK_ERR_HIP), mk.last_error()


def test_options_roundtrip():
    old = mk.get_option(mk.OPT_CTRL_PERIOD)
    mk.set_option(mk.OPT_CTRL_PERIOD, 4)
    assert mk.get_option(mk.OPT_CTRL_PERIOD) == 4
    mk.set_option(mk.OPT_CTRL_PERIOD, old)
    with pytest.raises(mk.MkError):
        mk.set_option(mk.OPT_SPIN_TIMEOUT_US, 0)
    for shape in range(6):  # automatic, 256, 128, 64 and the two wave-specialised tiles
        mk.set_option(mk.OPT_TILE_SHAPE, shape)
        assert mk.get_option(mk.OPT_TILE_SHAPE) == shape
    mk.set_option(mk.OPT_TILE_SHAPE, 0)
    for bad in (-1, 6, 7):
        with pytest.raises(mk.MkError):
            mk.set_option(mk.OPT_TILE_SHAPE, bad)
    with pytest.raises(mk.MkError):
        mk.set_option(99, 1)
    old = mk.get_option(mk.OPT_INPLACE)
    assert old == -1
    mk.set_option(mk.OPT_INPLACE, 0)
    assert mk.get_option(mk.OPT_INPLACE) == 0
    mk.set_option(mk.OPT_INPLACE, -2)  # dynamic hand-over
    assert mk.get_option(mk.OPT_INPLACE) == -2
    mk.set_option(mk.OPT_INPLACE, old)
    with pytest.raises(mk.MkError):
        mk.set_option(mk.OPT_INPLACE, -3)
    assert mk.get_option(mk.OPT_EARLY) == -1
    mk.set_option(mk.OPT_EARLY, 1)
    assert mk.get_option(mk.OPT_EARLY) == 1
    mk.set_option(mk.OPT_EARLY, -1)
    for bad in (-2, 2):
        with pytest.raises(mk.MkError):
            mk.set_option(mk.OPT_EARLY, bad)


def test_telemetry_struct_size():
    # 5 u64 + 10 i32, 2 u64 + 2 i32 of flag overhead, MK_TRACE_CAP entries of 24 bytes
    assert mk.TELEMETRY_BYTES == 5 * 8 + 10 * 4 + 2 * 8 + 2 * 4 + mk.MK_TRACE_CAP * 24
    assert mk.Telemetry.trace.offset == 104


S16 = 0xC0000000


def rs(A=A16, B=B16, peers=P16, n_peers=3, C=C16, send=S16, M=64, N=64, K=64, o0=0, o1=32,
       pdt=0, cdt=0):
    return mk.library().mk_gemm_rs_local(A, B, peers, n_peers, C, send, M, N, K, o0, o1, pdt,
                                         cdt, None, -1)


def rs_base(**kw):
    a = dict(A=A16, B=B16, peers=P16, n_peers=3, C=C16, send=S16, M=64, N=64, K=64, o0=0, o1=32,
             pdt=0, cdt=0)
    a.update(kw)
    return mk.library().mk_gemm_rs_baseline(a["A"], a["B"], a["peers"], a["n_peers"], a["C"],
                                            a["send"], a["M"], a["N"], a["K"], a["o0"], a["o1"],
                                            a["pdt"], a["cdt"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(o0=-1), mk.MK_ERR_INVALID_ARG),
    (dict(o0=40, o1=32), mk.MK_ERR_INVALID_ARG),
    (dict(o1=65), mk.MK_ERR_INVALID_ARG),
    (dict(send=None), mk.MK_ERR_INVALID_ARG),             # rows outside [o0, o1) need send
    (dict(send=S16 + 8), mk.MK_ERR_INVALID_ARG),
    (dict(send=C16 + 64), mk.MK_ERR_INVALID_ARG),          # send overlaps C
    (dict(send=P16 + 64), mk.MK_ERR_INVALID_ARG),          # send overlaps the peers
    (dict(C=A16 + 64 * 64), mk.MK_ERR_INVALID_ARG),        # C inside A's last rows
    (dict(N=60), mk.MK_ERR_UNSUPPORTED),
])
def test_reduce_scatter_validation(kw, status):
    assert rs(**kw) == status, mk.last_error()
    assert rs_base(**kw) == status, mk.last_error()


def test_reduce_scatter_send_may_be_null_when_every_row_is_owned():
    st = rs(send=None, o0=0, o1=64)
    assert st in (mk.MK_OK, mk.MK_ERR_NO_DEVICE, mk.MK_ERR_HIP), mk.last_error()


F16 = 0xC0000000  # fake gathered-matrix address


def ag(A_local=A16, peers_A=P16, n_peers=3, A_full=F16, B=B16, C=C16, Ms=128, N=64, K=64, rank=1,
       cdt=0, nc=-1):
    return mk.library().mk_gemm_ag_local(A_local, peers_A, n_peers, A_full, B, C, Ms, N, K, rank,
                                         cdt, None, nc)


def ag_base(A_local=A16, peers_A=P16, n_peers=3, A_full=F16, B=B16, C=C16, Ms=128, N=64, K=64,
            rank=1, cdt=0):
    return mk.library().mk_gemm_ag_baseline(A_local, peers_A, n_peers, A_full, B, C, Ms, N, K,
                                            rank, cdt, None)


@pytest.mark.parametrize("kw,status", [
    (dict(A_local=None), mk.MK_ERR_INVALID_ARG),
    (dict(peers_A=None), mk.MK_ERR_INVALID_ARG),
    (dict(A_full=None), mk.MK_ERR_INVALID_ARG),
    (dict(B=None), mk.MK_ERR_INVALID_ARG),
    (dict(C=None), mk.MK_ERR_INVALID_ARG),
    (dict(A_full=F16 + 4), mk.MK_ERR_INVALID_ARG),
    (dict(rank=4), mk.MK_ERR_INVALID_ARG),               # rank beyond P-1
    (dict(rank=-1), mk.MK_ERR_INVALID_ARG),
    (dict(n_peers=65), mk.MK_ERR_INVALID_ARG),
    (dict(Ms=-128), mk.MK_ERR_INVALID_ARG),
    (dict(cdt=2), mk.MK_ERR_INVALID_ARG),
    (dict(Ms=192), mk.MK_ERR_UNSUPPORTED),               # bands of 128 rows
    (dict(N=60), mk.MK_ERR_UNSUPPORTED),
    (dict(K=12), mk.MK_ERR_UNSUPPORTED),
    (dict(A_full=A16), mk.MK_ERR_INVALID_ARG),           # gathered matrix over the local shard
    (dict(A_full=P16 + 64), mk.MK_ERR_INVALID_ARG),      # ... over a peer shard
    (dict(C=F16 + 64), mk.MK_ERR_INVALID_ARG),           # C over the gathered matrix
    (dict(C=B16), mk.MK_ERR_INVALID_ARG),                # C over B
])
def test_allgather_validation_rejects(kw, status):
    assert ag(**kw) == status, mk.last_error()
    assert ag_base(**kw) == status, mk.last_error()


def test_allgather_static_count_below_minus_one_is_rejected():
    assert ag(nc=-2) == mk.MK_ERR_INVALID_ARG


@pytest.mark.parametrize("iters,scope,out,status", [
    (0, 0, A16, mk.MK_ERR_INVALID_ARG),
    ((1 << 24) + 1, 0, A16, mk.MK_ERR_INVALID_ARG),
    (10, 3, A16, mk.MK_ERR_INVALID_ARG),
    (10, 0, None, mk.MK_ERR_INVALID_ARG),
    (10, 0, A16 + 8, mk.MK_ERR_INVALID_ARG),
])
def test_flag_handoff_validation_rejects(iters, scope, out, status):
    assert mk.library().mk_flag_handoff(iters, scope, 0, None, out) == status, mk.last_error()


def test_flag_handoff_rejects_a_bad_xcd_choice():
    assert mk.library().mk_flag_handoff(10, 0, 2, None, A16) == mk.MK_ERR_INVALID_ARG


def test_ksplit_option_accepts_only_auto_off_and_two():
    old = mk.get_option(mk.OPT_KSPLIT)
    try:
        for v in (3, 4, 0, -2):
            with pytest.raises(mk.MkError):
                mk.set_option(mk.OPT_KSPLIT, v)
        for v in (-1, 1, 2):
            mk.set_option(mk.OPT_KSPLIT, v)
            assert mk.get_option(mk.OPT_KSPLIT) == v
    finally:
        mk.set_option(mk.OPT_KSPLIT, old)


def test_stream_cu_split_option_takes_multiples_of_eight():
    """The two-stream CU split is 0 (no masks) or a multiple of 8 compute units;
    whether it fits the device (below its unit count, 8 per mask word) is checked
    at the call."""
    old = mk.get_option(mk.OPT_STREAM_CU_SPLIT)
    assert old == 0
    try:
        for v in (-8, 7, 60, 4104):
            with pytest.raises(mk.MkError):
                mk.set_option(mk.OPT_STREAM_CU_SPLIT, v)
        for v in (0, 64, 128, 192, 72):
            mk.set_option(mk.OPT_STREAM_CU_SPLIT, v)
            assert mk.get_option(mk.OPT_STREAM_CU_SPLIT) == v
    finally:
        mk.set_option(mk.OPT_STREAM_CU_SPLIT, old)


def test_static_tiles_option_range():
    """The in-place kernel's switch: 2 (default: eight waves where they fit), 1
    (four waves) or 0 (the claim-queue kernel); anything else is rejected without
    changing the setting."""
    old = mk.get_option(mk.OPT_STATIC_TILES)
    assert old == 2
    try:
        for v in (-1, 3, 7):
            with pytest.raises(mk.MkError):
                mk.set_option(mk.OPT_STATIC_TILES, v)
            assert mk.get_option(mk.OPT_STATIC_TILES) == old
        for v in (0, 1, 2):
            mk.set_option(mk.OPT_STATIC_TILES, v)
            assert mk.get_option(mk.OPT_STATIC_TILES) == v
    finally:
        mk.set_option(mk.OPT_STATIC_TILES, old)


@pytest.mark.parametrize("iters,grid,out,status", [
    (0, 1, A16, mk.MK_ERR_INVALID_ARG),
    ((1 << 24) + 1, 1, A16, mk.MK_ERR_INVALID_ARG),
    (1, 0, A16, mk.MK_ERR_INVALID_ARG),
    (1, (1 << 16) + 1, A16, mk.MK_ERR_INVALID_ARG),
    (1, 1, None, mk.MK_ERR_INVALID_ARG),
    (1, 1, A16 + 2, mk.MK_ERR_INVALID_ARG),
])
def test_mfma_peak_validates_before_touching_the_device(iters, grid, out, status):
    assert mk.library().mk_mfma_peak(iters, grid, out, None) == status, mk.last_error()


@pytest.mark.parametrize("cus,grid,scope,want", [
    (256, 256, 0, (8, 0)),    # MI355X: eight XCDs of 32 compute units, one queue each
    (256, 512, 0, (8, 0)),
    (256, 256, 1, (8, 1)),
    (256, 100, 0, (1, 1)),    # grid not a multiple of the XCD count: one queue, agent scope
    (240, 240, 0, (1, 1)),    # compute units not whole XCDs of 32: layout unknown
    (32, 64, 0, (1, 0)),      # one XCD
    (128, 64, 0, (4, 0)),
    (1024, 1024, 0, (1, 1)),  # more than 16 queues: one queue, agent scope
])
def test_queue_plan(cus, grid, scope, want):
    """Tiles are queued per XCD, under the XCD-local flag protocol, only where each
    queue is served by one XCD; otherwise one queue with agent-scope flags."""
    assert mk.queue_plan(cus, grid, scope) == want


def test_queue_plan_rejects_bad_arguments():
    n = ctypes.c_int(0)
    lib = mk.library()
    assert lib.mk_queue_plan(0, 256, 0, ctypes.byref(n)) == -mk.MK_ERR_INVALID_ARG
    assert lib.mk_queue_plan(256, 0, 0, ctypes.byref(n)) == -mk.MK_ERR_INVALID_ARG
    assert lib.mk_queue_plan(256, 256, 2, ctypes.byref(n)) == -mk.MK_ERR_INVALID_ARG
    assert lib.mk_queue_plan(256, 256, 0, None) == -mk.MK_ERR_INVALID_ARG


def test_fused_schedule_validates_before_touching_the_device():
    lib = mk.library()
    for args in ((64, 64, 64, 1, 7, 0), (64, 64, 64, 1, 0, 7), (-1, 64, 64, 1, 0, 0),
                 (64, 64, 64, -1, 0, 0)):
        assert lib.mk_fused_schedule(*args) == -mk.MK_ERR_INVALID_ARG
    # valid arguments need the device (its compute-unit count): a schedule or an error
    v = lib.mk_fused_schedule(4096, 8192, 1792, 15, 0, 0)
    assert v in (1, 2, 3, 4, 5) or -v in (mk.MK_ERR_NO_DEVICE, mk.MK_ERR_HIP)
