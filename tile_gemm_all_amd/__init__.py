"""Python binding of libmk.so: one GPU's share of a tile-granular fused GEMM+AllReduce
on AMD Instinct MI355X (gfx950).

The functions here only marshal torch tensors (device pointers, sizes, dtypes and
the current HIP stream) into the C ABI declared in include/mk.h. Every step of
the computation runs in the library's HIP kernels. There is no fallback: if
libmk.so is missing or fails to load, importing this package raises.

    import tile_gemm_all_amd as mk
    mk.gemm_ar_local(A, B, peers, C)                  # adaptive reducer count
    mk.gemm_ar_local(A, B, peers, C, n_reduce_wg=16)  # static reducer count
    mk.gemm_then_reduce_baseline(A, B, peers, C)      # two-kernel baseline
    mk.stream_status()                                # sync + device error word

Shapes: A [M,K] bf16, B [K,N] bf16, peers [P-1,M,N] bf16|fp32, C [M,N] bf16|fp32,
all contiguous on the current CUDA (HIP) device.
"""
import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmk.so")

MK_OK, MK_ERR_INVALID_ARG, MK_ERR_UNSUPPORTED, MK_ERR_HIP, MK_ERR_TIMEOUT = 0, 1, 2, 3, 4
MK_ERR_NO_DEVICE, MK_ERR_WORKSPACE = 5, 6
MK_DT_BF16, MK_DT_F32 = 0, 1
MK_ADAPTIVE = -1
MK_MAX_PEERS = 64
MK_MAX_CHUNKS = 64
MK_TRACE_CAP = 512
OPT_SPIN_TIMEOUT_US, OPT_WITHHOLD_TILE, OPT_CTRL_PERIOD, OPT_TILE_SHAPE = 0, 1, 2, 3
OPT_FLAG_SCOPE, OPT_REDUCER_CAP, OPT_INPLACE, OPT_EARLY, OPT_KSPLIT = 4, 5, 6, 7, 8
OPT_STREAM_CU_SPLIT = 9  # two-stream schedule: compute units of the CU-masked reduce stream
OPT_STATIC_TILES = 10  # all-in-place 256x256 tiles: 2 in-place kernel, 8 waves where they fit; 1 four; 0 claim queues

EXPORTS = ["mk_gemm_ar_local", "mk_gemm_ar_local_noalloc", "mk_gemm_then_reduce_baseline",
           "mk_gemm_ar_two_stream",
           "mk_gemm_rs_local", "mk_gemm_rs_baseline", "mk_gemm_ag_local", "mk_gemm_ag_baseline",
           "mk_ag_grid", "mk_flag_handoff", "mk_mfma_peak",
           "mk_stream_status",
           "mk_workspace_reset", "mk_queue_plan", "mk_num_workgroups", "mk_fused_grid",
           "mk_fused_schedule",
           "mk_set_option",
           "mk_get_option",
           "mk_controller_eval", "mk_status_string", "mk_last_error", "mk_version"]


class MkError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{msg} (status {status})")
        self.status = status


if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run tile_gemm_all_amd/build.py "
                      "(or __graft_entry__.build()) first")
_lib = ctypes.CDLL(LIB_PATH)

_vp, _i64, _int = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
_lib.mk_gemm_ar_local.argtypes = [_vp, _vp, _vp, _int, _vp, _i64, _i64, _i64, _int, _int, _vp,
                                  _int, _vp]
_lib.mk_gemm_ar_local.restype = _int
_lib.mk_gemm_ar_local_noalloc.argtypes = [_vp, _vp, _vp, _int, _vp, _i64, _i64, _i64, _int, _int,
                                          _vp, _int, _vp]
_lib.mk_gemm_ar_local_noalloc.restype = _int
_lib.mk_gemm_then_reduce_baseline.argtypes = [_vp, _vp, _vp, _int, _vp, _i64, _i64, _i64, _int,
                                              _int, _vp]
_lib.mk_gemm_then_reduce_baseline.restype = _int
_lib.mk_gemm_ar_two_stream.argtypes = [_vp, _vp, _vp, _int, _vp, _i64, _i64, _i64, _int, _int,
                                       _vp, _int]
_lib.mk_gemm_ar_two_stream.restype = _int
_lib.mk_gemm_rs_local.argtypes = [_vp, _vp, _vp, _int, _vp, _vp, _i64, _i64, _i64, _i64, _i64,
                                  _int, _int, _vp, _int]
_lib.mk_gemm_rs_baseline.argtypes = [_vp, _vp, _vp, _int, _vp, _vp, _i64, _i64, _i64, _i64,
                                     _i64, _int, _int, _vp]
_lib.mk_gemm_rs_local.restype = _int
_lib.mk_gemm_rs_baseline.restype = _int
_lib.mk_gemm_ag_local.argtypes = [_vp, _vp, _int, _vp, _vp, _vp, _i64, _i64, _i64, _int, _int,
                                  _vp, _int]
_lib.mk_gemm_ag_local.restype = _int
_lib.mk_gemm_ag_baseline.argtypes = [_vp, _vp, _int, _vp, _vp, _vp, _i64, _i64, _i64, _int, _int,
                                     _vp]
_lib.mk_gemm_ag_baseline.restype = _int
_lib.mk_ag_grid.argtypes = [_i64, _int, _i64, _i64, _int]
_lib.mk_ag_grid.restype = _int
_lib.mk_flag_handoff.argtypes = [_int, _int, _int, _vp, _vp]
_lib.mk_flag_handoff.restype = _int
_lib.mk_mfma_peak.argtypes = [_int, _int, _vp, _vp]
_lib.mk_mfma_peak.restype = _int
_lib.mk_stream_status.argtypes = [_vp]
_lib.mk_stream_status.restype = _int
_lib.mk_workspace_reset.argtypes = [_int]
_lib.mk_workspace_reset.restype = _int
_lib.mk_queue_plan.argtypes = [_int, _int, _int, ctypes.POINTER(_int)]
_lib.mk_queue_plan.restype = _int
_lib.mk_num_workgroups.argtypes = [_int]
_lib.mk_num_workgroups.restype = _int
_lib.mk_fused_grid.argtypes = [_i64, _i64, _i64, _int, _int, _int]
_lib.mk_fused_grid.restype = _int
_lib.mk_fused_schedule.argtypes = [_i64, _i64, _i64, _int, _int, _int]
_lib.mk_fused_schedule.restype = _int
_lib.mk_set_option.argtypes = [_int, _i64]
_lib.mk_set_option.restype = _int
_lib.mk_get_option.argtypes = [_int]
_lib.mk_get_option.restype = _i64
_lib.mk_controller_eval.argtypes = [_int, _int, _int, _int, _int, ctypes.c_uint64,
                                    ctypes.c_uint64, ctypes.c_float, _int, _int]
_lib.mk_controller_eval.restype = _int
_lib.mk_status_string.argtypes = [_int]
_lib.mk_status_string.restype = ctypes.c_char_p
_lib.mk_last_error.restype = ctypes.c_char_p
_lib.mk_version.restype = _int


class TraceEntry(ctypes.Structure):
    _fields_ = [("t", ctypes.c_uint64), ("computed", ctypes.c_int32),
                ("reduced", ctypes.c_int32), ("target", ctypes.c_int32),
                ("spare", ctypes.c_int32)]


class Telemetry(ctypes.Structure):
    """Host mirror of mk_telemetry_t."""
    _fields_ = [("t_start", ctypes.c_uint64), ("t_end", ctypes.c_uint64),
                ("busy_compute", ctypes.c_uint64), ("busy_reduce", ctypes.c_uint64),
                ("wait_reduce", ctypes.c_uint64), ("tiles", ctypes.c_int32),
                ("grid", ctypes.c_int32), ("initial_target", ctypes.c_int32),
                ("final_target", ctypes.c_int32), ("n_updates", ctypes.c_int32),
                ("n_trace", ctypes.c_int32), ("role_switches", ctypes.c_int32),
                ("reduced_by_compute", ctypes.c_int32), ("computed_by_reducers", ctypes.c_int32),
                ("n_xcd", ctypes.c_int32), ("publish_ticks", ctypes.c_uint64),
                ("acquire_ticks", ctypes.c_uint64), ("published", ctypes.c_int32),
                ("acquired", ctypes.c_int32), ("trace", TraceEntry * MK_TRACE_CAP)]


TELEMETRY_BYTES = ctypes.sizeof(Telemetry)


def library():
    """The loaded ctypes library (for tests that call the C ABI directly)."""
    return _lib


def last_error():
    return _lib.mk_last_error().decode()


def status_string(st):
    return _lib.mk_status_string(st).decode()


def _check(st):
    if st != MK_OK:
        raise MkError(st, f"{status_string(st)}: {last_error()}")


_DT = {torch.bfloat16: MK_DT_BF16, torch.float32: MK_DT_F32}


def _stream_ptr(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _args(A, B, peers, C):
    if A.dtype != torch.bfloat16 or B.dtype != torch.bfloat16:
        raise TypeError("A and B must be bfloat16")
    if C.dtype not in _DT:
        raise TypeError("C must be bfloat16 or float32")
    for name, t in (("A", A), ("B", B), ("C", C)):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous GPU tensor")
    M, K = A.shape
    K2, N = B.shape
    if K2 != K or tuple(C.shape) != (M, N):
        raise ValueError(f"shape mismatch A{tuple(A.shape)} B{tuple(B.shape)} C{tuple(C.shape)}")
    if peers is None or peers.numel() == 0:
        n_peers, pdt, pptr = 0, MK_DT_BF16, None
    else:
        if peers.dtype not in _DT or not peers.is_cuda or not peers.is_contiguous():
            raise ValueError("peers must be a contiguous bf16/fp32 GPU tensor")
        if peers.dim() != 3 or tuple(peers.shape[1:]) != (M, N):
            raise ValueError(f"peers must be [P-1, {M}, {N}], got {tuple(peers.shape)}")
        n_peers, pdt, pptr = peers.shape[0], _DT[peers.dtype], peers.data_ptr()
    return (A.data_ptr(), B.data_ptr(), pptr, n_peers, C.data_ptr(), M, N, K, pdt, _DT[C.dtype])


def gemm_ar_local(A, B, peers, C, n_reduce_wg=None, telemetry=None, stream=None):
    """C = A @ B + peers.sum(0) with the fused persistent kernel.

    n_reduce_wg: None (adaptive controller) or a static reducer workgroup count in
    [0, G-1]. telemetry: None or a uint8 GPU tensor of TELEMETRY_BYTES bytes."""
    a = _args(A, B, peers, C)
    nr = MK_ADAPTIVE if n_reduce_wg is None else int(n_reduce_wg)
    tel = None
    if telemetry is not None:
        if telemetry.numel() * telemetry.element_size() < TELEMETRY_BYTES or not telemetry.is_cuda:
            raise ValueError("telemetry buffer too small")
        tel = telemetry.data_ptr()
    _check(_lib.mk_gemm_ar_local(*a[:10], _stream_ptr(stream), nr, tel))
    return C


def gemm_ar_local_noalloc(A, B, peers, C, n_reduce_wg=None, telemetry=None, stream=None):
    """gemm_ar_local with the library's fixed per-GPU workspace: no device memory is
    allocated. Calls that overlap on one GPU race."""
    a = _args(A, B, peers, C)
    nr = MK_ADAPTIVE if n_reduce_wg is None else int(n_reduce_wg)
    tel = None
    if telemetry is not None:
        if telemetry.numel() * telemetry.element_size() < TELEMETRY_BYTES or not telemetry.is_cuda:
            raise ValueError("telemetry buffer too small")
        tel = telemetry.data_ptr()
    _check(_lib.mk_gemm_ar_local_noalloc(*a[:10], _stream_ptr(stream), nr, tel))
    return C


def gemm_then_reduce_baseline(A, B, peers, C, stream=None):
    """Same result as gemm_ar_local, by a GEMM kernel followed by a reduce kernel."""
    a = _args(A, B, peers, C)
    _check(_lib.mk_gemm_then_reduce_baseline(*a[:10], _stream_ptr(stream)))
    return C


def gemm_ar_two_stream(A, B, peers, C, n_chunks=0, stream=None):
    """Same result as gemm_ar_local, by per-chunk GEMM kernels on the stream and
    per-chunk reduce kernels on a second stream that overlap the next chunks' GEMMs."""
    a = _args(A, B, peers, C)
    _check(_lib.mk_gemm_ar_two_stream(*a[:10], _stream_ptr(stream), int(n_chunks)))
    return C


def _rs_args(A, B, peers, C, send, own_m0, own_m1):
    M, K = A.shape
    N = B.shape[1]
    own0, own1 = int(own_m0), int(own_m1)
    if not 0 <= own0 <= own1 <= M:
        raise ValueError(f"owned rows [{own0}, {own1}) outside [0, {M}]")
    own = own1 - own0
    # A, B, peers and C as for an AllReduce share of the owned rows
    a = _args(A[own0:own1] if own > 0 else A[:0], B, peers, C)
    if not A.is_contiguous():
        raise ValueError("A must be contiguous")
    sptr = None
    if own < M:
        if send is None or not send.is_cuda or not send.is_contiguous():
            raise ValueError("send must be a contiguous GPU tensor")
        if tuple(send.shape) != (M, N) or _DT.get(send.dtype) != a[8] and a[3] > 0:
            raise ValueError(f"send must be [{M}, {N}] of the peer type")
        if a[3] == 0 and send.dtype not in _DT:
            raise ValueError("send must be bfloat16 or float32")
        sptr = send.data_ptr()
    pdt = a[8] if a[3] > 0 else (_DT[send.dtype] if sptr is not None else MK_DT_BF16)
    return (A.data_ptr(), B.data_ptr(), a[2], a[3], a[4], sptr, M, N, K, own0, own1, pdt, a[9])


def gemm_rs_local(A, B, peers, C, send, own_m0, own_m1, n_reduce_wg=None, stream=None):
    """One GPU's share of GEMM+ReduceScatter: C = peers.sum(0) + (A @ B)[own_m0:own_m1]
    for the owned rows; send[i] = (A @ B)[i] in the peer type for every other row
    (with no peers, send's dtype is the peer type). Fused persistent kernel;
    n_reduce_wg: None (adaptive) or a static reducer count."""
    nr = MK_ADAPTIVE if n_reduce_wg is None else int(n_reduce_wg)
    _check(_lib.mk_gemm_rs_local(*_rs_args(A, B, peers, C, send, own_m0, own_m1),
                                 _stream_ptr(stream), nr))
    return C, send


def gemm_rs_baseline(A, B, peers, C, send, own_m0, own_m1, stream=None):
    """Same result as gemm_rs_local, by a GEMM kernel followed by reduce kernels."""
    _check(_lib.mk_gemm_rs_baseline(*_rs_args(A, B, peers, C, send, own_m0, own_m1),
                                    _stream_ptr(stream)))
    return C, send


def _ag_args(A_local, peers_A, A_full, B, C, rank):
    for name, t in (("A_local", A_local), ("A_full", A_full), ("B", B)):
        if t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous bfloat16 GPU tensor")
    if C.dtype not in _DT or not C.is_cuda or not C.is_contiguous():
        raise ValueError("C must be a contiguous bfloat16/float32 GPU tensor")
    Ms, K = A_local.shape
    K2, N = B.shape
    if peers_A is None:
        n_peers, pptr = 0, None
    else:
        if peers_A.dtype != torch.bfloat16 or not peers_A.is_cuda or not peers_A.is_contiguous():
            raise ValueError("peers_A must be a contiguous bfloat16 GPU tensor")
        if peers_A.dim() != 3 or tuple(peers_A.shape[1:]) != (Ms, K):
            raise ValueError(f"peers_A must be [P-1, {Ms}, {K}], got {tuple(peers_A.shape)}")
        # the peer count comes from the shape, also when K = 0 leaves no elements
        n_peers = peers_A.shape[0]
        pptr = peers_A.data_ptr() if peers_A.numel() > 0 else None
    M = (n_peers + 1) * Ms
    if K2 != K or tuple(A_full.shape) != (M, K) or tuple(C.shape) != (M, N):
        raise ValueError(f"shape mismatch A_local{tuple(A_local.shape)} A_full"
                         f"{tuple(A_full.shape)} B{tuple(B.shape)} C{tuple(C.shape)}")
    return (A_local.data_ptr(), pptr, n_peers, A_full.data_ptr(), B.data_ptr(), C.data_ptr(), Ms,
            N, K, int(rank), _DT[C.dtype])


def gemm_ag_local(A_local, peers_A, A_full, B, C, rank, n_comm_wg=None, stream=None):
    """One GPU's share of AllGather+GEMM: A_full = the shards in rank order (this
    GPU's A_local at `rank`, peers_A the others), C = A_full @ B. Persistent kernel
    whose tiles wait for their band of A_full to land; n_comm_wg: None (default)
    or the count of workgroups that prefer landing bands."""
    nc = MK_ADAPTIVE if n_comm_wg is None else int(n_comm_wg)
    _check(_lib.mk_gemm_ag_local(*_ag_args(A_local, peers_A, A_full, B, C, rank),
                                 _stream_ptr(stream), nc))
    return A_full, C


def gemm_ag_baseline(A_local, peers_A, A_full, B, C, rank, stream=None):
    """Same result as gemm_ag_local, by a gather kernel followed by a GEMM kernel."""
    _check(_lib.mk_gemm_ag_baseline(*_ag_args(A_local, peers_A, A_full, B, C, rank),
                                    _stream_ptr(stream)))
    return A_full, C


def ag_grid(A_local, peers_A, A_full, B, C):
    """G of gemm_ag_local for these tensors (n_comm_wg must be < G)."""
    a = _ag_args(A_local, peers_A, A_full, B, C, 0)
    g = _lib.mk_ag_grid(a[6], a[2], a[7], a[8], a[10])
    if g < 0:
        _check(-g)
    return g


def flag_handoff(iters=1000, flag_scope=0, cross_xcd=False, stream=None):
    """Flag hand-off microbenchmark and message-passing litmus: returns (ns per
    hand-off, stale data reads, XCD of each side). Synchronizes the stream."""
    out = torch.zeros(6, dtype=torch.int64, device="cuda")
    _check(_lib.mk_flag_handoff(int(iters), int(flag_scope), int(bool(cross_xcd)),
                                _stream_ptr(stream), out.data_ptr()))
    vals = out.cpu().tolist()
    if vals[1]:
        raise MkError(MK_ERR_TIMEOUT, "flag hand-off timed out")
    return vals[0] * 10.0 / (2 * iters), vals[4], (vals[2], vals[3])


def mfma_peak(iters, n_workgroups, out, stream=None):
    """Launches the matrix-core ceiling kernel (n_workgroups * 4 * 8 * iters bf16
    MFMAs of 32768 flops); out: float32 GPU tensor of n_workgroups * 256 elements.
    Does not synchronize; time it with events on the stream."""
    if out.dtype != torch.float32 or not out.is_cuda or out.numel() < n_workgroups * 256:
        raise ValueError("out must be a float32 GPU tensor of n_workgroups * 256 elements")
    _check(_lib.mk_mfma_peak(int(iters), int(n_workgroups), out.data_ptr(), _stream_ptr(stream)))


def stream_status(stream=None):
    """Synchronizes the stream and raises MkError if a kernel reported an error."""
    _check(_lib.mk_stream_status(_stream_ptr(stream)))


def workspace_reset(device=None):
    dev = torch.cuda.current_device() if device is None else int(device)
    _check(_lib.mk_workspace_reset(dev))


def queue_plan(cus, grid, flag_scope=0):
    """(tile queues, flag scope) of a persistent launch of `grid` workgroups on a device
    of `cus` compute units: one queue per 32-unit XCD with the requested scope, or one
    queue with agent-scope flags where the device's layout is not known."""
    n = _int(0)
    s = _lib.mk_queue_plan(int(cus), int(grid), int(flag_scope), ctypes.byref(n))
    if s < 0:
        _check(-s)
    return n.value, s


def num_workgroups(device=None):
    dev = torch.cuda.current_device() if device is None else int(device)
    g = _lib.mk_num_workgroups(dev)
    if g < 0:
        _check(-g)
    return g


def fused_grid(A, B, peers, C):
    """G of the fused kernel for these tensors (n_reduce_wg must be < G)."""
    a = _args(A, B, peers, C)
    g = _lib.mk_fused_grid(a[5], a[6], a[7], a[3], a[8], a[9])
    if g < 0:
        _check(-g)
    return g


SCHEDULES = {1: "256x256 tiles, every tile in place", 2: "128x128 tiles, every tile in place",
             3: "64x64 tiles, one workgroup per tile, in place",
             4: "wave-specialised, 64x256 tiles", 5: "wave-specialised, 128x128 tiles"}


def fused_schedule(A, B, peers, C):
    """Tile shape (MK_OPT_TILE_SHAPE value, 1-5) of the schedule gemm_ar_local takes
    for these tensors with the adaptive default and no telemetry."""
    a = _args(A, B, peers, C)
    v = _lib.mk_fused_schedule(a[5], a[6], a[7], a[3], a[8], a[9])
    if v < 0:
        _check(-v)
    return v


def set_option(option, value):
    _check(_lib.mk_set_option(int(option), int(value)))


def get_option(option):
    return int(_lib.mk_get_option(int(option)))


def controller_eval(G, T, computed, reduced, busy_c, busy_r, seed_x, current, cap=-1, T_r=None):
    """The controller rule; T_r (tiles handed to reducers) defaults to T; cap < 0 means
    up to G-1 reducers while compute remains, 0 none."""
    return int(_lib.mk_controller_eval(G, T, T if T_r is None else T_r, computed, reduced, busy_c,
                                       busy_r, seed_x, current, cap))


def read_telemetry(buf):
    """Copies a telemetry GPU buffer to the host and returns a Telemetry structure."""
    host = buf.detach().cpu().contiguous().numpy().tobytes()[:TELEMETRY_BYTES]
    return Telemetry.from_buffer_copy(host)


def new_telemetry(device=None):
    return torch.zeros(TELEMETRY_BYTES, dtype=torch.uint8,
                       device=device if device is not None else "cuda")
