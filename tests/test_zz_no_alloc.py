"""GPU test of the allocation-free entry point (mk_gemm_ar_local_noalloc): through the
C ABI, its output equals mk_gemm_ar_local's on the same inputs (bitwise on integer
inputs, which the oracle also fixes exactly; within the tolerance rule on Gaussian
inputs), on two calls in a row with the second smaller, and it refuses what does not
fit its fixed workspace."""
import ctypes

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


def poisoned(M, N, cdt):
    C = torch.empty((M, N), dtype=TORCH_DT[cdt], device=DEV)
    if cdt == "bf16":
        C.view(torch.int16).fill_(0x7FC1)
    else:
        C.view(torch.int32).fill_(0x7FC00001)
    return C


def abi_call(fn, A, B, peers, C, n_reduce_wg=-1):
    """Calls fn (a C ABI entry point) with raw pointers on torch's current stream."""
    n_peers = 0 if peers is None else peers.shape[0]
    pdt = mk.MK_DT_F32 if peers is not None and peers.dtype == torch.float32 else mk.MK_DT_BF16
    cdt = mk.MK_DT_F32 if C.dtype == torch.float32 else mk.MK_DT_BF16
    st = fn(ctypes.c_void_p(A.data_ptr()), ctypes.c_void_p(B.data_ptr()),
            ctypes.c_void_p(peers.data_ptr() if n_peers else 0), n_peers,
            ctypes.c_void_p(C.data_ptr()), A.shape[0], B.shape[1], A.shape[1], pdt, cdt,
            ctypes.c_void_p(torch.cuda.current_stream().cuda_stream), n_reduce_wg, None)
    return st


# pairs of calls: the second smaller than the first
PAIRS = [
    # a shape whose handed-over partial (64 MiB) would exceed the fixed region (the
    # adaptive call takes the wave-specialised kernel, a static count every
    # 256x256 tile in place), then a few-tile shape (64x64 tiles)
    ((4096, 4096, 256, 3, "bf16", "bf16"), (128, 2048, 448, 15, "bf16", "bf16")),
    # handed-over and in-place tiles with the partial in the fixed region, then fp32
    ((1024, 2048, 576, 7, "bf16", "bf16"), (256, 512, 512, 3, "f32", "f32")),
    # ragged edges, then a tiny one
    ((520, 776, 1032, 1, "bf16", "f32"), (130, 136, 72, 15, "bf16", "bf16")),
]


@pytest.mark.parametrize("pair", PAIRS, ids=lambda p: "-".join("x".join(map(str, s[:4])) for s in p))
@pytest.mark.parametrize("variant", ["integer", "gaussian"])
def test_noalloc_matches_gemm_ar_local(pair, variant):
    lib = mk.library()
    for i, (M, N, K, npeer, pdt, cdt) in enumerate(pair):
        announce(f"noalloc {variant} call {i}: {M}x{N}x{K} peers {npeer} {pdt}/{cdt}")
        A, B, peers = mk_inputs.make_inputs(M, N, K, npeer, pdt, variant, 300 + i, device="cpu")
        C64, want = oracle.gemm_ar(mk_inputs.bits(A), mk_inputs.bits(B), mk_inputs.bits(peers), cdt)
        A, B, peers = A.to(DEV), B.to(DEV), peers.to(DEV)
        ref = poisoned(M, N, cdt)
        assert abi_call(lib.mk_gemm_ar_local, A, B, peers, ref) == mk.MK_OK, mk.last_error()
        mk.stream_status()
        for nr in (-1, 0):
            got = poisoned(M, N, cdt)
            assert abi_call(lib.mk_gemm_ar_local_noalloc, A, B, peers, got, nr) == mk.MK_OK, \
                mk.last_error()
            mk.stream_status()
            check_exact(mk_inputs.bits(got), mk_inputs.bits(ref), f"noalloc vs gemm_ar_local {nr}")
            if variant == "integer":
                check_exact(mk_inputs.bits(got), want, f"noalloc vs oracle {nr}")
            else:
                check_tolerance(mk_inputs.bits(got), C64, cdt, f"noalloc vs oracle {nr}")


def test_noalloc_refuses_what_does_not_fit():
    """Five peers cannot be reduced in place, and this call's handed-over partial
    (64 MiB) exceeds the fixed region: refused before anything is launched."""
    announce("noalloc refusal")
    M, N, K, npeer = 4096, 4096, 64, 5
    A = torch.zeros((M, K), dtype=torch.bfloat16, device=DEV)
    B = torch.zeros((K, N), dtype=torch.bfloat16, device=DEV)
    peers = torch.zeros((npeer, M, N), dtype=torch.bfloat16, device=DEV)
    C = poisoned(M, N, "bf16")
    st = abi_call(mk.library().mk_gemm_ar_local_noalloc, A, B, peers, C)
    assert st == mk.MK_ERR_UNSUPPORTED, (st, mk.last_error())
    mk.stream_status()
    assert int(C.view(torch.int16)[0, 0]) == 0x7FC1  # untouched
