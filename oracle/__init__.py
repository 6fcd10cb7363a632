"""CPU oracle for one GPU's share of GEMM+AllReduce (and of GEMM+ReduceScatter and
AllGather+GEMM) -- TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import
this package. The product path (tile_gemm_all_amd, libmk.so) never does.

It computes, in double precision, the operation of the "GEMM + AllReduce (TP)"
row of Table 3 on the thelatestinai.com page of "mKernel: Fast Multi-GPU,
Multi-Node Fused Kernels": the local partial product A*B of a K-split matrix
product plus the sum of the peers' partial products,

    C[i,j] = sum_k A[i,k] B[k,j] + sum_p peers[p,i,j],

then rounds once to the output type (round to nearest even). The arithmetic is
in mk_oracle.c: exact peer sum first, ascending-k fp64 dot products, one
addition, one rounding. Every function here marshals numpy arrays only.
"""
import ctypes
import os

import numpy as np

from . import build as _build

BF16, F32 = 0, 1


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


class Oracle:
    """ctypes view of one build of mk_oracle.c."""

    def __init__(self, lib_path):
        lib = ctypes.CDLL(lib_path)
        i64, vp = ctypes.c_int64, ctypes.c_void_p
        lib.mko_gemm_ar.argtypes = [vp, vp, vp, ctypes.c_int, ctypes.c_int, i64, i64, i64, vp,
                                    i64, vp, vp, ctypes.c_int, ctypes.c_int]
        lib.mko_gemm_ar.restype = ctypes.c_int
        lib.mko_bf16_to_f64_array.argtypes = [vp, vp, i64]
        lib.mko_f64_to_bf16_array.argtypes = [vp, vp, i64]
        lib.mko_exact_sum.argtypes = [vp, ctypes.c_int]
        lib.mko_exact_sum.restype = ctypes.c_double
        lib.mko_max_threads.restype = ctypes.c_int
        self.lib = lib
        self.path = lib_path

    def gemm_ar(self, A_bits, B_bits, peers, c_dtype="bf16", rows=None, threads=0):
        """Reference C for the given rows.

        A_bits: uint16 [M,K] (bfloat16 bit patterns); B_bits: uint16 [K,N];
        peers: None, uint16 [P-1,M,N] (bfloat16 bits) or float32 [P-1,M,N];
        c_dtype: "bf16" or "f32"; rows: None (all) or int sequence.
        Returns (C64 float64 [R,N], C_out uint16 or float32 [R,N]).
        """
        A_bits = np.ascontiguousarray(A_bits, dtype=np.uint16)
        B_bits = np.ascontiguousarray(B_bits, dtype=np.uint16)
        M, K = A_bits.shape
        K2, N = B_bits.shape
        if K2 != K:
            raise ValueError("A and B disagree on K")
        if peers is None or len(peers) == 0:
            n_peers, peer_dt, pp = 0, BF16, None
        else:
            if peers.dtype == np.uint16:
                peer_dt = BF16
            elif peers.dtype == np.float32:
                peer_dt = F32
            else:
                raise ValueError("peers must be uint16 (bf16 bits) or float32")
            pp = np.ascontiguousarray(peers)
            n_peers = pp.shape[0]
            if pp.shape[1:] != (M, N):
                raise ValueError("peers must be [P-1, M, N]")
        if rows is None:
            r = None
            n_rows = M
        else:
            r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
            n_rows = r.shape[0]
        C64 = np.empty((n_rows, N), dtype=np.float64)
        cd = BF16 if c_dtype == "bf16" else F32
        Cout = np.empty((n_rows, N), dtype=np.uint16 if cd == BF16 else np.float32)
        st = self.lib.mko_gemm_ar(_ptr(A_bits), _ptr(B_bits), _ptr(pp), n_peers, peer_dt, M, N,
                                  K, _ptr(r), n_rows, _ptr(C64), _ptr(Cout), cd, int(threads))
        if st != 0:
            raise ValueError("oracle rejected its arguments")
        return C64, Cout

    def gemm_rs(self, A_bits, B_bits, peers_own, own_m0, own_m1, c_dtype="bf16",
                peer_dtype="bf16", rows=None, threads=0):
        """Reference for one GPU's share of GEMM+ReduceScatter ("GEMM + ReduceScatter
        (TP)" row of Table 3, thelatestinai.com page: compute -> communication, each
        output tile added into its owner's buffer). This GPU owns rows
        [own_m0, own_m1). An owned row is the AllReduce share of that row with the
        owner's peer partials (peers_own: [P-1, own, N]); every other row is this
        GPU's partial A*B rounded to the peer type, which its owner receives as a
        peer partial.

        rows: None (all M rows) or global row indices. Returns
        ((owned_rows, C64, C_out), (other_rows, S64, S_out)): owned_rows and
        other_rows are the given rows split by ownership (global indices), C* the
        reduced rows, S* the published rows (S64 = the fp64 partial).
        """
        A_bits = np.ascontiguousarray(A_bits, dtype=np.uint16)
        M = A_bits.shape[0]
        if not 0 <= own_m0 <= own_m1 <= M:
            raise ValueError("owned rows outside [0, M]")
        rows = np.arange(M) if rows is None else np.asarray(rows, dtype=np.int64)
        mine = (rows >= own_m0) & (rows < own_m1)
        owned, other = rows[mine], rows[~mine]
        C64, C_out = self.gemm_ar(A_bits[own_m0:own_m1], B_bits, peers_own, c_dtype,
                                  rows=owned - own_m0, threads=threads)
        S64, S_out = self.gemm_ar(A_bits, B_bits, None, peer_dtype, rows=other, threads=threads)
        return (owned, C64, C_out), (other, S64, S_out)

    def gemm_ag(self, A_local, peers_A, rank, B_bits, c_dtype="bf16", rows=None, threads=0):
        """Reference for one GPU's share of AllGather+GEMM ("AllGather + GEMM (TP)" row
        of Table 3, thelatestinai.com page: communication -> compute, each GPU's row
        shard of the activations broadcast to every GPU, which multiplies the
        gathered matrix by its own weight shard).

        A_local: uint16 [Ms, K], this GPU's shard (rank `rank` of P); peers_A: uint16
        [P-1, Ms, K], the other GPUs' shards in rank order with `rank` left out;
        B_bits: uint16 [K, N]. The gathered matrix holds shard q at rows
        [q*Ms, (q+1)*Ms). Returns (A_full uint16 [P*Ms, K], C64, C_out) with C the
        product of the gathered matrix and B (rows: None for all, else indices).
        """
        A_local = np.ascontiguousarray(A_local, dtype=np.uint16)
        peers_A = np.ascontiguousarray(peers_A, dtype=np.uint16)
        if peers_A.ndim != 3 or peers_A.shape[1:] != A_local.shape:
            raise ValueError("peers_A must be [P-1, Ms, K] like A_local")
        if not 0 <= rank <= peers_A.shape[0]:
            raise ValueError("rank outside [0, P)")
        shards = [peers_A[q] for q in range(peers_A.shape[0])]
        shards.insert(rank, A_local)
        A_full = np.concatenate(shards, axis=0)
        C64, C_out = self.gemm_ar(A_full, B_bits, None, c_dtype, rows=rows, threads=threads)
        return A_full, C64, C_out

    def bf16_to_f64(self, bits):
        b = np.ascontiguousarray(bits, dtype=np.uint16)
        out = np.empty(b.shape, dtype=np.float64)
        self.lib.mko_bf16_to_f64_array(_ptr(b), _ptr(out), b.size)
        return out

    def f64_to_bf16(self, x):
        a = np.ascontiguousarray(x, dtype=np.float64)
        out = np.empty(a.shape, dtype=np.uint16)
        self.lib.mko_f64_to_bf16_array(_ptr(a), _ptr(out), a.size)
        return out

    def exact_sum(self, values):
        a = np.ascontiguousarray(values, dtype=np.float64)
        if a.size > 64:
            raise ValueError("exact_sum takes at most 64 values (the most peers per element)")
        return self.lib.mko_exact_sum(_ptr(a), a.size)

    def max_threads(self):
        return self.lib.mko_max_threads()


_default = None


def default():
    """The oracle built from mk_oracle.c as committed (built on first use if absent)."""
    global _default
    if _default is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        _default = Oracle(_build.LIB)
    return _default


def gemm_ar(*a, **k):
    return default().gemm_ar(*a, **k)


def gemm_rs(*a, **k):
    return default().gemm_rs(*a, **k)


def gemm_ag(*a, **k):
    return default().gemm_ag(*a, **k)


def bf16_to_f64(bits):
    return default().bf16_to_f64(bits)


def f64_to_bf16(x):
    return default().f64_to_bf16(x)


def exact_sum(values):
    return default().exact_sum(values)


def max_threads():
    return default().max_threads()
