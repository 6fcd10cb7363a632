"""Seeded synthetic inputs for one GPU's share of GEMM+AllReduce.

This module only draws random numbers and lays them out; it holds none of the
operation's arithmetic. Both the GPU path's tests/benchmark and the CPU oracle
take their inputs from here, so the two sides see the same bits.

Workloads (model-shaped, synthetic; no dataset or weights are involved):

  tiny     M=256   N=512  K=512   P=4   fp32 peers, fp32 C
  mlp      M=4096  N=8192 K=1792  P=16  Llama-70B-like MLP down projection,
                                        row-parallel shard (28672/16)
  attn     M=16384 N=8192 K=512   P=16  attention output projection shard (8192/16)
  large    M=8192  N=8192 K=8192  P=8   compute-bound shard
  decode   M=128   N=8192 K=1792  P=16  decode-sized skinny shard

AllGather+GEMM share (the "AllGather + GEMM (TP)" row of Table 3):

  ag_up    Ms=256 rows per GPU, P=16 (4096 gathered rows), K=8192, N=3584:
           Llama-70B-like MLP gate+up projection, column-parallel shard
           (2*28672/16 columns); bf16 C

Value distributions:
  gaussian  A, B ~ N(0,1)/sqrt(K) drawn in fp32 and rounded to bfloat16 by
            torch's conversion (round to nearest even); peers ~ N(0,1) in the
            peer dtype.
  integer   A, B and peers uniform integers in [-4, 4] (exact in bfloat16).
  zeropeer  gaussian A, B with all-zero peers (same traffic; C = A*B).

Seeds: 1000*config_index + {0: A, 1: B, 2: peers}, +100 for the integer
variant. Draws use torch.Generator on the requested device, so a CPU draw and
a GPU draw of the same seed differ; callers hand the oracle copies of the bits
that were actually used.
"""
import hashlib
import math
from dataclasses import dataclass

import torch


@dataclass(frozen=True)
class Workload:
    index: int
    name: str
    M: int
    N: int
    K: int
    P: int
    peer_dtype: str  # "bf16" | "f32"
    c_dtype: str  # "bf16" | "f32"
    description: str

    @property
    def n_peers(self):
        return self.P - 1

    @property
    def flops(self):
        return 2.0 * self.M * self.N * self.K

    def compulsory_bytes(self):
        """A + B + peers + C, read or written once each."""
        pb = 2 if self.peer_dtype == "bf16" else 4
        cb = 2 if self.c_dtype == "bf16" else 4
        return (2 * self.M * self.K + 2 * self.K * self.N + self.n_peers * pb * self.M * self.N
                + cb * self.M * self.N)


WORKLOADS = [
    Workload(1, "tiny", 256, 512, 512, 4, "f32", "f32", "tiny shard, fp32 peers and C"),
    Workload(2, "mlp", 4096, 8192, 1792, 16, "bf16", "bf16",
             "Llama-70B-like MLP down-proj row-parallel shard"),
    Workload(3, "attn", 16384, 8192, 512, 16, "bf16", "bf16",
             "attention out-proj shard, reduce-heavy"),
    Workload(4, "large", 8192, 8192, 8192, 8, "bf16", "bf16", "large compute-bound shard"),
    Workload(5, "decode", 128, 8192, 1792, 16, "bf16", "bf16", "decode-sized skinny shard"),
]
BY_NAME = {w.name: w for w in WORKLOADS}

_TORCH_DT = {"bf16": torch.bfloat16, "f32": torch.float32}


def _gen(seed, device):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def gaussian(shape, seed, scale=1.0, dtype="bf16", device="cpu"):
    """N(0,1)*scale drawn in fp32, then converted to dtype by torch."""
    x = torch.randn(*shape, generator=_gen(seed, device), device=device, dtype=torch.float32)
    if scale != 1.0:
        x.mul_(scale)
    return x.to(_TORCH_DT[dtype])


def integers(shape, seed, lo=-4, hi=4, dtype="bf16", device="cpu"):
    """Uniform integers in [lo, hi], exactly representable in dtype."""
    x = torch.randint(lo, hi + 1, tuple(shape), generator=_gen(seed, device), device=device,
                      dtype=torch.int32)
    return x.to(_TORCH_DT[dtype])


def make_inputs(M, N, K, n_peers, peer_dtype="bf16", variant="gaussian", seed_base=0,
                device="cpu"):
    """Returns (A [M,K] bf16, B [K,N] bf16, peers [n_peers,M,N] peer_dtype)."""
    if variant == "integer":
        sb = seed_base + 100
        A = integers((M, K), sb + 0, device=device)
        B = integers((K, N), sb + 1, device=device)
        peers = integers((n_peers, M, N), sb + 2, dtype=peer_dtype, device=device)
    elif variant in ("gaussian", "zeropeer"):
        s = 1.0 / math.sqrt(K) if K > 0 else 1.0
        A = gaussian((M, K), seed_base + 0, s, device=device)
        B = gaussian((K, N), seed_base + 1, s, device=device)
        if variant == "gaussian":
            peers = gaussian((n_peers, M, N), seed_base + 2, 1.0, dtype=peer_dtype, device=device)
        else:
            peers = torch.zeros((n_peers, M, N), dtype=_TORCH_DT[peer_dtype], device=device)
    else:
        raise ValueError(f"unknown variant {variant}")
    return A, B, peers


@dataclass(frozen=True)
class AgWorkload:
    index: int
    name: str
    Ms: int  # rows per GPU's shard
    P: int
    N: int
    K: int
    c_dtype: str
    description: str

    @property
    def M(self):
        return self.P * self.Ms

    @property
    def flops(self):
        return 2.0 * self.M * self.N * self.K

    def compulsory_bytes(self):
        """Shards read once, gathered matrix written once, B read once, C written once."""
        cb = 2 if self.c_dtype == "bf16" else 4
        return 2 * self.M * self.K * 2 + 2 * self.K * self.N + cb * self.M * self.N


AG_WORKLOADS = [
    AgWorkload(6, "ag_up", 256, 16, 3584, 8192, "bf16",
               "Llama-70B-like MLP gate+up column-parallel shard, activations gathered"),
]
AG_BY_NAME = {w.name: w for w in AG_WORKLOADS}


def make_ag_inputs(Ms, P, N, K, variant="gaussian", seed_base=0, device="cpu"):
    """Returns (shards [P,Ms,K] bf16: every GPU's row shard of the activations,
    B [K,N] bf16). A GPU of rank r takes shards[r] as its own and the others as
    its peers' (shard_split)."""
    if variant == "integer":
        sb = seed_base + 100
        shards = integers((P, Ms, K), sb + 0, device=device)
        B = integers((K, N), sb + 1, device=device)
    elif variant == "gaussian":
        s = 1.0 / math.sqrt(K) if K > 0 else 1.0
        shards = gaussian((P, Ms, K), seed_base + 0, s, device=device)
        B = gaussian((K, N), seed_base + 1, s, device=device)
    else:
        raise ValueError(f"unknown variant {variant}")
    return shards, B


def shard_split(shards, rank):
    """(own shard [Ms,K], the others [P-1,Ms,K] in rank order with `rank` left out)."""
    idx = [q for q in range(shards.shape[0]) if q != rank]
    return shards[rank].contiguous(), shards[idx].contiguous()


def workload_inputs(w: Workload, variant="gaussian", device="cpu"):
    return make_inputs(w.M, w.N, w.K, w.n_peers, w.peer_dtype, variant, 1000 * w.index, device)


def bits(t):
    """Raw bit patterns of a CPU/GPU tensor as a numpy array (uint16 for bf16)."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view("uint16")
    if t.dtype == torch.float32:
        return t.numpy()
    raise ValueError(t.dtype)


def sha256(t):
    return hashlib.sha256(bits(t).tobytes()).hexdigest()[:16]
