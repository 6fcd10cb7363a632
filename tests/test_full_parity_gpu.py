"""GPU, opt-in (MK_FULL_PARITY=1; minutes): every workload at full size, EVERY row,
against the CPU oracle -- integer inputs bit-exact, Gaussian inputs within the
tolerance rule of tests/compare.py -- for the fused kernel (default options) and
the two-kernel baseline. The default suite checks the same workloads on sampled
rows (test_parity_gpu.py::test_workload_parity); this is the one full pass per
workload."""
import json
import os

import numpy as np
import pytest
import torch

import mk_inputs
import oracle
from tests.compare import check_exact, tolerance_stats

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(os.environ.get("MK_FULL_PARITY") != "1",
                                 reason="opt-in full-size pass: set MK_FULL_PARITY=1")]

if torch.cuda.is_available():
    import tile_gemm_all_amd as mk
else:  # collected on CPU-only machines, never run there
    mk = None


@pytest.mark.parametrize("variant", ["integer", "gaussian"])
@pytest.mark.parametrize("w", mk_inputs.WORKLOADS, ids=lambda w: w.name)
def test_full_parity(w, variant):
    print(f"\n[case] full parity {w.name} {variant}", flush=True)
    cdt = torch.bfloat16 if w.c_dtype == "bf16" else torch.float32
    A, B, peers = mk_inputs.workload_inputs(w, variant, device="cuda")
    C64, want = oracle.gemm_ar(mk_inputs.bits(A), mk_inputs.bits(B), mk_inputs.bits(peers),
                               w.c_dtype)
    rec = {}
    for mode in ("fused", "baseline"):
        C = torch.empty((w.M, w.N), dtype=cdt, device="cuda")
        (mk.gemm_ar_local if mode == "fused" else mk.gemm_then_reduce_baseline)(A, B, peers, C)
        mk.stream_status()
        got = mk_inputs.bits(C)
        if variant == "integer":
            check_exact(got, want, f"{w.name} {mode}")
            rec[mode] = {"elements": int(got.size), "bit_mismatches": 0}
        else:
            st = tolerance_stats(got, C64, w.c_dtype)
            rec[mode] = {"elements": int(got.size), "within_tolerance": st["ok"],
                         "max_abs_err": st["max_abs_err"],
                         "rms_err_over_rms": st["rms_err_over_rms"],
                         "literal_bound": st["literal_bound"]}
            assert st["ok"], (w.name, mode, st)
    print("[full-parity] " + json.dumps({"workload": w.name, "variant": variant, **rec}),
          flush=True)
