"""GPU: the tile-flag hand-off microbenchmark (one publish and its acquire between
two workgroups, nothing else in flight) completes, within its bounded waits, for
both flag protocols; every later call sees only its own steps."""
import pytest
import torch

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import tile_gemm_all_amd as mk
else:  # collected on CPU-only machines, never run there
    mk = None


@pytest.mark.parametrize("scope", [0, 1], ids=["xcd-local", "agent-scope"])
def test_flag_handoff_completes(scope):
    print(f"\n[case] flag hand-off, scope {scope}", flush=True)
    torch.cuda.set_device(0)
    for iters in (1, 1000, 7):  # repeated calls on one workspace
        ns, xcds = mk.flag_handoff(iters, scope)
        assert 0.0 < ns < 100_000.0, (iters, ns)
        assert 0 <= xcds[0] < 16 and 0 <= xcds[1] < 16
    mk.stream_status()
