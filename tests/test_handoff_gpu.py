"""GPU: the tile-flag hand-off microbenchmark and message-passing litmus
(mk_flag_handoff). Every call completes within its bounded waits; every later
call sees only its own steps; and the fused kernel's flag protocol (stores
complete + relaxed flag store, agent-scope acquire) carries the data written
before the flag in every same-XCD hand-off, as does agent-scope release/acquire
on one XCD or across two."""
import pytest
import torch

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import tile_gemm_all_amd as mk
else:  # collected on CPU-only machines, never run there
    mk = None


@pytest.mark.parametrize("scope,cross", [(2, False), (1, False), (1, True)],
                         ids=["fused-protocol-same-xcd", "agent-same-xcd", "agent-cross-xcd"])
def test_flag_handoff_carries_the_data(scope, cross):
    print(f"\n[case] flag hand-off scope {scope} cross-XCD {cross}", flush=True)
    torch.cuda.set_device(0)
    for iters in (1, 20000, 7):  # repeated calls on one workspace
        ns, stale, xcds = mk.flag_handoff(iters, scope, cross)
        assert 0.0 < ns < 100_000.0, (iters, ns)
        if (xcds[0] == xcds[1]) == (not cross):  # the two sides landed as intended
            assert stale == 0, (iters, stale, xcds)
    mk.stream_status()


def test_flag_handoff_workgroup_scope_invalidate_completes():
    """The workgroup-scope invalidate (scope 0) is only timed and counted: it is
    known not to carry the data (its stale count is reported, not asserted)."""
    print("\n[case] flag hand-off scope 0", flush=True)
    ns, stale, _ = mk.flag_handoff(1000, 0, False)
    assert 0.0 < ns < 100_000.0 and 0 <= stale <= 1000
    mk.stream_status()


@pytest.mark.gpu
def test_mfma_peak_runs_every_chain():
    """The matrix-core ceiling kernel does the work it is timed for: each lane's sum
    of its eight accumulators after n rounds is exactly n times the sum after one
    (small integer operands, exact in fp32), and no lane's sum is zero."""
    import torch
    print("\n[case] mfma peak linearity", flush=True)
    grid = 4
    outs = {}
    for n in (1, 3):
        out = torch.full((grid * 256,), float("nan"), dtype=torch.float32, device="cuda")
        mk.mfma_peak(n, grid, out)
        mk.stream_status()
        outs[n] = out.cpu()
    assert torch.isfinite(outs[1]).all()
    assert (outs[1] != 0).all()
    assert torch.equal(outs[3], 3 * outs[1])
