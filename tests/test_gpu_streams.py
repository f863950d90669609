"""Entry points hold no global state: two layers enqueued on two streams at
once give bit for bit what each gives alone on the default stream (bf16 and
fp8 attention, a mean-gate and a TripPool layer of different shapes)."""
import pytest

from tests import gpu_support as gs
from workloads.configs import HEAD_AWARE_CYCLE, Workload

pytestmark = pytest.mark.gpu

A = Workload("st-a", "bf16", 1, 3, 128, (5, 16, 20), (40, 300, 24), ((4, 4, 4),),
             "mean_gate", 0.75, 4401)
B = Workload("st-b", "bf16", 2, 3, 128, (4, 12, 24), (100, 700, 30), HEAD_AWARE_CYCLE,
             "trippool", 0.8, 4402)


def _layer(w, fp8, fused=False):
    import torch
    from block_sparse_video_map_amd import vsa
    from workloads.inputs import make_weights
    layer = vsa.Layer(gs.problem_of(w), w.sparsity, vsa.score_mode(w.scorer, w.tripool_mode),
                      w.d if w.scorer == "mean_gate" else w.proj_dim, fp8=fp8, fused=fused)
    W = make_weights(w)
    if w.scorer == "mean_gate":
        weights = (torch.from_numpy(W["gate"]).cuda(), None)
    else:
        weights = (torch.from_numpy(W["proj_q"]).cuda(), torch.from_numpy(W["proj_k"]).cuda())
    return layer, gs.to_device(w), weights


@pytest.mark.parametrize("fp8_a,fp8_b,fused",
                         [(False, False, False), (True, True, False), (False, False, True),
                          (False, True, False)],
                         ids=["bf16", "fp8", "bf16-fused-select", "bf16-beside-fp8"])
def test_two_streams_match_sequential_runs(fp8_a, fp8_b, fused):
    """The fused case also guards the bf16 attention kernel against stale LDS:
    its V rings must not feed bytes another kernel left there (possibly NaN
    patterns) into the products of a step without a unit. The mixed case runs
    the two attention kernels beside each other."""
    import torch
    la, ia, wa = _layer(A, fp8_a, fused)
    lb, ib, wb = _layer(B, fp8_b, fused)
    la.forward(*ia, *wa)
    lb.forward(*ib, *wb)
    torch.cuda.synchronize()
    ref = [la.out.clone(), la.lse.clone(), lb.out.clone(), lb.lse.clone()]
    for t in (la.out, la.lse, lb.out, lb.lse):
        t.zero_()
    torch.cuda.synchronize()
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    for _ in range(3):
        with torch.cuda.stream(sa):
            la.forward(*ia, *wa)
        with torch.cuda.stream(sb):
            lb.forward(*ib, *wb)
    torch.cuda.synchronize()
    got = [la.out, la.lse, lb.out, lb.lse]
    gs.log(f"[streams] fp8={fp8_a},{fp8_b} fused={fused}: comparing {len(got)} buffers")
    for r, g in zip(ref, got):
        assert torch.equal(r, g)
