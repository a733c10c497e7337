"""The library allocates nothing and issues only kernel launches on the
caller's stream, so the whole path can be captured in a HIP graph.  The FA4
autotuning page ("Validation") lists graph replay in the numerical matrix of a
dense attention kernel; here each replay of a captured quantize + forward is
checked bit for bit against the eager result on the same inputs, with eager
work and new input values between replays."""
import numpy as np
import pytest

import precision_flash_attention_amd as sattn
import testkit
from gpu_helpers import from_dev, log, to_dev

pytestmark = pytest.mark.gpu


def _eager(qd, kd, vd, packed, work, scale):
    p = sattn.quantize_qkv(qd, kd, vd, packed=packed, workspace=work)
    attend = sattn.fwd if p.Nq == p.Nkv else sattn.fwd_cross
    return attend(p, scale, num_splits=0)


# (32760, 512): 384 query tiles of 256 against 4 key tiles, more tiles than
# CUs, so the short-key kernel runs
@pytest.mark.parametrize("Nq,Nkv", [(300, 300), (700, 200), (64, 4608), (32760, 512)])
def test_graph_replay_matches_eager(device, Nq, Nkv):
    import torch
    log(f"graph capture / replay, Nq={Nq} Nkv={Nkv}")
    cfg = testkit.CONFIGS[2]
    scale = cfg.softmax_scale
    inputs = [testkit.make_inputs(cfg, seed=900 + i, B=1, H=3, Nq=Nq, Nkv=Nkv) for i in range(3)]
    qd, kd, vd = (to_dev(a) for a in inputs[0])
    pb, wb = sattn.packed_bytes(1, 3, Nq, Nkv)
    packed = torch.empty(pb, dtype=torch.uint8, device=device)
    work = torch.empty(wb, dtype=torch.uint8, device=device)
    out = torch.empty((1, Nq, 3, 128), dtype=torch.bfloat16, device=device)
    # (64, 4608) runs split-KV (4 key ranges and the merge kernel); its
    # workspace is allocated before the capture
    swb, splits = sattn.fwd_workspace_bytes(1, 3, Nq, Nkv)
    assert splits == (4 if Nkv == 4608 else 1)
    sws = torch.empty(swb, dtype=torch.uint8, device=device) if swb else None

    # eager references on separate buffers, one per input set
    refs = []
    for q, k, v in inputs:
        refs.append(from_dev(_eager(to_dev(q), to_dev(k), to_dev(v), None, None, scale)))
    torch.cuda.synchronize()

    # warm up on a side stream (first-call device checks and attributes
    # happen outside the capture), then capture on it
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        p = sattn.quantize_qkv(qd, kd, vd, packed=packed, workspace=work)
        (sattn.fwd if Nq == Nkv else sattn.fwd_cross)(p, scale, out=out, num_splits=0, workspace=sws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        p = sattn.quantize_qkv(qd, kd, vd, packed=packed, workspace=work)
        (sattn.fwd if Nq == Nkv else sattn.fwd_cross)(p, scale, out=out, num_splits=0, workspace=sws)

    for rep in range(6):
        i = rep % 3
        q, k, v = inputs[i]
        # new input values (eager copies) and some unrelated eager work
        qd.copy_(to_dev(q))
        kd.copy_(to_dev(k))
        vd.copy_(to_dev(v))
        out.fill_(0)
        _ = torch.ones(1 << 20, device=device).sum()
        g.replay()
        torch.cuda.synchronize()
        got = from_dev(out)
        assert np.array_equal(got, refs[i]), f"replay {rep} (inputs {i}) differs from eager"
    log("  6 replays equal to eager")
