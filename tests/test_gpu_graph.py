"""The attention path under HIP graph capture: a captured segkv_attn_prefill
(persistent two-block kernel with its queue-zeroing kernel, split runs and
the merge pass) and its allocation-free twin, each replayed several times
with eager work and synchronisation between the replays; every replay equals
the eager result bit for bit."""

import pytest
import torch

import head_segmented_paged_amd as H
from tests.common import adhoc
from tests.gpu_helpers import GpuLayer, say
from workloads import layer_tensors, realize

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


@pytest.mark.parametrize("noalloc", [False, True], ids=["workspace", "noalloc"])
def test_graph_replays_match_eager(noalloc):
    w = adhoc(hq=8, hkv=2, d=128, page=64, window=1500, classes=(1, 0), seqs=((2500, 8300),), seed=5)
    r = realize(w)
    say(f"[graph] noalloc {noalloc}: hq {w.hq} hkv {w.hkv} seqs {list(zip(r.cached_len, r.new_len))}")
    # runs of at most 24 tiles, or 48 (partial results within the no-alloc scratch)
    gl = GpuLayer(w, r, 0, layer_tensors(w, r, 0, device="cuda"), max_unit_tiles=48 if noalloc else 24)
    gl.write()
    host = gl.tables()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert host["num_units"] > cus and host["num_parts"] > 0 and host["num_merges"] > 0
    rows = int(r.new_len.sum())
    q = gl.t["q"]
    ws = torch.empty(max(host["workspace_bytes"], 1), dtype=torch.uint8, device="cuda")

    def run(o, lse):
        if noalloc:
            H.segkv_attn_prefill_noalloc(gl.ctx, gl.dev, q, o, lse)
        else:
            H.segkv_attn_prefill(gl.ctx, gl.dev, q, o, lse, workspace=ws)

    o_ref = torch.empty((rows, w.hq, w.d), dtype=torch.bfloat16, device="cuda")
    lse_ref = torch.empty((w.hq, rows), dtype=torch.float32, device="cuda")
    run(o_ref, lse_ref)
    torch.cuda.synchronize()
    o, lse = torch.empty_like(o_ref), torch.empty_like(lse_ref)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run(o, lse)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(o, lse)
    torch.cuda.synchronize()
    for i in range(3):
        o.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        say(f"[graph] replay {i}")
        assert torch.equal(o, o_ref), f"replay {i}: output differs"
        assert torch.equal(lse, lse_ref), f"replay {i}: lse differs"
