"""A call captured into a HIP graph (torch.cuda.CUDAGraph) replays to the
eager result every time: with a workspace and output buffers passed in, the
library enqueues kernels only (no allocation, memset or host
synchronisation). Replays are interleaved with eager calls and host
synchronisations, and every replay is checked."""
import numpy as np
import pytest
import torch

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X GPU")]

import speculative_decoding_verification_11_amd as sv  # noqa: E402
from speculative_decoding_verification_11_amd import workloads as wl  # noqa: E402
from test_gpu_parity import DEV, say  # noqa: E402


@pytest.mark.parametrize("entry", ["spec_verify", "spec_verify_early_exit"])
def test_graph_replay_matches_eager(entry):
    fn = getattr(sv, entry)
    b = wl.generate(wl.WORKLOADS["c3"], DEV)
    seed = wl.philox_seeds("c3", 1)[0]
    ws = torch.empty(sv.workspace_size(b.B, b.k, b.V, b.workload.dtype_code), dtype=torch.uint8,
                     device=DEV)
    out = (torch.empty((b.B, b.k + 1), dtype=torch.int32, device=DEV),
           torch.empty((b.B,), dtype=torch.int32, device=DEV))
    args = (b.target, b.draft, b.draft_tokens, b.draft_len, b.temperature, seed)
    fn(*args, workspace=ws, out=out)
    torch.cuda.synchronize()
    ref = (out[0].cpu().numpy(), out[1].cpu().numpy())

    side = torch.cuda.Stream(device=DEV)  # default priority
    side.wait_stream(torch.cuda.current_stream(DEV))
    with torch.cuda.stream(side):  # warm the binding on the capture stream
        fn(*args, workspace=ws, out=out)
    torch.cuda.current_stream(DEV).wait_stream(side)
    torch.cuda.synchronize()
    say(f"[case] graph capture: {entry}")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn(*args, workspace=ws, out=out)
    eager_out = (torch.empty_like(out[0]), torch.empty_like(out[1]))
    for rep in range(4):
        out[0].fill_(-9)
        out[1].fill_(-9)
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out[0].cpu().numpy(), ref[0]), f"replay {rep}: tokens"
        assert np.array_equal(out[1].cpu().numpy(), ref[1]), f"replay {rep}: counts"
        fn(*args, workspace=ws, out=eager_out)  # eager work between replays
        torch.cuda.synchronize()
        assert np.array_equal(eager_out[0].cpu().numpy(), ref[0])
