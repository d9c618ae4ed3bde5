"""The mixer stack captured in a HIP graph: every replay equals the eager result bitwise,
with eager launches and synchronisations between the replays (the benchmark replays the
same capture)."""
import numpy as np
import pytest
import torch

import ternary_weight_selective_amd as tws
import workloads as wl
from gpu_helpers import DEV, gpu_config, host, quantize_layer, to_dev, torch_dtype

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,layers,batch", [("trissm", 3, 8), ("ternaryssm50m", 2, 2), ("mamba2_ssd", 1, 1)])
def test_graph_replay_matches_eager(name, layers, batch):
    cfg = wl.CONFIGS[name]
    lat, u = wl.mixer_problem(cfg, seed=5, layers=layers, batch=batch)
    gws = [quantize_layer(cfg, l, check=False)[0] for l in lat]
    c = gpu_config(cfg)
    mws = [tws.mixer_weights(g) for g in gws]
    u_dev = to_dev(u, torch_dtype(cfg))
    bufs = [torch.empty_like(u_dev), torch.empty_like(u_dev)]
    ws = torch.empty(tws.ssm_mixer_workspace_bytes(c, batch, cfg.seqlen), dtype=torch.uint8, device=DEV)

    def step(stream=None):
        h = u_dev
        for i, mw in enumerate(mws):
            h = tws.ssm_mixer_fwd(c, mw, h, add_residual=True, out=bufs[i % 2], workspace=ws, stream=stream)
        return h

    eager = host(step()).copy()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step(s)
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            out = step(s)
    torch.cuda.synchronize()
    for _ in range(4):
        bufs[0].fill_(7.0)
        bufs[1].fill_(-3.0)
        g.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(out), eager)
        other = host(step())  # eager work between replays
        np.testing.assert_array_equal(other, eager)
