"""The whole path (grouping, demean/quantise, attention) captured in one HIP graph through
torch's graph API: the library allocates, synchronises and clears nothing itself, so the
captured launches replay to bit-identical results (checked on every replay, with eager work of
the same calls between replays)."""
import pytest
import torch

import bit_attention_video_amd as vc

from gpu_util import bf16_dev, config_inputs, note

pytestmark = pytest.mark.gpu


def test_path_captured_in_a_graph_replays_bit_exactly():
    cfg, Q, K, V = config_inputs("medium", [0, 1])
    Qd, Kd, Vd = bf16_dev(Q), bf16_dev(K), bf16_dev(V)

    def path():
        g = vc.vc_vsmooth_group(Vd, cfg.k, 3)
        ops = vc.vc_vsmooth_demean_quant(Kd, Vd, g["perm"])
        O = vc.vc_attn_fwd(Qd, ops["Kq"], ops["sK"], ops["Rq"], ops["mu"], ops["sV"])
        return g, O

    g_ref, O_ref = path()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        path()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    note("capturing grouping + demean/quantise + attention")
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        g_cap, O_cap = path()
    for rep in range(3):
        path()                    # eager work between the replays
        graph.replay()
        torch.cuda.synchronize()
        note(f"replay {rep}")
        assert torch.equal(O_cap, O_ref)
        for key in ("labels", "perm", "offsets", "C", "J"):
            assert torch.equal(g_cap[key], g_ref[key]), key
