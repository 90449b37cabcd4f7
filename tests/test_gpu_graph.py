"""The layer captured in a HIP graph: every replay equals the eager result."""
import pytest
import torch

import bit_quantized_moe_top_amd as mq
import workloads as W

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


@pytest.mark.parametrize("name", ["tiny", "decode_small"])
def test_graph_replays_match_eager(name):
    if name == "tiny":
        cfg = W.get_config("tiny")
    else:        # decode shape with fewer experts, so the test stays small
        cfg = W.get_config("decode", E=32)
    inp = W.make_layer_inputs(cfg, device=DEV)
    layer = mq.MoELayer(cfg.H, cfg.I, cfg.E, cfg.k, "w4a8", device=DEV)
    layer.quantize_weights(inp["w13"], inp["w2"])
    x = inp["x"].clone()
    logits = inp["logits"].clone()
    y_eager = layer.forward(x, logits).clone()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        y_graph = layer.forward(x, logits)
    gen = torch.Generator(device=DEV)
    for rep in range(3):
        # new inputs written into the captured buffers, eager work in between
        gen.manual_seed(rep)
        x.copy_(inp["x"] * (1 + rep) if rep else inp["x"])
        logits.copy_(inp["logits"] + rep * torch.randn(logits.shape, generator=gen, device=DEV))
        torch.cuda.synchronize()
        expect = layer.forward(x.clone(), logits.clone()).clone()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y_graph, expect), f"replay {rep}"
        if rep == 0:
            assert torch.equal(y_graph, y_eager)
