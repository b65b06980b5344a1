"""Captured forwards replay like eager forwards: the prefill path (tiled
GEMMs, the separate re-quantization / bf16 conversion kernel) for the NVFP4
layer, the W4A16 layer and the layer with a shared expert, the forward on
handed-over codes, and the decode-sized path (one-block prologue, stream
GEMMs) in both finalize modes; every replay is checked, with eager work and
synchronizations between the replays."""
import numpy as np
import pytest
import torch

from nvfp4_token_quant_amd import binding, synth
from tests.layer_fixtures import gpu_weights, to_device_bf16

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("mode", ["nvfp4", "w4a16", "shared"])
def test_tiled_forward_graph_replay(mode):
    L = synth.LAYERS[1]
    T = 256
    print(f"graph replay, layer 1 T={T} mode={mode}", flush=True)
    shared = "sum" if mode == "shared" else None
    wts = gpu_weights(1, n_experts=L.E + (1 if shared else 0))
    layer = binding.MoeLayer(T, L.H, L.I, L.E, L.k, True, shared_expert=shared, w4a16=(mode == "w4a16"))
    layer.bind(wts)
    x = to_device_bf16(synth.activations(1, T))
    logits = torch.from_numpy(synth.router_logits(1, T)).cuda()
    out = torch.empty_like(x)
    layer.forward_into(x, logits, out)
    torch.cuda.synchronize()
    eager = out.clone()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        layer.forward_into(x, logits, out)
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            layer.forward_into(x, logits, out)
    torch.cuda.synchronize()
    other = torch.empty_like(x)
    for _ in range(3):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager)
        layer.forward_into(x[:17], logits[:17], other, T=17)   # eager work between replays
        torch.cuda.synchronize()
    layer.close()


@pytest.mark.parametrize("T", [64, 256])
def test_prequantized_forward_graph_replay(T):
    """The forward on handed-over codes (decode-sized stream path at T = 64,
    tiled path at T = 256) captured and replayed equals the eager forward on
    x, whose codes they are."""
    L = synth.LAYERS[1]
    print(f"graph replay, layer 1 T={T} pre-quantized", flush=True)
    layer = binding.MoeLayer(T, L.H, L.I, L.E, L.k, True)
    layer.bind(gpu_weights(1))
    x = to_device_bf16(synth.activations(1, T))
    logits = torch.from_numpy(synth.router_logits(1, T)).cuda()
    codes, scales, gs = binding.quantize_per_token(x)
    eager = layer.forward(x, logits)
    out = torch.empty_like(x)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        layer.forward_quantized_into(codes, scales, gs, logits, out)
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            layer.forward_quantized_into(codes, scales, gs, logits, out)
    torch.cuda.synchronize()
    other = torch.empty_like(x)
    for _ in range(3):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16))
        layer.forward_into(x[:17], logits[:17], other, T=17)   # eager work between replays
        torch.cuda.synchronize()
    layer.close()


@pytest.mark.parametrize("T,deterministic", [(1, True), (7, True), (64, True), (7, False)])
def test_stream_forward_graph_replay(T, deterministic):
    """Decode-sized forwards (one-block prologue with either router, stream
    GEMMs) captured and replayed: every replay equals the eager forward, bit
    for bit in the slot-ordered finalize, within a few bf16 ulps with the
    atomic one (fp32 adds in arrival order)."""
    L = synth.LAYERS[2]
    print(f"graph replay, layer 2 T={T} deterministic={deterministic}", flush=True)
    layer = binding.MoeLayer(64, L.H, L.I, L.E, L.k, deterministic)
    layer.bind(gpu_weights(2))
    x = to_device_bf16(synth.activations(2, T))
    logits = torch.from_numpy(synth.router_logits(2, T)).cuda()
    out = torch.empty_like(x)
    layer.forward_into(x, logits, out)
    torch.cuda.synchronize()
    eager = out.float().cpu().numpy()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        layer.forward_into(x, logits, out)
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            layer.forward_into(x, logits, out)
    torch.cuda.synchronize()
    other = torch.empty((64, L.H), dtype=torch.bfloat16, device="cuda")
    xo = to_device_bf16(synth.activations(2, 64))
    lo = torch.from_numpy(synth.router_logits(2, 64)).cuda()
    for _ in range(3):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        got = out.float().cpu().numpy()
        if deterministic:
            np.testing.assert_array_equal(got, eager)
        else:
            assert np.abs(got - eager).max() <= 4 * 2.0 ** -8 * np.abs(eager).max()
        layer.forward_into(xo, lo, other)   # eager work on another batch between replays
        torch.cuda.synchronize()
    layer.close()
