"""GPU parity of the forward for activations handed over already quantized
([P1] sglang PR #28354 summary, "Implementation breakdown" item 2: the runner
is given the FP4 codes, the block scales and the per-token scale).

Bit-exact: codes of x from the oracle's per-token Q give moe_nvfp4_forward(x)'s
output bit for bit (deterministic finalize), at the decode, small-batch and
prefill sizes (all three prologues, stream and tiled GEMMs).  Tolerance: the
output on arbitrary codes, scales and global scales (codes no bf16 row
quantizes to) against the oracle's pre-quantized layer, both finalize modes."""
import numpy as np
import pytest
import torch

import oracle
from nvfp4_token_quant_amd import binding, synth
from tests.layer_fixtures import bf16_tensor_to_f64, check_layer_tolerance, gpu_weights, oracle_weights, to_device_bf16

pytestmark = pytest.mark.gpu

_W = {}


def _weights(layer_id):
    if layer_id not in _W:
        _W.clear()
        torch.cuda.empty_cache()
        _W[layer_id] = gpu_weights(layer_id)
    return _W[layer_id]


def _sample(T, n=24):
    if T <= n:
        return np.arange(T)
    return np.unique(np.concatenate([[0, T - 1], np.random.default_rng(T).choice(T, n - 2, replace=False)]))


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


@pytest.mark.timeout(900)
@pytest.mark.parametrize("layer_id,T", [(1, 16), (2, 64), (2, 301), (3, 4096), (5, 1), (5, 7)])
def test_prequantized_forward_equals_forward(layer_id, T):
    L = synth.LAYERS[layer_id]
    print(f"layer {layer_id} T={T} pre-quantized vs forward", flush=True)
    x, logits = synth.activations(layer_id, T), synth.router_logits(layer_id, T)
    xc, xs, xg = oracle.quantize_rows(x)
    layer = binding.MoeLayer(T, L.H, L.I, L.E, L.k, True)
    layer.bind(_weights(layer_id))
    lg = torch.from_numpy(logits).cuda()
    ref = layer.forward(to_device_bf16(x), lg)
    got = layer.forward_quantized(_dev(xc), _dev(xs), _dev(xg), lg)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
    # the handed-over arrays are read, never written
    np.testing.assert_array_equal(xc, oracle.quantize_rows(x)[0])
    toks = _sample(T)
    ids, w = oracle.router(logits, L.k)
    qw = oracle_weights(layer_id, np.unique(ids[toks]))
    want = oracle.moe_layer_quantized(xc, xs, xg, ids, w, toks, L.H, L.I, qw)
    check_layer_tolerance(bf16_tensor_to_f64(got)[toks], want)


def _arbitrary(T, H, seed):
    """Random codes (every nibble, negative zeros included), block scales in
    [0.5, 448] and global scales around the ones N(0, 1) rows get; row 1
    (if present) is all zero codes."""
    rng = np.random.default_rng(seed)
    xc = rng.integers(0, 256, (T, H // 2), dtype=np.uint8)
    xs = rng.integers(0x30, 0x7F, (T, H // 16), dtype=np.uint8)
    xg = (672.0 * 2.0 ** rng.uniform(-1, 1, T)).astype(np.float32)
    if T > 1:
        xc[1] = 0
    return xc, xs, xg


@pytest.mark.parametrize("layer_id,T,det", [(1, 16, True), (2, 64, True), (2, 64, False), (2, 200, True),
                                            (3, 4096, True), (3, 4096, False)])
def test_prequantized_arbitrary_codes_parity(layer_id, T, det):
    L = synth.LAYERS[layer_id]
    print(f"layer {layer_id} T={T} det={det} arbitrary codes", flush=True)
    logits = synth.router_logits(layer_id, T)
    xc, xs, xg = _arbitrary(T, L.H, 100 + T)
    layer = binding.MoeLayer(T, L.H, L.I, L.E, L.k, det)
    layer.bind(_weights(layer_id))
    got = layer.forward_quantized(_dev(xc), _dev(xs), _dev(xg), torch.from_numpy(logits).cuda())
    torch.cuda.synchronize()
    toks = _sample(T)
    ids, w = oracle.router(logits, L.k)
    qw = oracle_weights(layer_id, np.unique(ids[toks]))
    want = oracle.moe_layer_quantized(xc, xs, xg, ids, w, toks, L.H, L.I, qw)
    got = bf16_tensor_to_f64(got)
    if T > 1:
        assert np.all(got[1] == 0.0)
    check_layer_tolerance(got[toks], want)


def test_prequantized_errors_and_empty():
    L = synth.LAYERS[1]
    T = 16
    xc, xs, xg = _arbitrary(T, L.H, 7)
    logits = torch.from_numpy(synth.router_logits(1, T)).cuda()
    a16 = binding.MoeLayer(T, L.H, L.I, L.E, L.k, True, w4a16=True)
    a16.bind(_weights(1))
    with pytest.raises(binding.Nvfp4Error):
        a16.forward_quantized(_dev(xc), _dev(xs), _dev(xg), logits)
    layer = binding.MoeLayer(T, L.H, L.I, L.E, L.k, True)
    layer.bind(_weights(1))
    # T = 0 is a no-op; more tokens than the workspace holds is refused
    out = torch.empty((0, L.H), dtype=torch.bfloat16, device="cuda")
    layer.forward_quantized_into(_dev(xc), _dev(xs), _dev(xg), logits, out, T=0)
    with pytest.raises(binding.Nvfp4Error):
        layer.forward_quantized_into(_dev(xc), _dev(xs), _dev(xg), logits,
                                     torch.empty((T, L.H), dtype=torch.bfloat16, device="cuda"), T=T + 1)
    # out over the codes: refused (not in-place)
    buf = torch.zeros(T * L.H * 2, dtype=torch.uint8, device="cuda")
    codes_in_out = buf[: T * L.H // 2].view(T, L.H // 2)
    with pytest.raises(binding.Nvfp4Error):
        layer.forward_quantized_into(codes_in_out, _dev(xs), _dev(xg), logits, buf.view(torch.bfloat16).view(T, L.H))
    torch.cuda.synchronize()


@pytest.mark.parametrize("T", [64, 1024])
def test_prequantized_with_shared_expert_and_static_scales(T):
    """With a shared expert ('average'), and with static activation scales
    (x's codes made with the static g_x, the GEMM2 input re-quantized with the
    static g_a), the forward on handed-over codes equals the forward on x bit
    for bit (stream path at T = 64, tiled at T = 1024)."""
    L = synth.LAYERS[2]
    print(f"layer 2 T={T} pre-quantized: shared expert, static scales", flush=True)
    x, logits = synth.activations(2, T), synth.router_logits(2, T)
    lg = torch.from_numpy(logits).cuda()
    xd = to_device_bf16(x)
    # shared expert: the weights hold E + 1 experts
    wts = gpu_weights(2, n_experts=L.E + 1)
    xc, xs, xg = oracle.quantize_rows(x)
    layer = binding.MoeLayer(T, L.H, L.I, L.E, L.k, True, shared_expert="average")
    layer.bind(wts)
    ref = layer.forward(xd, lg)
    got = layer.forward_quantized(_dev(xc), _dev(xs), _dev(xg), lg)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
    layer.close()
    del wts
    # static scales: g_x for x's codes, g_a for the GEMM2 input
    gx = float(oracle.global_scale(synth.bf16_to_f32(x)))
    ga = 40.0
    sc, ss = oracle.quantize_rows_given_g(synth.bf16_to_f32(x), gx)
    sg = np.full(T, gx, np.float32)
    layer = binding.MoeLayer(T, L.H, L.I, L.E, L.k, True, static_act_scales=True)
    layer.bind(_weights(2))
    layer.set_act_scales(torch.tensor([gx, ga], dtype=torch.float32, device="cuda"))
    ref = layer.forward(xd, lg)
    got = layer.forward_quantized(_dev(sc), _dev(ss), _dev(sg), lg)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
    layer.close()
