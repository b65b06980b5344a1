"""Pins of the oracle's router, expandInputRows permutation and layer.

  * router: torch.topk + torch.softmax over all experts, gathered and
    renormalized (library route); weights sum to 1; ties -> smaller index;
  * permutation: numpy bincount / cumsum / stable argsort (library);
  * layer: the oracle's expert-grouped layer equals the brute-force dense
    variant (every expert on every token, routed ones kept) on the tiny
    layer; each intermediate (SwiGLU activation, its re-quantization, the
    down projection, the weighted sum) is recomputed with numpy matmuls and
    scipy's expit from lookup-table dequantization;
  * lossless case: with weights and activations on the NVFP4 grid the gate/up
    projection equals a plain float64 matmul of the unquantized values.
"""
import numpy as np
import pytest
import torch
from scipy.special import expit

import oracle
from nvfp4_token_quant_amd import synth
from tests import npref


def test_router_matches_torch_topk_softmax():
    rng = np.random.default_rng(10)
    logits = rng.standard_normal((300, 64)).astype(np.float32) * 2
    ids, w = oracle.router(logits, 8)
    lt = torch.from_numpy(logits)
    vals, tids = torch.topk(lt, 8, dim=-1, sorted=True)
    np.testing.assert_array_equal(ids, tids.numpy())
    p = torch.softmax(lt.double(), dim=-1).gather(1, tids)
    p = (p / p.sum(dim=-1, keepdim=True)).numpy()
    np.testing.assert_allclose(w, p, rtol=0, atol=1e-12)
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-12)
    assert np.all(np.diff(w, axis=1) <= 0)


def test_router_ties_go_to_smaller_index():
    logits = np.array([[1.0, 3.0, 3.0, 0.5, 3.0, -1.0]], np.float32)
    ids, w = oracle.router(logits, 4)
    assert ids.tolist() == [[1, 2, 4, 0]]
    np.testing.assert_allclose(w[0, :3], w[0, 0])


def test_router_signed_zero_ties():
    """-0.0 and +0.0 compare equal in binary32, so they tie like any equal
    logits: the smaller expert index wins and the slot order follows the
    index.  Checked against a sort on (-value, index) in Python floats,
    where -0.0 == 0.0 as well."""
    rng = np.random.default_rng(12)
    vals = np.array([-0.0, 0.0, 1.0, -1.0, 0.5], np.float32)
    logits = rng.choice(vals, size=(200, 12)).astype(np.float32)
    ids, w = oracle.router(logits, 5)
    for t in range(logits.shape[0]):
        want = sorted(range(12), key=lambda e: (-float(logits[t, e]), e))[:5]
        assert ids[t].tolist() == want
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-12)


def test_permutation_matches_stable_argsort():
    rng = np.random.default_rng(11)
    T, k, E = 500, 8, 40
    ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    counts, offsets, perm, inv = oracle.permute(ids, E)
    flat = ids.ravel()
    np.testing.assert_array_equal(counts, np.bincount(flat, minlength=E))
    np.testing.assert_array_equal(offsets, np.concatenate([[0], np.cumsum(counts)]))
    np.testing.assert_array_equal(perm, np.argsort(flat, kind="stable"))
    np.testing.assert_array_equal(inv[perm], np.arange(T * k))


def _tiny_weights(layer_id=1, E=None):
    L = synth.LAYERS[layer_id]
    E = L.E if E is None else E
    (r13, c13), (r2, c2) = synth.weight_shapes(layer_id)
    w13 = np.stack([oracle.synth_weights(*synth.weight_key(layer_id, 1), e, (r13, c13), L.sigma)
                    for e in range(E)])
    w2 = np.stack([oracle.synth_weights(*synth.weight_key(layer_id, 2), e, (r2, c2), L.sigma)
                   for e in range(E)])
    q13 = oracle.quantize_groups(w13)
    q2 = oracle.quantize_groups(w2)
    return w13, w2, q13, q2


def test_layer_equals_dense_bruteforce():
    L = synth.LAYERS[1]
    x = synth.activations(1)
    logits = synth.router_logits(1)
    ids, w = oracle.router(logits, L.k)
    _, _, q13, q2 = _tiny_weights()
    qw = oracle.QuantWeights(np.arange(L.E), *q13, *q2)
    out = oracle.moe_layer(x, ids, w, np.arange(L.T), L.H, L.I, qw)
    dense = oracle.moe_layer_dense(x, ids, w, L.H, L.I, L.E, *q13, *q2)
    np.testing.assert_allclose(out, dense, rtol=1e-12, atol=1e-12 * np.abs(dense).max())
    assert np.all(np.isfinite(out))


def test_layer_and_routing_invariant_under_token_order():
    """Shuffling the tokens (rows of x and of the logits) shuffles the router
    output and the layer output the same way, value for value: each token's
    result depends on that token alone.  The expandInputRows permutation is
    rebuilt for the new order and stays a stable counting sort (rows of one
    expert in ascending (token, slot) order), so it is not simply permuted."""
    L = synth.LAYERS[1]
    x = synth.activations(1)
    logits = synth.router_logits(1)
    _, _, q13, q2 = _tiny_weights()
    qw = oracle.QuantWeights(np.arange(L.E), *q13, *q2)
    ids, w = oracle.router(logits, L.k)
    out = oracle.moe_layer(x, ids, w, np.arange(L.T), L.H, L.I, qw)
    pi = np.random.default_rng(17).permutation(L.T)
    ids_p, w_p = oracle.router(logits[pi], L.k)
    np.testing.assert_array_equal(ids_p, ids[pi])
    np.testing.assert_array_equal(w_p, w[pi])
    out_p = oracle.moe_layer(x[pi], ids_p, w_p, np.arange(L.T), L.H, L.I, qw)
    np.testing.assert_array_equal(out_p, out[pi])
    counts, offsets, perm, inv = oracle.permute(ids_p, L.E)
    flat = ids_p.ravel()
    for e in range(L.E):
        rows = perm[offsets[e]:offsets[e + 1]]
        assert np.all(flat[rows] == e) and np.all(np.diff(rows) > 0)


def test_layer_intermediates_against_numpy():
    L = synth.LAYERS[1]
    x = synth.activations(1)
    logits = synth.router_logits(1)
    ids, w = oracle.router(logits, L.k)
    _, _, q13, q2 = _tiny_weights()
    qw = oracle.QuantWeights(np.arange(L.E), *q13, *q2)
    toks = np.arange(L.T)
    out, dbg = oracle.moe_layer(x, ids, w, toks, L.H, L.I, qw, debug=True)
    xc, xs, xg = oracle.quantize_rows(x)
    xh = npref.dequant(xc, xs, xg)
    W13 = npref.dequant(q13[0], q13[1], q13[2][:, None, None], g_per_row=False)
    W2 = npref.dequant(q2[0], q2[1], q2[2][:, None, None], g_per_row=False)
    for t in toks:
        for j in range(L.k):
            e = ids[t, j]
            h = W13[e] @ xh[t]
            gate, up = h[:L.I], h[L.I:]
            act = (gate * expit(gate) * up).astype(np.float32)
            np.testing.assert_allclose(dbg["act"][t, j], act, rtol=2e-6,
                                       atol=1e-9 * np.abs(act).max())
            c2, S2, g2 = oracle.quantize_rows(dbg["act"][t, j][None])
            np.testing.assert_array_equal(dbg["c2"][t, j], c2[0])
            np.testing.assert_array_equal(dbg["S2"][t, j], S2[0])
            assert dbg["g2"][t, j] == g2[0]
            ah = npref.dequant(c2, S2, g2)[0]
            np.testing.assert_allclose(dbg["y"][t, j], W2[e] @ ah, rtol=1e-12,
                                       atol=1e-12 * np.abs(W2[e] @ ah).max())
    ref = np.einsum("tk,tkh->th", w, dbg["y"])
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-14)


def test_gate_up_projection_lossless_case():
    """On-grid activations and weights: act equals silu(x W1^T) * (x W3^T)
    computed from the unquantized float values."""
    rng = np.random.default_rng(12)
    H, I, E, k = 64, 32, 3, 2
    mags = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    def grid(shape):
        v = rng.choice(mags, shape) * rng.choice([-1.0, 1.0], shape)
        v.reshape(-1, 16)[:, 0] = 6.0   # every block amax 6: scale 448 everywhere
        return v
    x = grid((5, H)).astype(np.float32)
    w13 = grid((E, 2 * I, H)).astype(np.float32) * np.float32(0.125)
    w2 = grid((E, H, I)).astype(np.float32) * np.float32(0.25)
    q13 = oracle.quantize_groups(w13)
    q2 = oracle.quantize_groups(w2)
    xb = synth.bf16_bits(x)
    ids = np.array([[0, 1], [1, 2], [2, 0], [0, 2], [1, 0]], np.int32)
    w = np.full((5, k), 0.5)
    qw = oracle.QuantWeights(np.arange(E), *q13, *q2)
    _, dbg = oracle.moe_layer(xb, ids, w, np.arange(5), H, I, qw, debug=True)
    for t in range(5):
        for j in range(k):
            h = w13[ids[t, j]].astype(np.float64) @ x[t].astype(np.float64)
            want = (h[:I] * expit(h[:I]) * h[I:]).astype(np.float32)
            np.testing.assert_allclose(dbg["act"][t, j], want, rtol=2e-6)


def test_synth_weights_match_numpy_philox():
    sigma = 0.02
    seed, tag = synth.weight_key(2, 1)
    for e in (0, 3):
        n = 1000
        got = oracle.synth_weights(seed, tag, e, (n,), sigma)
        if e == 0:
            ctr = np.array([2**64 - 1] * 4, np.uint64)
        else:
            ctr = np.array([2**64 - 1, e - 1, 0, 0], np.uint64)
        # numpy's Philox increments the counter (with carry) before each block
        bg = np.random.Philox(counter=ctr, key=np.array([seed, tag], np.uint64))
        raw = bg.random_raw(n)
        fields = sum(((raw >> np.uint64(16 * q)) & np.uint64(0xFFFF)).astype(np.int64)
                     for q in range(4))
        want = (fields - 131070).astype(np.float32) * np.float32(synth.synth_scale_reference(sigma))
        np.testing.assert_array_equal(got, want)


def test_synth_weights_statistics():
    w = oracle.synth_weights(*synth.weight_key(5, 2), 7, (2000, 512), 0.01)
    assert abs(float(w.mean())) < 2e-5
    assert abs(float(w.std()) / 0.01 - 1) < 0.01
    assert float(np.abs(w).max()) <= 131070 * synth.synth_scale_reference(0.01) * (1 + 1e-6)
