"""GPU parity for w4a16_moe_layer (TurboFieldfare article, Gemma 4 26B-A4B
section and 量化和精度): the router, the top-k and the expert FFN from x.

By default one token takes three launches; switched on, it runs as a single
launch whose work items hand results to each other through device-scope words.
On either path its ids, weights and y must equal, bit for bit,
those of w4_moe_route followed by w4a16_moe_gemv (the same per-row arithmetic in
the same order), on consecutive calls sharing one workspace; at the Gemma shape
they are also checked against the oracle: the selection against a full sort of
the oracle's logits, y within 2e-3*S + 1e-5 of the oracle evaluating only the
selected experts. The give-up path of the launch's waits is forced from the host
(the expert selection is withheld and the poll limit is small): the call must
complete, report it, and leave the workspace usable."""
import numpy as np
import pytest
import torch

import bit_weight_only_quantize_amd as w4
import oracle
import synth
from gpu_util import TOL_ABS, TOL_REL, dev_bf16, dev_f32, tolerance_ratio

pytestmark = pytest.mark.gpu

_LAYERS = {}


@pytest.fixture
def single_launch():
    w4.moe_layer_set_single_launch(True)
    yield
    w4.moe_layer_set_single_launch(False)


def _stack(E, N, K, seed, name, scheme):
    q = w4.empty_quantized(scheme, N, K, num_experts=E)
    cs, ss, bs = [], [], []
    for e in range(E):
        W = synth.weights(N, K, 0.02, seed, f"{name}.{e}")
        c, s, b = oracle.quantize_pack(W, scheme)
        cs.append(c), ss.append(s), bs.append(b)
        w4.quantize_pack(dev_f32(W), scheme, out=q, expert=e)
    return (np.stack(cs), np.stack(ss), None if bs[0] is None else np.stack(bs)), q


def _single(N, K, seed, name, scheme):
    W = synth.weights(N, K, 0.02, seed, name)
    return oracle.quantize_pack(W, scheme), w4.quantize_pack(dev_f32(W), scheme)


def _layer(E, D, F, Fs, scheme, rscheme, tag):
    key = (E, D, F, Fs, scheme, rscheme, tag)
    if key not in _LAYERS:
        host, dev = {}, {}
        host["router"], dev["router"] = _single(E, D, 7, f"{tag}.router", rscheme)
        for nm, N, K in (("gate", F, D), ("up", F, D), ("down", D, F)):
            host[nm], dev[nm] = _stack(E, N, K, 7, f"{tag}.{nm}", scheme)
        if Fs:
            hs, ds = [], []
            for nm, N, K in (("sg", Fs, D), ("su", Fs, D), ("sd", D, Fs)):
                h, d = _single(N, K, 7, f"{tag}.{nm}", scheme)
                hs.append(h), ds.append(d)
            host["shared"], dev["shared"] = tuple(hs), ds
        else:
            host["shared"], dev["shared"] = None, None
        _LAYERS[key] = (host, dev)
    return _LAYERS[key]


def _reference_path(dev, x, k):
    """w4_moe_route then w4a16_moe_gemv: the launches the single launch replaces."""
    ids, wts, _ = w4.moe_route(dev["router"], x, top_k=k)
    y = w4.moe_gemv(dev["gate"], dev["up"], dev["down"], x, ids, wts, shared=dev["shared"])
    return y, ids, wts


@pytest.mark.parametrize("E,D,F,Fs,k,scheme,rscheme", [
    (128, 2048, 768, 2048, 8, "aff4_g64", "aff8_g64"),   # Gemma-4-26B-A4B-shaped
    (64, 2048, 256, 0, 4, "sym4_g128", "aff8_g64"),     # no shared expert
    (128, 4096, 512, 1024, 8, "aff4_g64", "aff8_g64"),  # D = 4096: two vectors per lane
    (16, 2048, 1024, 4096, 2, "sym4_g128", "aff8_g64"), # the longest expert and shared rows
    (37, 2048, 192, 64, 3, "aff4_g64", "aff8_g64"),     # ragged router tile (37 rows), short rows
])
def test_single_launch_layer_equals_route_then_moe_gemv(E, D, F, Fs, k, scheme, rscheme, single_launch):
    tag = f"layer.{E}.{D}.{F}.{Fs}.{scheme}"
    print(f"[moe_layer] E={E} D={D} F={F} Fs={Fs} k={k} {scheme} router {rscheme}", flush=True)
    _, dev = _layer(E, D, F, Fs, scheme, rscheme, tag)
    ws = w4.moe_layer_workspace(1, k, E, D, F, Fs)
    for seed in range(3):                         # consecutive calls on one workspace
        x = dev_bf16(synth.activations_bf16(1, D, seed, f"{tag}.x"))
        y, ids, wts = w4.moe_layer(dev["router"], dev["gate"], dev["up"], dev["down"], x, top_k=k,
                                   shared=dev["shared"], workspace=ws)
        assert w4.moe_layer_status(ws) == 0
        yr, idr, wr = _reference_path(dev, x, k)
        assert torch.equal(ids, idr), seed
        assert torch.equal(wts, wr), seed
        assert torch.equal(y, yr), seed


@pytest.mark.parametrize("single", [True, False])
def test_layer_matches_oracle_at_the_gemma_shape(single):
    E, D, F, Fs, k = 128, 2048, 768, 2048, 8
    tag = f"layer.{E}.{D}.{F}.{Fs}.aff4_g64"
    host, dev = _layer(E, D, F, Fs, "aff4_g64", "aff8_g64", tag)
    xh = synth.activations_bf16(1, D, 11, f"{tag}.xo")
    w4.moe_layer_set_single_launch(single)
    try:
        y, ids, wts = w4.moe_layer(dev["router"], dev["gate"], dev["up"], dev["down"], dev_bf16(xh),
                                   top_k=k, shared=dev["shared"])
        yr, idr, wr = _reference_path(dev, dev_bf16(xh), k)
    finally:
        w4.moe_layer_set_single_launch(False)
    assert torch.equal(y, yr) and torch.equal(ids, idr) and torch.equal(wts, wr)
    y, ids, wts = y.cpu().numpy(), ids.cpu().numpy(), wts.cpu().numpy()
    lref, rids, rp, margin = oracle.route(xh, *host["router"], top_k=k)
    _, S = oracle.gemv_reference(*host["router"], "aff8_g64", xh)
    tol_l = float((TOL_REL * S + TOL_ABS).max())
    assert len(set(ids[0].tolist())) == k
    if margin[0] > 2 * tol_l:
        assert list(ids[0]) == list(rids[0])
        assert np.all(np.abs(wts[0] - rp[0]) <= rp[0] * 2.5 * tol_l + 1e-7)
    yr, Sr = oracle.moe_sparse(xh, ids, wts.astype(np.float64), host["gate"], host["up"], host["down"],
                               host["shared"], scheme="aff4_g64")
    r = tolerance_ratio(y, yr, Sr)
    assert r <= 1.0, f"worst error {r:.3f} x tolerance"


def test_several_tokens_and_other_routers_take_the_launch_sequence():
    E, D, F, Fs, k = 128, 2048, 768, 2048, 8
    tag = f"layer.{E}.{D}.{F}.{Fs}.aff4_g64"
    _, dev = _layer(E, D, F, Fs, "aff4_g64", "aff8_g64", tag)
    for M in (32, 3):
        x = dev_bf16(synth.activations_bf16(M, D, 5, f"{tag}.xm{M}"))
        y, ids, wts = w4.moe_layer(dev["router"], dev["gate"], dev["up"], dev["down"], x, top_k=k,
                                   shared=dev["shared"])
        yr, idr, wr = _reference_path(dev, x, k)
        assert torch.equal(ids, idr) and torch.equal(wts, wr) and torch.equal(y, yr)
    # a 4-bit router at one token: the launch sequence, same results
    _, dev4 = _layer(64, 2048, 256, 0, "sym4_g128", "aff4_g64", "layer.r4")
    x = dev_bf16(synth.activations_bf16(1, 2048, 6, "layer.r4.x"))
    y, ids, wts = w4.moe_layer(dev4["router"], dev4["gate"], dev4["up"], dev4["down"], x, top_k=4)
    yr, idr, wr = _reference_path(dev4, x, 4)
    assert torch.equal(ids, idr) and torch.equal(y, yr)


def test_withheld_selection_gives_up_and_the_workspace_recovers(single_launch):
    E, D, F, Fs, k = 64, 2048, 256, 0, 4
    tag = f"layer.{E}.{D}.{F}.{Fs}.sym4_g128"
    _, dev = _layer(E, D, F, Fs, "sym4_g128", "aff8_g64", tag)
    ws = w4.moe_layer_workspace(1, k, E, D, F, Fs)
    x = dev_bf16(synth.activations_bf16(1, D, 0, f"{tag}.x"))
    try:
        w4.moe_layer_set_wait(max_polls=2000, withhold=True)
        w4.moe_layer(dev["router"], dev["gate"], dev["up"], dev["down"], x, top_k=k, workspace=ws)
        status = w4.moe_layer_status(ws)            # the launch completed (synchronized)
    finally:
        w4.moe_layer_set_wait(0, False)
    assert status & w4.MOE_LAYER_GAVE_UP_IDS
    y, ids, wts = w4.moe_layer(dev["router"], dev["gate"], dev["up"], dev["down"], x, top_k=k, workspace=ws)
    assert w4.moe_layer_status(ws) == 0
    yr, idr, _ = _reference_path(dev, x, k)
    assert torch.equal(ids, idr) and torch.equal(y, yr)
