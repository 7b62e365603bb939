"""GPU parity for the MoE path (TurboFieldfare article, Gemma 4 26B-A4B section
and 量化和精度): router logits within the GEMV tolerance, top-k identical to the
oracle's wherever the oracle's 8th/9th logit margin exceeds the logit tolerance,
softmax weights within the propagated tolerance, and the expert FFN output
within 2e-3·sum|w||h| + 1e-5 against the oracle evaluating only the selected
experts."""
import numpy as np
import pytest
import torch

import bit_weight_only_quantize_amd as w4
import oracle
import synth
from gpu_util import TOL_ABS, TOL_REL, dev_bf16, dev_f32, tolerance_ratio

pytestmark = pytest.mark.gpu


def _router(E, D, seed, name):
    W = synth.weights(E, D, 0.02, seed, name)
    c, s, b = oracle.quantize_pack(W, "aff8_g64")
    return W, (c, s, b), w4.quantize_pack(dev_f32(W), "aff8_g64")


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


@pytest.mark.parametrize("M", [1, 32])
def test_route_matches_oracle(M):
    E, D = 128, 2048
    print(f"[route] E={E} D={D} M={M}", flush=True)
    _, (c, s, b), qr = _router(E, D, 0, "moe.router")
    x = synth.activations_bf16(M, D, 0, "moe.x")
    ids, wts, logits = w4.moe_route(qr, dev_bf16(x), top_k=8)
    ids, wts, logits = ids.cpu().numpy(), wts.cpu().numpy(), logits.cpu().numpy()
    lref, S = oracle.gemv_reference(c, s, b, "aff8_g64", x)
    assert tolerance_ratio(logits, lref, S) <= 1.0
    _, rids, rp, margin = oracle.route(x, c, s, b, top_k=8)
    tol_l = (TOL_REL * S + TOL_ABS).max(axis=1)
    for m in range(M):
        assert len(set(ids[m].tolist())) == 8 and ids[m].min() >= 0 and ids[m].max() < E, m
        if margin[m] > 2 * tol_l[m]:
            assert list(ids[m]) == list(rids[m]), m
        else:  # a near tie: the GPU's set must still be a valid top-8 of the oracle's logits
            kth = np.sort(lref[m])[::-1][7]
            assert np.all(lref[m][ids[m]] >= kth - 2 * tol_l[m])
        # weights: softmax of logits that are each within tol_l -> relative error <= 2 tol_l
        sel = [list(ids[m]).index(e) for e in rids[m]] if list(ids[m]) == list(rids[m]) else None
        if sel is not None:
            assert np.all(np.abs(wts[m] - rp[m]) <= rp[m] * (2.5 * tol_l[m]) + 1e-7)
        assert np.all(np.diff(wts[m]) <= 0) and wts[m].sum() <= 1.0 + 1e-6


def test_route_ties_go_to_lower_index():
    E, D = 64, 2048
    W = np.tile(synth.weights(1, D, 0.02, 1, "tie"), (E, 1))
    q = w4.quantize_pack(dev_f32(W), "aff8_g64")
    x = dev_bf16(synth.activations_bf16(3, D, 1, "tie.x"))
    ids, wts, _ = w4.moe_route(q, x, top_k=5)
    assert ids.cpu().tolist() == [[0, 1, 2, 3, 4]] * 3
    assert torch.allclose(wts, torch.full_like(wts, 1.0 / E))


def _moe_case(M, E, D, F, Fs, k, scheme, seed, tag, ids=None, p=None):
    print(f"[moe] {tag} M={M} E={E} D={D} F={F} Fs={Fs} k={k} {scheme}", flush=True)
    gate_h, gate = _stack(E, F, D, seed, f"{tag}.gate", scheme)
    up_h, up = _stack(E, F, D, seed, f"{tag}.up", scheme)
    down_h, down = _stack(E, D, F, seed, f"{tag}.down", scheme)
    shared_h = shared = None
    if Fs:
        trip = [_single(n, kk, seed, f"{tag}.s{nm}", scheme) for n, kk, nm in ((Fs, D, "g"), (Fs, D, "u"), (D, Fs, "d"))]
        shared_h = tuple(t[0] for t in trip)
        shared = [t[1] for t in trip]
    x = synth.activations_bf16(M, D, seed, f"{tag}.x")
    if ids is None:
        _, (rc, rs, rb), _ = _router(E, D, seed, f"{tag}.router")
        _, ids, p, _ = oracle.route(x, rc, rs, rb, top_k=k)
    p32 = np.asarray(p, dtype=np.float32)
    y = w4.moe_gemv(gate, up, down, dev_bf16(x), torch.from_numpy(np.ascontiguousarray(ids, np.int32)).cuda(),
                    torch.from_numpy(p32).cuda(), shared=shared).cpu().numpy()
    yr, S = oracle.moe_sparse(x, ids, p32.astype(np.float64), gate_h, up_h, down_h, shared_h, scheme)
    r = tolerance_ratio(y, yr, S)
    assert r <= 1.0, f"worst error {r:.3f} x tolerance"
    return y


@pytest.mark.parametrize("M", [1, 32])
def test_moe_gemma_shaped_layer(M):
    """128 experts (gate/up 768x2048, down 2048x768, aff4 g64), top-8, shared FFN 2048."""
    _moe_case(M, 128, 2048, 768, 2048, 8, "aff4_g64", 0, "gemma")


@pytest.mark.parametrize("M,E,D,F,Fs,k", [
    (256, 64, 512, 256, 512, 8),    # the most tokens: 2048 pairs, experts with > 8 pairs in several descriptors
    (256, 32, 256, 128, 0, 32),     # the most slots: 8192 pairs (the bucketing limit), no shared expert
    (64, 128, 2048, 768, 2048, 8),  # Gemma-shaped, twice the bench's decode batch
])
def test_moe_largest_batches(M, E, D, F, Fs, k):
    _moe_case(M, E, D, F, Fs, k, "aff4_g64", 5, f"big.{M}.{E}.{k}")


@pytest.mark.parametrize("scheme", ["sym4_g128", "aff4_g64"])
def test_moe_small_ragged_and_edge_ids(scheme):
    E, D, F, M, k = 16, 256, 384, 5, 3
    ids = np.array([[3, 3, 7], [0, 15, -1], [7, 3, 0], [99, 2, 2], [5, 6, 7]], dtype=np.int32)
    p = np.array([[0.5, 0.25, 0.125], [0.3, 0.2, 0.9], [0.1, 0.1, 0.1], [1.0, 0.4, 0.4], [0.2, 0.3, 0.5]])
    _moe_case(M, E, D, F, 256, k, scheme, 3, f"edge.{scheme}", ids=ids, p=p)
    _moe_case(M, E, D, F, 0, k, scheme, 4, f"noshared.{scheme}", ids=ids, p=p)


@pytest.mark.parametrize("scheme", ["sym4_g128", "aff4_g64"])
@pytest.mark.parametrize("M", [20, 32])
def test_moe_expert_with_more_than_16_pairs(scheme, M):
    """Every token sends slot 0 to expert 1: its M pairs span several work
    descriptors (at most 8 pairs each; the routed passes stage one
    descriptor's activation rows per workgroup)."""
    E, D, F, k = 8, 256, 384, 2
    ids = np.stack([np.ones(M, np.int32), (np.arange(M) * 3 % E).astype(np.int32)], axis=1)
    p = np.stack([np.full(M, 0.75), np.full(M, 0.25)], axis=1)
    _moe_case(M, E, D, F, 256, k, scheme, 7, f"split.{scheme}.{M}", ids=ids, p=p)


def test_moe_end_to_end_route_then_experts_and_determinism():
    M, E, D, F, Fs = 4, 128, 2048, 768, 2048
    _, (rc, rs, rb), qr = _router(E, D, 5, "e2e.router")
    gate_h, gate = _stack(E, F, D, 5, "e2e.gate", "aff4_g64")
    up_h, up = _stack(E, F, D, 5, "e2e.up", "aff4_g64")
    down_h, down = _stack(E, D, F, 5, "e2e.down", "aff4_g64")
    trip = [_single(n, kk, 5, f"e2e.s{nm}", "aff4_g64") for n, kk, nm in ((Fs, D, "g"), (Fs, D, "u"), (D, Fs, "d"))]
    x = synth.activations_bf16(M, D, 5, "e2e.x")
    xd = dev_bf16(x)
    ids, wts, _ = w4.moe_route(qr, xd, top_k=8)
    y1 = w4.moe_gemv(gate, up, down, xd, ids, wts, shared=[t[1] for t in trip])
    y2 = w4.moe_gemv(gate, up, down, xd, ids, wts, shared=[t[1] for t in trip])
    assert torch.equal(y1, y2)
    _, rids, rp, margin = oracle.route(x, rc, rs, rb, top_k=8)
    assert np.array_equal(ids.cpu().numpy(), rids), "no near ties expected for this seed"
    yr, S = oracle.moe_sparse(x, rids, rp, gate_h, up_h, down_h, tuple(t[0] for t in trip))
    # weights differ from the oracle's by the softmax tolerance; add that term to the bound
    pw = np.abs(wts.cpu().numpy() - rp).sum(axis=1, keepdims=True)
    assert np.all(np.abs(y1.cpu().numpy() - yr) <= TOL_REL * S + TOL_ABS + pw * np.abs(yr).max())


def test_moe_rejects_bad_arguments():
    _, gate = _stack(4, 64, 128, 6, "bad.gate", "aff4_g64")
    _, up = _stack(4, 64, 128, 6, "bad.up", "aff4_g64")
    _, down = _stack(4, 128, 64, 6, "bad.down", "aff4_g64")
    x = dev_bf16(synth.activations_bf16(2, 128, 6, "bad.x"))
    ids = torch.zeros((2, 2), dtype=torch.int32, device="cuda")
    wts = torch.ones((2, 2), dtype=torch.float32, device="cuda")
    with pytest.raises(w4.W4Error):
        w4.moe_gemv(gate, up, gate, x, ids, wts)                   # down has the wrong shape
    with pytest.raises(w4.W4Error) as ei:
        w4.moe_gemv(gate, up, down, x, ids, wts, workspace=torch.empty(16, dtype=torch.uint8, device="cuda"))
    assert ei.value.code == -5


@pytest.mark.parametrize("scheme", ["aff4_g64", "sym4_g128"])
@pytest.mark.parametrize("k,ids_row,shared", [
    (8, [5, 9, 5, -1, 31, 0, 200, 17], True),     # duplicate expert, invalid ids
    (3, [2, 30, 7], True),                        # fewer than 8 slots
    (8, [1, 2, 3, 4, 5, 6, 7, 8], False),         # no shared expert
])
def test_moe_single_token_fast_path_edges(scheme, k, ids_row, shared):
    E, D, F, Fs = 32, 2048, 768, 2048
    ids = np.array([ids_row], dtype=np.int32)
    p = np.linspace(0.3, 0.05, k)[None, :]
    _moe_case(1, E, D, F, Fs if shared else 0, k, scheme, 7, f"m1.{scheme}.{k}.{int(shared)}", ids=ids, p=p)


def _dev_stack(E, N, K, seed, name, scheme):
    q = w4.empty_quantized(scheme, N, K, num_experts=E)
    for e in range(E):
        w4.quantize_pack(dev_f32(synth.weights(N, K, 0.02, seed, f"{name}.{e}")), scheme, out=q, expert=e)
    return q


@pytest.mark.parametrize("M,E,F,Fs,k", [
    (1, 128, 768, 2048, 8),   # one token, E <= 128: selection inside the gate/up pass
    (1, 64, 256, 0, 3),       # same path, fewer slots, no shared expert
    (1, 256, 256, 512, 8),    # one token, E > 128: a top-k launch first
    (2, 128, 256, 512, 8),    # several tokens: top-k launch, then the bucketed passes
    (32, 128, 768, 2048, 8),  # the decode batch of the MoE bench
    (20, 256, 256, 512, 8),   # > 16 tokens (two per wavefront), E > 128
])
def test_moe_gemv_logits_equals_route_then_gemv(M, E, F, Fs, k):
    """w4a16_moe_gemv_logits from router logits gives, bit for bit, the ids and
    weights w4_moe_route selects and the output w4a16_moe_gemv computes with them."""
    D, scheme, seed = 2048, "aff4_g64", 11
    tag = f"logits.{M}.{E}.{F}.{Fs}.{k}"
    qr = w4.quantize_pack(dev_f32(synth.weights(E, D, 0.02, seed, f"{tag}.router")), "aff8_g64")
    gate = _dev_stack(E, F, D, seed, f"{tag}.gate", scheme)
    up = _dev_stack(E, F, D, seed, f"{tag}.up", scheme)
    down = _dev_stack(E, D, F, seed, f"{tag}.down", scheme)
    shared = None
    if Fs:
        shared = [w4.quantize_pack(dev_f32(synth.weights(n, kk, 0.02, seed, f"{tag}.s{nm}")), scheme)
                  for n, kk, nm in ((Fs, D, "g"), (Fs, D, "u"), (D, Fs, "d"))]
    x = dev_bf16(synth.activations_bf16(M, D, seed, f"{tag}.x"))
    ids_r, w_r, logits = w4.moe_route(qr, x, top_k=k)
    y_r = w4.moe_gemv(gate, up, down, x, ids_r, w_r, shared=shared)
    for _ in range(2):  # the second call also checks nothing is left over from the first
        y, ids, w = w4.moe_gemv_logits(gate, up, down, x, logits, top_k=k, shared=shared)
        torch.cuda.synchronize()
        assert torch.equal(ids, ids_r)
        assert torch.equal(w, w_r)
        assert torch.equal(y, y_r)


@pytest.mark.parametrize("E,k", [(128, 8), (100, 8), (9, 8), (8, 8)])
def test_single_token_selection_ties_signed_zeros_and_minus_inf(E, k):
    """The selection inside the one-token gate/up pass (ranks over the
    workgroup) and the top-k launch of the several-token path agree bit for
    bit on logits with exact ties, +0 against -0 and -inf entries, and both
    follow the stable-sort rule: largest first, equal logits (-0 equal to +0)
    in expert order."""
    D, F, scheme, seed = 2048, 256, "aff4_g64", 5
    tag = f"ties.{E}.{k}"
    print(f"[moe] {tag}", flush=True)
    gate = _dev_stack(E, F, D, seed, f"{tag}.gate", scheme)
    up = _dev_stack(E, F, D, seed, f"{tag}.up", scheme)
    down = _dev_stack(E, D, F, seed, f"{tag}.down", scheme)
    rng = np.random.default_rng(17)
    vals = np.array([0.75, 0.5, 0.0, -0.0, -1.0, -np.inf], np.float32)
    row = vals[rng.integers(0, len(vals), E)]
    row[rng.integers(0, E)] = 0.75  # at least one finite logit
    x = dev_bf16(synth.activations_bf16(2, D, seed, f"{tag}.x"))
    ref_ids = sorted(range(E), key=lambda e: (-float(row[e]), e))[:k]
    one = torch.from_numpy(row[None, :].copy()).cuda()
    two = torch.from_numpy(np.stack([row, row])).cuda()
    y1, ids1, w1 = w4.moe_gemv_logits(gate, up, down, x[:1], one, top_k=k)
    y2, ids2, w2 = w4.moe_gemv_logits(gate, up, down, x, two, top_k=k)
    torch.cuda.synchronize()
    assert ids1.cpu().tolist() == [ref_ids]
    assert torch.equal(ids1[0], ids2[0]) and torch.equal(ids2[0], ids2[1])
    assert torch.equal(w1[0], w2[0])
    lr = row.astype(np.float64)
    p = np.exp(lr - lr.max()) / np.exp(lr - lr.max()).sum()
    assert np.allclose(w1[0].cpu().numpy(), p[ref_ids], rtol=1e-6, atol=0)
