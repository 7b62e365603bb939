"""GPU parity of the INT4 KV cache ([Shimmy] §3.2): codes and scales bit-exact against
the oracle's codec, the fused-dequant scores and weighted sums within
2e-3 * sum|a||b| + 1e-5 of the oracle's fp64 products."""
import numpy as np
import pytest
import torch

import bit_weight_only_quantize_amd as w4
import oracle
import synth
from gpu_util import tolerance_ratio

pytestmark = pytest.mark.gpu
D = 128


def _vectors(shape, name, seed=0):
    """Seeded fp32 head vectors with a spread of magnitudes, plus the special cases."""
    x = synth.normal_f32(shape, 1.0, seed, name)
    mag = synth.normal_f32(shape[:-1] + (1,), 1.0, seed, name + ".mag")
    x = (x * np.exp2(np.round(mag * 3)).astype(np.float32)).astype(np.float32)
    flat = x.reshape(-1, D)
    if flat.shape[0] >= 3:
        flat[0] = 0.0                                   # zero vector: scale 0, nibbles 8
        flat[1] = 0.0
        flat[1, :11] = [7.5, 0.5, -0.5, 1.5, -1.5, 2.5, -2.5, 3.5, -3.5, 6.5, -6.5]  # exact halves
        flat[2] = -3.0                                  # constant vector
    return x


def _cache(x_tkd):
    """Oracle cache of vectors x [Hkv][T][D] -> device codes/scales (inputs, not results)."""
    c, s = oracle.kv_quantize(x_tkd)
    return c, s, torch.from_numpy(c).cuda(), torch.from_numpy(s).cuda()


@pytest.mark.parametrize("n,Hkv,pos,T_max", [(1, 8, 0, 16), (5, 4, 3, 11), (64, 32, 100, 200), (1, 1, 9, 10)])
def test_kv_quantize_bit_exact(n, Hkv, pos, T_max):
    print(f"[kv_quantize] n={n} Hkv={Hkv} pos={pos} T_max={T_max}", flush=True)
    x = _vectors((n, Hkv, D), f"kvq.{n}.{Hkv}")
    codes, scales = w4.kv_cache(Hkv, T_max)
    codes.fill_(0x5A)
    scales.fill_(-1.0)
    w4.kv_quantize(torch.from_numpy(x).cuda(), codes, scales, pos)
    c_ref, s_ref = oracle.kv_quantize(np.ascontiguousarray(x.transpose(1, 0, 2)))   # [Hkv][n][D]
    c, s = codes.cpu().numpy(), scales.cpu().numpy()
    assert np.array_equal(c[:, pos:pos + n], c_ref), "codes differ"
    assert np.array_equal(s[:, pos:pos + n].view(np.uint32), s_ref.view(np.uint32)), "scales differ"
    # positions outside [pos, pos + n) untouched
    assert np.all(c[:, :pos] == 0x5A) and np.all(c[:, pos + n:] == 0x5A)
    assert np.all(s[:, :pos] == -1.0) and np.all(s[:, pos + n:] == -1.0)


@pytest.mark.parametrize("Hq,Hkv,T,T_max", [
    (4, 4, 128, 128),       # one chunk, no grouping
    (32, 8, 1000, 1024),    # query heads in groups of 4; ragged last chunk
    (8, 2, 1, 5),           # one position
    (6, 3, 300, 300),
    (32, 32, 8192, 8192),   # a 7B-shaped layer's cache at 8K context, as the bench runs it
])
def test_kv_scores_and_weighted_sum_match_oracle(Hq, Hkv, T, T_max):
    print(f"[kv_products] Hq={Hq} Hkv={Hkv} T={T} T_max={T_max}", flush=True)
    name = f"kv.{Hq}.{Hkv}.{T}"
    K = _vectors((Hkv, T_max, D), name + ".K")
    V = _vectors((Hkv, T_max, D), name + ".V", seed=1)
    kc, ks, kcd, ksd = _cache(K)
    vc, vs, vcd, vsd = _cache(V)
    q = synth.normal_f32((Hq, D), 1.0, 0, name + ".q")
    qd = torch.from_numpy(q).cuda()
    sc = w4.kv_scores(qd, kcd, ksd, T).cpu().numpy()
    y, S = oracle.kv_scores(q, kc[:, :T], ks[:, :T])
    r = tolerance_ratio(sc, y, S)
    assert r <= 1.0, f"scores: worst error {r:.3f} x tolerance"
    # weights: the softmax of the scaled scores (fp32, from the GPU scores)
    lg = torch.from_numpy(sc).cuda() / np.float32(np.sqrt(D))
    p = torch.softmax(lg, dim=1).contiguous()
    ws = torch.full((w4.kv_weighted_sum_workspace_bytes(Hq, T),), 0xFF, dtype=torch.uint8, device="cuda")
    out = w4.kv_weighted_sum(p, vcd, vsd, workspace=ws).cpu().numpy()
    yo, So = oracle.kv_weighted_sum(p.cpu().numpy(), vc[:, :T], vs[:, :T])
    r = tolerance_ratio(out, yo, So)
    assert r <= 1.0, f"weighted sum: worst error {r:.3f} x tolerance"
    out2 = w4.kv_weighted_sum(p, vcd, vsd, workspace=ws).cpu().numpy()
    sc2 = w4.kv_scores(qd, kcd, ksd, T).cpu().numpy()
    assert np.array_equal(out, out2) and np.array_equal(sc, sc2)      # deterministic


def test_kv_append_equals_two_quantize_calls():
    n, Hkv, pos, T_max = 3, 8, 5, 12
    k = _vectors((n, Hkv, D), "kva.k")
    v = _vectors((n, Hkv, D), "kva.v", seed=1)
    kd, vd = torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda()
    kc, vc = w4.kv_cache(Hkv, T_max), w4.kv_cache(Hkv, T_max)
    kc2, vc2 = w4.kv_cache(Hkv, T_max), w4.kv_cache(Hkv, T_max)
    for t in kc + vc + kc2 + vc2:
        t.zero_()
    w4.kv_append(kd, vd, kc, vc, pos)
    w4.kv_quantize(kd, kc2[0], kc2[1], pos)
    w4.kv_quantize(vd, vc2[0], vc2[1], pos)
    for a, b in zip(kc + vc, kc2 + vc2):
        assert torch.equal(a, b)
    c_ref, s_ref = oracle.kv_quantize(np.ascontiguousarray(v.transpose(1, 0, 2)))
    assert np.array_equal(vc[0].cpu().numpy()[:, pos:pos + n], c_ref)
    assert np.array_equal(vc[1].cpu().numpy()[:, pos:pos + n].view(np.uint32), s_ref.view(np.uint32))


@pytest.mark.parametrize("Hq,Hkv,pos,n,T_max", [
    (32, 32, 8192, 1, 8193),   # a 7B-shaped layer's decode step at 8K context, as the bench runs it
    (32, 8, 999, 1, 1024),     # query heads in groups of 4, ragged last chunk
    (8, 2, 0, 1, 5),           # empty cache: the new position is all there is
    (4, 4, 0, 16, 16),         # sixteen new positions, nothing cached
    (6, 3, 120, 16, 300),      # new positions across a chunk boundary
    (6, 3, 128, 1, 300),       # the new position opens a chunk
    (4, 2, 29, 5, 64),         # across a 16-position step
    (4, 2, 10, 17, 64),        # more than sixteen: the append is a launch of its own
    (4, 2, 100, 40, 200),
])
def test_kv_append_fused_into_products(Hq, Hkv, pos, n, T_max):
    """w4_kv_scores_append / w4_kv_weighted_sum_append against the append launch
    followed by the plain products: caches and outputs bit for bit, and the
    outputs against the oracle over the whole cache."""
    print(f"[kv_fused_append] Hq={Hq} Hkv={Hkv} pos={pos} n={n} T_max={T_max}", flush=True)
    name = f"kvf.{Hq}.{Hkv}.{pos}.{n}"
    T = pos + n
    K = _vectors((Hkv, T_max, D), name + ".K")
    V = _vectors((Hkv, T_max, D), name + ".V", seed=1)
    k_new = np.ascontiguousarray(K[:, pos:T].transpose(1, 0, 2))      # [n][Hkv][D]
    v_new = np.ascontiguousarray(V[:, pos:T].transpose(1, 0, 2))
    kc, ks = oracle.kv_quantize(K)
    vc, vs = oracle.kv_quantize(V)

    def old_cache(c, s):
        """The cache with positions < pos filled (from the oracle), the rest stale."""
        cd = torch.full((Hkv, T_max, D // 2), 0x5A, dtype=torch.uint8, device="cuda")
        sd = torch.full((Hkv, T_max), float("nan"), dtype=torch.float32, device="cuda")
        cd[:, :pos] = torch.from_numpy(c[:, :pos]).cuda()
        sd[:, :pos] = torch.from_numpy(s[:, :pos]).cuda()
        return cd, sd

    q = torch.from_numpy(synth.normal_f32((Hq, D), 1.0, 0, name + ".q")).cuda()
    knd, vnd = torch.from_numpy(k_new).cuda(), torch.from_numpy(v_new).cuda()
    # the launch sequence
    ka = old_cache(kc, ks)
    w4.kv_quantize(knd, ka[0], ka[1], pos)
    sc_a = w4.kv_scores(q, ka[0], ka[1], T)
    p = torch.softmax(sc_a / np.float32(np.sqrt(D)), dim=1).contiguous()
    va = old_cache(vc, vs)
    w4.kv_quantize(vnd, va[0], va[1], pos)
    out_a = w4.kv_weighted_sum(p, va[0], va[1])
    # fused
    kb = old_cache(kc, ks)
    sc_b = w4.kv_scores_append(q, knd, kb[0], kb[1], pos)
    vb = old_cache(vc, vs)
    ws = torch.full((w4.kv_weighted_sum_workspace_bytes(Hq, T),), 0xFF, dtype=torch.uint8, device="cuda")
    out_b = w4.kv_weighted_sum_append(p, vnd, vb[0], vb[1], pos, workspace=ws)
    torch.cuda.synchronize()
    for a, b in ((ka, kb), (va, vb)):
        assert torch.equal(a[0], b[0]), "codes differ"
        assert torch.equal(a[1][:, :T].view(torch.int32), b[1][:, :T].view(torch.int32)), "scales differ"
        assert torch.isnan(b[1][:, T:]).all(), "positions past pos + n written"
    assert torch.equal(sc_a.view(torch.int32), sc_b.view(torch.int32)), "scores differ"
    assert torch.equal(out_a.view(torch.int32), out_b.view(torch.int32)), "weighted sums differ"
    # the new positions' codes against the oracle's codec
    assert np.array_equal(kb[0][:, pos:T].cpu().numpy(), kc[:, pos:T])
    assert np.array_equal(vb[1][:, pos:T].cpu().numpy().view(np.uint32), vs[:, pos:T].view(np.uint32))
    y, S = oracle.kv_scores(q.cpu().numpy(), kc[:, :T], ks[:, :T])
    assert tolerance_ratio(sc_b.cpu().numpy(), y, S) <= 1.0
    yo, So = oracle.kv_weighted_sum(p.cpu().numpy(), vc[:, :T], vs[:, :T])
    assert tolerance_ratio(out_b.cpu().numpy(), yo, So) <= 1.0


def test_kv_quantize_then_read_back():
    """The device codec feeds the device products: quantize K on the GPU, score
    one-hot queries, and read the dequantized cache back element by element."""
    Hkv, T = 2, 40
    x = _vectors((T, Hkv, D), "kv.rt")
    codes, scales = w4.kv_cache(Hkv, T)
    w4.kv_quantize(torch.from_numpy(x).cuda(), codes, scales, 0)
    c_ref, s_ref = oracle.kv_quantize(np.ascontiguousarray(x.transpose(1, 0, 2)))
    Kd = oracle.kv_dequant(c_ref, s_ref)                        # [Hkv][T][D]
    for i in (0, 1, 63, 127):
        q = np.zeros((Hkv, D), dtype=np.float32)
        q[:, i] = 1
        sc = w4.kv_scores(torch.from_numpy(q).cuda(), codes, scales, T).cpu().numpy()
        # (nibble - 8) exactly, times the scale with one fp32 rounding
        assert np.array_equal(sc, Kd[:, :, i].astype(np.float32))


def test_kv_weighted_sum_rejects_small_workspace():
    codes, scales = w4.kv_cache(2, 64)
    p = torch.zeros((4, 64), dtype=torch.float32, device="cuda")
    need = w4.kv_weighted_sum_workspace_bytes(4, 64)
    with pytest.raises(w4.W4Error) as e:
        w4.kv_weighted_sum(p, codes, scales, workspace=torch.empty(need - 16, dtype=torch.uint8, device="cuda"))
    assert e.value.code == -5
