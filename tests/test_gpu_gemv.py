"""GPU parity: the fused-dequant decode GEMV / skinny GEMM against the oracle's
fp64 product, per element within 2e-3·sum|w||x| + 1e-5 (fp32 accumulation of
bf16 activations), and bit-exact on dyadic toys where fp32 is exact."""
from fractions import Fraction

import numpy as np
import pytest
import torch

import bit_weight_only_quantize_amd as w4
import oracle
import synth
from gpu_util import dev_bf16, dev_f32, tolerance_ratio, upload

pytestmark = pytest.mark.gpu


def _run(scheme, N, K, M, name, rows=None, quantize_on_gpu=True):
    print(f"[gemv] {name} scheme={scheme} N={N} K={K} M={M}", flush=True)
    W = synth.weights(N, K, 0.02, seed=0, name=name)
    x = synth.activations_bf16(M, K, seed=0, name=name + ".x")
    c, s, b = oracle.quantize_pack(W, scheme)
    q = w4.quantize_pack(dev_f32(W), scheme) if quantize_on_gpu else upload(c, s, b, scheme)
    y = w4.gemv(q, dev_bf16(x)).cpu().numpy()
    yr, S = oracle.gemv_reference(c, s, b, scheme, x, rows=rows)
    if rows is not None:
        y = y[:, rows]
    r = tolerance_ratio(y, yr, S)
    assert r <= 1.0, f"worst error is {r:.3f} x tolerance"
    return r


@pytest.mark.parametrize("scheme,N,K,M", [
    ("aff4_g64", 1024, 1024, 1),      # single-GEMV workload
    ("sym4_g128", 1000, 4096, 1),
    ("sym4_g128", 1000, 4096, 2),
    ("sym4_g128", 1000, 4096, 3),
    ("sym4_g128", 1000, 4096, 5),
    ("aff4_g64", 333, 768, 1),
    ("aff4_g64", 333, 768, 4),
    ("sym4_g128", 257, 11008, 1),
    ("aff8_g64", 128, 2048, 1),
    ("aff8_g64", 130, 2048, 7),
    ("aff4_g64", 64, 64, 1),
    ("aff4_g64", 7, 192, 2),
    ("sym4_g128", 1, 128, 1),
    ("aff4_g64", 520, 13824, 2),
    ("sym4_g128", 1000, 4096, 16),    # skinny MFMA path: full token tile, ragged rows
    ("aff4_g64", 333, 768, 13),
    ("aff4_g64", 17, 64, 6),          # one group: a half step, activations in LDS
    ("sym4_g128", 31, 128, 11),
    ("sym4_g128", 12370, 512, 3),     # > 256 row tiles: 4 per workgroup, ragged last workgroup
    ("aff4_g64", 600, 13888, 8),      # activations staged in chunks; odd group count
    ("aff8_g64", 128, 2048, 32),      # router shape, several tokens: token tiles split over workgroups
    ("sym4_g128", 40, 4096, 37),      # > 16 tokens (VALU multi-token path), ragged token split
    ("aff8_g64", 96, 13824, 1),       # one token, long rows: 14 code vectors per lane
    ("aff4_g64", 50, 20480, 1),       # 11 per lane, ragged last vector column
    ("sym4_g128", 70, 28672, 1),      # the longest rows (14 per lane)
    ("aff8_g64", 333, 4160, 16),      # 8-bit codes on the matrix cores: odd group count, ragged rows
    ("aff8_g64", 50, 64, 3),          # one group
    ("aff8_g64", 12370, 512, 4),      # > 256 row tiles
    ("aff4_g64", 100, 1024, 64),      # the most tokens the GEMV takes
])
def test_gemv_matches_oracle(scheme, N, K, M):
    _run(scheme, N, K, M, f"small.{scheme}.{N}x{K}")


@pytest.mark.parametrize("scheme,N,K,M", [
    ("sym4_g128", 300, 11008, 16),    # K in parts, ragged rows
    ("aff4_g64", 600, 13888, 8),      # odd group count: the last part ends in a half step
    ("aff4_g64", 200, 13824, 16),
    ("sym4_g128", 40, 28672, 16),     # the most parts (8)
    ("sym4_g128", 77, 11008, 9),      # ragged token tile (9 of 16), ragged rows
    ("sym4_g128", 4096, 11008, 16),   # the 7B down projection as the decode stack runs it
    ("aff4_g64", 5120, 13824, 8),     # the 13B down projection
    ("aff8_g64", 300, 11008, 16),     # 8-bit codes
])
def test_gemv_ws_k_parts_match_oracle(scheme, N, K, M):
    name = f"ws.{scheme}.{N}x{K}"
    print(f"[gemv_ws] {name} M={M}", flush=True)
    W = synth.weights(N, K, 0.02, seed=0, name=name)
    x = synth.activations_bf16(M, K, seed=0, name=name + ".x")
    c, s, b = oracle.quantize_pack(W, scheme)
    q = upload(c, s, b, scheme)
    need = w4.gemv_workspace_bytes(q, M)
    assert need > 0 and need % (M * N * 4) == 0 and 2 <= need // (M * N * 4) <= 8
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")   # NaN bits: contents do not matter
    xd = dev_bf16(x)
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    w4.gemv_ws_into(q, xd, y, ws)
    yr, S = oracle.gemv_reference(c, s, b, scheme, x)
    r = tolerance_ratio(y.cpu().numpy(), yr, S)
    assert r <= 1.0, f"worst error is {r:.3f} x tolerance"
    y2 = torch.empty_like(y)
    w4.gemv_ws_into(q, xd, y2, ws)
    assert torch.equal(y, y2)                       # deterministic
    with pytest.raises(w4.W4Error) as e:
        w4.gemv_ws_into(q, xd, y2, ws[: need - 16])
    assert e.value.code == -5


def test_gemv_ws_without_k_parts_is_gemv():
    W = synth.weights(4096, 4096, 0.02, seed=0, name="ws.none")
    x = dev_bf16(synth.activations_bf16(4, 4096, seed=0, name="ws.none.x"))
    q = w4.quantize_pack(dev_f32(W), "sym4_g128")
    assert w4.gemv_workspace_bytes(q, 4) == 0
    y = torch.empty((4, 4096), dtype=torch.float32, device="cuda")
    w4.gemv_ws_into(q, x, y, None)
    assert torch.equal(y, w4.gemv(q, x))


@pytest.mark.parametrize("M", [1, 4, 16])
@pytest.mark.parametrize("N,K,mat", [(4096, 4096, "wq"), (11008, 4096, "gate"), (4096, 11008, "down")])
def test_gemv_llama7b_shapes(N, K, mat, M):
    _run("sym4_g128", N, K, M, f"llama7b.{mat}")


@pytest.mark.parametrize("M", [1, 4, 16])
@pytest.mark.parametrize("N,K,mat", [(4096, 4096, "wq"), (11008, 4096, "gate"), (4096, 11008, "down")])
def test_gemv_w8a16_llama7b_shapes(N, K, mat, M):
    """Whole layers in the router's 8-bit affine g64 scheme (W8A16)."""
    _run("aff8_g64", N, K, M, f"w8.llama7b.{mat}")


@pytest.mark.parametrize("M", [1, 8])
@pytest.mark.parametrize("N,K,mat", [(5120, 5120, "wq"), (13824, 5120, "gate"), (5120, 13824, "down")])
def test_gemv_llama13b_shapes(N, K, mat, M):
    _run("aff4_g64", N, K, M, f"llama13b.{mat}")


@pytest.mark.parametrize("scheme,N,K,M", [
    ("sym4_g128", 70000, 256, 4),     # 4375 row tiles: more than 16 per CU
    ("aff4_g64", 66000, 192, 3),      # affine, odd group count (a half step)
    ("sym4_g128", 65537, 384, 16),    # one row past 4096 tiles, a full token tile
])
def test_gemv_split_k_kernel_matches_oracle(scheme, N, K, M):
    """Launches with more than 16 row tiles of 16 rows per CU (N > 65536) take the
    split-K skinny kernel (K interleaved over wavefronts, two row tiles each)."""
    assert (N + 15) // 16 > 16 * 256
    _run(scheme, N, K, M, f"splitk.{scheme}.{N}x{K}")


_HEAD = {}


def _head():
    """The 13B-shaped tied head, 152064 x 5120 affine 4-bit g64, quantized on the
    GPU once; the oracle quantizes only the sampled rows (rows are independent)."""
    if not _HEAD:
        N, K = 152064, 5120
        rows = np.sort(np.random.default_rng(0).choice(N, 1536, replace=False))
        rows = np.unique(np.concatenate([rows, [0, 1, 15, 16, 31, N - 17, N - 2, N - 1]]))
        W = synth.weights(N, K, 0.02, seed=0, name="llama13b.head")
        Wd = dev_f32(W)
        q = w4.quantize_pack(Wd, "aff4_g64")
        del Wd
        torch.cuda.synchronize()
        c, s, b = oracle.quantize_pack(np.ascontiguousarray(W[rows]), "aff4_g64")
        del W
        assert np.array_equal(q.codes[torch.from_numpy(rows).cuda()].cpu().numpy(), c)
        _HEAD.update(q=q, rows=rows, ref=(c, s, b))
    return _HEAD


@pytest.mark.parametrize("M", [1, 2, 8, 16])
def test_gemv_head_sampled_rows(M):
    """The tied head of the 13B-shaped stack on sampled rows (first and last
    tiles among them); at M > 1 this is the split-K skinny kernel (9504 row tiles)."""
    h = _head()
    print(f"[gemv] llama13b.head 152064x5120 M={M}", flush=True)
    x = synth.activations_bf16(M, 5120, seed=0, name=f"llama13b.head.x{M}")
    y = w4.gemv(h["q"], dev_bf16(x)).cpu().numpy()[:, h["rows"]]
    yr, S = oracle.gemv_reference(*h["ref"], "aff4_g64", x)
    r = tolerance_ratio(y, yr, S)
    assert r <= 1.0, f"worst error is {r:.3f} x tolerance"


@pytest.mark.parametrize("ngroups", [2, 3])
@pytest.mark.parametrize("scheme", ["aff4_g64", "sym4_g128", "aff8_g64"])
def test_gemv_exact_on_dyadic_toy(scheme, ngroups):
    """8 x 64/128 toy with dyadic scales/biases and small-integer activations:
    every partial sum is exactly representable, so the fp32 result is exact.
    Two tokens take the matrix-core path; an odd group count covers the
    4-bit affine half step."""
    rng = np.random.default_rng(21)
    g = 128 if scheme == "sym4_g128" else 64
    K, N = ngroups * g, 8
    if scheme == "sym4_g128":
        q = rng.integers(-7, 8, size=(N, K))
        s = np.array([2.0 ** -(2 + n % 3) for n in range(N)] * (K // g), np.float32).reshape(K // g, N).T.copy()
        codes, sb, bb = oracle.pack(q, 4), s, None
        sf, bf = s.astype(np.float64), None
    else:
        bits = 8 if scheme == "aff8_g64" else 4
        q = rng.integers(0, 2 ** bits, size=(N, K))
        sf = np.array([[2.0 ** -(3 + (n + j) % 3) for j in range(K // g)] for n in range(N)])
        bf = np.array([[-(n + j + 1) * 2.0 ** -5 for j in range(K // g)] for n in range(N)])
        sb = (sf.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
        bb = (bf.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
        codes = oracle.pack(q, bits)
    xi = rng.integers(-3, 4, size=(2, K))
    xb = (xi.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    y = w4.gemv(upload(codes, sb, bb, scheme), dev_bf16(xb)).cpu().numpy()
    for m in range(2):
        for n in range(N):
            ex = Fraction(0)
            for k in range(K):
                w_ = Fraction(float(sf[n, k // g])) * int(q[n, k])
                if bf is not None:
                    w_ += Fraction(float(bf[n, k // g]))
                ex += w_ * int(xi[m, k])
            assert Fraction(float(y[m, n])) == ex, (m, n)


def test_gemv_is_deterministic_and_noops():
    W = synth.weights(2048, 4096, 0.02, seed=3, name="det")
    q = w4.quantize_pack(dev_f32(W), "sym4_g128")
    x = dev_bf16(synth.activations_bf16(3, 4096, seed=3, name="det.x"))
    a = w4.gemv(q, x)
    b = w4.gemv(q, x)
    assert torch.equal(a, b)
    y = torch.full((1, 2048), 7.0, device="cuda")
    w4.gemv_into(q, x[:0], y)           # M == 0: nothing is written
    torch.cuda.synchronize()
    assert torch.equal(y, torch.full((1, 2048), 7.0, device="cuda"))


def test_gemv_rejects_bad_arguments():
    q = w4.quantize_pack(dev_f32(synth.weights(64, 256, 0.02, 4, "bad")), "aff4_g64")
    x = dev_bf16(synth.activations_bf16(65, 256, 4, "bad.x"))
    with pytest.raises(w4.W4Error):
        w4.gemv(q, x)                    # M > 64
    xs = torch.empty(257, dtype=torch.int16, device="cuda")[1:].view(1, 256)
    with pytest.raises(w4.W4Error):
        w4.gemv(q, xs)


@pytest.mark.parametrize("M", [1, 2])
@pytest.mark.parametrize("scheme,K,Ns", [
    ("sym4_g128", 4096, [1000, 1000, 1000]),      # Q/K/V-like
    ("sym4_g128", 4096, [700, 0, 333]),           # an empty member
    ("aff4_g64", 5120, [1300, 1300]),             # gate/up-like
    ("aff4_g64", 2048, [768, 768, 2048, 5]),      # four members, ragged
])
def test_gemv_multi_matches_oracle_and_separate_calls(scheme, K, Ns, M):
    print(f"[gemv_multi] {scheme} K={K} Ns={Ns} M={M}", flush=True)
    x = synth.activations_bf16(M, K, seed=1, name=f"multi.x.{K}")
    xd = dev_bf16(x)
    qs, refs = [], []
    for i, N in enumerate(Ns):
        W = synth.weights(max(N, 1), K, 0.02, seed=1, name=f"multi.{scheme}.{i}")[:N]
        c, s, b = oracle.quantize_pack(np.ascontiguousarray(W), scheme)
        qs.append(w4.quantize_pack(dev_f32(W), scheme) if N else
                  w4.empty_quantized(scheme, 0, K))
        refs.append(oracle.gemv_reference(c, s, b, scheme, x) if N else None)
    ys = w4.gemv_multi(qs, xd)
    for q, y, ref in zip(qs, ys, refs):
        if ref is None:
            assert y.shape[1] == 0
            continue
        assert tolerance_ratio(y.cpu().numpy(), *ref) <= 1.0
        assert torch.equal(y, w4.gemv(q, xd))       # one launch == separate launches, bit for bit
