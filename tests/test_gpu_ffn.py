"""GPU parity for w4a16_ffn, the dense gated FFN of a decode layer:
h = bf16(gelu_tanh(W_gate x) * (W_up x)), y = W_down h.

One token takes two launches by default (gate/up rows with the activation in
their epilogue, then the down GEMV), 4-bit and 8-bit codes alike; switched on,
the 7B / 13B shapes run as a single launch whose down rows wait for h through
device-scope words; several tokens take the skinny kernel in gated-pair mode
(gate and up tiles of the same rows in one workgroup) where the tiles pair up;
the rest (and any shape on request) take the three-launch sequence. The paths
must give the same bits (the same per-row arithmetic in the same order), on
consecutive calls sharing one workspace and inside a replayed HIP graph. Against the oracle (its own quantization of the same seeded weights and
its fp64 chain): every h within the interval the gate/up tolerance allows plus
one bf16 rounding, y within 2e-3*S + 1e-5 with S = sum|w_down||h|. The give-up
path of the single launch's wait is forced from the host (the "h complete" flag
is withheld, the poll limit small): the call must complete, report it, and leave
the workspace usable."""
import numpy as np
import pytest
import torch

import bit_weight_only_quantize_amd as w4
import oracle
import synth
from gpu_util import TOL_ABS, TOL_REL, U_BF16, dev_bf16, dev_f32, host_bits16, tolerance_ratio

pytestmark = pytest.mark.gpu

_FFN = {}


@pytest.fixture(autouse=True)
def _restore_settings():
    yield
    w4.ffn_set_path(w4.FFN_PATH_DEFAULT)
    w4.ffn_set_wait(0, withhold=False)


def _with_path(path, fn):
    w4.ffn_set_path(path)
    try:
        return fn()
    finally:
        w4.ffn_set_path(w4.FFN_PATH_DEFAULT)


def _ffn(D, F, scheme, tag):
    """Host (oracle) and device storage of one FFN's three matrices, cached."""
    key = (D, F, scheme, tag)
    if key not in _FFN:
        host, dev = [], []
        for nm, N, K in (("gate", F, D), ("up", F, D), ("down", D, F)):
            W = synth.weights(N, K, 0.02, 13, f"{tag}.{nm}")
            host.append(oracle.quantize_pack(W, scheme))
            dev.append(w4.quantize_pack(dev_f32(W), scheme))
        _FFN.clear()  # one FFN at a time keeps host memory small
        _FFN[key] = (host, dev)
    return _FFN[key]


def _check_oracle(x, h, y, host, scheme):
    """h: interval bound from the gate/up tolerance plus one bf16 rounding;
    y: 2e-3 * S + 1e-5 against the oracle's chain."""
    g_trip, u_trip, d_trip = host
    yr, S, hr = oracle.ffn(x, g_trip, u_trip, d_trip, scheme)
    Wg = oracle.dequantize(*g_trip, scheme)
    Wu = oracle.dequantize(*u_trip, scheme)
    g = oracle.matmul_f64(x, Wg)
    u = oracle.matmul_f64(x, Wu)
    tg = TOL_REL * oracle.abs_matmul_f64(x, Wg) + TOL_ABS
    tu = TOL_REL * oracle.abs_matmul_f64(x, Wu) + TOL_ABS
    a = oracle.gelu_tanh(g) * u
    # gelu_tanh is 1.13-Lipschitz: |a' - a| <= 1.13 tg (|u| + tu) + |gelu(g)| tu + tg tu
    da = 1.13 * tg * (np.abs(u) + tu) + np.abs(oracle.gelu_tanh(g)) * tu + 1e-6 * np.abs(a)
    hg = oracle.bf16_to_f32(host_bits16(h)).astype(np.float64).reshape(a.shape)
    bound = da + U_BF16 * (np.abs(a) + da) + 1e-30
    worst = float((np.abs(hg - a) / bound).max())
    assert worst <= 1.0, f"h: worst error {worst:.3f} x bound"
    same = float(np.mean(host_bits16(h).reshape(hr.shape) == hr))
    assert same > 0.98, f"only {same:.4f} of h equals the oracle's bits"
    r = tolerance_ratio(y.cpu().numpy(), yr, S)
    assert r <= 1.0, f"y: worst error {r:.3f} x tolerance"


@pytest.mark.parametrize("D,F,scheme", [
    (4096, 11008, "sym4_g128"),   # 7B: gate/up 2 x 11008 x 4096, down 4096 x 11008
    (5120, 13824, "aff4_g64"),    # 13B
    (2176, 10368, "sym4_g128"),   # smallest instance: 68 and 324 code vectors per row
    (8192, 16384, "aff4_g64"),    # largest instance
])
def test_every_path_gives_the_same_bits(D, F, scheme):
    print(f"[ffn] paths D={D} F={F} {scheme}", flush=True)
    host, (gate, up, down) = _ffn(D, F, scheme, f"ffn.{D}.{F}.{scheme}")
    ws = w4.ffn_workspace(down, 1)
    for call in range(3):
        x = dev_bf16(synth.activations_bf16(1, D, 40 + call, f"ffn.x.{D}"))
        y0, h0 = w4.ffn(gate, up, down, x, workspace=ws, want_h=True)
        y1, h1 = _with_path(w4.FFN_PATH_SINGLE_LAUNCH,
                            lambda: w4.ffn(gate, up, down, x, workspace=ws, want_h=True))
        assert w4.ffn_status(ws) == 0
        y2, h2 = _with_path(w4.FFN_PATH_SEQUENCE,
                            lambda: w4.ffn(gate, up, down, x, workspace=ws, want_h=True))
        torch.cuda.synchronize()
        for hh, yy, nm in ((h1, y1, "single launch"), (h2, y2, "sequence")):
            assert torch.equal(h0.view(torch.int16), hh.view(torch.int16)), f"call {call}: {nm} h differs"
            assert torch.equal(y0, yy), f"call {call}: {nm} y differs"
    assert torch.count_nonzero(ws[:16384]).item() == 0  # hand-off words left zero


@pytest.mark.parametrize("path", [0, 1])
@pytest.mark.parametrize("D,F,scheme", [(4096, 11008, "sym4_g128"), (5120, 13824, "aff4_g64")])
def test_one_token_matches_oracle(D, F, scheme, path):
    print(f"[ffn] oracle D={D} F={F} {scheme} path {path}", flush=True)
    host, (gate, up, down) = _ffn(D, F, scheme, f"ffn.{D}.{F}.{scheme}")
    xh = synth.activations_bf16(1, D, 3, f"ffn.xo.{D}")
    y, h = _with_path(path, lambda: w4.ffn(gate, up, down, dev_bf16(xh), want_h=True))
    torch.cuda.synchronize()
    _check_oracle(xh, h, y, host, scheme)


@pytest.mark.parametrize("M", [4, 16])
def test_several_tokens_match_oracle(M):
    """Three launches: gate+up (skinny MFMA), the activation, down (K parts at M = 16)."""
    D, F, scheme = 4096, 11008, "sym4_g128"
    print(f"[ffn] oracle M={M}", flush=True)
    host, (gate, up, down) = _ffn(D, F, scheme, f"ffn.{D}.{F}.{scheme}")
    xh = synth.activations_bf16(M, D, 5, f"ffn.xm.{M}")
    y, h = w4.ffn(gate, up, down, dev_bf16(xh), want_h=True)
    torch.cuda.synchronize()
    _check_oracle(xh, h, y, host, scheme)


@pytest.mark.parametrize("M,D,F,scheme", [
    (1, 2048, 768, "aff4_g64"),    # two launches (outside the single launch's shapes)
    (1, 9216, 1024, "sym4_g128"),  # D / 32 > 256: the sequence
    (3, 2048, 768, "aff4_g64"),
    (64, 2048, 768, "aff4_g64"),   # the most tokens the FFN takes: multi-token VALU launches
])
def test_other_shapes_take_the_sequence(M, D, F, scheme):
    print(f"[ffn] sequence M={M} D={D} F={F} {scheme}", flush=True)
    host, (gate, up, down) = _ffn(D, F, scheme, f"ffn.{D}.{F}.{scheme}")
    xh = synth.activations_bf16(M, D, 9, f"ffn.xs.{M}")
    y, h = w4.ffn(gate, up, down, dev_bf16(xh), want_h=True)
    torch.cuda.synchronize()
    _check_oracle(xh, h, y, host, scheme)


@pytest.mark.parametrize("path", [0, 1])
def test_graph_replays_equal_eager(path):
    """Captured in a HIP graph (the single launch clears its own hand-off words,
    no memset node): every replay equals the eager result."""
    D, F, scheme = 4096, 11008, "sym4_g128"
    print(f"[ffn] graph path {path}", flush=True)
    w4.ffn_set_path(path)
    _, (gate, up, down) = _ffn(D, F, scheme, f"ffn.{D}.{F}.{scheme}")
    x = dev_bf16(synth.activations_bf16(1, D, 21, "ffn.xg"))
    ws = w4.ffn_workspace(down, 1)
    y = torch.empty((1, D), dtype=torch.float32, device="cuda")
    ref = w4.ffn(gate, up, down, x, workspace=ws).clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        w4.ffn(gate, up, down, x, workspace=ws, y=y)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        w4.ffn(gate, up, down, x, workspace=ws, y=y)
    for rep in range(4):
        y.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, ref), f"replay {rep}"
        assert w4.ffn_status(ws) == 0
        _ = (x.float() * 2).sum().item()  # unrelated eager work between replays
    w4.ffn_set_path(w4.FFN_PATH_DEFAULT)


def test_withheld_flag_gives_up_and_the_workspace_recovers():
    D, F, scheme = 4096, 11008, "sym4_g128"
    print("[ffn] give-up", flush=True)
    _, (gate, up, down) = _ffn(D, F, scheme, f"ffn.{D}.{F}.{scheme}")
    x = dev_bf16(synth.activations_bf16(1, D, 23, "ffn.xw"))
    ws = w4.ffn_workspace(down, 1)
    w4.ffn_set_path(w4.FFN_PATH_SINGLE_LAUNCH)
    try:
        w4.ffn_set_wait(2000, withhold=True)
        w4.ffn(gate, up, down, x, workspace=ws)
        assert w4.ffn_status(ws) == w4.FFN_GAVE_UP_H
        w4.ffn_set_wait(0, withhold=False)
        y1 = w4.ffn(gate, up, down, x, workspace=ws)
        assert w4.ffn_status(ws) == 0
    finally:
        w4.ffn_set_wait(0, withhold=False)
        w4.ffn_set_path(w4.FFN_PATH_DEFAULT)
    y2 = w4.ffn(gate, up, down, x, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)


@pytest.mark.parametrize("M,D,F,scheme", [(1, 4096, 11008, "sym4_g128"), (4, 4096, 11008, "sym4_g128"),
                                          (1, 2048, 768, "aff4_g64")])
def test_gate_up_half_equals_the_ffn_h(M, D, F, scheme):
    print(f"[ffn] gate/up half M={M} D={D} F={F}", flush=True)
    _, (gate, up, down) = _ffn(D, F, scheme, f"ffn.{D}.{F}.{scheme}")
    x = dev_bf16(synth.activations_bf16(M, D, 31, f"ffn.xh.{M}"))
    _, h_ref = w4.ffn(gate, up, down, x, want_h=True)
    h = w4.ffn_gate_up(gate, up, x)
    torch.cuda.synchronize()
    assert torch.equal(h.view(torch.int16), h_ref.view(torch.int16))


@pytest.mark.parametrize("M,D,F,scheme", [
    (4, 4096, 11008, "sym4_g128"),   # 7B: 6 tile pairs per workgroup
    (16, 4096, 11008, "sym4_g128"),
    (13, 4096, 11008, "sym4_g128"),  # 8 staging loads in flight per lane
    (4, 2048, 4096, "aff4_g64"),     # affine regrouping, 2 tiles per workgroup
    (2, 2048, 768, "aff4_g64"),      # 1 tile per CU becomes a pair on half the CUs
    (8, 5120, 13824, "aff4_g64"),    # 13B: 7 tiles per CU, so gate/up + activation launches
])
def test_several_tokens_gated_launch_equals_the_sequence(M, D, F, scheme):
    """Several tokens: gate and up in one skinny launch whose epilogue writes h
    (tile pairs in one workgroup) against gate/up GEMV + activation launches."""
    print(f"[ffn] gated M={M} D={D} F={F} {scheme}", flush=True)
    _, (gate, up, down) = _ffn(D, F, scheme, f"ffn.{D}.{F}.{scheme}")
    x = dev_bf16(synth.activations_bf16(M, D, 33, f"ffn.xq.{M}"))
    y0, h0 = w4.ffn(gate, up, down, x, want_h=True)
    y1, h1 = _with_path(w4.FFN_PATH_SEQUENCE, lambda: w4.ffn(gate, up, down, x, want_h=True))
    torch.cuda.synchronize()
    assert torch.equal(h0.view(torch.int16), h1.view(torch.int16))
    assert torch.equal(y0, y1)



@pytest.mark.parametrize("M,D,F", [
    (1, 1024, 2048),
    (1, 4096, 11008),   # 7B shape: 256 code vectors per row, one staged per thread
    (1, 5120, 13824),   # 13B shape: 320 vectors, two staged per thread
    (4, 4096, 11008),   # several tokens: the gated skinny launch with 8-bit steps
    (16, 4096, 11008),
    (8, 5120, 13824),
])
def test_8bit_codes_equal_the_sequence_and_match_the_oracle(M, D, F):
    """W8A16 (the router's affine g64 8-bit scheme for whole layers): the gate/up
    launch with the activation in its epilogue against gate/up GEMV + activation
    launches, bit for bit, and the chain against the oracle."""
    scheme = "aff8_g64"
    print(f"[ffn] 8-bit M={M} D={D} F={F}", flush=True)
    host, (gate, up, down) = _ffn(D, F, scheme, f"ffn.{D}.{F}.{scheme}")
    xh = synth.activations_bf16(M, D, 37, f"ffn.x8.{M}")
    x = dev_bf16(xh)
    y0, h0 = w4.ffn(gate, up, down, x, want_h=True)
    y1, h1 = _with_path(w4.FFN_PATH_SEQUENCE, lambda: w4.ffn(gate, up, down, x, want_h=True))
    torch.cuda.synchronize()
    assert torch.equal(h0.view(torch.int16), h1.view(torch.int16))
    assert torch.equal(y0, y1)
    _check_oracle(xh, h0, y0, host, scheme)
