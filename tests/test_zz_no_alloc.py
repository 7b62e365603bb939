"""The allocation-free MoE entry point (w4a16_moe_gemv_noalloc) against the
workspace entry point it mirrors (w4a16_moe_gemv): the same kernels run on a
library-owned static scratch instead of a caller buffer, so the outputs must be
identical bit for bit, on two calls in a row (the second with fewer tokens and
the one-token path) and after the other entry point has run; sizes beyond the
scratch are refused before anything is launched."""
import numpy as np
import pytest
import torch

import bit_weight_only_quantize_amd as w4
import synth

pytestmark = pytest.mark.gpu

E, D, F, Fs, K_TOP = 32, 2048, 768, 2048, 8


def _layer():
    dev = torch.device("cuda:0")
    mats = []
    for nm, N, K in (("gate", F, D), ("up", F, D), ("down", D, F)):
        q = w4.empty_quantized("aff4_g64", N, K, num_experts=E, device=dev)
        for e in range(E):
            w4.quantize_pack(synth.device_weights(N, K, 0.02, 0, f"na.{nm}.{e}", dev), "aff4_g64",
                             out=q, expert=e)
        mats.append(q)
    shared = [w4.quantize_pack(synth.device_weights(N, K, 0.02, 0, f"na.s{nm}", dev), "aff4_g64")
              for nm, N, K in (("g", Fs, D), ("u", Fs, D), ("d", D, Fs))]
    return mats, shared


def _routing(M, seed):
    g = torch.Generator().manual_seed(seed)
    ids = torch.stack([torch.randperm(E, generator=g)[:K_TOP] for _ in range(M)]).to(torch.int32)
    ids[0, -1] = -1                                   # an empty slot contributes nothing
    p = torch.rand((M, K_TOP), generator=g) / K_TOP
    return ids.cuda(), p.cuda()


def _x(M, seed):
    bits = synth.activations_bf16(M, D, seed, f"na.x{M}")
    return torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)


def test_noalloc_matches_the_workspace_entry_point_on_consecutive_calls():
    (gate, up, down), shared = _layer()
    cases = [(32, 1), (1, 2)]                         # the second call is smaller (one token)
    ins = [(_x(M, s), *_routing(M, s)) for M, s in cases]
    print(f"[noalloc] E={E} D={D} F={F} Fs={Fs} M={[c[0] for c in cases]}", flush=True)
    got = [w4.moe_gemv_noalloc(gate, up, down, x, ids, p, shared=shared) for x, ids, p in ins]
    torch.cuda.synchronize()
    for (x, ids, p), y in zip(ins, got):
        ref = w4.moe_gemv(gate, up, down, x, ids, p, shared=shared)
        assert torch.equal(y, ref)
        assert torch.isfinite(y).all()
    # again after the workspace entry point ran, and with no shared expert
    x, ids, p = ins[0]
    y = w4.moe_gemv_noalloc(gate, up, down, x, ids, p)
    assert torch.equal(y, w4.moe_gemv(gate, up, down, x, ids, p))


def test_noalloc_refuses_sizes_beyond_the_scratch():
    (gate, up, down), shared = _layer()
    M = 256
    need = w4.moe_workspace_bytes(M, K_TOP, E, D, F, Fs)
    assert need > w4.MOE_SCRATCH_BYTES
    x, (ids, p) = _x(M, 3), _routing(M, 3)
    with pytest.raises(w4.W4Error) as e:
        w4.moe_gemv_noalloc(gate, up, down, x, ids, p, shared=shared)
    assert e.value.code == -5
