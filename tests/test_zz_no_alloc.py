"""The decode entry point that allocates nothing (bifocal_decode_noalloc), for callers that
cannot allocate device memory: its split partials live in the library's static per-device
scratch. Two calls in a row (the second smaller, so it runs over what the first left in the
scratch) must give the bits of bifocal_decode with a workspace, and the oracle's values."""
import ctypes

import numpy as np
import pytest
import torch

from oracle import bifocal_decode
from zero_shot_rope_amd import bifocal as Z
from zero_shot_rope_amd import workloads as W

MAX_ABS, REL_L2, LSE_ABS = 2e-2, 5e-3, 2e-2
ESCRATCH = -5
SCRATCH_BYTES = 16 << 20
FAKE = 0x1000  # never dereferenced: the call below fails its host-side size check first


def test_noalloc_rejects_shapes_beyond_the_scratch_before_any_hip_call():
    lib = Z.load_library()
    fp = ctypes.cast(ctypes.c_void_p(FAKE), ctypes.POINTER(ctypes.c_float))
    # batch 512 x 64 query heads of head_dim 128: one split per sequence, 512 * 64 * 130 * 4 B
    # = 17 MB of partials, past the 16 MiB scratch.
    need = Z.bifocal_decode_workspace_bytes(512, 64, 8, 128, 1000)
    assert need > SCRATCH_BYTES
    st = lib.bifocal_decode_noalloc(FAKE, FAKE, FAKE, FAKE, fp, 512, 64, 8, 128, 1000, 1000, 64, 256, 1e6, None)
    assert st == ESCRATCH
    assert "static scratch" in Z.bifocal_status_string(st)
    # Invalid arguments are still reported as such (checked before the scratch size).
    assert lib.bifocal_decode_noalloc(None, FAKE, FAKE, FAKE, fp, 1, 4, 1, 128, 10, 10, 4, 8, 1e6, None) == -1


def _draw(seed, B, cap, Hq, Hkv, D):
    rng = np.random.default_rng(seed)
    kb = W.round_to_bf16_bits(rng.standard_normal((B, cap, Hkv, D), dtype=np.float32))
    vb = W.round_to_bf16_bits(rng.standard_normal((B, cap, Hkv, D), dtype=np.float32))
    qb = W.round_to_bf16_bits(rng.standard_normal((B, Hq, D), dtype=np.float32))
    return qb, kb, vb


def _dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


@pytest.mark.gpu
def test_noalloc_decode_matches_decode_on_two_calls():
    # (batch, cap, Hq, Hkv, D, w_pretrained, w0, theta, L): the second call is smaller in every
    # dimension, so its split partials occupy a prefix of what the first call wrote.
    cases = [(2, 3000, 32, 8, 128, 1000, 128, 1e6, 2999), (1, 700, 8, 2, 64, 200, 60, 1e4, 650)]
    for i, (B, cap, Hq, Hkv, D, wp, w0, theta, L) in enumerate(cases):
        print(f"noalloc call {i}: B={B} L={L} Hq={Hq} Hkv={Hkv} D={D}", flush=True)
        qb, kb, vb = _draw(500 + i, B, cap, Hq, Hkv, D)
        q, kc, vc = _dev(qb), _dev(kb), _dev(vb)
        o_na = torch.full((B, Hq, D), -7.0, dtype=torch.bfloat16, device="cuda")
        l_na = torch.full((B, Hq), -7.0, dtype=torch.float32, device="cuda")
        # Through the C ABI itself (raw pointers, the current stream).
        Z.bifocal_decode_noalloc(q, kc, vc, o_na, l_na, B, Hq, Hkv, D, L, cap, w0, wp, theta)
        ws_bytes = Z.bifocal_decode_workspace_bytes(B, Hq, Hkv, D, L)
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
        o_ws = torch.empty((B, Hq, D), dtype=torch.bfloat16, device="cuda")
        l_ws = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
        Z.bifocal_decode(q, kc, vc, o_ws, l_ws, B, Hq, Hkv, D, L, cap, w0, wp, theta, ws, ws_bytes)
        torch.cuda.synchronize()
        # Same kernels, same split plan: the same bits.
        assert torch.equal(o_na, o_ws) and torch.equal(l_na, l_ws), f"call {i}: differs from bifocal_decode"
        ref_o, ref_lse = bifocal_decode(W.bf16_bits_to_float32(qb), W.bf16_bits_to_float32(kb),
                                        W.bf16_bits_to_float32(vb), L=L, w0=w0, w_pretrained=wp, theta=theta)
        got = o_na.float().cpu().numpy().astype(np.float64)
        err = got - ref_o
        rel = float(np.linalg.norm(err) / np.linalg.norm(ref_o))
        print(f"  max_abs={np.abs(err).max():.3e} rel_l2={rel:.3e}", flush=True)
        assert np.abs(err).max() <= MAX_ABS and rel <= REL_L2
        assert np.max(np.abs(l_na.cpu().numpy() - ref_lse)) <= LSE_ABS
    # The convenience wrapper runs the same entry point.
    o2 = Z.decode_noalloc(q, kc, vc, L=L, w0=w0, w_pretrained=wp, rope_theta=theta)
    torch.cuda.synchronize()
    assert torch.equal(o2, o_ws)
