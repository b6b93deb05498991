"""The attention entry point for callers that cannot allocate (kq_attn_quant_fwd_noalloc): its
key-split workspace lives in the library's static device array.  Checked through the C ABI
against kq_attn_quant_fwd_ws with a caller workspace, bit for bit, on two calls in a row, the
second on a smaller input (the array keeps the first call's partial results)."""
import numpy as np
import pytest
import torch

import precision_quantized_attention_amd as kq

pytestmark = pytest.mark.gpu


def _inputs(B, H, N, seed):
    """E4M3 codes of N(0, 2^2) Q, K and V (V transposed, zero beyond N) on the device."""
    g = torch.Generator().manual_seed(seed)
    codes = []
    for _ in range(3):
        x = torch.randn((B, H, N, 128), generator=g) * 2
        codes.append(x.clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8))
    q8, k8, v8 = codes
    ld = kq.kq_vt_ld(N)
    vt = torch.zeros((B * H, 128, ld), dtype=torch.uint8)
    vt[:, :, :N] = v8.reshape(B * H, N, 128).transpose(1, 2)
    return q8.cuda(), k8.cuda(), vt.contiguous().cuda()


@pytest.mark.parametrize("shapes", [((1, 2, 2560), (1, 1, 1000))])
def test_noalloc_matches_the_workspace_entry_point(shapes):
    for i, (B, H, N) in enumerate(shapes):
        print(f"no-alloc attention call {i}: B={B} H={H} N={N}", flush=True)
        nbytes = kq.kq_attn_workspace_size(B, H, N)
        assert nbytes > 0          # the shape takes the key split, so the array is used
        q8, k8, vt = _inputs(B, H, N, seed=11 + i)
        s_q, s_k, s_v, sm = 0.02, 0.03, 0.05, float(np.float32(1 / np.sqrt(128)))
        ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        o_ref = torch.empty((B, H, N, 128), dtype=torch.float32, device="cuda")
        st_ref = torch.empty((B, H, N, 2), dtype=torch.float32, device="cuda")
        kq.kq_attn_quant_fwd_ws(q8, k8, vt, s_q, s_k, s_v, sm, o_ref, ws, row_stats=st_ref)
        o = torch.full_like(o_ref, float("nan"))
        st = torch.full_like(st_ref, float("nan"))
        kq.kq_attn_quant_fwd_noalloc(q8, k8, vt, s_q, s_k, s_v, sm, o, row_stats=st)
        torch.cuda.synchronize()
        assert torch.isfinite(o_ref).all()
        assert torch.equal(o, o_ref), float((o - o_ref).abs().max())
        assert torch.equal(st, st_ref)
