"""GPU: path_decode_step_noalloc (the decode step with the library's own
partials array, for callers that cannot allocate) against path_decode_step
(the same step with a caller workspace): outputs, lse and the updated caches
bit-identical, on two calls in a row, the second smaller than the first."""
import numpy as np
import pytest
import torch

import softmax_attention_ut_amd as pa

pytestmark = pytest.mark.gpu


def _case(B, H, T_max, t, d, seed):
    g = torch.Generator().manual_seed(seed)
    bf = lambda *s: torch.randn(*s, generator=g).to(torch.bfloat16).cuda()
    kc, vc = bf(B, H, T_max, d), bf(B, H, T_max, d)
    q, k, v = bf(B, H, d), bf(B, H, d), bf(B, H, d)
    w = torch.randn(B, H, d, generator=g, dtype=torch.float64)
    w = (w / w.norm(dim=-1, keepdim=True)).to(torch.bfloat16).cuda()
    beta = (2 * torch.sigmoid(torch.randn(B, H, generator=g))).clamp(0.02, 1.98).float().cuda()
    return kc, vc, q, k, v, w, beta


def _both(B, H, T_max, t, d, seed):
    kc, vc, q, k, v, w, beta = _case(B, H, T_max, t, d, seed)
    scale = d ** -0.5
    ka, va = kc.clone(), vc.clone()
    oa = torch.empty(B, H, d, dtype=torch.bfloat16, device="cuda")
    la = torch.empty(B, H, dtype=torch.float32, device="cuda")
    ws = pa.decode_workspace(B, H, T_max, d, pa.PATH_BF16, kc.device)
    pa.path_decode_step(ka, va, q, k, v, w, beta, oa, la, t, scale, ws)
    kb, vb = kc.clone(), vc.clone()
    ob = torch.full((B, H, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    lb = torch.full((B, H), float("nan"), dtype=torch.float32, device="cuda")
    pa.path_decode_step_noalloc(kb, vb, q, k, v, w, beta, ob, lb, t, scale)
    torch.cuda.synchronize()
    print(f"B={B} H={H} T_max={T_max} t={t} d={d}: out max |a-b| "
          f"{(oa.float() - ob.float()).abs().max().item():.3e}", flush=True)
    assert torch.isfinite(ob.float()).all() and torch.isfinite(lb).all()
    assert torch.equal(oa, ob)
    assert torch.equal(la, lb)
    assert torch.equal(ka, kb)
    assert torch.equal(va, vb)
    # the step did update the cache and store the new key and value
    assert not torch.equal(ka[:, :, :t], kc[:, :, :t])
    assert torch.equal(va[:, :, t], v)


def test_noalloc_decode_matches_workspace_decode_twice():
    _both(2, 32, 8448, 8300, 128, seed=1)       # the d=128 decode shape: 19 splits per head
    _both(1, 3, 300, 150, 64, seed=2)           # then a smaller call (the array holds the
                                                # previous call's partials)
