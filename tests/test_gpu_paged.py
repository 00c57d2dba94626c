"""GPU: the paged K/V cache (path_kcache_from_prefill_paged,
path_decode_step_paged) against the contiguous cache and the oracle.

The paged calls run the same arithmetic with the same split of the keys as
the contiguous ones, so outputs, lse and every cached key and value must be
bit-identical to them; the block table is a shuffled assignment of pages
(with unused pages in the pool) and the decode crosses page boundaries.  The
decode outputs are also held to the bf16 tolerances against the fp64 oracle
(max-abs 2e-2, mean-abs 2e-3).
"""
import numpy as np
import pytest
import torch

import oracle
import softmax_attention_ut_amd as pa
from softmax_attention_ut_amd.inputs import generate

pytestmark = pytest.mark.gpu


def _gather(pool, table, T):
    """[num_blocks, H, P, d] pool -> [B, H, T, d] through the table."""
    B = table.shape[0]
    P = pool.shape[2]
    nb = (T + P - 1) // P
    rows = [torch.cat([pool[int(table[b, i])] for i in range(nb)], dim=1)[:, :T] for b in range(B)]
    return torch.stack(rows)


@pytest.mark.parametrize("d,gate,page", [(64, False, 64), (128, False, 64), (64, True, 128),
                                         (128, True, 64)])
def test_paged_equals_contiguous(d, gate, page):
    B, H, L, n = 2, 3, 200, 70
    print(f"paged d={d} gate={gate} page={page}: B={B} H={H} L={L} steps={n}", flush=True)
    inp = generate(B, H, L + n, d, dtype="bf16", gate=gate, seed=40 + d + page)
    g = {k: (None if t is None else t.cuda()) for k, t in vars(inp).items()}
    max_blocks = (L + n + page - 1) // page + 1
    T = max_blocks * page
    num_blocks = B * max_blocks + 3
    perm = torch.randperm(num_blocks, generator=torch.Generator().manual_seed(7))
    table = perm[:B * max_blocks].reshape(B, max_blocks).to(torch.int32).cuda()
    pre = lambda t: t[:, :, :L].contiguous()

    kc, vc = pa.kcache_from_prefill(pre(g["k"]), pre(g["v"]), pre(g["w"]), pre(g["beta"]), T)
    kp = torch.zeros(num_blocks, H, page, d, dtype=torch.bfloat16, device="cuda")
    vp = torch.zeros_like(kp)
    kws = torch.empty(pa.path_kcache_workspace_bytes(B, H, L, d, pa.PATH_BF16), dtype=torch.uint8,
                      device="cuda")
    pa.path_kcache_from_prefill_paged(pre(g["k"]), pre(g["v"]), pre(g["w"]), pre(g["beta"]),
                                      kp, vp, table, kws)
    torch.cuda.synchronize()
    assert torch.equal(_gather(kp, table, L), kc[:, :, :L])
    assert torch.equal(_gather(vp, table, L), vc[:, :, :L])

    fc = fp = None
    if gate:
        fc = pa.fcache_from_prefill(pre(g["log_f"]), T)
        fp = fc.clone()
    ws1 = pa.decode_workspace(B, H, T, d, pa.PATH_BF16, "cuda")
    ws2 = pa.decode_workspace(B, H, T, d, pa.PATH_BF16, "cuda")
    outs = []
    for i in range(n):
        t = L + i
        s = {k: g[k][:, :, t].contiguous() for k in ("q", "k", "v", "w", "beta")}
        lf = g["log_f"][:, :, t].contiguous() if gate else None
        o1 = torch.empty(B, H, d, dtype=torch.bfloat16, device="cuda")
        l1 = torch.empty(B, H, dtype=torch.float32, device="cuda")
        o2, l2 = torch.empty_like(o1), torch.empty_like(l1)
        if gate:
            pa.path_decode_step_gated(kc, vc, fc, s["q"], s["k"], s["v"], s["w"], s["beta"], lf,
                                      o1, l1, t, d ** -0.5, ws1)
        else:
            pa.path_decode_step(kc, vc, s["q"], s["k"], s["v"], s["w"], s["beta"], o1, l1, t,
                                d ** -0.5, ws1)
        pa.path_decode_step_paged(kp, vp, table, s["q"], s["k"], s["v"], s["w"], s["beta"], o2,
                                  l2, t, d ** -0.5, f_cache=fp, log_f_t=lf, workspace=ws2)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2), f"step {t}"
        outs.append(o2.double().cpu().numpy())
    assert torch.equal(_gather(kp, table, L + n), kc[:, :, :L + n])
    assert torch.equal(_gather(vp, table, L + n), vc[:, :, :L + n])
    if gate:
        assert torch.equal(fp, fc)

    ref, _, _, _ = oracle.recurrent(inp.q, inp.k, inp.v, inp.w, inp.beta, inp.log_f, d ** -0.5)
    got = np.stack(outs, axis=2)                  # [B, H, n, d]
    err = np.abs(got - ref[:, :, L:])
    print(f"paged decode vs oracle: max {err.max():.2e} mean {err.mean():.2e}", flush=True)
    assert err.max() <= 2e-2 and err.mean() <= 2e-3


def test_paged_page_outside_pool_is_not_touched():
    """A table entry outside [0, num_blocks) is never dereferenced: the other
    pages are updated as usual and nothing faults (the call's output is then
    not the defined attention and is not checked)."""
    B, H, L, d, page = 1, 2, 128, 64, 64
    inp = generate(B, H, L + 1, d, dtype="bf16", seed=3)
    g = {k: (None if t is None else t.cuda()) for k, t in vars(inp).items()}
    kp = torch.zeros(3, H, page, d, dtype=torch.bfloat16, device="cuda")
    vp = torch.zeros_like(kp)
    table = torch.tensor([[0, 5, 1]], dtype=torch.int32, device="cuda")   # page 5 does not exist
    kws = torch.empty(pa.path_kcache_workspace_bytes(B, H, L, d, pa.PATH_BF16), dtype=torch.uint8,
                      device="cuda")
    pre = lambda t: t[:, :, :L].contiguous()
    pa.path_kcache_from_prefill_paged(pre(g["k"]), pre(g["v"]), pre(g["w"]), pre(g["beta"]),
                                      kp, vp, table, kws)
    ws = pa.decode_workspace(B, H, 3 * page, d, pa.PATH_BF16, "cuda")
    o = torch.empty(B, H, d, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(B, H, dtype=torch.float32, device="cuda")
    s = {k: g[k][:, :, L].contiguous() for k in ("q", "k", "v", "w", "beta")}
    pa.path_decode_step_paged(kp, vp, table, s["q"], s["k"], s["v"], s["w"], s["beta"], o, lse, L,
                              d ** -0.5, workspace=ws)
    torch.cuda.synchronize()
    # slots 0..63 (page 0) were written by the prefill and updated once by step L
    assert torch.all(torch.isfinite(kp[0].float()))
    assert not torch.equal(kp[0], torch.zeros_like(kp[0]))
    # slot L = 128 is slot 0 of page 1 (table entry 2): the new key, unchanged
    assert torch.equal(kp[1][:, 0], g["k"][0, :, L])
    assert torch.equal(kp[2], torch.zeros_like(kp[2]))     # page 2 is in no table entry
