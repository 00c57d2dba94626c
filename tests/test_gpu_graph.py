"""GPU: decode steps captured in a HIP graph (torch.cuda.CUDAGraph on ROCm)
and replayed give the same outputs, lse, key cache and gate cache as the same
steps launched eagerly, bit for bit, on every replay.  Between replays the
caches are restored by eager copies and the stream is synchronised.  Nothing
in the captured launches is a memset (the decode workspace needs no
clearing)."""
import pytest
import torch

import softmax_attention_ut_amd as pa
from softmax_attention_ut_amd.inputs import generate

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("gate", [False, True])
def test_decode_graph_replays_equal_eager(gate):
    B, H, L, n, d = 1, 2, 130, 24, 128
    print(f"graph decode gate={gate}: B={B} H={H} L={L} steps={n} d={d}", flush=True)
    inp = generate(B, H, L + n, d, dtype="bf16", gate=gate, seed=61)
    g = {k: (None if t is None else t.cuda()) for k, t in vars(inp).items()}
    T = L + n
    pre = lambda t: t[:, :, :L].contiguous()
    kc, vc = pa.kcache_from_prefill(pre(g["k"]), pre(g["v"]), pre(g["w"]), pre(g["beta"]), T)
    fc = pa.fcache_from_prefill(pre(g["log_f"]), T) if gate else None
    ws = pa.decode_workspace(B, H, T, d, pa.PATH_BF16, kc.device)
    names = ("q", "k", "v", "w", "beta") + (("log_f",) if gate else ())
    steps = [{k: g[k][:, :, t].contiguous() for k in names} for t in range(L, T)]
    outs = torch.empty(n, B, H, d, dtype=torch.bfloat16, device="cuda")
    lses = torch.empty(n, B, H, dtype=torch.float32, device="cuda")
    kc0, vc0 = kc.clone(), vc.clone()
    fc0 = fc.clone() if gate else None
    torch.cuda.synchronize()

    def run(stream):
        for i, s in enumerate(steps):
            if gate:
                pa.path_decode_step_gated(kc, vc, fc, s["q"], s["k"], s["v"], s["w"], s["beta"],
                                          s["log_f"], outs[i], lses[i], L + i, d ** -0.5, ws, stream)
            else:
                pa.path_decode_step(kc, vc, s["q"], s["k"], s["v"], s["w"], s["beta"], outs[i],
                                    lses[i], L + i, d ** -0.5, ws, stream)

    def restore():
        kc.copy_(kc0)
        vc.copy_(vc0)
        if gate:
            fc.copy_(fc0)
        torch.cuda.synchronize()

    run(torch.cuda.current_stream())
    torch.cuda.synchronize()
    ref = (outs.clone(), lses.clone(), kc.clone(), vc.clone(), fc.clone() if gate else None)

    restore()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            run(side)
    torch.cuda.synchronize()
    for rep in range(3):
        restore()
        outs.zero_()
        lses.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(outs, ref[0]) and torch.equal(lses, ref[1]), f"replay {rep}"
        assert torch.equal(kc, ref[2]) and torch.equal(vc, ref[3]), f"replay {rep} caches"
        if gate:
            assert torch.equal(fc, ref[4]), f"replay {rep} gate cache"
