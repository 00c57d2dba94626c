"""GPU parity of the transition-parameter kernel (path_transition_prep,
through the C ABI) against the fp64 oracle ``oracle.transition_prep``.

Tolerances, from the arithmetic: every product accumulates in fp32 and the
low-rank intermediate enters the second product as a bf16 (high, low) pair,
so before the final rounding w is within ~1e-5 of the fp64 value (w has unit
norm); rounding to bf16 (nearest even) then adds at most 2^-8 |w| (half an
ulp of 8 significant bits).  The bound is 2^-8 |w_ref| + 1e-4 per element.
beta is fp32: within 1e-5.  The oracle sees exactly the bf16/fp32 tensors
the GPU receives.
"""
import numpy as np
import pytest
import torch

import oracle
import softmax_attention_ut_amd as pa
from softmax_attention_ut_amd.inputs import TRANSITION_CONFIGS, generate_transition

pytestmark = pytest.mark.gpu


def _run(inp, d):
    g = {k: t.cuda() for k, t in vars(inp).items()}
    w, beta = pa.transition_prep(g["x"], g["w_down"], g["w_up"], g["conv"], g["u"], g["b"], d)
    torch.cuda.synchronize()
    return w.double().cpu().numpy(), beta.double().cpu().numpy()


def _ref(inp, d):
    return oracle.transition_prep(inp.x.double().numpy(), inp.w_down.double().numpy(),
                                  inp.w_up.double().numpy(), inp.conv.double().numpy(),
                                  inp.u.double().numpy(), inp.b.double().numpy(), d)


def _check(w, beta, w_ref, beta_ref, what):
    err = np.abs(w - w_ref)
    bound = 2.0 ** -8 * np.abs(w_ref) + 1e-4
    berr = np.abs(beta - beta_ref)
    print(f"{what}: w max-abs {err.max():.2e} mean {err.mean():.2e}; beta max-abs "
          f"{berr.max():.2e}", flush=True)
    assert np.all(np.isfinite(w)) and np.all(np.isfinite(beta)), what
    assert np.all(err <= bound), (what, float((err - bound).max()))
    assert berr.max() <= 1e-5, what
    # the bf16-mode output tolerances hold with a wide margin
    assert err.max() <= 2e-2 and err.mean() <= 2e-3, what


# (B, L, Dm, r, H, d): ragged lengths across several 62-token tiles, a single
# token, each supported (d, r), H not a multiple of the four waves
CASES = [
    (2, 200, 256, 64, 4, 64),
    (1, 1, 128, 32, 1, 64),
    (1, 62, 128, 64, 5, 64),
    (1, 63, 256, 32, 3, 64),
    (2, 125, 384, 64, 3, 128),
    (1, 190, 128, 32, 6, 128),
    (1, 300, 512, 64, 64, 64),      # r + H = 128
    (1, 1000, 4096, 64, 32, 128),   # the width of 32 heads of 128 (32 column steps)
]


@pytest.mark.parametrize("B,L,Dm,r,H,d", CASES)
def test_transition_small(B, L, Dm, r, H, d):
    print(f"transition B={B} L={L} Dm={Dm} r={r} H={H} d={d}", flush=True)
    inp = generate_transition(B, L, Dm, r, H, d, seed=100 + L)
    w, beta = _run(inp, d)
    w_ref, beta_ref = _ref(inp, d)
    _check(w, beta, w_ref, beta_ref, f"L={L} d={d} r={r}")
    nrm = np.linalg.norm(w, axis=-1)
    assert np.all(np.abs(nrm - 1.0) <= 2e-2)          # unit rows after bf16 rounding


def test_transition_zero_head_stays_zero():
    """A head whose map is zero has c_t = 0: its w must be exactly 0 (no
    division by zero), while the other heads are unaffected."""
    B, L, Dm, r, H, d = 1, 100, 256, 64, 3, 64
    inp = generate_transition(B, L, Dm, r, H, d, seed=7)
    inp.w_up[d:2 * d] = 0
    w, beta = _run(inp, d)
    w_ref, beta_ref = _ref(inp, d)
    assert np.all(w[:, 1] == 0.0)
    _check(w, beta, w_ref, beta_ref, "zero head")


def test_transition_full_size():
    """The ~760M layer shape at 4K tokens (the benchmarked launch), every
    output compared with the oracle."""
    cfg = TRANSITION_CONFIGS["transition_L4k"]
    print(f"transition full size {cfg}", flush=True)
    inp = generate_transition(cfg.B, cfg.L, cfg.Dm, cfg.r, cfg.H, cfg.d, seed=cfg.seed)
    w, beta = _run(inp, cfg.d)
    w_ref, beta_ref = _ref(inp, cfg.d)
    _check(w, beta, w_ref, beta_ref, cfg.name)


@pytest.mark.parametrize("gate", [False, True])
def test_transition_then_attention(gate):
    """The layer's chain: w and beta from path_transition_prep feed
    path_attn_fwd directly (bf16 w, fp32 beta, the layouts both use).  The
    oracle runs its own chain from the same layer input and weights:
    oracle.transition_prep in fp64, w rounded to bf16 (nearest even) and
    beta to fp32 as the attention's inputs, then the recurrent forward.  The
    two chains may round a w element differently by an ulp; the outputs are
    held to the bf16 tolerances."""
    B, L, Dm, r, H, d = 2, 300, 512, 64, 4, 64
    inp = generate_transition(B, L, Dm, r, H, d, seed=71)
    rng = np.random.default_rng(72)
    shape = (B, H, L, d)
    q, k, v = (torch.from_numpy(rng.standard_normal(shape)).to(torch.bfloat16) for _ in range(3))
    log_f = (torch.from_numpy(-np.logaddexp(0.0, -(3.0 + rng.standard_normal((B, H, L)))))
             .to(torch.float32) if gate else None)
    gw, gbeta = (t.cuda() for t in _run_gpu_params(inp, d))
    out, lse = pa.attention(q.cuda(), k.cuda(), v.cuda(), gw, gbeta,
                            None if log_f is None else log_f.cuda(), scale=d ** -0.5)
    torch.cuda.synchronize()
    w_ref, beta_ref = _ref(inp, d)
    w_in = torch.from_numpy(w_ref).to(torch.bfloat16)
    beta_in = torch.from_numpy(beta_ref).to(torch.float32)
    ro, rl, _, _ = oracle.recurrent(q, k, v, w_in, beta_in, log_f, d ** -0.5)
    err = np.abs(out.double().cpu().numpy() - ro)
    lerr = np.abs(lse.double().cpu().numpy() - rl)
    print(f"transition -> attention gate={gate}: out max {err.max():.2e} mean {err.mean():.2e}; "
          f"lse max {lerr.max():.2e}", flush=True)
    assert err.max() <= 2e-2 and err.mean() <= 2e-3
    assert lerr.max() <= 2e-2 and lerr.mean() <= 2e-3


def _run_gpu_params(inp, d):
    g = {k: t.cuda() for k, t in vars(inp).items()}
    return pa.transition_prep(g["x"], g["w_down"], g["w_up"], g["conv"], g["u"], g["b"], d)
