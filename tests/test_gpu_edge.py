"""GPU parity on the method's edge cases, whole output against the oracle.

* Logits far above a row's diagonal maximum, up to overflowing fp32 if they
  were exponentiated unshifted: the online softmax must raise its running
  maximum (the scans' row-sum trigger) and recover from an infinite row
  sum.
* Forget gates that cut the past (log f = -1e4 at single tokens, inside a
  chunk and on a chunk boundary): every earlier key gets weight 0, the key at
  the cut keeps its weight (the product runs over s = j+1 .. i).
* beta at the clip bounds 0.02 and 1.98, and the same w repeated over long
  runs with beta near 2: the region where products of Householder-like
  transitions in bf16 are least stable (PaTH paper summary, Limitations).

Large logits.  The offsets are built so that the arithmetic that makes them
is exact on both sides: every w_t has a zero first coordinate, so every
transition H_t = I - beta_t w_t w_t^T leaves the first coordinate of a vector
unchanged, and q_i, k_j carry their large values in that coordinate only.
The logit of key j then holds the term scale * q_i[0] * k_j[0].  The scan
forms it two ways: in the query's own chunk from the unscaled bf16 query
(exact, then scaled in fp32), in chunks to its left from the query carried
pre-scaled by c2 = scale*log2(e) as a bf16 operand.  A bf16 rounding of
c2 * q_i[0] would shift the second form against the first by up to 2^-9 of
the logit (0.25 at a logit of 128), an error of the test's construction,
which puts a whole large logit into one coordinate, not of the rescaling
under test.  So q_i[0] is chosen such that c2 * q_i[0] lies within 4e-5
(relative) of a bf16 number, and the two forms agree to better than 0.01.
lse is off by at most that rounding of the largest logit; its bound in these
tests is 2e-2 + 2^-8 * max |logit|.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import softmax_attention_ut_amd as pa
from softmax_attention_ut_amd.inputs import generate

pytestmark = pytest.mark.gpu

BF16_MAX, BF16_MEAN = 2e-2, 2e-3


def _run(inp, scale):
    g = {k: (None if t is None else t.cuda()) for k, t in vars(inp).items()}
    out, lse = pa.attention(g["q"], g["k"], g["v"], g["w"], g["beta"], g["log_f"], scale=scale)
    torch.cuda.synchronize()
    return out.double().cpu().numpy(), lse.double().cpu().numpy()


def _compare(inp, scale, what, lse_slack=0.0):
    out, lse = _run(inp, scale)
    ro, rl, _, _ = oracle.recurrent(inp.q, inp.k, inp.v, inp.w, inp.beta, inp.log_f, scale)
    e = np.abs(out - ro)
    el = np.abs(lse - rl)
    where = np.unravel_index(np.argmax(e), e.shape)
    print(f"{what}: out max-abs {e.max():.3e} (at {tuple(int(x) for x in where)}) "
          f"mean-abs {e.mean():.3e}; lse max-abs {el.max():.3e} mean-abs {el.mean():.3e} "
          f"(lse slack {lse_slack:.3e})", flush=True)
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse)), what
    assert e.max() <= BF16_MAX and e.mean() <= BF16_MEAN, (what, e.max(), e.mean())
    assert el.max() <= BF16_MAX + lse_slack and el.mean() <= BF16_MEAN + lse_slack, (
        what, el.max(), el.mean())
    return ro


def _exact_query_coordinate(scale, lo=16.0, hi=64.0):
    """The bf16 value b in [lo, hi) for which fp32(c2 * b), c2 =
    fp32(scale * log2(e)), is nearest (relatively) to a bf16 number."""
    c2 = np.float32(np.float32(scale) * np.float32(math.log2(math.e)))
    best = None
    for b in np.arange(lo, hi, 0.125):
        b = float(torch.tensor(float(b)).to(torch.bfloat16))
        p = np.float32(c2 * np.float32(b))
        r = abs(float(torch.tensor(float(p)).to(torch.bfloat16)) - float(p)) / float(p)
        if best is None or r < best[0]:
            best = (r, b)
    assert best[0] < 4e-5
    return best[1]


def _big_logit_inputs(BH, L, d, gate, seed, scale):
    """Keys with large first coordinates at chosen places; q[..., 0] = b
    (about 32, see _exact_query_coordinate) for every query; w orthogonal to
    the first axis.  Returns (inputs, the largest |q[0] * k[0]|)."""
    inp = generate(1, BH, L, d, dtype="bf16", gate=gate, seed=seed)
    w = inp.w.double()
    w[..., 0] = 0.0
    w /= w.norm(dim=-1, keepdim=True)
    inp.w = w.to(torch.bfloat16)
    big = torch.zeros(L, dtype=torch.float64)

    def put(lo, hi, a):
        big[max(lo, 0):min(hi, L)] = a
    put(64, 96, 32.0)       # keys 0..31 of chunk 1: about 130 natural units (scale 1/8)
    put(160, 192, 8.0)      # keys 32..63 of chunk 2: 32 units
    put(320, 384, 4.0)      # all of chunk 5: 16 units
    put(449, 450, 16.0)     # single keys
    put(700, 701, 32.0)
    put(L - 70, L - 66, 8.0)
    k = inp.k.double()
    k[..., 0] = big
    inp.k = k.to(torch.bfloat16)
    q = inp.q.double()
    b = _exact_query_coordinate(scale)
    q[..., 0] = b
    inp.q = q.to(torch.bfloat16)
    return inp, float(big.abs().max()) * b


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("gate", [False, True])
def test_large_logits_rescale_and_overflow(d, gate):
    """Left-chunk logits up to 128 (fp32 exp overflows above 88) above a
    row's diagonal maximum, on either half of a chunk, in whole chunks and
    single keys; L = 1000 leaves a ragged last chunk."""
    scale = 0.125 if d == 64 else 1 / math.sqrt(128)
    inp, zmax = _big_logit_inputs(4, 1000, d, gate, 60 + d + gate, scale)
    _compare(inp, scale, f"large logits d={d} gate={gate}", lse_slack=2.0 ** -8 * zmax * scale)


def test_large_logits_persistent_pairs():
    """The same construction with B*H = 64 heads of 4096 tokens: 512 pairs of
    query blocks, two per persistent workgroup, dealt by XCD."""
    inp, zmax = _big_logit_inputs(64, 4096, 64, True, 66, 0.125)
    _compare(inp, 0.125, "large logits BH=64 L=4096", lse_slack=2.0 ** -8 * zmax * 0.125)


@pytest.mark.parametrize("d", [64, 128])
def test_gate_cuts_the_past(d):
    """log f = -1e4 at a token inside a chunk, at the first token of a chunk
    and at the last token of one: rows after a cut give weight 0 to every key
    before it; the key at the cut keeps its weight."""
    L = 900
    inp = generate(1, 3, L, d, dtype="bf16", gate=True, seed=70 + d)
    for t in (100, 320, 575, 576, 831):
        inp.log_f[..., t] = -1e4
    ro = _compare(inp, 1 / math.sqrt(d), f"gate cuts d={d}")
    # the oracle's rows right after a cut attend to the suffix only
    suffix = oracle.recurrent(inp.q[:, :, 576:], inp.k[:, :, 576:], inp.v[:, :, 576:],
                              inp.w[:, :, 576:], inp.beta[:, :, 576:], inp.log_f[:, :, 576:],
                              1 / math.sqrt(d))[0]
    np.testing.assert_allclose(ro.reshape(3, L, d)[:, 576:831],
                               suffix.reshape(3, L - 576, d)[:, :255], atol=1e-12)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("mode", ["all_1.98", "all_0.02", "alternating"])
def test_beta_at_clip_bounds(d, mode):
    L = 1000
    inp = generate(1, 4, L, d, dtype="bf16", gate=(mode == "alternating"), seed=80 + d)
    if mode == "all_1.98":
        inp.beta.fill_(1.98)
    elif mode == "all_0.02":
        inp.beta.fill_(0.02)
    else:
        inp.beta[..., 0::2] = 0.02
        inp.beta[..., 1::2] = 1.98
    _compare(inp, 1 / math.sqrt(d), f"beta {mode} d={d}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("run", [8, 4096])
def test_repeated_w_beta_near_two(d, run):
    """The same unit w over runs of `run` tokens (4096: one w per head for
    the whole sequence) with beta = 1.98: long products of one near
    reflection, (1 - 1.98)^n along w."""
    L = 2000
    inp = generate(1, 4, L, d, dtype="bf16", gate=False, seed=90 + d + run)
    w = inp.w.double()
    idx = (torch.arange(L) // run) * run
    w = w[:, :, idx]
    inp.w = w.to(torch.bfloat16).contiguous()
    inp.beta.fill_(1.98)
    _compare(inp, 1 / math.sqrt(d), f"repeated w run={run} d={d}")
