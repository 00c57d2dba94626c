"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle.

Tolerances: fp32 mode max-abs <= 1e-4; bf16 mode max-abs <= 2e-2 and
mean-abs <= 2e-3 on the outputs (lse is held to the same bounds).  Inputs
come from the seeded generator; the oracle sees exactly the rounded tensors
the GPU receives.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import softmax_attention_ut_amd as pa
from softmax_attention_ut_amd.inputs import CONFIGS, generate, generate_config

pytestmark = pytest.mark.gpu

F32_TOL = 1e-4
BF16_MAX, BF16_MEAN = 2e-2, 2e-3


def _dev(inp):
    return {k: (None if t is None else t.cuda()) for k, t in vars(inp).items()}


def _run_fwd(inp, scale, chunk=0, L=None):
    g = _dev(inp)
    sl = (lambda t: t) if L is None else (lambda t: None if t is None else t[:, :, :L].contiguous())
    out, lse = pa.attention(sl(g["q"]), sl(g["k"]), sl(g["v"]), sl(g["w"]), sl(g["beta"]),
                            sl(g["log_f"]), scale=scale, chunk=chunk)
    torch.cuda.synchronize()
    return out.double().cpu().numpy(), lse.double().cpu().numpy()


def _oracle_full(inp, scale, L=None):
    sl = (lambda t: t) if L is None else (lambda t: None if t is None else t[:, :, :L])
    out, lse, _, _ = oracle.recurrent(sl(inp.q), sl(inp.k), sl(inp.v), sl(inp.w),
                                      sl(inp.beta), sl(inp.log_f), scale)
    return out, lse


def _check_cache(got, ref, n_roundings, what):
    """Cached keys are stored in bf16 and re-rounded (round-to-nearest-even,
    relative error <= 2^-9 per element) every time they are carried or
    updated, so their error grows like sqrt(n_roundings) * 2^-9 in relative
    norm; the bound below is twice 2^-8 * sqrt(n + 1) per key.  (The outputs
    computed from the cache are held to the bf16 output tolerances.)"""
    rel = np.linalg.norm(got - ref, axis=-1) / np.maximum(np.linalg.norm(ref, axis=-1), 1e-30)
    bound = 2.0 * 2.0 ** -8 * math.sqrt(n_roundings + 1)
    print(f"{what}: max rel-norm {rel.max():.3e} mean {rel.mean():.3e} (bound {bound:.3e})",
          flush=True)
    assert np.all(np.isfinite(got)), what
    assert rel.max() <= bound, (what, rel.max(), bound)


def _check(got, ref, dtype, what=""):
    err = np.abs(got - ref)
    mx, mean = float(err.max()), float(err.mean())
    print(f"{what}: max-abs {mx:.3e} mean-abs {mean:.3e}", flush=True)
    assert np.all(np.isfinite(got)), what
    if dtype == "f32":
        assert mx <= F32_TOL, (what, mx)
    else:
        assert mx <= BF16_MAX and mean <= BF16_MEAN, (what, mx, mean)


# ---------------------------------------------------------------------------
# small and medium shapes: every output row against the recurrent oracle
# ---------------------------------------------------------------------------

def test_tiny_f32_config():
    cfg = CONFIGS["tiny_f32"]
    inp = generate_config(cfg)
    out, lse = _run_fwd(inp, cfg.scale, chunk=cfg.chunk)
    ro, rl = _oracle_full(inp, cfg.scale)
    _check(out, ro, "f32", "tiny_f32 out")
    _check(lse, rl, "f32", "tiny_f32 lse")


@pytest.mark.parametrize("chunk", [16, 32, 64])
@pytest.mark.parametrize("gate", [False, True])
def test_f32_chunk_invariance_ragged(chunk, gate):
    """The blockwise result does not depend on the chunk size; L = 203 leaves
    a ragged last chunk for every chunk size."""
    inp = generate(1, 2, 203, 32, dtype="f32", gate=gate, seed=21, clip_beta=False)
    s = 1 / math.sqrt(32)
    out, lse = _run_fwd(inp, s, chunk=chunk)
    ro, rl = _oracle_full(inp, s)
    _check(out, ro, "f32", f"f32 chunk={chunk} gate={gate} out")
    _check(lse, rl, "f32", f"f32 chunk={chunk} gate={gate} lse")


@pytest.mark.parametrize("d,chunk", [(16, 16), (64, 64), (128, 32)])
def test_f32_head_dims(d, chunk):
    inp = generate(2, 1, 150, d, dtype="f32", gate=True, seed=22, clip_beta=False)
    s = 1 / math.sqrt(d)
    out, lse = _run_fwd(inp, s, chunk=chunk)
    ro, rl = _oracle_full(inp, s)
    _check(out, ro, "f32", f"f32 d={d} out")
    _check(lse, rl, "f32", f"f32 d={d} lse")


def test_bf16_L1k_config_full():
    cfg = CONFIGS["bf16_L1k"]
    inp = generate_config(cfg)
    out, lse = _run_fwd(inp, cfg.scale)
    ro, rl = _oracle_full(inp, cfg.scale)
    _check(out, ro, "bf16", "bf16_L1k out")
    _check(lse, rl, "bf16", "bf16_L1k lse")


@pytest.mark.parametrize("L", [1, 5, 64, 65, 127, 129, 777])
@pytest.mark.parametrize("gate", [False, True])
def test_bf16_ragged_lengths(L, gate):
    inp = generate(1, 3, L, 64, dtype="bf16", gate=gate, seed=30 + L)
    s = 0.125
    out, lse = _run_fwd(inp, s)
    ro, rl = _oracle_full(inp, s)
    _check(out, ro, "bf16", f"bf16 L={L} gate={gate} out")
    _check(lse, rl, "bf16", f"bf16 L={L} gate={gate} lse")


@pytest.mark.parametrize("gate", [False, True])
def test_bf16_d128(gate):
    inp = generate(1, 2, 333, 128, dtype="bf16", gate=gate, seed=40)
    s = 1 / math.sqrt(128)
    out, lse = _run_fwd(inp, s)
    ro, rl = _oracle_full(inp, s)
    _check(out, ro, "bf16", f"bf16 d=128 gate={gate} out")
    _check(lse, rl, "bf16", f"bf16 d=128 gate={gate} lse")


def test_bf16_heads_not_multiple_of_8():
    inp = generate(1, 5, 300, 64, dtype="bf16", gate=True, seed=41)
    out, lse = _run_fwd(inp, 0.125)
    ro, rl = _oracle_full(inp, 0.125)
    _check(out, ro, "bf16", "bf16 BH=5 out")


def test_bf16_odd_query_block_count():
    """N = 11 chunks: three blocks of four query chunks per head (24 blocks,
    fewer than the CUs: one block per workgroup)."""
    inp = generate(2, 4, 700, 64, dtype="bf16", gate=True, seed=45)
    out, lse = _run_fwd(inp, 0.125)
    ro, rl = _oracle_full(inp, 0.125)
    _check(out, ro, "bf16", "bf16 BH=8 L=700 out")
    _check(lse, rl, "bf16", "bf16 BH=8 L=700 lse")


def test_bf16_odd_query_block_count_paired():
    """N = 11 chunks and B*H = 96: 288 query blocks, more than the CUs, so
    the blocks are dealt in pairs of equal weight, with the lone middle block
    of each head (odd block count) dealt on its own."""
    inp = generate(4, 24, 700, 64, dtype="bf16", gate=True, seed=47)
    out, lse = _run_fwd(inp, 0.125)
    ro, rl = _oracle_full(inp, 0.125)
    _check(out, ro, "bf16", "bf16 BH=96 L=700 out")
    _check(lse, rl, "bf16", "bf16 BH=96 L=700 lse")


def test_bf16_more_block_pairs_than_workgroups():
    """B*H = 9 heads of 16384 tokens: 9 * 32 pairs of query blocks, more than
    one per CU, dealt without the per-XCD grouping (9 is not a multiple of 8).
    Sampled rows of the first, a middle and the last head."""
    L, s = 16384, 0.125
    inp = generate(1, 9, L, 64, dtype="bf16", gate=True, seed=46)
    out, lse = _run_fwd(inp, s)
    rng = np.random.default_rng(146)
    rows = _sample_rows(L, rng)
    heads = [0, 4, 8]
    hi = np.repeat(heads, len(rows))
    ri = np.tile(rows, len(heads))
    ro, rl, _, _ = oracle.rows(inp.q, inp.k, inp.v, inp.w, inp.beta, inp.log_f, s, hi, ri)
    _check(out.reshape(-1, L, 64)[hi, ri], ro, "bf16", f"BH=9 L=16k sampled out ({len(hi)} rows)")
    _check(lse.reshape(-1, L)[hi, ri], rl, "bf16", "BH=9 L=16k sampled lse")


def test_bf16_beta_zero_is_causal_attention():
    inp = generate(1, 2, 256, 64, dtype="bf16", gate=False, seed=42)
    inp.beta.zero_()
    out, _ = _run_fwd(inp, 0.125)
    q, k, v = (t.float() for t in (inp.q, inp.k, inp.v))
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True, scale=0.125)
    _check(out, ref.double().numpy(), "bf16", "beta=0 vs causal SDPA (fp32 CPU)")


def test_bf16_first_transition_never_enters():
    """H_0, beta_0 and f_0 do not enter any logit: perturbing them leaves the
    GPU result bit-identical."""
    inp = generate(1, 2, 200, 64, dtype="bf16", gate=True, seed=43)
    a, la = _run_fwd(inp, 0.125)
    inp.w[:, :, 0] = inp.w[:, :, 0].flip(-1)
    inp.beta[:, :, 0] = 1.9
    inp.log_f[:, :, 0] = -30.0
    b, lb = _run_fwd(inp, 0.125)
    np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(la, lb)


# ---------------------------------------------------------------------------
# full-size configurations: sampled rows against the per-row oracle
# ---------------------------------------------------------------------------

def _sample_rows(L, rng, n_extra=12):
    base = {0, 1, 63, 64, 65, 127, 128, L // 2, L - 65, L - 64, L - 2, L - 1}
    base |= set(rng.integers(0, L, n_extra).tolist())
    return sorted(r for r in base if 0 <= r < L)


def _check_sampled(cfg, inp, out, lse, heads, L):
    rng = np.random.default_rng(cfg.seed + 100)
    rows = _sample_rows(L, rng)
    hi = np.repeat(heads, len(rows))
    ri = np.tile(rows, len(heads))
    sl = lambda t: None if t is None else t[:, :, :L]
    ro, rl, _, _ = oracle.rows(sl(inp.q), sl(inp.k), sl(inp.v), sl(inp.w), sl(inp.beta),
                               sl(inp.log_f), cfg.scale, hi, ri)
    d = inp.q.shape[-1]
    go = out.reshape(-1, L, d)[hi, ri]
    gl = lse.reshape(-1, L)[hi, ri]
    _check(go, ro, "bf16", f"{cfg.name} sampled out ({len(hi)} rows)")
    _check(gl, rl, "bf16", f"{cfg.name} sampled lse")


@pytest.mark.parametrize("name", ["fox_L4k", "fox_L16k"])
def test_full_size_sampled(name):
    cfg = CONFIGS[name]
    inp = generate_config(cfg)
    out, lse = _run_fwd(inp, cfg.scale)
    BH = cfg.B * cfg.H
    heads = sorted({0, 1, 7, BH // 2, BH - 1})
    _check_sampled(cfg, inp, out, lse, heads, cfg.L)


def test_d128_prefill_kcache_and_decode():
    """The d=128 workload: prefill (sampled rows), the transformed key cache
    after the prefill (sampled keys) and 256 decode steps (every step, sampled
    heads), each against the oracle."""
    cfg = CONFIGS["d128_L8k_decode"]
    inp = generate_config(cfg)
    L, T = cfg.L, cfg.L_total
    out, lse = _run_fwd(inp, cfg.scale, L=L)
    BH = cfg.B * cfg.H
    heads = [0, 5, BH - 1]
    _check_sampled(cfg, inp, out, lse, heads, L)
    del out, lse
    _decode_and_check(inp, cfg.scale, L, T, heads, key_samples=64)


def test_fox_d128_prefill_kcache_and_gated_decode():
    """The PaTH-FoX variant of the d=128 workload (B=2, H=32, L=8192 + 256
    steps, forget gate): the gated prefill (sampled rows), the key cache, the
    gate cache and 256 gated decode steps (sampled heads) against the oracle."""
    cfg = CONFIGS["fox_d128_L8k_decode"]
    inp = generate_config(cfg)
    L, T = cfg.L, cfg.L_total
    out, lse = _run_fwd(inp, cfg.scale, L=L)
    BH = cfg.B * cfg.H
    heads = [0, 33, BH - 1]
    _check_sampled(cfg, inp, out, lse, heads, L)
    del out, lse
    _decode_and_check(inp, cfg.scale, L, T, heads, key_samples=64)


def _decode_and_check(inp, scale, L, T, heads, key_samples):
    g = _dev(inp)
    B, H, _, d = inp.q.shape
    gated = inp.log_f is not None
    pre = lambda t: t[:, :, :L].contiguous()
    kc, vc = pa.kcache_from_prefill(pre(g["k"]), pre(g["v"]), pre(g["w"]), pre(g["beta"]), T)
    fc = pa.fcache_from_prefill(pre(g["log_f"]), T) if gated else None
    torch.cuda.synchronize()
    rng = np.random.default_rng(7)
    keys = sorted(set(rng.integers(0, L, key_samples).tolist()) | {0, L - 1, max(L - 64, 0)})
    hi = np.repeat(heads, len(keys))
    ki = np.tile(keys, len(heads))
    ref_k = oracle.transported_keys(inp.k, inp.w, inp.beta, L - 1, hi, ki)
    got_k = kc.double().cpu().numpy().reshape(B * H, T, d)[hi, ki]
    n_chunks = (L + 63) // 64
    _check_cache(got_k, ref_k, n_chunks + 2, "kcache after prefill")
    ws = pa.decode_workspace(B, H, T, d, pa.PATH_BF16, kc.device)
    outs, lses = [], []
    for t in range(L, T):
        o = torch.empty(B, H, d, dtype=kc.dtype, device=kc.device)
        ls = torch.empty(B, H, dtype=torch.float32, device=kc.device)
        step_in = [g[n][:, :, t].contiguous() for n in ("q", "k", "v", "w", "beta")]
        if gated:
            pa.path_decode_step_gated(kc, vc, fc, *step_in, g["log_f"][:, :, t].contiguous(), o, ls,
                                      t, scale, ws)
        else:
            pa.path_decode_step(kc, vc, *step_in, o, ls, t, scale, ws)
        outs.append(o)
        lses.append(ls)
    torch.cuda.synchronize()
    got = torch.stack(outs, 2).double().cpu().numpy().reshape(B * H, T - L, d)
    gotl = torch.stack(lses, 2).double().cpu().numpy().reshape(B * H, T - L)
    rows = np.arange(L, T)
    hi = np.repeat(heads, len(rows))
    ri = np.tile(rows, len(heads))
    ro, rl, _, _ = oracle.rows(inp.q, inp.k, inp.v, inp.w, inp.beta, inp.log_f, scale, hi, ri)
    _check(got[hi, ri - L], ro, "bf16", f"decode {T - L} steps out")
    if gated:   # the gate cache holds the prefix sums of log f (fp32)
        ref_f = np.cumsum(inp.log_f.double().numpy().reshape(B * H, -1)[:, :T], axis=1)
        got_f = fc.double().cpu().numpy().reshape(B * H, T)
        err = np.max(np.abs(got_f - ref_f) / np.maximum(1.0, np.abs(ref_f)))
        print(f"gate cache: max rel err {err:.2e}")
        assert err < 1e-5
    _check(gotl[hi, ri - L], rl, "bf16", f"decode {T - L} steps lse")
    # the cache after the last step against the oracle's in-place updated keys
    keys = sorted(set(rng.integers(0, T, key_samples).tolist()) | {0, T - 1})
    hi = np.repeat(heads, len(keys))
    ki = np.tile(keys, len(heads))
    ref_k = oracle.transported_keys(inp.k, inp.w, inp.beta, T - 1, hi, ki)
    got_k = kc.double().cpu().numpy().reshape(B * H, T, d)[hi, ki]
    _check_cache(got_k, ref_k, n_chunks + 2 + (T - L), "kcache after decode")


@pytest.mark.parametrize("d", [64, 128])
def test_decode_small_ragged(d):
    inp = generate(1, 3, 231, d, dtype="bf16", gate=False, seed=50)
    _decode_and_check(inp, 1 / math.sqrt(d), 170, 231, [0, 1, 2], key_samples=40)


@pytest.mark.parametrize("d", [64, 128])
def test_decode_gated(d):
    # PaTH-FoX decode: the gate cache from the prefill, then gated steps
    inp = generate(1, 3, 231, d, dtype="bf16", gate=True, seed=53)
    _decode_and_check(inp, 1 / math.sqrt(d), 170, 231, [0, 1, 2], key_samples=30)


def test_decode_short_prefix():
    # t from 5 to 69: one split of 64 keys, then two (the split size is a
    # multiple of 64 keys)
    inp = generate(1, 2, 70, 64, dtype="bf16", gate=False, seed=52)
    _decode_and_check(inp, 0.125, 5, 70, [0, 1], key_samples=10)
