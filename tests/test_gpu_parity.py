"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle.

Tolerances: fp32 mode max-abs <= 1e-4; bf16 mode max-abs <= 2e-2 and
mean-abs <= 2e-3 on the outputs (lse is held to the same bounds).  Inputs
come from the seeded generator; the oracle sees exactly the rounded tensors
the GPU receives.
"""
import concurrent.futures
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


def _check_cache(got, ref, k_in, what, n_roundings):
    """Cached (bf16) keys against the oracle's fp64 transported keys, per key,
    as the error norm over the norm of the key as it entered (k_in).  No
    transition increases a norm (the eigenvalues of I - beta w w^T are 1 and
    1 - beta, in [-1, 1] for beta in [0, 2]), so every intermediate value of a
    key, and of any product applied to it, is bounded by its input norm, and
    each bf16 rounding on its path adds at most 2^-9 of that.  Such errors add
    up like a random walk: the bound is 2^-8 * sqrt(n + 1) for n roundings,
    twice the walk's size.  A key's logit error is scale * |q| times this
    error, so the bound is what the outputs' tolerance can absorb; the outputs
    computed from the cache are checked against the oracle separately.  The
    error relative to the key's current norm is printed too: keys carried
    through thousands of transitions shrink by orders of magnitude, and the
    same absolute error is then a large relative one."""
    err = np.linalg.norm(got - ref, axis=-1)
    rel_in = err / np.maximum(np.linalg.norm(k_in, axis=-1), 1e-30)
    rel_cur = err / np.maximum(np.linalg.norm(ref, axis=-1), 1e-30)
    bound = 2.0 ** -8 * math.sqrt(n_roundings + 1)
    print(f"{what}: error / input norm max {rel_in.max():.3e} mean {rel_in.mean():.3e} "
          f"(bound {bound:.3e}); error / current norm max {rel_cur.max():.3e} "
          f"median {np.median(rel_cur):.3e}", flush=True)
    assert np.all(np.isfinite(got)), what
    assert rel_in.max() <= bound, (what, rel_in.max(), bound)


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
@pytest.mark.parametrize("d", [64, 128])
def test_bf16_ragged_lengths(L, gate, d):
    """One chunk of one token up to thirteen chunks with a ragged last one:
    the scan's single-chunk start (no left chunk), a last chunk of one key,
    and blocks of fewer than four query chunks."""
    inp = generate(1, 3, L, d, dtype="bf16", gate=gate, seed=30 + L)
    s = 1 / math.sqrt(d)
    out, lse = _run_fwd(inp, s)
    ro, rl = _oracle_full(inp, s)
    _check(out, ro, "bf16", f"bf16 d={d} L={L} gate={gate} out")
    _check(lse, rl, "bf16", f"bf16 d={d} L={L} gate={gate} lse")


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


@pytest.mark.parametrize("d", [64, 128])
def test_bf16_odd_query_block_count_paired(d):
    """N = 11 chunks and B*H = 96: 288 query blocks, more than the CUs, so
    the blocks are dealt in pairs of equal weight (each workgroup's heads in
    one XCD group), with the lone middle block of each head (odd block count)
    dealt on its own; L = 700 leaves a ragged last chunk."""
    inp = generate(4, 24, 700, d, dtype="bf16", gate=True, seed=47)
    s = 1 / math.sqrt(d)
    out, lse = _run_fwd(inp, s)
    ro, rl = _oracle_full(inp, s)
    _check(out, ro, "bf16", f"bf16 d={d} BH=96 L=700 out")
    _check(lse, rl, "bf16", f"bf16 d={d} BH=96 L=700 lse")


@pytest.mark.parametrize("d", [64, 128])
def test_bf16_paired_heads_not_multiple_of_8(d):
    """B*H = 90 (not a multiple of 8) and N = 11: 270 query blocks, dealt in
    pairs round-robin without the XCD grouping of heads."""
    inp = generate(2, 45, 700, d, dtype="bf16", gate=False, seed=48)
    s = 1 / math.sqrt(d)
    out, lse = _run_fwd(inp, s)
    ro, rl = _oracle_full(inp, s)
    _check(out, ro, "bf16", f"bf16 d={d} BH=90 L=700 out")
    _check(lse, rl, "bf16", f"bf16 d={d} BH=90 L=700 lse")


def test_bf16_beta_zero_is_causal_attention():
    inp = generate(1, 2, 256, 64, dtype="bf16", gate=False, seed=42)
    inp.beta.zero_()
    out, _ = _run_fwd(inp, 0.125)
    q, k, v = (t.float() for t in (inp.q, inp.k, inp.v))
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True, scale=0.125)
    _check(out, ref.double().numpy(), "bf16", "beta=0 vs causal SDPA (fp32 CPU)")


@pytest.mark.parametrize("d", [64, 128])
def test_bf16_first_transition_never_enters(d):
    """H_0, beta_0 and f_0 do not enter any logit: perturbing them leaves the
    GPU result bit-identical."""
    inp = generate(1, 2, 200, d, dtype="bf16", gate=True, seed=43)
    s = 1 / math.sqrt(d)
    a, la = _run_fwd(inp, s)
    inp.w[:, :, 0] = inp.w[:, :, 0].flip(-1)
    inp.beta[:, :, 0] = 1.9
    inp.log_f[:, :, 0] = -30.0
    b, lb = _run_fwd(inp, s)
    np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(la, lb)


# ---------------------------------------------------------------------------
# full-size configurations: every head and every row against the recurrent
# oracle (run on a host thread while the GPU works; ctypes releases the GIL)
# ---------------------------------------------------------------------------

_POOL = concurrent.futures.ThreadPoolExecutor(max_workers=1)


def _oracle_bg(inp, scale, Lcache=0):
    return _POOL.submit(oracle.recurrent, inp.q, inp.k, inp.v, inp.w, inp.beta, inp.log_f,
                        scale, Lcache=Lcache)


@pytest.mark.parametrize("name", ["fox_L4k", "fox_L16k"])
def test_full_size_whole_output(name):
    """The 4k PaTH-FoX workload (B=8, H=24: every head, so every XCD group
    and every persistent workgroup's pairs) and the 16k one (B=1, H=16), the
    whole out and lse against the oracle."""
    cfg = CONFIGS[name]
    inp = generate_config(cfg)
    fut = _oracle_bg(inp, cfg.scale)
    out, lse = _run_fwd(inp, cfg.scale)
    ro, rl, _, used = fut.result()
    print(f"{name}: oracle on {used} threads", flush=True)
    _check(out, ro, "bf16", f"{name} whole out ({out.size} values)")
    _check(lse, rl, "bf16", f"{name} whole lse")


def test_bf16_more_block_pairs_than_workgroups():
    """B*H = 9 heads of 16384 tokens: 9 * 32 pairs of query blocks, more than
    one per CU, dealt without the per-XCD grouping (9 is not a multiple of 8).
    Whole output."""
    L, s = 16384, 0.125
    inp = generate(1, 9, L, 64, dtype="bf16", gate=True, seed=46)
    fut = _oracle_bg(inp, s)
    out, lse = _run_fwd(inp, s)
    ro, rl, _, _ = fut.result()
    _check(out, ro, "bf16", "BH=9 L=16k whole out")
    _check(lse, rl, "bf16", "BH=9 L=16k whole lse")


def _prefill_decode_whole(cfg):
    """One oracle recurrence over all L + 256 tokens of every head gives the
    prefill rows, the 256 decode rows and the key cache after the prefill;
    the GPU runs the prefill forward, the key-cache hand-off and the 256
    decode steps."""
    inp = generate_config(cfg)
    L, T = cfg.L, cfg.L_total
    fut = _oracle_bg(inp, cfg.scale, Lcache=L)
    out, lse = _run_fwd(inp, cfg.scale, L=L)
    dec = _decode_gpu(inp, cfg.scale, L, T)
    kf, vf = _kcache_from_forward(inp, cfg.scale, L, T)
    ro, rl, rkc, used = fut.result()
    BH, d = cfg.B * cfg.H, cfg.d
    ro, rl = ro.reshape(BH, T, d), rl.reshape(BH, T)
    print(f"{cfg.name}: oracle on {used} threads", flush=True)
    _check_cache(kf[:, :L], rkc.reshape(BH, L, d), inp.k.double().numpy().reshape(BH, -1, d)[:, :L],
                 f"{cfg.name} kcache from the forward's workspace (every key)", (L + 63) // 64 + 2)
    assert np.array_equal(vf[:, :L], dec["vc_pre"])
    del kf, vf
    _check(out.reshape(BH, L, d), ro[:, :L], "bf16", f"{cfg.name} prefill whole out")
    _check(lse.reshape(BH, L), rl[:, :L], "bf16", f"{cfg.name} prefill whole lse")
    del out, lse
    _check_decode(inp, cfg.scale, L, T, dec, ro[:, L:], rl[:, L:], rkc.reshape(BH, L, d),
                  key_samples=64)


def test_d128_prefill_kcache_and_decode():
    """The d=128 workload (B=2, H=32, L=8192, then 256 decode steps): the
    prefill, the whole key cache after it, every decode step of every head."""
    _prefill_decode_whole(CONFIGS["d128_L8k_decode"])


def test_fox_d128_prefill_kcache_and_gated_decode():
    """The PaTH-FoX variant of the d=128 workload (forget gate): gated
    prefill, key cache, gate cache and 256 gated decode steps, whole."""
    _prefill_decode_whole(CONFIGS["fox_d128_L8k_decode"])


def _kcache_from_forward(inp, scale, L, T):
    """A bf16 forward over the first L tokens with an explicit workspace, then
    path_kcache_from_forward from that workspace, which must leave it as it
    was.  Returns the key and value caches (host, [B*H][T][d])."""
    g = _dev(inp)
    B, H, _, d = inp.q.shape
    pre = lambda t: None if t is None else t[:, :, :L].contiguous()
    n = pa.path_attn_fwd_workspace_bytes(B, H, L, d, pa.PATH_BF16, 0)
    fws = torch.empty(n, dtype=torch.uint8, device="cuda")
    out = torch.empty(B, H, L, d, dtype=g["q"].dtype, device="cuda")
    lse = torch.empty(B, H, L, dtype=torch.float32, device="cuda")
    pa.path_attn_fwd(pre(g["q"]), pre(g["k"]), pre(g["v"]), pre(g["w"]), pre(g["beta"]),
                     pre(g["log_f"]), out, lse, scale, 0, fws)
    fws_before = fws.clone()
    kc, vc = pa.kcache_from_forward(fws, pre(g["v"]), T)
    torch.cuda.synchronize()
    assert torch.equal(fws, fws_before), "the forward's workspace was modified"
    return (kc.double().cpu().numpy().reshape(B * H, T, d),
            vc.double().cpu().numpy().reshape(B * H, T, d))


@pytest.mark.parametrize("L", [64, 700, 1100])
@pytest.mark.parametrize("gate", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_kcache_from_forward_workspace(L, gate, d):
    """path_kcache_from_forward after a bf16 forward on the same inputs: every
    cached key against the oracle's transported keys (the bound of the
    prefill hand-off), the values copied exactly, the slots past L untouched,
    and the keys of path_kcache_from_prefill for comparison.  L = 1100: 18
    chunks, a ragged last chunk and a partial last group of eight chunks."""
    B, H, T = 1, 3, L + 40
    inp = generate(B, H, L, d, dtype="bf16", gate=gate, seed=50 + L + d)
    BH = B * H
    kf, vf = _kcache_from_forward(inp, 1 / math.sqrt(d), L, T)
    g = _dev(inp)
    kcp, _ = pa.kcache_from_prefill(g["k"], g["v"], g["w"], g["beta"], T)
    kp = kcp.double().cpu().numpy().reshape(BH, T, d)
    hi = np.repeat(np.arange(BH), L)
    ki = np.tile(np.arange(L), BH)
    ref = oracle.transported_keys(inp.k, inp.w, inp.beta, L - 1, hi, ki).reshape(BH, L, d)
    k_in = inp.k.double().numpy().reshape(BH, L, d)
    n_chunks = (L + 63) // 64
    _check_cache(kf[:, :L], ref, k_in, f"kcache from the forward, d={d} L={L} gate={gate}",
                 n_chunks + 2)
    _check_cache(kp[:, :L], ref, k_in, f"kcache from the prefill, d={d} L={L} gate={gate}",
                 n_chunks + 2)
    assert np.array_equal(vf[:, :L], inp.v.double().numpy().reshape(BH, L, d))
    assert not np.any(kf[:, L:]) and not np.any(vf[:, L:])


def _decode_gpu(inp, scale, L, T):
    """Prefill hand-off (key, value and gate caches) then decode steps
    t = L .. T-1 on the GPU.  Returns the caches after the hand-off (host
    copies), the per-step outputs and lse, and the caches after the last
    step."""
    g = _dev(inp)
    B, H, _, d = inp.q.shape
    gated = inp.log_f is not None
    pre = lambda t: t[:, :, :L].contiguous()
    kc, vc = pa.kcache_from_prefill(pre(g["k"]), pre(g["v"]), pre(g["w"]), pre(g["beta"]), T)
    fc = pa.fcache_from_prefill(pre(g["log_f"]), T) if gated else None
    torch.cuda.synchronize()
    kc_pre = kc.double().cpu().numpy().reshape(B * H, T, d)[:, :L]
    vc_pre = vc.double().cpu().numpy().reshape(B * H, T, d)[:, :L]
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
    return {"kc_pre": kc_pre, "vc_pre": vc_pre, "out": got, "lse": gotl,
            "kc": kc.double().cpu().numpy().reshape(B * H, T, d),
            "fc": None if fc is None else fc.double().cpu().numpy().reshape(B * H, T)}


def _check_decode(inp, scale, L, T, dec, ro, rl, rkc, key_samples):
    """ro, rl: the oracle's rows L .. T-1 of every head; rkc: the oracle's
    key cache after the prefill, every key of every head.  Every check runs
    and prints before the first failure is raised."""
    B, H, _, d = inp.q.shape
    BH = B * H
    n_chunks = (L + 63) // 64
    k_in = inp.k.double().numpy().reshape(BH, -1, d)
    failures = []

    def run(fn, *args):
        try:
            fn(*args)
        except AssertionError as e:
            failures.append(e)
    run(_check, dec["out"], ro, "bf16", f"decode {T - L} steps out (every head)")
    run(_check, dec["lse"], rl, "bf16", f"decode {T - L} steps lse (every head)")
    run(_check_cache, dec["kc_pre"], rkc, k_in[:, :L], "kcache after prefill (every key)",
        n_chunks + 2)
    np.testing.assert_array_equal(dec["vc_pre"], inp.v.double().numpy().reshape(BH, -1, d)[:, :L])
    if dec["fc"] is not None:   # the gate cache holds the prefix sums of log f (fp32)
        ref_f = np.cumsum(inp.log_f.double().numpy().reshape(BH, -1)[:, :T], axis=1)
        err = np.max(np.abs(dec["fc"] - ref_f) / np.maximum(1.0, np.abs(ref_f)))
        print(f"gate cache: max rel err {err:.2e}")
        assert err < 1e-5
    # the cache after the last step against the oracle's in-place updated keys
    rng = np.random.default_rng(7)
    keys = sorted(set(rng.integers(0, T, key_samples).tolist()) | {0, L - 1, L, T - 1})
    hi = np.repeat(np.arange(BH), len(keys))
    ki = np.tile(keys, BH)
    ref_k = oracle.transported_keys(inp.k, inp.w, inp.beta, T - 1, hi, ki)
    run(_check_cache, dec["kc"][hi, ki], ref_k, k_in[hi, ki],
        f"kcache after decode ({len(hi)} keys)", n_chunks + 2 + (T - L))
    if failures:
        raise failures[0]


def _decode_and_check(inp, scale, L, T, key_samples=40):
    """Small cases: the oracle recurrence over all T tokens, then every
    decode row, the whole prefill key cache and sampled final keys."""
    fut = _oracle_bg(inp, scale, Lcache=L)
    dec = _decode_gpu(inp, scale, L, T)
    ro, rl, rkc, _ = fut.result()
    B, H, _, d = inp.q.shape
    ro, rl = ro.reshape(B * H, T, d), rl.reshape(B * H, T)
    _check_decode(inp, scale, L, T, dec, ro[:, L:], rl[:, L:], rkc.reshape(B * H, L, d),
                  key_samples)


@pytest.mark.parametrize("d", [64, 128])
def test_decode_small_ragged(d):
    inp = generate(1, 3, 231, d, dtype="bf16", gate=False, seed=50)
    _decode_and_check(inp, 1 / math.sqrt(d), 170, 231, key_samples=40)


@pytest.mark.parametrize("d", [64, 128])
def test_decode_gated(d):
    # PaTH-FoX decode: the gate cache from the prefill, then gated steps
    inp = generate(1, 3, 231, d, dtype="bf16", gate=True, seed=53)
    _decode_and_check(inp, 1 / math.sqrt(d), 170, 231, key_samples=30)


def test_decode_short_prefix():
    # t from 5 to 69: one split of 64 keys, then two (the split size is a
    # multiple of 64 keys)
    inp = generate(1, 2, 70, 64, dtype="bf16", gate=False, seed=52)
    _decode_and_check(inp, 0.125, 5, 70, key_samples=10)
