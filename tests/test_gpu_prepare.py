"""GPU unit tests of the prepare stage's per-chunk quantities (the UT
transform, Chinese notes, training strategy) against fp64 numpy evaluations
of the pages' formulas, read straight out of the forward's workspace.

The workspace layout is the library's internal one (path_internal.h,
plan_workspace): these tests replicate its section order to find the tiles,
and the k-slot permutation permk of the transposed tiles.  Checked, per head
and chunk, on the bf16-rounded inputs the GPU receives:
  K~   every key carried to its chunk end, H_end ... H_{j+1} k_j
       (oracle.transported_keys);
  M^T (forward, d = 64 and 128), from T^{-1} = (I + strictLower(D W
       W^T))^{-1} D (oracle.ut_tinv): I - M = I - W^T U = oracle.ut_product;
  U = T^{-1} W and Y = T^{-1} strictLower(W K^T) (the backward's prepare
       stage, read back from its workspace after path_attn_bwd, where they
       are row-major tiles);
  V^T  (d = 128) an exact copy;
  the chunk-local gate sums loc_j = -sum_{s>j}^{end} log2 f_s and the chunk
       totals csum;
  (forward) the own-chunk step: the query carried to the chunk start times
       scale log2(e), the row maximum m_i and sum l_i of exp2(z_ij - m_i) over
       the own keys, and those probabilities, z_ij the logits in log2 units
       from the full-matrix form (oracle.full_matrix_logits) plus the gate.
Tolerances: every stored value is bf16 (relative rounding 2^-9) of a value
computed with bf16 operands and fp32 sums (hi/lo splits for the fp32 factors
T^{-1}, R, Y, U, about 16 bits), so a tile's max error is held to 2^-7 of
its largest entry and a key's (row's) error norm to 2^-7 of its norm; the
gate sums are fp64 sums rounded to fp32 (1e-5 relative); m_i, computed from
logits whose operands X = Q W^T and Y are bf16, to 2e-2 (log2 units).
"""
import math

import numpy as np
import pytest
import torch

import oracle
import softmax_attention_ut_amd as pa
from softmax_attention_ut_amd.inputs import generate

pytestmark = pytest.mark.gpu

C = 64


def permk(s):
    p = s & 15
    return (s & ~15) | ((p & ~12) | ((p & 4) << 1) | ((p & 8) >> 1))


PK = np.array([permk(s) for s in range(C)])


def _a256(x):
    return (x + 255) & ~255


def _sections(BH, L, D, diag):
    """Byte offsets of the forward workspace sections (bf16 mode, gate on,
    no key-cache tiles), in the library's order."""
    N = (L + C - 1) // C
    Lp = N * C
    off = 0
    sec = {}

    def take(name, nbytes):
        nonlocal off
        sec[name] = (off, nbytes)
        off += _a256(nbytes)
    take("kt", BH * Lp * D * 2)
    if not diag:
        take("ut", BH * Lp * D * 2)
    if D != 64:
        take("vt", BH * Lp * D * 2)
    if not diag:
        take("yt", BH * N * C * C * 2)
    if diag:
        take("mt", BH * N * D * D * 2)
        take("qt", BH * Lp * D * 2)
        take("pd", BH * Lp * C * 2)
        take("ml", BH * Lp * 2 * 4)
    take("loc", BH * Lp * 4)
    take("csum", BH * N * 4)
    return sec, off


def _view(ws, sec, name, dtype, shape):
    off, nbytes = sec[name]
    t = ws[off:off + nbytes].view(dtype).reshape(shape)
    return t.double().cpu().numpy()


def _prepare(inp, scale, diag):
    B, H, L, D = inp.q.shape
    g = {k: (None if t is None else t.cuda()) for k, t in vars(inp).items()}
    n = pa.path_attn_fwd_workspace_bytes(B, H, L, D, pa.PATH_BF16, 0)
    sec, total = _sections(B * H, L, D, diag)
    assert total <= n, (total, n)
    ws = torch.zeros(n, dtype=torch.uint8, device="cuda")
    pa.path_attn_fwd_prepare(g["q"], g["k"], g["v"], g["w"], g["beta"], g["log_f"], scale, 0, ws)
    torch.cuda.synchronize()
    return ws, sec


def _tile_close(got, ref, what, rel=2.0 ** -7):
    e = np.abs(got - ref).max()
    m = np.abs(ref).max()
    print(f"{what}: max-abs {e:.3e} of max |ref| {m:.3e}", flush=True)
    assert e <= rel * m + 1e-6, (what, e, m)


def _chunk(inp, h, c, L):
    sl = slice(c * C, min((c + 1) * C, L))
    f = lambda t: t[0, h, sl].double().numpy()
    return f(inp.q), f(inp.k), f(inp.v), f(inp.w), f(inp.beta), f(inp.log_f)


def _pad(a, rows):
    out = np.zeros((rows,) + a.shape[1:])
    out[:a.shape[0]] = a
    return out


def _common(inp, ws, sec, D, L):
    """K~ and the gate sums, both variants."""
    BH = inp.q.shape[1]
    N = (L + C - 1) // C
    Lp = N * C
    kt = _view(ws, sec, "kt", torch.bfloat16, (BH, Lp, D))
    loc = _view(ws, sec, "loc", torch.float32, (BH, Lp))
    csum = _view(ws, sec, "csum", torch.float32, (BH, N))
    worst = 0.0
    for h in range(BH):
        for c in range(N):
            n = min(C, L - c * C)
            end = c * C + n - 1
            keys = np.arange(c * C, end + 1)
            ref = oracle.transported_keys(inp.k[0, h], inp.w[0, h], inp.beta[0, h], end,
                                          np.zeros_like(keys), keys)
            got = kt[h, c * C:c * C + n]
            err = np.linalg.norm(got - ref, axis=1) / np.maximum(np.linalg.norm(ref, axis=1), 1e-30)
            worst = max(worst, err.max())
            lf2 = inp.log_f[0, h, c * C:end + 1].double().numpy() * math.log2(math.e)
            suffix = np.cumsum(lf2[::-1])[::-1]                  # sum_{s >= j}
            np.testing.assert_allclose(loc[h, c * C:end + 1], -(suffix - lf2), rtol=1e-5, atol=1e-5)
            np.testing.assert_allclose(csum[h, c], suffix[0], rtol=1e-5, atol=1e-5)
    print(f"K~ per-key relative error max {worst:.3e}", flush=True)
    assert worst <= 2.0 ** -7


def _bwd_sections(BH, L):
    """Byte offsets of the backward workspace's prepare-stage sections (d =
    64), in the library's order."""
    D = 64
    N = (L + C - 1) // C
    Lp = N * C
    off = 0
    sec = {}
    for name, nbytes in (("kt", BH * Lp * D * 2), ("ut", BH * Lp * D * 2), ("yt", BH * N * C * C * 2),
                         ("mt", BH * N * D * D * 2), ("loc", BH * Lp * 4), ("csum", BH * N * 4)):
        sec[name] = (off, nbytes)
        off += _a256(nbytes)
    return sec, off


def test_prepare_backward_u_and_y():
    """d = 64, the backward's prepare stage: K~, U, Y, -M^T, gate sums; L =
    200 leaves a ragged last chunk (w = 0, beta = 0 padding: H = I there).
    After path_attn_bwd the U and Y sections hold row-major U[m][e] and
    Y[m][j] (the backward's layout pass rewrites them in place)."""
    B, H, L, D = 1, 2, 200, 64
    scale = 0.125
    inp = generate(B, H, L, D, dtype="bf16", gate=True, seed=401)
    g = {k: (None if t is None else t.cuda()) for k, t in vars(inp).items()}
    n = pa.path_attn_bwd_workspace_bytes(B, H, L, D, pa.PATH_BF16)
    sec, total = _bwd_sections(B * H, L)
    assert total <= n, (total, n)
    ws = torch.zeros(n, dtype=torch.uint8, device="cuda")
    out = torch.zeros_like(g["q"])
    lse = torch.zeros(B, H, L, dtype=torch.float32, device="cuda")
    dout = torch.zeros_like(g["q"])
    grads = [torch.zeros(B, H, L, D, dtype=torch.float32, device="cuda") for _ in range(4)]
    dbeta = torch.zeros(B, H, L, dtype=torch.float32, device="cuda")
    dlogf = torch.zeros(B, H, L, dtype=torch.float32, device="cuda")
    pa.path_attn_bwd(g["q"], g["k"], g["v"], g["w"], g["beta"], g["log_f"], out, lse, dout,
                     *grads, dbeta, dlogf, scale, workspace=ws)
    torch.cuda.synchronize()
    _common(inp, ws, sec, D, L)
    N = (L + C - 1) // C
    U_ = _view(ws, sec, "ut", torch.bfloat16, (H, N, C, D))
    Y_ = _view(ws, sec, "yt", torch.bfloat16, (H, N, C, C))
    mt = _view(ws, sec, "mt", torch.bfloat16, (H, N, D, D))
    for h in range(H):
        for c in range(N):
            q, k, v, w, beta, lf = (_pad(x, C) for x in _chunk(inp, h, c, L))
            tinv = oracle.ut_tinv(w, beta)
            _tile_close(U_[h, c], tinv @ w, f"U h={h} c={c}")
            _tile_close(Y_[h, c], tinv @ np.tril(w @ k.T, -1), f"Y h={h} c={c}")
            M = np.eye(D) - oracle.ut_product(w, beta)
            _tile_close(mt[h, c], -M[:, PK].T, f"-M^T h={h} c={c}")


@pytest.mark.parametrize("D,L", [(64, 333), (128, 200)])
def test_prepare_dense_carry_and_own_chunk(D, L):
    """The forward's prepare stage (dense d x d carry, the own-chunk step):
    K~, -M^T, the carried queries, the own chunk's row maximum and sum and
    its probabilities, gate sums, and at d = 128 the V^T tiles; ragged L."""
    B, H = 1, 2
    scale = 1 / math.sqrt(D)
    s2 = scale * math.log2(math.e)
    inp = generate(B, H, L, D, dtype="bf16", gate=True, seed=402)
    ws, sec = _prepare(inp, scale, diag=True)
    _common(inp, ws, sec, D, L)
    N = (L + C - 1) // C
    Lp = N * C
    mt = _view(ws, sec, "mt", torch.bfloat16, (H, N, D, D))
    qt = _view(ws, sec, "qt", torch.bfloat16, (H, Lp, D))
    pd = _view(ws, sec, "pd", torch.bfloat16, (H, Lp, C))
    ml = _view(ws, sec, "ml", torch.float32, (H, Lp, 2))
    vt = _view(ws, sec, "vt", torch.bfloat16, (H, N, D, C)) if D != 64 else None
    pk_d = np.array([permk(r) for r in range(D)])
    worst_m = 0.0
    for h in range(H):
        for c in range(N):
            n = min(C, L - c * C)
            q, k, v, w, beta, lf = (_pad(x, C) for x in _chunk(inp, h, c, L))
            M = np.eye(D) - oracle.ut_product(w, beta)          # I - M = chunk product
            _tile_close(mt[h, c], -M[:, pk_d].T, f"-M^T h={h} c={c}")
            if vt is not None:                                  # vt[rho][sigma] = V[permk(sigma)][permk(rho)]
                np.testing.assert_array_equal(vt[h, c], v[PK][:, pk_d].T)
            U = oracle.ut_tinv(w, beta) @ w
            qc = (q - np.tril(q @ w.T) @ U) * s2
            got = qt[h, c * C:c * C + n]
            err = np.linalg.norm(got - qc[:n], axis=1) / np.linalg.norm(qc[:n], axis=1)
            assert err.max() <= 2.0 ** -7, ("carried query", h, c, err.max())
            # own-chunk logits in log2 units: full-matrix form + gate
            z = oracle.full_matrix_logits(q, k, w, beta, scale) * math.log2(math.e)
            lf2 = lf * math.log2(math.e)
            F = np.cumsum(lf2)
            z = z + (F[:, None] - F[None, :])
            z = z[:n, :n]
            m = z.max(axis=1)
            p = np.exp2(z - m[:, None])
            worst_m = max(worst_m, np.abs(ml[h, c * C:c * C + n, 0] - m).max())
            assert np.abs(ml[h, c * C:c * C + n, 0] - m).max() <= 2e-2
            np.testing.assert_allclose(ml[h, c * C:c * C + n, 1], p.sum(axis=1), rtol=2e-2)
            # pd[i][s] = exp2(z_{i, permk(s)} - m_i), zero for keys past i
            pref = np.zeros((n, C))
            pref[:, :n] = p
            got_p = pd[h, c * C:c * C + n][:, np.argsort(PK)]   # back to key order
            e = np.abs(got_p - pref).max()
            assert e <= 2e-2, ("probabilities", h, c, e)
    print(f"own-chunk row maximum: max error {worst_m:.3e} (log2 units)", flush=True)
