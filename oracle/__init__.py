"""PaTH attention CPU oracle (fp64).  TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It shares no code with the HIP path
(``softmax_attention_ut_amd``) and never imports it.

Two kinds of functions live here:

* ctypes wrappers around ``path_oracle.c`` (plain C, fp64, OpenMP over heads):
  the recurrent in-place key-update evaluation, the per-row evaluation of the
  definition, and selected transported keys;
* numpy fp64 evaluations written straight from the pages' formulas, used to
  pin the C code and each other on tiny inputs: explicit d x d transition
  matrices, the UT transform, and the full-matrix form of the logits;
* the transition parameters w_t, beta_t from the layer input (low-rank map,
  short convolution, L2 normalisation; 2 sigmoid), the reference of the
  transition-prep kernel;
* the gradients of the forward (the backward pass used in training), by
  reverse-mode differentiation of the recurrent form in plain fp64 PyTorch
  CPU ops.

Every function cites the passage it follows (PaTH paper pages: the Dutch
technical summary and the Chinese paper notes).  All parts are pinned by
tests in ``tests/test_oracle_pins.py``; none is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "path_oracle.c")
_LIB = os.path.join(_HERE, "libpath_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile path_oracle.c with gcc (plain -O2, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC",
                               "-shared", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        Lg = ctypes.c_long
        lib.path_oracle_recurrent.restype = ctypes.c_int
        lib.path_oracle_recurrent.argtypes = [Lg, Lg, Lg, P, P, P, P, P, P,
                                              ctypes.c_double, P, P, Lg, P,
                                              ctypes.c_int]
        lib.path_oracle_rows.restype = ctypes.c_int
        lib.path_oracle_rows.argtypes = [Lg, Lg, Lg, P, P, P, P, P, P,
                                         ctypes.c_double, Lg, P, P, P, P, P,
                                         ctypes.c_int]
        lib.path_oracle_transported_keys.restype = ctypes.c_int
        lib.path_oracle_transported_keys.argtypes = [Lg, Lg, Lg, P, P, P, Lg,
                                                     Lg, P, P, P]
        lib.path_oracle_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def _f64(x):
    """Exact float64 copy of a tensor/array, flattened to [BH, L, ...]."""
    if x is None:
        return None
    if hasattr(x, "detach"):
        x = x.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a):
    return None if a is None else a.ctypes.data


def max_threads() -> int:
    return _load().path_oracle_threads()


# ---------------------------------------------------------------------------
# C oracle wrappers
# ---------------------------------------------------------------------------

def recurrent(q, k, v, w, beta, log_f, scale, *, Lcache=0, nthreads=0):
    """Every output row by the in-place key-update recurrence (Dutch summary
    section 3 "Inferentie"; Chinese notes, inference paragraph): at step t all
    cached keys are multiplied by H_t = I - beta_t w_t w_t^T, key t is
    appended, and query t attends over keys 0..t with the FoX bias
    sum_{s=j+1}^{t} log f_s (Chinese notes, PaTH-FoX).

    q,k,v,w: [..., L, d]; beta, log_f: [..., L].  Returns (out, lse, kcache,
    threads) with kcache [..., Lcache, d] (the transformed cache after step
    Lcache-1) or None.
    """
    lib = _load()
    q, k, v, w = (_f64(t) for t in (q, k, v, w))
    beta = _f64(beta)
    log_f = _f64(log_f)
    lead = q.shape[:-2]
    L, d = q.shape[-2:]
    BH = int(np.prod(lead)) if lead else 1
    out = np.empty((BH, L, d))
    lse = np.empty((BH, L))
    kc = np.empty((BH, Lcache, d)) if Lcache > 0 else None
    used = lib.path_oracle_recurrent(BH, L, d, _ptr(q), _ptr(k), _ptr(v),
                                     _ptr(w), _ptr(beta), _ptr(log_f),
                                     float(scale), _ptr(out), _ptr(lse),
                                     int(Lcache), _ptr(kc), int(nthreads))
    out = out.reshape(*lead, L, d)
    lse = lse.reshape(*lead, L)
    if kc is not None:
        kc = kc.reshape(*lead, Lcache, d)
    return out, lse, kc, used


def rows(q, k, v, w, beta, log_f, scale, head_idx, row_idx, *,
         want_logits=False, nthreads=0):
    """Selected output rows straight from the definition
    A_ij ~ exp(k_j^T (H_{j+1}...H_i) q_i) (Dutch summary section 2,
    Kernmechanisme; Chinese notes, overall framework): the query is carried
    leftwards one transition at a time.  Heads are indexed in the flattened
    [B*H] order.  Returns (out [n,d], lse [n], logits [n,L] or None, threads).
    """
    lib = _load()
    q, k, v, w = (_f64(t) for t in (q, k, v, w))
    beta = _f64(beta)
    log_f = _f64(log_f)
    L, d = q.shape[-2:]
    BH = q.size // (L * d)
    hi = np.ascontiguousarray(np.asarray(head_idx, dtype=np.int64))
    ri = np.ascontiguousarray(np.asarray(row_idx, dtype=np.int64))
    n = hi.size
    out = np.empty((n, d))
    lse = np.empty(n)
    lg = np.empty((n, L)) if want_logits else None
    used = lib.path_oracle_rows(BH, L, d, _ptr(q), _ptr(k), _ptr(v), _ptr(w),
                                _ptr(beta), _ptr(log_f), float(scale), n,
                                _ptr(hi), _ptr(ri), _ptr(out), _ptr(lse),
                                _ptr(lg), int(nthreads))
    return out, lse, lg, used


def transported_keys(k, w, beta, T, head_idx, key_idx):
    """Selected in-place-updated cache entries H_T ... H_{j+1} k_j (Dutch
    summary section 3 "Inferentie")."""
    lib = _load()
    k, w = _f64(k), _f64(w)
    beta = _f64(beta)
    L, d = k.shape[-2:]
    BH = k.size // (L * d)
    hi = np.ascontiguousarray(np.asarray(head_idx, dtype=np.int64))
    ki = np.ascontiguousarray(np.asarray(key_idx, dtype=np.int64))
    out = np.empty((hi.size, d))
    lib.path_oracle_transported_keys(BH, L, d, _ptr(k), _ptr(w), _ptr(beta),
                                     int(T), hi.size, _ptr(hi), _ptr(ki),
                                     _ptr(out))
    return out


# ---------------------------------------------------------------------------
# numpy fp64 evaluations from the pages' formulas (tiny inputs)
# ---------------------------------------------------------------------------

def transition(w_t, beta_t):
    """H_t = I - beta_t w_t w_t^T as an explicit d x d matrix (Dutch summary
    section 2, "Data-afhankelijke Transitie-matrix")."""
    w_t = np.asarray(w_t, dtype=np.float64)
    return np.eye(w_t.size) - beta_t * np.outer(w_t, w_t)


def bruteforce_logits(q, k, w, beta, log_f, scale):
    """Unnormalised logit matrix of one head from explicit d x d products:
    logit_ij = scale * k_j^T (H_{j+1} ... H_i) q_i + sum_{s=j+1}^{i} log f_s
    for j <= i, -inf above the diagonal (Chinese notes, overall framework and
    PaTH-FoX).  q, k, w: [L, d]; beta, log_f: [L]."""
    q, k, w = (np.asarray(t, dtype=np.float64) for t in (q, k, w))
    beta = np.asarray(beta, dtype=np.float64)
    L, d = q.shape
    out = np.full((L, L), -np.inf)
    for i in range(L):
        M = np.eye(d)                      # H_{j+1} ... H_i, starts empty
        for j in range(i, -1, -1):
            bias = 0.0 if log_f is None else float(np.sum(log_f[j + 1:i + 1]))
            out[i, j] = scale * (k[j] @ M @ q[i]) + bias
            M = transition(w[j], beta[j]) @ M
    return out


def softmax_from_logits(logits, v):
    """o_i = sum_j softmax_j(logit_ij) v_j and lse_i = log sum_j exp(logit_ij)
    (Chinese notes, softmax form o_t = (1/Z_t) sum_j v_j exp(...))."""
    m = np.max(logits, axis=-1, keepdims=True)
    p = np.exp(logits - m)
    z = np.sum(p, axis=-1, keepdims=True)
    return (p / z) @ np.asarray(v, dtype=np.float64), (m + np.log(z))[..., 0]


def ut_tinv(w, beta):
    """T^{-1} = (I + strictLower(D W W^T))^{-1} D with D = diag(beta), rows of
    W = w_t (Chinese notes, training strategy, UT transform)."""
    w = np.asarray(w, dtype=np.float64)
    D = np.diag(np.asarray(beta, dtype=np.float64))
    A = np.tril(D @ w @ w.T, -1)
    return np.linalg.solve(np.eye(w.shape[0]) + A, D)


def ut_product(w, beta):
    """I - W^T T^{-1} W, the UT-transform form of a product of transitions
    (Chinese notes, training strategy; Dutch summary section 3)."""
    w = np.asarray(w, dtype=np.float64)
    return np.eye(w.shape[1]) - w.T @ ut_tinv(w, beta) @ w


def full_matrix_logits(q, k, w, beta, scale):
    """The full-matrix form  lower(Q K^T) - lower(Q W^T) T^{-1}
    strictLower(W K^T)  of the (unscaled) logits (Chinese notes, training
    strategy), scaled; entries above the diagonal set to -inf."""
    q, k, w = (np.asarray(t, dtype=np.float64) for t in (q, k, w))
    tinv = ut_tinv(w, beta)
    a = np.tril(q @ k.T) - np.tril(q @ w.T) @ tinv @ np.tril(w @ k.T, -1)
    a = scale * a
    a[np.triu_indices(q.shape[0], 1)] = -np.inf
    return a


def transition_prep(x, w_down, w_up, conv, u, b, d):
    """The transition parameters of every token from the layer input
    (Chinese notes, key design; Dutch summary section 2): w_t = L2-normalised
    short convolution (filter size 3) of a low-rank linear map of x_t, per
    head, and beta_t = 2 sigmoid(u^T x_t + b) per head.

    Readings where the pages are silent: the low-rank map is
    z_t = W_up (W_down x_t); the convolution is causal and depthwise,
    c_t = conv[:, 0] z_t + conv[:, 1] z_{t-1} + conv[:, 2] z_{t-2} (zero
    before the first token), with no bias or activation; each head's d-vector
    is divided by its norm, a zero vector staying zero.

    x [B, L, Dm]; w_down [r, Dm]; w_up [H*d, r]; conv [H*d, 3]; u [H, Dm];
    b [H].  Returns w [B, H, L, d] and beta [B, H, L], fp64."""
    x, w_down, w_up, conv, u, b = (np.asarray(t, dtype=np.float64)
                                   for t in (x, w_down, w_up, conv, u, b))
    B, L, _ = x.shape
    H = u.shape[0]
    z = (x @ w_down.T) @ w_up.T                        # [B, L, H*d]
    c = conv[:, 0] * z
    c[:, 1:] += conv[:, 1] * z[:, :-1]
    c[:, 2:] += conv[:, 2] * z[:, :-2]
    c = c.reshape(B, L, H, d).transpose(0, 2, 1, 3)    # [B, H, L, d]
    n = np.linalg.norm(c, axis=-1, keepdims=True)
    w = np.divide(c, n, out=np.zeros_like(c), where=n > 0)
    logit = x @ u.T + b                                # [B, L, H]
    beta = 2.0 / (1.0 + np.exp(-logit))
    return w, beta.transpose(0, 2, 1)


# ---------------------------------------------------------------------------
# Backward pass (gradients of the forward)
# ---------------------------------------------------------------------------

def _forward_torch(q, k, v, w, beta, log_f, scale):
    """The recurrent in-place key-update form (Dutch summary section 3,
    "Inferentie"; Chinese notes, inference paragraph) in fp64 torch ops, all
    heads at once: at step t every cached key is multiplied by H_t, key t is
    appended, and query t attends over the cache with the optional PaTH-FoX
    bias F_t - F_j (Chinese notes, PaTH-FoX).  q, k, v, w: [..., L, d];
    beta, log_f: [..., L].  Returns out [..., L, d]."""
    import torch
    L = q.shape[-2]
    F = None if log_f is None else torch.cumsum(log_f, dim=-1)
    keys = None
    outs = []
    for t in range(L):
        if keys is None:
            keys = k[..., :1, :]
        else:
            wt = w[..., t, :]                                         # [..., d]
            proj = (keys * wt[..., None, :]).sum(-1)                  # w_t . k_j, [..., t]
            keys = keys - beta[..., t, None, None] * proj[..., None] * wt[..., None, :]
            keys = torch.cat([keys, k[..., t:t + 1, :]], dim=-2)
        s = scale * (keys * q[..., t, None, :]).sum(-1)               # [..., t + 1]
        if F is not None:
            s = s + (F[..., t, None] - F[..., :t + 1])
        p = torch.softmax(s, dim=-1)
        outs.append((p[..., None] * v[..., :t + 1, :]).sum(-2))
    return torch.stack(outs, dim=-2)


def backward(q, k, v, w, beta, log_f, scale, d_out):
    """Gradients of sum(d_out * out) with respect to q, k, v, w, beta and
    log_f (None without the gate), out being the PaTH(-FoX) forward.  The
    pages say only that training uses the same blockwise algorithm (English
    summary; Dutch summary section 3); the backward is read as the exact
    gradient of the forward.  Reverse-mode differentiation of the recurrent
    form above, fp64, for small inputs (its graph holds O(L^2 d) values per
    head).  Returns a dict of fp64 numpy arrays: dq, dk, dv, dw, dbeta and,
    with the gate, dlog_f."""
    import torch
    names = ["q", "k", "v", "w", "beta"] + ([] if log_f is None else ["log_f"])
    vals = [q, k, v, w, beta] + ([] if log_f is None else [log_f])
    ts = [torch.tensor(_f64(x), dtype=torch.float64, requires_grad=True) for x in vals]
    tq, tk, tv, tw, tb = ts[:5]
    tf = ts[5] if log_f is not None else None
    out = _forward_torch(tq, tk, tv, tw, tb, tf, float(scale))
    loss = (out * torch.tensor(_f64(d_out), dtype=torch.float64)).sum()
    grads = torch.autograd.grad(loss, ts)
    return {"d" + n: g.numpy() for n, g in zip(names, grads)}
