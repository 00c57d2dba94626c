"""PaTH attention for MI355X (gfx950): Python binding of libpath_attn.so.

Argument marshalling only: every step of the computation runs in the HIP
kernels of libpath_attn.so (C ABI in include/path_attn.h).  PyTorch provides
device memory and streams.  There is no CPU fallback: if the library is
missing or no GPU is present, calls raise.

Functions with the C names take torch tensors (device memory) and pass raw
pointers; ``attention`` / ``kcache_from_prefill`` / ``decode_step`` are
conveniences that allocate outputs and workspaces with torch.
"""
from __future__ import annotations

import ctypes
import os

import torch

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libpath_attn.so")

PATH_F32, PATH_BF16 = 0, 1
PATH_OK = 0
STATUS = {0: "ok", -1: "invalid argument", -2: "unsupported size or chunk",
          -3: "HIP runtime or launch error", -4: "workspace missing or too small"}

# every symbol declared in include/path_attn.h
EXPORTS = ("path_status_string", "path_version", "path_attn_fwd_workspace_bytes",
           "path_attn_fwd", "path_attn_fwd_prepare", "path_attn_fwd_scan",
           "path_kcache_workspace_bytes", "path_kcache_from_prefill",
           "path_decode_workspace_bytes", "path_decode_step", "path_fcache_from_prefill",
           "path_decode_step_gated", "path_transition_prep",
           "path_kcache_from_prefill_paged", "path_decode_step_paged",
           "path_decode_step_noalloc", "path_attn_bwd_workspace_bytes", "path_attn_bwd",
           "path_kcache_from_forward")


class PathError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {STATUS.get(status, 'unknown')} ({status})")
        self.status = status


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libpath_attn.so (torch is imported first so that the library binds
    to the same HIP runtime as torch)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m softmax_attention_ut_amd.build` "
            "(there is no CPU fallback)")
    lib = ctypes.CDLL(path)
    P, I, F, S = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.path_status_string.restype = ctypes.c_char_p
    lib.path_status_string.argtypes = [I]
    lib.path_version.restype = ctypes.c_char_p
    lib.path_version.argtypes = []
    lib.path_attn_fwd_workspace_bytes.restype = S
    lib.path_attn_fwd_workspace_bytes.argtypes = [I, I, I, I, I, I]
    lib.path_attn_fwd.restype = I
    lib.path_attn_fwd.argtypes = [P, P, P, P, P, P, P, P, I, I, I, I, F, I, I, P, S, P]
    lib.path_attn_fwd_prepare.restype = I
    lib.path_attn_fwd_prepare.argtypes = [P, P, P, P, P, P, I, I, I, I, F, I, I, P, S, P]
    lib.path_attn_fwd_scan.restype = I
    lib.path_attn_fwd_scan.argtypes = [P, P, P, P, P, P, P, I, I, I, I, F, I, I, P, S, P]
    lib.path_attn_bwd_workspace_bytes.restype = S
    lib.path_attn_bwd_workspace_bytes.argtypes = [I, I, I, I, I]
    lib.path_attn_bwd.restype = I
    lib.path_attn_bwd.argtypes = [P] * 15 + [I, I, I, I, F, I, P, S, P]
    lib.path_kcache_workspace_bytes.restype = S
    lib.path_kcache_workspace_bytes.argtypes = [I, I, I, I, I]
    lib.path_kcache_from_prefill.restype = I
    lib.path_kcache_from_prefill.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, P, S, P]
    lib.path_kcache_from_forward.restype = I
    lib.path_kcache_from_forward.argtypes = [P, S, P, P, P, I, I, I, I, I, I, P, S, P]
    lib.path_decode_workspace_bytes.restype = S
    lib.path_decode_workspace_bytes.argtypes = [I, I, I, I, I]
    lib.path_decode_step.restype = I
    lib.path_decode_step.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I, I, F, I, P, S, P]
    lib.path_decode_step_noalloc.restype = I
    lib.path_decode_step_noalloc.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I, I, F, I, P]
    lib.path_fcache_from_prefill.restype = I
    lib.path_fcache_from_prefill.argtypes = [P, P, I, I, I, I, P]
    lib.path_decode_step_gated.restype = I
    lib.path_decode_step_gated.argtypes = [P, P, P, P, P, P, P, P, P, P, P, I, I, I, I, I, F, I, P, S, P]
    lib.path_kcache_from_prefill_paged.restype = I
    lib.path_kcache_from_prefill_paged.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, I, I,
                                                   P, S, P]
    lib.path_decode_step_paged.restype = I
    lib.path_decode_step_paged.argtypes = [P, P, P, I, I, I, P, P, P, P, P, P, P, P, P, I, I, I,
                                           I, F, I, P, S, P]
    lib.path_transition_prep.restype = I
    lib.path_transition_prep.argtypes = [P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, P]
    _lib = lib
    return lib


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return PATH_F32
    if t.dtype == torch.bfloat16:
        return PATH_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(st: int, where: str):
    if st != PATH_OK:
        raise PathError(st, where)


def _require_cuda(*ts):
    for t in ts:
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError("tensors must be contiguous device tensors")


# ---------------------------------------------------------------------------
# C-ABI names
# ---------------------------------------------------------------------------

def path_attn_fwd_workspace_bytes(B, H, L, d, dtype, chunk=0) -> int:
    return load_library().path_attn_fwd_workspace_bytes(B, H, L, d, dtype, chunk)


def path_attn_fwd(q, k, v, w, beta, log_f, out, lse, scale, chunk=0,
                  workspace=None, stream=None):
    """q,k,v,w,out [B,H,L,d]; beta, log_f (or None), lse (or None) [B,H,L]."""
    lib = load_library()
    _require_cuda(q, k, v, w, beta, log_f, out, lse, workspace)
    B, H, L, d = q.shape
    dt = _dt(q)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = lib.path_attn_fwd(_p(q), _p(k), _p(v), _p(w), _p(beta), _p(log_f), _p(out),
                           _p(lse), B, H, L, d, float(scale), dt, int(chunk),
                           _p(workspace), ws_bytes, _stream(stream))
    _check(st, "path_attn_fwd")


def path_attn_fwd_prepare(q, k, v, w, beta, log_f, scale, chunk=0, workspace=None, stream=None):
    """The per-chunk stage of path_attn_fwd (fills workspace)."""
    lib = load_library()
    _require_cuda(q, k, v, w, beta, log_f, workspace)
    B, H, L, d = k.shape
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = lib.path_attn_fwd_prepare(_p(q), _p(k), _p(v), _p(w), _p(beta), _p(log_f), B, H, L, d,
                                   float(scale), _dt(k), int(chunk), _p(workspace), ws_bytes,
                                   _stream(stream))
    _check(st, "path_attn_fwd_prepare")


def path_attn_fwd_scan(q, k, v, w, log_f, out, lse, scale, chunk=0, workspace=None,
                       stream=None):
    """The right-to-left scan stage of path_attn_fwd (reads workspace)."""
    lib = load_library()
    _require_cuda(q, k, v, w, log_f, out, lse, workspace)
    B, H, L, d = q.shape
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = lib.path_attn_fwd_scan(_p(q), _p(k), _p(v), _p(w), _p(log_f), _p(out), _p(lse),
                                B, H, L, d, float(scale), _dt(q), int(chunk), _p(workspace),
                                ws_bytes, _stream(stream))
    _check(st, "path_attn_fwd_scan")


def path_attn_bwd_workspace_bytes(B, H, L, d, dtype) -> int:
    return load_library().path_attn_bwd_workspace_bytes(B, H, L, d, dtype)


def path_attn_bwd(q, k, v, w, beta, log_f, out, lse, d_out, dq, dk, dv, dw, dbeta, dlog_f,
                  scale, workspace=None, stream=None):
    """Gradients of path_attn_fwd: q,k,v,w,out,d_out bf16 [B,H,L,d]; dq,dk,dv,dw
    fp32 [B,H,L,d]; beta, log_f (or None), lse, dbeta, dlog_f (or None) fp32 [B,H,L]."""
    lib = load_library()
    _require_cuda(q, k, v, w, beta, log_f, out, lse, d_out, dq, dk, dv, dw, dbeta, dlog_f,
                  workspace)
    B, H, L, d = q.shape
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = lib.path_attn_bwd(_p(q), _p(k), _p(v), _p(w), _p(beta), _p(log_f), _p(out), _p(lse),
                           _p(d_out), _p(dq), _p(dk), _p(dv), _p(dw), _p(dbeta), _p(dlog_f),
                           B, H, L, d, float(scale), _dt(q), _p(workspace), ws_bytes,
                           _stream(stream))
    _check(st, "path_attn_bwd")


def path_kcache_workspace_bytes(B, H, L, d, dtype) -> int:
    return load_library().path_kcache_workspace_bytes(B, H, L, d, dtype)


def path_kcache_from_prefill(k, v, w, beta, k_cache, v_cache, workspace=None, stream=None):
    """k,v,w [B,H,L,d]; beta [B,H,L]; k_cache, v_cache [B,H,T_max,d]."""
    lib = load_library()
    _require_cuda(k, v, w, beta, k_cache, v_cache, workspace)
    B, H, L, d = k.shape
    T_max = k_cache.shape[2]
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = lib.path_kcache_from_prefill(_p(k), _p(v), _p(w), _p(beta), _p(k_cache),
                                      _p(v_cache), B, H, L, T_max, d, _dt(k),
                                      _p(workspace), ws_bytes, _stream(stream))
    _check(st, "path_kcache_from_prefill")


def path_kcache_from_forward(fwd_workspace, v, k_cache, v_cache, workspace=None, stream=None):
    """The caches from the workspace of a bf16 path_attn_fwd on the same k, w,
    beta: v [B,H,L,d]; k_cache, v_cache [B,H,T_max,d]."""
    lib = load_library()
    _require_cuda(fwd_workspace, v, k_cache, v_cache, workspace)
    B, H, L, d = v.shape
    T_max = k_cache.shape[2]
    fws_bytes = fwd_workspace.numel() * fwd_workspace.element_size()
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = lib.path_kcache_from_forward(_p(fwd_workspace), fws_bytes, _p(v), _p(k_cache),
                                      _p(v_cache), B, H, L, T_max, d, _dt(v),
                                      _p(workspace), ws_bytes, _stream(stream))
    _check(st, "path_kcache_from_forward")


def path_decode_workspace_bytes(B, H, T_max, d, dtype) -> int:
    return load_library().path_decode_workspace_bytes(B, H, T_max, d, dtype)


def path_decode_step(k_cache, v_cache, q_t, k_t, v_t, w_t, beta_t, out_t, lse_t, t,
                     scale, workspace=None, stream=None):
    """caches [B,H,T_max,d]; q_t,k_t,v_t,w_t,out_t [B,H,d]; beta_t, lse_t [B,H]."""
    lib = load_library()
    _require_cuda(k_cache, v_cache, q_t, k_t, v_t, w_t, beta_t, out_t, lse_t, workspace)
    B, H, T_max, d = k_cache.shape
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = lib.path_decode_step(_p(k_cache), _p(v_cache), _p(q_t), _p(k_t), _p(v_t), _p(w_t),
                              _p(beta_t), _p(out_t), _p(lse_t), B, H, int(t), T_max, d,
                              float(scale), _dt(k_cache), _p(workspace), ws_bytes,
                              _stream(stream))
    _check(st, "path_decode_step")


def path_decode_step_noalloc(k_cache, v_cache, q_t, k_t, v_t, w_t, beta_t, out_t, lse_t, t,
                             scale, stream=None):
    """path_decode_step with the library's own partials buffer (no workspace)."""
    lib = load_library()
    _require_cuda(k_cache, v_cache, q_t, k_t, v_t, w_t, beta_t, out_t, lse_t)
    B, H, T_max, d = k_cache.shape
    st = lib.path_decode_step_noalloc(_p(k_cache), _p(v_cache), _p(q_t), _p(k_t), _p(v_t),
                                      _p(w_t), _p(beta_t), _p(out_t), _p(lse_t), B, H, int(t),
                                      T_max, d, float(scale), _dt(k_cache), _stream(stream))
    _check(st, "path_decode_step_noalloc")


def path_fcache_from_prefill(log_f, f_cache, stream=None):
    """log_f [B,H,L] float32; f_cache [B,H,T_max] float32 (slots [0,L) written)."""
    lib = load_library()
    _require_cuda(log_f, f_cache)
    B, H, L = log_f.shape
    T_max = f_cache.shape[2]
    st = lib.path_fcache_from_prefill(_p(log_f), _p(f_cache), B, H, L, T_max, _stream(stream))
    _check(st, "path_fcache_from_prefill")


def path_decode_step_gated(k_cache, v_cache, f_cache, q_t, k_t, v_t, w_t, beta_t, log_f_t,
                           out_t, lse_t, t, scale, workspace=None, stream=None):
    """path_decode_step with the PaTH-FoX gate: f_cache [B,H,T_max] float32
    (F_0 .. F_{t-1} in, F_t written), log_f_t [B,H] float32."""
    lib = load_library()
    _require_cuda(k_cache, v_cache, f_cache, q_t, k_t, v_t, w_t, beta_t, log_f_t, out_t, lse_t,
                  workspace)
    B, H, T_max, d = k_cache.shape
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = lib.path_decode_step_gated(_p(k_cache), _p(v_cache), _p(f_cache), _p(q_t), _p(k_t),
                                    _p(v_t), _p(w_t), _p(beta_t), _p(log_f_t), _p(out_t),
                                    _p(lse_t), B, H, int(t), T_max, d, float(scale),
                                    _dt(k_cache), _p(workspace), ws_bytes, _stream(stream))
    _check(st, "path_decode_step_gated")


def path_kcache_from_prefill_paged(k, v, w, beta, k_pool, v_pool, block_table,
                                   workspace=None, stream=None):
    """k,v,w [B,H,L,d]; beta [B,H,L]; k_pool, v_pool [num_blocks,H,page,d];
    block_table [B,max_blocks] int32."""
    lib = load_library()
    _require_cuda(k, v, w, beta, k_pool, v_pool, block_table, workspace)
    B, H, L, d = k.shape
    num_blocks, _, page, _ = k_pool.shape
    max_blocks = block_table.shape[1]
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = lib.path_kcache_from_prefill_paged(_p(k), _p(v), _p(w), _p(beta), _p(k_pool),
                                            _p(v_pool), _p(block_table), num_blocks,
                                            max_blocks, page, B, H, L, d, _dt(k),
                                            _p(workspace), ws_bytes, _stream(stream))
    _check(st, "path_kcache_from_prefill_paged")


def path_decode_step_paged(k_pool, v_pool, block_table, q_t, k_t, v_t, w_t, beta_t, out_t,
                           lse_t, t, scale, f_cache=None, log_f_t=None, workspace=None,
                           stream=None):
    """pools [num_blocks,H,page,d]; block_table [B,max_blocks] int32;
    q_t,k_t,v_t,w_t,out_t [B,H,d]; beta_t, lse_t [B,H]; optional PaTH-FoX gate
    f_cache [B,H,max_blocks*page] and log_f_t [B,H]."""
    lib = load_library()
    _require_cuda(k_pool, v_pool, block_table, q_t, k_t, v_t, w_t, beta_t, out_t, lse_t,
                  f_cache, log_f_t, workspace)
    num_blocks, H, page, d = k_pool.shape
    B, max_blocks = block_table.shape
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = lib.path_decode_step_paged(_p(k_pool), _p(v_pool), _p(block_table), num_blocks,
                                    max_blocks, page, _p(f_cache), _p(log_f_t), _p(q_t),
                                    _p(k_t), _p(v_t), _p(w_t), _p(beta_t), _p(out_t),
                                    _p(lse_t), B, H, int(t), d, float(scale), _dt(k_pool),
                                    _p(workspace), ws_bytes, _stream(stream))
    _check(st, "path_decode_step_paged")


def path_transition_prep(x, w_down, w_up, conv, u, b, w, beta, stream=None):
    """x [B,L,Dm]; w_down [r,Dm]; w_up [H*d,r]; conv [H*d,3] float32; u [H,Dm];
    b [H] float32 -> w [B,H,L,d] (written), beta [B,H,L] float32 (written)."""
    lib = load_library()
    _require_cuda(x, w_down, w_up, conv, u, b, w, beta)
    B, L, Dm = x.shape
    r = w_down.shape[0]
    H = u.shape[0]
    d = w.shape[-1]
    st = lib.path_transition_prep(_p(x), _p(w_down), _p(w_up), _p(conv), _p(u), _p(b),
                                  _p(w), _p(beta), B, L, Dm, r, H, d, _dt(x),
                                  _stream(stream))
    _check(st, "path_transition_prep")


# ---------------------------------------------------------------------------
# conveniences (allocate with torch, then call the C ABI)
# ---------------------------------------------------------------------------

def _workspace(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def attention(q, k, v, w, beta, log_f=None, scale=None, chunk=0, want_lse=True,
              stream=None):
    """PaTH attention forward; returns (out, lse)."""
    B, H, L, d = q.shape
    if scale is None:
        scale = d ** -0.5
    n = path_attn_fwd_workspace_bytes(B, H, L, d, _dt(q), chunk)
    if n == 0:
        raise PathError(-2, "path_attn_fwd_workspace_bytes")
    ws = _workspace(n, q.device)
    out = torch.empty_like(q)
    lse = torch.empty(B, H, L, dtype=torch.float32, device=q.device) if want_lse else None
    path_attn_fwd(q, k, v, w, beta, log_f, out, lse, scale, chunk, ws, stream)
    return out, lse


def attention_backward(q, k, v, w, beta, log_f, out, lse, d_out, scale=None, stream=None):
    """Gradients of attention(): returns (dq, dk, dv, dw, dbeta, dlog_f or None),
    float32, from the forward's out and lse and d_out = dLoss/d out."""
    B, H, L, d = q.shape
    if scale is None:
        scale = d ** -0.5
    n = path_attn_bwd_workspace_bytes(B, H, L, d, _dt(q))
    if n == 0:
        raise PathError(-2, "path_attn_bwd_workspace_bytes")
    ws = _workspace(n, q.device)
    f32 = dict(dtype=torch.float32, device=q.device)
    dq, dk, dv, dw = (torch.empty(B, H, L, d, **f32) for _ in range(4))
    dbeta = torch.empty(B, H, L, **f32)
    dlog_f = torch.empty(B, H, L, **f32) if log_f is not None else None
    path_attn_bwd(q, k, v, w, beta, log_f, out, lse, d_out, dq, dk, dv, dw, dbeta, dlog_f,
                  scale, ws, stream)
    return dq, dk, dv, dw, dbeta, dlog_f


def kcache_from_prefill(k, v, w, beta, T_max, stream=None):
    B, H, L, d = k.shape
    n = path_kcache_workspace_bytes(B, H, L, d, _dt(k))
    if n == 0:
        raise PathError(-2, "path_kcache_workspace_bytes")
    ws = _workspace(n, k.device)
    kc = torch.zeros(B, H, T_max, d, dtype=k.dtype, device=k.device)
    vc = torch.zeros(B, H, T_max, d, dtype=k.dtype, device=k.device)
    path_kcache_from_prefill(k, v, w, beta, kc, vc, ws, stream)
    return kc, vc


def kcache_from_forward(fwd_workspace, v, T_max, stream=None):
    """Key and value caches from the workspace of a bf16 forward on the same
    k, w, beta (v is needed for the value cache)."""
    B, H, L, d = v.shape
    n = path_kcache_workspace_bytes(B, H, L, d, _dt(v))
    if n == 0:
        raise PathError(-2, "path_kcache_workspace_bytes")
    ws = _workspace(n, v.device)
    kc = torch.zeros(B, H, T_max, d, dtype=v.dtype, device=v.device)
    vc = torch.zeros(B, H, T_max, d, dtype=v.dtype, device=v.device)
    path_kcache_from_forward(fwd_workspace, v, kc, vc, ws, stream)
    return kc, vc


def fcache_from_prefill(log_f, T_max, stream=None):
    B, H, L = log_f.shape
    fc = torch.zeros(B, H, T_max, dtype=torch.float32, device=log_f.device)
    path_fcache_from_prefill(log_f, fc, stream)
    return fc


def decode_workspace(B, H, T_max, d, dtype, device):
    n = path_decode_workspace_bytes(B, H, T_max, d, dtype)
    if n == 0:
        raise PathError(-2, "path_decode_workspace_bytes")
    return _workspace(n, device)


def transition_prep(x, w_down, w_up, conv, u, b, d, stream=None):
    """Transition parameters (w, beta) of every token; returns
    w [B,H,L,d] in x's dtype and beta [B,H,L] float32."""
    B, L, _ = x.shape
    H = u.shape[0]
    w = torch.empty(B, H, L, d, dtype=x.dtype, device=x.device)
    beta = torch.empty(B, H, L, dtype=torch.float32, device=x.device)
    path_transition_prep(x, w_down, w_up, conv, u, b, w, beta, stream)
    return w, beta
