"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every symbol include/path_attn.h declares, and rejects bad arguments before
any HIP call."""
import ctypes
import os
import re
import shutil
import subprocess

import pytest

import softmax_attention_ut_amd as pa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _header_symbols():
    txt = open(os.path.join(ROOT, "include", "path_attn.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return set(re.findall(r"\b(path_[a-z_0-9]+)\s*\(", txt))


def test_library_exports_every_declared_symbol():
    lib = pa.load_library()
    syms = _header_symbols()
    assert syms == set(pa.EXPORTS)
    for s in syms:
        assert hasattr(lib, s), s
    assert b"gfx950" in lib.path_version()


def test_status_strings():
    lib = pa.load_library()
    for code in (0, -1, -2, -3, -4):
        assert lib.path_status_string(code).decode() == pa.STATUS[code]


def test_workspace_sizes():
    f = pa.path_attn_fwd_workspace_bytes
    assert f(2, 8, 1024, 64, pa.PATH_BF16, 0) > 0
    assert f(2, 8, 1000, 64, pa.PATH_BF16, 0) == f(2, 8, 1024, 64, pa.PATH_BF16, 0)
    assert f(1, 1, 64, 16, pa.PATH_F32, 16) > 0
    assert f(1, 1, 0, 64, pa.PATH_BF16, 0) == 0          # empty sequence
    assert f(1, 1, 64, 48, pa.PATH_BF16, 0) == 0         # unsupported d
    assert f(1, 1, 64, 64, pa.PATH_BF16, 32) == 0        # bf16 chunk is 64
    assert f(1, 1, 64, 128, pa.PATH_F32, 64) == 0        # f32 d=128 needs chunk <= 32
    assert f(1, 1, 64, 64, 7, 0) == 0                    # bad dtype
    assert pa.path_kcache_workspace_bytes(2, 32, 8192, 128, pa.PATH_BF16) > 0
    assert pa.path_kcache_workspace_bytes(2, 32, 8192, 128, pa.PATH_F32) == 0
    assert pa.path_decode_workspace_bytes(2, 32, 8448, 128, pa.PATH_BF16) > 0
    assert pa.path_decode_workspace_bytes(2, 32, 8448, 96, pa.PATH_BF16) == 0


def _fwd_raw(ptr=1, L=64, d=64, dt=pa.PATH_BF16, chunk=0, ws=None, ws_bytes=None,
             log_f=None, B=1, H=1):
    lib = pa.load_library()
    p = ctypes.c_void_p(ptr) if ptr else None
    need = lib.path_attn_fwd_workspace_bytes(B, H, L, d, dt, chunk)
    if ws is None:
        ws = ctypes.c_void_p(4096)              # 256-aligned fake address, never touched
    if ws_bytes is None:
        ws_bytes = need
    return lib.path_attn_fwd(p, p, p, p, p, log_f, p, None, B, H, L, d, 0.125, dt, chunk,
                             ws, ws_bytes, None)


def test_fwd_argument_errors_before_launch():
    assert _fwd_raw(ptr=0) == -1                 # null inputs
    assert _fwd_raw(L=0) == -1                   # empty sequence
    assert _fwd_raw(B=0) == -1
    assert _fwd_raw(dt=3) == -1
    assert _fwd_raw(d=80) == -2
    assert _fwd_raw(chunk=32) == -2              # bf16 supports chunk 64 only
    assert _fwd_raw(d=128, dt=pa.PATH_F32, chunk=64) == -2
    assert _fwd_raw(ws=None, ws_bytes=0) == -4   # no room
    assert _fwd_raw(ws_bytes=100) == -4
    assert _fwd_raw(ws=ctypes.c_void_p(4096 + 8)) == -4    # misaligned workspace


def test_decode_argument_errors_before_launch():
    lib = pa.load_library()
    p = ctypes.c_void_p(4096)
    ws = lib.path_decode_workspace_bytes(1, 1, 16, 64, pa.PATH_BF16)
    args = lambda t, T, d, dt, wsb: (p, p, p, p, p, p, p, p, None, 1, 1, t, T, d, 0.1, dt, p, wsb, None)
    assert lib.path_decode_step(*args(16, 16, 64, pa.PATH_BF16, ws)) == -1   # t >= T_max
    assert lib.path_decode_step(*args(-1, 16, 64, pa.PATH_BF16, ws)) == -1
    assert lib.path_decode_step(*args(3, 16, 96, pa.PATH_BF16, ws)) == -2
    assert lib.path_decode_step(*args(3, 16, 64, pa.PATH_F32, ws)) == -2
    assert lib.path_decode_step(*args(3, 16, 64, pa.PATH_BF16, 8)) == -4


def test_noalloc_decode_argument_errors_before_launch():
    """path_decode_step_noalloc checks its arguments like path_decode_step
    and rejects calls whose partials exceed its 8 MiB array, all before any
    HIP call (the fake pointers are never dereferenced)."""
    lib = pa.load_library()
    p = ctypes.c_void_p(4096)
    args = lambda B, H, t, T, d, dt, q=p: (p, p, q, p, p, p, p, p, None, B, H, t, T, d, 0.1, dt,
                                           None)
    assert lib.path_decode_step_noalloc(*args(1, 1, 16, 16, 64, pa.PATH_BF16)) == -1  # t >= T_max
    assert lib.path_decode_step_noalloc(*args(1, 1, 3, 16, 64, pa.PATH_BF16, None)) == -1
    assert lib.path_decode_step_noalloc(*args(0, 1, 3, 16, 64, pa.PATH_BF16)) == -1
    assert lib.path_decode_step_noalloc(*args(1, 1, 3, 16, 96, pa.PATH_BF16)) == -2
    assert lib.path_decode_step_noalloc(*args(1, 1, 3, 16, 64, pa.PATH_F32)) == -2
    # 64 heads, d = 128: 64 * ceil((t+1)/64) * 130 * 4 bytes <= 8 MiB holds up to t = 16127
    assert lib.path_decode_step_noalloc(*args(2, 32, 16128, 20000, 128, pa.PATH_BF16)) == -4
    assert lib.path_decode_step_noalloc(*args(128, 64, 100, 200, 128, pa.PATH_BF16)) == -4


def test_bwd_workspace_and_argument_errors_before_launch():
    """path_attn_bwd: bf16 with d = 64 only; log_f and dlog_f both or
    neither; the workspace holds two bf16 64 x 64 tiles per pair of chunks
    per head.  Every call here is rejected on the host (the fake pointers are
    never dereferenced)."""
    lib = pa.load_library()
    f = lib.path_attn_bwd_workspace_bytes
    assert f(1, 1, 128, 128, pa.PATH_BF16) == 0
    assert f(1, 1, 128, 64, pa.PATH_F32) == 0
    assert f(1, 1, 0, 64, pa.PATH_BF16) == 0
    # 64 -> 128 chunks adds 64 * 127 / 2 - 32 * 31 / 2 pairs, 16 KiB each
    assert f(1, 1, 8192, 64, pa.PATH_BF16) - f(1, 1, 4096, 64, pa.PATH_BF16) >= 3568 * 16384
    assert f(1, 1, 1000, 64, pa.PATH_BF16) == f(1, 1, 1024, 64, pa.PATH_BF16)
    p = ctypes.c_void_p(4096)
    ws = f(1, 1, 128, 64, pa.PATH_BF16)

    def call(lf=p, dlf=p, d=64, dt=pa.PATH_BF16, wsb=ws, L=128, q=p, w_=p):
        return lib.path_attn_bwd(q, p, p, p, p, lf, p, p, p, p, p, p, p, p, dlf,
                                 1, 1, L, d, 0.125, dt, w_, wsb, None)
    assert call(dlf=None) == -1
    assert call(lf=None) == -1
    assert call(q=None) == -1
    assert call(L=0) == -1
    assert call(d=128) == -2
    assert call(dt=pa.PATH_F32) == -2
    assert call(wsb=ws - 1) == -4
    assert call(w_=ctypes.c_void_p(4096 + 16)) == -4


def test_gated_decode_argument_errors_before_launch():
    lib = pa.load_library()
    p = ctypes.c_void_p(4096)
    ws = lib.path_decode_workspace_bytes(1, 1, 16, 64, pa.PATH_BF16)
    # (k_cache, v_cache, f_cache, q, k, v, w, beta, log_f, out, lse, B, H, t, T_max, d, ...)
    args = lambda fc, lf, t: (p, p, fc, p, p, p, p, p, lf, p, None, 1, 1, t, 16, 64, 0.1,
                              pa.PATH_BF16, p, ws, None)
    assert lib.path_decode_step_gated(*args(None, p, 3)) == -1     # no gate cache
    assert lib.path_decode_step_gated(*args(p, None, 3)) == -1     # no log f
    assert lib.path_decode_step_gated(*args(p, p, 16)) == -1       # t >= T_max
    assert lib.path_fcache_from_prefill(p, p, 1, 1, 20, 16, None) == -1   # T_max < L
    assert lib.path_fcache_from_prefill(None, p, 1, 1, 8, 16, None) == -1
    assert lib.path_fcache_from_prefill(p, p, 0, 1, 8, 16, None) == -1


def test_kcache_argument_errors_before_launch():
    lib = pa.load_library()
    p = ctypes.c_void_p(4096)
    ws = lib.path_kcache_workspace_bytes(1, 1, 128, 64, pa.PATH_BF16)
    assert lib.path_kcache_from_prefill(p, p, p, p, p, p, 1, 1, 128, 100, 64, pa.PATH_BF16,
                                        p, ws, None) == -1          # T_max < L
    assert lib.path_kcache_from_prefill(p, p, p, p, p, p, 1, 1, 128, 200, 64, pa.PATH_F32,
                                        p, ws, None) == -2
    assert lib.path_kcache_from_prefill(None, p, p, p, p, p, 1, 1, 128, 200, 64,
                                        pa.PATH_BF16, p, ws, None) == -1
    assert lib.path_kcache_from_prefill(p, p, p, p, p, p, 1, 1, 128, 200, 64, pa.PATH_BF16,
                                        p, ws - 1, None) == -4


def test_kcache_from_forward_argument_errors_before_launch():
    lib = pa.load_library()
    p = ctypes.c_void_p(4096)
    ws = lib.path_kcache_workspace_bytes(1, 1, 128, 64, pa.PATH_BF16)
    fws = lib.path_attn_fwd_workspace_bytes(1, 1, 128, 64, pa.PATH_BF16, 0)
    f = lib.path_kcache_from_forward
    assert f(p, fws, p, p, p, 1, 1, 128, 100, 64, pa.PATH_BF16, p, ws, None) == -1   # T_max < L
    assert f(p, fws, p, p, p, 1, 1, 128, 200, 64, pa.PATH_F32, p, ws, None) == -2
    assert f(p, fws, p, p, p, 1, 1, 128, 200, 32, pa.PATH_BF16, p, ws, None) == -2   # d = 32
    assert f(p, fws, None, p, p, 1, 1, 128, 200, 64, pa.PATH_BF16, p, ws, None) == -1
    assert f(None, fws, p, p, p, 1, 1, 128, 200, 64, pa.PATH_BF16, p, ws, None) == -4
    assert f(p, fws - 1, p, p, p, 1, 1, 128, 200, 64, pa.PATH_BF16, p, ws, None) == -4
    assert f(ctypes.c_void_p(4096 + 16), fws, p, p, p, 1, 1, 128, 200, 64, pa.PATH_BF16, p, ws,
             None) == -4                                                            # not 256-aligned
    assert f(p, fws, p, p, p, 1, 1, 128, 200, 64, pa.PATH_BF16, p, ws - 1, None) == -4


def test_transition_argument_errors_before_launch():
    """Every call here is rejected on the host (fake pointers are never
    dereferenced): null pointers and sizes below 1 are invalid, shapes outside
    d in {64, 128}, r in {32, 64}, r + H <= 128, Dm % 128 == 0 unsupported."""
    lib = pa.load_library()
    p = ctypes.c_void_p(4096)

    def call(B=1, L=64, Dm=256, r=64, H=4, d=64, dt=pa.PATH_BF16, x=p, conv=p):
        return lib.path_transition_prep(x, p, p, conv, p, p, p, p, B, L, Dm, r, H, d, dt, None)

    assert call(x=None) == -1
    assert call(conv=None) == -1
    assert call(B=0) == -1
    assert call(L=0) == -1
    assert call(dt=5) == -1
    assert call(dt=pa.PATH_F32) == -2
    assert call(d=32) == -2
    assert call(r=48) == -2
    assert call(r=64, H=65) == -2          # r + H > 128
    assert call(Dm=200) == -2              # not a multiple of 128


def test_paged_argument_errors_before_launch():
    """Paged decode and prefill hand-off: a null table, bad page counts, a page
    that is not a multiple of 64, t beyond the capacity and a half-given gate
    are rejected on the host (fake pointers are never dereferenced)."""
    lib = pa.load_library()
    p = ctypes.c_void_p(4096)
    ws = lib.path_decode_workspace_bytes(1, 1, 256, 64, pa.PATH_BF16)

    def dec(table=p, nb=4, mb=4, page=64, fc=None, lf=None, t=10, d=64, wsb=ws):
        return lib.path_decode_step_paged(p, p, table, nb, mb, page, fc, lf, p, p, p, p, p, p,
                                          None, 1, 1, t, d, 0.1, pa.PATH_BF16, p, wsb, None)

    assert dec(table=None) == -1
    assert dec(nb=0) == -1
    assert dec(mb=0) == -1
    assert dec(page=0) == -1
    assert dec(page=48) == -2
    assert dec(t=256) == -1                 # capacity is max_blocks * page = 256
    assert dec(fc=p) == -1                  # gate cache without log f
    assert dec(lf=p) == -1
    assert dec(d=96) == -2
    assert dec(wsb=8) == -4
    kws = lib.path_kcache_workspace_bytes(1, 1, 128, 64, pa.PATH_BF16)

    def pre(table=p, mb=2, page=64, L=128):
        return lib.path_kcache_from_prefill_paged(p, p, p, p, p, p, table, 4, mb, page, 1, 1, L,
                                                  64, pa.PATH_BF16, p, kws, None)

    assert pre(table=None) == -1
    assert pre(page=100) == -2
    assert pre(mb=1) == -1                  # 128 tokens do not fit one 64-slot page


C_CLIENT = r"""
#include <stdio.h>
#include <string.h>
#include "path_attn.h"
int main(void) {
    /* host-only calls: no device is touched */
    if (strstr(path_version(), "gfx950") == NULL) return 1;
    if (strcmp(path_status_string(PATH_ERR_WORKSPACE), "workspace missing or too small")) return 2;
    if (path_attn_fwd_workspace_bytes(8, 24, 4096, 64, PATH_BF16, 0) == 0) return 3;
    if (path_attn_fwd(NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 1, 1, 64, 64, 0.125f,
                      PATH_BF16, 0, NULL, 0, NULL) != PATH_ERR_INVALID) return 4;
    printf("ok\n");
    return 0;
}
"""


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_plain_c_client_compiles_links_and_calls(tmp_path):
    """The boundary is a C ABI: a C99 program compiles against the header
    alone, links against libpath_attn.so and calls its host queries (no
    Python, no torch, no device access)."""
    lib = pa.load_library()
    src = tmp_path / "client.c"
    src.write_text(C_CLIENT)
    exe = tmp_path / "client"
    libdir = os.path.dirname(pa.LIB_PATH)
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
                        str(src), "-o", str(exe), "-L", libdir, "-l:libpath_attn.so",
                        f"-Wl,-rpath,{libdir}"], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert out.returncode == 0 and out.stdout.strip() == "ok", (out.returncode, out.stdout, out.stderr)
    assert lib is not None


def test_missing_library_fails_loudly(tmp_path):
    with pytest.raises(RuntimeError, match="no CPU fallback"):
        pa._lib_backup = pa._lib
        try:
            pa._lib = None
            pa.load_library(str(tmp_path / "nope.so"))
        finally:
            pa._lib = pa._lib_backup
