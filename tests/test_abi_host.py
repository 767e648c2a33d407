"""Host-side checks of the C ABI (no GPU): the library loads, exports every
function include/moe.h declares, and rejects bad arguments before launching
anything. Every call here fails validation, so no HIP API is reached."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _ensure_built():
    import sparse_moe_transformer_gemm_amd as m
    if not os.path.exists(m.library_path()):
        from sparse_moe_transformer_gemm_amd import build
        build.build()
    return m


@pytest.fixture(scope="module")
def moe():
    return _ensure_built()


def _declared_functions():
    with open(os.path.join(ROOT, "include", "moe.h")) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_four_calls():
    names = _declared_functions()
    for n in ("moe_route", "moe_permute", "moe_expert_ffn_mxfp4", "moe_combine",
              "moe_workspace_bytes"):
        assert n in names


def test_every_declared_symbol_is_exported(moe):
    L = moe.lib()
    for name in _declared_functions():
        assert hasattr(L, name), name
    assert set(_declared_functions()) == set(moe.EXPORTED)


def test_library_is_gfx950_and_dynamic(moe):
    out = os.popen(f"readelf -d {moe.library_path()}").read()
    assert "libamdhip64.so" in out


def test_workspace_bytes(moe):
    L = moe.lib()
    D = moe.Dims
    assert L.moe_workspace_bytes(D(16, 2880, 2880, 32, 4)) > 0
    assert L.moe_workspace_bytes(D(8192, 2880, 2880, 32, 4)) >= 8192 * 4 * 2880
    assert L.moe_workspace_bytes(D(0, 2880, 2880, 32, 4)) == 0       # T < 1
    assert L.moe_workspace_bytes(D(16, 2880 + 32, 2880, 32, 4)) == 0  # d % 64
    assert L.moe_workspace_bytes(D(16, 2880, 2880, 3, 4)) == 0       # k > E
    assert L.moe_workspace_bytes(D(16, 2880, 2880, 512, 4)) == 0     # E > 256
    assert L.moe_workspace_bytes(D(16, 2880, 2880, 32, 9)) == 0      # k > 8


FAKE = 0x10000  # an aligned, non-null address that is never dereferenced


def test_route_validation(moe):
    L = moe.lib()
    D = moe.Dims
    ok = D(16, 512, 512, 32, 4)
    ws = L.moe_workspace_bytes(ok)
    assert L.moe_route(ok, None, FAKE, None, FAKE, FAKE, FAKE, ws, None) == -1
    assert L.moe_route(ok, FAKE + 2, FAKE, None, FAKE, FAKE, FAKE, ws, None) == -1  # misaligned
    assert b"aligned" in L.moe_last_error()
    assert L.moe_route(ok, FAKE, FAKE, None, FAKE, FAKE, FAKE, ws - 256, None) == -3
    assert L.moe_route(D(16, 512, 512, 300, 4), FAKE, FAKE, None, FAKE, FAKE, FAKE, ws, None) == -2
    assert L.moe_route(D(16, 500, 512, 32, 4), FAKE, FAKE, None, FAKE, FAKE, FAKE, ws, None) == -1
    assert L.moe_route(ok, FAKE, FAKE, FAKE + 4, FAKE, FAKE, FAKE, ws, None) == -1


def test_permute_validation(moe):
    L = moe.lib()
    D = moe.Dims
    ok = D(16, 512, 512, 32, 4)
    ws = L.moe_workspace_bytes(ok)
    assert L.moe_permute(ok, FAKE, FAKE, None, FAKE, FAKE, FAKE, ws, None) == -1
    assert L.moe_permute(D(16, 512, 512, 32, 0), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws, None) == -1
    assert L.moe_permute(ok, FAKE, FAKE, FAKE, FAKE, FAKE, None, ws, None) == -1


def test_ffn_validation(moe):
    L = moe.lib()
    D = moe.Dims
    ok = D(16, 512, 512, 32, 4)
    ws = L.moe_workspace_bytes(ok)
    m = moe.MXFP4(FAKE, FAKE)
    bad = moe.MXFP4(FAKE, None)
    args = [FAKE, FAKE, FAKE, m, m, m, FAKE, FAKE, FAKE, FAKE, FAKE, ws, None]
    a = list(args); a[3] = bad
    assert L.moe_expert_ffn_mxfp4(ok, *a) == -1
    a = list(args); a[11] = 16
    assert L.moe_expert_ffn_mxfp4(ok, *a) == -3
    assert L.moe_expert_ffn_mxfp4(D(16, 512, 544, 32, 4), *args) == -1  # F % 64
    assert L.moe_expert_ffn_mxfp4(D(70000, 512, 512, 32, 4), *args) == -2  # T too big
    # contraction lengths below MOE_MIN_FFN_K: the encoding's error tail
    for dd, ff in ((448, 512), (512, 448), (64, 64)):
        small = D(16, dd, ff, 32, 4)
        a = list(args); a[11] = L.moe_workspace_bytes(small)
        assert a[11] > 0  # routing and dispatch still accept the widths
        assert L.moe_expert_ffn_mxfp4(small, *a) == -2, (dd, ff)
        assert b"512" in L.moe_last_error()
    # many tokens at a width no prefill column tile divides (d = 64 mod 128, not a
    # multiple of 192 or 320): the down GEMM streams, which needs F <= 4096
    wide = D(100, 832, 8192, 32, 4)
    a = list(args); a[11] = L.moe_workspace_bytes(wide)
    assert L.moe_expert_ffn_mxfp4(wide, *a) == -2
    assert b"4096" in L.moe_last_error()
    fine = D(100, 832, 4096, 32, 4)
    a = list(args); a[3] = bad; a[11] = L.moe_workspace_bytes(fine)
    assert L.moe_expert_ffn_mxfp4(fine, *a) == -1   # accepted dims, rejected for the null pointer


def test_pack_sizes_and_validation(moe):
    L = moe.lib()
    # K = 2880: 23 steps of 128 (the last half used); 2 KB of codes and 128 B of
    # scales per (32-row group, step)
    assert L.moe_mxfp4_packed_bytes(32, 2880, 2880, 0) == 32 * 90 * 23 * 2048
    assert L.moe_mxfp4_packed_bytes(32, 2880, 2880, 1) == 32 * 90 * 23 * 128
    assert L.moe_mxfp4_packed_bytes(1, 64, 128, 0) == 2 * 1 * 2048
    assert L.moe_mxfp4_packed_bytes(32, 2880, 2880, 2) == 0      # which
    assert L.moe_mxfp4_packed_bytes(32, 2880, 2880 + 32, 0) == 0  # K % 64
    assert L.moe_mxfp4_packed_bytes(0, 2880, 2880, 0) == 0       # E < 1
    assert L.moe_mxfp4_packed_bytes(257, 2880, 2880, 0) == 0     # E > 256
    src = moe.MXFP4(FAKE, FAKE)
    assert L.moe_pack_mxfp4(32, 2880, 2880, moe.MXFP4(FAKE, None), FAKE, FAKE, None) == -1
    assert L.moe_pack_mxfp4(32, 2880, 2880, src, FAKE + 8, FAKE, None) == -1  # misaligned
    assert L.moe_pack_mxfp4(32, 2880, 2900, src, FAKE, FAKE, None) == -1
    assert L.moe_pack_mxfp4(32, 20000, 2880, src, FAKE, FAKE, None) == -1


def test_forward_validation(moe):
    L = moe.lib()
    D = moe.Dims
    ok = D(16, 512, 512, 32, 4)
    ws = L.moe_workspace_bytes(ok)
    m = moe.MXFP4(FAKE, FAKE)
    # x, w_router, b_router, w_gate, w_up, w_down, b_gate, b_up, b_down, topk_idx,
    # topk_w, counts, offsets, sorted_pair, pair_row, y_sorted, out, ws, ws_bytes, stream
    args = [FAKE, FAKE, None, m, m, m, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
            FAKE, FAKE, FAKE, ws, None]
    for i in (0, 1, 6, 9, 11, 14, 16, 17):
        a = list(args); a[i] = None
        assert L.moe_forward(ok, *a) == -1, i
    a = list(args); a[4] = moe.MXFP4(None, FAKE)
    assert L.moe_forward(ok, *a) == -1
    a = list(args); a[2] = FAKE + 4                          # misaligned b_router
    assert L.moe_forward(ok, *a) == -1
    a = list(args); a[18] = ws - 256
    assert L.moe_forward(ok, *a) == -3
    assert L.moe_forward(D(16, 512, 512, 300, 4), *args) == -2
    a = list(args); a[18] = L.moe_workspace_bytes(D(16, 256, 512, 32, 4))
    assert L.moe_forward(D(16, 256, 512, 32, 4), *a) == -2  # d below MOE_MIN_FFN_K


def test_ffn_stage_validation(moe):
    """The staged FFN call rejects a stage outside 0..2 and checks the rest of
    its arguments as moe_expert_ffn_mxfp4 does, before any launch."""
    L = moe.lib()
    D = moe.Dims
    ok = D(16, 512, 512, 32, 4)
    ws = L.moe_workspace_bytes(ok)
    m = moe.MXFP4(FAKE, FAKE)
    # x, sorted_pair, offsets, w_gate, w_up, w_down, b_gate, b_up, b_down, y_sorted,
    # stage, ws, ws_bytes, stream
    args = [FAKE, FAKE, FAKE, m, m, m, FAKE, FAKE, FAKE, FAKE, 1, FAKE, ws, None]
    for stage in (-1, 3):
        a = list(args); a[10] = stage
        assert L.moe_expert_ffn_mxfp4_stage(ok, *a) == -1, stage
        assert b"stage" in L.moe_last_error()
    for i in (0, 1, 2, 6, 9, 11):
        a = list(args); a[i] = None
        assert L.moe_expert_ffn_mxfp4_stage(ok, *a) == -1, i
    a = list(args); a[12] = ws - 256
    assert L.moe_expert_ffn_mxfp4_stage(ok, *a) == -3
    assert L.moe_expert_ffn_mxfp4_stage(D(16, 512, 512, 300, 4), *args) == -2
    a = list(args); a[12] = L.moe_workspace_bytes(D(16, 512, 384, 32, 4))
    assert L.moe_expert_ffn_mxfp4_stage(D(16, 512, 384, 32, 4), *a) == -2  # F below the minimum


def test_workspace_covers_the_fused_call(moe):
    """The whole-block call's scratch (router partials and an arrival counter
    after the FFN regions) is part of moe_workspace_bytes at decode sizes."""
    L = moe.lib()
    D = moe.Dims
    for T, d, F, E, k in [(16, 2880, 2880, 32, 4), (64, 4096, 4096, 256, 8), (1, 64, 64, 4, 4)]:
        ws = L.moe_workspace_bytes(D(T, d, F, E, k))
        P = T * k
        steps = lambda K: (K + 127) // 128
        enc = T * steps(d) * 208 + P * steps(F) * 208
        assert ws >= enc + (d // 64) * T * E * 8 + 256, (T, d, F, E, k)


def test_combine_norm_validation(moe):
    L = moe.lib()
    D = moe.Dims
    assert L.moe_combine(D(16, 512, 512, 32, 4), FAKE, FAKE, None, FAKE, None) == -1
    assert L.moe_rmsnorm(16, 12, FAKE, FAKE, 1e-5, FAKE, None) == -1
    assert L.moe_rmsnorm(16, 512, FAKE, FAKE, -1.0, FAKE, None) == -1
    assert L.moe_residual_add(0, 512, FAKE, FAKE, FAKE, None) == -1
    # the fused residual + norm: bad d, bad eps, a null pointer, n_out aliasing x
    FAKE2 = 0x20000
    assert L.moe_residual_rmsnorm(16, 12, FAKE, FAKE2, FAKE, 1e-5, FAKE, FAKE2, None) == -1
    assert L.moe_residual_rmsnorm(16, 512, FAKE, FAKE2, FAKE, -1.0, FAKE, FAKE2, None) == -1
    assert L.moe_residual_rmsnorm(16, 512, FAKE, None, FAKE, 1e-5, FAKE, FAKE2, None) == -1
    assert L.moe_residual_rmsnorm(16, 512, FAKE, FAKE2, FAKE, 1e-5, FAKE2, FAKE, None) == -1
    assert b"alias" in L.moe_last_error()


def test_combine_residual_norm_validation(moe):
    """The fused combine + residual + norm and the whole block with it: null or
    misaligned pointers, a negative eps and forbidden aliases are rejected on the
    host; the block output and, without a gain, n_out may be null."""
    L = moe.lib()
    D = moe.Dims
    ok = D(16, 512, 512, 32, 4)
    R, RO, N, M = 0x20000, 0x30000, 0x40000, 0x50000
    # y_sorted, pair_row, topk_w, resid, gain, eps, m_out, resid_out, n_out, stream
    args = [FAKE, FAKE, FAKE, R, FAKE, 1e-5, M, RO, N, None]
    for i in (0, 1, 2, 3, 7, 8):
        a = list(args); a[i] = None
        assert L.moe_combine_residual_rmsnorm(ok, *a) == -1, i
    a = list(args); a[5] = -1.0
    assert L.moe_combine_residual_rmsnorm(ok, *a) == -1
    for i, v in ((8, R), (8, RO), (8, M), (6, R), (6, RO)):
        a = list(args); a[i] = v
        assert L.moe_combine_residual_rmsnorm(ok, *a) == -1, (i, v)
        assert b"alias" in L.moe_last_error()
    a = list(args); a[3] = R + 8
    assert L.moe_combine_residual_rmsnorm(ok, *a) == -1
    assert L.moe_combine_residual_rmsnorm(D(16, 512, 512, 300, 4), *args) == -2
    ws = L.moe_workspace_bytes(ok)
    m = moe.MXFP4(FAKE, FAKE)
    # moe_forward's arguments (out may be null), then resid, gain, eps, resid_out,
    # n_out, ws, ws_bytes, stream
    fw = [FAKE, FAKE, None, m, m, m, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
          FAKE, None, R, FAKE, 1e-5, RO, N, FAKE, ws, None]
    for i in (0, 9, 15, 17, 20, 21, 22):
        a = list(fw); a[i] = None
        assert L.moe_forward_residual_rmsnorm(ok, *a) == -1, i
    a = list(fw); a[21] = RO
    assert L.moe_forward_residual_rmsnorm(ok, *a) == -1
    a = list(fw); a[19] = -1.0
    assert L.moe_forward_residual_rmsnorm(ok, *a) == -1
    a = list(fw); a[23] = ws - 256
    assert L.moe_forward_residual_rmsnorm(ok, *a) == -3
    a = list(fw); a[16] = R                                   # the block output on resid
    assert L.moe_forward_residual_rmsnorm(ok, *a) == -1
    a = list(fw); a[23] = L.moe_workspace_bytes(D(16, 256, 512, 32, 4))
    assert L.moe_forward_residual_rmsnorm(D(16, 256, 512, 32, 4), *a) == -2


def test_status_strings(moe):
    L = moe.lib()
    for s, txt in ((0, b"ok"), (-1, b"invalid argument"), (-3, b"workspace too small"),
                   (-4, b"HIP runtime error")):
        assert L.moe_status_string(s) == txt


def test_binding_raises_without_library(monkeypatch, tmp_path):
    import sparse_moe_transformer_gemm_amd as m
    monkeypatch.setattr(m, "_lib", None)
    monkeypatch.setenv("MOE_MI355X_LIB", str(tmp_path / "missing.so"))
    with pytest.raises(m.MoeError):
        m.lib()


def test_header_is_c99_and_usable_from_c(moe, tmp_path):
    """include/moe.h compiles as strict C99 (gcc -std=c99 -pedantic -Werror), and
    a C program linked against the library gets the same host-side answers as the
    Python binding (workspace and packed sizes, validation before any launch)."""
    import shutil
    import subprocess
    if shutil.which("gcc") is None:
        pytest.skip("no C compiler")
    src = tmp_path / "client.c"
    src.write_text(r'''
#include <stdio.h>
#include "moe.h"
int main(void) {
  moe_dims d = {16, 2880, 2880, 32, 4};
  moe_dims bad = {16, 2880, 2880, 3, 4};   /* k > E */
  moe_status st = moe_route(d, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL);
  printf("%zu %zu %zu %d\n", moe_workspace_bytes(d), moe_workspace_bytes(bad),
         moe_mxfp4_packed_bytes(32, 2880, 2880, 0), (int)st);
  return 0;
}
''')
    exe = tmp_path / "client"
    lib = moe.library_path()
    libdir = os.path.dirname(lib)
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror", f"-I{ROOT}/include",
           str(src), "-o", str(exe), f"-L{libdir}", f"-l:{os.path.basename(lib)}",
           f"-Wl,-rpath,{libdir}"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split()
    L = moe.lib()
    assert int(out[0]) == L.moe_workspace_bytes(moe.Dims(16, 2880, 2880, 32, 4))
    assert int(out[1]) == 0
    assert int(out[2]) == 32 * 90 * 23 * 2048
    assert int(out[3]) == -1   # MOE_ERR_INVALID_ARG: null pointers, nothing launched
