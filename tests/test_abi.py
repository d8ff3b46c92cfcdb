"""Host-side checks of the C ABI (no GPU needed, no kernel launched).

The library must load, export every function ``include/dn.h`` declares, and
reject invalid arguments on the host with the documented status codes before
it touches the GPU.
"""
import ctypes
import os
import re

import pytest

import chunkwise_delta_rule_wy_amd as dn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DN_OK, DN_EINVAL, DN_EUNSUPPORTED, DN_ENOWS, DN_EHIP, DN_ESCRATCH = range(6)


def declared_functions():
    src = open(os.path.join(ROOT, "include", "dn.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(dn_[a-z_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    return dn.load_library()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert {"dn_chunk_fwd", "dn_chunk_bwd", "dn_recurrent_step", "dn_status_str",
            "dn_chunk_fwd_workspace", "dn_chunk_bwd_workspace"} <= set(names)
    for name in names:
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for code in range(6):
        assert lib.dn_status_str(code).decode().startswith("DN_")


FAKE = 0x10000  # 16-byte aligned, never dereferenced: validation fails first


def shape(**kw):
    d = dict(B=2, T=128, H=2, Dk=64, Dv=64, n_seqs=2, chunk=64, dtype=1)
    d.update(kw)
    return dn._Shape(**d)


def fwd(lib, s, q=FAKE, k=FAKE, v=FAKE, beta=FAKE, g=None, h0=None, cu=None, o=FAKE, hT=None):
    P = ctypes.c_void_p
    return lib.dn_chunk_fwd(ctypes.byref(s), P(q), P(k), P(v), P(beta), P(g), P(h0), P(cu),
                            P(o), P(hT), None, 0, None)


def bwd(lib, s, g=None, dg=None, ws=FAKE, wsb=1 << 40, cu=None, q=FAKE):
    P = ctypes.c_void_p
    return lib.dn_chunk_bwd(ctypes.byref(s), P(q), P(FAKE), P(FAKE), P(FAKE), P(g), None, P(cu),
                            P(FAKE), None, P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(dg), None,
                            P(ws), wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(B=0), DN_EINVAL), (dict(H=0), DN_EINVAL), (dict(T=-1), DN_EINVAL),
    (dict(Dk=0), DN_EINVAL), (dict(dtype=7), DN_EINVAL), (dict(n_seqs=3), DN_EINVAL),
    (dict(chunk=16), DN_EUNSUPPORTED), (dict(chunk=32, dtype=0), DN_EUNSUPPORTED),
    (dict(chunk=128), DN_EUNSUPPORTED), (dict(Dk=96), DN_EUNSUPPORTED),
    (dict(Dk=256), DN_EUNSUPPORTED), (dict(Dv=48), DN_EUNSUPPORTED),
    (dict(Dv=2048), DN_EUNSUPPORTED), (dict(dtype=0, Dk=128), DN_EUNSUPPORTED),
    # one chunk's rows must stay within 32-bit byte offsets: 256 H max(Dk, Dv) < 2^31
    (dict(H=8192, Dv=1024), DN_EUNSUPPORTED), (dict(H=1 << 21, Dk=128, Dv=64), DN_EUNSUPPORTED),
])
def test_fwd_rejects_bad_shapes(lib, kw, code):
    assert fwd(lib, shape(**kw)) == code


def test_fwd_accepts_largest_chunk_span(lib):
    # 256 * 8191 * 1024 < 2^31: accepted by validation, which then fails on the null output
    assert fwd(lib, shape(H=8191, Dv=1024), o=None) == DN_EINVAL


def test_32_token_chunks_in_bf16(lib):
    # accepted by validation (which then fails on the null output)
    assert fwd(lib, shape(chunk=32), o=None) == DN_EINVAL
    # the training pair takes them too, with a workspace for twice the chunk states
    s32, s64 = shape(chunk=32), shape()
    need32 = lib.dn_chunk_bwd_workspace(ctypes.byref(s32))
    need64 = lib.dn_chunk_bwd_workspace(ctypes.byref(s64))
    assert need32 == 2 * need64 > 0
    assert fwd_save(lib, s32, o=None) == DN_EINVAL
    assert fwd_save(lib, s32, wsb=need64) == DN_ENOWS
    assert fwd_save(lib, shape(chunk=32, dtype=0)) == DN_EUNSUPPORTED
    assert bwd_saved(lib, s32, wsb=need64) == DN_ENOWS


def test_fwd_rejects_null_and_misaligned(lib):
    assert fwd(lib, shape(), q=None) == DN_EINVAL
    assert fwd(lib, shape(), beta=None) == DN_EINVAL
    assert fwd(lib, shape(), o=None) == DN_EINVAL
    assert fwd(lib, shape(), k=FAKE + 2) == DN_EINVAL
    # packed sequences need B == 1
    assert fwd(lib, shape(B=2, n_seqs=3), cu=FAKE) == DN_EINVAL


def test_fwd_workspace_holds_the_sequence_order(lib):
    # packed input: 4 bytes per sequence (the longest-first order), rounded to 256
    s = shape(B=1, T=1000, n_seqs=7)
    assert lib.dn_chunk_fwd_workspace(ctypes.byref(s)) == 256
    assert lib.dn_chunk_fwd_workspace(ctypes.byref(shape(B=1, T=10 ** 6, n_seqs=65536))) == 4 * 65536
    assert lib.dn_chunk_fwd_workspace(ctypes.byref(shape(B=1, T=10 ** 6, n_seqs=65537))) == 0  # own order
    assert lib.dn_chunk_fwd_workspace(ctypes.byref(shape())) == 0  # fixed length: none
    P = ctypes.c_void_p

    def call(ws, wsb):
        return lib.dn_chunk_fwd(ctypes.byref(s), P(FAKE), P(FAKE), P(FAKE), P(FAKE), None, None, P(FAKE),
                                P(FAKE), None, P(ws) if ws else None, wsb, None)
    assert call(None, 0) == DN_ENOWS
    assert call(FAKE, 255) == DN_ENOWS
    assert call(FAKE + 4, 256) == DN_ENOWS  # misaligned
    # the backward workspace: bf16 states and state gradients for at most
    # T/64 + n_seqs chunks, then chunk_base [N + 1], chunk_seq [chunks] and the
    # order [N] as int32 (each part rounded up to 256 bytes)
    nch, per = 1000 // 64 + 7, 2 * 64 * 64 * 2
    assert lib.dn_chunk_bwd_workspace(ctypes.byref(s)) == 2 * nch * per + 256 * -(-4 * (8 + nch + 7) // 256)
    big = shape(B=1, T=64 * 1000, n_seqs=1000)
    nch = 2000
    assert lib.dn_chunk_bwd_workspace(ctypes.byref(big)) == 2 * nch * per + 256 * -(-4 * (1001 + nch + 1000) // 256)


def test_bwd_validation(lib):
    s = shape()
    assert bwd(lib, s, g=FAKE, dg=None) == DN_EINVAL
    assert bwd(lib, s, g=None, dg=FAKE) == DN_EINVAL
    assert bwd(lib, s, q=None) == DN_EINVAL
    need = lib.dn_chunk_bwd_workspace(ctypes.byref(s))
    assert need > 0
    assert bwd(lib, s, wsb=need - 1) == DN_ENOWS
    assert bwd(lib, s, ws=None) == DN_ENOWS
    assert bwd(lib, shape(chunk=128)) == DN_EUNSUPPORTED
    assert bwd(lib, shape(chunk=32), q=None) == DN_EINVAL  # accepted chunk length, then the null input
    assert bwd(lib, shape(chunk=32), wsb=need) == DN_ENOWS  # twice the states of 64-token chunks
    assert bwd(lib, shape(chunk=32, dtype=0)) == DN_EUNSUPPORTED


def test_bwd_workspace_covers_varlen_bound(lib):
    # packed input: sum ceil(L/64) <= T/64 + n_seqs chunks; each chunk stores
    # its state and state gradient, H*Dk*Dv bf16 each
    s1 = shape(B=1, T=1000, n_seqs=7)
    per = 2 * 64 * 64 * 2
    assert lib.dn_chunk_bwd_workspace(ctypes.byref(s1)) >= 2 * (1000 // 64 + 7) * per


def test_step_validation(lib):
    P = ctypes.c_void_p
    f = lib.dn_recurrent_step
    assert f(0, 1, 64, 64, 1, P(FAKE), P(FAKE), P(FAKE), P(FAKE), None, P(FAKE), P(FAKE), None) == DN_EINVAL
    assert f(1, 1, 96, 64, 1, P(FAKE), P(FAKE), P(FAKE), P(FAKE), None, P(FAKE), P(FAKE), None) == DN_EUNSUPPORTED
    assert f(1, 1, 64, 64, 1, P(FAKE), P(FAKE), P(FAKE), P(FAKE), None, None, P(FAKE), None) == DN_EINVAL
    assert f(1, 1, 64, 64, 1, P(FAKE), P(FAKE), P(FAKE), P(FAKE), None, P(FAKE + 4), P(FAKE), None) == DN_EINVAL


def test_binding_refuses_cpu_tensors():
    import torch
    q = torch.zeros(1, 64, 1, 64)
    with pytest.raises(ValueError):
        dn.chunk_fwd(q, q, q, torch.zeros(1, 64, 1))


def test_longhorn_validation(lib):
    P = ctypes.c_void_p
    f = lib.dn_longhorn_eps
    assert f(0, 1, 1, 64, 1, P(FAKE), P(FAKE), P(FAKE), None) == DN_EINVAL
    assert f(1, -1, 1, 64, 1, P(FAKE), P(FAKE), P(FAKE), None) == DN_EINVAL
    assert f(1, 1, 1, 96, 1, P(FAKE), P(FAKE), P(FAKE), None) == DN_EUNSUPPORTED
    assert f(1, 1, 1, 64, 7, P(FAKE), P(FAKE), P(FAKE), None) == DN_EINVAL
    assert f(1, 1, 1, 64, 1, P(FAKE + 4), P(FAKE), P(FAKE), None) == DN_EINVAL
    assert f(1, 1, 1, 64, 1, P(FAKE), None, P(FAKE), None) == DN_EINVAL
    assert f(1, 0, 1, 64, 1, None, None, None, None) == DN_OK  # nothing to do, nothing launched
    fb = lib.dn_longhorn_eps_bwd
    assert fb(1, 1, 1, 64, 1, P(FAKE), P(FAKE), P(FAKE), P(FAKE), None, None) == DN_EINVAL
    assert fb(1, 1, 1, 64, 1, P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(FAKE + 4), None) == DN_EINVAL
    assert fb(1, 1, 1, 128, 0, P(FAKE), P(FAKE), None, P(FAKE), P(FAKE), None) == DN_EINVAL
    assert fb(2, 3, 1, 32, 0, P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(FAKE), None) == DN_EUNSUPPORTED


def test_prologue_validation(lib):
    P = ctypes.c_void_p
    f = lib.dn_prologue
    ok = [P(FAKE)] * 4
    assert f(1, 1, 1, 96, 1, *ok, 1.0, P(FAKE), P(FAKE), P(FAKE), P(FAKE), None) == DN_EUNSUPPORTED
    assert f(1, 1, 1, 64, 1, P(FAKE), P(FAKE), P(FAKE), P(FAKE), 1.0, P(FAKE), P(FAKE), P(FAKE), None, None) == DN_EINVAL
    assert f(1, 1, 1, 64, 1, P(FAKE + 8), P(FAKE), P(FAKE), None, 1.0, P(FAKE), P(FAKE), P(FAKE), None, None) == DN_EINVAL
    assert f(1, 1, 1, 64, 1, P(FAKE), P(FAKE), None, None, 1.0, P(FAKE), P(FAKE), P(FAKE), None, None) == DN_EINVAL
    assert f(1, 0, 1, 64, 1, None, None, None, None, 1.0, None, None, None, None, None) == DN_OK
    fb = lib.dn_prologue_bwd
    args = [P(FAKE)] * 3 + [None, 1.0] + [P(FAKE)] * 3 + [None] + [P(FAKE)] * 3 + [None, None]
    assert fb(1, 1, 1, 64, 1, *args[:-6], P(FAKE), *args[-5:]) == DN_EINVAL  # dg without x_in
    bad = list(args)
    bad[9] = P(FAKE + 4)  # misaligned dq_in
    assert fb(1, 1, 1, 64, 0, *bad) == DN_EINVAL


def fwd_save(lib, s, q=FAKE, o=FAKE, ws=FAKE, wsb=1 << 40):
    P = ctypes.c_void_p
    return lib.dn_chunk_fwd_save(ctypes.byref(s), P(q), P(FAKE), P(FAKE), P(FAKE), None, None, None,
                                 P(o), None, P(ws), wsb, None)


def bwd_saved(lib, s, g=None, dg=None, ws=FAKE, wsb=1 << 40):
    P = ctypes.c_void_p
    return lib.dn_chunk_bwd_saved(ctypes.byref(s), P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(g), None, None,
                                  P(FAKE), None, P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(dg), None,
                                  P(ws), wsb, None, None)


def test_saved_state_pair_validation(lib):
    s = shape()
    need = lib.dn_chunk_bwd_workspace(ctypes.byref(s))
    # the saving forward pass: bf16 only, the backward workspace, the forward's own checks
    assert fwd_save(lib, shape(dtype=0)) == DN_EUNSUPPORTED
    assert fwd_save(lib, s, q=None) == DN_EINVAL
    assert fwd_save(lib, s, o=None) == DN_EINVAL
    assert fwd_save(lib, s, o=FAKE + 8) == DN_EINVAL
    assert fwd_save(lib, s, wsb=need - 1) == DN_ENOWS
    assert fwd_save(lib, s, ws=None) == DN_ENOWS
    assert fwd_save(lib, shape(chunk=32), wsb=need) == DN_ENOWS
    # the backward pass from saved states validates as the recomputing one
    assert bwd_saved(lib, s, g=FAKE, dg=None) == DN_EINVAL
    assert bwd_saved(lib, s, g=None, dg=FAKE) == DN_EINVAL
    assert bwd_saved(lib, s, wsb=need - 1) == DN_ENOWS
    assert bwd_saved(lib, shape(dtype=0)) == DN_EUNSUPPORTED


def test_probe_library_exports_and_validates():
    # the benchmark's machine probes: own library, host-side argument checks
    path = os.path.join(ROOT, "chunkwise_delta_rule_wy_amd", "libdnprobe.so")
    plib = ctypes.CDLL(path)
    for name in ("dnp_mfma_loop", "dnp_mfma_loop_flops", "dnp_clock", "dnp_copy", "dnp_event_create",
                 "dnp_event_destroy", "dnp_event_record", "dnp_event_elapsed_ms"):
        assert hasattr(plib, name), name
    plib.dnp_event_create.argtypes = [ctypes.c_void_p]
    assert plib.dnp_event_create(None) == -1
    plib.dnp_event_elapsed_ms.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    assert plib.dnp_event_elapsed_ms(ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE), None) == -1
    plib.dnp_mfma_loop_flops.argtypes = [ctypes.c_int, ctypes.c_int]
    plib.dnp_mfma_loop_flops.restype = ctypes.c_double
    assert plib.dnp_mfma_loop_flops(2, 3) == 2 * 4 * 3 * 16 * 16384
    plib.dnp_mfma_loop.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    assert plib.dnp_mfma_loop(0, 1, ctypes.c_void_p(FAKE), None) == -1
    assert plib.dnp_mfma_loop(1, 1, None, None) == -1
    plib.dnp_clock.argtypes = [ctypes.c_ulonglong, ctypes.c_void_p, ctypes.c_void_p]
    assert plib.dnp_clock(0, ctypes.c_void_p(FAKE), None) == -1
    assert plib.dnp_clock(1 << 33, ctypes.c_void_p(FAKE), None) == -1
    plib.dnp_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p]
    assert plib.dnp_copy(ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE), 24, 1, None) == -1  # not 16-byte units
    assert plib.dnp_copy(ctypes.c_void_p(FAKE + 8), ctypes.c_void_p(FAKE), 32, 1, None) == -1
    assert plib.dnp_copy(None, ctypes.c_void_p(FAKE), 32, 1, None) == -1
    assert plib.dnp_copy(ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE), 0, 1, None) == 0  # nothing launched


def test_bwd_prologue_validation(lib):
    P = ctypes.c_void_p
    s = shape()
    f = lib.dn_chunk_bwd_prologue
    f.argtypes = ([ctypes.c_void_p] + [P] * 7 + [P, P] + [P, P, P, ctypes.c_float] + [P] * 6
                  + [P, ctypes.c_size_t, P, P])

    def call(g=None, x_in=None, q_in=FAKE, k_in=FAKE, wsb=1 << 40, dtype_shape=s):
        return f(ctypes.byref(dtype_shape), P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(g), None, None,
                 P(FAKE), None, P(q_in), P(k_in), P(x_in), 0.1, P(FAKE), P(FAKE), P(FAKE), P(FAKE),
                 P(g), None, P(FAKE), wsb, None, None)
    assert call(g=FAKE, x_in=None) == DN_EINVAL      # gate without its raw input
    assert call(g=None, x_in=FAKE) == DN_EINVAL
    assert call(q_in=None) == DN_EINVAL
    assert call(k_in=FAKE + 4) == DN_EINVAL          # misaligned raw keys
    need = lib.dn_chunk_bwd_workspace(ctypes.byref(s))
    assert call(wsb=need - 1) == DN_ENOWS
    assert call(dtype_shape=shape(dtype=0)) == DN_EUNSUPPORTED
    assert call(dtype_shape=shape(chunk=32)) == DN_EUNSUPPORTED  # the folded variants: 64-token chunks


def test_bwd_longhorn_validation(lib):
    P = ctypes.c_void_p
    s = shape()
    f = lib.dn_chunk_bwd_longhorn
    f.argtypes = [ctypes.c_void_p] + [P] * 7 + [P, P] + [P] + [P] * 6 + [P, ctypes.c_size_t, P, P]

    def call(beta=FAKE, g=None, dg=None, wsb=1 << 40, sh=s):
        return f(ctypes.byref(sh), P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(g), None, None, P(FAKE), None,
                 P(beta), P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(dg), None, P(FAKE), wsb, None, None)
    assert call(beta=None) == DN_EINVAL
    assert call(g=FAKE, dg=None) == DN_EINVAL
    need = lib.dn_chunk_bwd_workspace(ctypes.byref(s))
    assert call(wsb=need - 1) == DN_ENOWS
    assert call(sh=shape(dtype=0)) == DN_EUNSUPPORTED
    assert call(sh=shape(chunk=32)) == DN_EUNSUPPORTED  # the folded variants: 64-token chunks


def test_empty_shape_needs_no_workspace(lib):
    # T = 0 with B > 1: no chunk, so the backward workspace is empty and may be null;
    # the call then enqueues only the pass-through of dhT to dh0 (not run here:
    # validation is all this checks, with an output pointer left null on purpose)
    s = shape(T=0)
    assert lib.dn_chunk_bwd_workspace(ctypes.byref(s)) == 0
    P = ctypes.c_void_p
    st = lib.dn_chunk_fwd_save(ctypes.byref(shape(T=0, dtype=0)), P(FAKE), P(FAKE), P(FAKE), P(FAKE), None, None,
                               None, P(FAKE), None, None, 0, None)
    assert st == DN_EUNSUPPORTED  # dtype is checked before the workspace


def test_bwd_rejects_too_many_chunk_head_pairs(lib):
    # 2^24 chunks x 8192 heads exceeds the chunk-parallel kernel's grid
    s = shape(B=1, T=1 << 30, H=8192, n_seqs=1)
    assert bwd(lib, s) == DN_EUNSUPPORTED
    assert fwd_save(lib, s) == DN_EUNSUPPORTED


def test_binding_checks_caller_workspaces():
    import torch
    cpu = torch.device("cpu")
    ok = torch.empty(64, dtype=torch.uint8)
    assert dn._workspace(ok, cpu, 64, "ws") is ok
    with pytest.raises(ValueError):
        dn._workspace(ok, cpu, 65, "ws")  # too small: never silently replaced
    with pytest.raises(TypeError):
        dn._workspace(torch.empty(16, dtype=torch.float32), cpu, 8, "ws")
    with pytest.raises(TypeError):
        dn._workspace(torch.empty(64, dtype=torch.uint8)[::2], cpu, 8, "ws")
    with pytest.raises(ValueError):
        dn._workspace(ok, torch.device("cuda:0"), 8, "ws")  # on another device than the inputs


def test_short_conv_validation(lib):
    P = ctypes.c_void_p
    f, fb = lib.dn_short_conv, lib.dn_short_conv_bwd
    ok = [P(FAKE), P(FAKE), None, P(FAKE), None]  # x, w, cu, y, stream
    assert f(1, 4, 2, 12, 4, 1, 1, *ok) == DN_EUNSUPPORTED   # D not a multiple of 8
    assert f(1, 4, 2, 16, 5, 1, 1, *ok) == DN_EUNSUPPORTED   # W beyond 4
    assert f(1, 4, 2, 16, 0, 1, 1, *ok) == DN_EUNSUPPORTED
    assert f(2, 4, 2, 16, 4, 1, 1, *ok) == DN_EINVAL         # n_seqs != B without cu_seqlens
    assert f(2, 4, 2, 16, 4, 2, 1, P(FAKE), P(FAKE), P(FAKE), P(FAKE), None) == DN_EINVAL  # packed needs B == 1
    assert f(1, 4, 2, 16, 4, 1, 5, *ok) == DN_EINVAL         # dtype
    assert f(1, 4, 2, 16, 4, 1, 1, P(FAKE + 8), P(FAKE), None, P(FAKE), None) == DN_EINVAL  # misaligned x
    assert f(1, 4, 2, 16, 4, 1, 1, P(FAKE), None, None, P(FAKE), None) == DN_EINVAL
    assert f(1, 0, 2, 16, 4, 1, 1, None, None, None, None, None) == DN_OK  # nothing to do
    okb = [P(FAKE), P(FAKE), None, P(FAKE), P(FAKE), P(FAKE), None]  # x, w, cu, dy, dx, dw, stream
    assert fb(1, 4, 2, 16, 4, 1, 0, *okb[:5], None, None) == DN_EINVAL  # dw is required
    assert fb(1, 4, 2, 16, 4, 1, 0, P(FAKE), P(FAKE), None, P(FAKE), P(FAKE + 4), P(FAKE), None) == DN_EINVAL
    assert fb(1, 4, 2, 24, 3, 1, 0, P(FAKE), P(FAKE), None, None, P(FAKE), P(FAKE), None) == DN_EINVAL
    assert fb(1, 4, 2, 20, 3, 1, 0, *okb) == DN_EUNSUPPORTED


def test_short_conv_l2_validation(lib):
    P = ctypes.c_void_p
    f, fb = lib.dn_short_conv_l2, lib.dn_short_conv_l2_bwd
    assert f(1, 4, 2, 32, 4, 1, 1, P(FAKE), P(FAKE), None, P(FAKE), None) == DN_EUNSUPPORTED  # D not 64 or 128
    assert f(1, 4, 2, 128, 5, 1, 1, P(FAKE), P(FAKE), None, P(FAKE), None) == DN_EUNSUPPORTED
    assert f(1, 4, 2, 128, 4, 1, 1, P(FAKE + 8), P(FAKE), None, P(FAKE), None) == DN_EINVAL
    assert f(1, 0, 2, 128, 4, 1, 1, None, None, None, None, None) == DN_OK
    assert fb(1, 4, 2, 64, 4, 1, 0, P(FAKE), P(FAKE), None, P(FAKE), P(FAKE), None, None) == DN_EINVAL
    assert fb(1, 4, 2, 256, 4, 1, 0, P(FAKE), P(FAKE), None, P(FAKE), P(FAKE), P(FAKE), None) == DN_EUNSUPPORTED


def test_short_conv_grid_limits(lib):
    # channel groups of 512 sit on the grid's y axis (at most 65535 of them); tokens on x
    P = ctypes.c_void_p
    f = lib.dn_short_conv
    assert f(1, 4, 262144, 128, 4, 1, 1, P(FAKE), P(FAKE), None, P(FAKE), None) == DN_EUNSUPPORTED
    assert f(1, 4, 262141, 128, 4, 1, 1, P(FAKE), P(FAKE), None, P(FAKE), None) == DN_EUNSUPPORTED
    assert f(1, 4, 262140, 128, 4, 1, 1, None, P(FAKE), None, P(FAKE), None) == DN_EINVAL  # 65535 groups: x checked next


def noalloc(lib, s, g=None, dg=None, q=FAKE):
    P = ctypes.c_void_p
    return lib.dn_chunk_bwd_noalloc(ctypes.byref(s), P(q), P(FAKE), P(FAKE), P(FAKE), P(g), None, None,
                                    P(FAKE), None, P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(dg), P(FAKE), None)


def test_noalloc_validates_before_touching_the_device(lib):
    # argument errors, then the size limit of the static buffer (64 MiB), are
    # reported before the device is looked up or anything is enqueued
    assert lib.dn_chunk_bwd_noalloc(None, *([None] * 15), None) == DN_EINVAL
    assert noalloc(lib, shape(B=0)) == DN_EINVAL
    assert noalloc(lib, shape(), g=FAKE) == DN_EINVAL          # g without dg
    assert noalloc(lib, shape(), q=FAKE + 4) == DN_EINVAL      # misaligned
    assert noalloc(lib, shape(dtype=0)) == DN_EUNSUPPORTED     # bf16 only
    big = shape(B=4, T=4096, H=16, Dk=128, Dv=256, n_seqs=4)
    assert lib.dn_chunk_bwd_workspace(ctypes.byref(big)) > 64 << 20
    assert noalloc(lib, big, g=FAKE, dg=FAKE) == DN_ESCRATCH
    assert lib.dn_status_str(DN_ESCRATCH).decode().startswith("DN_ESCRATCH")
