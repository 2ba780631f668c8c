"""C-ABI checks that need no GPU: the library loads, exports every function
include/fp4q.h declares, and rejects invalid arguments on the host before any
HIP call (status codes as documented in the header)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp4q.h")

INVALID, UNSUPPORTED, WORKSPACE, HIP_ERR = -1, -2, -3, -4


def declared_functions(header=HEADER):
    src = open(header).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(fp4q_[a-z_0-9]+)\s*\(", src)))


@pytest.fixture(scope="module")
def L():
    from fp4_w4a4_quantized_amd import binding
    return binding.lib()


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert {"fp4q_quantize", "fp4q_gemm", "fp4q_grouped_gemm", "fp4q_error_decompose"} <= set(names)
    for n in names:
        assert hasattr(L, n), n


def test_peaks_library_exports_and_rejects():
    """libfp4q_peaks.so (the attainable-peak microbenchmarks) exports what
    include/fp4q_peaks.h declares and rejects bad arguments on the host."""
    path = os.path.join(ROOT, "fp4_w4a4_quantized_amd", "libfp4q_peaks.so")
    P = ctypes.CDLL(path)
    names = declared_functions(os.path.join(ROOT, "include", "fp4q_peaks.h"))
    assert {"fp4q_peak_mfma", "fp4q_peak_read", "fp4q_peak_copy"} <= set(names)
    for n in names:
        assert hasattr(P, n), n
    P.fp4q_peak_mfma.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                 ctypes.POINTER(ctypes.c_double), ctypes.c_void_p]
    P.fp4q_peak_read.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int32,
                                 ctypes.c_void_p, ctypes.c_void_p]
    P.fp4q_peak_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint64,
                                 ctypes.c_int32, ctypes.c_void_p]
    P.fp4q_peak_mfma_out_floats.restype = ctypes.c_int64
    fl = ctypes.c_double()
    assert P.fp4q_peak_mfma(2, 4, 1, A, ctypes.byref(fl), None) == -1      # bad kind
    assert P.fp4q_peak_mfma(0, 0, 1, A, ctypes.byref(fl), None) == -1      # no blocks
    assert P.fp4q_peak_mfma(0, 4, 1, None, ctypes.byref(fl), None) == -1   # no output
    assert P.fp4q_peak_read(A, 15, 4, B, None) == -1                       # not 16-byte units
    assert P.fp4q_peak_read(ctypes.c_void_p(0x10008), 64, 4, B, None) == -1  # misaligned
    assert P.fp4q_peak_copy(A, B, 64, 0, None) == -1
    assert P.fp4q_peak_mfma_out_floats(4) == 4 * 256


def test_status_strings(L):
    assert L.fp4q_status_str(0) == b"ok"
    assert L.fp4q_status_str(-4) == b"HIP error"
    assert L.fp4q_status_str(12345) == b"unknown status"
    assert L.fp4q_last_hip_error() == 0


def test_workspace_queries(L):
    assert L.fp4q_quantize_workspace_bytes(0, 100, 64, 5) >= 20
    assert L.fp4q_quantize_workspace_bytes(0, 100, 64, 3000) >= 12000
    assert L.fp4q_quantize_workspace_bytes(1, 100, 64, 5) == 0
    assert L.fp4q_error_decompose_workspace_bytes(8192, 4096) >= 256


# Fake, never-dereferenced device addresses: validation fails before use.
A = ctypes.c_void_p(0x10000)
B = ctypes.c_void_p(0x20000)


def q(L, fmt=0, x=A, rows=4, cols=64, ldx=64, off=None, G=1, chan=None, nS=0, qq=B, sc=B,
      ts=B, R=None, ws=A, wsb=64, layout=0):
    return L.fp4q_quantize(fmt, layout, x, rows, cols, ldx, off, G, chan, nS, qq, sc, ts, R, ws,
                           wsb, None)


def test_quantize_rejects(L):
    assert q(L, fmt=7) == INVALID
    assert q(L, cols=40) == INVALID              # not a multiple of 16
    assert q(L, fmt=1, ts=None, cols=48) == INVALID   # MXFP4 needs cols % 32
    assert q(L, ldx=32) == INVALID               # ldx < cols
    assert q(L, ldx=68) == INVALID               # ldx % 8
    assert q(L, rows=-1) == INVALID
    assert q(L, G=0) == INVALID
    assert q(L, G=3, off=None) == INVALID
    assert q(L, nS=2, chan=None, R=B) == INVALID
    assert q(L, nS=2, chan=A, R=None) == INVALID
    assert q(L, nS=65, chan=A, R=B) == INVALID   # more channels than columns
    assert q(L, ts=None) == INVALID              # NVFP4 needs the tensor scale
    assert q(L, fmt=1) == INVALID                # MXFP4 takes none
    assert q(L, x=None) == INVALID
    assert q(L, x=ctypes.c_void_p(0x10008)) == INVALID   # misaligned
    assert q(L, ws=None) == WORKSPACE
    assert q(L, wsb=2) == WORKSPACE
    assert q(L, rows=1 << 28) == UNSUPPORTED     # 2^31 chunks of 8 elements
    assert q(L, layout=2) == INVALID
    assert q(L, layout=1, cols=64) == INVALID    # tiled needs cols % 128
    assert q(L, layout=1, cols=128, ldx=128, sc=ctypes.c_void_p(0x20002)) == INVALID
    assert q(L, sc=ctypes.c_void_p(0x20002)) == INVALID  # scales 4-byte aligned


def test_quantize_workspace_alignment(L):
    """The NVFP4 workspace holds 64-bit exchange slots: 8-byte alignment and
    the 512-byte state block in front of the amax words."""
    need = L.fp4q_quantize_workspace_bytes(0, 4, 64, 1)
    assert need >= 512 + 4 * 1024
    assert L.fp4q_quantize_workspace_bytes(0, 4, 64, 5000) >= 512 + 4 * 5000
    assert q(L, ws=ctypes.c_void_p(0x10004), wsb=need) == WORKSPACE
    assert q(L, wsb=need - 1) == WORKSPACE


def test_test_hook_rejects(L):
    assert L.fp4q_test_hook(99, 0) == INVALID
    assert L.fp4q_test_hook(1, 0) == INVALID        # no error code to report
    assert L.fp4q_test_hook(1, -5) == INVALID
    assert L.fp4q_test_hook(2, -1) == INVALID       # negative spin limit
    assert L.fp4q_test_hook(3, -2) == INVALID       # skip slot below -1
    assert L.fp4q_test_hook(0, 0) == 0


def test_injected_launch_failure(L):
    """The test fault hook makes the launch path report FP4Q_ERR_HIP with the
    given hipError_t, without launching (the pointers here are fake); a call
    that fails its argument checks first leaves the hook armed, and the hook
    fires once."""
    need = L.fp4q_quantize_workspace_bytes(0, 4, 64, 1)
    try:
        assert L.fp4q_test_hook(1, 719) == 0
        assert q(L, fmt=7) == INVALID                 # rejected before the hook
        assert q(L, wsb=need) == HIP_ERR               # the injected failure
        assert L.fp4q_last_hip_error() == 719
        assert L.fp4q_status_str(HIP_ERR) == b"HIP error"
        # the GEMM, the decomposition and the status query take the same path
        assert L.fp4q_test_hook(1, 98) == 0
        assert g(L) == HIP_ERR
        assert L.fp4q_last_hip_error() == 98
        assert L.fp4q_test_hook(1, 700) == 0
        ws = L.fp4q_error_decompose_workspace_bytes(16, 64)
        assert L.fp4q_error_decompose(1, A, 16, 64, 64, B, A, ws, None) == HIP_ERR
        assert L.fp4q_last_hip_error() == 700
        st = ctypes.c_int32(-1)
        assert L.fp4q_test_hook(1, 4) == 0
        assert L.fp4q_quantize_status(A, need, ctypes.byref(st), None) == HIP_ERR
        assert L.fp4q_last_hip_error() == 4 and st.value == -1
    finally:
        L.fp4q_test_hook(0, 0)


def test_qdq_fallback_rejects(L):
    P = ctypes.c_void_p
    L.fp4q_qdq_fallback.argtypes = [ctypes.c_int, P, ctypes.c_int64, ctypes.c_int64,
                                    ctypes.c_int64, P, ctypes.c_int64, P, P, ctypes.c_size_t, P]
    need = L.fp4q_qdq_fallback_workspace_bytes(0, 4, 64)
    assert need > 0 and L.fp4q_qdq_fallback_workspace_bytes(1, 4, 64) == 0

    def f(fmt=0, x=A, rows=4, cols=64, ldx=64, y=B, ldy=64, n=None, ws=A, wsb=need):
        return L.fp4q_qdq_fallback(fmt, x, rows, cols, ldx, y, ldy, n, ws, wsb, None)
    assert f(fmt=3) == INVALID
    assert f(cols=40) == INVALID
    assert f(fmt=1, cols=48) == INVALID            # MXFP4 blocks of 32
    assert f(ldx=60) == INVALID
    assert f(ldy=60) == INVALID
    assert f(ldy=66) == INVALID                    # rows of float4 stores
    assert f(y=ctypes.c_void_p(0x20008)) == INVALID
    assert f(x=None) == INVALID
    assert f(n=ctypes.c_void_p(0x30004)) == INVALID
    assert f(ws=None) == WORKSPACE
    assert f(wsb=need - 1) == WORKSPACE
    assert f(rows=1 << 28) == UNSUPPORTED
    assert f(rows=0, n=None) == 0                  # nothing to do, no HIP call
    try:
        assert L.fp4q_test_hook(1, 77) == 0
        assert f() == HIP_ERR and L.fp4q_last_hip_error() == 77
    finally:
        L.fp4q_test_hook(0, 0)


def test_gemm_decode_fused_rejects(L):
    P, i64 = ctypes.c_void_p, ctypes.c_int64
    L.fp4q_gemm_decode_fused.argtypes = [ctypes.c_int, ctypes.c_int, i64, i64, i64, P, i64, P, P,
                                         P, P, ctypes.c_int32, P, ctypes.c_size_t, P, ctypes.c_int,
                                         i64, P, P, P, P, P]

    def f(fmt=0, layout=1, M=64, N=256, K=2048, x=A, ldx=2048, bq=B, bs=B, bts=B, chan=None,
          nS=0, cw=None, cwb=0, y=A, dt=0, ldy=256, qo=None, so=None, tso=None, ro=None):
        return L.fp4q_gemm_decode_fused(fmt, layout, M, N, K, x, ldx, bq, bs, bts, chan, nS, cw,
                                        cwb, y, dt, ldy, qo, so, tso, ro, None)
    assert f(fmt=2) == INVALID
    assert f(ldx=2000) == INVALID
    assert f(ldy=100) == INVALID
    assert f(bts=None) == INVALID
    assert f(nS=4, chan=None) == INVALID
    assert f(qo=B) == INVALID                     # optional outputs all or none
    assert f(x=ctypes.c_void_p(0x10008)) == INVALID
    assert f(fmt=1) == UNSUPPORTED                # NVFP4 only
    assert f(M=65) == UNSUPPORTED
    assert f(K=2176, ldx=2176) == UNSUPPORTED     # at most 16 K steps
    assert f(K=2000, ldx=2000) == UNSUPPORTED
    assert f(nS=65, chan=A) == UNSUPPORTED
    assert f(nS=8, chan=A) == WORKSPACE           # prepared weights missing
    assert f(nS=8, chan=A, cw=A, cwb=16) == WORKSPACE
    assert f(M=0) == 0                            # nothing to do, no HIP call
    try:
        assert L.fp4q_test_hook(1, 55) == 0
        assert f() == HIP_ERR and L.fp4q_last_hip_error() == 55
    finally:
        L.fp4q_test_hook(0, 0)


def test_grouped_gemm_gather_rejects(L):
    def f(fmt=0, wl=0, rows=64, N=256, K=256, off=A, G=2, src=B, tokens=10, aq=A, as_=A, ats=B,
          bq=B, bs=B, bts=B, chan=None, nS=0, R=None, cw=None, cwb=0, y=A, dt=0):
        return L.fp4q_grouped_gemm_gather(fmt, wl, rows, N, K, off, G, src, tokens, aq, as_, ats,
                                          bq, bs, bts, chan, nS, R, cw, cwb, y, dt, None)
    assert f(src=None) == INVALID
    assert f(tokens=0) == INVALID
    assert f(off=None) == INVALID
    assert f(N=200) == UNSUPPORTED                 # the 256-tile kernel only
    assert f(K=200) == INVALID                     # not a multiple of the block
    assert f(G=3000) == UNSUPPORTED
    assert f(nS=8, chan=A, R=B) == WORKSPACE       # prepared weights missing
    assert f(wl=2) == INVALID                      # no such weight layout
    assert f(wl=1, fmt=1, ats=None, bts=None) == UNSUPPORTED  # tiled weights: NVFP4 only
    # tiled weights keep 32-bit offsets into the token matrix's codes
    assert f(wl=1, K=512, tokens=1 << 24) == UNSUPPORTED
    assert f(wl=1, rows=0) == 0
    assert f(rows=0) == 0
    try:
        assert L.fp4q_test_hook(1, 33) == 0
        assert f() == HIP_ERR and L.fp4q_last_hip_error() == 33
    finally:
        L.fp4q_test_hook(0, 0)


def test_grouped_gemm_residual_fp4_rejects(L):
    def f(fmt=0, wl=0, rows=64, N=256, K=256, off=A, G=2, aq=A, as_=A, ats=B, bq=B, bs=B, bts=B,
          chan=A, nS=16, rq=A, rs=A, rts=B, y=A, dt=0, ws=A, wsb=1 << 30):
        return L.fp4q_grouped_gemm_residual_fp4(fmt, wl, rows, N, K, off, G, aq, as_, ats, bq, bs,
                                                bts, chan, nS, rq, rs, rts, y, dt, ws, wsb, None)
    assert f(nS=8) == INVALID                      # not a multiple of the block
    assert f(rq=None) == INVALID
    assert f(rts=None) == INVALID                  # NVFP4: one residual scale per group
    assert f(fmt=1, ats=None, bts=None, nS=32) == INVALID   # MXFP4 takes none
    assert f(off=None) == INVALID
    assert f(G=3000) == UNSUPPORTED
    assert f(ws=None) == WORKSPACE
    assert f(wsb=16) == WORKSPACE
    assert f(wl=2) == INVALID
    assert f(wl=1, N=128) == UNSUPPORTED           # tiled weights: the 128 x 512 kernel only
    assert f(wl=1, fmt=1, ats=None, bts=None, nS=32, rts=None) == UNSUPPORTED
    assert f(rows=0) == 0
    need = L.fp4q_grouped_gemm_residual_fp4_workspace_bytes(0, 0, 64, 256, 256, 2, 16)
    assert need >= 64 * 16 * 2                     # the decoded residual at least
    # tiled weights: the compensation weights are always gathered
    # the compensation weights are gathered for either weight layout
    need_t = L.fp4q_grouped_gemm_residual_fp4_workspace_bytes(0, 1, 64, 256, 256, 2, 16)
    assert need_t == need == 64 * 16 * 2 + 2 * (256 // 16) * 1024
    try:
        assert L.fp4q_test_hook(1, 34) == 0
        assert f() == HIP_ERR and L.fp4q_last_hip_error() == 34
    finally:
        L.fp4q_test_hook(0, 0)


def test_quantize_status_rejects(L):
    need = L.fp4q_quantize_workspace_bytes(0, 4, 64, 1)
    st = ctypes.c_int32(0)
    assert L.fp4q_quantize_status(A, need, None, None) == INVALID
    assert L.fp4q_quantize_status(None, need, ctypes.byref(st), None) == WORKSPACE
    assert L.fp4q_quantize_status(ctypes.c_void_p(0x10004), need, ctypes.byref(st), None) == WORKSPACE
    assert L.fp4q_quantize_status(A, 100, ctypes.byref(st), None) == WORKSPACE


def g(L, fmt=0, M=4, N=8, K=256, aq=A, as_=A, ats=B, bq=B, bs=B, bts=B, chan=None, nS=0, R=None,
      y=A, dt=0, ldy=8, layout=0, ws=None, wsb=0):
    return L.fp4q_gemm(fmt, layout, M, N, K, aq, as_, ats, bq, bs, bts, chan, nS, R, y, dt, ldy,
                       ws, wsb, None)


def test_gemm_rejects(L):
    assert g(L, fmt=2) == INVALID
    assert g(L, dt=5) == INVALID
    assert g(L, K=40) == INVALID
    assert g(L, K=144) == UNSUPPORTED            # valid NVFP4 K, not a multiple of 128
    assert g(L, ldy=4) == INVALID
    assert g(L, ats=None) == INVALID
    assert g(L, fmt=1) == INVALID                # MXFP4 with tensor scales
    assert g(L, nS=3, chan=A, R=None) == INVALID
    assert g(L, nS=300, chan=A, R=B) == INVALID
    assert g(L, aq=ctypes.c_void_p(0x10004)) == INVALID
    assert g(L, y=None) == INVALID
    assert g(L, layout=5) == INVALID
    assert g(L, layout=1, K=144) == UNSUPPORTED
    assert g(L, nS=8, chan=A, R=ctypes.c_void_p(0x20008)) == INVALID   # resid 16-byte aligned
    # the large-tile kernels stream B_S, gathered into the workspace first
    need = L.fp4q_gemm_workspace_bytes(0, 1, 512, 512, 256, 128)
    assert need == (512 // 16) * 4 * 1024
    assert L.fp4q_gemm_workspace_bytes(0, 1, 512, 512, 256, 104) == (512 // 16) * 4 * 1024
    assert L.fp4q_gemm_workspace_bytes(0, 1, 512, 500, 256, 136) == (512 // 16) * 5 * 1024
    assert L.fp4q_gemm_workspace_bytes(0, 1, 512, 512, 256, 0) == 0
    for fmt in (0, 1):
        for nS in (8, 32, 40, 96):
            assert (L.fp4q_gemm_workspace_bytes(fmt, 1, 512, 512, 256, nS)
                    == (512 // 16) * ((nS + 31) // 32) * 1024)
    assert L.fp4q_gemm_workspace_bytes(0, 1, 64, 11008, 2048, 128) == 0   # decode shape
    assert L.fp4q_gemm_workspace_bytes(0, 1, 512, 512, 256, 12) == 0      # |S| % 8: other path
    big = dict(M=512, N=512, K=256, nS=128, chan=A, R=B, ldy=512)
    assert g(L, **big) == WORKSPACE
    assert g(L, **big, ws=A, wsb=need - 1) == WORKSPACE
    assert g(L, **big, ws=ctypes.c_void_p(0x10008), wsb=need) == WORKSPACE


def _packed(L, fmt, layout, rows, cols):
    cb, sb = ctypes.c_size_t(7), ctypes.c_size_t(7)
    rc = L.fp4q_packed_bytes(fmt, layout, rows, cols, ctypes.byref(cb), ctypes.byref(sb))
    return rc, cb.value, sb.value


def test_packed_bytes(L):
    # row-major: exact sizes
    assert _packed(L, 0, 0, 5, 64) == (0, 160, 20)
    assert _packed(L, 1, 0, 5, 64) == (0, 160, 10)
    # tiled: codes padded to 16 rows, scales to 64 rows
    assert _packed(L, 0, 1, 5, 256) == (0, 16 * 128, 64 * 16)
    assert _packed(L, 1, 1, 5, 256) == (0, 16 * 128, 64 * 8)
    assert _packed(L, 0, 1, 64, 128) == (0, 64 * 64, 64 * 8)
    assert _packed(L, 0, 1, 65, 128) == (0, 80 * 64, 128 * 8)
    assert _packed(L, 0, 1, 0, 128) == (0, 0, 0)
    assert _packed(L, 0, 1, 5, 64)[0] == INVALID     # tiled needs cols % 128
    assert _packed(L, 1, 0, 5, 48)[0] == INVALID     # MXFP4 needs cols % 32
    assert _packed(L, 0, 3, 5, 128)[0] == INVALID
    assert _packed(L, 0, 0, -1, 128)[0] == INVALID


def test_grouped_gemm_rejects(L):
    f = L.fp4q_grouped_gemm

    def gg(fmt=0, wl=0, rows=10, N=8, K=256, off=A, G=2, ats=B, bts=B, chan=None, nS=0, R=None,
           ws=None, wsb=0):
        return f(fmt, wl, rows, N, K, off, G, A, A, ats, B, B, bts, chan, nS, R, A, 0, ws, wsb,
                 None)

    assert gg(off=None) == INVALID
    assert gg(G=0) == INVALID
    assert gg(G=5000) == UNSUPPORTED
    assert gg(fmt=1, bts=None) == INVALID        # MXFP4 takes no tensor scales
    # the staged 256-column path gathers every group's compensation weights
    # when there are more than 96 channels
    need = L.fp4q_grouped_gemm_workspace_bytes(0, 0, 1000, 512, 256, 4, 128)
    assert need == 4 * (512 // 16) * 4 * 1024
    # every group's compensation weights are gathered at any channel count
    assert L.fp4q_grouped_gemm_workspace_bytes(0, 0, 1000, 512, 256, 4, 32) == 4 * 32 * 1024
    assert L.fp4q_grouped_gemm_workspace_bytes(1, 0, 1000, 512, 256, 4, 32) == 4 * 32 * 1024
    assert L.fp4q_grouped_gemm_workspace_bytes(0, 0, 1000, 128, 256, 4, 128) == 0   # N < 256
    assert L.fp4q_grouped_gemm_workspace_bytes(0, 0, 1000, 512, 256, 4, 0) == 0
    # tiled weights gather the compensation weights for any channel count
    assert L.fp4q_grouped_gemm_workspace_bytes(0, 1, 1000, 512, 256, 4, 32) == 4 * 32 * 1024
    assert gg(wl=2) == INVALID
    assert gg(wl=1) == UNSUPPORTED               # N < 256: the general kernel, row-major only
    assert gg(wl=1, N=512, K=192) == UNSUPPORTED   # K % 128 (checked as for row-major)
    assert gg(wl=1, N=512, chan=A, nS=32, R=B) == WORKSPACE
    big = dict(rows=1000, N=512, K=256, G=4, chan=A, nS=128, R=B)
    assert gg(**big) == WORKSPACE
    assert gg(**big, ws=A, wsb=need - 16) == WORKSPACE


def test_error_decompose_rejects(L):
    f = L.fp4q_error_decompose
    assert f(1, A, 4, 48, 48, B, A, 1 << 20, None) == INVALID     # cols % 32
    assert f(1, A, 4, 64, 64, None, A, 1 << 20, None) == INVALID  # no output
    assert f(0, A, 4, 40, 40, B, A, 1 << 20, None) == INVALID  # NVFP4: whole 16-blocks
    assert f(2, A, 4, 64, 64, B, A, 1 << 20, None) == INVALID  # no such format
    assert f(1, A, 4, 64, 64, B, None, 0, None) == WORKSPACE
    assert f(1, A, 4, 64, 64, B, A, 8, None) == WORKSPACE


def g4(L, fmt=0, M=4, N=8, K=256, aq=A, as_=A, ats=B, bq=B, bs=B, bts=B, chan=A, nS=16, rq=B,
       rs=B, rts=B, y=A, dt=0, ldy=8, layout=0, ws=A, wsb=1 << 20):
    return L.fp4q_gemm_residual_fp4(fmt, layout, M, N, K, aq, as_, ats, bq, bs, bts, chan, nS, rq,
                                    rs, rts, y, dt, ldy, ws, wsb, None)


def test_gemm_residual_fp4_rejects(L):
    assert g4(L, nS=8) == INVALID                 # not a whole NVFP4 block of channels
    assert g4(L, fmt=1, ats=None, bts=None, rts=None, nS=16) == INVALID   # MXFP4 blocks are 32
    assert g4(L, rts=None) == INVALID             # NVFP4 residual needs its tensor scale
    assert g4(L, fmt=1, ats=None, bts=None, nS=32) == INVALID             # MXFP4 takes none
    assert g4(L, rq=None) == INVALID
    assert g4(L, rs=None) == INVALID
    assert g4(L, ws=None) == WORKSPACE
    assert g4(L, wsb=64) == WORKSPACE
    assert g4(L, ws=ctypes.c_void_p(0x10008)) == WORKSPACE                 # misaligned
    assert g4(L, layout=3) == INVALID
    assert g4(L, chan=None) == INVALID
    # workspace: the decoded residual (256-byte rounded) then the GEMM's own
    assert L.fp4q_gemm_residual_fp4_workspace_bytes(0, 0, 4, 8, 256, 16) == 256
    assert (L.fp4q_gemm_residual_fp4_workspace_bytes(1, 1, 512, 512, 256, 128)
            == 512 * 128 * 2 + L.fp4q_gemm_workspace_bytes(1, 1, 512, 512, 256, 128))
    assert L.fp4q_gemm_residual_fp4_workspace_bytes(0, 0, 4, 8, 256, 0) == 0


def sel(L, fmt=0, layout=0, x=A, rows=4, cols=64, ldx=64, qq=B, sc=B, ts=B, k=8, chan=A, R=B,
        ws=A, wsb=1 << 20):
    return L.fp4q_select_channels(fmt, layout, x, rows, cols, ldx, qq, sc, ts, k, chan, R, ws,
                                  wsb, None)


def test_select_channels_rejects(L):
    assert sel(L, fmt=2) == INVALID
    assert sel(L, layout=3) == INVALID
    assert sel(L, cols=40, ldx=40) == INVALID           # not whole NVFP4 blocks
    assert sel(L, fmt=1, ts=None, cols=48, ldx=48) == INVALID  # nor MXFP4 blocks
    assert sel(L, layout=1) == INVALID                  # tiled needs cols % 128 == 0
    assert sel(L, ldx=60) == INVALID
    assert sel(L, ldx=68) == INVALID                    # ldx % 8
    assert sel(L, k=-1) == INVALID
    assert sel(L, k=65) == INVALID                      # more channels than columns
    assert sel(L, ts=None) == INVALID                   # NVFP4 needs its tensor scale
    assert sel(L, fmt=1) == INVALID                     # MXFP4 takes none
    assert sel(L, chan=None) == INVALID
    assert sel(L, R=None) == INVALID
    assert sel(L, qq=None) == INVALID
    assert sel(L, sc=None) == INVALID
    assert sel(L, x=ctypes.c_void_p(0x10008)) == INVALID   # x 16-byte aligned
    assert sel(L, qq=ctypes.c_void_p(0x20002)) == INVALID  # codes 4-byte aligned
    assert sel(L, ws=None) == WORKSPACE
    assert sel(L, wsb=16) == WORKSPACE
    assert sel(L, ws=ctypes.c_void_p(0x10008)) == WORKSPACE
    assert sel(L, rows=1 << 27, cols=64, k=32) == UNSUPPORTED   # rows * k >= 2^31
    # nothing to choose: accepted without launching anything
    assert sel(L, k=0, chan=None, R=None, ws=None, wsb=0) == 0
    assert sel(L, rows=0, x=None, qq=None, sc=None, R=None, k=0, chan=None) == 0


def qsel(L, fmt=0, layout=0, x=A, rows=4, cols=64, ldx=64, k=8, qq=B, sc=B, ts=B, chan=A, R=B,
         ws=A, wsb=1 << 20):
    return L.fp4q_quantize_select(fmt, layout, x, rows, cols, ldx, k, qq, sc, ts, chan, R, ws, wsb,
                                  None)


def test_quantize_select_rejects(L):
    assert qsel(L, fmt=2) == INVALID
    assert qsel(L, layout=3) == INVALID
    assert qsel(L, cols=40, ldx=40) == INVALID           # not whole NVFP4 blocks
    assert qsel(L, layout=1) == INVALID                  # tiled needs cols % 128 == 0
    assert qsel(L, ldx=68) == INVALID                    # ldx % 8
    assert qsel(L, k=-1) == INVALID
    assert qsel(L, k=65) == INVALID                      # more channels than columns
    assert qsel(L, ts=None) == INVALID                   # NVFP4 writes its tensor scale
    assert qsel(L, fmt=1) == INVALID                     # MXFP4 has none
    assert qsel(L, chan=None) == INVALID
    assert qsel(L, R=None) == INVALID
    assert qsel(L, qq=None) == INVALID
    assert qsel(L, x=ctypes.c_void_p(0x10008)) == INVALID   # x 16-byte aligned
    assert qsel(L, qq=ctypes.c_void_p(0x20002)) == INVALID  # codes 4-byte aligned
    assert qsel(L, ws=None) == WORKSPACE
    assert qsel(L, wsb=16) == WORKSPACE
    assert qsel(L, ws=ctypes.c_void_p(0x10008)) == WORKSPACE
    assert qsel(L, rows=1 << 27, cols=64, k=32) == UNSUPPORTED   # rows * k >= 2^31


def test_quantize_select_workspace(L):
    f = L.fp4q_quantize_select_workspace_bytes
    q = L.fp4q_quantize_workspace_bytes
    rq = lambda b: (b + 255) // 256 * 256
    # the quantize workspace, then the larger of the two selection paths'
    assert f(0, 0, 4, 64) >= rq(q(0, 4, 64, 1)) + L.fp4q_select_channels_workspace_bytes(4, 64)
    assert f(1, 0, 4, 64) >= L.fp4q_select_channels_workspace_bytes(4, 64)
    # prefill activations, tiled: 64 bands of 128 rows, scores [64, 4096] BF16
    big = f(0, 1, 8192, 4096)
    assert big >= rq(q(0, 8192, 4096, 1)) + 64 * 4096 * 2 and big % 256 == 0
    assert f(0, 0, -1, 64) == 0 and f(0, 0, 4, 0) == 0 and f(5, 0, 4, 64) == 0


def test_select_channels_grouped_rejects(L):
    P, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
    L.fp4q_select_channels_grouped.argtypes = [ctypes.c_int, P, i64, i64, i64, P, i32, P, P, P,
                                               i32, P, P, P, sz, P]

    def f(fmt=0, x=A, rows=32, cols=64, ldx=64, off=A, G=2, qq=A, sc=A, ts=B, k=8, chan=A, R=A,
          ws=A, wsb=1 << 20):
        return L.fp4q_select_channels_grouped(fmt, x, rows, cols, ldx, off, G, qq, sc, ts, k,
                                              chan, R, ws, wsb, None)
    assert f(fmt=2) == INVALID
    assert f(cols=40, ldx=40) == INVALID           # not whole NVFP4 blocks
    assert f(k=65) == INVALID
    assert f(off=None) == INVALID
    assert f(G=0) == INVALID
    assert f(G=3000) == UNSUPPORTED
    assert f(ts=None) == INVALID                   # NVFP4: one tensor scale per group
    assert f(fmt=1) == INVALID                     # MXFP4 takes none
    assert f(cols=32768, ldx=32768) == UNSUPPORTED  # more columns than the pick keeps in LDS
    assert f(ws=None) == WORKSPACE
    assert f(wsb=16) == WORKSPACE
    assert f(k=0, chan=None, R=None, ws=None, wsb=0) == 0
    assert L.fp4q_select_channels_grouped_workspace_bytes(32, 64, 2) >= 2 * 64 * 2


def test_select_channels_workspace(L):
    f = L.fp4q_select_channels_workspace_bytes
    assert f(4, 64) == 256                     # one row block: its partial maxima
    # many row blocks: partial maxima of every block plus the reduced scores
    big = f(8192, 7168)
    assert big > 7168 * 2 * 2 and big % 256 == 0
    assert f(-1, 64) == 0 and f(4, 0) == 0


def pq(L, fmt=0, x=A, tokens=8, cols=64, ldx=64, qq=B, sc=B, ts=B, src=A, rows=16, off=A, G=2,
       chan=A, nS=4, qo=B, so=B, tso=B, R=A):
    return L.fp4q_permute_quantized(fmt, x, tokens, cols, ldx, qq, sc, ts, src, rows, off, G,
                                    chan, nS, qo, so, tso, R, None)


def test_permute_quantized_rejects(L):
    assert pq(L, fmt=5) == INVALID
    assert pq(L, cols=40, ldx=40) == INVALID       # not whole NVFP4 blocks
    assert pq(L, tokens=0) == INVALID              # rows to fill but no tokens
    assert pq(L, G=0) == INVALID
    assert pq(L, off=None) == INVALID
    assert pq(L, nS=65) == INVALID
    assert pq(L, chan=None) == INVALID
    assert pq(L, R=None) == INVALID
    assert pq(L, ts=None) == INVALID               # NVFP4 needs the token tensor scale
    assert pq(L, tso=None) == INVALID              # ... and somewhere to put the groups' copies
    assert pq(L, fmt=1) == INVALID                 # MXFP4 takes neither
    assert pq(L, src=None) == INVALID
    assert pq(L, qo=None) == INVALID
    assert pq(L, qq=ctypes.c_void_p(0x20004)) == INVALID   # codes 8-byte aligned
    assert pq(L, x=None) == INVALID                # the residual reads x
    assert pq(L, ldx=32) == INVALID
    # nothing to do: accepted without touching memory
    assert pq(L, fmt=1, ts=None, tso=None, rows=0, src=None, qq=None, sc=None, qo=None, so=None,
              chan=None, nS=0, R=None, x=None, tokens=0) == 0


def test_comp_weights_rejects(L):
    def cw(fmt=0, layout=0, N=32, K=256, bq=B, bs=B, chan=A, nS=8, out=A, nb=4096):
        return L.fp4q_comp_weights(fmt, layout, N, K, bq, bs, chan, nS, out, nb, None)
    # 1 KB per 16 columns and 32 channels
    assert L.fp4q_comp_weights_bytes(0, 1, 11008, 2048, 64) == 688 * 2 * 1024
    assert L.fp4q_comp_weights_bytes(1, 0, 17, 256, 33) == 2 * 2 * 1024
    assert L.fp4q_comp_weights_bytes(0, 0, 17, 256, 0) == 0
    assert L.fp4q_comp_weights_bytes(0, 0, 0, 256, 8) == 0
    assert cw(fmt=2) == INVALID
    assert cw(layout=3) == INVALID
    assert cw(chan=None) == INVALID
    assert cw(out=ctypes.c_void_p(0x10008)) == INVALID          # 16-byte aligned
    assert cw(K=144) == UNSUPPORTED
    assert cw(nb=2047) == WORKSPACE
    assert cw(nS=0, chan=None) == 0                               # nothing to write
    assert cw(N=0) == 0


def test_gemm_prepared_rejects(L):
    def gp(fmt=0, layout=0, M=4, N=8, K=256, ats=B, bts=B, chan=A, nS=8, R=B, cw=A, nb=1024,
           y=A, ldy=8):
        return L.fp4q_gemm_prepared(fmt, layout, M, N, K, A, A, ats, B, B, bts, chan, nS, R, cw,
                                    nb, y, 0, ldy, None)
    assert gp(fmt=2) == INVALID
    assert gp(layout=4) == INVALID
    assert gp(ldy=4) == INVALID
    assert gp(R=None) == INVALID
    assert gp(K=144) == UNSUPPORTED
    assert gp(cw=None) == WORKSPACE
    assert gp(nb=1023) == WORKSPACE
    assert gp(cw=ctypes.c_void_p(0x10008)) == WORKSPACE


def test_grouped_prepared_rejects(L):
    assert L.fp4q_grouped_comp_weights_bytes(0, 1536, 2048, 128, 32) == 128 * 96 * 1024
    assert L.fp4q_grouped_comp_weights_bytes(0, 1536, 2048, 0, 32) == 0

    def gcw(fmt=0, wl=0, N=32, K=256, G=2, chan=A, nS=8, out=A, nb=4096):
        return L.fp4q_grouped_comp_weights(fmt, wl, N, K, G, B, B, chan, nS, out, nb, None)
    assert gcw(fmt=3) == INVALID
    assert gcw(wl=2) == INVALID
    assert gcw(G=0) == INVALID
    assert gcw(G=5000) == UNSUPPORTED
    assert gcw(chan=None) == INVALID
    assert gcw(K=144) == UNSUPPORTED
    assert gcw(nb=4095) == WORKSPACE
    assert gcw(out=ctypes.c_void_p(0x10008)) == INVALID

    def ggp(G=2, off=A, cw=A, nb=1 << 20, nS=8, chan=A, R=B, wl=0, N=256, fmt=0, ts=B):
        return L.fp4q_grouped_gemm_prepared(fmt, wl, 64, N, 256, off, G, A, A, ts, B, B, ts, chan,
                                            nS, R, cw, nb, A, 0, None)
    assert ggp(wl=2) == INVALID
    assert ggp(wl=1, N=200) == UNSUPPORTED
    assert ggp(wl=1, fmt=1, ts=None, nS=32) == UNSUPPORTED
    assert ggp(off=None) == INVALID
    assert ggp(G=5000) == UNSUPPORTED
    assert ggp(cw=None) == WORKSPACE
    assert ggp(nb=100) == WORKSPACE


def test_tiled_weight_wrappers_need_shapes():
    """The binding cannot read N (and K) from packed tiled weights: it asks
    for them instead of guessing from padded byte counts."""
    import torch
    import fp4_w4a4_quantized_amd as fq
    bq = torch.zeros((2, 4096), dtype=torch.uint8)
    chan = torch.zeros((2, 8), dtype=torch.int32)
    with pytest.raises(ValueError):
        fq.grouped_comp_weights(0, bq, bq, chan, w_layout=fq.TILED, N=256)
    a = {"q": torch.zeros((4, 128), dtype=torch.uint8), "scales": None, "tscale": None,
         "resid": None}
    off = torch.tensor([0, 2, 4], dtype=torch.int32)
    with pytest.raises(ValueError):
        fq.grouped_gemm(0, off, a, bq, bq, None, w_layout=fq.TILED)
    with pytest.raises(ValueError):
        fq.grouped_gemm_prepared(0, off, a, bq, bq, None, chan, bq, w_layout=fq.TILED)
