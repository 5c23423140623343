"""The C ABI loads, exports every declared entry point and rejects bad
arguments with the documented status before touching a device.

These tests run without a GPU.  The pointers passed are fake addresses; every
call but the last one carries an argument error, so nothing is launched.  The
last one (all arguments valid) is only run where no GPU is present, and
checks that the library reports the missing device instead of launching.
"""
import pytest
import torch

from bit_gemm_block_amd import w4a4 as W

P = 0x10000      # a 16-byte-aligned fake address (never dereferenced)
Q = 0x10001      # misaligned


@pytest.fixture(scope="module")
def lib():
    return W.lib()


def test_exports_every_declared_symbol(lib):
    names = W.header_functions()
    assert len(names) == 25
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(W._SIGS)


def test_version_and_status_strings(lib):
    assert lib.w4a4_abi_version() == 1
    assert lib.w4a4_status_string(0) == b"ok"
    for s in range(1, 6):
        assert lib.w4a4_status_string(s) not in (b"ok", b"unknown status")
    assert lib.w4a4_status_string(99) == b"unknown status"
    assert lib.w4a4_last_hip_error() == 0


def test_quantize_act_argument_errors(lib):
    f = lib.w4a4_quantize_act_int4
    L = W.CODES_PACKED
    assert f(P, 7, 4, 256, 0, P, L, P, None) == W.ERR_INVALID_ARG          # dtype
    assert f(P, W.F16, 4, 256, 0, P, 6, P, None) == W.ERR_INVALID_ARG      # layout
    assert f(P, W.F16, 4, 192, 0, P, W.CODES_F6_TILED, P, None) == W.ERR_UNSUPPORTED  # K % 128
    assert f(P, W.F16, -1, 256, 0, P, L, P, None) == W.ERR_INVALID_ARG     # M < 0
    assert f(P, W.F16, 4, 0, 0, P, L, P, None) == W.ERR_INVALID_ARG        # K = 0
    assert f(None, W.F16, 4, 256, 0, P, L, P, None) == W.ERR_INVALID_ARG   # null x
    assert f(P, W.F16, 4, 256, 0, None, L, P, None) == W.ERR_INVALID_ARG   # null xq
    assert f(P, W.F16, 4, 100, 0, P, L, P, None) == W.ERR_UNSUPPORTED      # K % 64
    assert f(P, W.F16, 4, 32768, 0, P, L, P, None) == W.ERR_UNSUPPORTED    # K too big
    assert f(P, W.F16, 4, 256, 3, P, L, P, None) == W.ERR_UNSUPPORTED      # b not pow2
    assert f(P, W.F16, 4, 8192, 8192, P, L, P, None) == W.ERR_UNSUPPORTED  # b > 4096
    assert f(P, W.F16, 4, 192, 128, P, L, P, None) == W.ERR_UNSUPPORTED    # b does not divide K
    assert f(Q, W.F16, 4, 256, 0, P, L, P, None) == W.ERR_MISALIGNED
    assert f(P, W.F16, 4, 256, 0, P, L, Q, None) == W.ERR_MISALIGNED
    assert f(None, W.F16, 0, 256, 64, None, L, None, None) == W.OK         # empty: no-op


def test_int8_activation_quantizer_argument_errors(lib):
    f = lib.w4a4_quantize_act_int8
    assert f(P, W.F16, 4, 256, 0, P, W.CODES_PACKED, P, None) == W.ERR_INVALID_ARG         # 4-bit layout
    assert f(P, W.F16, 4, 256, 0, P, W.CODES_PACKED_TILED, P, None) == W.ERR_INVALID_ARG
    assert f(P, W.F16, 4, 256, 0, P, W.CODES_F6_TILED, P, None) == W.ERR_INVALID_ARG   # FP6: 4-bit
    assert f(P, W.F16, 4, 192, 0, P, W.CODES_I8_TILED, P, None) == W.ERR_UNSUPPORTED       # K % 128
    assert f(P, W.F16, 4, 256, 3, P, W.CODES_I8, P, None) == W.ERR_UNSUPPORTED             # b
    assert f(Q, W.F16, 4, 256, 0, P, W.CODES_I8, P, None) == W.ERR_MISALIGNED
    assert f(None, W.F16, 0, 256, 0, None, W.CODES_I8, None, None) == W.OK


def test_w4a8_forward_argument_errors(lib):
    f = lib.w4a8_qlinear_forward
    need = lib.w4a4_qlinear_workspace_size(16, 32, 256, 8)
    args = [P, W.F16, P, 0, P, W.F16, 16, 32, 256, 256, 0, P, P, 8, P, P, need, None]
    bad = list(args); bad[11] = None
    assert f(*bad) == W.ERR_INVALID_ARG
    bad = list(args); bad[16] = need - 1
    assert f(*bad) == W.ERR_WORKSPACE
    bad = list(args); bad[6] = 0
    assert f(*bad) == W.OK


def test_rotate_and_weight_argument_errors(lib):
    r = lib.w4a4_hadamard_rotate
    assert r(P, W.F32, P, 4, 256, 0, None) == W.ERR_UNSUPPORTED         # rotation needed
    assert r(P, W.F32, None, 4, 256, 256, None) == W.ERR_INVALID_ARG
    assert r(P, W.F32, Q, 4, 256, 256, None) == W.ERR_MISALIGNED
    w = lib.w4a4_quantize_weight_int4
    assert w(P, W.F32, 8, 256, 0, 96, P, 0, P, W.F16, None) == W.ERR_UNSUPPORTED   # group % 64
    assert w(P, W.F32, 8, 192, 0, 128, P, 0, P, W.F16, None) == W.ERR_UNSUPPORTED  # group | K
    assert w(P, W.F32, 8, 384, 0, 192, P, 0, P, W.F16, None) == W.ERR_UNSUPPORTED  # not pow2
    assert w(P, W.F32, 8, 256, 0, -64, P, 0, P, W.F16, None) == W.ERR_INVALID_ARG
    assert w(P, W.F32, 8, 256, 0, 0, P, 0, P, 5, None) == W.ERR_INVALID_ARG       # scale dtype
    assert w(P, W.F32, 8, 256, 0, 0, P, 0, None, W.F16, None) == W.ERR_INVALID_ARG
    assert w(P, W.F32, 0, 256, 0, 0, None, 0, None, W.F16, None) == W.OK


def test_gemm_and_lowrank_argument_errors(lib):
    g = lib.w4a4_qgemm_w4a4
    L = W.CODES_I8
    assert g(P, L, P, P, 0, P, W.F16, 0, 4, 8, 256, None, None, None) == W.ERR_INVALID_ARG  # no output
    assert g(P, 9, P, P, 0, P, W.F16, 0, 4, 8, 256, P, None, None) == W.ERR_INVALID_ARG    # layout
    assert g(P, L, None, P, 0, P, W.F16, 0, 4, 8, 256, P, None, None) == W.ERR_INVALID_ARG  # y needs scales
    assert g(P, L, P, P, 0, P, W.F16, 96, 4, 8, 256, P, None, None) == W.ERR_UNSUPPORTED
    assert g(P, L, P, P, 0, P, W.F16, 0, 4, 8, 200, P, None, None) == W.ERR_UNSUPPORTED
    assert g(P, L, P, Q, 0, P, W.F16, 0, 4, 8, 256, P, None, None) == W.ERR_MISALIGNED
    assert g(None, L, None, None, 0, None, W.F16, 0, 4, 0, 256, None, None, None) == W.OK
    T, WT = W.CODES_I8_TILED, W.WEIGHTS_TILED
    assert g(P, L, P, P, 7, P, W.F16, 0, 4, 8, 256, P, None, None) == W.ERR_INVALID_ARG    # w layout
    assert g(P, L, P, P, WT, P, W.F16, 0, 4, 8, 256, P, None, None) == W.ERR_INVALID_ARG   # mixed
    assert g(P, T, P, P, 0, P, W.F16, 0, 4, 8, 256, P, None, None) == W.ERR_INVALID_ARG    # mixed
    assert g(P, T, P, P, WT, P, W.F16, 0, 4, 8, 192, P, None, None) == W.ERR_UNSUPPORTED   # K % 128
    assert g(P, T, P, P, WT, P, W.F16, 64, 4, 8, 256, P, None, None) == W.ERR_UNSUPPORTED  # group
    assert lib.w4a4_quantize_act_int4(P, W.F16, 4, 192, 0, P, T, P, None) == W.ERR_UNSUPPORTED
    assert lib.w4a4_quantize_weight_int4(P, W.F32, 8, 192, 0, 0, P, WT, P, W.F16,
                                         None) == W.ERR_UNSUPPORTED
    lr = lib.w4a4_lowrank_project
    assert lr(P, W.F16, P, 4, 256, 0, P, None) == W.ERR_INVALID_ARG
    assert lr(P, W.F16, P, 4, 256, 257, P, None) == W.ERR_UNSUPPORTED
    assert lr(P, W.F16, None, 4, 256, 8, P, None) == W.ERR_INVALID_ARG


def test_qlinear_argument_errors(lib):
    f = lib.w4a4_qlinear_forward
    need = lib.w4a4_qlinear_workspace_size(16, 32, 256, 8)
    assert need >= 16 * 128 + 16 * 4 + 16 * 8 * 4
    assert lib.w4a4_qlinear_workspace_size(0, 32, 256, 8) == 0
    args = [P, W.F16, P, 0, P, W.F16, 16, 32, 256, 256, 0, P, P, 8, P, P, need, None]
    bad = list(args); bad[11] = None                                  # rank > 0 without A
    assert f(*bad) == W.ERR_INVALID_ARG
    bad = list(args); bad[13] = 300
    assert f(*bad) == W.ERR_UNSUPPORTED
    bad = list(args); bad[16] = need - 1
    assert f(*bad) == W.ERR_WORKSPACE
    bad = list(args); bad[15] = Q
    assert f(*bad) == W.ERR_MISALIGNED
    bad = list(args); bad[10] = 100
    assert f(*bad) == W.ERR_UNSUPPORTED
    bad = list(args); bad[3] = 4                                      # weight layout
    assert f(*bad) == W.ERR_INVALID_ARG
    bad = list(args); bad[3] = W.WEIGHTS_TILED_F6                     # FP6: 4-bit codes only
    assert lib.w4a8_qlinear_forward(*bad) == W.ERR_UNSUPPORTED
    bad = list(args); bad[3] = W.WEIGHTS_TILED_F6; bad[10] = 64       # FP6: groups of 128 k
    assert f(*bad) == W.ERR_UNSUPPORTED
    bad = list(args); bad[3] = W.WEIGHTS_TILED_OB; bad[10] = 128      # offset-binary: no groups
    assert f(*bad) == W.ERR_UNSUPPORTED
    bad = list(args); bad[3] = W.WEIGHTS_TILED_OB                     # offset-binary: no W4A8
    assert lib.w4a8_qlinear_forward(*bad) == W.ERR_UNSUPPORTED
    bad = list(args); bad[3] = W.WEIGHTS_TILED; bad[10] = 64          # tiled needs group % 128
    assert f(*bad) == W.ERR_UNSUPPORTED
    bad = list(args); bad[6] = 0
    assert f(*bad) == W.OK


def test_offset_binary_argument_errors(lib):
    g = lib.w4a4_qgemm_w4a4
    OB, WOB = W.CODES_PACKED_TILED_OB, W.WEIGHTS_TILED_OB
    PT, WT = W.CODES_PACKED_TILED, W.WEIGHTS_TILED
    assert g(P, OB, P, P, WT, P, W.F16, 0, 64, 8, 256, P, None, None) == W.ERR_INVALID_ARG  # codes need OB weights
    assert g(P, OB, P, P, 0, P, W.F16, 0, 64, 8, 256, P, None, None) == W.ERR_INVALID_ARG   # row-major weights
    assert g(P, OB, P, P, WOB, P, W.F16, 128, 64, 8, 256, P, None, None) == W.ERR_UNSUPPORTED
    assert g(P, PT, P, P, WOB, P, W.F16, 0, 33, 8, 256, P, None, None) == W.ERR_UNSUPPORTED  # M > 32
    assert g(P, W.CODES_I8_TILED, P, P, WOB, P, W.F16, 0, 8, 8, 256, P, None, None) == W.ERR_UNSUPPORTED
    assert g(P, OB, P, P, WOB, P, W.F16, 0, 64, 8, 192, P, None, None) == W.ERR_UNSUPPORTED  # K % 128
    assert lib.w4a4_quantize_act_int4(P, W.F16, 4, 192, 0, P, OB, P, None) == W.ERR_UNSUPPORTED
    assert lib.w4a4_quantize_act_int8(P, W.F16, 4, 256, 0, P, OB, P, None) == W.ERR_INVALID_ARG
    assert lib.w4a4_quantize_weight_int4(P, W.F32, 8, 256, 0, 0, P, WOB, P, W.F16,
                                         None) == W.ERR_INVALID_ARG
    c = lib.w4a4_weights_tiled_to_ob
    assert c(P, 8, 192, P, None) == W.ERR_UNSUPPORTED
    assert c(P, -1, 256, P, None) == W.ERR_INVALID_ARG
    assert c(None, 8, 256, P, None) == W.ERR_INVALID_ARG
    assert c(P, 8, 256, Q, None) == W.ERR_MISALIGNED
    assert c(None, 0, 256, None, None) == W.OK


def test_mxfp4_argument_errors(lib):
    q = lib.w4a4_quantize_mxfp4
    assert q(P, W.F16, 4, 256, 0, P, W.CODES_I8, P, None) == W.ERR_INVALID_ARG          # layout
    assert q(P, W.F16, 4, 192, 0, P, W.CODES_PACKED_TILED, P, None) == W.ERR_UNSUPPORTED  # K % 128
    assert q(P, W.F16, 4, 256, 0, P, W.CODES_PACKED, None, None) == W.ERR_INVALID_ARG
    assert q(P, W.F16, 4, 256, 0, P, W.CODES_PACKED, Q, None) == W.ERR_MISALIGNED
    assert q(None, W.F16, 0, 256, 0, None, W.CODES_PACKED, None, None) == W.OK
    g = lib.w4a4_qgemm_mxfp4
    assert g(P, P, P, None, 4, 8, 256, P, None) == W.ERR_INVALID_ARG
    assert g(P, P, P, P, 4, 8, 192, P, None) == W.ERR_UNSUPPORTED
    assert g(P, Q, P, P, 4, 8, 256, P, None) == W.ERR_MISALIGNED
    assert g(None, None, None, None, 4, 0, 256, None, None) == W.OK
    f = lib.w4a4_qlinear_forward_mxfp4
    need = lib.w4a4_qlinear_workspace_size(16, 32, 512, 8)
    args = [P, W.F16, P, P, 16, 32, 512, 128, P, P, 8, P, P, need, None]
    bad = list(args); bad[8] = None
    assert f(*bad) == W.ERR_INVALID_ARG
    bad = list(args); bad[13] = need - 1
    assert f(*bad) == W.ERR_WORKSPACE
    bad = list(args); bad[6] = 448
    assert f(*bad) == W.ERR_UNSUPPORTED
    bad = list(args); bad[4] = 0
    assert f(*bad) == W.OK


def test_residual_argument_errors(lib):
    w = lib.w4a4_quantize_weight_residual_int4
    assert w(P, W.F32, 8, 256, 0, -1, P, P, W.F16, None) == W.ERR_INVALID_ARG      # r < 0
    assert w(P, W.F32, 8, 256, 0, 300, P, P, W.F16, None) == W.ERR_UNSUPPORTED     # r > K
    assert w(P, W.F32, 8, 192, 0, 32, P, P, W.F16, None) == W.ERR_UNSUPPORTED      # K % 128
    assert w(P, W.F32, 8, 16384, 0, 32, P, P, W.F16, None) == W.ERR_UNSUPPORTED    # int32 bound
    assert w(P, W.F32, 8, 256, 0, 32, None, P, W.F16, None) == W.ERR_INVALID_ARG
    assert w(P, W.F32, 8, 256, 0, 32, P, Q, W.F16, None) == W.ERR_MISALIGNED
    assert w(None, W.F32, 0, 256, 0, 32, None, None, W.F16, None) == W.OK
    g = lib.w4a4_qgemm_residual
    assert g(P, P, P, P, W.F16, 32, 4, 8, 256, None, None, None) == W.ERR_INVALID_ARG  # no output
    assert g(P, None, P, P, W.F16, 32, 4, 8, 256, P, None, None) == W.ERR_INVALID_ARG  # y needs scales
    assert g(P, P, P, P, W.F16, 32, 4, 8, 320, P, None, None) == W.ERR_UNSUPPORTED     # K % 128
    assert g(P, P, Q, P, W.F16, 32, 4, 8, 256, P, None, None) == W.ERR_MISALIGNED
    assert g(None, None, None, None, W.F16, 32, 0, 8, 256, None, None, None) == W.OK
    f = lib.w4a4_qlinear_forward_residual
    need = lib.w4a4_qlinear_workspace_size(16, 32, 512, 0)
    args = [P, W.F16, P, P, W.F16, 64, 16, 32, 512, 128, P, P, need, None]
    bad = list(args); bad[5] = 600
    assert f(*bad) == W.ERR_UNSUPPORTED
    bad = list(args); bad[12] = need - 1
    assert f(*bad) == W.ERR_WORKSPACE
    bad = list(args); bad[2] = None
    assert f(*bad) == W.ERR_INVALID_ARG
    bad = list(args); bad[6] = 0
    assert f(*bad) == W.OK


def test_asymmetric_argument_errors(lib):
    q = lib.w4a4_quantize_act_asym_int4
    L, LT = W.CODES_PACKED, W.CODES_PACKED_TILED
    assert q(P, W.F16, 4, 512, 0, 128, P, W.CODES_I8, P, P, None) == W.ERR_INVALID_ARG   # layout
    assert q(P, W.F16, 4, 512, 0, 128, P, L, P, None, None) == W.ERR_INVALID_ARG         # no zeros
    assert q(P, W.F16, 4, 512, 0, 0, P, L, P, P, None) == W.ERR_INVALID_ARG              # group 0
    assert q(P, W.F16, 4, 512, 0, 64, P, L, P, P, None) == W.ERR_UNSUPPORTED             # group < 128
    assert q(P, W.F16, 4, 384, 0, 256, P, L, P, P, None) == W.ERR_UNSUPPORTED            # group | K
    assert q(P, W.F16, 4, 512, 256, 128, P, L, P, P, None) == W.ERR_UNSUPPORTED          # b != group
    assert q(P, W.F16, 4, 512, 0, 128, P, L, P, Q, None) == W.ERR_MISALIGNED
    assert q(None, W.F16, 0, 512, 128, 128, None, LT, None, None, None) == W.OK
    s = lib.w4a4_weight_group_sums
    assert s(P, 3, 8, 256, 128, P, None) == W.ERR_INVALID_ARG                           # layout
    assert s(P, 0, 8, 256, 96, P, None) == W.ERR_UNSUPPORTED                            # group % 64
    assert s(P, 0, 8, 256, 128, None, None) == W.ERR_INVALID_ARG
    assert s(None, 0, 0, 256, 128, None, None) == W.OK
    g = lib.w4a4_qgemm_asym
    args = [P, P, P, 128, P, P, W.F16, P, 4, 8, 512, P, None]
    bad = list(args); bad[2] = None
    assert g(*bad) == W.ERR_INVALID_ARG
    bad = list(args); bad[3] = 64
    assert g(*bad) == W.ERR_UNSUPPORTED
    bad = list(args); bad[10] = 448                                                     # K % 128
    assert g(*bad) == W.ERR_UNSUPPORTED
    bad = list(args); bad[7] = Q
    assert g(*bad) == W.ERR_MISALIGNED
    bad = list(args); bad[9] = 0
    assert g(*bad) == W.OK
    f = lib.w4a4_qlinear_forward_asym
    need = lib.w4a4_qlinear_workspace_size(16, 32, 512, 8)
    args = [P, W.F16, P, P, W.F16, P, 16, 32, 512, 128, P, P, 8, P, P, need, None]
    bad = list(args); bad[5] = None
    assert f(*bad) == W.ERR_INVALID_ARG
    bad = list(args); bad[9] = 64
    assert f(*bad) == W.ERR_UNSUPPORTED
    bad = list(args); bad[15] = need - 1
    assert f(*bad) == W.ERR_WORKSPACE
    bad = list(args); bad[6] = 0
    assert f(*bad) == W.OK


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the no-device path")
def test_valid_call_without_device_reports_unsupported(lib):
    need = lib.w4a4_qlinear_workspace_size(16, 32, 256, 8)
    assert lib.w4a4_qlinear_forward(P, W.F16, P, 0, P, W.F16, 16, 32, 256, 256, 0, P, P, 8, P,
                                    P, need, None) == W.ERR_UNSUPPORTED
    assert lib.w4a4_quantize_act_int4(P, W.F16, 4, 256, 0, P, W.CODES_PACKED, P,
                                      None) == W.ERR_UNSUPPORTED
    assert lib.w4a4_weights_tiled_to_ob(P, 8, 256, P, None) == W.ERR_UNSUPPORTED


def test_workspace_layout_query(lib):
    # Host logic only: where the forward leaves its codes and scales (codes,
    # then scales); the codes layout is the one the GEMM of that call reads.
    M, N, K = 40, 96, 4096
    size = W.qlinear_workspace_size(M, N, K, 16)
    cases = {("rowmajor", 4): "i8", ("tiled", 4): "packed_tiled",
             ("tiled_ob", 4): "packed_tiled_ob", ("tiled", 8): "i8_tiled",
             ("rowmajor", 8): "i8"}
    for (wl, bits), want in cases.items():
        co, cl, so = W.qlinear_workspace_layout(M, N, K, 16, wl, 0, bits)
        assert cl == want
        assert co % 256 == 0
        assert so >= co + W.pad16(M) * K and so + 4 * M <= size
    # decode-sized calls on offset-binary weights read plain packed codes
    assert W.qlinear_workspace_layout(8, N, K, 0, "tiled_ob", 0, 4)[1] == "packed_tiled"
    import ctypes
    c, i = ctypes.c_size_t(0), ctypes.c_int(0)
    f = lib.w4a4_qlinear_workspace_layout
    assert f(0, N, K, 0, 0, 0, 4, ctypes.byref(c), ctypes.byref(i), ctypes.byref(c)) == W.ERR_INVALID_ARG
    assert f(M, N, K, 0, 7, 0, 4, ctypes.byref(c), ctypes.byref(i), ctypes.byref(c)) == W.ERR_INVALID_ARG
    assert f(M, N, K, 0, 0, 0, 5, ctypes.byref(c), ctypes.byref(i), ctypes.byref(c)) == W.ERR_INVALID_ARG
    assert f(M, N, K, 0, 0, 0, 4, None, ctypes.byref(i), ctypes.byref(c)) == W.ERR_INVALID_ARG


def test_noalloc_argument_errors(lib):
    # Checked on the host before any device call: sizes beyond the library's
    # scratch array, negative sizes, and the empty no-op.
    f = lib.w4a4_qlinear_forward_noalloc
    import re
    with open(W.HEADER) as fh:
        m = re.search(r"#define W4A4_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", fh.read())
    assert m and int(m.group(1)) << int(m.group(2)) == W.NOALLOC_SCRATCH_BYTES
    big = (4096, 4096, 16384)          # 64 MiB of int8 codes room
    assert W.qlinear_workspace_size(*big, 0) > W.NOALLOC_SCRATCH_BYTES
    assert f(P, W.F16, P, 1, P, W.F16, *big, 128, 0, None, None, 0, P, None) == W.ERR_WORKSPACE
    assert f(P, W.F16, P, 1, P, W.F16, -1, 16, 256, 256, 0, None, None, 0, P, None) == W.ERR_INVALID_ARG
    assert f(P, W.F16, P, 1, P, W.F16, 16, 16, 256, 256, 0, None, None, -1, P, None) == W.ERR_INVALID_ARG
    assert f(None, W.F16, None, 1, None, W.F16, 0, 16, 256, 256, 0, None, None, 0, None, None) == W.OK
