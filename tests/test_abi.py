"""The C ABI: libqlin loads, exports every function include/qlin.h declares with
the argument count the binding uses, and its host-side validation returns the
documented status before any HIP call (CPU only, no kernel is launched)."""
import ctypes as C
import os
import re

import pytest

from outlier_aware_bit_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qlin.h")


def _declarations():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    decls = {}
    for m in re.finditer(r"\b(qlin_\w+)\s*\(([^;{]*?)\)\s*;", text, flags=re.S):
        params = m.group(2).strip()
        n = 0 if params in ("", "void") else params.count(",") + 1
        decls[m.group(1)] = n
    return decls


def test_header_declares_the_entry_points():
    d = _declarations()
    for name in ["qlin_quant_act", "qlin_hadamard_offset", "qlin_gemm_w8a8", "qlin_gemm_w4a8",
                 "qlin_outlier_comp", "qlin_momentum_update", "qlin_gemm_w4a4", "qlin_pack_weight"]:
        assert name in d


def test_library_exports_every_declared_symbol_with_matching_arity():
    lib = _lib.load()
    decls = _declarations()
    assert set(decls) == set(_lib.SIGNATURES), set(decls) ^ set(_lib.SIGNATURES)
    for name, nargs in decls.items():
        assert hasattr(lib, name), name
        assert len(_lib.SIGNATURES[name][1]) == nargs, name


def test_exported_symbols_via_nm_style_lookup():
    # dlsym through a fresh handle, independent of the binding's table.
    handle = C.CDLL(_lib.LIB_PATH)
    for name in _declarations():
        assert C.cast(getattr(handle, name), C.c_void_p).value


def test_status_strings_and_version():
    lib = _lib.load()
    assert lib.qlin_abi_version() == 3
    names = [lib.qlin_status_string(i).decode() for i in range(6)]
    assert names == ["QLIN_OK", "QLIN_ERR_INVALID_ARG", "QLIN_ERR_SHAPE", "QLIN_ERR_ALIGN",
                     "QLIN_ERR_UNSUPPORTED", "QLIN_ERR_HIP"]
    assert lib.qlin_status_string(99).decode() == "QLIN_ERR_UNKNOWN"


def test_packed_bytes():
    lib = _lib.load()
    assert lib.qlin_packed_bytes(_lib.QLIN_LAYOUT_W8, 4096, 4096) == 4096 * 4096
    assert lib.qlin_packed_bytes(_lib.QLIN_LAYOUT_W4S, 4096, 11008) == 4096 * 11008 // 2
    assert lib.qlin_packed_bytes(_lib.QLIN_LAYOUT_W4U, 4096, 14336) == 4096 * 14336 // 2
    assert lib.qlin_packed_bytes(7, 4096, 4096) == 0
    assert lib.qlin_packed_bytes(_lib.QLIN_LAYOUT_W8, 100, 4096) == 0
    assert lib.qlin_packed_bytes(_lib.QLIN_LAYOUT_W8, 4096, 100) == 0
    assert lib.qlin_packed_bytes(_lib.QLIN_LAYOUT_WO, 205, 4096) == 208 * 4096 * 2
    assert lib.qlin_packed_bytes(_lib.QLIN_LAYOUT_WO, 0, 4096) == 0
    # the transposed int8 layout packs [N x K]: N % 128, K % 64
    assert lib.qlin_packed_bytes(_lib.QLIN_LAYOUT_W8T, 4096, 4096) == 4096 * 4096
    assert lib.qlin_packed_bytes(_lib.QLIN_LAYOUT_W8T, 64, 128) == 64 * 128
    assert lib.qlin_packed_bytes(_lib.QLIN_LAYOUT_W8T, 4096, 64) == 0
    assert lib.qlin_packed_bytes(_lib.QLIN_LAYOUT_W8T, 100, 4096) == 0
    assert [lib.qlin_outlier_ld(n) for n in (0, 1, 16, 17, 205)] == [0, 16, 16, 32, 208]


# Fake but 16-byte aligned "device" addresses: validation never dereferences
# them, and every case below fails (or returns for M == 0) before a HIP call.
A = 0x10000
B = 0x20000
MIS = 0x10008  # 8-byte aligned only


def _err(status, code):
    assert status == code, (_lib.load().qlin_status_string(status), _lib.load().qlin_last_error())


def test_quant_act_validation():
    lib = _lib.load()
    def qa(*head, O=None, nO=0, s=None, qO=None, xO=None):
        return lib.qlin_quant_act(*head, O, nO, s, qO, xO, None)
    _err(qa(None, 4, 256, None, B, A), _lib.QLIN_ERR_INVALID_ARG)
    assert b"x" in lib.qlin_last_error()
    _err(qa(A, 4, 200, None, B, A), _lib.QLIN_ERR_SHAPE)
    _err(qa(A, -1, 256, None, B, A), _lib.QLIN_ERR_INVALID_ARG)
    _err(qa(MIS, 4, 256, None, B, A), _lib.QLIN_ERR_ALIGN)
    _err(qa(A, 4, 256, MIS, B, A), _lib.QLIN_ERR_ALIGN)
    _err(qa(A, 4, 256, None, B, A, O=A), _lib.QLIN_ERR_INVALID_ARG)
    _err(qa(A, 4, 256, None, B, A, nO=3), _lib.QLIN_ERR_INVALID_ARG)
    _err(qa(A, 4, 256, None, B, A, O=A, nO=3), _lib.QLIN_ERR_INVALID_ARG)
    _err(qa(A, 4, 256, None, B, A, O=A, nO=3, xO=B), _lib.QLIN_ERR_INVALID_ARG)
    _err(qa(A, 4, 256, None, B, A, O=A, nO=300, qO=B), _lib.QLIN_ERR_SHAPE)
    _err(qa(A, 0, 256, None, B, A), _lib.QLIN_OK)


def test_hadamard_validation():
    lib = _lib.load()
    args = [A, 4, 256, B, 128, A, A, A, A, None, None]
    _err(lib.qlin_hadamard_offset(*args[:4], 64, *args[5:]), _lib.QLIN_ERR_UNSUPPORTED)
    _err(lib.qlin_hadamard_offset(A, 4, 192, B, 128, A, A, A, A, None, None), _lib.QLIN_ERR_SHAPE)
    _err(lib.qlin_hadamard_offset(A, 4, 256, None, 128, A, A, A, A, None, None), _lib.QLIN_ERR_INVALID_ARG)
    _err(lib.qlin_hadamard_offset(A, 4, 256, B, 128, A, A, A, A, MIS, None), _lib.QLIN_ERR_ALIGN)
    _err(lib.qlin_hadamard_offset(A, 0, 256, B, 128, A, A, A, A, None, None), _lib.QLIN_OK)


def test_momentum_validation():
    lib = _lib.load()
    _err(lib.qlin_momentum_update(A, 8, 256, A, 4, A, 1.5, A, B, None, None), _lib.QLIN_ERR_INVALID_ARG)
    _err(lib.qlin_momentum_update(A, 8, 256, A, 400, A, 0.9, A, B, None, None), _lib.QLIN_ERR_SHAPE)
    _err(lib.qlin_momentum_update(A, 8, 256, None, 4, A, 0.9, A, B, None, None), _lib.QLIN_ERR_INVALID_ARG)
    _err(lib.qlin_momentum_update(A, 8, 256, A, 4, A, 0.9, None, B, None, None), _lib.QLIN_ERR_INVALID_ARG)
    _err(lib.qlin_momentum_update(A, -2, 256, A, 4, A, 0.9, A, B, None, None), _lib.QLIN_ERR_INVALID_ARG)
    _err(lib.qlin_momentum_update(A, 8, 256, A, 4, A, 0.9, A, B, A + 4, None), _lib.QLIN_ERR_ALIGN)
    # Workspace: up to 16 row blocks of 128 tokens, one float per outlier each.
    assert lib.qlin_momentum_work_bytes(0, 205) == 205 * 4
    assert lib.qlin_momentum_work_bytes(128, 205) == 205 * 4
    assert lib.qlin_momentum_work_bytes(129, 205) == 2 * 205 * 4
    assert lib.qlin_momentum_work_bytes(2048, 205) == 16 * 205 * 4
    assert lib.qlin_momentum_work_bytes(100000, 7) == 16 * 7 * 4
    assert lib.qlin_momentum_work_bytes(-1, 7) == 0


def test_momentum_quant_validation():
    lib = _lib.load()
    def mq(x=A, M=8, K=256, O=A, nO=4, wm=A, gamma=0.9, s=A, r=B, work=None, q=A, scale=B, xO=A):
        return lib.qlin_quaff_momentum_quant(x, M, K, O, nO, wm, gamma, s, r, work, q, scale, xO, None)
    _err(mq(gamma=1.5), _lib.QLIN_ERR_INVALID_ARG)
    _err(mq(nO=400), _lib.QLIN_ERR_SHAPE)
    _err(mq(K=200), _lib.QLIN_ERR_SHAPE)
    _err(mq(M=-1), _lib.QLIN_ERR_INVALID_ARG)
    _err(mq(O=None), _lib.QLIN_ERR_INVALID_ARG)
    _err(mq(wm=None), _lib.QLIN_ERR_INVALID_ARG)
    _err(mq(xO=None), _lib.QLIN_ERR_INVALID_ARG)
    _err(mq(nO=0, O=None, wm=None), _lib.QLIN_ERR_INVALID_ARG)  # xO given without outliers
    _err(mq(q=None), _lib.QLIN_ERR_INVALID_ARG)
    _err(mq(scale=None), _lib.QLIN_ERR_INVALID_ARG)
    _err(mq(s=None), _lib.QLIN_ERR_INVALID_ARG)
    _err(mq(x=MIS), _lib.QLIN_ERR_ALIGN)
    _err(mq(work=A + 4), _lib.QLIN_ERR_ALIGN)
    # Workspace: five rows of nO floats (four row blocks and the old s), or
    # what the momentum update's two-launch form needs, if more.
    assert lib.qlin_quaff_momentum_quant_work_bytes(128, 205) == 5 * 205 * 4
    assert lib.qlin_quaff_momentum_quant_work_bytes(2048, 205) == 16 * 205 * 4
    assert lib.qlin_quaff_momentum_quant_work_bytes(0, 7) == 5 * 7 * 4
    assert lib.qlin_quaff_momentum_quant_work_bytes(-1, 7) == 0


def test_weight_prep_validation():
    lib = _lib.load()
    _err(lib.qlin_quant_weight_sym(A, 256, 128, 3, A, B, None), _lib.QLIN_ERR_UNSUPPORTED)
    _err(lib.qlin_quant_weight_sym(A, 256, 100, 8, A, B, None), _lib.QLIN_ERR_SHAPE)
    _err(lib.qlin_quant_weight_group(A, 256, 128, 64, A, B, A, B, None), _lib.QLIN_ERR_UNSUPPORTED)
    _err(lib.qlin_quant_weight_offq(A, 256, 128, None, 128, A, B, A, B, None), _lib.QLIN_ERR_INVALID_ARG)
    _err(lib.qlin_pack_weight(9, A, 256, 128, B, None), _lib.QLIN_ERR_INVALID_ARG)
    _err(lib.qlin_pack_weight(_lib.QLIN_LAYOUT_W8, A, 256, 128, MIS, None), _lib.QLIN_ERR_ALIGN)
    _err(lib.qlin_weight_row_absmax(A, 0, 128, None, None), _lib.QLIN_OK)


def test_gemm_validation():
    lib = _lib.load()
    ok = [A, A, B, A, 16, 128, 256, None, 0, None, A, None, None]
    _err(lib.qlin_gemm_w8a8(*ok[:4], 16, 100, 256, *ok[7:]), _lib.QLIN_ERR_SHAPE)
    _err(lib.qlin_gemm_w8a8(*ok[:4], 16, 128, 250, *ok[7:]), _lib.QLIN_ERR_SHAPE)
    _err(lib.qlin_gemm_w8a8(None, *ok[1:]), _lib.QLIN_ERR_INVALID_ARG)
    _err(lib.qlin_gemm_w8a8(*ok[:7], A, 5, None, A, None, None), _lib.QLIN_ERR_INVALID_ARG)
    _err(lib.qlin_gemm_w8a8(*ok[:7], A, 0, None, A, None, None), _lib.QLIN_ERR_INVALID_ARG)
    _err(lib.qlin_gemm_w8a8(*ok[:7], None, 300, None, A, None, None), _lib.QLIN_ERR_SHAPE)
    _err(lib.qlin_gemm_w8a8(*ok[:10], A, MIS, None), _lib.QLIN_ERR_ALIGN)
    _err(lib.qlin_gemm_w8a8(*ok[:4], 0, *ok[5:]), _lib.QLIN_OK)
    _err(lib.qlin_gemm_w4a8(A, A, B, A, None, 64, 16, 128, 256, A, None, None, None), _lib.QLIN_ERR_UNSUPPORTED)
    _err(lib.qlin_gemm_w4a8(A, A, B, A, None, 128, 16, 128, 256, A, None, None, None), _lib.QLIN_ERR_INVALID_ARG)
    _err(lib.qlin_gemm_w4a8(A, A, B, A, A, 0, 16, 128, 256, A, None, None, None), _lib.QLIN_ERR_INVALID_ARG)
    _err(lib.qlin_gemm_w4a8(A, A, B, A, A, 128, 256, 128, 256, A, None, MIS, None), _lib.QLIN_ERR_ALIGN)
    _err(lib.qlin_gemm_w4a8(A, A, B, A, None, 0, 0, 128, 256, A, None, None, None), _lib.QLIN_OK)
    # Workspace of the once-per-call requantization: per group, above 128 tokens.
    assert lib.qlin_gemm_w4a8_work_bytes(129, 4096, 11008, 128) == 11008 * 4096
    assert lib.qlin_gemm_w4a8_work_bytes(128, 4096, 11008, 128) == 0
    assert lib.qlin_gemm_w4a8_work_bytes(4096, 4096, 11008, 0) == 0
    assert lib.qlin_gemm_w4a8_work_bytes(4096, 100, 11008, 128) == 0
    assert lib.qlin_gemm_w4a8_work_bytes(1 << 40, 4096, 11008, 128) == 0
    _err(lib.qlin_gemm_w4a4(A, A, A, A, B, A, A, None, 16, 128, 256, A, None, None), _lib.QLIN_ERR_INVALID_ARG)
    _err(lib.qlin_gemm_w4a4(A, A, A, A, B, A, A, A, 16, 128, 384 + 64, A, None, None), _lib.QLIN_ERR_SHAPE)
    _err(lib.qlin_gemm_w4a4(A, A, A, A, B, A, A, A, 0, 128, 256, A, None, None), _lib.QLIN_OK)
    _err(lib.qlin_outlier_comp(A, A, 4, A, 16, 100, A, None), _lib.QLIN_ERR_SHAPE)
    _err(lib.qlin_outlier_comp(None, A, 4, A, 16, 128, A, None), _lib.QLIN_ERR_INVALID_ARG)
    _err(lib.qlin_outlier_comp(A, A, 4, MIS, 16, 128, A, None), _lib.QLIN_ERR_ALIGN)
    _err(lib.qlin_outlier_comp(A, A, 0, A, 16, 128, A, None), _lib.QLIN_OK)
    _err(lib.qlin_pack_weight(_lib.QLIN_LAYOUT_WO, A, 0, 128, B, None), _lib.QLIN_ERR_SHAPE)


def test_group_and_backward_validation():
    lib = _lib.load()
    _err(lib.qlin_hadamard_offset_group(A, 4, 256, B, 64, A, A, A, A, None, None), _lib.QLIN_ERR_UNSUPPORTED)
    _err(lib.qlin_hadamard_offset_group(A, 4, 192, B, 128, A, A, A, A, None, None), _lib.QLIN_ERR_SHAPE)
    _err(lib.qlin_hadamard_offset_group(A, 4, 256, B, 128, A, None, A, A, None, None), _lib.QLIN_ERR_INVALID_ARG)
    _err(lib.qlin_hadamard_offset_group(A, 0, 256, B, 128, A, A, A, A, None, None), _lib.QLIN_OK)
    _err(lib.qlin_weight_colsum_group(A, 256, 128, 64, A, None), _lib.QLIN_ERR_UNSUPPORTED)
    _err(lib.qlin_weight_colsum_group(A, 200, 128, 128, A, None), _lib.QLIN_ERR_SHAPE)
    _err(lib.qlin_weight_colsum_group(A, 256, 128, 128, MIS, None), _lib.QLIN_ERR_ALIGN)
    _err(lib.qlin_gemm_w4a4_group(A, A, A, A, B, A, A, None, 16, 128, 256, A, None, None), _lib.QLIN_ERR_INVALID_ARG)
    _err(lib.qlin_gemm_w4a4_group(A, A, A, A, B, A, A, A, 16, 100, 256, A, None, None), _lib.QLIN_ERR_SHAPE)
    _err(lib.qlin_gemm_w4a4_group(A, A, A, A, B, A, A, A, 16, 128, 256, A, A + 4, None), _lib.QLIN_ERR_ALIGN)
    _err(lib.qlin_gemm_w4a4_group(A, A, A, A, B, A, A, A, 0, 128, 256, A, None, None), _lib.QLIN_OK)
    bw = [A, 8, 256, 128, A, B, A, A, A, 3, A, A, A, A, A, None, None]
    _err(lib.qlin_quaff_backward(A, 8, 192, 128, *bw[4:]), _lib.QLIN_ERR_SHAPE)
    _err(lib.qlin_quaff_backward(A, 8, 256, 192, *bw[4:]), _lib.QLIN_ERR_SHAPE)
    _err(lib.qlin_quaff_backward(A, 8, 256, 128, *bw[4:9], 200, *bw[10:]), _lib.QLIN_ERR_SHAPE)
    _err(lib.qlin_quaff_backward(A, 8, 256, 128, *bw[4:10], None, *bw[11:]), _lib.QLIN_ERR_INVALID_ARG)
    _err(lib.qlin_quaff_backward(A, 8, 256, 128, *bw[4:8], None, 0, None, A, A, A, A, None, None),
         _lib.QLIN_ERR_INVALID_ARG)
    _err(lib.qlin_quaff_backward(A, 8, 256, 128, *bw[4:14], MIS, None, None), _lib.QLIN_ERR_ALIGN)
    _err(lib.qlin_quaff_backward(A, 0, 256, 128, *bw[4:]), _lib.QLIN_OK)
    _err(lib.qlin_pack_weight(_lib.QLIN_LAYOUT_W8T, A, 128, 200, B, None), _lib.QLIN_ERR_SHAPE)


def test_pca_validation():
    lib = _lib.load()
    _err(lib.qlin_pca_select(A, 4, 16, 100, A, B, None), _lib.QLIN_ERR_SHAPE)
    _err(lib.qlin_pca_select(A, 4, 0, 128, A, B, None), _lib.QLIN_ERR_INVALID_ARG)
    _err(lib.qlin_pca_select(A, 4, 16, 128, None, B, None), _lib.QLIN_ERR_INVALID_ARG)
    _err(lib.qlin_pca_select(A, 0, 16, 128, A, B, None), _lib.QLIN_OK)
    _err(lib.qlin_pca_leading_eigvec(A, 1, 128, 10, 1e-9, A, A, A, A, None), _lib.QLIN_ERR_SHAPE)
    _err(lib.qlin_pca_leading_eigvec(A, 8, 128, 0, 1e-9, A, A, A, A, None), _lib.QLIN_ERR_INVALID_ARG)
    _err(lib.qlin_pca_leading_eigvec(A, 8, 128, 10, -1.0, A, A, A, A, None), _lib.QLIN_ERR_INVALID_ARG)
    _err(lib.qlin_pca_leading_eigvec(A, 8, 128, 10, 1e-9, A, A, A, MIS, None), _lib.QLIN_ERR_ALIGN)
    _err(lib.qlin_pca_leading_eigvec(A, 8, 100, 10, 1e-9, A, A, A, A, None), _lib.QLIN_ERR_SHAPE)
    _err(lib.qlin_pca_leading_eigvec(A, 8, 16384, 10, 1e-9, A, A, A, A, None), _lib.QLIN_ERR_SHAPE)
    _err(lib.qlin_pca_leading_eigvec(A, 4096, 128, 10, 1e-9, A, A, A, A, None), _lib.QLIN_ERR_SHAPE)
    _err(lib.qlin_pca_fold_weight(A, 70000, 64, A, B, A, None), _lib.QLIN_ERR_SHAPE)
    _err(lib.qlin_pca_fold_weight(A, 128, 60, A, B, A, None), _lib.QLIN_ERR_SHAPE)
    _err(lib.qlin_pca_rotate(A, 4, 100, A, B, None), _lib.QLIN_ERR_SHAPE)
    _err(lib.qlin_pca_rotate(A, 4, 16384, A, B, None), _lib.QLIN_ERR_SHAPE)
    _err(lib.qlin_pca_rotate(A, 0, 128, A, B, None), _lib.QLIN_OK)
    _err(lib.qlin_pca_fold_weight(A, 128, 64, None, B, A, None), _lib.QLIN_ERR_INVALID_ARG)
    _err(lib.qlin_pca_rotate(A, 0, 128, A, B, None), _lib.QLIN_OK)
    _err(lib.qlin_pca_rotate(A, 4, 0, A, B, None), _lib.QLIN_ERR_SHAPE)


def test_binding_refuses_cpu_tensors():
    import torch
    from outlier_aware_bit_amd import qlin
    with pytest.raises(ValueError):
        qlin.qlin_quant_act(torch.zeros((4, 256), dtype=torch.float16))
    with pytest.raises(TypeError):
        qlin.qlin_quant_act(torch.zeros((4, 256), dtype=torch.float32))


def test_size_limits():
    # Every dimension below 2^31 and every operand at most 2^40 elements:
    # larger sizes are rejected before any size arithmetic can overflow.
    lib = _lib.load()
    big, bigger = 1 << 40, 1 << 62
    assert lib.qlin_packed_bytes(_lib.QLIN_LAYOUT_W8, big, big) == 0
    assert lib.qlin_packed_bytes(_lib.QLIN_LAYOUT_WO, bigger, 128) == 0
    assert lib.qlin_packed_bytes(_lib.QLIN_LAYOUT_W8, 1 << 20, 1 << 20) == 1 << 40
    _err(lib.qlin_gemm_w8a8(A, A, B, A, bigger, 128, 256, None, 0, None, A, None, None), _lib.QLIN_ERR_SHAPE)
    _err(lib.qlin_gemm_w8a8(A, A, B, A, 1 << 31, 128, 256, None, 0, None, A, None, None), _lib.QLIN_ERR_SHAPE)
    _err(lib.qlin_gemm_w4a8(A, A, B, A, None, 0, big, big, big, A, None, None, None), _lib.QLIN_ERR_SHAPE)
    _err(lib.qlin_quant_act(A, bigger, 256, None, B, A, None, 0, None, None, None, None), _lib.QLIN_ERR_SHAPE)
    _err(lib.qlin_momentum_update(A, bigger, 256, A, 4, A, 0.9, A, B, None, None), _lib.QLIN_ERR_SHAPE)
    _err(lib.qlin_pack_weight(_lib.QLIN_LAYOUT_W8, A, big, big, B, None), _lib.QLIN_ERR_SHAPE)
    _err(lib.qlin_pca_fold_weight(A, 128, bigger, A, B, A, None), _lib.QLIN_ERR_SHAPE)
