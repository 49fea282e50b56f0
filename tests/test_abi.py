"""The C ABI library on the CPU: it loads, exports what include/kq.h declares,
and rejects bad arguments on the host before any HIP call (no GPU needed)."""
import ctypes
import os
import re

import numpy as np
import pytest

import mxfp4_activation_quantizer_amd as kq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_symbols():
    text = open(os.path.join(ROOT, "include", "kq.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kq_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    return kq.lib()


def test_exports_every_declared_symbol(L):
    syms = declared_symbols()
    assert len(syms) >= 8
    for s in syms:
        assert hasattr(L, s), s
    assert sorted(kq.EXPORTS) == syms


P = ctypes.c_void_p
GOOD = P(0x10000)  # never dereferenced: every case below fails before a launch


@pytest.mark.parametrize("fn,args,status", [
    ("kq_quantize_mxfp4", (GOOD, 4, 33, 33, GOOD, GOOD, None), kq.KQ_ERR_SHAPE),
    ("kq_quantize_mxfp4", (GOOD, 4, 64, 32, GOOD, GOOD, None), kq.KQ_ERR_SHAPE),
    ("kq_quantize_mxfp4", (GOOD, -1, 64, 64, GOOD, GOOD, None), kq.KQ_ERR_SHAPE),
    ("kq_quantize_mxfp4", (None, 4, 64, 64, GOOD, GOOD, None), kq.KQ_ERR_NULL),
    ("kq_quantize_mxfp4", (GOOD, 4, 64, 64, None, GOOD, None), kq.KQ_ERR_NULL),
    ("kq_quantize_mxfp4", (GOOD, 4, 64, 64, GOOD, None, None), kq.KQ_ERR_NULL),
    ("kq_quantize_mxfp4", (P(0x10002), 4, 64, 64, GOOD, GOOD, None), kq.KQ_ERR_ALIGN),
    ("kq_quantize_mxfp4", (GOOD, 4, 64, 68, GOOD, GOOD, None), kq.KQ_ERR_ALIGN),
    ("kq_quantize_mxfp4", (GOOD, 4, 64, 64, P(0x10004), GOOD, None), kq.KQ_ERR_ALIGN),
    ("kq_quantize_mxfp4", (None, 0, 64, 64, None, None, None), kq.KQ_OK),
    ("kq_quantize_mxfp4", (None, 5, 0, 0, None, None, None), kq.KQ_OK),
    ("kq_transform_quantize_mxfp4", (GOOD, 4, 64, 64, None, GOOD, GOOD, None, None), kq.KQ_ERR_NULL),
    ("kq_transform_quantize_mxfp4", (GOOD, 4, 64, 64, P(0x10008), GOOD, GOOD, None, None), kq.KQ_ERR_ALIGN),
    ("kq_transform_quantize_mxfp4", (GOOD, 4, 64, 64, GOOD, GOOD, GOOD, P(0x10004), None), kq.KQ_ERR_ALIGN),
    ("kq_transform_quantize_mxfp4", (GOOD, 4, 48, 64, GOOD, GOOD, GOOD, None, None), kq.KQ_ERR_SHAPE),
    ("kq_transform_quantize_mxfp4_form", (GOOD, 4, 64, 64, GOOD, GOOD, GOOD, None, 3, None), kq.KQ_ERR_UNSUPPORTED),
    ("kq_transform_quantize_mxfp4_form", (GOOD, 4, 64, 64, GOOD, GOOD, GOOD, None, -1, None), kq.KQ_ERR_UNSUPPORTED),
    ("kq_transform_quantize_mxfp4_form", (GOOD, 4, 64, 64, None, GOOD, GOOD, None, 1, None), kq.KQ_ERR_NULL),
    ("kq_transform_quantize_mxfp4_form", (GOOD, 4, 48, 64, GOOD, GOOD, GOOD, None, 2, None), kq.KQ_ERR_SHAPE),
    ("kq_transform_quantize_mxfp4_form", (None, 0, 64, 64, None, None, None, None, 0, None), kq.KQ_OK),
    ("kq_smoothquant_quantize_mxfp4", (GOOD, 4, 64, 64, None, GOOD, GOOD, None), kq.KQ_ERR_NULL),
    ("kq_smoothquant_quantize_mxfp4", (GOOD, 4, 64, 64, P(0x10004), GOOD, GOOD, None), kq.KQ_ERR_ALIGN),
    ("kq_quantize_mxfp4_f32", (GOOD, 4, 64, 66, GOOD, GOOD, None), kq.KQ_ERR_ALIGN),
    ("kq_quantize_mxfp4_f32", (GOOD, 4, 64, 32, GOOD, GOOD, None), kq.KQ_ERR_SHAPE),
    ("kq_quantize_mxfp4_f32", (None, 4, 64, 64, GOOD, GOOD, None), kq.KQ_ERR_NULL),
    ("kq_inverse_fold_weights", (GOOD, 4, 40, GOOD, GOOD, None), kq.KQ_ERR_SHAPE),
    ("kq_inverse_fold_weights", (GOOD, 4, 64, None, GOOD, None), kq.KQ_ERR_NULL),
    ("kq_inverse_fold_weights", (GOOD, 4, 64, GOOD, P(0x10004), None), kq.KQ_ERR_ALIGN),
    ("kq_inverse_fold_weights", (None, 0, 64, None, None, None), kq.KQ_OK),
    ("kq_mxfp4_gemm", (GOOD, GOOD, GOOD, GOOD, 4, 4, 48, GOOD, 4, None), kq.KQ_ERR_SHAPE),
    ("kq_mxfp4_gemm", (GOOD, GOOD, GOOD, GOOD, 4, 4, 64, GOOD, 3, None), kq.KQ_ERR_SHAPE),
    ("kq_mxfp4_gemm", (GOOD, None, GOOD, GOOD, 4, 4, 64, GOOD, 4, None), kq.KQ_ERR_NULL),
    ("kq_mxfp4_gemm", (P(0x10008), GOOD, GOOD, GOOD, 4, 4, 64, GOOD, 4, None), kq.KQ_ERR_ALIGN),
    ("kq_mxfp4_gemm", (None, None, None, None, 0, 4, 64, None, 4, None), kq.KQ_OK),
    ("kq_mxfp4_gemm_wide", (GOOD, GOOD, GOOD, GOOD, 4, 4, 48, GOOD, 4, None), kq.KQ_ERR_SHAPE),
    ("kq_mxfp4_gemm_wide", (GOOD, GOOD, GOOD, GOOD, 4, 4, 64, GOOD, 3, None), kq.KQ_ERR_SHAPE),
    ("kq_mxfp4_gemm_wide", (GOOD, None, GOOD, GOOD, 4, 4, 64, GOOD, 4, None), kq.KQ_ERR_NULL),
    ("kq_mxfp4_gemm_wide", (GOOD, GOOD, None, GOOD, 4, 4, 64, GOOD, 4, None), kq.KQ_ERR_NULL),
    ("kq_mxfp4_gemm_wide", (P(0x10008), GOOD, GOOD, GOOD, 4, 4, 64, GOOD, 4, None), kq.KQ_ERR_ALIGN),
    ("kq_mxfp4_gemm_wide", (GOOD, GOOD, GOOD, P(0x10002), 4, 4, 128, GOOD, 4, None), kq.KQ_ERR_ALIGN),
    ("kq_mxfp4_gemm_wide", (None, None, None, None, 0, 4, 64, None, 4, None), kq.KQ_OK),
    ("kq_lowrank_project_bf16", (GOOD, 4, 48, 48, GOOD, 32, GOOD, None), kq.KQ_ERR_SHAPE),
    ("kq_lowrank_project_bf16", (GOOD, 4, 64, 64, GOOD, 48, GOOD, None), kq.KQ_ERR_SHAPE),
    ("kq_lowrank_project_bf16", (GOOD, 4, 64, 32, GOOD, 32, GOOD, None), kq.KQ_ERR_SHAPE),
    ("kq_lowrank_project_bf16", (GOOD, 4, 64, 64, None, 32, GOOD, None), kq.KQ_ERR_NULL),
    ("kq_lowrank_project_bf16", (GOOD, 4, 64, 64, P(0x10008), 32, GOOD, None), kq.KQ_ERR_ALIGN),
    ("kq_lowrank_project_bf16", (GOOD, 4, 64, 68, GOOD, 32, GOOD, None), kq.KQ_ERR_ALIGN),
    ("kq_lowrank_project_bf16", (None, 0, 64, 64, None, 32, None, None), kq.KQ_OK),
    ("kq_dequantize_mxfp4_bf16", (GOOD, GOOD, 4, 48, GOOD, None), kq.KQ_ERR_SHAPE),
    ("kq_dequantize_mxfp4_bf16", (None, GOOD, 4, 64, GOOD, None), kq.KQ_ERR_NULL),
    ("kq_dequantize_mxfp4_bf16", (GOOD, GOOD, 4, 64, P(0x10008), None), kq.KQ_ERR_ALIGN),
    ("kq_dequantize_mxfp4_bf16", (None, None, 0, 64, None, None), kq.KQ_OK),
    ("kq_pack_mxfp4_scales", (GOOD, 4, 128, GOOD, None), kq.KQ_ERR_SHAPE),
    ("kq_pack_mxfp4_scales", (GOOD, -1, 256, GOOD, None), kq.KQ_ERR_SHAPE),
    ("kq_pack_mxfp4_scales", (None, 4, 256, GOOD, None), kq.KQ_ERR_NULL),
    ("kq_pack_mxfp4_scales", (GOOD, 4, 256, None, None), kq.KQ_ERR_NULL),
    ("kq_pack_mxfp4_scales", (GOOD, 4, 256, P(0x10004), None), kq.KQ_ERR_ALIGN),
    ("kq_pack_mxfp4_scales", (None, 0, 256, None, None), kq.KQ_OK),
    ("kq_pack_mxfp4_scales", (None, 4, 0, None, None), kq.KQ_OK),
    ("kq_mxfp4_gemm_packed", (GOOD, GOOD, GOOD, GOOD, 4, 4, 128, GOOD, 4, None), kq.KQ_ERR_SHAPE),
    ("kq_mxfp4_gemm_packed", (GOOD, GOOD, GOOD, GOOD, 4, 4, 256, GOOD, 3, None), kq.KQ_ERR_SHAPE),
    ("kq_mxfp4_gemm_packed", (GOOD, GOOD, GOOD, GOOD, -1, 4, 256, GOOD, 4, None), kq.KQ_ERR_SHAPE),
    ("kq_mxfp4_gemm_packed", (GOOD, None, GOOD, GOOD, 4, 4, 256, GOOD, 4, None), kq.KQ_ERR_NULL),
    ("kq_mxfp4_gemm_packed", (GOOD, GOOD, GOOD, GOOD, 4, 4, 256, None, 4, None), kq.KQ_ERR_NULL),
    ("kq_mxfp4_gemm_packed", (P(0x10008), GOOD, GOOD, GOOD, 4, 4, 256, GOOD, 4, None), kq.KQ_ERR_ALIGN),
    ("kq_mxfp4_gemm_packed", (GOOD, P(0x10008), GOOD, GOOD, 4, 4, 256, GOOD, 4, None), kq.KQ_ERR_ALIGN),
    ("kq_mxfp4_gemm_packed", (GOOD, GOOD, GOOD, GOOD, 4, 4, 256, P(0x10002), 4, None), kq.KQ_ERR_ALIGN),
    ("kq_mxfp4_gemm_packed", (GOOD, GOOD, GOOD, GOOD, 4, 4, 1 << 24, GOOD, 4, None), kq.KQ_ERR_UNSUPPORTED),
    ("kq_mxfp4_gemm_packed", (None, None, None, None, 0, 4, 256, None, 4, None), kq.KQ_OK),
    ("kq_mxfp4_gemm_packed_lowrank_split", (GOOD, GOOD, GOOD, GOOD, 4, 4, 256, GOOD, GOOD, GOOD, 48, GOOD, 4, None),
     kq.KQ_ERR_SHAPE),
    ("kq_mxfp4_gemm_packed_lowrank_split", (GOOD, GOOD, GOOD, GOOD, 4, 4, 128, GOOD, GOOD, GOOD, 32, GOOD, 4, None),
     kq.KQ_ERR_SHAPE),
    ("kq_mxfp4_gemm_packed_lowrank_split", (GOOD, GOOD, GOOD, GOOD, 4, 4, 256, GOOD, None, GOOD, 32, GOOD, 4, None),
     kq.KQ_ERR_NULL),
    ("kq_mxfp4_gemm_packed_lowrank_split", (GOOD, GOOD, GOOD, GOOD, 4, 4, 256, GOOD, GOOD, P(0x10008), 32, GOOD, 4,
                                            None), kq.KQ_ERR_ALIGN),
    ("kq_mxfp4_gemm_packed_lowrank_split", (GOOD, GOOD, GOOD, GOOD, 4, 4, 256, GOOD, GOOD, GOOD, 1 << 22, GOOD, 4,
                                            None), kq.KQ_ERR_UNSUPPORTED),
    ("kq_mxfp4_gemm_packed_lowrank_split", (None, None, None, None, 0, 4, 256, None, None, None, 32, None, 4, None),
     kq.KQ_OK),
    ("kq_lowrank_project_bf16_split", (GOOD, 4, 64, 64, GOOD, 48, GOOD, GOOD, None), kq.KQ_ERR_SHAPE),
    ("kq_lowrank_project_bf16_split", (GOOD, 4, 64, 64, GOOD, 32, GOOD, None, None), kq.KQ_ERR_NULL),
    ("kq_lowrank_project_bf16_split", (GOOD, 4, 64, 64, GOOD, 32, P(0x10008), GOOD, None), kq.KQ_ERR_ALIGN),
    ("kq_lowrank_project_bf16_split", (None, 0, 64, 64, None, 32, None, None, None), kq.KQ_OK),
    ("kq_lowrank_project_split", (GOOD, 4, 64, 64, GOOD, GOOD, 48, GOOD, GOOD, None), kq.KQ_ERR_SHAPE),
    ("kq_lowrank_project_split", (GOOD, 4, 64, 64, GOOD, None, 32, GOOD, GOOD, None), kq.KQ_ERR_NULL),
    ("kq_lowrank_project_split", (GOOD, 4, 64, 64, P(0x10008), GOOD, 32, GOOD, GOOD, None), kq.KQ_ERR_ALIGN),
    ("kq_lowrank_project_split", (None, 0, 64, 64, None, None, 32, None, None, None), kq.KQ_OK),
    ("kq_mxfp4_gemm_packed_bf16", (GOOD, GOOD, GOOD, GOOD, 4, 4, 128, GOOD, 4, None), kq.KQ_ERR_SHAPE),
    ("kq_mxfp4_gemm_packed_bf16", (GOOD, GOOD, GOOD, GOOD, 4, 4, 256, GOOD, 3, None), kq.KQ_ERR_SHAPE),
    ("kq_mxfp4_gemm_packed_bf16", (GOOD, GOOD, GOOD, GOOD, 4, 4, 256, None, 4, None), kq.KQ_ERR_NULL),
    ("kq_mxfp4_gemm_packed_bf16", (GOOD, GOOD, GOOD, GOOD, 4, 4, 256, P(0x10001), 4, None), kq.KQ_ERR_ALIGN),
    ("kq_mxfp4_gemm_packed_bf16", (GOOD, GOOD, GOOD, GOOD, 4, 4, 1 << 24, GOOD, 4, None), kq.KQ_ERR_UNSUPPORTED),
    ("kq_mxfp4_gemm_packed_bf16", (None, None, None, None, 4, 0, 256, None, 4, None), kq.KQ_OK),
    ("kq_mxfp4_gemm_packed_lowrank", (GOOD, GOOD, GOOD, GOOD, 4, 4, 256, GOOD, GOOD, GOOD, 48, GOOD, 4, None),
     kq.KQ_ERR_SHAPE),
    ("kq_mxfp4_gemm_packed_lowrank", (GOOD, GOOD, GOOD, GOOD, 4, 4, 128, GOOD, GOOD, GOOD, 32, GOOD, 4, None),
     kq.KQ_ERR_SHAPE),
    ("kq_mxfp4_gemm_packed_lowrank", (GOOD, GOOD, GOOD, GOOD, 4, 4, 256, None, GOOD, GOOD, 32, GOOD, 4, None),
     kq.KQ_ERR_NULL),
    ("kq_mxfp4_gemm_packed_lowrank", (GOOD, GOOD, GOOD, GOOD, 4, 4, 256, P(0x10008), GOOD, GOOD, 32, GOOD, 4, None),
     kq.KQ_ERR_ALIGN),
    ("kq_mxfp4_gemm_packed_lowrank", (None, None, None, None, 0, 4, 256, None, None, None, 32, None, 4, None),
     kq.KQ_OK),
    ("kq_transform_quantize_mxfp4_gemm", (GOOD, 4, 48, 48, GOOD, GOOD, GOOD, 4, GOOD, 4, None),
     kq.KQ_ERR_SHAPE),
    ("kq_transform_quantize_mxfp4_gemm", (GOOD, 4, 64, 64, GOOD, GOOD, GOOD, 4, GOOD, 3, None),
     kq.KQ_ERR_SHAPE),
    ("kq_transform_quantize_mxfp4_gemm", (GOOD, 4, 64, 32, GOOD, GOOD, GOOD, 4, GOOD, 4, None),
     kq.KQ_ERR_SHAPE),
    ("kq_transform_quantize_mxfp4_gemm", (GOOD, 4, 64, 64, None, GOOD, GOOD, 4, GOOD, 4, None),
     kq.KQ_ERR_NULL),
    ("kq_transform_quantize_mxfp4_gemm", (GOOD, 4, 64, 64, GOOD, GOOD, GOOD, 4, None, 4, None),
     kq.KQ_ERR_NULL),
    ("kq_transform_quantize_mxfp4_gemm", (P(0x10008), 4, 64, 64, GOOD, GOOD, GOOD, 4, GOOD, 4, None),
     kq.KQ_ERR_ALIGN),
    ("kq_transform_quantize_mxfp4_gemm", (GOOD, 4, 64, 68, GOOD, GOOD, GOOD, 4, GOOD, 4, None),
     kq.KQ_ERR_ALIGN),
    ("kq_transform_quantize_mxfp4_gemm", (GOOD, 4, 64, 64, P(0x10004), GOOD, GOOD, 4, GOOD, 4, None),
     kq.KQ_ERR_ALIGN),
    ("kq_transform_quantize_mxfp4_gemm", (None, 0, 64, 64, None, None, None, 4, None, 4, None), kq.KQ_OK),
    ("kq_hadamard_quantize_mxfp4", (GOOD, 4, 96, 96, 48, GOOD, GOOD, None, None), kq.KQ_ERR_SHAPE),
    ("kq_hadamard_quantize_mxfp4", (GOOD, 4, 64, 64, 16, GOOD, GOOD, None, None), kq.KQ_ERR_SHAPE),
    ("kq_hadamard_quantize_mxfp4", (GOOD, 4, 96, 96, 64, GOOD, GOOD, None, None), kq.KQ_ERR_SHAPE),
    ("kq_hadamard_quantize_mxfp4", (GOOD, 4, 32768, 32768, 32768, GOOD, GOOD, None, None),
     kq.KQ_ERR_UNSUPPORTED),
    ("kq_hadamard_quantize_mxfp4", (None, 4, 64, 64, 64, GOOD, GOOD, None, None), kq.KQ_ERR_NULL),
    ("kq_hadamard_quantize_mxfp4", (GOOD, 4, 64, 64, 64, GOOD, GOOD, P(0x10004), None), kq.KQ_ERR_ALIGN),
    ("kq_hadamard_quantize_mxfp4", (GOOD, 4, 64, 68, 64, GOOD, GOOD, None, None), kq.KQ_ERR_ALIGN),
    ("kq_hadamard_quantize_mxfp4", (None, 0, 1024, 1024, 1024, None, None, None, None), kq.KQ_OK),
    ("kq_transform_quantize_mxfp4_y16", (GOOD, 4, 64, 64, GOOD, GOOD, GOOD, None, None), kq.KQ_ERR_NULL),
    ("kq_transform_quantize_mxfp4_y16", (GOOD, 4, 64, 64, GOOD, GOOD, GOOD, P(0x10008), None), kq.KQ_ERR_ALIGN),
    ("kq_transform_quantize_mxfp4_packed", (GOOD, 4, 128, 128, GOOD, GOOD, GOOD, None, None), kq.KQ_ERR_SHAPE),
    ("kq_transform_quantize_mxfp4_packed", (GOOD, 4, 256, 256, None, GOOD, GOOD, None, None), kq.KQ_ERR_NULL),
    ("kq_transform_quantize_mxfp4_packed", (GOOD, 4, 256, 256, GOOD, GOOD, None, None, None), kq.KQ_ERR_NULL),
    ("kq_transform_quantize_mxfp4_packed", (GOOD, 4, 256, 256, GOOD, GOOD, GOOD, P(0x10008), None),
     kq.KQ_ERR_ALIGN),
    ("kq_transform_quantize_mxfp4_packed", (GOOD, 4, 256, 256, P(0x10004), GOOD, GOOD, None, None),
     kq.KQ_ERR_ALIGN),
    ("kq_transform_quantize_mxfp4_packed", (GOOD, 1 << 30, 256, 256, GOOD, GOOD, GOOD, None, None),
     kq.KQ_ERR_UNSUPPORTED),
    ("kq_transform_quantize_mxfp4_packed", (None, 0, 256, 256, None, None, None, None, None), kq.KQ_OK),
    ("kq_lowrank_project", (GOOD, 4, 64, 64, GOOD, GOOD, 48, GOOD, None), kq.KQ_ERR_SHAPE),
    ("kq_lowrank_project", (GOOD, 4, 64, 60, GOOD, GOOD, 32, GOOD, None), kq.KQ_ERR_SHAPE),
    ("kq_lowrank_project", (GOOD, 4, 64, 72, GOOD, GOOD, 32, P(0x10004), None), kq.KQ_ERR_ALIGN),
    ("kq_lowrank_project", (None, 4, 64, 64, GOOD, GOOD, 32, GOOD, None), kq.KQ_ERR_NULL),
    ("kq_mxfp4_gemm_lowrank", (GOOD, GOOD, GOOD, GOOD, 4, 4, 64, GOOD, GOOD, GOOD, 0, GOOD, 4, None),
     kq.KQ_ERR_SHAPE),
    ("kq_mxfp4_gemm_lowrank", (GOOD, GOOD, GOOD, GOOD, 4, 4, 64, None, GOOD, GOOD, 32, GOOD, 4, None),
     kq.KQ_ERR_NULL),
    ("kq_mxfp4_gemm_lowrank", (GOOD, GOOD, GOOD, GOOD, 4, 4, 64, P(0x10004), GOOD, GOOD, 32, GOOD, 4, None),
     kq.KQ_ERR_ALIGN),
    ("kq_gemm_f32", (0, 0, 4, 4, 4, 1.0, None, 4, GOOD, 4, 0.0, None, 4, GOOD, 4, None), kq.KQ_ERR_NULL),
    ("kq_gemm_f32", (0, 0, 4, 4, 8, 1.0, GOOD, 4, GOOD, 4, 0.0, None, 4, GOOD, 4, None), kq.KQ_ERR_SHAPE),
    ("kq_gemm_f32", (0, 0, 4, 4, 4, 1.0, GOOD, 4, GOOD, 4, 1.0, None, 4, GOOD, 4, None), kq.KQ_ERR_NULL),
    ("kq_gemm_f32", (0, 0, -1, 4, 4, 1.0, GOOD, 4, GOOD, 4, 0.0, None, 4, GOOD, 4, None), kq.KQ_ERR_SHAPE),
    ("kq_gemm_f32", (0, 0, 0, 4, 4, 1.0, None, 4, None, 4, 0.0, None, 4, None, 4, None), kq.KQ_OK),
    ("kq_calib_init", (GOOD, 64, 48, GOOD, 16, GOOD, 1 << 30, None), kq.KQ_ERR_SHAPE),
    ("kq_calib_init", (None, 64, 64, GOOD, 16, GOOD, 1 << 30, None), kq.KQ_ERR_NULL),
    ("kq_calib_init", (GOOD, 64, 64, GOOD, 16, P(0x10010), 1 << 30, None), kq.KQ_ERR_ALIGN),
    ("kq_calib_init", (GOOD, 64, 64, GOOD, 16, GOOD, 1024, None), kq.KQ_ERR_SHAPE),
    ("kq_calib_step", (GOOD, 64, 64, 16, GOOD, GOOD, GOOD, 0, 1e-3, 0.9, 0.999, 1e-8, GOOD, 1, GOOD, None,
                       GOOD, 1 << 30, None), kq.KQ_ERR_SHAPE),
    ("kq_calib_step", (GOOD, 64, 64, 16, GOOD, GOOD, GOOD, 1, 1e-3, 1.0, 0.999, 1e-8, GOOD, 1, GOOD, None,
                       GOOD, 1 << 30, None), kq.KQ_ERR_SHAPE),
    ("kq_calib_step", (GOOD, 64, 64, 16, GOOD, GOOD, GOOD, 1, -1.0, 0.9, 0.999, 1e-8, GOOD, 1, GOOD, None,
                       GOOD, 1 << 30, None), kq.KQ_ERR_SHAPE),
    ("kq_calib_step", (GOOD, 64, 64, 16, GOOD, None, GOOD, 1, 1e-3, 0.9, 0.999, 1e-8, GOOD, 1, GOOD, None,
                       GOOD, 1 << 30, None), kq.KQ_ERR_NULL),
    ("kq_calib_step", (GOOD, 64, 64, 16, GOOD, GOOD, GOOD, 1, 1e-3, 0.9, 0.999, 1e-8, GOOD, 1, GOOD, None,
                       GOOD, 4096, None), kq.KQ_ERR_SHAPE),
    ("kq_calib_step_noalloc", (GOOD, GOOD, 4096, 1152, 1152, GOOD, GOOD, GOOD, 1, 1e-3, 0.9, 0.999, 1e-8, GOOD, 1,
                               GOOD, None, None), kq.KQ_ERR_UNSUPPORTED),
    ("kq_calib_step_noalloc", (None, GOOD, 256, 256, 128, GOOD, GOOD, GOOD, 1, 1e-3, 0.9, 0.999, 1e-8, GOOD, 1,
                               GOOD, None, None), kq.KQ_ERR_NULL),
    ("kq_calib_step_noalloc", (GOOD, GOOD, 256, 250, 128, GOOD, GOOD, GOOD, 1, 1e-3, 0.9, 0.999, 1e-8, GOOD, 1,
                               GOOD, None, None), kq.KQ_ERR_SHAPE),
    ("kq_calib_step_noalloc", (GOOD, GOOD, 256, 256, 128, GOOD, GOOD, GOOD, 0, 1e-3, 0.9, 0.999, 1e-8, GOOD, 1,
                               GOOD, None, None), kq.KQ_ERR_SHAPE),
    ("kq_calib_step_noalloc", (P(0x10008), GOOD, 256, 256, 128, GOOD, GOOD, GOOD, 1, 1e-3, 0.9, 0.999, 1e-8, GOOD,
                               1, GOOD, None, None), kq.KQ_ERR_ALIGN),
])
def test_host_argument_checks(L, fn, args, status):
    assert getattr(L, fn)(*args) == status


def test_status_strings(L):
    for s in range(6):
        assert L.kq_status_string(s).startswith(b"KQ_")
    assert L.kq_last_hip_error() == 0


def test_factors_from_lu_matches_eq6(orc):
    rng = np.random.default_rng(2)
    abc = rng.standard_normal((9, 5, 3))
    abc[..., 0] = np.where(np.abs(abc[..., 0]) < 0.1, 0.5, abc[..., 0])
    got = kq.factors_from_lu(abc)
    want = orc.factors_from_lu(abc).astype(np.float32)
    assert np.array_equal(got, want)
    bad = abc.copy()
    bad[3, 2, 0] = 0.0
    with pytest.raises(kq.KQError):
        kq.factors_from_lu(bad)


def test_calib_workspace_bytes(L):
    n = ctypes.c_int64(0)
    assert L.kq_calib_workspace_bytes(4096, 1152, 1152, ctypes.byref(n)) == kq.KQ_OK
    floats = 4096 * 1152 * 6 + 1152 * 1152 * 3  # A, X, Q(X), grad (M x d); C0, E (M x o); Y, Q(Y), grad (o x d)
    assert n.value >= floats * 4
    assert L.kq_calib_workspace_bytes(4096, 1000, 16, ctypes.byref(n)) == kq.KQ_ERR_SHAPE
    assert L.kq_calib_workspace_bytes(4096, 1024, 16, None) == kq.KQ_ERR_NULL
    assert L.kq_calib_workspace_bytes(1 << 20, 4096, 16, ctypes.byref(n)) == kq.KQ_ERR_UNSUPPORTED
