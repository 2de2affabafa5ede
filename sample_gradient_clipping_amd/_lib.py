"""ctypes declarations for libdpfused.so (the C ABI in include/dpfused.h).

Loading fails loudly when the library has not been built: there is no
fallback path.  Build it with ``python -m sample_gradient_clipping_amd.build``.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdpfused.so")

DPF_OK = 0
DPF_ERR_INVALID_ARGUMENT = 1
DPF_ERR_UNSUPPORTED = 2
DPF_ERR_OUT_OF_MEMORY = 3
DPF_ERR_HIP = 4

DPF_F32 = 0
DPF_BF16 = 1


class DpfAct(ctypes.Structure):
    """Mirror of dpf_act: one [B, T, D] tensor, last dim contiguous, strides in elements."""
    _fields_ = [
        ("data", ctypes.c_void_p),
        ("dtype", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
        ("B", ctypes.c_int64),
        ("T", ctypes.c_int64),
        ("D", ctypes.c_int64),
        ("stride_b", ctypes.c_int64),
        ("stride_t", ctypes.c_int64),
    ]


class DpfError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{status_name(status)}: {message}")
        self.status = status


_lib = None

# name -> (restype, argtypes)
_SIGNATURES = {
    "dpfused_linear_clip_accumulate": (ctypes.c_int, [
        ctypes.POINTER(DpfAct), ctypes.POINTER(DpfAct), ctypes.c_void_p, ctypes.c_float,
        ctypes.c_float, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_void_p]),
    "dpfused_linear_clip_accumulate_ex": (ctypes.c_int, [
        ctypes.POINTER(DpfAct), ctypes.POINTER(DpfAct), ctypes.c_void_p, ctypes.c_float,
        ctypes.c_float, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_float, ctypes.c_int32,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    "dpfused_linear_clip_accumulate_noalloc": (ctypes.c_int, [
        ctypes.POINTER(DpfAct), ctypes.POINTER(DpfAct), ctypes.c_void_p, ctypes.c_float,
        ctypes.c_float, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_void_p]),
    "dpfused_linear_clip_accumulate_projected": (ctypes.c_int, [
        ctypes.POINTER(DpfAct), ctypes.POINTER(DpfAct), ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_int64, ctypes.c_float, ctypes.c_float, ctypes.c_uint64, ctypes.c_uint64,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    "dpfused_linear_clip_accumulate_projected_seeded": (ctypes.c_int, [
        ctypes.POINTER(DpfAct), ctypes.POINTER(DpfAct), ctypes.c_void_p, ctypes.c_int64,
        ctypes.c_uint64, ctypes.c_uint64, ctypes.c_float, ctypes.c_float, ctypes.c_float,
        ctypes.c_uint64, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    "dpfused_linear_clip_accumulate_bias": (ctypes.c_int, [
        ctypes.POINTER(DpfAct), ctypes.POINTER(DpfAct), ctypes.c_void_p, ctypes.c_float,
        ctypes.c_float, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_void_p, ctypes.c_void_p]),
    "dpfused_linear_clip_accumulate_projected_many": (ctypes.c_int, [
        ctypes.c_int32, ctypes.POINTER(DpfAct), ctypes.POINTER(DpfAct),
        ctypes.POINTER(ctypes.c_void_p), ctypes.POINTER(ctypes.c_void_p), ctypes.c_int64,
        ctypes.c_float, ctypes.c_float, ctypes.c_uint64, ctypes.POINTER(ctypes.c_uint64),
        ctypes.POINTER(ctypes.c_void_p), ctypes.POINTER(ctypes.c_void_p), ctypes.c_void_p]),
    "dpfused_group_clip_accumulate": (ctypes.c_int, [
        ctypes.c_int32, ctypes.POINTER(DpfAct), ctypes.POINTER(DpfAct), ctypes.c_void_p,
        ctypes.c_float, ctypes.c_float, ctypes.c_uint64, ctypes.POINTER(ctypes.c_uint64),
        ctypes.POINTER(ctypes.c_void_p), ctypes.c_void_p, ctypes.c_void_p]),
    "dpfused_projected_adam_step": (ctypes.c_int, [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
        ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_float, ctypes.c_float,
        ctypes.c_float, ctypes.c_float, ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint64,
        ctypes.c_uint64, ctypes.c_float, ctypes.c_void_p]),
    "dpfused_per_sample_sqnorms": (ctypes.c_int, [
        ctypes.POINTER(DpfAct), ctypes.POINTER(DpfAct), ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_int32, ctypes.c_void_p]),
    "dpfused_clip_factors": (ctypes.c_int, [
        ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_void_p]),
    "dpfused_scaled_accumulate": (ctypes.c_int, [
        ctypes.POINTER(DpfAct), ctypes.POINTER(DpfAct), ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_float, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_void_p]),
    "dpfused_philox4x32_10": (ctypes.c_int, [
        ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]),
    "dpfused_gaussian_fill": (ctypes.c_int, [
        ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int64, ctypes.c_float, ctypes.c_int32,
        ctypes.c_void_p, ctypes.c_void_p]),
    "dpfused_noise_blocks": (ctypes.c_uint64, [ctypes.c_int64]),
    "dpfused_set_option": (ctypes.c_int, [ctypes.c_char_p, ctypes.c_int64]),
    "dpfused_get_option": (ctypes.c_int64, [ctypes.c_char_p]),
    "dpfused_timing_reset": (None, []),
    "dpfused_timing_collect": (ctypes.c_int32, []),
    "dpfused_timing_name": (ctypes.c_char_p, [ctypes.c_int32]),
    "dpfused_project": (ctypes.c_int, [ctypes.POINTER(DpfAct), ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]),
    "dpfused_timing_total_ms": (ctypes.c_double, [ctypes.c_int32]),
    "dpfused_timing_launches": (ctypes.c_int64, [ctypes.c_int32]),
    "dpfused_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "dpfused_last_error": (ctypes.c_char_p, []),
    "dpfused_abi_version": (ctypes.c_int32, []),
}

EXPECTED_ABI_VERSION = 1


def lib():
    """The loaded library (loaded once).  Raises if it is missing or stale."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build the HIP library first "
                "(python -m sample_gradient_clipping_amd.build)")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        if handle.dpfused_abi_version() != EXPECTED_ABI_VERSION:
            raise ImportError("libdpfused ABI version mismatch; rebuild the library")
        _lib = handle
    return _lib


def status_name(status: int) -> str:
    return lib().dpfused_status_string(int(status)).decode()


def check(status: int) -> None:
    if status != DPF_OK:
        raise DpfError(status, lib().dpfused_last_error().decode())
