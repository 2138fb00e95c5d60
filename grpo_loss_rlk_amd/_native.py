"""ctypes loader and signatures for librlk.so (the C ABI of include/rlk.h).

The library is built in-tree (``python -m grpo_loss_rlk_amd.build``). There is
no fallback: if it is missing, loading raises.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "librlk.so")

c_i32, c_i64, c_f32, c_sz, c_vp = (ctypes.c_int32, ctypes.c_int64, ctypes.c_float,
                                   ctypes.c_size_t, ctypes.c_void_p)

RLK_OK, RLK_EINVAL, RLK_EUNSUPPORTED, RLK_EWORKSPACE, RLK_EHIP = 0, 1, 2, 3, 4
DTYPE_F32, DTYPE_BF16 = 0, 1
FLAG_OUTSIDE, FLAG_BAD_TARGET, FLAG_NONFINITE, FLAG_BOUNDARY, FLAG_BAD_PARAM = 1, 2, 4, 8, 16
FLAG_BAD_SUPPORT, FLAG_MISMATCH = 32, 64


class GrpoParams(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32), ("tis_cap", c_f32), ("eps_low", c_f32),
                ("eps_high", c_f32), ("kl_coef", c_f32), ("adv_eps", c_f32),
                ("std_ddof", c_i32), ("normalize_std", c_i32), ("loss_type", c_i32),
                ("correction", c_i32), ("aggregation", c_i32), ("filter_zero_adv", c_i32),
                ("baseline", c_i32), ("ipo_eps", c_f32), ("icepop_lo", c_f32),
                ("icepop_hi", c_f32)]


LOSS_TYPES = {"dapo": 0, "ipo": 1, "icepop": 2, "cispo": 3, "tis_pg": 4}
CORRECTIONS = {"tis": 0, "mis": 1}
AGGREGATIONS = {"token_mean": 0, "prompt_mean": 1}
BASELINES = {"mean": 0, "length": 1}


# name -> (restype, argtypes); every symbol include/rlk.h declares
SIGNATURES = {
    "rlk_abi_version": (c_i32, []),
    "rlk_status_str": (ctypes.c_char_p, [c_i32]),
    "rlk_last_error": (ctypes.c_char_p, []),
    "rlk_logprob_from_logits_workspace_size": (c_sz, [c_i64, c_i64, c_i32]),
    "rlk_logprob_from_logits": (c_i32, [
        c_vp, c_i32, c_i64, c_i64, c_i64, c_vp, c_f32, c_f32, c_vp, c_vp, c_i32, c_vp,
        c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_sz, c_vp]),
    "rlk_logprob_from_logits_noalloc": (c_i32, [
        c_vp, c_i32, c_i64, c_i64, c_i64, c_vp, c_f32, c_f32, c_vp, c_vp, c_i32, c_vp,
        c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp]),
    "rlk_logprob_from_support_workspace_size": (c_sz, [c_i64, c_i64, c_i32, c_f32]),
    "rlk_logprob_from_support": (c_i32, [
        c_vp, c_i32, c_i64, c_i64, c_i64, c_vp, c_f32, c_vp, c_vp, c_i64, c_f32, c_i32,
        c_vp, c_vp, c_vp, c_vp, c_sz, c_vp]),
    "rlk_sample_top_p_workspace_size": (c_sz, [c_i64, c_i64, c_i32]),
    "rlk_sample_top_p": (c_i32, [
        c_vp, c_i32, c_i64, c_i64, c_i64, c_f32, c_f32, c_i32, c_vp, c_vp, c_vp,
        ctypes.c_uint64, ctypes.c_uint32, c_vp,
        c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_sz, c_vp]),
    "rlk_logprob_fused_linear_workspace_size": (c_sz, [c_i64, c_i64, c_i64, c_f32, c_i32]),
    "rlk_logprob_fused_linear": (c_i32, [
        c_vp, c_vp, c_i64, c_i64, c_i64, c_i64, c_i64, c_vp, c_f32, c_f32, c_i32,
        c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_sz, c_vp]),
    "rlk_logprob_fused_linear_bwd_workspace_size": (c_sz, [c_i64, c_i64, c_i64, c_f32]),
    "rlk_logprob_fused_linear_bwd": (c_i32, [
        c_vp, c_vp, c_i64, c_i64, c_i64, c_i64, c_i64, c_vp, c_vp, c_vp, c_vp,
        c_f32, c_f32, c_i32, c_vp, c_vp, c_vp, c_sz, c_vp]),
    "rlk_grpo_token_loss_workspace_size": (c_sz, [c_i64, c_i64]),
    "rlk_grpo_token_loss": (c_i32, [
        c_vp, c_vp, c_vp, c_vp, c_i64, c_i64, c_vp, c_vp, c_i32, ctypes.POINTER(GrpoParams),
        c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_sz, c_vp]),
}

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library with typed signatures (raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m grpo_loss_rlk_amd.build` (there is no fallback path)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype, fn.argtypes = res, args
        _lib = L
    return _lib


class RlkError(RuntimeError):
    def __init__(self, status: int, where: str):
        L = lib()
        msg = L.rlk_last_error().decode() or L.rlk_status_str(status).decode()
        super().__init__(f"{where}: status {status} ({L.rlk_status_str(status).decode()}): {msg}")
        self.status = status


def check(status: int, where: str) -> None:
    if status != RLK_OK:
        raise RlkError(status, where)
