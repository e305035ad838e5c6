"""ctypes binding of libegs.so (include/egs.h).

Argument marshalling only: torch tensors supply device pointers and the
current HIP stream; every step of the method runs in the library's kernels.
Importing this module fails loudly when the library has not been built.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libegs.so")

EGS_OK, EGS_EINVAL, EGS_ENOTSUP, EGS_EWORKSPACE, EGS_EHIP = range(5)
EGS_BF16, EGS_F32 = 0, 1
EGS_SHANNON, EGS_RENYI = 0, 1
EGS_POOL_MEAN_PROBE, EGS_POOL_MAXMIN = 0, 1
EGS_BUDGET_FIXED, EGS_BUDGET_TWO_LEVEL, EGS_BUDGET_PROPORTIONAL, EGS_BUDGET_ALG3 = range(4)
EGS_PAGE_GROUP, EGS_PAGE_LAYER_UNION, EGS_PAGE_HEAD_UNION = 0, 1, 2
EGS_STATIC_SCRATCH_BYTES = 64 << 20
ABI_VERSION = 7


class PrefillShapeC(ctypes.Structure):
    _fields_ = [("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("seq_len", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("segment_size", ctypes.c_int32),
                ("probe_len", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("sm_scale", ctypes.c_float)]


class BudgetPolicyC(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int32), ("frac", ctypes.c_double),
                ("frac_rigid", ctypes.c_double), ("frac_dynamic", ctypes.c_double),
                ("frac_min", ctypes.c_double), ("frac_max", ctypes.c_double),
                ("entropy_threshold", ctypes.c_double), ("base_tokens", ctypes.c_double),
                ("alg3_alpha", ctypes.c_double), ("alg3_delta_t", ctypes.c_double)]


class DecodeShapeC(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("cache_len", ctypes.c_int32), ("n_obs", ctypes.c_int32),
                ("n_sink", ctypes.c_int32), ("n_recent", ctypes.c_int32),
                ("n_keep", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("sm_scale", ctypes.c_float)]


class RetainParamsC(ctypes.Structure):
    _fields_ = [("entropy_kind", ctypes.c_int32), ("renyi_alpha", ctypes.c_float),
                ("zeta", ctypes.c_double), ("tau", ctypes.c_double),
                ("raw_logit_mode", ctypes.c_int32), ("info_alpha", ctypes.c_double)]


class LatentStateC(ctypes.Structure):
    _fields_ = [("length", ctypes.c_int32), ("generated", ctypes.c_int32),
                ("n_delay", ctypes.c_int32), ("interval", ctypes.c_int32),
                ("compressed", ctypes.c_int32)]


class PruneParamsC(ctypes.Structure):
    _fields_ = [("eps_s", ctypes.c_double), ("lam", ctypes.c_double), ("eps", ctypes.c_double),
                ("m0", ctypes.c_int32), ("target", ctypes.c_int32), ("zeta", ctypes.c_double),
                ("tau", ctypes.c_double)]


_P = ctypes.c_void_p
_PS = ctypes.POINTER(PrefillShapeC)
_DS = ctypes.POINTER(DecodeShapeC)
_ST = ctypes.c_int32

# name -> (restype, argtypes); mirrors include/egs.h
SIGNATURES = {
    "egs_entropy_score_workspace": (ctypes.c_size_t, [_PS]),
    "egs_entropy_score": (_ST, [_PS, ctypes.c_int32, ctypes.c_int32, ctypes.c_float, _P, _P,
                                _P, _P, _P, ctypes.c_size_t, _P]),
    "egs_entropy_score_static": (_ST, [_PS, ctypes.c_int32, ctypes.c_int32, ctypes.c_float, _P,
                                       _P, _P, _P, _P]),
    "egs_allocate_budget": (_ST, [_PS, ctypes.POINTER(BudgetPolicyC), _P, _P, _P, _P]),
    "egs_select_blocks": (_ST, [_PS, _P, _P, ctypes.c_int32, _P, _P, _P]),
    "egs_score_select": (_ST, [_PS, ctypes.c_int32, ctypes.c_int32, ctypes.c_float,
                               ctypes.POINTER(BudgetPolicyC), _P, _P, ctypes.c_int32, _P, _P, _P,
                               _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "egs_sparse_prefill_attn_workspace": (ctypes.c_size_t, [_PS]),
    "egs_sparse_prefill_attn": (_ST, [_PS, _P, _P, _P, _P, _P, ctypes.c_int32, _P, _P, _P,
                                      ctypes.c_size_t, _P]),
    "egs_kv_retain_total": (ctypes.c_int32, [_DS]),
    "egs_kv_retain_workspace": (ctypes.c_size_t, [_DS]),
    "egs_kv_retain": (_ST, [_DS, ctypes.POINTER(RetainParamsC), _P, _P, _P, _P, _P, _P, _P,
                            _P, _P, _P, ctypes.c_size_t, _P]),
    "egs_sparse_decode_attn_workspace": (ctypes.c_size_t, [_DS, ctypes.c_int32]),
    "egs_sparse_decode_attn": (_ST, [_DS, _P, _P, _P, ctypes.c_int32, _P, _P,
                                     ctypes.c_size_t, _P]),
    "egs_chunk_prune_workspace": (ctypes.c_size_t, [_DS, ctypes.c_int32]),
    "egs_chunk_prune": (_ST, [_DS, ctypes.POINTER(PruneParamsC), _P, _P, _P, ctypes.c_int32, _P,
                              _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "egs_prune_certificate_workspace": (ctypes.c_size_t, [ctypes.c_int32]),
    "egs_prune_certificate": (_ST, [_P, ctypes.c_int32, ctypes.c_int32, _P, _P, ctypes.c_double,
                                    ctypes.c_int32, ctypes.c_double, _P, _P, ctypes.c_size_t,
                                    _P]),
    "egs_latent_decode_workspace": (ctypes.c_size_t, [_DS]),
    "egs_latent_decode_step": (_ST, [_DS, ctypes.POINTER(RetainParamsC),
                                     ctypes.POINTER(LatentStateC), _P, _P, _P, _P, _P, _P, _P,
                                     _P, _P, ctypes.c_size_t, _P]),
    "egs_page_retain_capacity": (ctypes.c_int32, [_DS, ctypes.c_int32, ctypes.c_int32,
                                                  ctypes.c_int32]),
    "egs_page_retain_workspace": (ctypes.c_size_t, [_DS, ctypes.c_int32, ctypes.c_int32,
                                                    ctypes.c_int32]),
    "egs_page_retain": (_ST, [_DS, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _P, _P, _P,
                              _P, ctypes.c_size_t, _P]),
    "egs_status_string": (ctypes.c_char_p, [ctypes.c_int32]),
    "egs_last_error": (ctypes.c_char_p, []),
    "egs_abi_version": (ctypes.c_int32, []),
}


class EgsError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built: run `python -m entropy_guided_sparse_amd.build` "
            "(the HIP extension is required; there is no fallback)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if lib.egs_abi_version() != ABI_VERSION:
        raise ImportError("libegs.so ABI version mismatch")
    return lib


LIB = _load()


def check(status: int) -> None:
    if status != EGS_OK:
        msg = LIB.egs_last_error().decode()
        name = LIB.egs_status_string(status).decode()
        raise EgsError(status, f"{name}: {msg}")
