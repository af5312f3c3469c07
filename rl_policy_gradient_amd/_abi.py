"""ctypes mirror of include/plp.h and the raw library handle.

Argument marshalling only: every computation happens in libplp.so.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libplp.so")

PLP_OK = 0
PLP_E_INVALID = -1
PLP_E_UNSUPPORTED = -2
PLP_E_WORKSPACE = -3
PLP_E_HIP = -4

DTYPE_F32, DTYPE_BF16 = 0, 1
LOSS_GMPO, LOSS_GSPO_TOKEN, LOSS_GRPO, LOSS_BNPO, LOSS_DAPO = 0, 1, 2, 3, 4
ABI_VERSION = 5
IS_TOKEN, IS_SEQUENCE = 0, 1
REDUCE_SEQ_MEAN, REDUCE_TOKEN_SUM = 0, 1

METRIC_NAMES = (
    "clip_fraction",
    "seq_log_ratio_mean",
    "clipped_seq_fraction",
    "mean_kl",
    "entropy_threshold",
    "entropy_kept_fraction",
    "active_tokens",
    "clipped_tokens",
)
NUM_METRICS = len(METRIC_NAMES)

_vp = ctypes.c_void_p


class PlpArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("dtype", ctypes.c_int32),
        ("B", ctypes.c_int64),
        ("T", ctypes.c_int64),
        ("H", ctypes.c_int32),
        ("V", ctypes.c_int32),
        ("hidden", _vp),
        ("weight", _vp),
        ("bias", _vp),
        ("targets", _vp),
        ("old_logp", _vp),
        ("ref_logp", _vp),
        ("completion_mask", _vp),
        ("ratio_mask", _vp),
        ("advantages", _vp),
        ("loss_type", ctypes.c_int32),
        ("is_level", ctypes.c_int32),
        ("reduction", ctypes.c_int32),
        ("pad0", ctypes.c_int32),
        ("epsilon_low", ctypes.c_double),
        ("epsilon_high", ctypes.c_double),
        ("beta", ctypes.c_double),
        ("temperature", ctypes.c_double),
        ("top_entropy_quantile", ctypes.c_double),
        ("chunk_sequences", ctypes.c_int64),
        ("global_tokens", ctypes.c_int64),
        ("token_advantages", _vp),
        ("kl_bias_correction", ctypes.c_int32),
        ("pad1", ctypes.c_int32),
        ("weight_prepared", _vp),
    ]


class PlpOutputs(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("pad0", ctypes.c_uint32),
        ("loss", _vp),
        ("metrics", _vp),
        ("grad_hidden", _vp),
        ("grad_weight", _vp),
        ("grad_bias", _vp),
        ("logp_out", _vp),
        ("entropy_out", _vp),
        ("entropy_mask_out", _vp),
        ("dlogp_out", _vp),
    ]


class PlpError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"plp error {code}: {msg}")
        self.code = code


_lib = None


def lib() -> ctypes.CDLL:
    """Load libplp.so once. Raises ImportError when it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m rl_policy_gradient_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    sz = ctypes.c_size_t
    P = ctypes.POINTER
    L.plp_abi_version.restype = ctypes.c_int
    L.plp_last_error.restype = ctypes.c_char_p
    L.plp_workspace_size.argtypes = [P(PlpArgs), P(sz)]
    L.plp_fused_lmhead_policy_loss_fwd_bwd.argtypes = [P(PlpArgs), P(PlpOutputs), _vp, sz, _vp]
    L.plp_selective_entropy_workspace_size.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                                       ctypes.c_int32, P(sz)]
    L.plp_selective_entropy.argtypes = [_vp, _vp, _vp, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                        ctypes.c_int32, ctypes.c_float, _vp, _vp, _vp, _vp, sz, _vp]
    L.plp_selective_entropy_prepared_workspace_size.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                                                ctypes.c_int32, P(sz)]
    L.plp_selective_entropy_prepared.argtypes = [_vp, _vp, _vp, _vp, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                                 ctypes.c_int32, ctypes.c_float, _vp, _vp, _vp, _vp, sz, _vp]
    L.plp_entropy_quantile_mask_workspace_size.argtypes = [ctypes.c_int64, P(sz)]
    L.plp_entropy_quantile_mask.argtypes = [_vp, _vp, ctypes.c_int64, ctypes.c_double, _vp, _vp, _vp, sz, _vp]
    L.plp_entropy_quantile_mask_noalloc.argtypes = [_vp, _vp, ctypes.c_int64, ctypes.c_double, _vp, _vp, _vp]
    L.plp_policy_loss_workspace_size.argtypes = [P(PlpArgs), P(sz)]
    L.plp_policy_loss_from_logprobs.argtypes = [P(PlpArgs), _vp, _vp, P(PlpOutputs), _vp, sz, _vp]
    L.plp_prepared_weight_size.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, P(sz)]
    L.plp_prepare_weight.argtypes = [_vp, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _vp, sz, _vp]
    L.plp_profile_start.argtypes = [ctypes.c_int32]
    L.plp_profile_stop.argtypes = [P(ctypes.c_double), P(ctypes.c_int32)]
    L.plp_profile_stop_n.argtypes = [P(ctypes.c_double), P(ctypes.c_int32), ctypes.c_int32]
    L.plp_profile_stop_n.restype = ctypes.c_int
    L.plp_profile_start.restype = ctypes.c_int
    L.plp_profile_stop.restype = ctypes.c_int
    for name in ("plp_workspace_size", "plp_fused_lmhead_policy_loss_fwd_bwd", "plp_selective_entropy_workspace_size",
                 "plp_selective_entropy", "plp_selective_entropy_prepared_workspace_size",
                 "plp_selective_entropy_prepared", "plp_entropy_quantile_mask_workspace_size", "plp_entropy_quantile_mask",
                 "plp_entropy_quantile_mask_noalloc", "plp_prepared_weight_size", "plp_prepare_weight",
                 "plp_policy_loss_workspace_size", "plp_policy_loss_from_logprobs"):
        getattr(L, name).restype = ctypes.c_int
    if L.plp_abi_version() != ABI_VERSION:
        raise ImportError(f"{LIB_PATH} has ABI version {L.plp_abi_version()}, this binding {ABI_VERSION}: "
                          "rebuild it with `python -m rl_policy_gradient_amd.build`")
    _lib = L
    return L


def check(rc: int) -> None:
    if rc != PLP_OK:
        raise PlpError(rc, lib().plp_last_error().decode(errors="replace"))


def new_args() -> PlpArgs:
    a = PlpArgs()
    a.struct_size = ctypes.sizeof(PlpArgs)
    a.temperature = 1.0
    a.top_entropy_quantile = 1.0
    return a


def new_outputs() -> PlpOutputs:
    o = PlpOutputs()
    o.struct_size = ctypes.sizeof(PlpOutputs)
    return o
