"""ctypes view of include/dllm.h (argument marshalling only)."""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, Structure, c_float, c_int32, c_size_t, c_void_p

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdllm.so")
CHECK_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdllm_check.so")

DLLM_F32, DLLM_BF16 = 0, 1
VAR_L1N, VAR_COS, VAR_L2REL, VAR_KL, VAR_NONE = 0, 1, 2, 3, 4
SEL_TOPK, SEL_THRESH_CAP, SEL_UNLOCKED = 0, 1, 2
FORCE_NONE, FORCE_ON, FORCE_EXCLUDED = 0, 1, 2
UNMASK_CONF, UNMASK_FORCED = 0, 1
MAX_NESTED = 3
NOALLOC_SCRATCH_BYTES = 64 << 20   # DLLM_NOALLOC_SCRATCH_BYTES

EXPORTED = (
    "dllm_workspace_size", "dllm_score_select", "dllm_gather_rows", "dllm_scatter_rows",
    "dllm_layer_sparse", "dllm_confidence_kl", "dllm_skip_step", "dllm_status_string", "dllm_version",
    "dllm_dus_mark", "dllm_pack_weight", "dllm_layer_sparse_noalloc", "dllm_check_word", "dllm_peak_probe",
    "dllm_packed_plan",
)
TK_NONE, TK_QKV, TK_ATTN, TK_O, TK_FFN_UP, TK_FFN_DOWN, TK_LM_HEAD, TK_VOCAB, TK_SCORE, TK_SELECT = range(10)


class Dims(Structure):
    _fields_ = [(n, c_int32) for n in ("B", "S", "d", "n_heads", "n_kv_heads", "head_dim", "d_ff", "vocab", "n_layers")]


class LayerW(Structure):
    _fields_ = [(n, c_void_p) for n in ("attn_norm", "w_qkv", "w_o", "ffn_norm", "w_gate_up", "w_down",
                                        "w_gate_up_packed", "w_down_packed", "w_qkv_packed")]


class ModelC(Structure):
    _fields_ = [("dims", Dims), ("dtype", c_int32), ("rope_base", c_float), ("rms_eps", c_float),
                ("mask_id", c_int32), ("embed", c_void_p), ("layers", POINTER(LayerW)),
                ("final_norm", c_void_p), ("lm_head", c_void_p), ("lm_head_packed", c_void_p)]


class ScoreCfg(Structure):
    _fields_ = [("alpha", c_float), ("conf_inverted", c_int32), ("var", c_int32), ("sel", c_int32),
                ("k", c_int32), ("tau", c_float)]


class StateC(Structure):
    _fields_ = [("tokens", c_void_p), ("k_cache", POINTER(c_void_p)), ("v_cache", POINTER(c_void_p)),
                ("h_bnd", c_void_p * 2), ("bnd_cur", c_int32), ("h_fin", c_void_p), ("conf", c_void_p),
                ("kl", c_void_p), ("argmax", c_void_p), ("logits_prev", c_void_p), ("force", c_void_p),
                ("idx", c_void_p), ("n_active", c_void_p), ("k_max", c_int32), ("have_prev", c_int32),
                ("logits_prev_dtype", c_int32), ("h_nested", c_void_p * MAX_NESTED),
                ("x_in_cache", POINTER(c_void_p)), ("x_out_cache", POINTER(c_void_p))]


class Timing(Structure):
    _fields_ = [("kernel", c_int32), ("max_rows", c_int32), ("capacity", c_int32), ("count", c_int32),
                ("start", POINTER(c_void_p)), ("stop", POINTER(c_void_p))]


class StepCfg(Structure):
    _fields_ = [("boundary_layer", c_int32), ("full_step", c_int32), ("score", ScoreCfg),
                ("lock_kl_eps", c_float), ("lock_conf_min", c_float), ("unmask_n", c_int32),
                ("block_lo", c_int32), ("block_hi", c_int32), ("unmask_mode", c_int32), ("ws", c_void_p),
                ("ws_bytes", c_size_t), ("n_nested", c_int32), ("nested_layer", c_int32 * MAX_NESTED),
                ("nested_k", c_int32 * MAX_NESTED), ("layer_cache", c_int32), ("timing", POINTER(Timing))]


_LIB = None
_CHECK_LIB = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libdllm.so; raises if it has not been built (there is no fallback path)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    _LIB = _open(path)
    return _LIB


def load_check() -> ctypes.CDLL:
    """Load the checking build libdllm_check.so (device-side precondition checks, for debugging)."""
    global _CHECK_LIB
    if _CHECK_LIB is None:
        _CHECK_LIB = _open(CHECK_LIB_PATH)
    return _CHECK_LIB


def _open(path: str) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with token_skipping_denoise_amd.build.build()")
    lib = ctypes.CDLL(path)
    lib.dllm_workspace_size.restype = c_size_t
    lib.dllm_workspace_size.argtypes = [POINTER(Dims), c_int32, c_int32]
    lib.dllm_score_select.restype = c_int32
    lib.dllm_score_select.argtypes = [c_void_p, c_void_p, c_void_p, c_int32, c_void_p, c_void_p, c_void_p,
                                      c_int32, c_int32, c_int32, POINTER(ScoreCfg), c_void_p, c_void_p, c_void_p,
                                      c_int32, c_void_p]
    lib.dllm_gather_rows.restype = c_int32
    lib.dllm_gather_rows.argtypes = [c_void_p, c_void_p, c_void_p, c_int32, c_int32, c_int32, c_int32, c_int32,
                                     c_void_p, c_void_p]
    lib.dllm_scatter_rows.restype = c_int32
    lib.dllm_scatter_rows.argtypes = list(lib.dllm_gather_rows.argtypes)
    lib.dllm_layer_sparse.restype = c_int32
    lib.dllm_layer_sparse.argtypes = [POINTER(ModelC), c_int32, c_void_p, c_void_p, c_void_p, c_int32, c_void_p,
                                      c_void_p, c_void_p, c_size_t, c_void_p]
    lib.dllm_layer_sparse_noalloc.restype = c_int32
    lib.dllm_layer_sparse_noalloc.argtypes = [POINTER(ModelC), c_int32, c_void_p, c_void_p, c_void_p, c_int32,
                                              c_void_p, c_void_p, c_void_p]
    lib.dllm_confidence_kl.restype = c_int32
    lib.dllm_confidence_kl.argtypes = [c_void_p, c_void_p, c_int32, c_void_p, c_int32, c_int32, c_int32, c_int32,
                                       c_void_p, c_void_p, c_void_p, c_void_p]
    lib.dllm_pack_weight.restype = c_int32
    lib.dllm_pack_weight.argtypes = [c_void_p, c_void_p, c_int32, c_int32, c_int32, c_void_p]
    lib.dllm_dus_mark.restype = c_int32
    lib.dllm_dus_mark.argtypes = [c_void_p, c_int32, c_int32, c_int32, c_int32, c_int32, c_int32, c_int32, c_int32,
                                  c_void_p]
    lib.dllm_skip_step.restype = c_int32
    lib.dllm_skip_step.argtypes = [POINTER(ModelC), POINTER(StateC), POINTER(StepCfg), c_void_p]
    lib.dllm_status_string.restype = ctypes.c_char_p
    lib.dllm_status_string.argtypes = [c_int32]
    lib.dllm_version.restype = c_int32
    lib.dllm_version.argtypes = []
    lib.dllm_packed_plan.restype = c_int32
    lib.dllm_packed_plan.argtypes = [c_int32, c_int32, c_int32, c_int32, POINTER(c_int32), POINTER(c_int32)]
    lib.dllm_peak_probe.restype = c_int32
    lib.dllm_peak_probe.argtypes = [c_int32, c_void_p, c_size_t, c_int32, POINTER(ctypes.c_double), c_void_p]
    lib.dllm_check_word.restype = c_int32
    lib.dllm_check_word.argtypes = [POINTER(ctypes.c_uint32), c_int32]
    return lib
