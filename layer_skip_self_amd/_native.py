"""ctypes declarations of the C ABI in include/lss.h (argument marshalling only)."""
import ctypes as C
import os

_LIB_PATH = os.environ.get("LSS_LIB_PATH") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                             "liblss.so")

LSS_OK, LSS_EINVAL, LSS_ESTATE, LSS_ECAPACITY, LSS_EHIP, LSS_ENOTIMPL = 0, -1, -2, -3, -4, -5
LSS_F32, LSS_BF16 = 0, 1
LSS_MODE_AR, LSS_MODE_STATIC, LSS_MODE_DP, LSS_MODE_CASCADE = 0, 1, 2, 3
LSS_WINDOW_MAX = 31
LSS_TREE_NODES_MAX = 15
LSS_ROWS_MAX = 64
LSS_SEQS_MAX = 64
LSS_BATCH_PASS_SEQS = 16
LSS_LEVELS_MAX = 4
LSS_STOP_MAX = 8
LSS_ACCEPT_ROWS_MAX = 64
LSS_ACCEPT_VOCAB_MAX = 262144

STATUS_NAMES = {0: "LSS_OK", -1: "LSS_EINVAL", -2: "LSS_ESTATE", -3: "LSS_ECAPACITY",
                -4: "LSS_EHIP", -5: "LSS_ENOTIMPL"}


class lss_config(C.Structure):
    _fields_ = [("n_layers", C.c_int32), ("d_model", C.c_int32), ("n_heads", C.c_int32),
                ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32), ("ffn_dim", C.c_int32),
                ("vocab", C.c_int32), ("rope_theta", C.c_float), ("rms_eps", C.c_float),
                ("dtype", C.c_int32), ("max_seq", C.c_int32), ("max_rows", C.c_int32),
                ("kv_dtype", C.c_int32), ("max_seqs", C.c_int32)]


class lss_tensor(C.Structure):
    _fields_ = [("name", C.c_char_p), ("dev_ptr", C.c_void_p), ("numel", C.c_int64)]


class lss_policy(C.Structure):
    _fields_ = [("mode", C.c_int32), ("k_max", C.c_int32), ("exit_tau", C.c_float),
                ("quant", C.c_int32), ("static_mask", C.POINTER(C.c_uint8)),
                ("n_skip", C.c_int32), ("interval", C.c_int32), ("n_levels", C.c_int32),
                ("level_skip", C.c_int32 * LSS_LEVELS_MAX), ("level_exit", C.c_int32 * LSS_LEVELS_MAX),
                ("level_quant", C.c_int32 * LSS_LEVELS_MAX), ("beta", C.c_double * 3),
                ("tree_width", C.c_int32), ("tree_depth", C.c_int32),
                ("row_cost", C.c_double * (LSS_TREE_NODES_MAX + 1)),
                ("n_stop", C.c_int32), ("stop_tokens", C.c_int32 * LSS_STOP_MAX)]


class lss_stats(C.Structure):
    _fields_ = [("rounds", C.c_int32), ("drafted", C.c_int32), ("accepted", C.c_int32),
                ("dp_runs", C.c_int32), ("emitted", C.c_int32)]


# name -> (restype, argtypes); every symbol include/lss.h declares
SIGNATURES = {
    "lss_workspace_bytes": (C.c_size_t, [C.POINTER(lss_config)]),
    "lss_load_weights": (C.c_int, [C.POINTER(lss_config), C.POINTER(lss_tensor), C.c_int32, C.c_void_p,
                                   C.c_size_t, C.c_void_p, C.POINTER(C.c_void_p)]),
    "lss_create": (C.c_int, [C.POINTER(lss_config), C.POINTER(C.c_void_p), C.c_int32, C.c_void_p,
                             C.c_size_t, C.c_void_p, C.POINTER(C.c_void_p)]),
    "lss_destroy": (None, [C.c_void_p]),
    "lss_last_error": (C.c_char_p, [C.c_void_p]),
    "lss_prefill": (C.c_int, [C.c_void_p, C.POINTER(C.c_int32), C.c_int32, C.POINTER(C.c_int32)]),
    "lss_seq_select": (C.c_int, [C.c_void_p, C.c_int32]),
    "lss_batch_draft": (C.c_int, [C.c_void_p, C.c_int32, C.POINTER(C.c_int32), C.POINTER(C.c_uint8), C.c_int32,
                                  C.POINTER(C.c_int32), C.c_float, C.POINTER(C.c_int32), C.POINTER(C.c_int32)]),
    "lss_batch_verify": (C.c_int, [C.c_void_p, C.c_int32, C.POINTER(C.c_int32)]),
    "lss_batch_accept": (C.c_int, [C.c_void_p, C.c_int32, C.POINTER(C.c_int32), C.POINTER(C.c_int32),
                                   C.POINTER(C.c_int32), C.POINTER(C.c_int32)]),
    "lss_generate_batch": (C.c_int, [C.c_void_p, C.c_int32, C.POINTER(C.c_int32), C.POINTER(C.c_int32), C.c_int32,
                                     C.POINTER(lss_policy), C.POINTER(C.c_int32), C.POINTER(lss_stats)]),
    "lss_draft": (C.c_int, [C.c_void_p, C.POINTER(C.c_uint8), C.c_int32, C.c_int32, C.c_float,
                            C.POINTER(C.c_int32), C.POINTER(C.c_int32)]),
    "lss_draft_tree": (C.c_int, [C.c_void_p, C.POINTER(C.c_uint8), C.c_int32, C.c_int32, C.c_int32,
                                 C.POINTER(C.c_int32)]),
    "lss_draft_tree_levels": (C.c_int, [C.c_void_p, C.POINTER(C.c_uint8), C.POINTER(C.c_int32), C.c_int32,
                                        C.c_int32, C.POINTER(C.c_int32)]),
    "lss_verify": (C.c_int, [C.c_void_p, C.POINTER(C.c_int32), C.c_int32]),
    "lss_accept_and_rollback": (C.c_int, [C.c_void_p, C.POINTER(C.c_int32), C.POINTER(C.c_int32),
                                          C.POINTER(C.c_int32)]),
    "lss_select_layers_dp": (C.c_int, [C.c_void_p, C.c_int32, C.POINTER(C.c_uint8), C.POINTER(C.c_float)]),
    "lss_select_layers_dp_exit": (C.c_int, [C.c_void_p, C.c_int32, C.c_int32, C.POINTER(C.c_uint8),
                                            C.POINTER(C.c_float)]),
    "lss_seq_len": (C.c_int32, [C.c_void_p]),
    "lss_set_sampling": (C.c_int, [C.c_void_p, C.c_float, C.c_uint64]),
    "lss_set_gemv_grid": (C.c_int, [C.c_void_p, C.c_int32]),
    "lss_set_decode_kernel": (C.c_int, [C.c_void_p, C.c_int32]),
    "lss_read_logits": (C.c_int, [C.c_void_p, C.c_int32, C.POINTER(C.c_float)]),
    "lss_read_states": (C.c_int, [C.c_void_p, C.c_int32, C.POINTER(C.c_float)]),
    "lss_read_dp_decisions": (C.c_int, [C.c_void_p, C.POINTER(C.c_float)]),
    "lss_generate": (C.c_int, [C.c_void_p, C.POINTER(C.c_int32), C.c_int32, C.c_int32,
                               C.POINTER(lss_policy), C.POINTER(C.c_int32), C.POINTER(lss_stats)]),
    "lss_router_plan": (C.c_int, [C.POINTER(C.c_double), C.POINTER(C.c_double), C.c_int32, C.c_double,
                                  C.c_int32, C.POINTER(C.c_int32)]),
    "lss_router_update": (C.c_int, [C.POINTER(C.c_double), C.c_int32, C.POINTER(C.c_int32), C.c_int32,
                                    C.c_int32]),
    "lss_router_plan_tree": (C.c_int, [C.POINTER(C.c_double), C.POINTER(C.c_double), C.c_int32, C.c_double,
                                       C.POINTER(C.c_double), C.c_int32, C.c_int32, C.c_int32,
                                       C.POINTER(C.c_int32), C.POINTER(C.c_int32)]),
    "lss_router_update_tree": (C.c_int, [C.POINTER(C.c_double), C.c_int32, C.POINTER(C.c_int32), C.c_int32,
                                         C.c_int32, C.c_int32]),
    "lss_latency_fit": (C.c_int, [C.POINTER(C.c_double), C.c_int32, C.POINTER(C.c_double)]),
    "lss_profile_kernel": (C.c_int, [C.c_void_p, C.c_int32, C.c_int32, C.c_int32]),
    "lss_profile_read": (C.c_int, [C.c_void_p, C.POINTER(C.c_double), C.POINTER(C.c_int64),
                                   C.POINTER(C.c_int64)]),
    "lss_op_accept_greedy_workspace_bytes": (C.c_size_t, [C.c_int32, C.c_int32]),
    "lss_op_accept_greedy": (C.c_int, [C.c_void_p, C.c_int32, C.c_int32, C.c_void_p, C.c_void_p, C.c_void_p,
                                       C.c_size_t, C.c_void_p]),
    "lss_op_accept_greedy_noalloc": (C.c_int, [C.c_void_p, C.c_int32, C.c_int32, C.c_void_p, C.c_void_p,
                                               C.c_void_p]),
    "lss_op_quantize_rows": (C.c_int, [C.c_void_p, C.c_int32, C.c_int32, C.c_void_p, C.c_void_p,
                                       C.c_void_p]),
    "lss_w8_bytes": (C.c_size_t, [C.POINTER(lss_config)]),
    "lss_attach_w8": (C.c_int, [C.c_void_p, C.c_void_p, C.c_size_t]),
    "lss_op_w8_quantize": (C.c_int, [C.c_void_p, C.c_int32, C.c_int32, C.c_int32, C.c_void_p, C.c_void_p,
                                     C.c_void_p]),
    "lss_op_w8a8_gemv": (C.c_int, [C.c_void_p, C.c_void_p, C.c_int32, C.c_int32, C.c_void_p, C.c_void_p,
                                   C.c_void_p, C.c_void_p]),
    "lss_op_w8a8_gemv_f32": (C.c_int, [C.c_void_p, C.c_void_p, C.c_int32, C.c_int32, C.c_void_p, C.c_void_p,
                                       C.c_void_p]),
}

_lib = None


def lib_path():
    return _LIB_PATH


def load():
    """Load liblss.so; raises if it has not been built (no fallback exists)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is not built; run __graft_entry__.build() "
                           "(python -m layer_skip_self_amd.build)")
    lib = C.CDLL(_LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib
