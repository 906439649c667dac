"""ctypes view of libtreeverify.so (the C ABI declared in include/treeverify.h)."""

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtreeverify.so")

TV_OK = 0
STATUS_NAMES = {0: "TV_OK", 1: "TV_ERR_NULL", 2: "TV_ERR_SHAPE", 3: "TV_ERR_DTYPE",
                4: "TV_ERR_UNSUPPORTED", 5: "TV_ERR_WORKSPACE", 6: "TV_ERR_HIP"}
TV_F32, TV_BF16 = 0, 1

EXPORTS = ("tv_abi_version", "tv_status_string", "tree_build", "tree_expand_workspace_size",
           "tree_expand_rerank", "tree_draft_continue", "tree_cost_lookup", "tree_budget_thresholds",
           "tree_verify_attn_workspace_size", "tree_verify_attn_plan", "tree_verify_attn",
           "tree_verify_attn_noalloc",
           "tree_accept", "tree_accept_stochastic_workspace_size", "tree_accept_stochastic",
           "tree_kv_compact",
           "tree_candidate_workspace_size", "tree_candidate_logits")

_P = ctypes.c_void_p
_I = ctypes.c_int
_S = ctypes.c_size_t
_F = ctypes.c_float

_SIGNATURES = {
    "tv_abi_version": (_I, []),
    "tv_status_string": (ctypes.c_char_p, [_I]),
    "tree_build": (_I, [_I, _I, _P, _P, _P, _P, _P, _P, _P, _P]),
    "tree_expand_workspace_size": (_S, [_I, _I, _I]),
    "tree_expand_rerank": (_I, [_P, _S, _I, _I, _I, _I, _I, _P, _I, _P, _P, _P, _I, _P, _P, _P,
                                _P, _P, _P, _P]),
    "tree_draft_continue": (_I, [_P, _S, _I, _I, _I, _I, _P, _P, _P, _P]),
    "tree_cost_lookup": (_I, [_P, _I, _P, _I, _P, _I, _P, _I, _I, _I, _P]),
    "tree_budget_thresholds": (_I, [_P, _I, _F, _P]),
    "tree_verify_attn_workspace_size": (_S, [_I, _I, _I, _I, _I, _I, _I]),
    "tree_verify_attn_plan": (_I, [_I, _I, _I, _I, _I, _I, _I, _P]),
    "tree_verify_attn": (_I, [_I, _I, _I, _I, _I, _I, _I, _F, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                              _P, _P, _S, _P, _P]),
    "tree_verify_attn_noalloc": (_I, [_I, _I, _I, _I, _I, _I, _I, _F, _P, _P, _P, _P, _P, _P, _P,
                                      _P, _P, _P, _P, _P]),
    "tree_accept": (_I, [_I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "tree_accept_stochastic_workspace_size": (_S, [_I, _I, _I]),
    "tree_accept_stochastic": (_I, [_I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                    _P, _S, _P]),
    "tree_kv_compact": (_I, [_I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, ctypes.c_int64, _P]),
    "tree_candidate_workspace_size": (_S, [_I, _I, _I]),
    "tree_candidate_logits": (_I, [_I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _S, _P]),
}

_lib = None


class TreeVerifyError(RuntimeError):
    def __init__(self, fn, code):
        self.code = code
        super().__init__(f"{fn} returned {STATUS_NAMES.get(code, code)}")


def load(path):
    """A build of the library at `path` with the C signatures set (loaded RTLD_LOCAL, so
    several builds can live in one process)."""
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing; build it with "
                          "`python -m tree_attention_verify_ancestor_amd.build`")
    handle = ctypes.CDLL(path, mode=ctypes.RTLD_LOCAL)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(handle, name)
        fn.restype = res
        fn.argtypes = args
    return handle


def lib():
    """The loaded library.  Raises when it has not been built: there is no fallback."""
    global _lib
    if _lib is None:
        _lib = load(LIB_PATH)
    return _lib


def check(fn, code):
    if code != TV_OK:
        raise TreeVerifyError(fn, code)
