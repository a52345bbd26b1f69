"""ctypes loader for libspectree.so (the C ABI in include/spec_tree.h).

Loading fails loudly: there is no fallback implementation anywhere in this
package. Build the library first with ``python -m tree_attention_verification_03_amd.build``.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libspectree.so")

c_i32, c_i64, c_u64, c_f32, c_sz, c_vp = (ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64, ctypes.c_float,
                                          ctypes.c_size_t, ctypes.c_void_p)

# name -> (restype, argtypes); mirrors include/spec_tree.h
SIGNATURES = {
    "spec_abi_version": (c_i32, []),
    "spec_last_error": (ctypes.c_char_p, []),
    "spec_tree_build_workspace_size": (c_sz, [c_i32, c_i32, c_i32]),
    "spec_tree_build_step": (c_i32, [c_vp, c_sz, c_i32, c_vp, c_i64, c_vp, c_vp, c_i32, c_i32, c_i32, c_i32, c_vp, c_vp]),
    "spec_tree_build_step_finish": (c_i32, [c_vp, c_sz, c_i32, c_vp, c_i64, c_vp, c_vp, c_i32, c_i32, c_i32, c_i32,
                                            c_vp, c_vp, c_vp, c_i32, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp]),
    "spec_tree_build_step_map": (c_i32, [c_vp, c_sz, c_i32, c_vp, c_vp, c_i64, c_vp, c_vp, c_i32, c_i32, c_i32, c_i32,
                                         c_vp, c_vp]),
    "spec_tree_build_step_finish_map": (c_i32, [c_vp, c_sz, c_i32, c_vp, c_vp, c_i64, c_vp, c_vp, c_i32, c_i32, c_i32,
                                                c_i32, c_vp, c_vp, c_vp, c_i32, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp]),
    "spec_tree_build_finish": (c_i32, [c_vp, c_sz, c_vp, c_vp, c_vp, c_vp, c_i32, c_i32, c_i32, c_i32, c_vp, c_vp,
                                       c_vp, c_vp, c_vp, c_vp]),
    "spec_tree_mask": (c_i32, [c_vp, c_vp, c_i32, c_i32, c_vp, c_vp, c_vp, c_vp]),
    "spec_tree_attention_workspace_size": (c_sz, [c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_i32]),
    "spec_tree_attention": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_i32, c_i32, c_i32, c_i32, c_i32,
                                    c_i32, c_i32, c_i32, c_f32, c_vp, c_vp, c_vp, c_vp, c_sz, c_vp]),
    "spec_tree_attention_fp8": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_i32, c_i32, c_i32,
                                        c_i32, c_i32, c_i32, c_i32, c_i32, c_f32, c_vp, c_vp, c_vp, c_vp, c_sz, c_vp]),
    "spec_tree_attention_noalloc": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_i32, c_i32, c_i32, c_i32,
                                            c_i32, c_i32, c_i32, c_i32, c_f32, c_vp, c_vp, c_vp, c_vp]),
    "spec_tree_verify_workspace_size": (c_sz, [c_i32, c_i32, c_i32]),
    "spec_tree_verify": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_u64, c_u64, c_u64, c_i32, c_i32, c_i32,
                                 c_i32, c_vp, c_vp, c_vp, c_vp, c_vp, c_sz, c_vp]),
    "spec_tree_verify_logits_workspace_size": (c_sz, [c_i32, c_i32, c_i32]),
    "spec_tree_verify_logits": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_u64, c_u64, c_u64, c_i32, c_i32,
                                        c_i32, c_i32, c_vp, c_vp, c_vp, c_vp, c_vp, c_sz, c_vp]),
    "spec_kv_compact": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_i32,
                                c_i32, c_i64, c_vp, c_vp]),
    "spec_kv_prune": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_vp, c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_vp, c_vp, c_vp,
                              c_vp, c_vp]),
}

_lib = None


def load():
    """Return the loaded library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -m tree_attention_verification_03_amd.build` "
            "(hipcc, gfx950). There is no CPU fallback.")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


class SpecError(RuntimeError):
    def __init__(self, code: int, where: str, message: str):
        super().__init__(f"{where} failed with code {code}: {message}")
        self.code = code


def check(rc: int, where: str):
    if rc != 0:
        msg = load().spec_last_error().decode(errors="replace")
        raise SpecError(rc, where, msg)
