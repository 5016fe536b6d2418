"""ctypes view of libmoe.so: one Python name per C entry point, argument
types declared once.  Fails loudly when the library is missing: there is no
fallback path."""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = \
    0, -1, -2, -3, -4
MOE_F32, MOE_BF16 = 0, 1
MOE_ACT_GELU, MOE_ACT_SWIGLU = 0, 1

_P = ctypes.c_void_p
_I = ctypes.c_int
_Z = ctypes.c_size_t

# name -> (restype, argtypes), mirroring include/moe.h
SIGNATURES = {
    "moe_status_string": (ctypes.c_char_p, [_I]),
    "moe_abi_version": (_I, []),
    "moe_init": (_I, [_I]),
    "moe_set_overlap": (_I, [_I]),
    "moe_gate_topk": (_I, [_P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P]),
    "moe_permute_workspace_bytes": (_Z, [_I, _I, _I]),
    "moe_permute": (_I, [_P, _P, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _Z, _P]),
    "moe_ffn_workspace_bytes": (_Z, [_I, _I, _I, _I, _I, _I, _I]),
    "moe_expert_ffn_fwd": (_I, [_P, _P, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P,
                                _P, _P, _Z, _P]),
    "moe_expert_ffn_fwd_noalloc": (_I, [_P, _P, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P,
                                        _P, _P, _P]),
    "moe_expert_ffn_bwd": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _P,
                                _P, _P, _P, _P, _P, _P, _Z, _P]),
    "moe_expert_ffn_bwd_accumulate": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I,
                                           _P, _P, _P, _P, _P, _P, _P, _P, _Z, _P]),
    "moe_expert_ffn_fwd_gather": (_I, [_P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _P, _P,
                                       _P, _P, _P, _P, _P, _Z, _P]),
    "moe_expert_ffn_bwd_gather": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I,
                                       _I, _P, _P, _P, _P, _P, _P, _P, _P, _Z, _P]),
    "moe_combine": (_I, [_P, _P, _P, _I, _I, _I, _I, _P, _P]),
    "moe_combine_bwd": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _P, _P, _P]),
    "moe_unpermute_grad": (_I, [_P, _P, _I, _I, _I, _I, _P, _I, _P]),
    "moe_gate_bwd_workspace_bytes": (_Z, [_I, _I, _I]),
    "moe_gate_topk_bwd": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _I,
                               _P, _P, _Z, _P]),
    "moe_mfma_loop": (_I, [_I, _I, _P, _Z, _P]),
    "moe_mfma_loop_random": (_I, [_I, _I, _P, _Z, _P]),
    "moe_lds_probe": (_I, [_I, _I, _I, _P, _Z, _P, _Z, _P]),
    "moe_profile_enable": (_I, [_I]),
    "moe_profile_disable": (None, []),
    "moe_profile_reset": (None, []),
    "moe_profile_count": (_I, []),
    "moe_profile_get": (_I, [_I, ctypes.POINTER(ctypes.c_char_p),
                             ctypes.POINTER(ctypes.c_float)]),
}

_lib = None


class MoEError(RuntimeError):
    pass


def load(path: str = LIB_PATH):
    """Load libmoe.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise MoEError(
            "libmoe.so not found at %s: build it first (python -c "
            "'import __graft_entry__ as g; g.build()')" % path)
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def profile_records():
    """[(kernel name, ms)] of every launch timed since the last reset."""
    L = load()
    out = []
    name = ctypes.c_char_p()
    ms = ctypes.c_float()
    for i in range(L.moe_profile_count()):
        check(L.moe_profile_get(i, ctypes.byref(name), ctypes.byref(ms)),
              "moe_profile_get")
        out.append((name.value.decode(), float(ms.value)))
    return out


def check(status: int, what: str):
    if status != MOE_OK:
        msg = load().moe_status_string(status).decode()
        raise MoEError("%s failed: %s (%d)" % (what, msg, status))
