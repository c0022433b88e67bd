"""ctypes loader for libmoe_ffn.so (the C ABI declared in include/moe_ffn.h).

The library is built in-tree by expert_ffn_dispatch_amd.build.  Loading fails
loudly if it is missing: there is no fallback implementation.
"""
import ctypes
import os

# MOE_FFN_LIB names another build of the same library (the host-sanitizer
# build, libmoe_ffn_san.so) to load instead of the in-tree one.
LIB_PATH = os.environ.get("MOE_FFN_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe_ffn.so")

MOE_OK = 0
MOE_ERR_INVALID = 1
MOE_ERR_UNSUPPORTED = 2
MOE_ERR_WORKSPACE = 3
MOE_ERR_DEVICE = 4
MOE_FLAG_IDS_IN = 1

EXPORTS = (
    "moe_abi_version", "moe_last_error", "moe_layer_workspace_bytes", "moe_route_workspace_bytes",
    "moe_permute_workspace_bytes",
    "moe_grouped_ffn_workspace_bytes", "moe_route", "moe_permute", "moe_grouped_ffn", "moe_combine",
    "moe_layer", "moe_set_stage_events", "moe_quantize_fp8", "moe_grouped_ffn_fp8", "moe_layer_fp8",
    "moe_layer_pipelined_workspace_bytes", "moe_layer_pipelined", "moe_layer_single_launch",
    "moe_layer_noalloc",
)
# bytes of the library's own workspace array (moe_layer_noalloc)
MOE_NOALLOC_SCRATCH_BYTES = 64 << 20
MOE_STAGE_EVENTS = 7


class MoeDims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "n_tokens", "hidden", "n_experts", "top_k", "expert_width", "n_shared", "shared_width")]


class MoeFp8Ffn(ctypes.Structure):
    """struct moe_fp8_ffn: device pointers of E4M3 codes and per-channel scales."""
    _fields_ = [(n, ctypes.c_void_p) for n in ("gate", "up", "down", "gate_scale", "up_scale", "down_scale")]


class MoeError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"[{code}] {msg}")
        self.code = code


_lib = None

P = ctypes.c_void_p
DIMS = ctypes.POINTER(MoeDims)


def load() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing; build it with `python -m expert_ffn_dispatch_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    lib.moe_abi_version.restype = ctypes.c_int
    lib.moe_last_error.restype = ctypes.c_char_p
    for name in ("moe_layer_workspace_bytes",):
        getattr(lib, name).argtypes = [DIMS, ctypes.c_uint32, ctypes.POINTER(ctypes.c_size_t)]
    for name in ("moe_route_workspace_bytes", "moe_permute_workspace_bytes", "moe_grouped_ffn_workspace_bytes"):
        getattr(lib, name).argtypes = [DIMS, ctypes.POINTER(ctypes.c_size_t)]
    lib.moe_route.argtypes = [DIMS, P, P, P, P, P, P, ctypes.c_size_t, P]
    lib.moe_permute.argtypes = [DIMS, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
    lib.moe_grouped_ffn.argtypes = [DIMS, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
    lib.moe_combine.argtypes = [DIMS, P, P, P, P, P, P]
    lib.moe_layer.argtypes = [DIMS, ctypes.c_uint32] + [P] * 13 + [ctypes.c_size_t, P]
    lib.moe_set_stage_events.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_int]
    F8 = ctypes.POINTER(MoeFp8Ffn)
    lib.moe_quantize_fp8.argtypes = [P, ctypes.c_int64, ctypes.c_int32, P, P, P]
    lib.moe_grouped_ffn_fp8.argtypes = [DIMS, P, P, F8, P, P, P, ctypes.c_size_t, P]
    lib.moe_layer_fp8.argtypes = [DIMS, ctypes.c_uint32, P, P, P, F8, F8, P, P, P, P, ctypes.c_size_t, P]
    lib.moe_layer_pipelined_workspace_bytes.argtypes = [DIMS, ctypes.c_uint32, ctypes.c_int32,
                                                        ctypes.POINTER(ctypes.c_size_t)]
    lib.moe_layer_pipelined.argtypes = [DIMS, ctypes.c_uint32, ctypes.c_int32] + [P] * 13 + [ctypes.c_size_t, P]
    lib.moe_layer_single_launch.argtypes = [DIMS, ctypes.c_uint32, ctypes.c_int, ctypes.POINTER(ctypes.c_int)]
    lib.moe_layer_noalloc.argtypes = [DIMS, ctypes.c_uint32] + [P] * 12 + [P]
    for name in EXPORTS[2:]:
        getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def check(code: int) -> None:
    if code != MOE_OK:
        raise MoeError(code, load().moe_last_error().decode())
