"""ctypes binding of libspear_w4ec.so (argument marshalling only).

Every computation runs in the library's HIP kernels.  PyTorch provides device
memory (tensors) and the stream (torch.cuda.current_stream()); nothing here
computes any part of the layer.  If the library is missing or fails to load,
the binding raises: there is no fallback path.
"""
import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libspear_w4ec.so")

SPEAR_OK = 0
STATUS_NAMES = {
    0: "SPEAR_OK",
    1: "SPEAR_ERR_NULL_POINTER",
    2: "SPEAR_ERR_INVALID_SHAPE",
    3: "SPEAR_ERR_UNSUPPORTED",
    4: "SPEAR_ERR_MISALIGNED",
    5: "SPEAR_ERR_WORKSPACE_TOO_SMALL",
    6: "SPEAR_ERR_INVALID_PLAN",
    7: "SPEAR_ERR_HIP",
    8: "SPEAR_ERR_INVALID_ARGUMENT",
}
VARIANTS = {"auto": 0, "fused": 1, "split": 2, "no_ec": 3}
GROUP_SIZE = 128   # SPEAR_GROUP_SIZE
VARIANT_NAMES = {v: k for k, v in VARIANTS.items()}

# Entry points declared in include/spear_w4ec.h.
EXPORTS = (
    "spear_status_str",
    "spear_abi_version",
    "spear_packed_bytes",
    "spear_pack_w4",
    "spear_pack_w4_grouped",
    "spear_dispatch_plan",
    "spear_schedule_ec",
    "spear_schedule_ec_costs",
    "spear_w4ec_linear",
    "spear_ec_workspace_bytes",
    "spear_ec_project",
    "spear_debug_unpack_w4",
    "spear_ec_init_workspace_bytes",
    "spear_ec_init",
    "spear_take_error",
    "spear_w4ec_linear_noalloc",
    "spear_debug_set_spin_limit",
    "spear_debug_fail_waits",
    "spear_debug_stream_read",
    "spear_debug_mfma_rate",
)


class LinearDesc(ctypes.Structure):
    _fields_ = [
        ("M", ctypes.c_int32), ("K", ctypes.c_int32), ("N", ctypes.c_int32), ("rank", ctypes.c_int32),
        ("gate_bias", ctypes.c_float), ("skip_tau", ctypes.c_float),
        ("variant", ctypes.c_int32), ("device_cus", ctypes.c_int32),
        ("group_size", ctypes.c_int32),
    ]


class Plan(ctypes.Structure):
    _fields_ = [
        ("abi_version", ctypes.c_uint32), ("layout_id", ctypes.c_uint32),
        ("variant", ctypes.c_int32), ("kernel", ctypes.c_int32),
        ("M", ctypes.c_int32), ("K", ctypes.c_int32), ("N", ctypes.c_int32), ("rank", ctypes.c_int32),
        ("tile_m", ctypes.c_int32), ("tile_n", ctypes.c_int32), ("split_k", ctypes.c_int32),
        ("grid", ctypes.c_int32), ("producers", ctypes.c_int32), ("ec_split", ctypes.c_int32),
        ("cus", ctypes.c_int32), ("ec_local", ctypes.c_int32),
        ("group_size", ctypes.c_int32),
        ("predicted_us", ctypes.c_float), ("predicted_no_ec_us", ctypes.c_float),
        ("workspace_bytes", ctypes.c_size_t),
    ]

    def as_dict(self):
        d = {name: getattr(self, name) for name, _ in self._fields_}
        d["variant_name"] = VARIANT_NAMES.get(self.variant, "?")
        return d


class SchedLayer(ctypes.Structure):
    _fields_ = [("K", ctypes.c_int32), ("N", ctypes.c_int32), ("rank", ctypes.c_int32),
                ("group_size", ctypes.c_int32), ("weight", ctypes.c_float)]


class SpearError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)} ({_status_str(status)})")


_lib = None


def load(path=None):
    """Load the shared library (once) and declare the entry-point signatures."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    path = path or LIB_PATH
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m w4_gemm_gated_amd.build` "
                           "(there is no fallback implementation)")
    lib = ctypes.CDLL(path)
    vp, i32, sz, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.c_float
    lib.spear_status_str.restype = ctypes.c_char_p
    lib.spear_status_str.argtypes = [ctypes.c_int]
    lib.spear_abi_version.restype = ctypes.c_uint32
    lib.spear_abi_version.argtypes = []
    lib.spear_packed_bytes.restype = ctypes.c_int
    lib.spear_packed_bytes.argtypes = [i32, i32, ctypes.POINTER(sz)]
    lib.spear_pack_w4.restype = ctypes.c_int
    lib.spear_pack_w4.argtypes = [vp, i32, i32, vp, vp, vp]
    lib.spear_pack_w4_grouped.restype = ctypes.c_int
    lib.spear_pack_w4_grouped.argtypes = [vp, i32, i32, i32, vp, vp, vp]
    lib.spear_dispatch_plan.restype = ctypes.c_int
    lib.spear_dispatch_plan.argtypes = [ctypes.POINTER(LinearDesc), ctypes.POINTER(Plan)]
    lib.spear_schedule_ec.restype = ctypes.c_int
    lib.spear_schedule_ec.argtypes = [ctypes.POINTER(SchedLayer), i32, i32, ctypes.c_double, i32,
                                      ctypes.POINTER(ctypes.c_uint8), ctypes.POINTER(ctypes.c_double)]
    lib.spear_schedule_ec_costs.restype = ctypes.c_int
    lib.spear_schedule_ec_costs.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_float), i32,
                                            ctypes.c_double, ctypes.POINTER(ctypes.c_uint8),
                                            ctypes.POINTER(ctypes.c_double)]
    lib.spear_w4ec_linear.restype = ctypes.c_int
    lib.spear_w4ec_linear.argtypes = [ctypes.POINTER(LinearDesc), ctypes.POINTER(Plan),
                                      vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.spear_ec_workspace_bytes.restype = ctypes.c_int
    lib.spear_ec_workspace_bytes.argtypes = [i32, i32, i32, ctypes.POINTER(sz)]
    lib.spear_ec_project.restype = ctypes.c_int
    lib.spear_ec_project.argtypes = [i32, i32, i32, vp, vp, vp, f32, f32, vp, vp, vp, sz, vp]
    lib.spear_debug_unpack_w4.restype = ctypes.c_int
    lib.spear_debug_unpack_w4.argtypes = [vp, i32, i32, vp, vp]
    lib.spear_w4ec_linear_noalloc.restype = ctypes.c_int
    lib.spear_w4ec_linear_noalloc.argtypes = [ctypes.POINTER(LinearDesc), ctypes.POINTER(Plan),
                                              vp, vp, vp, vp, vp, vp, vp, vp]
    lib.spear_ec_init_workspace_bytes.restype = ctypes.c_int
    lib.spear_ec_init_workspace_bytes.argtypes = [i32, i32, i32, ctypes.POINTER(sz)]
    lib.spear_ec_init.restype = ctypes.c_int
    lib.spear_ec_init.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, vp, vp, vp, sz, vp]
    lib.spear_take_error.restype = ctypes.c_int
    lib.spear_take_error.argtypes = [vp, sz, vp, vp]
    lib.spear_debug_set_spin_limit.restype = None
    lib.spear_debug_set_spin_limit.argtypes = [ctypes.c_int64]
    lib.spear_debug_fail_waits.restype = None
    lib.spear_debug_fail_waits.argtypes = [ctypes.c_int32]
    lib.spear_debug_stream_read.restype = ctypes.c_int
    lib.spear_debug_stream_read.argtypes = [vp, sz, i32, vp, vp]
    lib.spear_debug_mfma_rate.restype = ctypes.c_int
    lib.spear_debug_mfma_rate.argtypes = [i32, i32, i32, vp, vp, ctypes.POINTER(ctypes.c_double)]
    if path == LIB_PATH:
        _lib = lib
    return lib


def _status_str(status):
    try:
        return load().spear_status_str(int(status)).decode()
    except Exception:  # noqa: BLE001 - only used to decorate an error message
        return "?"


def check(status, where):
    if status != SPEAR_OK:
        raise SpearError(status, where)
