"""ctypes view of libcpa.so: loads the in-tree library and declares every exported symbol."""
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcpa.so")

EXPORTS = ("cpa_append_kv", "cpa_build_block_plans", "cpa_build_block_tables", "cpa_build_block_tables_bits",
           "cpa_chunked_prefill", "cpa_chunked_prefill_direct", "cpa_chunked_prefill_fp8kv", "cpa_chunked_prefill_fused",
           "cpa_chunked_prefill_fused_bits",
           "cpa_chunked_prefill_split", "cpa_chunked_prefill_split_static", "cpa_chunked_prefill_vt",
           "cpa_split_workspace_bytes", "cpa_status_string", "cpa_version")

_lib = None


def load():
    """Load libcpa.so once; raises if it has not been built (there is no fallback path)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m sparse_attention_long_reduce_amd.build` first")
    lib = ctypes.CDLL(LIB_PATH)
    c = ctypes
    vp, i32, i64, f32 = c.c_void_p, c.c_int, c.c_int64, c.c_float
    lib.cpa_build_block_tables.restype = i32
    lib.cpa_build_block_tables.argtypes = [vp, i32, i32, i32, i32, i32, vp, vp, vp, i32, vp, vp]
    lib.cpa_build_block_tables_bits.restype = i32
    lib.cpa_build_block_tables_bits.argtypes = [vp, i32, i32, i32, i32, i32, i32, vp, vp, vp, i32, vp, vp]
    lib.cpa_build_block_plans.restype = i32
    lib.cpa_build_block_plans.argtypes = [vp, i32, i32, i32, i32, vp, vp, vp, i32, vp, vp]
    lib.cpa_chunked_prefill_direct.restype = i32
    lib.cpa_chunked_prefill_direct.argtypes = [vp, i32, vp, i64, i64, i64, vp, i64, i64, i64, i64, vp, i32, vp, i32,
                                               vp, i32, vp, vp, i32, i32, i32, i32, i32, f32, vp, vp, vp]
    lib.cpa_chunked_prefill_fp8kv.restype = i32
    lib.cpa_chunked_prefill_fp8kv.argtypes = [vp, vp, vp, i64, i64, i64, i32, i64, i64, i64, f32, f32, i64, vp, i32,
                                              vp, i32, vp, vp, vp, i32, i32, i32, i32, i32, f32, vp, vp, i32, i32, vp,
                                              c.c_size_t, vp]
    lib.cpa_chunked_prefill_fused.restype = i32
    lib.cpa_chunked_prefill_fused.argtypes = [vp, i32, vp, i64, i64, i64, vp, i32, i64, i64, i64, i32, f32, f32, i64, vp,
                                              i32, vp,
                                              i32, i32, vp, vp, i32, i32, i32, i32, i32, f32, vp, vp, i32, i32,
                                              vp, c.c_size_t, vp]
    lib.cpa_chunked_prefill_fused_bits.restype = i32
    lib.cpa_chunked_prefill_fused_bits.argtypes = [vp, i32, vp, i64, i64, i64, vp, i32, i64, i64, i64, i32, f32, f32,
                                                   i64, vp, i32,
                                                   vp, i32, i32, i32, vp, vp, i32, i32, i32, i32, i32, f32, vp, vp,
                                                   i32, i32, vp, c.c_size_t, vp]
    lib.cpa_chunked_prefill.restype = i32
    lib.cpa_chunked_prefill.argtypes = [vp, i32, vp, vp, i64, i64, i64, i64, vp, i32, vp, i32, vp,
                                        vp, vp, i32, i32, i32, i32, i32, f32, vp, vp, vp]
    lib.cpa_chunked_prefill_split.restype = i32
    lib.cpa_chunked_prefill_split.argtypes = [vp, i32, vp, vp, i64, i64, i64, i64, vp, i32, vp, i32, vp,
                                              vp, vp, i32, i32, i32, i32, i32, f32, vp, vp, i32, i32,
                                              vp, c.c_size_t, vp]
    lib.cpa_chunked_prefill_split_static.restype = i32
    lib.cpa_chunked_prefill_split_static.argtypes = [vp, i32, vp, vp, i64, i64, i64, i64, vp, i32, vp, i32, vp,
                                                     vp, vp, i32, i32, i32, i32, i32, f32, vp, vp, i32, i32, vp]
    lib.cpa_chunked_prefill_vt.restype = i32
    lib.cpa_chunked_prefill_vt.argtypes = [vp, i32, vp, i64, i64, i64, vp, i64, i64, i64, i64, vp, i32, vp, i32,
                                           vp, vp, vp, i32, i32, i32, i32, i32, f32, vp, vp, i32, i32, vp,
                                           c.c_size_t, vp]
    lib.cpa_append_kv.restype = i32
    lib.cpa_append_kv.argtypes = [vp, vp, i32, vp, i64, i64, i64, vp, i32, i64, i64, i64, i64, vp, i32, vp, vp,
                                  i32, i32, i32, i32, vp]
    lib.cpa_split_workspace_bytes.restype = c.c_size_t
    lib.cpa_split_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
    lib.cpa_status_string.restype = c.c_char_p
    lib.cpa_status_string.argtypes = [i32]
    lib.cpa_version.restype = i32
    lib.cpa_version.argtypes = []
    _lib = lib
    return lib


DIAG_LIB_PATH = os.path.join(_HERE, "libcpa_diag.so")
DIAG_EXPORTS = ("cpa_diag_clock_rates", "cpa_diag_mfma_loop")
_diag = None


def load_diag():
    """Load libcpa_diag.so (the measurement helpers of include/cpa_diag.h) once."""
    global _diag
    if _diag is not None:
        return _diag
    if not os.path.exists(DIAG_LIB_PATH):
        raise RuntimeError(f"{DIAG_LIB_PATH} is missing: build it with "
                           "`python -m sparse_attention_long_reduce_amd.build` first")
    lib = ctypes.CDLL(DIAG_LIB_PATH)
    c = ctypes
    lib.cpa_diag_mfma_loop.restype = c.c_int
    lib.cpa_diag_mfma_loop.argtypes = [c.c_int, c.c_int, c.c_int, c.c_void_p, c.c_void_p, c.c_void_p]
    lib.cpa_diag_clock_rates.restype = c.c_int
    lib.cpa_diag_clock_rates.argtypes = [c.c_int, c.POINTER(c.c_int), c.POINTER(c.c_int)]
    _diag = lib
    return lib


class CpaError(RuntimeError):
    def __init__(self, status: int, where: str):
        msg = load().cpa_status_string(status).decode()
        super().__init__(f"{where}: status {status} ({msg})")
        self.status = status
