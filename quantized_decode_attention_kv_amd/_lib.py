"""ctypes view of include/kvq.h.  Loading fails loudly if libkvq.so was not built."""

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# KVQ_LIBRARY names another build of the same sources (the host sanitizer test
# loads a host-only build through it); by default the in-tree libkvq.so
LIB_PATH = os.environ.get("KVQ_LIBRARY") or os.path.join(HERE, "libkvq.so")

KVQ_OK, KVQ_ERR_INVALID, KVQ_ERR_UNSUPPORTED, KVQ_ERR_HIP = 0, 1, 2, 3
KVQ_F32, KVQ_F16, KVQ_BF16 = 0, 1, 2
KVQ_GROUP = 32
KVQ_NUM_CACHE_BUFFERS = 8
KVQ_STREAM_MAX_ROWS = 4096

LAYOUT_FIELDS = ["B", "Hq", "Hkv", "Dk", "Dv", "T", "k_bits", "v_bits", "n_recent", "log_window", "k_group", "v_group",
                 "R", "Tq", "n_groups", "flags"]
CACHE_FIELDS = ["k_codes", "k_scale", "k_zero", "v_codes", "v_scale", "v_zero", "k_fp16", "v_fp16"]

# every entry point declared in include/kvq.h
EXPORTS = ["kvq_layout_init", "kvq_cache_sizes", "kvq_retained_positions", "kvq_quantized_before",
           "kvq_decode_workspace_bytes", "kv_quant_pack", "kv_decode_attn", "kv_decode_attn_ex", "kvq_status_string",
           "kvq_last_error", "kvq_read_probe", "kvq_layout_init_ex", "kvq_stream_init", "kvq_stream_init_ex",
           "kvq_stream_cache_sizes",
           "kvq_stream_workspace_bytes", "kvq_stream_plan", "kv_stream_prefill", "kv_stream_append",
           "kv_stream_decode", "kvq_side_sizes", "kv_side_pack", "kv_decode_attn_side", "kvq_decode_plan",
           "kv_decode_attn_noalloc", "kv_decode_attn_timed", "kvq_layout_set_flags", "kvq_stream_set_flags"]

KVQ_KERNEL_MFMA, KVQ_KERNEL_VALU = 1, 2
KVQ_STATIC_SCRATCH_BYTES = 16 << 20
KVQ_KEY_ROTATION = 1


class KvqSide(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scale", ctypes.c_void_p), ("zero", ctypes.c_void_p)]


class KvqDecodeInfo(ctypes.Structure):
    _fields_ = [("kernel", ctypes.c_int32), ("units", ctypes.c_int32), ("ring_depth", ctypes.c_int32),
                ("waves_per_simd", ctypes.c_int32), ("waves", ctypes.c_int64)]


class KvqLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in LAYOUT_FIELDS]


class KvqCache(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in CACHE_FIELDS]


STREAM_FIELDS = ["t", "n_groups", "n_rows", "n_pending", "g_cap", "r_cap"]


class KvqStream(ctypes.Structure):
    _fields_ = ([("L", KvqLayout)] + [(n, ctypes.c_int32) for n in STREAM_FIELDS]
                + [("row_pos", ctypes.c_int32 * KVQ_STREAM_MAX_ROWS),
                   ("row_pending", ctypes.c_uint8 * KVQ_STREAM_MAX_ROWS)])


class KvqStreamStep(ctypes.Structure):
    _fields_ = [("new_row", ctypes.c_int32), ("group", ctypes.c_int32),
                ("member_rows", ctypes.c_int32 * KVQ_GROUP), ("member_pos", ctypes.c_int32 * KVQ_GROUP),
                ("n_moves", ctypes.c_int32), ("move_src", ctypes.c_int32 * KVQ_GROUP),
                ("move_dst", ctypes.c_int32 * KVQ_GROUP)]


_lib = None


def load() -> ctypes.CDLL:
    """Load libkvq.so and declare the signatures.  Raises if the library is missing:
    there is no fallback path."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libkvq.so is not built (%s); run `python -m quantized_decode_attention_kv_amd.build`"
                           % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    c_int, c_i32, c_i64, c_sz, vp = ctypes.c_int, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p
    LP = ctypes.POINTER(KvqLayout)
    CP = ctypes.POINTER(KvqCache)
    lib.kvq_layout_init.argtypes = [LP] + [c_int] * 10
    lib.kvq_layout_init.restype = c_int
    lib.kvq_layout_init_ex.argtypes = [LP] + [c_int] * 12
    lib.kvq_layout_init_ex.restype = c_int
    lib.kvq_layout_set_flags.argtypes = [LP, c_int]
    lib.kvq_layout_set_flags.restype = c_int
    lib.kvq_cache_sizes.argtypes = [LP, ctypes.POINTER(c_sz)]
    lib.kvq_cache_sizes.restype = c_int
    lib.kvq_retained_positions.argtypes = [LP, ctypes.POINTER(c_i32), c_i32]
    lib.kvq_retained_positions.restype = c_int
    lib.kvq_quantized_before.argtypes = [LP, c_i64]
    lib.kvq_quantized_before.restype = c_i64
    lib.kvq_decode_workspace_bytes.argtypes = [LP, c_int]
    lib.kvq_decode_workspace_bytes.restype = c_sz
    lib.kv_quant_pack.argtypes = [LP, c_i64, c_i64, vp, vp, c_int, CP, vp]
    lib.kv_quant_pack.restype = c_int
    lib.kv_decode_attn.argtypes = [LP, vp, c_int, CP, ctypes.c_float, c_int, vp, c_sz, vp, vp]
    lib.kv_decode_attn.restype = c_int
    lib.kv_decode_attn_ex.argtypes = [LP, vp, c_int, CP, ctypes.c_float, c_int, vp, c_sz, vp, vp, vp]
    lib.kv_decode_attn_ex.restype = c_int
    lib.kv_decode_attn_timed.argtypes = [LP, vp, c_int, CP, ctypes.c_float, c_int, vp, c_sz, vp, vp, vp, vp]
    lib.kv_decode_attn_timed.restype = c_int
    lib.kv_decode_attn_noalloc.argtypes = [LP, vp, c_int, CP, ctypes.c_float, c_int, vp, vp]
    lib.kv_decode_attn_noalloc.restype = c_int
    lib.kvq_decode_plan.argtypes = [LP, c_int, c_int, ctypes.POINTER(KvqDecodeInfo)]
    lib.kvq_decode_plan.restype = c_int
    SDP = ctypes.POINTER(KvqSide)
    lib.kvq_side_sizes.argtypes = [LP, c_int, ctypes.POINTER(c_sz)]
    lib.kvq_side_sizes.restype = c_int
    lib.kv_side_pack.argtypes = [LP, c_int, c_int, vp, vp, c_int, CP, SDP, vp]
    lib.kv_side_pack.restype = c_int
    lib.kv_decode_attn_side.argtypes = [LP, vp, c_int, CP, c_int, vp, SDP, ctypes.c_float, c_int, vp, c_sz, vp, vp]
    lib.kv_decode_attn_side.restype = c_int
    lib.kvq_read_probe.argtypes = [vp, c_sz, vp, vp]
    lib.kvq_read_probe.restype = c_int
    SP = ctypes.POINTER(KvqStream)
    lib.kvq_stream_init.argtypes = [SP] + [c_int] * 10
    lib.kvq_stream_init.restype = c_int
    lib.kvq_stream_init_ex.argtypes = [SP] + [c_int] * 11
    lib.kvq_stream_init_ex.restype = c_int
    lib.kvq_stream_set_flags.argtypes = [SP, c_int]
    lib.kvq_stream_set_flags.restype = c_int
    lib.kvq_stream_cache_sizes.argtypes = [SP, ctypes.POINTER(c_sz)]
    lib.kvq_stream_cache_sizes.restype = c_int
    lib.kvq_stream_workspace_bytes.argtypes = [SP, c_int]
    lib.kvq_stream_workspace_bytes.restype = c_sz
    lib.kvq_stream_plan.argtypes = [SP, ctypes.POINTER(KvqStreamStep)]
    lib.kvq_stream_plan.restype = c_int
    lib.kv_stream_prefill.argtypes = [SP, c_int, vp, vp, c_int, CP, vp]
    lib.kv_stream_prefill.restype = c_int
    lib.kv_stream_append.argtypes = [SP, vp, vp, c_int, CP, vp]
    lib.kv_stream_append.restype = c_int
    lib.kv_stream_decode.argtypes = [SP, vp, c_int, CP, ctypes.c_float, c_int, vp, c_sz, vp, vp]
    lib.kv_stream_decode.restype = c_int
    lib.kvq_status_string.argtypes = [c_int]
    lib.kvq_status_string.restype = ctypes.c_char_p
    lib.kvq_last_error.argtypes = []
    lib.kvq_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


class KvqError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("%s (%s)" % (message, status_name(status)))
        self.status = status


def status_name(status: int) -> str:
    return {KVQ_OK: "KVQ_OK", KVQ_ERR_INVALID: "KVQ_ERR_INVALID", KVQ_ERR_UNSUPPORTED: "KVQ_ERR_UNSUPPORTED",
            KVQ_ERR_HIP: "KVQ_ERR_HIP"}.get(status, "status %d" % status)


def check(status: int):
    if status != KVQ_OK:
        raise KvqError(status, load().kvq_last_error().decode())
