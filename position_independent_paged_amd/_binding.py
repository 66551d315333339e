"""ctypes binding of libminipic.so (argument marshalling only).

Each function takes torch tensors that already live on the GPU, passes their
data pointers and the current HIP stream to the C entry point of the same
name, and raises MinipicError on a non-zero status. No arithmetic of the
method happens here.
"""
import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libminipic.so")

MINIPIC_OK = 0
MINIPIC_ERR_INVALID_ARG = -1
MINIPIC_ERR_UNSUPPORTED = -2
MINIPIC_ERR_WORKSPACE = -3
MINIPIC_ERR_HIP = -4
MINIPIC_F32 = 0
MINIPIC_BF16 = 1
MINIPIC_BLK_PDEP = 1
MINIPIC_BLK_GLOBAL = 2
MINIPIC_FLAG_ROTATE_Q = 1
MINIPIC_EW_BLOCK = 1
MINIPIC_EW_POS = 2
MINIPIC_EW_QCTX = 4
MINIPIC_EW_CTX = 8
MINIPIC_EW_SPAN = 16
MINIPIC_EW_PLAN = 32

EXPORTS = [
    "minipic_version", "minipic_status_string", "minipic_last_error", "minipic_rope_table",
    "minipic_write_kv", "minipic_workspace_size", "minipic_get_launch_info", "minipic_prefill_attn",
    "minipic_reference_prerotated", "minipic_set_kernel_timing", "minipic_kernel_times",
    "minipic_kernel_times_all",
    "minipic_decode_workspace_size", "minipic_decode_attn", "minipic_decode_prerotated",
    "minipic_describe_blocks", "minipic_block_cache_create", "minipic_block_cache_destroy",
    "minipic_block_cache_assign", "minipic_slot_mapping", "minipic_prefill_attn_static",
    "minipic_prefill_plan", "minipic_prefill_run",
]


MINIPIC_ERR_CONTRACT = -5
MINIPIC_ERR_CACHE_FULL = -6
MINIPIC_STATIC_WORKSPACE_BYTES = 128 * 1024 * 1024


class minipic_markers(ctypes.Structure):
    """Marker token ids (-1 disables one) and the hash seed h_0."""
    _fields_ = [("ssep", ctypes.c_int32), ("pdep", ctypes.c_int32), ("global_", ctypes.c_int32),
                ("seed", ctypes.c_uint64)]


class MinipicError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"minipic status {status}: {msg}")
        self.status = status


class minipic_batch(ctypes.Structure):
    _fields_ = [
        ("num_reqs", ctypes.c_int32), ("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("block_size", ctypes.c_int32), ("max_blocks_per_req", ctypes.c_int32),
        ("total_q", ctypes.c_int64), ("max_q_len", ctypes.c_int32), ("max_ctx_len", ctypes.c_int32),
        ("q_indptr", ctypes.c_void_p), ("q_ctx_idx", ctypes.c_void_p), ("ctx_len", ctypes.c_void_p),
        ("block_table", ctypes.c_void_p), ("logical_pos", ctypes.c_void_p), ("span_id", ctypes.c_void_p),
        ("blk_flags", ctypes.c_void_p),
    ]


class minipic_launch_info(ctypes.Structure):
    _fields_ = [
        ("rows_per_tile", ctypes.c_int32), ("tokens_per_tile", ctypes.c_int32), ("num_q_tiles", ctypes.c_int32),
        ("num_splits", ctypes.c_int32), ("split_blocks", ctypes.c_int32), ("threads", ctypes.c_int32),
        ("num_workgroups", ctypes.c_int64), ("num_tiles", ctypes.c_int64), ("partial_slots", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
    ]


_lib = None


def load_library(path: str = None):
    """Load libminipic.so; fails loudly if it has not been built.

    MINIPIC_LIBRARY names another build of the same library (the tests load a
    copy whose host code is built with address and undefined-behaviour
    sanitizers this way)."""
    global _lib
    if _lib is not None:
        return _lib
    if path is None:
        path = os.environ.get("MINIPIC_LIBRARY") or LIB_PATH
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m position_independent_paged_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    lib.minipic_version.restype = ctypes.c_char_p
    lib.minipic_status_string.restype = ctypes.c_char_p
    lib.minipic_status_string.argtypes = [ctypes.c_int]
    lib.minipic_last_error.restype = ctypes.c_char_p
    lib.minipic_rope_table.argtypes = [vp, i32, i32, ctypes.c_double, vp]
    lib.minipic_write_kv.argtypes = [vp, vp, vp, i64, i32, i32, i32, vp, vp, i64, i32, vp]
    lib.minipic_workspace_size.argtypes = [ctypes.POINTER(minipic_batch), i32, ctypes.POINTER(sz)]
    lib.minipic_get_launch_info.argtypes = [ctypes.POINTER(minipic_batch), i32, ctypes.POINTER(minipic_launch_info)]
    attn = [vp, vp, vp, i64, ctypes.POINTER(minipic_batch), vp, i32, ctypes.c_float, vp, vp, sz, ctypes.c_uint32,
            i32, vp]
    lib.minipic_prefill_attn.argtypes = attn
    lib.minipic_reference_prerotated.argtypes = attn
    lib.minipic_prefill_run.argtypes = attn
    lib.minipic_prefill_plan.argtypes = [i64, ctypes.POINTER(minipic_batch), vp, i32, vp, sz, ctypes.c_uint32, i32,
                                         vp]
    lib.minipic_prefill_attn_static.argtypes = [vp, vp, vp, i64, ctypes.POINTER(minipic_batch), vp, i32,
                                                ctypes.c_float, vp, vp, ctypes.c_uint32, i32, vp]
    lib.minipic_decode_workspace_size.argtypes = [ctypes.POINTER(minipic_batch), i32, ctypes.POINTER(sz)]
    lib.minipic_decode_attn.argtypes = attn
    lib.minipic_decode_prerotated.argtypes = [vp, vp, vp, i64, ctypes.POINTER(minipic_batch), ctypes.c_float, vp,
                                              vp, sz, ctypes.c_uint32, i32, vp]
    lib.minipic_describe_blocks.argtypes = [vp, i64, ctypes.POINTER(minipic_markers), i32, vp, vp, vp, i64,
                                            ctypes.POINTER(i64)]
    lib.minipic_block_cache_create.argtypes = [i64]
    lib.minipic_block_cache_create.restype = ctypes.c_void_p
    lib.minipic_block_cache_destroy.argtypes = [ctypes.c_void_p]
    lib.minipic_block_cache_destroy.restype = None
    lib.minipic_block_cache_assign.argtypes = [ctypes.c_void_p, vp, i64, vp, vp, ctypes.POINTER(i64)]
    lib.minipic_slot_mapping.argtypes = [vp, vp, i64, i32, vp, vp, ctypes.POINTER(i64)]
    lib.minipic_set_kernel_timing.argtypes = [ctypes.c_int]
    lib.minipic_kernel_times.argtypes = [ctypes.POINTER(ctypes.c_float)]
    lib.minipic_kernel_times_all.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_int32,
                                             ctypes.POINTER(ctypes.c_int32)]
    for name in EXPORTS[3:]:
        if name not in ("minipic_block_cache_create", "minipic_block_cache_destroy"):
            getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def _check(status):
    if status != MINIPIC_OK:
        lib = load_library()
        raise MinipicError(status, lib.minipic_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is not None:
        return ctypes.c_void_p(stream)
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return MINIPIC_BF16
    if t.dtype == torch.float32:
        return MINIPIC_F32
    raise MinipicError(MINIPIC_ERR_UNSUPPORTED, f"unsupported tensor dtype {t.dtype}")


def minipic_version() -> str:
    return load_library().minipic_version().decode()


def minipic_rope_table(cos_sin, max_pos: int, head_dim: int, base: float, stream=None):
    _check(load_library().minipic_rope_table(_ptr(cos_sin), max_pos, head_dim, float(base), _stream(stream)))


def minipic_write_kv(k, v, slot_mapping, k_cache, v_cache, *, num_kv_heads: int, head_dim: int,
                     block_size: int = 16, num_blocks: int, stream=None):
    _check(load_library().minipic_write_kv(
        _ptr(k), _ptr(v), _ptr(slot_mapping), int(slot_mapping.shape[0]), num_kv_heads, head_dim, block_size,
        _ptr(k_cache), _ptr(v_cache), int(num_blocks), _dtype_code(k_cache), _stream(stream)))


def minipic_workspace_size(batch: minipic_batch, dtype_code: int) -> int:
    n = ctypes.c_size_t(0)
    _check(load_library().minipic_workspace_size(ctypes.byref(batch), dtype_code, ctypes.byref(n)))
    return int(n.value)


def minipic_get_launch_info(batch: minipic_batch, dtype_code: int) -> dict:
    info = minipic_launch_info()
    _check(load_library().minipic_get_launch_info(ctypes.byref(batch), dtype_code, ctypes.byref(info)))
    return {f: getattr(info, f) for f, _ in minipic_launch_info._fields_}


def _attn(fn, q, k_cache, v_cache, num_blocks, batch, cos_sin, max_pos, out, workspace, flags, softmax_scale,
          stream):
    _check(fn(_ptr(q), _ptr(k_cache), _ptr(v_cache), int(num_blocks), ctypes.byref(batch), _ptr(cos_sin),
              int(max_pos), float(softmax_scale), _ptr(out), _ptr(workspace),
              0 if workspace is None else workspace.numel() * workspace.element_size(), int(flags),
              _dtype_code(q), _stream(stream)))


def minipic_prefill_attn(q, k_cache, v_cache, num_blocks, batch, cos_sin, max_pos, out, workspace, *,
                         flags: int = 0, softmax_scale: float = 0.0, stream=None):
    _attn(load_library().minipic_prefill_attn, q, k_cache, v_cache, num_blocks, batch, cos_sin, max_pos, out,
          workspace, flags, softmax_scale, stream)


def minipic_prefill_plan(num_blocks, batch, cos_sin, max_pos, workspace, *, dtype_code: int, flags: int = 0,
                         stream=None):
    """The planning kernels of minipic_prefill_attn only (the plan serves minipic_prefill_run calls)."""
    _check(load_library().minipic_prefill_plan(
        int(num_blocks), ctypes.byref(batch), _ptr(cos_sin), int(max_pos), _ptr(workspace),
        0 if workspace is None else workspace.numel() * workspace.element_size(), int(flags), int(dtype_code),
        _stream(stream)))


def minipic_prefill_run(q, k_cache, v_cache, num_blocks, batch, cos_sin, max_pos, out, workspace, *,
                        flags: int = 0, softmax_scale: float = 0.0, stream=None):
    """The attention and merge kernels of minipic_prefill_attn on a workspace holding a plan of the batch."""
    _attn(load_library().minipic_prefill_run, q, k_cache, v_cache, num_blocks, batch, cos_sin, max_pos, out,
          workspace, flags, softmax_scale, stream)


def minipic_prefill_attn_static(q, k_cache, v_cache, num_blocks, batch, cos_sin, max_pos, out, err_word=None, *,
                                flags: int = 0, softmax_scale: float = 0.0, stream=None):
    """minipic_prefill_attn on the library's own workspace (no allocation); err_word: None or a device int32/uint32."""
    _check(load_library().minipic_prefill_attn_static(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), int(num_blocks), ctypes.byref(batch), _ptr(cos_sin), int(max_pos),
        float(softmax_scale), _ptr(out), _ptr(err_word), int(flags), _dtype_code(q), _stream(stream)))


def minipic_reference_prerotated(q, k_cache, v_cache, num_blocks, batch, out, workspace, *, cos_sin=None,
                                 max_pos: int = 0, flags: int = 0, softmax_scale: float = 0.0, stream=None):
    _attn(load_library().minipic_reference_prerotated, q, k_cache, v_cache, num_blocks, batch, cos_sin, max_pos,
          out, workspace, flags, softmax_scale, stream)


def minipic_set_kernel_timing(enable: bool):
    _check(load_library().minipic_set_kernel_timing(1 if enable else 0))


def minipic_kernel_times() -> tuple:
    """(plan, attention, merge) milliseconds of the latest timed attention call of this thread."""
    ms = (ctypes.c_float * 3)()
    _check(load_library().minipic_kernel_times(ms))
    return float(ms[0]), float(ms[1]), float(ms[2])


def minipic_kernel_times_all(max_calls: int = 4096) -> list:
    """(plan, attention, merge) milliseconds of every attention call timed since timing was switched on."""
    ms = (ctypes.c_float * (3 * max_calls))()
    n = ctypes.c_int32(0)
    _check(load_library().minipic_kernel_times_all(ms, max_calls, ctypes.byref(n)))
    return [(float(ms[3 * c]), float(ms[3 * c + 1]), float(ms[3 * c + 2])) for c in range(n.value)]


def minipic_decode_workspace_size(batch: minipic_batch, dtype_code: int) -> int:
    n = ctypes.c_size_t(0)
    _check(load_library().minipic_decode_workspace_size(ctypes.byref(batch), dtype_code, ctypes.byref(n)))
    return int(n.value)


def minipic_decode_attn(q, k_cache, v_cache, num_blocks, batch, cos_sin, max_pos, out, workspace, *,
                        flags: int = 0, softmax_scale: float = 0.0, stream=None):
    _attn(load_library().minipic_decode_attn, q, k_cache, v_cache, num_blocks, batch, cos_sin, max_pos, out,
          workspace, flags, softmax_scale, stream)


def minipic_decode_prerotated(q, k_cache, v_cache, num_blocks, batch, out, workspace, *, flags: int = 0,
                              softmax_scale: float = 0.0, stream=None):
    _check(load_library().minipic_decode_prerotated(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), int(num_blocks), ctypes.byref(batch), float(softmax_scale),
        _ptr(out), _ptr(workspace), int(workspace.numel() * workspace.element_size()), int(flags),
        _dtype_code(q), _stream(stream)))


def _np_ptr(a):
    return ctypes.c_void_p(a.ctypes.data) if a is not None and a.size else None


def minipic_describe_blocks(tokens, *, ssep=-1, pdep=-1, global_=-1, seed=0):
    """(hashes uint64, span_id int32, flags uint8) of one request's blocks."""
    import numpy as np
    tok = np.ascontiguousarray(tokens, dtype=np.int32)
    nb = (len(tok) + 15) // 16
    hashes = np.zeros(max(nb, 1), np.uint64)
    span = np.zeros(max(nb, 1), np.int32)
    flags = np.zeros(max(nb, 1), np.uint8)
    m = minipic_markers(ssep, pdep, global_, seed)
    out = ctypes.c_int64(0)
    _check(load_library().minipic_describe_blocks(_np_ptr(tok), len(tok), ctypes.byref(m), 16, _np_ptr(hashes),
                                                  _np_ptr(span), _np_ptr(flags), nb, ctypes.byref(out)))
    return hashes[:nb], span[:nb], flags[:nb]


class BlockCache:
    """Hash -> physical block map of the library (host memory)."""

    def __init__(self, num_blocks: int):
        self._lib = load_library()
        self._h = self._lib.minipic_block_cache_create(int(num_blocks))
        if not self._h:
            raise MinipicError(MINIPIC_ERR_INVALID_ARG, "minipic_block_cache_create failed")

    def assign(self, hashes):
        """(block_table int32, hit uint8, num_hits) for one request's block hashes."""
        import numpy as np
        h = np.ascontiguousarray(hashes, dtype=np.uint64)
        bt = np.zeros(max(len(h), 1), np.int32)
        hit = np.zeros(max(len(h), 1), np.uint8)
        n = ctypes.c_int64(0)
        _check(self._lib.minipic_block_cache_assign(ctypes.c_void_p(self._h), _np_ptr(h), len(h), _np_ptr(bt),
                                                    _np_ptr(hit), ctypes.byref(n)))
        return bt[:len(h)], hit[:len(h)], int(n.value)

    def close(self):
        if self._h:
            self._lib.minipic_block_cache_destroy(ctypes.c_void_p(self._h))
            self._h = None

    def __del__(self):
        self.close()


def minipic_slot_mapping(block_table, hit, n: int):
    """(slots int64, ctx_index int32) of the tokens whose blocks missed."""
    import numpy as np
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    hi = np.ascontiguousarray(hit, dtype=np.uint8)
    slots = np.zeros(max(n, 1), np.int64)
    idx = np.zeros(max(n, 1), np.int32)
    k = ctypes.c_int64(0)
    _check(load_library().minipic_slot_mapping(_np_ptr(bt), _np_ptr(hi), int(n), 16, _np_ptr(slots), _np_ptr(idx),
                                               ctypes.byref(k)))
    return slots[:k.value], idx[:k.value]
