"""Python binding of libmoe_mi355x.so, the gfx950 fused MXFP4 MoE (see include/moe_mi355x.h).

Argument marshalling only: tensors are allocated with torch on the current CUDA (HIP) device,
their data pointers and torch's current stream are passed to the C entry points, and every
step of the operator runs in the library's HIP kernels.  If the library is not built the
calls raise; there is no fallback path.
"""
import ctypes
import os

import torch

DT_BF16, DT_FP8, DT_FP4 = 0, 1, 2
ACT_SITUV2, ACT_SILU, ACT_NONE_TEST = 0, 1, 2
STAGE_1, STAGE_2, STAGE_ALL = 1, 2, 3
W_ROW_MAJOR, W1_PACKED, W_PACKED = 0, 1, 2
DTYPES = {"bf16": DT_BF16, "fp8": DT_FP8, "fp4": DT_FP4}
ACTS = {"situv2": ACT_SITUV2, "silu": ACT_SILU, "none_test": ACT_NONE_TEST}

STATUS = {0: "MOE_OK", 1: "MOE_ERR_INVALID_ARG", 2: "MOE_ERR_UNSUPPORTED", 3: "MOE_ERR_CAPACITY",
          4: "MOE_ERR_HIP", 5: "MOE_ERR_WORKSPACE", 6: "MOE_ERR_DEBUG_CHECK"}
SORT_CHUNK = 4096
SORT_MIN_CHUNK = 1024

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe_mi355x.so")
# the same library built with MOE_DEBUG_CHECKS (device-side index checks; every call waits for
# the device and returns MOE_ERR_DEBUG_CHECK when a check failed)
DEBUG_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe_mi355x_debug.so")
EXPORTS = ("moe_sort", "moe_quant_act", "moe_pack_w1", "moe_pack_w2", "moe_fused", "moe_fused_noalloc",
           "moe_last_hip_error")
NOALLOC_SCRATCH_BYTES = 128 << 20


class MoeError(RuntimeError):
    def __init__(self, fn, status, hip_error=0):
        self.status = status
        msg = f"{fn} returned {STATUS.get(status, status)}"
        if status == 4:
            msg += f" (hipError_t {hip_error})"
        super().__init__(msg)


class Layout(ctypes.Structure):
    _fields_ = [("sorted_token_ids", ctypes.c_void_p), ("sorted_weights", ctypes.c_void_p),
                ("expert_ids", ctypes.c_void_p), ("num_tiles", ctypes.c_void_p),
                ("row_of", ctypes.c_void_p), ("sync", ctypes.c_void_p), ("cap_tiles", ctypes.c_int32),
                ("block_m", ctypes.c_int32)]


class ActParams(ctypes.Structure):
    _fields_ = [("act", ctypes.c_int32), ("beta", ctypes.c_float), ("linear_beta", ctypes.c_float)]


_lib = None


def lib():
    """Load libmoe_mi355x.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run: python -m quantized_moe_expert_sort_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        L.moe_sort.argtypes = [vp, vp, i32, i32, i32, i32, ctypes.POINTER(Layout), vp, sz, vp]
        L.moe_sort.restype = i32
        L.moe_quant_act.argtypes = [vp, i64, i64, i32, vp, vp, vp]
        L.moe_quant_act.restype = i32
        L.moe_fused.argtypes = [vp, vp, i32, vp, i32, vp, vp, vp, vp, ctypes.POINTER(Layout), i32, i32,
                                i32, i32, i32, ctypes.POINTER(ActParams), vp, vp, sz, i32, vp]
        L.moe_fused.restype = i32
        L.moe_fused_noalloc.argtypes = [vp, vp, i32, vp, i32, vp, vp, vp, vp, ctypes.POINTER(Layout), i32, i32,
                                        i32, i32, i32, ctypes.POINTER(ActParams), vp, i32, vp]
        L.moe_fused_noalloc.restype = i32
        L.moe_pack_w1.argtypes = [vp, i32, i32, i32, vp, vp]
        L.moe_pack_w1.restype = i32
        L.moe_pack_w2.argtypes = [vp, i32, i32, i32, vp, vp]
        L.moe_pack_w2.restype = i32
        L.moe_last_hip_error.argtypes = []
        L.moe_last_hip_error.restype = i32
        _lib = L
    return _lib


def select_library(path):
    """Route later calls to the library at `path` (LIB_PATH or DEBUG_LIB_PATH); returns the
    previous path."""
    global LIB_PATH, _lib
    prev, LIB_PATH, _lib = LIB_PATH, path, None
    return prev


def _check(fn, status):
    if status != 0:
        raise MoeError(fn, status, lib().moe_last_hip_error() if status == 4 else 0)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


# ------------------------------------------------------------------ size helpers (mirror the
# static inline helpers of include/moe_mi355x.h)

def _align256(b):
    return (b + 255) & ~255


def block_m(tokens):
    """Rows per tile the kernels are tuned for (moe_block_m of the header)."""
    return 16 if tokens <= 512 else 32


def cap_tiles(tokens, topk, num_local_experts, block_m):
    n = tokens * topk
    return (n + block_m - 1) // block_m + min(num_local_experts, n)


SINGLE_LAUNCH_MAX_TOKENS = 2048
SYNC_CLASSES = 16


def sync_words(tokens, cap):
    return 16 * (1 + 2 * cap + SYNC_CLASSES * tokens)


def sort_ws_bytes(tokens, topk, num_local_experts):
    n = tokens * topk
    chunks = (n + SORT_MIN_CHUNK - 1) // SORT_MIN_CHUNK
    return _align256((chunks + 2) * num_local_experts * 4) + _align256(n * 4)


def row_bytes(cols, dt):
    return cols * 2 if dt == DT_BF16 else cols if dt == DT_FP8 else cols // 2


def rowout_elem_bytes(a_dtype):
    return 2


HOT_MAX = 16
WS_PARTS = ("rowout", "inter", "iscale", "groups", "cgroups", "tile_hot", "hot_e", "hotpos", "hotw", "hotmask",
            "hot_out", "dbg", "total")


def fused_ws_parts(tokens, model_dim, inter_dim, cap, block_m, a_dtype, act):
    """Byte offsets of the workspace parts and the total (moe_fused_ws_parts of the header)."""
    rows = cap * block_m
    t = max(tokens, 0)
    sizes = [_align256(rows * model_dim * rowout_elem_bytes(a_dtype)),
             _align256((rows + 1) * row_bytes(inter_dim, a_dtype)),
             _align256(0 if a_dtype == DT_BF16 else (rows + 1) * (inter_dim // 32)),
             _align256(cap * 8) + 256, _align256(cap * 8) + 256, _align256(cap * 4), 256,
             _align256(t * HOT_MAX * 4), _align256(t * HOT_MAX * 4), _align256(t * 4),
             _align256(t * model_dim * 2),
             _align256(rows * inter_dim * 2 * 4) if act == ACT_NONE_TEST else 0]
    out, o = {}, 0
    for name, sz in zip(WS_PARTS, sizes):
        out[name] = o
        o += sz
    out["total"] = o
    return out


def fused_debug_offset(tokens, model_dim, inter_dim, cap, block_m, a_dtype):
    return fused_ws_parts(tokens, model_dim, inter_dim, cap, block_m, a_dtype, ACT_NONE_TEST)["dbg"]


def fused_ws_bytes(tokens, model_dim, inter_dim, cap, block_m, a_dtype, act):
    return fused_ws_parts(tokens, model_dim, inter_dim, cap, block_m, a_dtype, act)["total"]


# ------------------------------------------------------------------ entry points

class MoeLayout:
    """Device buffers of a sorted layout (owned by torch) plus its ctypes view."""

    def __init__(self, tokens, topk, num_local_experts, block_m, with_weights=True, device="cuda",
                 cap=None, single_launch=False):
        """single_launch: allocate the sync words that let moe_fused run batches below
        SINGLE_LAUNCH_MAX_TOKENS as one launch (False: one launch per stage)."""
        self.block_m = block_m
        self.cap = cap_tiles(tokens, topk, num_local_experts, block_m) if cap is None else cap
        n = max(self.cap * block_m, 1)
        self.sorted_token_ids = torch.empty(n, dtype=torch.int32, device=device)
        self.sorted_weights = torch.empty(n, dtype=torch.float32, device=device) if with_weights else None
        self.expert_ids = torch.empty(max(self.cap, 1), dtype=torch.int32, device=device)
        self.num_tiles = torch.empty(1, dtype=torch.int32, device=device)
        self.row_of = torch.empty(max(tokens * topk, 1), dtype=torch.int32, device=device)
        self.sync = (torch.empty(sync_words(tokens, self.cap), dtype=torch.int32, device=device)
                     if single_launch else None)
        self.c = Layout(self.sorted_token_ids.data_ptr(),
                        None if self.sorted_weights is None else self.sorted_weights.data_ptr(),
                        self.expert_ids.data_ptr(), self.num_tiles.data_ptr(), self.row_of.data_ptr(),
                        None if self.sync is None else self.sync.data_ptr(), self.cap, block_m)


def moe_sort(topk_ids, topk_w, expert_begin, num_local_experts, block_m, with_weights=True,
             layout=None, ws=None, single_launch=False):
    """Route-sort on the GPU; returns a MoeLayout (see moe_sort in the header)."""
    T, K = topk_ids.shape
    if layout is None:
        layout = MoeLayout(T, K, num_local_experts, block_m, with_weights, topk_ids.device,
                           single_launch=single_launch)
    if ws is None:
        ws = torch.empty(max(sort_ws_bytes(T, K, num_local_experts), 1), dtype=torch.uint8,
                         device=topk_ids.device)
    _check("moe_sort", lib().moe_sort(_ptr(topk_ids), _ptr(topk_w) if with_weights else None, T, K,
                                      expert_begin, num_local_experts, ctypes.byref(layout.c),
                                      _ptr(ws), ws.numel(), _stream()))
    return layout


def moe_pack_w1(w1, out=None):
    """Stage1 weights [E, 2I, D/2] uint8 (row-major) -> the packed layout moe_fused reads."""
    E, rows, half_d = w1.shape
    if out is None:
        out = torch.empty_like(w1)
    _check("moe_pack_w1", lib().moe_pack_w1(_ptr(w1), E, half_d * 2, rows // 2, _ptr(out), _stream()))
    return out


def moe_pack_w2(w2, out=None):
    """Stage2 weights [E, D, I/2] uint8 (row-major) -> the packed layout moe_fused reads."""
    E, D, half_i = w2.shape
    if out is None:
        out = torch.empty_like(w2)
    _check("moe_pack_w2", lib().moe_pack_w2(_ptr(w2), E, D, half_i * 2, _ptr(out), _stream()))
    return out


def device_weights(w1, w1s, w2, w2s, device="cuda"):
    """Host MXFP4 weights (numpy, row-major) -> the device tuple moe_fused takes (w1 and w2
    packed, the scales as they are)."""
    w1_d, w1s_d, w2_d, w2s_d = (torch.from_numpy(a).to(device) for a in (w1, w1s, w2, w2s))
    p1, p2 = moe_pack_w1(w1_d), moe_pack_w2(w2_d)
    del w1_d, w2_d
    return p1, w1s_d, p2, w2s_d


def moe_quant_act(x_bf16, dt, q=None, scale=None):
    """bf16 [rows, cols] -> (codes, e8m0 scales); dt is "fp8" or "fp4"."""
    d = DTYPES[dt] if isinstance(dt, str) else dt
    rows, cols = x_bf16.shape
    if q is None:
        q = torch.empty((rows, cols if d == DT_FP8 else cols // 2), dtype=torch.uint8, device=x_bf16.device)
    if scale is None:
        scale = torch.empty((rows, cols // 32), dtype=torch.uint8, device=x_bf16.device)
    _check("moe_quant_act", lib().moe_quant_act(_ptr(x_bf16), rows, cols, d, _ptr(q), _ptr(scale), _stream()))
    return q, scale


def moe_fused(x, x_scale, a_dtype, w1, w1_scale, w2, w2_scale, topk_w, layout, num_local_experts,
              act="situv2", beta=None, linear_beta=None, out=None, ws=None, stages=STAGE_ALL,
              w_layout=W_PACKED):
    """Stage1 + Stage2 over a layout from moe_sort; returns out [T, D] bf16 (or, for
    act="none_test", the workspace tensor holding the raw gate/up sums).  w1 and w2 are in the
    layout named by w_layout (the library reads W_PACKED, as moe_pack_w1 / moe_pack_w2 write
    them; device_weights does both).  stages selects
    STAGE_1, STAGE_2 (reusing the intermediate a STAGE_1 call left in the same ws) or both."""
    d = DTYPES[a_dtype] if isinstance(a_dtype, str) else a_dtype
    a = ACTS[act] if isinstance(act, str) else act
    T, K = topk_w.shape
    D = w2.shape[1]
    I = w2.shape[2] * 2
    if a == ACT_SITUV2 and (beta is None or linear_beta is None):
        raise ValueError("SiTUv2 needs beta and linear_beta (there are no defaults)")
    params = ActParams(a, 0.0 if beta is None else beta, 0.0 if linear_beta is None else linear_beta)
    if ws is None:
        ws = torch.empty(fused_ws_bytes(T, D, I, layout.cap, layout.block_m, d, a), dtype=torch.uint8,
                         device=topk_w.device)
    if out is None and a != ACT_NONE_TEST:
        out = torch.empty((T, D), dtype=torch.bfloat16, device=topk_w.device)
    _check("moe_fused", lib().moe_fused(_ptr(x), _ptr(x_scale), d, _ptr(w1), w_layout, _ptr(w1_scale), _ptr(w2),
                                        _ptr(w2_scale), _ptr(topk_w), ctypes.byref(layout.c), T, K,
                                        num_local_experts, D, I, ctypes.byref(params), _ptr(out),
                                        _ptr(ws), ws.numel(), stages, _stream()))
    return ws if a == ACT_NONE_TEST else out


def moe_fused_noalloc(x, x_scale, a_dtype, w1, w1_scale, w2, w2_scale, topk_w, layout, num_local_experts,
                      act="situv2", beta=None, linear_beta=None, out=None, stages=STAGE_ALL,
                      w_layout=W_PACKED):
    """moe_fused with the library's fixed per-device scratch as its workspace (nothing allocated
    for the workspace; calls on one device share it and must not overlap).  Returns out."""
    d = DTYPES[a_dtype] if isinstance(a_dtype, str) else a_dtype
    a = ACTS[act] if isinstance(act, str) else act
    T, K = topk_w.shape
    D = w2.shape[1]
    I = w2.shape[2] * 2
    if a == ACT_SITUV2 and (beta is None or linear_beta is None):
        raise ValueError("SiTUv2 needs beta and linear_beta (there are no defaults)")
    params = ActParams(a, 0.0 if beta is None else beta, 0.0 if linear_beta is None else linear_beta)
    if out is None and a != ACT_NONE_TEST:
        out = torch.empty((T, D), dtype=torch.bfloat16, device=topk_w.device)
    _check("moe_fused_noalloc", lib().moe_fused_noalloc(_ptr(x), _ptr(x_scale), d, _ptr(w1), w_layout,
                                                        _ptr(w1_scale), _ptr(w2), _ptr(w2_scale), _ptr(topk_w),
                                                        ctypes.byref(layout.c), T, K, num_local_experts, D, I,
                                                        ctypes.byref(params), _ptr(out), stages, _stream()))
    return out
