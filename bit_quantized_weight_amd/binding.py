"""ctypes binding of ``libq4w.so`` -- argument marshalling only.

Every function takes torch tensors on the GPU, checks nothing the library
does not check itself beyond dtype/contiguity, and hands raw device pointers
plus torch's current HIP stream to the C ABI (``include/q4w.h``).  There is
no fallback: if the library is missing the call raises.
"""

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_NAME = "libq4w.so"
_lib = None

STATUS = {
    0: "OK",
    -1: "INVALID_ARG",
    -2: "UNSUPPORTED_SHAPE",
    -3: "MISALIGNED",
    -4: "WORKSPACE",
    -5: "HIP",
}


class GemvDesc(ctypes.Structure):
    """q4w_gemv_desc: one matmul of a batch."""
    _fields_ = [("x", ctypes.c_void_p), ("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("y", ctypes.c_void_p), ("N", ctypes.c_int64), ("K", ctypes.c_int64)]


class BatchedPlan(ctypes.Structure):
    """q4w_batched_plan, filled by q4_gemv_batched_plan."""
    _fields_ = [("M", ctypes.c_int), ("count", ctypes.c_int), ("total_items", ctypes.c_int),
                ("grid", ctypes.c_int), ("variant", ctypes.c_int), ("ws", ctypes.c_void_p)]


class Q4WError(RuntimeError):
    def __init__(self, fn, status, hip_err=0):
        self.status = status
        self.hip_error = hip_err
        super().__init__(f"{fn} failed: {STATUS.get(status, status)}"
                         + (f" (hipError {hip_err})" if status == -5 else ""))


def lib_path():
    return os.path.join(_HERE, "lib", LIB_NAME)


def lib():
    """Load the HIP library (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    path = lib_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'`")
    L = ctypes.CDLL(path)
    vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
    L.q4_pack.argtypes = [vp, i64, i64, vp, vp, vp]
    L.q4_pack.restype = i32
    L.q4_gemv_skinny_ws_bytes.argtypes = [i32, i64, i64, i32]
    L.q4_gemv_skinny_ws_bytes.restype = sz
    L.q4_gemv_skinny.argtypes = [vp, vp, vp, vp, i32, i64, i64, i32, vp, sz, vp]
    L.q4_gemv_skinny.restype = i32
    L.q4_gemv_skinny_noalloc.argtypes = [vp, vp, vp, vp, i32, i64, i64, i32, vp]
    L.q4_gemv_skinny_noalloc.restype = i32
    L.q4_attn_decode_ws_bytes.argtypes = [i32, i32, i32, i32, i64]
    L.q4_attn_decode_ws_bytes.restype = sz
    L.q4_attn_decode.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i64, vp, sz, vp]
    L.q4_attn_decode.restype = i32
    L.a8_quantize_act.argtypes = [vp, i64, i64, vp, vp, vp]
    L.a8_quantize_act.restype = i32
    L.a8w4_ws_bytes.argtypes = [i64, i64]
    L.a8w4_ws_bytes.restype = sz
    L.a8w4_gemm_prefill.argtypes = [vp, vp, vp, vp, i64, i64, i64, vp, sz, vp]
    L.a8w4_gemm_prefill.restype = i32
    L.a8w4_prepare_act.argtypes = [vp, i64, i64, vp, sz, vp]
    L.a8w4_prepare_act.restype = i32
    L.a8w4_gemm_prepared.argtypes = [vp, vp, vp, vp, i64, i64, i64, sz, vp]
    L.a8w4_gemm_prepared.restype = i32
    L.a8w4_debug_block_acc.argtypes = [vp, vp, vp, i64, i64, i64, vp, sz, vp]
    L.a8w4_debug_block_acc.restype = i32
    L.q4_gemv_batched_ws_bytes.argtypes = [i32, ctypes.POINTER(GemvDesc), i32]
    L.q4_gemv_batched_ws_bytes.restype = sz
    L.q4_gemv_batched_plan.argtypes = [i32, ctypes.POINTER(GemvDesc), i32, vp, sz,
                                       ctypes.POINTER(BatchedPlan)]
    L.q4_gemv_batched_plan.restype = i32
    L.q4_gemv_batched_run.argtypes = [ctypes.POINTER(BatchedPlan), vp]
    L.q4_gemv_batched_run.restype = i32
    L.q4w_stream_read.argtypes = [vp, sz, vp, i32, i32, vp]
    L.q4w_stream_read.restype = i32
    L.q4w_status_str.argtypes = [i32]
    L.q4w_status_str.restype = ctypes.c_char_p
    L.q4w_last_hip_error.argtypes = []
    L.q4w_last_hip_error.restype = i32
    _lib = L
    return L


def _check(fn, st):
    if st != 0:
        raise Q4WError(fn, st, lib().q4w_last_hip_error() if st == -5 else 0)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream():
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _need(t, dtype, name):
    if t.dtype != dtype or not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} CUDA tensor")


def _need_shape(t, shape, name):
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _need_packed(codes, scales, n, k, what="weights"):
    """codes uint8 [n, k/2] and scales fp16 [n, k/32], contiguous CUDA tensors:
    the library reads exactly these sizes, so a mismatch is refused here."""
    import torch
    _need(codes, torch.uint8, f"{what} codes")
    _need(scales, torch.float16, f"{what} scales")
    if k % 32 == 0:
        _need_shape(codes, (n, k // 2), f"{what} codes")
        _need_shape(scales, (n, k // 32), f"{what} scales")


# Workspaces are cached per (route, device, stream): calls on one stream run
# in order, so they may share one; calls on two streams could overlap in time
# and must not (their split-K counters, partials and quantized activations
# would race).  A cached workspace only grows.
_ws_cache = {}


def _workspace(nbytes, device, key):
    import torch
    if nbytes == 0:
        return None
    k = (key, str(device), torch.cuda.current_stream(device).cuda_stream)
    buf = _ws_cache.get(k)
    if buf is None or buf.numel() < nbytes:
        buf = torch.zeros(nbytes, dtype=torch.uint8, device=device)
        _ws_cache[k] = buf
    return buf


def pack(w):
    """fp32 W [N, K] (CUDA) -> (codes uint8 [N, K/2], scales fp16 [N, K/32])."""
    import torch
    _need(w, torch.float32, "w")
    n, k = w.shape
    codes = torch.empty((n, k // 2), dtype=torch.uint8, device=w.device)
    scales = torch.empty((n, k // 32), dtype=torch.float16, device=w.device)
    _check("q4_pack", lib().q4_pack(_ptr(w), n, k, _ptr(codes), _ptr(scales), _stream()))
    return codes, scales


def gemv_ws_bytes(m, n, k, split_k=0):
    return lib().q4_gemv_skinny_ws_bytes(m, n, k, split_k)


def q4_gemv_skinny_raw(x, codes, scales, y, split_k=0, ws=None):
    """Direct call into q4_gemv_skinny with a caller-provided output y [M, N]
    and, optionally, workspace ws (uint8; its whole size is passed, so the
    library rejects one that is too small)."""
    import torch
    _need(x, torch.float16, "x")
    m, k = x.shape
    n = codes.shape[0]
    _need_packed(codes, scales, n, k)
    _need(y, torch.float16, "y")
    _need_shape(y, (m, n), "y")
    if ws is None:
        ws = _workspace(gemv_ws_bytes(m, n, k, split_k), x.device, "gemv")
    else:
        _need(ws, torch.uint8, "ws")
    _check("q4_gemv_skinny", lib().q4_gemv_skinny(
        _ptr(x), _ptr(codes), _ptr(scales), _ptr(y), m, n, k, split_k,
        _ptr(ws), ws.numel() if ws is not None else 0, _stream()))
    return y


def gemv(x, codes, scales, split_k=0):
    """fp16 X [M<=16, K] against packed weights -> fp16 Y [M, N]."""
    import torch
    _need(x, torch.float16, "x")
    _need(codes, torch.uint8, "codes")
    _need(scales, torch.float16, "scales")
    y = torch.empty((x.shape[0], codes.shape[0]), dtype=torch.float16, device=x.device)
    return q4_gemv_skinny_raw(x, codes, scales, y, split_k)


# Q4W_NOALLOC_SCRATCH_BYTES of include/q4w.h: the largest split-K workspace
# q4_gemv_skinny_noalloc serves from its static device scratch.
NOALLOC_SCRATCH_BYTES = 256 * 1024 + 8 * 1024 * 1024


def gemv_noalloc(x, codes, scales, y, split_k=0):
    """q4_gemv_skinny_noalloc into a caller-provided fp16 y [M, N]: no
    workspace argument, nothing allocated (the library's static device
    scratch holds the split-K state)."""
    import torch
    _need(x, torch.float16, "x")
    m, k = x.shape
    n = codes.shape[0]
    _need_packed(codes, scales, n, k)
    _need(y, torch.float16, "y")
    _need_shape(y, (m, n), "y")
    _check("q4_gemv_skinny_noalloc", lib().q4_gemv_skinny_noalloc(
        _ptr(x), _ptr(codes), _ptr(scales), _ptr(y), m, n, k, split_k, _stream()))
    return y


def attn_decode_ws_bytes(m, n_q_heads, n_kv_heads, head_dim, t):
    return lib().q4_attn_decode_ws_bytes(m, n_q_heads, n_kv_heads, head_dim, t)


def attn_decode(q, k_codes, k_scales, v_codes, v_scales, n_kv_heads, out=None, ws=None):
    """Attention read of a 4-bit K/V cache: q fp16 [M, H_q, D]; caches as
    q4_pack output of the [T, H_kv * D] rows (codes uint8, scales fp16)
    -> fp16 o [M, H_q, D]."""
    import torch
    _need(q, torch.float16, "q")
    for t, dt, name in ((k_codes, torch.uint8, "k_codes"), (v_codes, torch.uint8, "v_codes"),
                        (k_scales, torch.float16, "k_scales"), (v_scales, torch.float16, "v_scales")):
        _need(t, dt, name)
    m, hq, d = q.shape
    t_len = k_codes.shape[0]
    _need_packed(k_codes, k_scales, t_len, n_kv_heads * d, "K cache")
    _need_packed(v_codes, v_scales, t_len, n_kv_heads * d, "V cache")
    if out is None:
        out = torch.empty_like(q)
    _need(out, torch.float16, "out")
    _need_shape(out, q.shape, "out")
    nb = attn_decode_ws_bytes(m, hq, n_kv_heads, d, t_len)
    if ws is None:
        ws = _workspace(nb, q.device, "attn")
    else:
        _need(ws, torch.uint8, "ws")
    _check("q4_attn_decode", lib().q4_attn_decode(
        _ptr(q), _ptr(k_codes), _ptr(k_scales), _ptr(v_codes), _ptr(v_scales), _ptr(out),
        m, hq, n_kv_heads, d, t_len, _ptr(ws), ws.numel() if ws is not None else 0, _stream()))
    return out


def a8_quantize_act(x):
    """fp16 X [M, K] -> (xq int8 [M, K], sa fp32 [M, K/64]) in the canonical layout."""
    import torch
    _need(x, torch.float16, "x")
    m, k = x.shape
    xq = torch.empty((m, k), dtype=torch.int8, device=x.device)
    sa = torch.empty((m, k // 64), dtype=torch.float32, device=x.device)
    _check("a8_quantize_act", lib().a8_quantize_act(_ptr(x), m, k, _ptr(xq), _ptr(sa), _stream()))
    return xq, sa


def a8w4_ws_bytes(m, k):
    return lib().a8w4_ws_bytes(m, k)


def a8w4_gemm(x, codes, scales, y=None):
    """A8 prefill route: fp16 X [M, K] -> fp16 Y [M, N]."""
    import torch
    _need(x, torch.float16, "x")
    m, k = x.shape
    n = codes.shape[0]
    _need_packed(codes, scales, n, k)
    if y is None:
        y = torch.empty((m, n), dtype=torch.float16, device=x.device)
    _need(y, torch.float16, "y")
    _need_shape(y, (m, n), "y")
    nb = a8w4_ws_bytes(m, k)
    ws = _workspace(nb, x.device, "a8")
    _check("a8w4_gemm_prefill", lib().a8w4_gemm_prefill(
        _ptr(x), _ptr(codes), _ptr(scales), _ptr(y), m, n, k, _ptr(ws), nb, _stream()))
    return y


def a8w4_prepare(x, ws=None):
    """Quantize fp16 X [M, K] once into a workspace (returned) for a8w4_gemm_prepared."""
    import torch
    _need(x, torch.float16, "x")
    m, k = x.shape
    nb = a8w4_ws_bytes(m, k)
    if ws is None:
        ws = torch.empty(max(nb, 1), dtype=torch.uint8, device=x.device)
    _check("a8w4_prepare_act", lib().a8w4_prepare_act(_ptr(x), m, k, _ptr(ws), ws.numel(), _stream()))
    return ws


def a8w4_gemm_prepared(ws, m, k, codes, scales, y=None):
    """A8 GEMM from a workspace filled by a8w4_prepare -> fp16 Y [M, N]."""
    import torch
    n = codes.shape[0]
    _need_packed(codes, scales, n, k)
    if y is None:
        y = torch.empty((m, n), dtype=torch.float16, device=codes.device)
    _need(y, torch.float16, "y")
    _need_shape(y, (m, n), "y")
    _need(ws, torch.uint8, "ws")
    _check("a8w4_gemm_prepared", lib().a8w4_gemm_prepared(
        _ptr(ws), _ptr(codes), _ptr(scales), _ptr(y), m, n, k, ws.numel(), _stream()))
    return y


def a8w4_debug_block_acc(x, codes, scales):
    """Exact int32 block sums [M, N, K/32] from the A8 kernel's debug epilogue."""
    import torch
    _need(x, torch.float16, "x")
    m, k = x.shape
    n = codes.shape[0]
    _need_packed(codes, scales, n, k)
    acc = torch.empty((m, n, k // 32), dtype=torch.int32, device=x.device)
    nb = a8w4_ws_bytes(m, k)
    ws = _workspace(nb, x.device, "a8")
    _check("a8w4_debug_block_acc", lib().a8w4_debug_block_acc(
        _ptr(x), _ptr(codes), _ptr(acc), m, n, k, _ptr(ws), nb, _stream()))
    return acc


class Batch:
    """A planned batch of independent skinny matmuls (same M): the plan, its
    workspace and references to every tensor it names (kept alive here)."""

    def __init__(self, plan, ws, tensors):
        self.plan = plan
        self.ws = ws
        self._tensors = tensors

    def run(self):
        """Enqueue the single persistent launch on torch's current stream."""
        _check("q4_gemv_batched_run", lib().q4_gemv_batched_run(ctypes.byref(self.plan), _stream()))


def _descs(items):
    arr = (GemvDesc * len(items))()
    for d, (x, codes, scales, y) in zip(arr, items):
        d.x, d.codes, d.scales, d.y = x.data_ptr(), codes.data_ptr(), scales.data_ptr(), y.data_ptr()
        d.N, d.K = codes.shape[0], x.shape[1]
    return arr


def batched_ws_bytes(m, items):
    return lib().q4_gemv_batched_ws_bytes(m, _descs(items), len(items))


def batched_plan(items):
    """items: list of (x fp16 [M, K], codes, scales, y fp16 [M, N]) CUDA tensors, one M.
    Plans them as one batch (blocking set-up call) and returns a Batch."""
    import torch
    m = items[0][0].shape[0]
    for x, codes, scales, y in items:
        _need(x, torch.float16, "x")
        _need(y, torch.float16, "y")
        if x.shape[0] != m or y.shape[0] != m:
            raise ValueError("every matmul of a batch has the same M")
        _need_packed(codes, scales, codes.shape[0], x.shape[1])
        _need_shape(y, (m, codes.shape[0]), "y")
    descs = _descs(items)
    nb = lib().q4_gemv_batched_ws_bytes(m, descs, len(items))
    if nb == 0:
        raise ValueError("invalid batch shapes")
    ws = torch.empty(nb, dtype=torch.uint8, device=items[0][0].device)
    plan = BatchedPlan()
    _check("q4_gemv_batched_plan", lib().q4_gemv_batched_plan(m, descs, len(items), _ptr(ws), nb,
                                                              ctypes.byref(plan)))
    return Batch(plan, ws, [t for it in items for t in it])


def stream_read(buf, grid=256, block=512, out=None):
    """Plain streaming read of a device tensor's bytes (a measurement helper):
    returns out, int32 [grid * block / 64], each wave's XOR of the words it read."""
    import torch
    if not buf.is_cuda or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous CUDA tensor")
    nout = grid * (block // 64)
    if out is None:
        out = torch.empty(nout, dtype=torch.int32, device=buf.device)
    _need(out, torch.int32, "out")
    _need_shape(out, (nout,), "out")
    nbytes = buf.numel() * buf.element_size()
    _check("q4w_stream_read", lib().q4w_stream_read(_ptr(buf), nbytes, _ptr(out), grid, block, _stream()))
    return out

