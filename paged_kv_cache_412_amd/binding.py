"""ctypes binding of libpa (``include/pa.h``): argument marshalling only.

Every function here takes torch tensors that already live on the GPU, checks
shapes on the host, passes raw device pointers and the current HIP stream to
the C ABI and raises :class:`PaError` on a non-OK status.  No arithmetic of
the path happens here; there is no CPU fallback.  If ``libpa.so`` is missing
the first call raises :class:`LibraryNotBuilt`.
"""

from __future__ import annotations

import ctypes
import os
import re

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libpa.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "pa.h")

PA_F32, PA_F16, PA_BF16, PA_FP8_E4M3, PA_FP8_E5M2 = 0, 1, 2, 3, 4
STATUS = {0: "PA_OK", 1: "PA_ERR_NULL", 2: "PA_ERR_SHAPE", 3: "PA_ERR_UNSUPPORTED",
          4: "PA_ERR_WORKSPACE", 5: "PA_ERR_LAUNCH", 6: "PA_ERR_OUT_OF_BLOCKS"}
PA_ERR_OUT_OF_BLOCKS = 6
# who combines split sequences (pa_decode_args.combine)
PA_COMBINE_AUTO, PA_COMBINE_IN_LAUNCH, PA_COMBINE_REDUCE = 0, 1, 2
DTYPE_NAMES = {"f32": PA_F32, "f16": PA_F16, "bf16": PA_BF16, "e4m3": PA_FP8_E4M3, "e5m2": PA_FP8_E5M2}
# uint8 pools are taken as e4m3 unless the caller names the format (kv_dtype)
TORCH_TO_PA = {torch.float32: PA_F32, torch.float16: PA_F16, torch.bfloat16: PA_BF16,
               torch.uint8: PA_FP8_E4M3, torch.float8_e4m3fn: PA_FP8_E4M3,
               torch.float8_e5m2: PA_FP8_E5M2}


class LibraryNotBuilt(RuntimeError):
    pass


class PaError(RuntimeError):
    def __init__(self, status: int, what: str, message: str):
        super().__init__(f"{what}: {STATUS.get(status, status)} ({message})")
        self.status = status


class DecodeArgs(ctypes.Structure):
    """Mirror of ``pa_decode_args``."""

    _fields_ = [
        ("out", ctypes.c_void_p), ("q", ctypes.c_void_p), ("k_cache", ctypes.c_void_p),
        ("v_cache", ctypes.c_void_p), ("block_tables", ctypes.c_void_p), ("seq_lens", ctypes.c_void_p),
        ("B", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32), ("D", ctypes.c_int32),
        ("block_size", ctypes.c_int32), ("num_blocks", ctypes.c_int32),
        ("max_blocks_per_seq", ctypes.c_int32), ("scale", ctypes.c_float), ("k_scale", ctypes.c_float),
        ("v_scale", ctypes.c_float), ("q_dtype", ctypes.c_int), ("kv_dtype", ctypes.c_int),
        ("out_dtype", ctypes.c_int), ("partition_size", ctypes.c_int32),
        ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
        ("k_scales", ctypes.c_void_p), ("v_scales", ctypes.c_void_p), ("combine", ctypes.c_int32),
    ]


class PrefillArgs(ctypes.Structure):
    """Mirror of ``pa_prefill_args``."""

    _fields_ = [
        ("out", ctypes.c_void_p), ("q", ctypes.c_void_p), ("k_cache", ctypes.c_void_p),
        ("v_cache", ctypes.c_void_p), ("block_tables", ctypes.c_void_p), ("seq_lens", ctypes.c_void_p),
        ("q_starts", ctypes.c_void_p), ("B", ctypes.c_int32), ("T", ctypes.c_int32),
        ("max_q_len", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32),
        ("D", ctypes.c_int32), ("block_size", ctypes.c_int32), ("num_blocks", ctypes.c_int32),
        ("max_blocks_per_seq", ctypes.c_int32), ("scale", ctypes.c_float), ("k_scale", ctypes.c_float),
        ("v_scale", ctypes.c_float), ("q_dtype", ctypes.c_int), ("kv_dtype", ctypes.c_int),
        ("out_dtype", ctypes.c_int), ("k_scales", ctypes.c_void_p), ("v_scales", ctypes.c_void_p),
    ]


_lib = None


def declared_functions() -> list:
    """Names of the functions ``include/pa.h`` declares."""
    text = open(HEADER, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pa_[a-z0-9_]+)\s*\(", text)))


def lib() -> ctypes.CDLL:
    """Load libpa.so (once)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise LibraryNotBuilt(f"{LIB_PATH} is missing: run `python -m paged_kv_cache_412_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float
    argp = ctypes.POINTER(DecodeArgs)
    L.pa_decode_workspace_size.argtypes = [argp]
    L.pa_decode_workspace_size.restype = ctypes.c_size_t
    L.pa_decode_workspace_zero_bytes.argtypes = [argp]
    L.pa_decode_workspace_zero_bytes.restype = ctypes.c_size_t
    L.pa_decode_partition_size.argtypes = [argp]
    L.pa_decode_partition_size.restype = ctypes.c_int32
    L.pa_read_blocks.argtypes = [vp, i32, ctypes.c_size_t, vp, i32, vp, i32, vp]
    L.pa_read_blocks.restype = ctypes.c_int
    for name in ("pa_decode", "pa_decode_partition", "pa_decode_reduce", "pa_decode_no_alloc"):
        getattr(L, name).argtypes = [argp, vp]
        getattr(L, name).restype = ctypes.c_int
    L.pa_decode_check.argtypes = [argp]
    L.pa_decode_check.restype = ctypes.c_int
    L.pa_slot_mapping.argtypes = [vp, vp, i32, i32, i32, vp, vp]
    L.pa_slot_mapping.restype = ctypes.c_int
    L.pa_reshape_and_cache.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, ctypes.c_int,
                                       ctypes.c_int, f32, f32, vp]
    L.pa_reshape_and_cache.restype = ctypes.c_int
    L.pa_reshape_and_cache_scales.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, ctypes.c_int,
                                              ctypes.c_int, vp, vp, vp]
    L.pa_reshape_and_cache_scales.restype = ctypes.c_int
    L.pa_append_kv.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, vp, i32, i32, i32, i32, ctypes.c_int,
                               ctypes.c_int, ctypes.c_float, ctypes.c_float, vp, vp, vp]
    L.pa_append_kv.restype = ctypes.c_int
    L.pa_copy_blocks.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, ctypes.c_int, vp]
    L.pa_copy_blocks.restype = ctypes.c_int
    L.pa_swap_blocks.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, ctypes.c_int, vp]
    L.pa_swap_blocks.restype = ctypes.c_int
    i32p = ctypes.POINTER(ctypes.c_int32)
    L.pa_bm_create.argtypes = [i32, i32, i32, vp]
    L.pa_bm_create.restype = vp
    L.pa_bm_destroy.argtypes = [vp]
    L.pa_bm_destroy.restype = None
    L.pa_bm_add.argtypes = [vp, vp, i32, i32p, i32p]
    L.pa_bm_add.restype = ctypes.c_int
    L.pa_bm_append.argtypes = [vp, i32, i32, i32p, i32p, i32p]
    L.pa_bm_append.restype = ctypes.c_int
    L.pa_bm_fork.argtypes = [vp, i32, i32p]
    L.pa_bm_fork.restype = ctypes.c_int
    L.pa_bm_free.argtypes = [vp, i32]
    L.pa_bm_free.restype = ctypes.c_int
    L.pa_bm_table.argtypes = [vp, i32, vp, i32]
    L.pa_bm_table.restype = i32
    for name in ("pa_bm_length",):
        getattr(L, name).argtypes = [vp, i32]
        getattr(L, name).restype = i32
    for name in ("pa_bm_free_blocks", "pa_bm_cached_blocks"):
        getattr(L, name).argtypes = [vp]
        getattr(L, name).restype = i32
    pargp = ctypes.POINTER(PrefillArgs)
    L.pa_prefill_check.argtypes = [pargp]
    L.pa_prefill_check.restype = ctypes.c_int
    L.pa_prefill.argtypes = [pargp, vp]
    L.pa_prefill.restype = ctypes.c_int
    L.pa_prefill_slot_mapping.argtypes = [vp, vp, vp, i32, i32, i32, i32, vp, vp]
    L.pa_prefill_slot_mapping.restype = ctypes.c_int
    L.pa_status_str.argtypes = [ctypes.c_int]
    L.pa_status_str.restype = ctypes.c_char_p
    L.pa_abi_version.argtypes = []
    L.pa_abi_version.restype = ctypes.c_int32
    _lib = L
    return L


def _check(status: int, what: str) -> None:
    if status != 0:
        raise PaError(status, what, lib().pa_status_str(status).decode())


def _ptr(t) -> int:
    return 0 if t is None else t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _pa_dtype(t: torch.Tensor, override=None) -> int:
    if override is not None:
        return DTYPE_NAMES[override] if isinstance(override, str) else int(override)
    return TORCH_TO_PA[t.dtype]


def _require(t: torch.Tensor, name: str, dtype=None, ndim=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU (the library has no CPU path)")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")


def _head_scales(args, k_scales, v_scales, Hkv):
    """Per-KV-head scale tensors (fp32 [Hkv] on the GPU) into args."""
    if k_scales is None and v_scales is None:
        return
    for t, n in ((k_scales, "k_scales"), (v_scales, "v_scales")):
        _require(t, n, torch.float32, 1)
        if t.shape[0] != Hkv:
            raise ValueError(f"{n} must hold one scale per KV head")
    args.k_scales, args.v_scales = k_scales.data_ptr(), v_scales.data_ptr()


def decode_args(out, q, k_cache, v_cache, block_tables, seq_lens, scale, k_scale=1.0, v_scale=1.0,
                partition_size=0, workspace=None, kv_dtype=None, k_scales=None,
                v_scales=None, combine=PA_COMBINE_AUTO) -> DecodeArgs:
    """Build ``pa_decode_args`` from tensors (shapes per include/pa.h)."""
    for t, n, nd in ((out, "out", 3), (q, "q", 3), (k_cache, "k_cache", 4), (v_cache, "v_cache", 4)):
        _require(t, n, ndim=nd)
    _require(block_tables, "block_tables", torch.int32, 2)
    _require(seq_lens, "seq_lens", torch.int32, 1)
    B, Hq, D = q.shape
    NB, bs, Hkv, Dk = k_cache.shape
    if tuple(v_cache.shape) != tuple(k_cache.shape) or Dk != D or tuple(out.shape) != (B, Hq, D):
        raise ValueError("inconsistent shapes")
    if block_tables.shape[0] != B or seq_lens.shape[0] != B:
        raise ValueError("block_tables / seq_lens batch mismatch")
    a = DecodeArgs()
    a.out, a.q, a.k_cache, a.v_cache = _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache)
    a.block_tables, a.seq_lens = _ptr(block_tables), _ptr(seq_lens)
    a.B, a.Hq, a.Hkv, a.D = B, Hq, Hkv, D
    a.block_size, a.num_blocks, a.max_blocks_per_seq = bs, NB, block_tables.shape[1]
    a.scale, a.k_scale, a.v_scale = float(scale), float(k_scale), float(v_scale)
    a.q_dtype = _pa_dtype(q)
    a.kv_dtype = _pa_dtype(k_cache, kv_dtype)
    a.out_dtype = _pa_dtype(out)
    a.partition_size = int(partition_size)
    a.combine = int(combine)
    _head_scales(a, k_scales, v_scales, Hkv)
    if workspace is not None:
        _require(workspace, "workspace")
        a.workspace, a.workspace_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    return a


def workspace_size(args: DecodeArgs) -> int:
    return int(lib().pa_decode_workspace_size(ctypes.byref(args)))


def partition_size(args: DecodeArgs) -> int:
    """Tokens per split-K partition the library uses for ``args``."""
    return int(lib().pa_decode_partition_size(ctypes.byref(args)))


def workspace_zero_bytes(args: DecodeArgs) -> int:
    """Bytes at the workspace's start that must be zero when a call starts."""
    return int(lib().pa_decode_workspace_zero_bytes(ctypes.byref(args)))


def alloc_workspace(args: DecodeArgs, device=None) -> torch.Tensor | None:
    """A zero-filled workspace tensor of the size ``pa_decode_workspace_size``
    asks for (or None).  Its arrival counters start at zero and every call
    leaves them zero, so the tensor serves any number of calls with these
    arguments' B and Hkv."""
    n = workspace_size(args)
    if n == 0:
        return None
    ws = torch.zeros(n, dtype=torch.uint8, device=device or "cuda")
    args.workspace, args.workspace_bytes = ws.data_ptr(), n
    return ws


def decode_check(args: DecodeArgs) -> int:
    return int(lib().pa_decode_check(ctypes.byref(args)))


def decode_run(args: DecodeArgs, stream=None) -> None:
    _check(lib().pa_decode(ctypes.byref(args), _stream(stream)), "pa_decode")


def decode_partition_run(args: DecodeArgs, stream=None) -> None:
    _check(lib().pa_decode_partition(ctypes.byref(args), _stream(stream)), "pa_decode_partition")


def decode_reduce_run(args: DecodeArgs, stream=None) -> None:
    _check(lib().pa_decode_reduce(ctypes.byref(args), _stream(stream)), "pa_decode_reduce")


def decode(out, q, k_cache, v_cache, block_tables, seq_lens, scale, k_scale=1.0, v_scale=1.0,
           partition_size=0, workspace=None, kv_dtype=None, stream=None, k_scales=None, v_scales=None,
           combine=PA_COMBINE_AUTO):
    """pa_decode on tensors; allocates the workspace with torch when none is given."""
    a = decode_args(out, q, k_cache, v_cache, block_tables, seq_lens, scale, k_scale, v_scale,
                    partition_size, workspace, kv_dtype, k_scales, v_scales, combine)
    keep = None
    if workspace is None:
        keep = alloc_workspace(a, q.device)
    decode_run(a, stream)
    return out, keep


def decode_no_alloc(out, q, k_cache, v_cache, block_tables, seq_lens, scale, k_scale=1.0,
                    v_scale=1.0, partition_size=0, kv_dtype=None, stream=None, k_scales=None,
                    v_scales=None, combine=PA_COMBINE_AUTO):
    """pa_decode_no_alloc on tensors: the library's own fixed workspace, nothing allocated."""
    a = decode_args(out, q, k_cache, v_cache, block_tables, seq_lens, scale, k_scale, v_scale,
                    partition_size, None, kv_dtype, k_scales, v_scales, combine)
    _check(lib().pa_decode_no_alloc(ctypes.byref(a), _stream(stream)), "pa_decode_no_alloc")
    return out


def slot_mapping(block_tables, positions, block_size, slots, stream=None):
    _require(block_tables, "block_tables", torch.int32, 2)
    _require(positions, "positions", torch.int32, 1)
    _require(slots, "slots", torch.int32, 1)
    B = positions.shape[0]
    if block_tables.shape[0] != B or slots.shape[0] != B:
        raise ValueError("batch mismatch")
    _check(lib().pa_slot_mapping(_ptr(block_tables), _ptr(positions), B, block_tables.shape[1],
                                 int(block_size), _ptr(slots), _stream(stream)), "pa_slot_mapping")
    return slots


def reshape_and_cache(k_new, v_new, k_cache, v_cache, slots, k_scale=1.0, v_scale=1.0,
                      kv_dtype=None, stream=None, k_scales=None, v_scales=None):
    """pa_reshape_and_cache, or pa_reshape_and_cache_scales when per-KV-head
    scale tensors (fp32 [Hkv] on the GPU) are given."""
    _require(k_new, "k_new", ndim=3)
    _require(v_new, "v_new", ndim=3)
    _require(k_cache, "k_cache", ndim=4)
    _require(v_cache, "v_cache", ndim=4)
    _require(slots, "slots", torch.int32, 1)
    T, Hkv, D = k_new.shape
    NB, bs, Hkv2, D2 = k_cache.shape
    if (Hkv2, D2) != (Hkv, D) or tuple(v_new.shape) != tuple(k_new.shape) or slots.shape[0] != T:
        raise ValueError("inconsistent shapes")
    if tuple(v_cache.shape) != tuple(k_cache.shape) or v_new.dtype != k_new.dtype:
        raise ValueError("K and V must match")
    if k_scales is not None or v_scales is not None:
        for t, n in ((k_scales, "k_scales"), (v_scales, "v_scales")):
            _require(t, n, torch.float32, 1)
            if t.shape[0] != Hkv:
                raise ValueError(f"{n} must hold one scale per KV head")
        _check(lib().pa_reshape_and_cache_scales(_ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
                                                 _ptr(slots), T, Hkv, D, bs, NB, _pa_dtype(k_new),
                                                 _pa_dtype(k_cache, kv_dtype), _ptr(k_scales),
                                                 _ptr(v_scales), _stream(stream)),
               "pa_reshape_and_cache_scales")
        return
    _check(lib().pa_reshape_and_cache(_ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
                                      _ptr(slots), T, Hkv, D, bs, NB, _pa_dtype(k_new),
                                      _pa_dtype(k_cache, kv_dtype), float(k_scale), float(v_scale),
                                      _stream(stream)), "pa_reshape_and_cache")


def append_kv(k_new, v_new, k_cache, v_cache, block_tables, positions, slots=None, k_scale=1.0,
              v_scale=1.0, kv_dtype=None, stream=None, k_scales=None, v_scales=None):
    """pa_append_kv: the slot mapping and the cache write of one new token per
    sequence in one launch; the slots go to ``slots`` when it is given."""
    _require(k_new, "k_new", ndim=3)
    _require(v_new, "v_new", ndim=3)
    _require(k_cache, "k_cache", ndim=4)
    _require(v_cache, "v_cache", ndim=4)
    _require(block_tables, "block_tables", torch.int32, 2)
    _require(positions, "positions", torch.int32, 1)
    B, Hkv, D = k_new.shape
    NB, bs, Hkv2, D2 = k_cache.shape
    if (Hkv2, D2) != (Hkv, D) or tuple(v_new.shape) != tuple(k_new.shape):
        raise ValueError("inconsistent shapes")
    if tuple(v_cache.shape) != tuple(k_cache.shape) or v_new.dtype != k_new.dtype:
        raise ValueError("K and V must match")
    if block_tables.shape[0] != B or positions.shape[0] != B:
        raise ValueError("batch mismatch")
    if slots is not None:
        _require(slots, "slots", torch.int32, 1)
        if slots.shape[0] != B:
            raise ValueError("batch mismatch")
    if (k_scales is None) != (v_scales is None):
        raise ValueError("per-head scales come in pairs")
    for t, n in ((k_scales, "k_scales"), (v_scales, "v_scales")):
        if t is not None:
            _require(t, n, torch.float32, 1)
            if t.shape[0] != Hkv:
                raise ValueError(f"{n} must hold one scale per KV head")
    _check(lib().pa_append_kv(_ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
                              _ptr(block_tables), _ptr(positions), B, block_tables.shape[1],
                              _ptr(slots) if slots is not None else None, Hkv, D, bs, NB,
                              _pa_dtype(k_new), _pa_dtype(k_cache, kv_dtype), float(k_scale),
                              float(v_scale), _ptr(k_scales) if k_scales is not None else None,
                              _ptr(v_scales) if v_scales is not None else None, _stream(stream)),
           "pa_append_kv")


def copy_blocks(k_cache, v_cache, block_mapping, kv_dtype=None, stream=None):
    _require(k_cache, "k_cache", ndim=4)
    _require(v_cache, "v_cache", ndim=4)
    _require(block_mapping, "block_mapping", torch.int32, 2)
    if block_mapping.shape[1] != 2 or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("block_mapping must be [P, 2] and K/V pools must match")
    NB, bs, Hkv, D = k_cache.shape
    _check(lib().pa_copy_blocks(_ptr(k_cache), _ptr(v_cache), _ptr(block_mapping),
                                block_mapping.shape[0], NB, bs, Hkv, D, _pa_dtype(k_cache, kv_dtype),
                                _stream(stream)), "pa_copy_blocks")


def prefill_args(out, q, k_cache, v_cache, block_tables, seq_lens, q_starts, max_q_len, scale,
                 k_scale=1.0, v_scale=1.0, kv_dtype=None, k_scales=None, v_scales=None) -> PrefillArgs:
    """Build ``pa_prefill_args`` from tensors (shapes per include/pa.h).
    ``max_q_len`` is a host integer: the most new tokens of any sequence."""
    for t, n, nd in ((out, "out", 3), (q, "q", 3), (k_cache, "k_cache", 4), (v_cache, "v_cache", 4)):
        _require(t, n, ndim=nd)
    _require(block_tables, "block_tables", torch.int32, 2)
    _require(seq_lens, "seq_lens", torch.int32, 1)
    _require(q_starts, "q_starts", torch.int32, 1)
    T, Hq, D = q.shape
    NB, bs, Hkv, Dk = k_cache.shape
    B = seq_lens.shape[0]
    if tuple(v_cache.shape) != tuple(k_cache.shape) or Dk != D or tuple(out.shape) != (T, Hq, D):
        raise ValueError("inconsistent shapes")
    if block_tables.shape[0] != B or q_starts.shape[0] != B + 1:
        raise ValueError("block_tables / q_starts batch mismatch")
    a = PrefillArgs()
    a.out, a.q, a.k_cache, a.v_cache = _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache)
    a.block_tables, a.seq_lens, a.q_starts = _ptr(block_tables), _ptr(seq_lens), _ptr(q_starts)
    a.B, a.T, a.max_q_len = B, T, int(max_q_len)
    a.Hq, a.Hkv, a.D = Hq, Hkv, D
    a.block_size, a.num_blocks, a.max_blocks_per_seq = bs, NB, block_tables.shape[1]
    a.scale, a.k_scale, a.v_scale = float(scale), float(k_scale), float(v_scale)
    a.q_dtype = _pa_dtype(q)
    a.kv_dtype = _pa_dtype(k_cache, kv_dtype)
    a.out_dtype = _pa_dtype(out)
    _head_scales(a, k_scales, v_scales, Hkv)
    return a


def prefill_check(args: PrefillArgs) -> int:
    return int(lib().pa_prefill_check(ctypes.byref(args)))


def prefill_run(args: PrefillArgs, stream=None) -> None:
    _check(lib().pa_prefill(ctypes.byref(args), _stream(stream)), "pa_prefill")


def prefill(out, q, k_cache, v_cache, block_tables, seq_lens, q_starts, max_q_len, scale,
            k_scale=1.0, v_scale=1.0, kv_dtype=None, stream=None, k_scales=None, v_scales=None):
    """pa_prefill on tensors."""
    prefill_run(prefill_args(out, q, k_cache, v_cache, block_tables, seq_lens, q_starts, max_q_len,
                             scale, k_scale, v_scale, kv_dtype, k_scales, v_scales), stream)
    return out


def prefill_slot_mapping(block_tables, seq_lens, q_starts, block_size, slots, stream=None):
    _require(block_tables, "block_tables", torch.int32, 2)
    _require(seq_lens, "seq_lens", torch.int32, 1)
    _require(q_starts, "q_starts", torch.int32, 1)
    _require(slots, "slots", torch.int32, 1)
    B = seq_lens.shape[0]
    if block_tables.shape[0] != B or q_starts.shape[0] != B + 1:
        raise ValueError("batch mismatch")
    _check(lib().pa_prefill_slot_mapping(_ptr(block_tables), _ptr(seq_lens), _ptr(q_starts), B,
                                         slots.shape[0], block_tables.shape[1], int(block_size),
                                         _ptr(slots), _stream(stream)), "pa_prefill_slot_mapping")
    return slots


def swap_blocks(src_k, src_v, dst_k, dst_v, block_mapping, kv_dtype=None, stream=None):
    """pa_swap_blocks: whole blocks from the source pools to the destination
    pools.  Each pool is a device tensor or a pinned host tensor
    (``pin_memory=True``); the mapping lives on the GPU."""
    for t, n in ((src_k, "src_k"), (src_v, "src_v"), (dst_k, "dst_k"), (dst_v, "dst_v")):
        if not isinstance(t, torch.Tensor) or t.dim() != 4 or not t.is_contiguous():
            raise ValueError(f"{n} must be a contiguous 4-d tensor")
        if not (t.is_cuda or t.is_pinned()):
            raise ValueError(f"{n} must be on the GPU or in pinned host memory")
    _require(block_mapping, "block_mapping", torch.int32, 2)
    if block_mapping.shape[1] != 2:
        raise ValueError("block_mapping must be [P, 2]")
    if src_k.shape != src_v.shape or dst_k.shape != dst_v.shape or src_k.shape[1:] != dst_k.shape[1:]:
        raise ValueError("pools must share the block shape [block_size, Hkv, D]")
    if not (src_k.dtype == src_v.dtype == dst_k.dtype == dst_v.dtype):
        raise ValueError("pools must share the dtype")
    NBs, bs, Hkv, D = src_k.shape
    _check(lib().pa_swap_blocks(_ptr(src_k), _ptr(src_v), _ptr(dst_k), _ptr(dst_v), _ptr(block_mapping),
                                block_mapping.shape[0], NBs, dst_k.shape[0], bs, Hkv, D,
                                _pa_dtype(src_k, kv_dtype), _stream(stream)), "pa_swap_blocks")


class OutOfBlocks(PaError):
    """The block manager has no free or evictable block; nothing changed."""


class BlockManager:
    """The library's host block manager with prefix caching (pa_bm_* in
    include/pa.h): argument marshalling only, all bookkeeping is native."""

    def __init__(self, num_blocks: int, block_size: int, prefix_caching: bool = True, free_order=None):
        import numpy as np
        self._lib = lib()
        self.block_size = int(block_size)
        self._order = None if free_order is None else np.ascontiguousarray(free_order, dtype=np.int32)
        ptr = None if self._order is None else self._order.ctypes.data
        self._h = self._lib.pa_bm_create(int(num_blocks), int(block_size), int(bool(prefix_caching)), ptr)
        if not self._h:
            raise ValueError("invalid block manager arguments")

    def close(self):
        if self._h:
            self._lib.pa_bm_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def _st(self, status, what):
        if status == PA_ERR_OUT_OF_BLOCKS:
            raise OutOfBlocks(status, what, "no free or evictable block")
        _check(status, what)

    def add(self, tokens):
        """Admit a prompt; returns (sequence id, cached tokens)."""
        import numpy as np
        t = np.ascontiguousarray(tokens, dtype=np.int32)
        sid, cached = ctypes.c_int32(), ctypes.c_int32()
        self._st(self._lib.pa_bm_add(self._h, t.ctypes.data if t.size else None, int(t.size),
                                     ctypes.byref(sid), ctypes.byref(cached)), "pa_bm_add")
        return sid.value, cached.value

    def append(self, seq: int, token: int):
        """Append a token; returns (slot, (src, dst) copy or None)."""
        slot, src, dst = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
        self._st(self._lib.pa_bm_append(self._h, int(seq), int(token), ctypes.byref(slot),
                                        ctypes.byref(src), ctypes.byref(dst)), "pa_bm_append")
        return slot.value, (None if src.value < 0 else (src.value, dst.value))

    def fork(self, seq: int) -> int:
        out = ctypes.c_int32()
        self._st(self._lib.pa_bm_fork(self._h, int(seq), ctypes.byref(out)), "pa_bm_fork")
        return out.value

    def free(self, seq: int) -> None:
        self._st(self._lib.pa_bm_free(self._h, int(seq)), "pa_bm_free")

    def table(self, seq: int) -> list:
        n = self._lib.pa_bm_table(self._h, int(seq), None, 0)
        if n < 0:
            raise KeyError(seq)
        buf = (ctypes.c_int32 * max(n, 1))()
        self._lib.pa_bm_table(self._h, int(seq), buf, n)
        return list(buf[:n])

    def length(self, seq: int) -> int:
        return int(self._lib.pa_bm_length(self._h, int(seq)))

    def free_blocks(self) -> int:
        return int(self._lib.pa_bm_free_blocks(self._h))

    def cached_blocks(self) -> int:
        return int(self._lib.pa_bm_cached_blocks(self._h))


def read_blocks(pool, piece_bytes, ids, sink, stream=None):
    """pa_read_blocks: read pieces ``ids`` of ``pool`` (a flat uint8 tensor of
    whole pieces) into the fold ``sink`` (int32); a measurement utility."""
    _require(pool, "pool", torch.uint8, 1)
    _require(ids, "ids", torch.int32, 1)
    _require(sink, "sink", torch.int32, 1)
    if pool.numel() % piece_bytes:
        raise ValueError("the pool must hold whole pieces")
    _check(lib().pa_read_blocks(_ptr(pool), pool.numel() // piece_bytes, piece_bytes, _ptr(ids),
                                ids.shape[0], _ptr(sink), sink.shape[0], _stream(stream)),
           "pa_read_blocks")
