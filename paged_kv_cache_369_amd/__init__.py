"""paged_kv_cache_369_amd -- paged-KV-cache decode attention for AMD MI355X (gfx950).

Thin ctypes binding over the C ABI in ``include/pkv.h`` (library
``libpkv.so`` next to this file).  The functions carry the C names, take torch
tensors that already live on the GPU, and only marshal arguments: every step
of the computation runs in the library's HIP kernels on torch's current
stream.  There is no CPU fallback: if the library is missing the first call
raises.

    paged_kv_write(k_new, v_new, k_cache, v_cache, slot_mapping, k_scale=1, v_scale=1)
    paged_attention_decode(out, q, k_cache, v_cache, block_table, context_lens, scale, ...)
    paged_attention_workspace_bytes(num_seqs, num_heads, head_dim, max_blocks_per_seq, ...)

Layouts: new tokens ``[T, H_kv, D]``; K pool ``[num_blocks, H_kv, D // X,
16, X]`` with ``X = 16 // element bytes`` (each token row as 16-byte chunks
of consecutive dimensions, chunk-major), V pool ``[num_blocks, H_kv, D, 16]``
(dimension-major) -- see ``k_cache_shape`` / ``v_cache_shape``; fp8 pools as
``torch.uint8`` or ``torch.float8_e4m3fn``; ``q`` and ``out`` ``[B, H_q, D]``;
``block_table`` ``[B, max_blocks]`` int32 (-1 padded); ``context_lens``
``[B]`` int32; ``slot_mapping`` ``[T]`` int32 (-1 = skip).
"""
from __future__ import annotations

import ctypes
import os
import threading

__all__ = ["paged_kv_write", "paged_attention_decode", "paged_attention_workspace_bytes", "pkv_check_inputs",
           "paged_attention_decode_noalloc", "paged_attention_decode_cascade", "prepare",
           "BlockManager", "paged_kv_copy_blocks", "paged_attention_varlen", "paged_attention_prefill",
           "pkv_abi_version", "pkv_stream_read", "pkv_tile_read", "PkvError", "library_path", "BLOCK_SIZE", "k_cache_shape", "v_cache_shape"]

BLOCK_SIZE = 16
_ELT = {"f32": 4, "bf16": 2, "fp8": 1}
_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libpkv.so")
_lib = None


class PkvError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{msg} (pkv status {status})")
        self.status = status


def library_path() -> str:
    return _LIB_PATH


_RECORDING = threading.local()  # prepare(): this thread's recorder, which stands in for the library


def _load():
    global _lib
    rec = getattr(_RECORDING, "lib", None)
    if rec is not None:
        return rec
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"HIP library {_LIB_PATH} is not built; run `python -m paged_kv_cache_369_amd.build`")
    lib = ctypes.CDLL(_LIB_PATH)
    p, i32, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    lib.pkv_abi_version.restype = ctypes.c_int
    lib.pkv_status_string.argtypes = [ctypes.c_int]
    lib.pkv_status_string.restype = ctypes.c_char_p
    lib.paged_kv_write.argtypes = [p, p, ctypes.c_int, p, p, ctypes.c_int, p, i32, i32, i32, i32, i32, f32, f32, p]
    lib.paged_kv_write.restype = ctypes.c_int
    lib.paged_attention_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32, i32]
    lib.paged_attention_workspace_bytes.restype = sz
    lib.paged_attention_decode.argtypes = [p, p, ctypes.c_int, p, p, ctypes.c_int, p, i32, p,
                                           i32, i32, i32, i32, i32, i32, f32, f32, f32, i32, p, sz, p]
    lib.paged_attention_decode.restype = ctypes.c_int
    lib.paged_attention_decode_noalloc.argtypes = [p, p, ctypes.c_int, p, p, ctypes.c_int, p, i32, p,
                                                   i32, i32, i32, i32, i32, i32, f32, f32, f32, i32, p]
    lib.paged_attention_decode_noalloc.restype = ctypes.c_int
    lib.paged_attention_cascade_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32, i32]
    lib.paged_attention_cascade_workspace_bytes.restype = sz
    lib.paged_attention_decode_cascade.argtypes = [p, p, ctypes.c_int, p, p, ctypes.c_int, p, i32, p, p, p,
                                                   i32, i32, i32, i32, i32, i32, f32, f32, f32, i32, p, sz, p]
    lib.paged_attention_decode_cascade.restype = ctypes.c_int
    lib.paged_attention_varlen_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32, i32]
    lib.paged_attention_varlen_workspace_bytes.restype = sz
    lib.paged_attention_varlen.argtypes = [p, p, ctypes.c_int, p, i32, p, p, ctypes.c_int, p, i32, p,
                                           i32, i32, i32, i32, i32, i32, f32, f32, f32, i32, p, sz, p]
    lib.paged_attention_varlen.restype = ctypes.c_int
    lib.paged_attention_prefill.argtypes = [p, p, ctypes.c_int, p, i32, i32, p, p, ctypes.c_int, p, i32, p,
                                            i32, i32, i32, i32, i32, i32, f32, f32, f32, p]
    lib.paged_attention_prefill.restype = ctypes.c_int
    lib.pkv_stream_read.argtypes = [p, sz, p, p]
    lib.pkv_stream_read.restype = ctypes.c_int
    lib.pkv_tile_read.argtypes = [p, p, p, i32, i32, i32, i32, i32, p, p]
    lib.pkv_tile_read.restype = ctypes.c_int
    lib.pkv_check_inputs.argtypes = [p, i32, p, i32, p, i32, i32, p, p]
    lib.pkv_check_inputs.restype = ctypes.c_int
    i64 = ctypes.c_int64
    lib.pkv_bm_create.argtypes = [i32, i32]
    lib.pkv_bm_create.restype = p
    lib.pkv_bm_destroy.argtypes = [p]
    lib.pkv_bm_destroy.restype = None
    for name in ("pkv_bm_add", "pkv_bm_free"):
        getattr(lib, name).argtypes = [p, i64]
        getattr(lib, name).restype = ctypes.c_int
    lib.pkv_bm_fork.argtypes = [p, i64, i64]
    lib.pkv_bm_fork.restype = ctypes.c_int
    lib.pkv_bm_append.argtypes = [p, i64, i32, p]
    lib.pkv_bm_append.restype = ctypes.c_int
    lib.pkv_bm_table.argtypes = [p, p, i32, i32, p, p]
    lib.pkv_bm_table.restype = ctypes.c_int
    lib.pkv_bm_take_copies.argtypes = [p, p, p, i32]
    lib.pkv_bm_take_copies.restype = i32
    lib.pkv_bm_stats.argtypes = [p, p]
    lib.pkv_bm_stats.restype = ctypes.c_int
    lib.pkv_bm_enable_prefix_caching.argtypes = [p]
    lib.pkv_bm_enable_prefix_caching.restype = ctypes.c_int
    lib.pkv_bm_add_prompt.argtypes = [p, i64, p, i32, p, p]
    lib.pkv_bm_add_prompt.restype = ctypes.c_int
    lib.pkv_bm_append_tokens.argtypes = [p, i64, p, i32, p]
    lib.pkv_bm_append_tokens.restype = ctypes.c_int
    lib.pkv_bm_cache_stats.argtypes = [p, p]
    lib.pkv_bm_cache_stats.restype = ctypes.c_int
    lib.paged_kv_copy_blocks.argtypes = [p, p, ctypes.c_int, i32, i32, i32, i32, p, p, i32, p]
    lib.paged_kv_copy_blocks.restype = ctypes.c_int
    _lib = lib
    return lib


def pkv_abi_version() -> int:
    return _load().pkv_abi_version()


def k_cache_shape(num_blocks: int, num_kv_heads: int, head_dim: int, dtype: str):
    """Shape of a K pool: [num_blocks, H_kv, D // X, 16, X], X = 16 // element bytes ("f32", "bf16", "fp8")."""
    x = 16 // _ELT[dtype]
    return (num_blocks, num_kv_heads, head_dim // x, BLOCK_SIZE, x)


def v_cache_shape(num_blocks: int, num_kv_heads: int, head_dim: int, dtype: str = ""):
    """Shape of a V pool: [num_blocks, H_kv, D, 16]."""
    return (num_blocks, num_kv_heads, head_dim, BLOCK_SIZE)


def _pools(k_cache, v_cache):
    """(num_blocks, H_kv, head_dim) of a K/V pool pair, checking both layouts."""
    if k_cache.dim() != 5 or v_cache.dim() != 4:
        raise ValueError("K pool must be [NB, H, D//X, 16, X] and V pool [NB, H, D, 16]")
    NB, H, nc, BS, X = k_cache.shape
    D = nc * X
    if X * k_cache.element_size() != 16 or BS != BLOCK_SIZE:
        raise ValueError("K pool chunks must be 16 bytes of 16-token blocks")
    if tuple(v_cache.shape) != (NB, H, D, BLOCK_SIZE) or v_cache.dtype != k_cache.dtype:
        raise ValueError("V pool shape/dtype does not match the K pool")
    return NB, H, D


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return 0
    if t.dtype == torch.bfloat16:
        return 1
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return 2
    raise TypeError(f"unsupported dtype {t.dtype}")


def _dev(t, name):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check(status: int, what: str):
    if status != 0:
        raise PkvError(status, f"{what}: {_load().pkv_status_string(status).decode()}")


# The C entry points that launch work on a stream (the rest answer queries).
_LAUNCHES = ("paged_kv_write", "paged_attention_decode", "paged_attention_decode_noalloc",
             "paged_attention_decode_cascade", "paged_attention_varlen", "paged_attention_prefill",
             "paged_kv_copy_blocks", "pkv_stream_read")


def prepare(call, *args, **kwargs):
    """Marshal the arguments of one launching binding call once; return a function that launches it again.

    `call` is one of this module's launching functions (paged_kv_write, paged_attention_decode, ...), with
    the arguments it would take.  Its checks and argument marshalling run here, once, and its C call is
    recorded instead of made; the returned function makes that C call (same tensors, scalars, workspace
    and stream) and checks its status.  The tensors stay referenced by the returned function.  This is for
    launch loops, such as one decode step per generated token, where Python's per-call marshalling would
    otherwise keep the GPU waiting."""
    real = _load()
    rec = []

    class _Recorder:
        def __getattr__(self, name):
            fn = getattr(real, name)
            if name not in _LAUNCHES:
                return fn

            def record(*a):
                rec.append((name, fn, a))
                return 0
            return record

    _RECORDING.lib = _Recorder()  # the call below looks the library up through _load, in this thread
    try:
        call(*args, **kwargs)
    finally:
        _RECORDING.lib = None
    if len(rec) != 1:
        raise ValueError(f"{getattr(call, '__name__', call)} made {len(rec)} launching calls; prepare needs one")
    name, fn, cargs = rec[0]

    def launch():
        st = fn(*cargs)
        if st != 0:
            _check(st, name)

    launch.keep_alive = (args, kwargs)
    return launch


def paged_kv_write(k_new, v_new, k_cache, v_cache, slot_mapping, k_scale: float = 1.0, v_scale: float = 1.0,
                   stream=None) -> None:
    """Store new tokens' K/V at their slots (copy, or quantise into an fp8 pool)."""
    lib = _load()
    T, H, D = k_new.shape
    NB, Hc, Dc = _pools(k_cache, v_cache)
    if (Hc, Dc) != (H, D) or v_new.shape != k_new.shape:
        raise ValueError("shape mismatch between new tokens and pools")
    if slot_mapping.shape != (T,):
        raise ValueError("slot_mapping must be [num_tokens]")
    st = lib.paged_kv_write(_dev(k_new, "k_new"), _dev(v_new, "v_new"), _dtype_code(k_new),
                            _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), _dtype_code(k_cache),
                            _dev(slot_mapping, "slot_mapping"), T, H, D, BLOCK_SIZE, NB,
                            float(k_scale), float(v_scale), _stream(stream))
    _check(st, "paged_kv_write")


def paged_attention_workspace_bytes(num_seqs: int, num_heads: int, num_kv_heads: int, head_dim: int,
                                    max_blocks_per_seq: int, block_size: int = BLOCK_SIZE,
                                    partition_size: int = 0) -> int:
    return int(_load().paged_attention_workspace_bytes(num_seqs, num_heads, num_kv_heads, head_dim,
                                                       max_blocks_per_seq, block_size, partition_size))


_WORKSPACES = {}


def _default_workspace(device, need: int, stream=None):
    """A zero-filled workspace per (device, stream), grown on demand.

    It is allocated and zero-filled on the stream the call runs on, so the
    fill is ordered before the kernel that first reads it, and the caching
    allocator keeps the memory for that stream (a buffer dropped when the
    workspace grows is reused only by later work on the same stream).  The
    decode leaves its counters at zero, so the buffer is reused without
    clearing.  Calls on different streams get different buffers."""
    import torch
    s = torch.cuda.current_stream(device) if stream is None else stream
    key = (device.type, device.index, int(s.cuda_stream))
    ws = _WORKSPACES.get(key)
    if ws is None or ws.numel() < need:
        with torch.cuda.stream(s):
            ws = torch.zeros(need, dtype=torch.uint8, device=device)
        _WORKSPACES[key] = ws
    return ws


def paged_attention_decode(out, q, k_cache, v_cache, block_table, context_lens, scale: float,
                           k_scale: float = 1.0, v_scale: float = 1.0, partition_size: int = 0,
                           workspace=None, stream=None) -> None:
    """out[s, h] = softmax(scale * q[s, h] . K_s^T) V_s over the paged context of sequence s.

    workspace: uint8 device tensor of at least paged_attention_workspace_bytes(...)
    bytes, zero-filled before its first use (torch.zeros); None uses a buffer
    the binding keeps per (device, stream), allocated and zeroed on that stream."""
    import torch
    lib = _load()
    B, Hq, D = q.shape
    NB, Hkv, Dc = _pools(k_cache, v_cache)
    if out.shape != q.shape or Dc != D:
        raise ValueError("shape mismatch")
    if block_table.dim() != 2 or block_table.shape[0] != B or context_lens.shape != (B,):
        raise ValueError("block_table must be [B, max_blocks] and context_lens [B]")
    MB = block_table.shape[1]
    need = paged_attention_workspace_bytes(B, Hq, Hkv, D, MB, BLOCK_SIZE, partition_size)
    if workspace is None and need > 0:
        workspace = _default_workspace(q.device, need, stream)
    ws_ptr = _dev(workspace, "workspace") if workspace is not None else ctypes.c_void_p(0)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = lib.paged_attention_decode(_dev(out, "out"), _dev(q, "q"), _dtype_code(q),
                                    _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), _dtype_code(k_cache),
                                    _dev(block_table, "block_table"), MB, _dev(context_lens, "context_lens"),
                                    B, Hq, Hkv, D, BLOCK_SIZE, NB, float(scale), float(k_scale), float(v_scale),
                                    int(partition_size), ws_ptr, ws_bytes, _stream(stream))
    _check(st, "paged_attention_decode")


NOALLOC_SCRATCH_BYTES = 32 << 20  # PKV_NOALLOC_SCRATCH_BYTES


def paged_attention_decode_noalloc(out, q, k_cache, v_cache, block_table, context_lens, scale: float,
                                   k_scale: float = 1.0, v_scale: float = 1.0, partition_size: int = 0,
                                   stream=None) -> None:
    """paged_attention_decode with the library's static per-GPU scratch as its workspace: no workspace
    argument and no allocation (see include/pkv.h).  Calls that overlap on one GPU race."""
    lib = _load()
    B, Hq, D = q.shape
    NB, Hkv, Dc = _pools(k_cache, v_cache)
    if out.shape != q.shape or Dc != D:
        raise ValueError("shape mismatch")
    if block_table.dim() != 2 or block_table.shape[0] != B or context_lens.shape != (B,):
        raise ValueError("block_table must be [B, max_blocks] and context_lens [B]")
    MB = block_table.shape[1]
    st = lib.paged_attention_decode_noalloc(_dev(out, "out"), _dev(q, "q"), _dtype_code(q),
                                            _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
                                            _dtype_code(k_cache), _dev(block_table, "block_table"), MB,
                                            _dev(context_lens, "context_lens"), B, Hq, Hkv, D, BLOCK_SIZE, NB,
                                            float(scale), float(k_scale), float(v_scale), int(partition_size),
                                            _stream(stream))
    _check(st, "paged_attention_decode_noalloc")


def paged_attention_cascade_workspace_bytes(num_seqs: int, num_heads: int, num_kv_heads: int, head_dim: int,
                                            max_blocks_per_seq: int, block_size: int = BLOCK_SIZE,
                                            partition_size: int = 0) -> int:
    return int(_load().paged_attention_cascade_workspace_bytes(num_seqs, num_heads, num_kv_heads, head_dim,
                                                               max_blocks_per_seq, block_size, partition_size))


def paged_attention_decode_cascade(out, q, k_cache, v_cache, block_table, context_lens, prefix_leader,
                                   prefix_blocks, scale: float, k_scale: float = 1.0, v_scale: float = 1.0,
                                   partition_size: int = 0, workspace=None, stream=None) -> None:
    """paged_attention_decode's result, with each shared prefix read once per chunk of sequences sharing it.

    prefix_leader, prefix_blocks: int32 [B] device tensors (see include/pkv.h): the first sequence of each
    sequence's sharing group (consecutive sequences) and the leading blocks the group shares."""
    lib = _load()
    B, Hq, D = q.shape
    NB, Hkv, Dc = _pools(k_cache, v_cache)
    if out.shape != q.shape or Dc != D:
        raise ValueError("shape mismatch")
    if block_table.dim() != 2 or block_table.shape[0] != B or context_lens.shape != (B,):
        raise ValueError("block_table must be [B, max_blocks] and context_lens [B]")
    if prefix_leader.shape != (B,) or prefix_blocks.shape != (B,):
        raise ValueError("prefix_leader and prefix_blocks must be [B]")
    MB = block_table.shape[1]
    need = paged_attention_cascade_workspace_bytes(B, Hq, Hkv, D, MB, BLOCK_SIZE, partition_size)
    if workspace is None and need > 0:
        workspace = _default_workspace(q.device, need, stream)
    ws_ptr = _dev(workspace, "workspace") if workspace is not None else ctypes.c_void_p(0)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = lib.paged_attention_decode_cascade(_dev(out, "out"), _dev(q, "q"), _dtype_code(q),
                                            _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
                                            _dtype_code(k_cache), _dev(block_table, "block_table"), MB,
                                            _dev(context_lens, "context_lens"), _dev(prefix_leader, "prefix_leader"),
                                            _dev(prefix_blocks, "prefix_blocks"), B, Hq, Hkv, D, BLOCK_SIZE, NB,
                                            float(scale), float(k_scale), float(v_scale), int(partition_size),
                                            ws_ptr, ws_bytes, _stream(stream))
    _check(st, "paged_attention_decode_cascade")


def paged_attention_varlen_workspace_bytes(num_seqs: int, num_heads: int, num_kv_heads: int, head_dim: int,
                                           max_blocks_per_seq: int, block_size: int = BLOCK_SIZE,
                                           partition_size: int = 0) -> int:
    return int(_load().paged_attention_varlen_workspace_bytes(num_seqs, num_heads, num_kv_heads, head_dim,
                                                              max_blocks_per_seq, block_size, partition_size))


def paged_attention_varlen(out, q, cu_seqlens_q, k_cache, v_cache, block_table, context_lens, scale: float,
                           k_scale: float = 1.0, v_scale: float = 1.0, partition_size: int = 0, workspace=None,
                           stream=None) -> None:
    """Several new query tokens per sequence: q and out are [T, H, D] (rows grouped by sequence through
    cu_seqlens_q [B + 1]); row i of sequence s attends causally to its first L_s - n_s + i + 1 cached tokens."""
    lib = _load()
    T, Hq, D = q.shape
    NB, Hkv, Dc = _pools(k_cache, v_cache)
    if out.shape != q.shape or Dc != D:
        raise ValueError("shape mismatch")
    B = context_lens.shape[0]
    if block_table.dim() != 2 or block_table.shape[0] != B or cu_seqlens_q.shape != (B + 1,):
        raise ValueError("block_table must be [B, max_blocks] and cu_seqlens_q [B + 1]")
    MB = block_table.shape[1]
    need = paged_attention_varlen_workspace_bytes(B, Hq, Hkv, D, MB, BLOCK_SIZE, partition_size)
    if workspace is None and need > 0:
        workspace = _default_workspace(q.device, need, stream)
    ws_ptr = _dev(workspace, "workspace") if workspace is not None else ctypes.c_void_p(0)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = lib.paged_attention_varlen(_dev(out, "out"), _dev(q, "q"), _dtype_code(q), _dev(cu_seqlens_q, "cu_seqlens_q"),
                                    T, _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), _dtype_code(k_cache),
                                    _dev(block_table, "block_table"), MB, _dev(context_lens, "context_lens"),
                                    B, Hq, Hkv, D, BLOCK_SIZE, NB, float(scale), float(k_scale), float(v_scale),
                                    int(partition_size), ws_ptr, ws_bytes, _stream(stream))
    _check(st, "paged_attention_varlen")


def paged_attention_prefill(out, q, cu_seqlens_q, k_cache, v_cache, block_table, context_lens, scale: float,
                            max_q_len: int, k_scale: float = 1.0, v_scale: float = 1.0, stream=None) -> None:
    """The result of paged_attention_varlen, computed 32 query columns per wave (long chunks of new
    tokens).  max_q_len bounds any sequence's new-token count; no workspace."""
    lib = _load()
    T, Hq, D = q.shape
    NB, Hkv, Dc = _pools(k_cache, v_cache)
    if out.shape != q.shape or Dc != D:
        raise ValueError("shape mismatch")
    B = context_lens.shape[0]
    if block_table.dim() != 2 or block_table.shape[0] != B or cu_seqlens_q.shape != (B + 1,):
        raise ValueError("block_table must be [B, max_blocks] and cu_seqlens_q [B + 1]")
    MB = block_table.shape[1]
    st = lib.paged_attention_prefill(_dev(out, "out"), _dev(q, "q"), _dtype_code(q), _dev(cu_seqlens_q, "cu_seqlens_q"),
                                     T, int(max_q_len), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
                                     _dtype_code(k_cache), _dev(block_table, "block_table"), MB,
                                     _dev(context_lens, "context_lens"), B, Hq, Hkv, D, BLOCK_SIZE, NB, float(scale),
                                     float(k_scale), float(v_scale), _stream(stream))
    _check(st, "paged_attention_prefill")


STREAM_SINK_WORDS = 8192  # PKV_STREAM_SINK_WORDS in include/pkv.h


def pkv_stream_read(buf, sink, stream=None) -> None:
    """A plain streaming read of a device tensor (measurement aid); sink: int32 device tensor of
    >= STREAM_SINK_WORDS elements."""
    lib = _load()
    if sink.numel() * sink.element_size() < 4 * STREAM_SINK_WORDS:
        raise ValueError(f"sink needs {STREAM_SINK_WORDS} 32-bit words")
    st = lib.pkv_stream_read(_dev(buf, "buf"), buf.numel() * buf.element_size(), _dev(sink, "sink"), _stream(stream))
    _check(st, "pkv_stream_read")


TILE_SINK_WORDS = 2048  # PKV_TILE_SINK_WORDS


def pkv_tile_read(k, v, ids, num_tiles: int, tile_bytes: int, v_load_bytes: int, depth: int, sink,
                  stream=None) -> None:
    """The decode's read pattern without its arithmetic (see include/pkv.h): the K then V tile of each entry
    of `ids` from the byte pools `k` and `v` (num_tiles tiles each), V read by v_load_bytes-byte loads."""
    import torch
    lib = _load()
    if ids.dtype != torch.int32:
        raise TypeError("ids must be int32")
    if sink.numel() * sink.element_size() < 4 * TILE_SINK_WORDS:
        raise ValueError(f"sink must hold {TILE_SINK_WORDS} 32-bit words")
    for name, t in (("k", k), ("v", v)):
        if t.numel() * t.element_size() < int(num_tiles) * int(tile_bytes):
            raise ValueError(f"{name} holds fewer than num_tiles tiles of tile_bytes")
    st = lib.pkv_tile_read(_dev(k, "k"), _dev(v, "v"), _dev(ids, "ids"), ids.numel(), int(num_tiles),
                           int(tile_bytes), int(v_load_bytes), int(depth), _dev(sink, "sink"), _stream(stream))
    _check(st, "pkv_tile_read")


def pkv_check_inputs(num_blocks: int, block_table=None, context_lens=None, slot_mapping=None, stream=None):
    """Counts of invalid index-array contents (see include/pkv.h), read back after the launch:
    (bad context lengths, bad table entries, bad slots, repeated slots)."""
    import torch
    dev = next((t.device for t in (block_table, context_lens, slot_mapping) if t is not None), None)
    if dev is None:
        raise ValueError("pass at least one of block_table/context_lens, slot_mapping")
    counts = torch.empty(4, dtype=torch.int32, device=dev)
    B = int(context_lens.shape[0]) if context_lens is not None else 0
    MB = int(block_table.shape[1]) if block_table is not None else 0
    T = int(slot_mapping.shape[0]) if slot_mapping is not None else 0
    none = ctypes.c_void_p(0)
    st = _load().pkv_check_inputs(_dev(block_table, "block_table") if block_table is not None else none, MB,
                                  _dev(context_lens, "context_lens") if context_lens is not None else none, B,
                                  _dev(slot_mapping, "slot_mapping") if slot_mapping is not None else none, T,
                                  int(num_blocks), _dev(counts, "counts"), _stream(stream))
    _check(st, "pkv_check_inputs")
    if stream is not None:
        stream.synchronize()  # the counts are written on `stream`; .cpu() below waits on torch's current one
    return tuple(int(x) for x in counts.cpu().tolist())


class BlockManager:
    """The library's host block manager (see include/pkv.h): blocks handed out on demand, sequences forked
    with shared blocks, copy-on-write of a shared partly filled last block.  Host numpy arrays in and out."""

    def __init__(self, num_blocks: int, max_blocks_per_seq: int):
        import numpy as np  # noqa: F401  (used by the methods)
        self._lib = _load()
        self._h = self._lib.pkv_bm_create(int(num_blocks), int(max_blocks_per_seq))
        if not self._h:
            raise PkvError(1, "pkv_bm_create")
        self.num_blocks, self.max_blocks_per_seq = int(num_blocks), int(max_blocks_per_seq)

    def close(self):
        if self._h:
            self._lib.pkv_bm_destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()

    def add(self, seq: int):
        _check(self._lib.pkv_bm_add(self._h, int(seq)), "pkv_bm_add")

    def fork(self, parent: int, child: int):
        _check(self._lib.pkv_bm_fork(self._h, int(parent), int(child)), "pkv_bm_fork")

    def append(self, seq: int, n: int):
        import numpy as np
        slots = np.empty(max(int(n), 1), dtype=np.int32)
        _check(self._lib.pkv_bm_append(self._h, int(seq), int(n), slots.ctypes.data), "pkv_bm_append")
        return slots[: int(n)]

    def free(self, seq: int):
        _check(self._lib.pkv_bm_free(self._h, int(seq)), "pkv_bm_free")

    def enable_prefix_caching(self):
        _check(self._lib.pkv_bm_enable_prefix_caching(self._h), "pkv_bm_enable_prefix_caching")

    def add_prompt(self, seq: int, tokens):
        """New sequence with its prompt token ids -> (slots of the tokens to compute, tokens reused)."""
        import numpy as np
        tok = np.ascontiguousarray(tokens, dtype=np.int32)
        slots = np.empty(max(len(tok), 1), dtype=np.int32)
        cached = ctypes.c_int32(0)
        _check(self._lib.pkv_bm_add_prompt(self._h, int(seq), tok.ctypes.data, len(tok), slots.ctypes.data,
                                           ctypes.byref(cached)), "pkv_bm_add_prompt")
        return slots[:len(tok) - cached.value].copy(), cached.value

    def append_tokens(self, seq: int, tokens):
        import numpy as np
        tok = np.ascontiguousarray(tokens, dtype=np.int32)
        slots = np.empty(max(len(tok), 1), dtype=np.int32)
        _check(self._lib.pkv_bm_append_tokens(self._h, int(seq), tok.ctypes.data, len(tok), slots.ctypes.data),
               "pkv_bm_append_tokens")
        return slots[:len(tok)].copy()

    def cache_stats(self):
        """(registered blocks, evictable blocks, prompt blocks looked up, reused, evictions)"""
        import numpy as np
        out = np.zeros(5, dtype=np.int64)
        _check(self._lib.pkv_bm_cache_stats(self._h, out.ctypes.data), "pkv_bm_cache_stats")
        return tuple(int(x) for x in out)

    def table(self, seqs, max_blocks: int):
        import numpy as np
        ids = np.ascontiguousarray(np.asarray(seqs, dtype=np.int64))
        tab = np.empty((max(len(ids), 1), max(int(max_blocks), 1)), dtype=np.int32)
        lens = np.empty(max(len(ids), 1), dtype=np.int32)
        _check(self._lib.pkv_bm_table(self._h, ids.ctypes.data, len(ids), int(max_blocks), tab.ctypes.data,
                                      lens.ctypes.data), "pkv_bm_table")
        return tab[: len(ids), : int(max_blocks)], lens[: len(ids)]

    def take_copies(self, max_copies: int = 1 << 16):
        import numpy as np
        src = np.empty(max(int(max_copies), 1), dtype=np.int32)
        dst = np.empty_like(src)
        k = self._lib.pkv_bm_take_copies(self._h, src.ctypes.data, dst.ctypes.data, int(max_copies))
        if k < 0:
            raise PkvError(1, "pkv_bm_take_copies")
        return src[:k].copy(), dst[:k].copy()

    def stats(self):
        import numpy as np
        out = np.zeros(5, dtype=np.int64)
        _check(self._lib.pkv_bm_stats(self._h, out.ctypes.data), "pkv_bm_stats")
        return tuple(int(x) for x in out)


def paged_kv_copy_blocks(k_cache, v_cache, src, dst, stream=None) -> None:
    """Copy whole blocks of both pools: block dst[i] <- block src[i] (device int32 tensors)."""
    NB, Hkv, D = _pools(k_cache, v_cache)
    n = int(src.numel())
    if dst.numel() != n:
        raise ValueError("src and dst differ in length")
    st = _load().paged_kv_copy_blocks(_dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), _dtype_code(k_cache), Hkv,
                                      D, BLOCK_SIZE, NB, _dev(src, "src") if n else ctypes.c_void_p(0),
                                      _dev(dst, "dst") if n else ctypes.c_void_p(0), n, _stream(stream))
    _check(st, "paged_kv_copy_blocks")
