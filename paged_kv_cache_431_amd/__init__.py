"""Python binding of libpkv: paged KV-cache decode attention for MI355X.

Argument marshalling only: every step of the hot path runs in the HIP
kernels of libpkv.so (built from csrc/ by ``python -m
paged_kv_cache_431_amd.build``).  There is no fallback: if the library is
missing, or a tensor is not on the GPU, the call raises.

PyTorch is used for device memory and streams; the functions take tensors,
check their shapes and dtypes, and pass raw device pointers plus the current
HIP stream to the C ABI declared in include/pkv.h (same function names).

  pkv_paged_attention_decode   paged decode attention (one launch)
  pkv_paged_attention_multi    several new query tokens per sequence, causal
  pkv_decode_step              scatter of the new tokens + decode in one launch
  pkv_reshape_and_cache        write new tokens' K/V into their slots
  pkv_copy_blocks              copy blocks (src -> dst) in both pools: copy-on-write
  pkv_swap_blocks              move blocks between a device pool and a pinned host pool
  pkv_decode_workspace_bytes   workspace size for a decode call (any h_kv, library's splits)
  pkv_decode_workspace_bytes_splits  ... for a forced split count
  pkv_decode_num_splits        split count the library will use
  pkv_multi_workspace_bytes    workspace size for a call with several query tokens
  pkv_multi_num_splits         its split count
  BlockManager                 the host block manager (pkv_bm_*)
"""

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpkv.so")

PKV_F32, PKV_F16, PKV_BF16, PKV_FP8_E4M3 = 0, 1, 2, 3
PKV_OK, PKV_EINVAL, PKV_EUNSUPPORTED, PKV_ENOSPC, PKV_EWORKSPACE, PKV_EHIP = range(6)

_lib = None


class PkvError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__(f"{what}: {lib().pkv_status_str(status).decode()}")


class OutOfBlocks(PkvError):
    pass


def lib():
    """The loaded libpkv.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m paged_kv_cache_431_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    c_int, c_i32, c_sz, c_f, c_p = ctypes.c_int, ctypes.c_int32, ctypes.c_size_t, ctypes.c_float, ctypes.c_void_p
    p_i32 = ctypes.POINTER(ctypes.c_int32)
    p_i64 = ctypes.POINTER(ctypes.c_int64)
    # (out, out_dtype, q, q_dtype, k_cache, v_cache, kv_dtype, k_scale, v_scale,
    #  block_tables, context_lens, S, Hq, Hkv, D, B, NB, MB, max_context_len,
    #  scale, workspace, workspace_bytes, stream); the *_splits calls take
    #  num_splits right after scale
    _DECODE_ARGS = [c_p, c_int, c_p, c_int, c_p, c_p, c_int, c_f, c_f, c_p, c_p, c_int, c_int, c_int, c_int, c_int,
                    c_int, c_int, c_int, c_f, c_p, c_sz, c_p]
    # decode's arguments with (new_k, new_v, new_dtype) after q_dtype
    _STEP_ARGS = [c_p, c_int, c_p, c_int, c_p, c_p, c_int, c_p, c_p, c_int, c_f, c_f, c_p, c_p, c_int, c_int, c_int,
                  c_int, c_int, c_int, c_int, c_int, c_f, c_p, c_sz, c_p]
    sig = {
        "pkv_status_str": (ctypes.c_char_p, [c_int]),
        "pkv_abi_version": (c_int, []),
        "pkv_decode_workspace_bytes": (c_sz, [c_int] * 5),
        "pkv_decode_workspace_bytes_splits": (c_sz, [c_int] * 7),
        "pkv_decode_num_splits": (c_int, [c_int] * 7),
        "pkv_paged_attention_decode": (c_int, _DECODE_ARGS),
        "pkv_paged_attention_decode_splits": (c_int, _DECODE_ARGS[:20] + [c_int] + _DECODE_ARGS[20:]),
        "pkv_paged_attention_decode_noalloc": (c_int, _DECODE_ARGS[:20] + _DECODE_ARGS[22:]),
        "pkv_decode_step": (c_int, _STEP_ARGS),
        "pkv_decode_step_splits": (c_int, _STEP_ARGS[:23] + [c_int] + _STEP_ARGS[23:]),
        "pkv_multi_workspace_bytes": (c_sz, [c_int] * 8),
        "pkv_multi_num_splits": (c_int, [c_int] * 8),
        "pkv_paged_attention_multi": (c_int, [c_p, c_int, c_p, c_int, c_p, c_int, c_int, c_p, c_p, c_int, c_f, c_f,
                                              c_p, c_p, c_int, c_int, c_int, c_int, c_int, c_int, c_int, c_int, c_f,
                                              c_int, c_p, c_sz, c_p]),
        "pkv_reshape_and_cache": (c_int, [c_p, c_p, c_int, c_p, c_p, c_int, c_f, c_f, c_p, c_int, c_int, c_int,
                                          c_int, c_int, c_p]),
        "pkv_copy_blocks": (c_int, [c_p, c_p, c_int, c_p, c_int, c_int, c_int, c_int, c_int, c_p]),
        "pkv_swap_blocks": (c_int, [c_p, c_p, c_int, c_p, c_p, c_int, c_int, c_p, c_int, c_int, c_int, c_int, c_p]),
        "pkv_bm_create": (c_int, [c_i32, c_i32, p_i32, ctypes.POINTER(c_p)]),
        "pkv_bm_destroy": (None, [c_p]),
        "pkv_bm_append": (c_int, [c_p, c_i32, c_i32, p_i64, p_i32, p_i32]),
        "pkv_bm_fork": (c_int, [c_p, c_i32, c_i32]),
        "pkv_bm_free": (c_int, [c_p, c_i32]),
        "pkv_bm_block_table": (c_int, [c_p, c_i32, p_i32, c_i32, p_i32, p_i32]),
        "pkv_bm_export": (c_int, [c_p, p_i32, c_i32, p_i32, c_i32, p_i32]),
        "pkv_bm_num_free": (c_i32, [c_p]),
        "pkv_bm_refcount": (c_i32, [c_p, c_i32]),
        "pkv_bm_free_list": (c_int, [c_p, p_i32, c_i32, p_i32]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _lib = L
    return L


def _check(status, what):
    if status != PKV_OK:
        if status == PKV_ENOSPC:
            raise OutOfBlocks(status, what)
        raise PkvError(status, what)


def dtype_code(t):
    import torch
    codes = {torch.float32: PKV_F32, torch.float16: PKV_F16, torch.bfloat16: PKV_BF16,
             torch.uint8: PKV_FP8_E4M3, torch.float8_e4m3fn: PKV_FP8_E4M3}
    if t.dtype not in codes:
        raise TypeError(f"unsupported tensor dtype {t.dtype}")
    return codes[t.dtype]


def _dev_ptr(t, name):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (there is no CPU path)")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def pkv_decode_workspace_bytes(num_seqs, h_q, head_dim, max_context_len, block_size):
    """Workspace bytes for any decode call with these sizes (any h_kv dividing
    h_q, the library's split count)."""
    return lib().pkv_decode_workspace_bytes(num_seqs, h_q, head_dim, max_context_len, block_size)


def pkv_decode_workspace_bytes_splits(num_seqs, h_q, h_kv, head_dim, block_size, max_context_len, num_splits):
    """Workspace bytes for a decode call with num_splits forced (0: the library's choice)."""
    return lib().pkv_decode_workspace_bytes_splits(num_seqs, h_q, h_kv, head_dim, block_size, max_context_len,
                                                   num_splits)


def pkv_decode_num_splits(num_seqs, h_q, h_kv, head_dim, block_size, max_context_len, num_splits=0):
    return lib().pkv_decode_num_splits(num_seqs, h_q, h_kv, head_dim, block_size, max_context_len, num_splits)


def make_workspace(num_seqs, h_q, h_kv, head_dim, block_size, max_context_len, num_splits=0, device="cuda"):
    """A zero-filled decode workspace (zero once; calls keep it reusable),
    sized by pkv_decode_workspace_bytes, or by pkv_decode_workspace_bytes_splits
    for a forced split count."""
    import torch
    if num_splits:
        n = pkv_decode_workspace_bytes_splits(num_seqs, h_q, h_kv, head_dim, block_size, max_context_len, num_splits)
    else:
        n = pkv_decode_workspace_bytes(num_seqs, h_q, head_dim, max_context_len, block_size)
    return torch.zeros(max(n, 256), dtype=torch.uint8, device=device)


def _decode_args(out, q, k_cache, v_cache, block_tables, context_lens, max_context_len, workspace, scale, k_scale,
                 v_scale, num_splits, stream):
    """Checked, marshalled arguments of pkv_paged_attention_decode (num_splits
    == 0), pkv_paged_attention_decode_splits (num_splits inserted after
    scale) or, with workspace None, pkv_paged_attention_decode_noalloc."""
    import torch
    S, h_q, D = q.shape
    NB, h_kv, B, D2 = k_cache.shape
    if D2 != D or tuple(v_cache.shape) != tuple(k_cache.shape) or tuple(out.shape) != (S, h_q, D):
        raise ValueError("shape mismatch between q / out / k_cache / v_cache")
    if k_cache.dtype != v_cache.dtype:
        raise ValueError("k_cache and v_cache must share a dtype")
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise TypeError("block_tables and context_lens must be int32")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or tuple(context_lens.shape) != (S,):
        raise ValueError("block_tables must be [S, MB] and context_lens [S]")
    split_arg = (int(num_splits),) if num_splits else ()
    ws_arg = () if workspace is None else (_dev_ptr(workspace, "workspace"),
                                           workspace.numel() * workspace.element_size())
    return (_dev_ptr(out, "out"), dtype_code(out), _dev_ptr(q, "q"), dtype_code(q),
            _dev_ptr(k_cache, "k_cache"), _dev_ptr(v_cache, "v_cache"), dtype_code(k_cache),
            float(k_scale), float(v_scale), _dev_ptr(block_tables, "block_tables"),
            _dev_ptr(context_lens, "context_lens"), S, h_q, h_kv, D, B, NB, block_tables.shape[1],
            int(max_context_len), float(scale), *split_arg, *ws_arg, _stream(stream))


def pkv_paged_attention_decode(out, q, k_cache, v_cache, block_tables, context_lens, *, max_context_len,
                               scale=0.0, k_scale=1.0, v_scale=1.0, num_splits=0, workspace=None, stream=None):
    """out[s, g, :] = attention of q[s, g, :] over sequence s's cached K/V.

    q, out [S, Hq, D]; k_cache, v_cache [NB, Hkv, B, D] (uint8 = FP8 E4M3);
    block_tables [S, MB] int32; context_lens [S] int32 (all on the GPU).
    num_splits > 0 calls pkv_paged_attention_decode_splits with that count.
    """
    if workspace is None:
        workspace = make_workspace(q.shape[0], q.shape[1], k_cache.shape[1], q.shape[2], k_cache.shape[2],
                                   max_context_len, num_splits, device=q.device)
    args = _decode_args(out, q, k_cache, v_cache, block_tables, context_lens, max_context_len, workspace, scale,
                        k_scale, v_scale, num_splits, stream)
    name = "pkv_paged_attention_decode_splits" if num_splits else "pkv_paged_attention_decode"
    _check(getattr(lib(), name)(*args), name)
    return out


def pkv_paged_attention_decode_noalloc(out, q, k_cache, v_cache, block_tables, context_lens, *, max_context_len,
                                       scale=0.0, k_scale=1.0, v_scale=1.0, stream=None):
    """pkv_paged_attention_decode without a workspace argument: the library
    uses its own per-GPU workspace and allocates nothing (for callers that
    cannot allocate).  Calls that overlap on one GPU race."""
    args = _decode_args(out, q, k_cache, v_cache, block_tables, context_lens, max_context_len, None, scale, k_scale,
                        v_scale, 0, stream)
    _check(lib().pkv_paged_attention_decode_noalloc(*args), "pkv_paged_attention_decode_noalloc")
    return out


def pkv_multi_workspace_bytes(num_seqs, h_q, h_kv, head_dim, block_size, max_query_len, max_context_len,
                              num_splits=0):
    return lib().pkv_multi_workspace_bytes(num_seqs, h_q, h_kv, head_dim, block_size, max_query_len,
                                           max_context_len, num_splits)


def pkv_multi_num_splits(num_seqs, h_q, h_kv, head_dim, block_size, max_query_len, max_context_len, num_splits=0):
    return lib().pkv_multi_num_splits(num_seqs, h_q, h_kv, head_dim, block_size, max_query_len, max_context_len,
                                      num_splits)


def make_multi_workspace(num_seqs, h_q, h_kv, head_dim, block_size, max_query_len, max_context_len, num_splits=0,
                         device="cuda"):
    """A zero-filled workspace for pkv_paged_attention_multi (zero once; calls keep it reusable)."""
    import torch
    n = pkv_multi_workspace_bytes(num_seqs, h_q, h_kv, head_dim, block_size, max_query_len, max_context_len,
                                  num_splits)
    return torch.zeros(max(n, 256), dtype=torch.uint8, device=device)


def _multi_args(out, q, k_cache, v_cache, block_tables, context_lens, query_start, max_query_len, max_context_len,
                workspace, scale, k_scale, v_scale, num_splits, stream):
    import torch
    T, h_q, D = q.shape
    NB, h_kv, B, D2 = k_cache.shape
    S = context_lens.shape[0] if context_lens.dim() == 1 else -1
    if D2 != D or tuple(v_cache.shape) != tuple(k_cache.shape) or tuple(out.shape) != (T, h_q, D):
        raise ValueError("shape mismatch between q / out / k_cache / v_cache")
    if k_cache.dtype != v_cache.dtype:
        raise ValueError("k_cache and v_cache must share a dtype")
    for t, n in ((block_tables, "block_tables"), (context_lens, "context_lens"), (query_start, "query_start")):
        if t.dtype != torch.int32:
            raise TypeError(f"{n} must be int32")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or tuple(query_start.shape) != (S + 1,):
        raise ValueError("block_tables must be [S, MB], context_lens [S] and query_start [S + 1]")
    return (_dev_ptr(out, "out"), dtype_code(out), _dev_ptr(q, "q"), dtype_code(q),
            _dev_ptr(query_start, "query_start"), T, int(max_query_len),
            _dev_ptr(k_cache, "k_cache"), _dev_ptr(v_cache, "v_cache"), dtype_code(k_cache),
            float(k_scale), float(v_scale), _dev_ptr(block_tables, "block_tables"),
            _dev_ptr(context_lens, "context_lens"), S, h_q, h_kv, D, B, NB, block_tables.shape[1],
            int(max_context_len), float(scale), int(num_splits), _dev_ptr(workspace, "workspace"),
            workspace.numel() * workspace.element_size(), _stream(stream))


def pkv_paged_attention_multi(out, q, k_cache, v_cache, block_tables, context_lens, query_start, *, max_query_len,
                              max_context_len, scale=0.0, k_scale=1.0, v_scale=1.0, num_splits=0, workspace=None,
                              stream=None):
    """Causal paged attention of several new query tokens per sequence.

    q, out [T, Hq, D]: rows query_start[s] .. query_start[s+1]-1 are the new
    tokens of sequence s, at positions ctx_s - m_s + i; context_lens [S]
    counts them; query_start [S + 1] int32 (all on the GPU).
    """
    if workspace is None:
        S = context_lens.shape[0]
        workspace = make_multi_workspace(S, q.shape[1], k_cache.shape[1], q.shape[2], k_cache.shape[2],
                                         max_query_len, max_context_len, num_splits, device=q.device)
    args = _multi_args(out, q, k_cache, v_cache, block_tables, context_lens, query_start, max_query_len,
                       max_context_len, workspace, scale, k_scale, v_scale, num_splits, stream)
    _check(lib().pkv_paged_attention_multi(*args), "pkv_paged_attention_multi")
    return out


def _step_args(out, q, new_k, new_v, k_cache, v_cache, block_tables, context_lens, max_context_len, workspace, scale,
               k_scale, v_scale, num_splits, stream):
    """Checked, marshalled arguments of pkv_decode_step (num_splits == 0) or
    pkv_decode_step_splits (num_splits inserted after scale)."""
    import torch
    S, h_q, D = q.shape
    NB, h_kv, B, D2 = k_cache.shape
    if D2 != D or tuple(v_cache.shape) != tuple(k_cache.shape) or tuple(out.shape) != (S, h_q, D):
        raise ValueError("shape mismatch between q / out / k_cache / v_cache")
    if tuple(new_k.shape) != (S, h_kv, D) or new_v.shape != new_k.shape or new_v.dtype != new_k.dtype:
        raise ValueError("new_k and new_v must be [S, Hkv, D] of one dtype")
    if k_cache.dtype != v_cache.dtype:
        raise ValueError("k_cache and v_cache must share a dtype")
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise TypeError("block_tables and context_lens must be int32")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or tuple(context_lens.shape) != (S,):
        raise ValueError("block_tables must be [S, MB] and context_lens [S]")
    split_arg = (int(num_splits),) if num_splits else ()
    return (_dev_ptr(out, "out"), dtype_code(out), _dev_ptr(q, "q"), dtype_code(q), _dev_ptr(new_k, "new_k"),
            _dev_ptr(new_v, "new_v"), dtype_code(new_k), _dev_ptr(k_cache, "k_cache"), _dev_ptr(v_cache, "v_cache"),
            dtype_code(k_cache), float(k_scale), float(v_scale), _dev_ptr(block_tables, "block_tables"),
            _dev_ptr(context_lens, "context_lens"), S, h_q, h_kv, D, B, NB, block_tables.shape[1],
            int(max_context_len), float(scale), *split_arg, _dev_ptr(workspace, "workspace"),
            workspace.numel() * workspace.element_size(), _stream(stream))


def pkv_decode_step(out, q, new_k, new_v, k_cache, v_cache, block_tables, context_lens, *, max_context_len,
                    scale=0.0, k_scale=1.0, v_scale=1.0, num_splits=0, workspace=None, stream=None):
    """One decode step in one launch: new_k / new_v [S, Hkv, D] go to position
    context_lens[s] - 1 of each sequence (slot from its block table), then
    out[s, g, :] is the attention of q[s, g, :] over the context including
    it.  Same bits as pkv_reshape_and_cache followed by the decode call.
    num_splits > 0 calls pkv_decode_step_splits with that count."""
    if workspace is None:
        S, h_q, D = q.shape
        workspace = make_workspace(S, h_q, k_cache.shape[1], D, k_cache.shape[2], max_context_len, num_splits,
                                   device=q.device)
    args = _step_args(out, q, new_k, new_v, k_cache, v_cache, block_tables, context_lens, max_context_len, workspace,
                      scale, k_scale, v_scale, num_splits, stream)
    name = "pkv_decode_step_splits" if num_splits else "pkv_decode_step"
    _check(getattr(lib(), name)(*args), name)
    return out


class PreparedCall:
    """A C-ABI call whose arguments were validated and marshalled once.

    Calling it re-issues the same launch (same tensors, same stream) with no
    Python-side work beyond the foreign call: for decode loops and benchmarks.
    The tensors must stay alive and keep their storage while it is used."""

    def __init__(self, fn, args, what, keep):
        self._fn, self._args, self._what, self._keep = fn, args, what, keep

    def __call__(self):
        st = self._fn(*self._args)
        if st != PKV_OK:
            _check(st, self._what)


def prepare_paged_attention_decode(out, q, k_cache, v_cache, block_tables, context_lens, *, max_context_len,
                                   workspace, scale=0.0, k_scale=1.0, v_scale=1.0, num_splits=0, stream=None):
    """PreparedCall of pkv_paged_attention_decode (or its _splits variant for
    num_splits > 0), same arguments."""
    args = _decode_args(out, q, k_cache, v_cache, block_tables, context_lens, max_context_len, workspace, scale,
                        k_scale, v_scale, num_splits, stream)
    name = "pkv_paged_attention_decode_splits" if num_splits else "pkv_paged_attention_decode"
    return PreparedCall(getattr(lib(), name), args, name,
                        (out, q, k_cache, v_cache, block_tables, context_lens, workspace))


def prepare_paged_attention_multi(out, q, k_cache, v_cache, block_tables, context_lens, query_start, *,
                                  max_query_len, max_context_len, workspace, scale=0.0, k_scale=1.0, v_scale=1.0,
                                  num_splits=0, stream=None):
    """PreparedCall of pkv_paged_attention_multi (same arguments)."""
    args = _multi_args(out, q, k_cache, v_cache, block_tables, context_lens, query_start, max_query_len,
                       max_context_len, workspace, scale, k_scale, v_scale, num_splits, stream)
    return PreparedCall(lib().pkv_paged_attention_multi, args, "pkv_paged_attention_multi",
                        (out, q, k_cache, v_cache, block_tables, context_lens, query_start, workspace))


def prepare_decode_step(out, q, new_k, new_v, k_cache, v_cache, block_tables, context_lens, *, max_context_len,
                        workspace, scale=0.0, k_scale=1.0, v_scale=1.0, num_splits=0, stream=None):
    """PreparedCall of pkv_decode_step (or pkv_decode_step_splits for
    num_splits > 0), same arguments."""
    args = _step_args(out, q, new_k, new_v, k_cache, v_cache, block_tables, context_lens, max_context_len, workspace,
                      scale, k_scale, v_scale, num_splits, stream)
    name = "pkv_decode_step_splits" if num_splits else "pkv_decode_step"
    return PreparedCall(getattr(lib(), name), args, name,
                        (out, q, new_k, new_v, k_cache, v_cache, block_tables, context_lens, workspace))


def prepare_reshape_and_cache(key, value, k_cache, v_cache, slot_mapping, *, k_scale=1.0, v_scale=1.0, stream=None):
    """PreparedCall of pkv_reshape_and_cache (same arguments)."""
    T, h_kv, D = key.shape
    NB, _, B, _ = k_cache.shape
    args = (_dev_ptr(key, "key"), _dev_ptr(value, "value"), dtype_code(key), _dev_ptr(k_cache, "k_cache"),
            _dev_ptr(v_cache, "v_cache"), dtype_code(k_cache), float(k_scale), float(v_scale),
            _dev_ptr(slot_mapping, "slot_mapping"), T, h_kv, D, B, NB, _stream(stream))
    return PreparedCall(lib().pkv_reshape_and_cache, args, "pkv_reshape_and_cache",
                        (key, value, k_cache, v_cache, slot_mapping))


def pkv_reshape_and_cache(key, value, k_cache, v_cache, slot_mapping, *, k_scale=1.0, v_scale=1.0, stream=None):
    """Write key/value [T, Hkv, D] into the pools at slot_mapping [T] (int64)."""
    import torch
    T, h_kv, D = key.shape
    NB, h_kv2, B, D2 = k_cache.shape
    if (h_kv2, D2) != (h_kv, D) or tuple(value.shape) != tuple(key.shape) or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("shape mismatch between key / value / caches")
    if slot_mapping.dtype != torch.int64 or tuple(slot_mapping.shape) != (T,):
        raise TypeError("slot_mapping must be int64 [T]")
    st = lib().pkv_reshape_and_cache(
        _dev_ptr(key, "key"), _dev_ptr(value, "value"), dtype_code(key), _dev_ptr(k_cache, "k_cache"),
        _dev_ptr(v_cache, "v_cache"), dtype_code(k_cache), float(k_scale), float(v_scale),
        _dev_ptr(slot_mapping, "slot_mapping"), T, h_kv, D, B, NB, _stream(stream))
    _check(st, "pkv_reshape_and_cache")


def pkv_copy_blocks(k_cache, v_cache, block_pairs, *, stream=None):
    """Copy block src -> dst for every row of block_pairs [n, 2] (int32, on
    the GPU) in both pools (the copy of copy-on-write)."""
    import torch
    if tuple(v_cache.shape) != tuple(k_cache.shape) or k_cache.dtype != v_cache.dtype:
        raise ValueError("k_cache and v_cache must have one shape and dtype")
    if block_pairs.dtype != torch.int32 or block_pairs.dim() != 2 or block_pairs.shape[1] != 2:
        raise TypeError("block_pairs must be int32 [n, 2]")
    NB, h_kv, B, D = k_cache.shape
    st = lib().pkv_copy_blocks(_dev_ptr(k_cache, "k_cache"), _dev_ptr(v_cache, "v_cache"), dtype_code(k_cache),
                               _dev_ptr(block_pairs, "block_pairs"), block_pairs.shape[0], h_kv, D, B, NB,
                               _stream(stream))
    _check(st, "pkv_copy_blocks")


def _pool_ptr(t, name):
    """Device pointer of a GPU tensor or address of a pinned host tensor."""
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if not (t.is_cuda or t.is_pinned()):
        raise ValueError(f"{name} must be a GPU tensor or a pinned host tensor (pin_memory=True)")
    return ctypes.c_void_p(t.data_ptr())


def pkv_swap_blocks(dst_k, dst_v, src_k, src_v, block_pairs, *, stream=None):
    """Copy block src of (src_k, src_v) to block dst of (dst_k, dst_v) for each
    row (src, dst) of block_pairs [n, 2] int32, in one launch.  Pools are
    [NB, Hkv, B, D] on the GPU or in pinned host memory (swap out: device ->
    host, swap in: host -> device); block_pairs on the GPU or pinned."""
    import torch
    if src_k.dtype != dst_k.dtype or src_v.dtype != src_k.dtype or dst_v.dtype != dst_k.dtype:
        raise ValueError("all four pools must share a dtype")
    if tuple(src_k.shape[1:]) != tuple(dst_k.shape[1:]) or src_v.shape != src_k.shape or dst_v.shape != dst_k.shape:
        raise ValueError("pools must agree in [Hkv, B, D], and K with V")
    if block_pairs.dtype != torch.int32 or block_pairs.dim() != 2 or block_pairs.shape[1] != 2:
        raise ValueError("block_pairs must be [n, 2] int32")
    _, h_kv, B, D = src_k.shape
    st = lib().pkv_swap_blocks(_pool_ptr(dst_k, "dst_k"), _pool_ptr(dst_v, "dst_v"), dst_k.shape[0],
                               _pool_ptr(src_k, "src_k"), _pool_ptr(src_v, "src_v"), src_k.shape[0],
                               dtype_code(src_k), _pool_ptr(block_pairs, "block_pairs"), block_pairs.shape[0],
                               h_kv, D, B, _stream(stream))
    _check(st, "pkv_swap_blocks")


class BlockManager:
    """Host block manager of libpkv (FIFO free list, refcounts, copy-on-write)."""

    def __init__(self, num_blocks, block_size, free_order=None):
        self._h = ctypes.c_void_p()
        order = None
        if free_order is not None:
            self._order = np.ascontiguousarray(free_order, dtype=np.int32)
            order = self._order.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
        _check(lib().pkv_bm_create(num_blocks, block_size, order, ctypes.byref(self._h)), "pkv_bm_create")
        self.num_blocks = num_blocks
        self.block_size = block_size

    def __del__(self):
        if getattr(self, "_h", None) and _lib is not None:
            _lib.pkv_bm_destroy(self._h)
            self._h = None

    def append(self, seq, n_tokens):
        slots = np.empty(max(n_tokens, 1), dtype=np.int64)
        src, dst = ctypes.c_int32(), ctypes.c_int32()
        _check(lib().pkv_bm_append(self._h, seq, n_tokens, slots.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                   ctypes.byref(src), ctypes.byref(dst)), "pkv_bm_append")
        return slots[:n_tokens].tolist(), (src.value, dst.value)

    def fork(self, parent, child):
        _check(lib().pkv_bm_fork(self._h, parent, child), "pkv_bm_fork")

    def free_seq(self, seq):
        _check(lib().pkv_bm_free(self._h, seq), "pkv_bm_free")

    def block_table(self, seq):
        nb, nt = ctypes.c_int32(), ctypes.c_int32()
        _check(lib().pkv_bm_block_table(self._h, seq, None, 0, ctypes.byref(nb), ctypes.byref(nt)), "pkv_bm_block_table")
        out = np.empty(max(nb.value, 1), dtype=np.int32)
        _check(lib().pkv_bm_block_table(self._h, seq, out.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), nb.value,
                                        ctypes.byref(nb), ctypes.byref(nt)), "pkv_bm_block_table")
        return out[:nb.value].tolist(), nt.value

    def export(self, seqs, max_blocks):
        """(block_tables [len(seqs), max_blocks] int32, context_lens [len(seqs)] int32)."""
        seqs = np.ascontiguousarray(seqs, dtype=np.int32)
        tables = np.empty((len(seqs), max_blocks), dtype=np.int32)
        lens = np.empty(len(seqs), dtype=np.int32)
        P = ctypes.POINTER(ctypes.c_int32)
        _check(lib().pkv_bm_export(self._h, seqs.ctypes.data_as(P), len(seqs), tables.ctypes.data_as(P), max_blocks,
                                   lens.ctypes.data_as(P)), "pkv_bm_export")
        return tables, lens

    def num_free(self):
        return lib().pkv_bm_num_free(self._h)

    def refcount(self, block):
        return lib().pkv_bm_refcount(self._h, block)

    def free_list(self):
        n = ctypes.c_int32()
        _check(lib().pkv_bm_free_list(self._h, None, 0, ctypes.byref(n)), "pkv_bm_free_list")
        out = np.empty(max(n.value, 1), dtype=np.int32)
        _check(lib().pkv_bm_free_list(self._h, out.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), n.value,
                                      ctypes.byref(n)), "pkv_bm_free_list")
        return out[:n.value].tolist()
