"""Fused attention forward for AMD Instinct MI355X (gfx950).

A thin ctypes binding over ``libfa.so`` (the C ABI in ``include/fa.h``).
``fa_fwd``, ``fa_visible_pairs``, ``fa_fwd_flops``, ``fa_fwd_varlen``,
``fa_fwd_varlen_flops``, ``fa_rope``, ``fa_fwd_rope``, ``fa_bwd``,
``fa_bwd_workspace_bytes``, ``fa_bwd_flops``, ``fa_decode``, ``fa_decode_rope``,
``fa_decode_paged_rope``,
``fa_decode_workspace_bytes``, ``fa_decode_flops``, ``fa_decode_paged``,
``fa_decode_paged_workspace_bytes``, ``fa_decode_noalloc`` and ``fa_strerror``
carry the C names and arguments (marshalling only). ``forward``,
``forward_varlen``, ``rope``, ``forward_rope``, ``backward``, ``decode``,
``decode_noalloc`` and ``decode_paged`` are the convenience entries
for torch tensors: torch supplies device memory and the stream; every step of
the computation runs in the library's HIP kernels.
There is no fallback: if the library is missing, importing this package
raises.
"""
import ctypes
import math
import os

__all__ = [
    "FA_MASK_FULL", "FA_MASK_CAUSAL", "FA_MASK_WINDOW", "FA_DTYPE_FP16",
    "FA_DTYPE_BF16", "FaError", "fa_fwd", "fa_visible_pairs", "fa_fwd_flops",
    "fa_fwd_schedule", "fa_fwd_varlen", "fa_fwd_varlen_flops", "fa_rope", "fa_fwd_rope", "FA_ROPE_HALVES",
    "FA_ROPE_INTERLEAVED", "fa_bwd", "fa_bwd_workspace_bytes", "fa_bwd_flops", "fa_decode",
    "fa_decode_rope", "fa_decode_paged_rope", "fa_decode_workspace_bytes", "fa_decode_flops", "fa_decode_paged",
    "fa_decode_paged_workspace_bytes", "fa_decode_noalloc", "fa_strerror", "forward",
    "forward_varlen", "rope", "forward_rope", "backward", "decode", "decode_noalloc",
    "decode_paged", "lib_path", "library", "load_library",
]

FA_MASK_FULL, FA_MASK_CAUSAL, FA_MASK_WINDOW = 0, 1, 2
FA_DTYPE_FP16, FA_DTYPE_BF16 = 0, 1
FA_ROPE_HALVES, FA_ROPE_INTERLEAVED = 0, 1
_ROPE_MODES = {"halves": FA_ROPE_HALVES, "interleaved": FA_ROPE_INTERLEAVED}
_MASKS = {"full": FA_MASK_FULL, "causal": FA_MASK_CAUSAL, "window": FA_MASK_WINDOW}

_HERE = os.path.dirname(os.path.abspath(__file__))


def lib_path():
    return os.environ.get("FA_LIBRARY", os.path.join(_HERE, "libfa.so"))


def _load(path=None):
    # torch ships its own HIP runtime (SONAME libamdhip64.so.7). Loading torch
    # first makes libfa bind to that same runtime instead of pulling a second
    # copy from /opt/rocm, so torch's streams and pointers stay valid in libfa.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    path = path or lib_path()
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is not built; run `python -m tiled_attention_11_amd._build` "
            "(hipcc, gfx950) first. There is no non-HIP fallback.")
    lib = ctypes.CDLL(path)
    vp, ci = ctypes.c_void_p, ctypes.c_int
    lib.fa_fwd.argtypes = [vp, vp, vp, vp, vp, ci, ci, ci, ci, ctypes.c_float, ci, ci, ci,
                           ci, vp]
    lib.fa_fwd.restype = ci
    lib.fa_visible_pairs.argtypes = [ci, ci, ci, ci]
    lib.fa_visible_pairs.restype = ctypes.c_int64
    lib.fa_fwd_flops.argtypes = [ci, ci, ci, ci, ci, ci, ci]
    lib.fa_fwd_flops.restype = ctypes.c_int64
    lib.fa_fwd_schedule.argtypes = [ci, ci, ci, ci, ci, ci, ci, ci, vp, ctypes.c_int64]
    lib.fa_fwd_schedule.restype = ctypes.c_int64
    i64 = ctypes.c_int64
    lib.fa_fwd_varlen.argtypes = [vp, vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ctypes.c_float,
                                  ci, ci, ci, ci, vp]
    lib.fa_fwd_varlen.restype = ci
    lib.fa_fwd_varlen_flops.argtypes = [ctypes.POINTER(ctypes.c_int32), ci, ci, ci, ci, ci, ci]
    lib.fa_fwd_varlen_flops.restype = i64
    lib.fa_rope.argtypes = [vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, ci, vp]
    lib.fa_rope.restype = ci
    lib.fa_fwd_rope.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ci,
                                ctypes.c_float, ci, ci, ci, ci, vp]
    lib.fa_fwd_rope.restype = ci
    lib.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, ci, ci, ci, ci, ctypes.c_float,
                           ci, ci, ci, ci, vp, i64, vp]
    lib.fa_bwd.restype = ci
    lib.fa_bwd_workspace_bytes.argtypes = [ci, ci, ci]
    lib.fa_bwd_workspace_bytes.restype = i64
    lib.fa_bwd_flops.argtypes = [ci, ci, ci, ci, ci, ci, ci]
    lib.fa_bwd_flops.restype = i64
    lib.fa_decode_rope.argtypes = [vp, vp, vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, ci,
                                   ctypes.c_float, ci, ci, ci, ci, vp, i64, vp]
    lib.fa_decode_rope.restype = ci
    lib.fa_decode_paged_rope.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, ci, ci, ci, ci, ci,
                                         ci, ci, ci, ci, ci, ctypes.c_float, ci, ci, ci, ci, vp,
                                         i64, vp]
    lib.fa_decode_paged_rope.restype = ci
    lib.fa_decode.argtypes = [vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ctypes.c_float, ci, ci,
                              ci, ci, vp, i64, vp]
    lib.fa_decode.restype = ci
    lib.fa_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ctypes.c_float,
                                      ci, ci, ci, ci, vp]
    lib.fa_decode_noalloc.restype = ci
    lib.fa_decode_workspace_bytes.argtypes = [ci, ci, ci, ci, ci, ci, ci, ci]
    lib.fa_decode_workspace_bytes.restype = i64
    lib.fa_decode_paged.argtypes = [vp, vp, vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, ci, ci,
                                    ctypes.c_float, ci, ci, ci, ci, vp, i64, vp]
    lib.fa_decode_paged.restype = ci
    lib.fa_decode_paged_workspace_bytes.argtypes = [ci, ci, ci, ci, ci, ci, ci, ci]
    lib.fa_decode_paged_workspace_bytes.restype = i64
    lib.fa_decode_flops.argtypes = [ci, ci, ci, ci, ci, ci, ci, ci]
    lib.fa_decode_flops.restype = i64
    lib.fa_strerror.argtypes = [ci]
    lib.fa_strerror.restype = ctypes.c_char_p
    return lib


_lib = _load()


def library():
    """The loaded ``ctypes.CDLL``."""
    return _lib


def load_library(path):
    """Another build of the same C ABI (e.g. the conservative-sync variant
    ``libfa_sync.so`` next to ``libfa.so``) as a ``ctypes.CDLL`` with the
    same argument types."""
    return _load(path)


class FaError(RuntimeError):
    def __init__(self, status, fn="fa_fwd"):
        self.status = status
        super().__init__(f"{fn} failed: {fa_strerror(status)} (status {status})")


# ---- the C functions, same names and arguments ------------------------------

def fa_fwd(q, k, v, o, lse, B, H, S, D, scale, mask_mode, win_l, win_r, dtype, stream):
    """Call ``fa_fwd`` with raw device addresses (ints); return its status."""
    return _lib.fa_fwd(q, k, v, o, lse, B, H, S, D, scale, mask_mode, win_l, win_r, dtype,
                       stream)


def fa_visible_pairs(S, mask_mode, win_l=-1, win_r=-1):
    return _lib.fa_visible_pairs(S, mask_mode, win_l, win_r)


def fa_fwd_flops(B, H, S, D, mask_mode, win_l=-1, win_r=-1):
    return _lib.fa_fwd_flops(B, H, S, D, mask_mode, win_l, win_r)


def fa_fwd_schedule(B, H, S, D, mask_mode, win_l, win_r, n_cu):
    """The forward's work plan on a GPU with ``n_cu`` compute units, as an
    int32 numpy array of rows (workgroup, round, head, first query row, rows
    per item, key tiles); raises FaError on bad arguments."""
    import numpy as np

    n = _lib.fa_fwd_schedule(B, H, S, D, mask_mode, win_l, win_r, n_cu, None, 0)
    if n < 0:
        raise FaError(n, "fa_fwd_schedule")
    out = np.zeros((max(n, 1), 6), dtype=np.int32)
    m = _lib.fa_fwd_schedule(B, H, S, D, mask_mode, win_l, win_r, n_cu,
                             out.ctypes.data_as(ctypes.c_void_p), n)
    if m != n:
        raise FaError(m if m < 0 else -1, "fa_fwd_schedule")
    return out[:n]


def fa_fwd_varlen(q, k, v, o, lse, cu_seqlens, nseq, max_seqlen, total_tokens, H, D, scale,
                  mask_mode, win_l, win_r, dtype, stream):
    """Call ``fa_fwd_varlen`` with raw device addresses (ints); return its status."""
    return _lib.fa_fwd_varlen(q, k, v, o, lse, cu_seqlens, nseq, max_seqlen, total_tokens, H, D,
                              scale, mask_mode, win_l, win_r, dtype, stream)


def fa_fwd_varlen_flops(cu_seqlens, H, D, mask_mode, win_l=-1, win_r=-1):
    """``cu_seqlens``: a host sequence of nseq + 1 ints."""
    n = len(cu_seqlens) - 1
    if n < 0:
        raise ValueError("cu_seqlens needs at least one entry")
    arr = (ctypes.c_int32 * (n + 1))(*[int(x) for x in cu_seqlens])
    return _lib.fa_fwd_varlen_flops(arr, n, H, D, mask_mode, win_l, win_r)


def fa_rope(x, y, cos_table, sin_table, n_pos, rope_mode, B, H, S, D, dtype, stream):
    """Call ``fa_rope`` with raw device addresses (ints); return its status."""
    return _lib.fa_rope(x, y, cos_table, sin_table, n_pos, rope_mode, B, H, S, D, dtype, stream)


def fa_fwd_rope(q, k, v, o, lse, k_rot, cos_table, sin_table, n_pos, rope_mode, B, H, S, D,
                scale, mask_mode, win_l, win_r, dtype, stream):
    """Call ``fa_fwd_rope`` with raw device addresses (ints); return its status."""
    return _lib.fa_fwd_rope(q, k, v, o, lse, k_rot, cos_table, sin_table, n_pos, rope_mode, B,
                            H, S, D, scale, mask_mode, win_l, win_r, dtype, stream)


def fa_bwd(q, k, v, o, lse, dout, dq, dk, dv, B, H, S, D, scale, mask_mode, win_l, win_r,
           dtype, workspace, workspace_bytes, stream):
    """Call ``fa_bwd`` with raw device addresses (ints); return its status."""
    return _lib.fa_bwd(q, k, v, o, lse, dout, dq, dk, dv, B, H, S, D, scale, mask_mode, win_l,
                       win_r, dtype, workspace, workspace_bytes, stream)


def fa_bwd_workspace_bytes(B, H, S):
    return _lib.fa_bwd_workspace_bytes(B, H, S)


def fa_bwd_flops(B, H, S, D, mask_mode, win_l=-1, win_r=-1):
    return _lib.fa_bwd_flops(B, H, S, D, mask_mode, win_l, win_r)


def fa_decode(q, k, v, o, lse, B, H, Sq, Sk, D, scale, mask_mode, win_l, win_r, dtype,
              workspace, workspace_bytes, stream):
    """Call ``fa_decode`` with raw device addresses (ints); return its status."""
    return _lib.fa_decode(q, k, v, o, lse, B, H, Sq, Sk, D, scale, mask_mode, win_l, win_r,
                          dtype, workspace, workspace_bytes, stream)


def fa_decode_noalloc(q, k, v, o, lse, B, H, Sq, Sk, D, scale, mask_mode, win_l, win_r, dtype,
                      stream):
    """Call ``fa_decode_noalloc`` with raw device addresses (ints); return its status."""
    return _lib.fa_decode_noalloc(q, k, v, o, lse, B, H, Sq, Sk, D, scale, mask_mode, win_l,
                                  win_r, dtype, stream)


def fa_decode_rope(q, k, v, o, lse, cos_table, sin_table, n_pos, rope_mode, B, H, Sq, Sk, D,
                   scale, mask_mode, win_l, win_r, dtype, workspace, workspace_bytes, stream):
    """Call ``fa_decode_rope`` with raw device addresses (ints); return its status."""
    return _lib.fa_decode_rope(q, k, v, o, lse, cos_table, sin_table, n_pos, rope_mode, B, H, Sq,
                               Sk, D, scale, mask_mode, win_l, win_r, dtype, workspace,
                               workspace_bytes, stream)


def fa_decode_paged_rope(q, k_pages, v_pages, o, lse, block_table, seq_lens, cos_table,
                         sin_table, n_pos, rope_mode, B, H, Sq, max_seq_len, D, num_pages,
                         page_size, max_pages, scale, mask_mode, win_l, win_r, dtype, workspace,
                         workspace_bytes, stream):
    """Call ``fa_decode_paged_rope`` with raw device addresses (ints); return its status."""
    return _lib.fa_decode_paged_rope(q, k_pages, v_pages, o, lse, block_table, seq_lens,
                                     cos_table, sin_table, n_pos, rope_mode, B, H, Sq,
                                     max_seq_len, D, num_pages, page_size, max_pages, scale,
                                     mask_mode, win_l, win_r, dtype, workspace, workspace_bytes,
                                     stream)


def fa_decode_workspace_bytes(B, H, Sq, Sk, D, mask_mode, win_l=-1, win_r=-1):
    return _lib.fa_decode_workspace_bytes(B, H, Sq, Sk, D, mask_mode, win_l, win_r)


def fa_decode_flops(B, H, Sq, Sk, D, mask_mode, win_l=-1, win_r=-1):
    return _lib.fa_decode_flops(B, H, Sq, Sk, D, mask_mode, win_l, win_r)


def fa_decode_paged(q, k_pages, v_pages, o, lse, block_table, seq_lens, B, H, Sq, max_seq_len,
                    D, num_pages, page_size, max_pages, scale, mask_mode, win_l, win_r, dtype,
                    workspace, workspace_bytes, stream):
    """Call ``fa_decode_paged`` with raw device addresses (ints); return its status."""
    return _lib.fa_decode_paged(q, k_pages, v_pages, o, lse, block_table, seq_lens, B, H, Sq,
                                max_seq_len, D, num_pages, page_size, max_pages, scale,
                                mask_mode, win_l, win_r, dtype, workspace, workspace_bytes,
                                stream)


def fa_decode_paged_workspace_bytes(B, H, Sq, max_seq_len, D, mask_mode, win_l=-1, win_r=-1):
    return _lib.fa_decode_paged_workspace_bytes(B, H, Sq, max_seq_len, D, mask_mode, win_l,
                                                win_r)


def fa_strerror(status):
    return _lib.fa_strerror(status).decode()


# ---- torch convenience ---------------------------------------------------------

def _mask_code(mask):
    if isinstance(mask, int):
        return mask
    try:
        return _MASKS[mask]
    except KeyError:
        raise ValueError(f"mask must be one of {sorted(_MASKS)}, got {mask!r}") from None


class _Nothing:
    def __enter__(self):
        return None

    def __exit__(self, *exc):
        return False


_NOTHING = _Nothing()


def _on_device(device):
    """A context that makes ``device`` current for the library call; nothing
    to do (and no device switch) when it already is, the common case."""
    import torch

    if device.index is None or device.index == torch.cuda.current_device():
        return _NOTHING
    return torch.cuda.device(device)


def forward(q, k, v, *, scale=None, mask="full", window=(-1, -1), out=None, lse=None,
            return_lse=True, stream=None):
    """Attention forward on torch device tensors.

    q, k, v: contiguous [B, H, S, D] float16 or bfloat16 tensors on one GPU.
    scale: defaults to 1/sqrt(D). mask: "full", "causal" or "window" with
    ``window=(win_l, win_r)`` (inclusive; negative = unbounded side).
    out / lse: optional preallocated outputs. Returns ``(o, lse)`` (``lse`` is
    None when ``return_lse`` is False and no buffer is given).
    """
    import torch

    if q.dim() != 4 or q.shape != k.shape or q.shape != v.shape:
        raise ValueError("q, k, v must share one [B, H, S, D] shape")
    if not (q.is_cuda and k.device == q.device and v.device == q.device):
        raise ValueError("q, k, v must be on the same GPU")
    if q.dtype not in (torch.float16, torch.bfloat16) or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must all be float16 or all bfloat16")
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    B, H, S, D = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype or out.device != q.device or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor like q")
    if lse is None and return_lse:
        lse = torch.empty((B, H, S), dtype=torch.float32, device=q.device)
    if lse is not None and (lse.shape != (B, H, S) or lse.dtype != torch.float32
                            or lse.device != q.device or not lse.is_contiguous()):
        raise ValueError("lse must be a contiguous float32 [B, H, S] tensor on q's device")
    wl, wr = window
    dtype = FA_DTYPE_FP16 if q.dtype == torch.float16 else FA_DTYPE_BF16
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    with _on_device(q.device):
        status = fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                        lse.data_ptr() if lse is not None else None, B, H, S, D,
                        float(scale), _mask_code(mask), int(wl), int(wr), dtype, stream)
    if status != 0:
        raise FaError(status)
    return out, lse


def forward_varlen(q, k, v, cu_seqlens, max_seqlen, *, scale=None, mask="full",
                   window=(-1, -1), out=None, lse=None, return_lse=True, stream=None):
    """Attention forward over packed variable-length sequences.

    q, k, v: contiguous [total_tokens, H, D] float16 or bfloat16 tensors on one
    GPU; sequence b is tokens ``cu_seqlens[b] .. cu_seqlens[b+1]-1``
    (``cu_seqlens``: int32 device tensor [nseq + 1]); ``max_seqlen``: a host int
    bounding every length. Other arguments as for ``forward``. Returns
    ``(o, lse)`` with ``lse`` of shape [total_tokens, H].
    """
    import torch

    if q.dim() != 3 or q.shape != k.shape or q.shape != v.shape:
        raise ValueError("q, k, v must share one [total_tokens, H, D] shape")
    if not (q.is_cuda and k.device == q.device and v.device == q.device):
        raise ValueError("q, k, v must be on the same GPU")
    if q.dtype not in (torch.float16, torch.bfloat16) or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must all be float16 or all bfloat16")
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if (cu_seqlens.dim() != 1 or cu_seqlens.numel() < 1 or cu_seqlens.dtype != torch.int32
            or cu_seqlens.device != q.device or not cu_seqlens.is_contiguous()):
        raise ValueError("cu_seqlens must be a contiguous int32 [nseq + 1] tensor on q's device")
    T, H, D = q.shape
    nseq = cu_seqlens.numel() - 1
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype or out.device != q.device or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor like q")
    if lse is None and return_lse:
        lse = torch.empty((T, H), dtype=torch.float32, device=q.device)
    if lse is not None and (lse.shape != (T, H) or lse.dtype != torch.float32
                            or lse.device != q.device or not lse.is_contiguous()):
        raise ValueError("lse must be a contiguous float32 [total_tokens, H] tensor on q's device")
    wl, wr = window
    dtype = FA_DTYPE_FP16 if q.dtype == torch.float16 else FA_DTYPE_BF16
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    with _on_device(q.device):
        status = fa_fwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                               lse.data_ptr() if lse is not None else None,
                               cu_seqlens.data_ptr(), nseq, int(max_seqlen), T, H, D,
                               float(scale), _mask_code(mask), int(wl), int(wr), dtype, stream)
    if status != 0:
        raise FaError(status, "fa_fwd_varlen")
    return out, lse


def _rope_code(mode):
    if isinstance(mode, int):
        return mode
    try:
        return _ROPE_MODES[mode]
    except KeyError:
        raise ValueError(f"rope mode must be one of {sorted(_ROPE_MODES)}, got {mode!r}") from None


def _check_tables(cos, sin, D, x):
    import torch
    if (cos.dim() != 2 or cos.shape != sin.shape or cos.shape[1] != D // 2
            or cos.dtype != torch.float32 or sin.dtype != torch.float32
            or cos.device != x.device or sin.device != x.device
            or not cos.is_contiguous() or not sin.is_contiguous()):
        raise ValueError("cos and sin must be contiguous float32 [n_pos, D/2] tensors on the "
                         "tensors' device")


def rope(x, cos, sin, *, mode="halves", out=None, stream=None):
    """Rotary embedding of a contiguous [B, H, S, D] float16/bfloat16 tensor:
    row s of every head turns by the angles of row s of ``cos``/``sin``
    (float32 [n_pos >= S, D/2]). ``out`` may be ``x`` (in place)."""
    import torch

    if x.dim() != 4 or not x.is_cuda or not x.is_contiguous():
        raise ValueError("x must be a contiguous [B, H, S, D] tensor on a GPU")
    if x.dtype not in (torch.float16, torch.bfloat16):
        raise ValueError("x must be float16 or bfloat16")
    B, H, S, D = x.shape
    _check_tables(cos, sin, D, x)
    if out is None:
        out = torch.empty_like(x)
    elif out.shape != x.shape or out.dtype != x.dtype or out.device != x.device or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor like x")
    dtype = FA_DTYPE_FP16 if x.dtype == torch.float16 else FA_DTYPE_BF16
    if stream is None:
        stream = torch.cuda.current_stream(x.device).cuda_stream
    with _on_device(x.device):
        status = fa_rope(x.data_ptr(), out.data_ptr(), cos.data_ptr(), sin.data_ptr(),
                         cos.shape[0], _rope_code(mode), B, H, S, D, dtype, stream)
    if status != 0:
        raise FaError(status, "fa_rope")
    return out


def forward_rope(q, k, v, cos, sin, *, mode="halves", k_rot=None, scale=None, mask="full",
                 window=(-1, -1), out=None, lse=None, return_lse=True, stream=None):
    """``forward`` of the rotary-embedded q and k (row i of each turned by row i
    of ``cos``/``sin``). The rotated keys are written to ``k_rot`` (allocated
    when not given; may be ``k`` to rotate in place). Returns ``(o, lse, k_rot)``."""
    import torch

    if q.dim() != 4 or q.shape != k.shape or q.shape != v.shape:
        raise ValueError("q, k, v must share one [B, H, S, D] shape")
    if not (q.is_cuda and k.device == q.device and v.device == q.device):
        raise ValueError("q, k, v must be on the same GPU")
    if q.dtype not in (torch.float16, torch.bfloat16) or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must all be float16 or all bfloat16")
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    B, H, S, D = q.shape
    _check_tables(cos, sin, D, q)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype or out.device != q.device or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor like q")
    if k_rot is None:
        k_rot = torch.empty_like(k)
    elif k_rot.shape != k.shape or k_rot.dtype != k.dtype or k_rot.device != k.device or not k_rot.is_contiguous():
        raise ValueError("k_rot must be a contiguous tensor like k")
    if lse is None and return_lse:
        lse = torch.empty((B, H, S), dtype=torch.float32, device=q.device)
    if lse is not None and (lse.shape != (B, H, S) or lse.dtype != torch.float32
                            or lse.device != q.device or not lse.is_contiguous()):
        raise ValueError("lse must be a contiguous float32 [B, H, S] tensor on q's device")
    wl, wr = window
    dtype = FA_DTYPE_FP16 if q.dtype == torch.float16 else FA_DTYPE_BF16
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    with _on_device(q.device):
        status = fa_fwd_rope(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                             lse.data_ptr() if lse is not None else None, k_rot.data_ptr(),
                             cos.data_ptr(), sin.data_ptr(), cos.shape[0], _rope_code(mode),
                             B, H, S, D, float(scale), _mask_code(mask), int(wl), int(wr), dtype,
                             stream)
    if status != 0:
        raise FaError(status, "fa_fwd_rope")
    return out, lse, k_rot


def backward(q, k, v, o, lse, dout, *, scale=None, mask="full", window=(-1, -1), dq=None,
             dk=None, dv=None, workspace=None, stream=None):
    """Gradients ``(dq, dk, dv)`` of the attention for ``dout`` = dL/dO, given the
    forward's ``o`` and ``lse`` (from ``forward`` with the same q, k, v, scale
    and mask). All of q, k, v, o, dout contiguous [B, H, S, D] of one dtype;
    lse float32 [B, H, S]. ``workspace``: optional uint8 device tensor of at
    least ``fa_bwd_workspace_bytes(B, H, S)`` bytes (allocated when not given)."""
    import torch

    ts = (q, k, v, o, dout)
    if q.dim() != 4 or any(t.shape != q.shape for t in ts):
        raise ValueError("q, k, v, o, dout must share one [B, H, S, D] shape")
    if not q.is_cuda or any(t.device != q.device for t in ts):
        raise ValueError("q, k, v, o, dout must be on the same GPU")
    if q.dtype not in (torch.float16, torch.bfloat16) or any(t.dtype != q.dtype for t in ts):
        raise ValueError("q, k, v, o, dout must all be float16 or all bfloat16")
    if not all(t.is_contiguous() for t in ts):
        raise ValueError("q, k, v, o, dout must be contiguous")
    B, H, S, D = q.shape
    if (lse.shape != (B, H, S) or lse.dtype != torch.float32 or lse.device != q.device
            or not lse.is_contiguous()):
        raise ValueError("lse must be a contiguous float32 [B, H, S] tensor on q's device")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    grads = []
    for name, g in (("dq", dq), ("dk", dk), ("dv", dv)):
        if g is None:
            g = torch.empty_like(q)
        elif g.shape != q.shape or g.dtype != q.dtype or g.device != q.device or not g.is_contiguous():
            raise ValueError(f"{name} must be a contiguous tensor like q")
        grads.append(g)
    need = fa_bwd_workspace_bytes(B, H, S)
    if need < 0:
        raise FaError(int(need), "fa_bwd")
    if workspace is None:
        workspace = torch.empty(max(int(need), 4), dtype=torch.uint8, device=q.device)
    wl, wr = window
    dtype = FA_DTYPE_FP16 if q.dtype == torch.float16 else FA_DTYPE_BF16
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    with _on_device(q.device):
        status = fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                        dout.data_ptr(), grads[0].data_ptr(), grads[1].data_ptr(),
                        grads[2].data_ptr(), B, H, S, D, float(scale), _mask_code(mask),
                        int(wl), int(wr), dtype, workspace.data_ptr(),
                        workspace.numel() * workspace.element_size(), stream)
    if status != 0:
        raise FaError(status, "fa_bwd")
    return tuple(grads)


def decode(q, k, v, *, scale=None, mask="causal", window=(-1, -1), out=None, lse=None,
           return_lse=True, workspace=None, rope=None, stream=None):
    """New query rows against a key/value cache on torch device tensors.

    q: contiguous [B, H, Sq, D] (Sq <= 32); k, v: contiguous [B, H, Sk, D]
    (Sk >= Sq), all float16 or all bfloat16 on one GPU. Query row i sits at
    position Sk - Sq + i; ``mask``/``window`` as for ``forward``, applied at
    that position. ``workspace``: optional uint8 device tensor of at least
    ``fa_decode_workspace_bytes(...)`` bytes (allocated here when needed and
    not given). ``rope``: optional ``(cos, sin, mode)`` (float32 [n_pos, D/2]
    tables, "halves" or "interleaved") to rotate the new rows at their
    positions; the cache holds rotated keys. Returns ``(o, lse)``.
    """
    import torch

    if q.dim() != 4 or k.dim() != 4 or k.shape != v.shape:
        raise ValueError("q must be [B, H, Sq, D] and k, v one [B, H, Sk, D] shape")
    B, H, Sq, D = q.shape
    if k.shape[0] != B or k.shape[1] != H or k.shape[3] != D:
        raise ValueError("q and k, v disagree on B, H or D")
    Sk = k.shape[2]
    if not (q.is_cuda and k.device == q.device and v.device == q.device):
        raise ValueError("q, k, v must be on the same GPU")
    if q.dtype not in (torch.float16, torch.bfloat16) or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must all be float16 or all bfloat16")
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype or out.device != q.device or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor like q")
    if lse is None and return_lse:
        lse = torch.empty((B, H, Sq), dtype=torch.float32, device=q.device)
    if lse is not None and (lse.shape != (B, H, Sq) or lse.dtype != torch.float32
                            or lse.device != q.device or not lse.is_contiguous()):
        raise ValueError("lse must be a contiguous float32 [B, H, Sq] tensor on q's device")
    wl, wr = window
    m = _mask_code(mask)
    dtype = FA_DTYPE_FP16 if q.dtype == torch.float16 else FA_DTYPE_BF16
    with _on_device(q.device):
        need = fa_decode_workspace_bytes(B, H, Sq, Sk, D, m, int(wl), int(wr))
        if need < 0:
            raise FaError(int(need), "fa_decode")
        if workspace is None and need > 0:
            workspace = torch.empty(int(need), dtype=torch.uint8, device=q.device)
        ws_ptr = workspace.data_ptr() if workspace is not None else None
        ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
        if stream is None:
            stream = torch.cuda.current_stream(q.device).cuda_stream
        if rope is None:
            status = fa_decode(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                               lse.data_ptr() if lse is not None else None, B, H, Sq, Sk, D,
                               float(scale), m, int(wl), int(wr), dtype, ws_ptr, int(ws_bytes),
                               stream)
        else:
            cos, sin, mode = rope
            _check_tables(cos, sin, D, q)
            status = fa_decode_rope(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                    lse.data_ptr() if lse is not None else None, cos.data_ptr(),
                                    sin.data_ptr(), cos.shape[0], _rope_code(mode), B, H, Sq,
                                    Sk, D, float(scale), m, int(wl), int(wr), dtype, ws_ptr,
                                    int(ws_bytes), stream)
    if status != 0:
        raise FaError(status, "fa_decode" if rope is None else "fa_decode_rope")
    return out, lse


def decode_noalloc(q, k, v, *, scale=None, mask="causal", window=(-1, -1), out=None, lse=None,
                   return_lse=True, stream=None):
    """``decode`` through ``fa_decode_noalloc``: the split partials go to the
    library's per-GPU scratch array instead of a workspace, so with ``out``
    (and ``lse``, or ``return_lse=False``) given nothing is allocated. Calls
    that overlap in time on one GPU race on that array. Returns ``(o, lse)``."""
    import torch

    if q.dim() != 4 or k.dim() != 4 or k.shape != v.shape:
        raise ValueError("q must be [B, H, Sq, D] and k, v one [B, H, Sk, D] shape")
    B, H, Sq, D = q.shape
    if k.shape[0] != B or k.shape[1] != H or k.shape[3] != D:
        raise ValueError("q and k, v disagree on B, H or D")
    Sk = k.shape[2]
    if not (q.is_cuda and k.device == q.device and v.device == q.device):
        raise ValueError("q, k, v must be on the same GPU")
    if q.dtype not in (torch.float16, torch.bfloat16) or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must all be float16 or all bfloat16")
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype or out.device != q.device or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor like q")
    if lse is None and return_lse:
        lse = torch.empty((B, H, Sq), dtype=torch.float32, device=q.device)
    if lse is not None and (lse.shape != (B, H, Sq) or lse.dtype != torch.float32
                            or lse.device != q.device or not lse.is_contiguous()):
        raise ValueError("lse must be a contiguous float32 [B, H, Sq] tensor on q's device")
    wl, wr = window
    m = _mask_code(mask)
    dtype = FA_DTYPE_FP16 if q.dtype == torch.float16 else FA_DTYPE_BF16
    with _on_device(q.device):
        if stream is None:
            stream = torch.cuda.current_stream(q.device).cuda_stream
        status = fa_decode_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                   lse.data_ptr() if lse is not None else None, B, H, Sq, Sk, D,
                                   float(scale), m, int(wl), int(wr), dtype, stream)
    if status != 0:
        raise FaError(status, "fa_decode_noalloc")
    return out, lse


def decode_paged(q, k_pages, v_pages, block_table, seq_lens, max_seq_len, *, scale=None,
                 mask="causal", window=(-1, -1), out=None, lse=None, return_lse=True,
                 workspace=None, rope=None, stream=None):
    """``decode`` over a paged cache on torch device tensors.

    q: contiguous [B, H, Sq, D]; k_pages, v_pages: contiguous
    [num_pages, page_size, H, D] (page_size a multiple of 32); block_table:
    int32 [B, max_pages]; seq_lens: int32 [B] (each >= Sq, <= max_seq_len,
    the host-side bound). Returns ``(o, lse)``.
    """
    import torch

    if q.dim() != 4 or k_pages.dim() != 4 or k_pages.shape != v_pages.shape:
        raise ValueError("q must be [B, H, Sq, D] and the pools one [P, page, H, D] shape")
    B, H, Sq, D = q.shape
    num_pages, page_size = k_pages.shape[0], k_pages.shape[1]
    if k_pages.shape[2] != H or k_pages.shape[3] != D:
        raise ValueError("the pools disagree with q on H or D")
    if block_table.dim() != 2 or block_table.shape[0] != B or block_table.dtype != torch.int32:
        raise ValueError("block_table must be int32 [B, max_pages]")
    if seq_lens.shape != (B,) or seq_lens.dtype != torch.int32:
        raise ValueError("seq_lens must be int32 [B]")
    max_pages = block_table.shape[1]
    for name, t in (("q", q), ("k_pages", k_pages), ("v_pages", v_pages),
                    ("block_table", block_table), ("seq_lens", seq_lens)):
        if not t.is_contiguous() or t.device != q.device:
            raise ValueError(f"{name} must be contiguous and on q's device")
    if q.dtype not in (torch.float16, torch.bfloat16) or k_pages.dtype != q.dtype \
            or v_pages.dtype != q.dtype:
        raise ValueError("q and the pools must all be float16 or all bfloat16")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and return_lse:
        lse = torch.empty((B, H, Sq), dtype=torch.float32, device=q.device)
    wl, wr = window
    m = _mask_code(mask)
    dtype = FA_DTYPE_FP16 if q.dtype == torch.float16 else FA_DTYPE_BF16
    with _on_device(q.device):
        need = fa_decode_paged_workspace_bytes(B, H, Sq, int(max_seq_len), D, m, int(wl), int(wr))
        if need < 0:
            raise FaError(int(need), "fa_decode_paged")
        if workspace is None and need > 0:
            workspace = torch.empty(int(need), dtype=torch.uint8, device=q.device)
        ws_ptr = workspace.data_ptr() if workspace is not None else None
        ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
        if stream is None:
            stream = torch.cuda.current_stream(q.device).cuda_stream
        if rope is None:
            status = fa_decode_paged(q.data_ptr(), k_pages.data_ptr(), v_pages.data_ptr(),
                                     out.data_ptr(), lse.data_ptr() if lse is not None else None,
                                     block_table.data_ptr(), seq_lens.data_ptr(), B, H, Sq,
                                     int(max_seq_len), D, num_pages, page_size, max_pages,
                                     float(scale), m, int(wl), int(wr), dtype, ws_ptr,
                                     int(ws_bytes), stream)
        else:
            cos, sin, mode = rope
            _check_tables(cos, sin, D, q)
            status = fa_decode_paged_rope(
                q.data_ptr(), k_pages.data_ptr(), v_pages.data_ptr(), out.data_ptr(),
                lse.data_ptr() if lse is not None else None, block_table.data_ptr(),
                seq_lens.data_ptr(), cos.data_ptr(), sin.data_ptr(), cos.shape[0],
                _rope_code(mode), B, H, Sq, int(max_seq_len), D, num_pages, page_size, max_pages,
                float(scale), m, int(wl), int(wr), dtype, ws_ptr, int(ws_bytes), stream)
    if status != 0:
        raise FaError(status, "fa_decode_paged" if rope is None else "fa_decode_paged_rope")
    return out, lse
