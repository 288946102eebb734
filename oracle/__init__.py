"""fp64 CPU oracle for the attention forward -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The product library never uses it.

It wraps ``attn_oracle.c`` (plain C, fp64, two-pass softmax over a
materialised score row). See that file's header for the definition it writes
out and the pages it follows. Inputs are numpy ``uint16`` arrays holding raw
fp16 or bf16 bit patterns, contiguous ``[B, H, S, D]``.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_DTYPES = {"f16": 0, "bf16": 1}
_MASKS = {"full": 0, "causal": 1, "window": 2}

_i64 = ctypes.c_int64
_ptr = ctypes.c_void_p


def _bind(lib):
    lib.oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
    lib.oracle_f16_to_f64.restype = ctypes.c_double
    lib.oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
    lib.oracle_bf16_to_f64.restype = ctypes.c_double
    lib.oracle_visible.argtypes = [_i64, _i64, ctypes.c_int, _i64, _i64]
    lib.oracle_visible.restype = ctypes.c_int
    lib.oracle_pair_count.argtypes = [_i64, ctypes.c_int, _i64, _i64]
    lib.oracle_pair_count.restype = _i64
    lib.oracle_attention_rows.argtypes = [
        _ptr, _ptr, _ptr, _i64, _i64, _i64, _i64, ctypes.c_double, ctypes.c_int,
        _i64, _i64, ctypes.c_int, _i64, _ptr, _ptr, _ptr, ctypes.c_int]
    lib.oracle_attention_rows.restype = ctypes.c_int
    lib.oracle_attention_probs.argtypes = [
        _ptr, _ptr, _ptr, _i64, _i64, ctypes.c_double, ctypes.c_int, _i64, _i64,
        ctypes.c_int, _ptr, _ptr, _ptr]
    lib.oracle_attention_probs.restype = ctypes.c_int
    lib.oracle_attention_kv.argtypes = [
        _ptr, _ptr, _ptr, _i64, _i64, _i64, _i64, _i64, ctypes.c_double, ctypes.c_int,
        _i64, _i64, ctypes.c_int, _ptr, _ptr, ctypes.c_int]
    lib.oracle_attention_kv.restype = ctypes.c_int
    lib.oracle_round.argtypes = [ctypes.c_double, ctypes.c_int]
    lib.oracle_round.restype = ctypes.c_double
    lib.oracle_rope_rows.argtypes = [_ptr, _i64, _i64, _ptr, _ptr, _ptr, ctypes.c_int,
                                     ctypes.c_int, _ptr]
    lib.oracle_rope_rows.restype = ctypes.c_int
    lib.oracle_attention_rope_rows.argtypes = [
        _ptr, _ptr, _ptr, _i64, _i64, _i64, _i64, ctypes.c_double, ctypes.c_int, _i64, _i64,
        ctypes.c_int, _ptr, _ptr, ctypes.c_int, _i64, _ptr, _ptr, _ptr, ctypes.c_int]
    lib.oracle_attention_rope_rows.restype = ctypes.c_int
    lib.oracle_attention_kv_rope.argtypes = [
        _ptr, _ptr, _ptr, _i64, _i64, _i64, _i64, _i64, ctypes.c_double, ctypes.c_int, _i64,
        _i64, ctypes.c_int, _ptr, _ptr, ctypes.c_int, _ptr, _ptr, ctypes.c_int]
    lib.oracle_attention_kv_rope.restype = ctypes.c_int
    lib.oracle_attention_bwd.argtypes = [
        _ptr, _ptr, _ptr, _ptr, _i64, _i64, _i64, _i64, ctypes.c_double, ctypes.c_int, _i64,
        _i64, ctypes.c_int, _ptr, _ptr, _ptr, _ptr, _ptr, _ptr, ctypes.c_int]
    lib.oracle_attention_bwd.restype = ctypes.c_int
    lib.oracle_decode.argtypes = [_ptr, _i64, ctypes.c_int, _ptr]
    lib.oracle_decode.restype = None
    lib.oracle_max_threads.argtypes = []
    lib.oracle_max_threads.restype = ctypes.c_int
    return lib


class Oracle:
    """One loaded build of the oracle (the real one, or a planted-mistake copy)."""

    def __init__(self, path):
        self.path = path
        self.lib = _bind(ctypes.CDLL(path))

    # -- masks ---------------------------------------------------------------
    @staticmethod
    def _mask_args(mask, window):
        if mask not in _MASKS:
            raise ValueError(f"mask must be one of {sorted(_MASKS)}, got {mask!r}")
        wl, wr = window if window is not None else (-1, -1)
        return _MASKS[mask], int(wl), int(wr)

    def visible(self, i, j, mask, window=(-1, -1)):
        m, wl, wr = self._mask_args(mask, window)
        return bool(self.lib.oracle_visible(i, j, m, wl, wr))

    def pair_count(self, S, mask, window=(-1, -1)):
        """Visible (i, j) pairs of one S x S head, by enumeration."""
        m, wl, wr = self._mask_args(mask, window)
        return int(self.lib.oracle_pair_count(S, m, wl, wr))

    # -- decoding ------------------------------------------------------------
    def decode(self, bits, dtype):
        bits = np.ascontiguousarray(bits, dtype=np.uint16)
        out = np.empty(bits.shape, dtype=np.float64)
        self.lib.oracle_decode(bits.ctypes.data, bits.size, _DTYPES[dtype], out.ctypes.data)
        return out

    # -- attention -----------------------------------------------------------
    def attention_rows(self, q, k, v, dtype, scale, mask, window=(-1, -1), rows=None,
                       nthreads=0):
        """fp64 output rows and LSE for the flat row indices ``rows``.

        ``q, k, v``: uint16 bit patterns, shape [B, H, S, D]. ``rows``: flat
        indices ``(b*H + h)*S + i`` (default: every row). Returns
        ``(o [n, D] float64, lse [n] float64)``.
        """
        q = np.ascontiguousarray(q, dtype=np.uint16)
        k = np.ascontiguousarray(k, dtype=np.uint16)
        v = np.ascontiguousarray(v, dtype=np.uint16)
        if q.ndim != 4 or q.shape != k.shape or q.shape != v.shape:
            raise ValueError("q, k, v must share one [B, H, S, D] shape")
        B, H, S, D = q.shape
        if rows is None:
            rows = np.arange(B * H * S, dtype=np.int64)
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        m, wl, wr = self._mask_args(mask, window)
        o = np.empty((rows.size, D), dtype=np.float64)
        lse = np.empty(rows.size, dtype=np.float64)
        rc = self.lib.oracle_attention_rows(
            q.ctypes.data, k.ctypes.data, v.ctypes.data, B, H, S, D, float(scale), m,
            wl, wr, _DTYPES[dtype], rows.size, rows.ctypes.data, o.ctypes.data,
            lse.ctypes.data, int(nthreads))
        if rc != 0:
            raise ValueError("oracle_attention_rows rejected its arguments")
        return o, lse

    def attention(self, q, k, v, dtype, scale, mask, window=(-1, -1), nthreads=0):
        """Every row: ``(o [B,H,S,D] float64, lse [B,H,S] float64)``."""
        B, H, S, D = q.shape
        o, lse = self.attention_rows(q, k, v, dtype, scale, mask, window, None, nthreads)
        return o.reshape(B, H, S, D), lse.reshape(B, H, S)

    def attention_probs(self, qh, kh, vh, dtype, scale, mask, window=(-1, -1)):
        """One head with its [S, S] probability matrix: ``(p, o, lse)``."""
        qh = np.ascontiguousarray(qh, dtype=np.uint16)
        kh = np.ascontiguousarray(kh, dtype=np.uint16)
        vh = np.ascontiguousarray(vh, dtype=np.uint16)
        S, D = qh.shape
        m, wl, wr = self._mask_args(mask, window)
        p = np.empty((S, S), dtype=np.float64)
        o = np.empty((S, D), dtype=np.float64)
        lse = np.empty(S, dtype=np.float64)
        rc = self.lib.oracle_attention_probs(
            qh.ctypes.data, kh.ctypes.data, vh.ctypes.data, S, D, float(scale), m, wl, wr,
            _DTYPES[dtype], p.ctypes.data, o.ctypes.data, lse.ctypes.data)
        if rc != 0:
            raise ValueError("oracle_attention_probs rejected its arguments")
        return p, o, lse

    def attention_kv(self, q, k, v, dtype, scale, mask, window=(-1, -1), nthreads=0):
        """New query rows against a key/value cache (incremental decoding).

        ``q``: [B, H, Sq, D]; ``k, v``: [B, H, Sk, D] (uint16 bit patterns),
        1 <= Sq <= Sk. Query row i sits at position Sk - Sq + i. Returns
        ``(o [B,H,Sq,D] float64, lse [B,H,Sq] float64)``.
        """
        q = np.ascontiguousarray(q, dtype=np.uint16)
        k = np.ascontiguousarray(k, dtype=np.uint16)
        v = np.ascontiguousarray(v, dtype=np.uint16)
        if q.ndim != 4 or k.ndim != 4 or k.shape != v.shape:
            raise ValueError("q must be [B, H, Sq, D] and k, v one [B, H, Sk, D] shape")
        B, H, Sq, D = q.shape
        if k.shape[:2] != (B, H) or k.shape[3] != D:
            raise ValueError("q and k, v disagree on B, H or D")
        Sk = k.shape[2]
        m, wl, wr = self._mask_args(mask, window)
        o = np.empty((B, H, Sq, D), dtype=np.float64)
        lse = np.empty((B, H, Sq), dtype=np.float64)
        rc = self.lib.oracle_attention_kv(
            q.ctypes.data, k.ctypes.data, v.ctypes.data, B, H, Sq, Sk, D, float(scale), m,
            wl, wr, _DTYPES[dtype], o.ctypes.data, lse.ctypes.data, int(nthreads))
        if rc != 0:
            raise ValueError("oracle_attention_kv rejected its arguments")
        return o, lse

    # -- rotary position embedding --------------------------------------------
    _ROPE_MODES = {"halves": 0, "interleaved": 1}

    @staticmethod
    def _tables(cos, sin, D):
        cos = np.ascontiguousarray(cos, dtype=np.float32)
        sin = np.ascontiguousarray(sin, dtype=np.float32)
        if cos.ndim != 2 or cos.shape != sin.shape or cos.shape[1] != D // 2:
            raise ValueError("cos and sin must share one [n_pos, D/2] float32 shape")
        return cos, sin

    def round_to(self, x, dtype):
        """Nearest ``dtype`` value of each float64 in ``x`` (ties to even), as float64."""
        return np.array([self.lib.oracle_round(float(t), _DTYPES[dtype])
                         for t in np.asarray(x, np.float64).ravel()]).reshape(np.shape(x))

    def rope(self, x, pos, cos, sin, mode, dtype):
        """RoPE of the rows of ``x`` (uint16 bits, [..., D]) at positions ``pos``
        (one per row), with [n_pos, D/2] float32 tables. ``mode``: "halves" or
        "interleaved". Returns float64 of x's shape."""
        x = np.ascontiguousarray(x, dtype=np.uint16)
        D = x.shape[-1]
        cos, sin = self._tables(cos, sin, D)
        n = x.size // D
        pos = np.ascontiguousarray(np.broadcast_to(np.asarray(pos, np.int64), (n,)))
        if n and (pos.min() < 0 or pos.max() >= cos.shape[0]):
            raise ValueError("a position is outside the tables")
        out = np.empty(x.shape, dtype=np.float64)
        rc = self.lib.oracle_rope_rows(x.ctypes.data, n, D, pos.ctypes.data, cos.ctypes.data,
                                       sin.ctypes.data, self._ROPE_MODES[mode], _DTYPES[dtype],
                                       out.ctypes.data)
        if rc != 0:
            raise ValueError("oracle_rope_rows rejected its arguments")
        return out

    def attention_rope_rows(self, q, k, v, dtype, scale, mask, window, cos, sin, mode,
                            rows=None, nthreads=0):
        """RoPE attention: q and k rows rotated at their positions 0..S-1 (tables
        [n_pos >= S, D/2] float32) and rounded to ``dtype``, then attention.
        Same conventions as :meth:`attention_rows`."""
        q = np.ascontiguousarray(q, dtype=np.uint16)
        k = np.ascontiguousarray(k, dtype=np.uint16)
        v = np.ascontiguousarray(v, dtype=np.uint16)
        if q.ndim != 4 or q.shape != k.shape or q.shape != v.shape:
            raise ValueError("q, k, v must share one [B, H, S, D] shape")
        B, H, S, D = q.shape
        cos, sin = self._tables(cos, sin, D)
        if cos.shape[0] < S:
            raise ValueError("the tables need a row per position")
        if rows is None:
            rows = np.arange(B * H * S, dtype=np.int64)
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        m, wl, wr = self._mask_args(mask, window)
        o = np.empty((rows.size, D), dtype=np.float64)
        lse = np.empty(rows.size, dtype=np.float64)
        rc = self.lib.oracle_attention_rope_rows(
            q.ctypes.data, k.ctypes.data, v.ctypes.data, B, H, S, D, float(scale), m, wl, wr,
            _DTYPES[dtype], cos.ctypes.data, sin.ctypes.data, self._ROPE_MODES[mode],
            rows.size, rows.ctypes.data, o.ctypes.data, lse.ctypes.data, int(nthreads))
        if rc != 0:
            raise ValueError("oracle_attention_rope_rows rejected its arguments")
        return o, lse

    def attention_rope(self, q, k, v, dtype, scale, mask, window, cos, sin, mode, nthreads=0):
        """Every row of RoPE attention: ``(o [B,H,S,D], lse [B,H,S])`` float64."""
        B, H, S, D = q.shape
        o, lse = self.attention_rope_rows(q, k, v, dtype, scale, mask, window, cos, sin, mode,
                                          None, nthreads)
        return o.reshape(B, H, S, D), lse.reshape(B, H, S)

    def attention_kv_rope(self, q, k, v, dtype, scale, mask, window, cos, sin, mode,
                          nthreads=0):
        """:meth:`attention_kv` with the new query rows rotated (RoPE) at their
        positions Sk - Sq + i and rounded to ``dtype``; the cache keys are used
        as given (already rotated)."""
        q = np.ascontiguousarray(q, dtype=np.uint16)
        k = np.ascontiguousarray(k, dtype=np.uint16)
        v = np.ascontiguousarray(v, dtype=np.uint16)
        B, H, Sq, D = q.shape
        Sk = k.shape[2]
        cos, sin = self._tables(cos, sin, D)
        if cos.shape[0] < Sk:
            raise ValueError("the tables need a row per cached position")
        m, wl, wr = self._mask_args(mask, window)
        o = np.empty((B, H, Sq, D), dtype=np.float64)
        lse = np.empty((B, H, Sq), dtype=np.float64)
        rc = self.lib.oracle_attention_kv_rope(
            q.ctypes.data, k.ctypes.data, v.ctypes.data, B, H, Sq, Sk, D, float(scale), m, wl,
            wr, _DTYPES[dtype], cos.ctypes.data, sin.ctypes.data, self._ROPE_MODES[mode],
            o.ctypes.data, lse.ctypes.data, int(nthreads))
        if rc != 0:
            raise ValueError("oracle_attention_kv_rope rejected its arguments")
        return o, lse

    def attention_varlen(self, q, k, v, cu_seqlens, dtype, scale, mask, window=(-1, -1),
                         nthreads=0):
        """Packed variable-length sequences, each attending only within itself.

        Ascend C FlashAttention-2 tile-fusion page, section 4.1 (data
        structures): the input is taken as contiguous [total_tokens, H, D].
        Sequence b is tokens ``cu_seqlens[b] .. cu_seqlens[b+1]-1`` (host ints,
        non-decreasing, within the tensors); its token ``cu_seqlens[b] + i`` is
        its row i, and its result is :meth:`attention` of that sequence alone.
        Returns ``(o [T,H,D] float64, lse [T,H] float64)``; tokens in no
        sequence are NaN.
        """
        q = np.ascontiguousarray(q, dtype=np.uint16)
        k = np.ascontiguousarray(k, dtype=np.uint16)
        v = np.ascontiguousarray(v, dtype=np.uint16)
        if q.ndim != 3 or q.shape != k.shape or q.shape != v.shape:
            raise ValueError("q, k, v must share one [total_tokens, H, D] shape")
        T, H, D = q.shape
        cu = [int(x) for x in cu_seqlens]
        if any(b < a for a, b in zip(cu, cu[1:])) or (cu and (cu[0] < 0 or cu[-1] > T)):
            raise ValueError("cu_seqlens must be non-decreasing within [0, total_tokens]")
        o = np.full((T, H, D), np.nan)
        lse = np.full((T, H), np.nan)
        for a, b in zip(cu, cu[1:]):
            if b == a:
                continue

            def head_major(x):  # [L, H, D] -> [1, H, L, D]
                return np.ascontiguousarray(x[a:b].transpose(1, 0, 2))[None]

            os_, ls = self.attention(head_major(q), head_major(k), head_major(v), dtype,
                                     scale, mask, window, nthreads)
            o[a:b] = os_[0].transpose(1, 0, 2)
            lse[a:b] = ls[0].T
        return o, lse

    def attention_bwd(self, q, k, v, dout, dtype, scale, mask, window=(-1, -1), nthreads=0):
        """Gradients of the attention: ``(dq, dk, dv)`` and the magnitude sums
        ``(mag_dq, mag_dk, mag_dv)``, float64 [B,H,S,D] each, for uint16 bit
        inputs q, k, v and dout (= dL/dO) of one [B,H,S,D] shape."""
        arrs = [np.ascontiguousarray(x, dtype=np.uint16) for x in (q, k, v, dout)]
        if arrs[0].ndim != 4 or any(a.shape != arrs[0].shape for a in arrs):
            raise ValueError("q, k, v, dout must share one [B, H, S, D] shape")
        B, H, S, D = arrs[0].shape
        m, wl, wr = self._mask_args(mask, window)
        outs = [np.empty((B, H, S, D), dtype=np.float64) for _ in range(6)]
        rc = self.lib.oracle_attention_bwd(
            *(a.ctypes.data for a in arrs), B, H, S, D, float(scale), m, wl, wr, _DTYPES[dtype],
            *(o.ctypes.data for o in outs), int(nthreads))
        if rc != 0:
            raise ValueError("oracle_attention_bwd rejected its arguments")
        return tuple(outs[:3]), tuple(outs[3:])

    def max_threads(self):
        return int(self.lib.oracle_max_threads())


_default = None


def load(rebuild=False):
    """The oracle, built from source first if no build exists yet."""
    global _default
    if _default is None or rebuild:
        path = _build.lib_path()
        if rebuild or not os.path.exists(path):
            _build.build()
        _default = Oracle(path)
    return _default


def load_planted(plant):
    """A copy of the oracle with deliberate mistake ``plant`` built in (tests only)."""
    path = _build.lib_path(plant)
    _build.build(plant=plant, out=path)
    return Oracle(path)
