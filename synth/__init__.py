"""Seeded synthetic inputs for the attention forward.

This module only draws and encodes inputs; it holds none of the attention
arithmetic. Both the GPU path's tests/benchmark and the CPU oracle receive the
same bytes from here.

Recipe (every workload):
  * ``numpy.random.default_rng(seed)`` (PCG64);
  * ``standard_normal(dtype=float32)`` in C order, drawn in the order q, k, v,
    each of shape [B, H, S, D];
  * optional large-logit outliers: for each (b, h) in order, ``round(frac*S)``
    distinct key rows picked with ``rng.choice(S, n, replace=False)`` are
    multiplied by ``outlier_scale`` in fp32 (before the single rounding);
  * one rounding to the storage type, round-to-nearest-even: fp16 through
    numpy's IEEE conversion, bf16 by integer rounding of the fp32 bit pattern.
Arrays come back as ``uint16`` bit patterns, contiguous [B, H, S, D].
"""
import hashlib

import numpy as np

# Workloads of the forward pass: shapes, masks, scales and seeds. The
# B4 H32 S4096 D128 fp16 shape is the one the catlass FlashAttention article
# benchmarks (section "performance data"); the sliding-window rows use a
# window that is, and one that is not, a multiple of a 64-key tile.
WORKLOADS = {
    "tiny_full":   dict(B=1, H=2, S=128, D=64, dtype="f16", mask="full",
                        window=(-1, -1), scale=0.125, seed=1),
    "tiny_causal": dict(B=1, H=2, S=128, D=64, dtype="f16", mask="causal",
                        window=(-1, -1), scale=0.125, seed=1),
    "d64_causal":  dict(B=1, H=32, S=2048, D=64, dtype="f16", mask="causal",
                        window=(-1, -1), scale=0.125, seed=2),
    "b4h32s4096_full":   dict(B=4, H=32, S=4096, D=128, dtype="f16", mask="full",
                              window=(-1, -1), scale=128 ** -0.5, seed=3),
    "b4h32s4096_causal": dict(B=4, H=32, S=4096, D=128, dtype="f16", mask="causal",
                              window=(-1, -1), scale=128 ** -0.5, seed=3),
    "b4h32s4096_win1024": dict(B=4, H=32, S=4096, D=128, dtype="f16", mask="window",
                               window=(1024, 0), scale=128 ** -0.5, seed=3),
    "b4h32s4096_win1000": dict(B=4, H=32, S=4096, D=128, dtype="f16", mask="window",
                               window=(1000, 0), scale=128 ** -0.5, seed=3),
    # the headline shape with rotary embedding of q and k (pairs of halves,
    # the usual 10000 frequency base; tables from rope_tables)
    "b4h32s4096_causal_rope": dict(B=4, H=32, S=4096, D=128, dtype="f16", mask="causal",
                                   window=(-1, -1), scale=128 ** -0.5, seed=3, rope="halves",
                                   rope_base=10000.0),
    # one GPU's share of the B4 H32 S4096 causal shape when its heads are
    # sharded over 8 GPUs (no communication: heads are independent)
    "b4h4s4096_causal": dict(B=4, H=4, S=4096, D=128, dtype="f16", mask="causal",
                             window=(-1, -1), scale=128 ** -0.5, seed=3),
    "long_bf16_outliers": dict(B=1, H=64, S=16384, D=128, dtype="bf16", mask="causal",
                               window=(-1, -1), scale=128 ** -0.5, seed=5,
                               outlier_frac=0.01, outlier_scale=20.0),
}

HEADLINE = "b4h32s4096_causal"

# Packed variable-length batches ([total_tokens, H, D], one token after the
# other; the tile-fusion page's data-structure section takes this layout).
# The lengths are drawn uniformly from [len_lo, len_hi] (varlen_lengths), so
# most are not multiples of a tile: the same 16384 tokens as the headline
# B4 x S4096 batch, in about eight sequences of ragged lengths.
VARLEN_WORKLOADS = {
    "varlen_h32_t16384_causal": dict(T=16384, H=32, D=128, dtype="f16", mask="causal",
                                     window=(-1, -1), scale=128 ** -0.5, seed=9,
                                     len_lo=256, len_hi=4096),
}

# New query rows against a key/value cache (incremental decoding): Sq rows at
# the end of sequences whose first Sk positions the cache holds. The NPU
# optimisation page's hands-on section runs batch 1, 32 heads, D = 128 against
# a cache; these stand in for a serving step at long context (one new token,
# and 16 new tokens as in speculative decoding or chunked prefill).
DECODE_WORKLOADS = {
    "decode_b1h32_q1_k8192":   dict(B=1, H=32, Sq=1, Sk=8192, D=128, dtype="f16",
                                    mask="causal", window=(-1, -1), scale=128 ** -0.5, seed=6),
    "decode_b4h32_q1_k16384":  dict(B=4, H=32, Sq=1, Sk=16384, D=128, dtype="f16",
                                    mask="causal", window=(-1, -1), scale=128 ** -0.5, seed=7),
    "decode_b4h32_q16_k16384": dict(B=4, H=32, Sq=16, Sk=16384, D=128, dtype="f16",
                                    mask="causal", window=(-1, -1), scale=128 ** -0.5, seed=8),
    # the same cache scattered over 64-key pages of a pool in a seeded random order
    "decode_paged_b4h32_q1_k16384": dict(B=4, H=32, Sq=1, Sk=16384, D=128, dtype="f16",
                                         mask="causal", window=(-1, -1), scale=128 ** -0.5,
                                         seed=7, page_size=64),
}


def paged_cache(k, v, page_size, seed):
    """Scatter contiguous caches k, v [B, H, Sk, D] (Sk a multiple of page_size)
    over the pages of pools [B * Sk / page_size, page_size, H, D] in a seeded
    random order; return the pools and the int32 block table [B, Sk / page_size]."""
    B, H, Sk, D = k.shape
    per = Sk // page_size
    order = np.random.default_rng(seed).permutation(B * per).astype(np.int32)
    table = order.reshape(B, per)
    kp = np.empty((B * per, page_size, H, D), dtype=k.dtype)
    vp = np.empty_like(kp)
    src_k = k.reshape(B, H, per, page_size, D).transpose(0, 2, 3, 1, 4).reshape(B * per, page_size, H, D)
    src_v = v.reshape(B, H, per, page_size, D).transpose(0, 2, 3, 1, 4).reshape(B * per, page_size, H, D)
    kp[table.reshape(-1)] = src_k
    vp[table.reshape(-1)] = src_v
    return kp, vp, table


def f32_to_bits(x, dtype):
    """Round fp32 values once to ``dtype`` ('f16' or 'bf16'); return uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f16":
        return x.astype(np.float16).view(np.uint16)
    if dtype == "bf16":
        u = x.view(np.uint32)
        # round to nearest, ties to even, on the 16 discarded bits
        bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
        return ((u + bias) >> np.uint32(16)).astype(np.uint16)
    raise ValueError(f"unknown dtype {dtype!r}")


def make_qkv(B, H, S, D, dtype, seed, outlier_frac=0.0, outlier_scale=20.0):
    """Draw q, k, v per the module recipe; return three uint16 [B,H,S,D] arrays."""
    rng = np.random.default_rng(seed)
    shape = (B, H, S, D)
    q = rng.standard_normal(shape, dtype=np.float32)
    k = rng.standard_normal(shape, dtype=np.float32)
    v = rng.standard_normal(shape, dtype=np.float32)
    if outlier_frac > 0.0 and S > 0:
        n = int(round(outlier_frac * S))
        for b in range(B):
            for h in range(H):
                if n:
                    rows = rng.choice(S, size=n, replace=False)
                    k[b, h, rows, :] *= np.float32(outlier_scale)
    return f32_to_bits(q, dtype), f32_to_bits(k, dtype), f32_to_bits(v, dtype)


def varlen_lengths(total_tokens, len_lo, len_hi, seed):
    """Sequence lengths for a packed batch of ``total_tokens`` tokens: integers
    drawn uniformly from [len_lo, len_hi] with ``default_rng(seed)`` until they
    reach the total, the last one cut so that they sum to it exactly."""
    rng = np.random.default_rng(seed)
    lengths, left = [], int(total_tokens)
    while left > 0:
        n = min(int(rng.integers(len_lo, len_hi + 1)), left)
        lengths.append(n)
        left -= n
    return lengths


def cu_seqlens_of(lengths):
    """int32 [nseq + 1] prefix sums of ``lengths`` (starting at 0)."""
    return np.concatenate([[0], np.cumsum(np.asarray(lengths, np.int64))]).astype(np.int32)


def make_varlen_qkv(total_tokens, H, D, dtype, seed):
    """Packed q, k, v of ``total_tokens`` tokens: standard normal fp32 drawn in
    the order q, k, v, each [total_tokens, H, D] in C order from one generator,
    each rounded once to ``dtype`` (uint16 bit patterns)."""
    rng = np.random.default_rng(seed)
    shape = (total_tokens, H, D)
    q = rng.standard_normal(shape, dtype=np.float32)
    k = rng.standard_normal(shape, dtype=np.float32)
    v = rng.standard_normal(shape, dtype=np.float32)
    return f32_to_bits(q, dtype), f32_to_bits(k, dtype), f32_to_bits(v, dtype)


def varlen_inputs(name):
    """(q, k, v, cu_seqlens) for a named packed workload."""
    w = VARLEN_WORKLOADS[name]
    lengths = varlen_lengths(w["T"], w["len_lo"], w["len_hi"], w["seed"])
    q, k, v = make_varlen_qkv(w["T"], w["H"], w["D"], w["dtype"], w["seed"] + 1)
    return q, k, v, cu_seqlens_of(lengths)


def rope_tables(n_pos, D, base=10000.0):
    """Rotary-embedding tables ``(cos, sin)``, float32 [n_pos, D/2]: pair t of a
    row at position p turns by p * base^(-2t/D) radians (the usual frequency
    ladder of rotary embeddings), evaluated in float64 and rounded once."""
    t = np.arange(D // 2, dtype=np.float64)
    ang = np.arange(n_pos, dtype=np.float64)[:, None] * base ** (-2.0 * t / D)[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def make_decode_qkv(B, H, Sq, Sk, D, dtype, seed):
    """q [B,H,Sq,D] and the cache k, v [B,H,Sk,D]: standard normal fp32 drawn in
    the order q, k, v from one generator, each rounded once to ``dtype``."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, Sq, D), dtype=np.float32)
    k = rng.standard_normal((B, H, Sk, D), dtype=np.float32)
    v = rng.standard_normal((B, H, Sk, D), dtype=np.float32)
    return f32_to_bits(q, dtype), f32_to_bits(k, dtype), f32_to_bits(v, dtype)


def decode_inputs(name):
    """(q, k, v) bit arrays for a named cache workload."""
    w = DECODE_WORKLOADS[name]
    return make_decode_qkv(w["B"], w["H"], w["Sq"], w["Sk"], w["D"], w["dtype"], w["seed"])


def workload_inputs(name):
    """(q, k, v) bit arrays for a named workload."""
    w = WORKLOADS[name]
    return make_qkv(w["B"], w["H"], w["S"], w["D"], w["dtype"], w["seed"],
                    w.get("outlier_frac", 0.0), w.get("outlier_scale", 20.0))


def digest(*arrays):
    """SHA-256 over the raw bytes of the arrays (for determinism checks)."""
    h = hashlib.sha256()
    for a in arrays:
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()
