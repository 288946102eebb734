"""Helpers for comparing the HIP path with the oracle (used by GPU tests,
the smoke check and the benchmark's spot check).

Tolerance rule (per output element o against the oracle's fp64 value r):
  fp16: max |o - r| <= 2e-3 and mean |o - r| <= 2e-4 over the compared outputs;
  bf16: against R = RNE_bf16(r), the oracle's value rounded to the output
        type: |o - R| <= max(4e-3, ulp_bf16(R)) for every element -- the
        absolute bound, relaxed to one bf16 unit in the last place where the
        format cannot resolve 4e-3 (|R| >= 0.5: a correctly rounded output
        already misses a literal 4e-3 bound against r once |r| >= 1) -- and
        mean |o - R| <= 4e-4.
  LSE (fp32, both types): max |lse - lse_ref| <= 1e-3.
The literal statistics (max/mean against the unrounded fp64 value) are always
reported next to the verdict.
"""
import numpy as np
import torch

TOL = {"f16": (2e-3, 2e-4), "bf16": (4e-3, 4e-4)}
LSE_TOL = 1e-3

_TORCH = {"f16": torch.float16, "bf16": torch.bfloat16}


def to_device(bits, dtype, device="cuda"):
    """uint16 bit array -> contiguous torch tensor of ``dtype`` on ``device``."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16).copy())
    return t.view(_TORCH[dtype]).to(device)


def to_bits(t):
    """torch fp16/bf16 tensor -> uint16 numpy bit array (host)."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def decode(bits, dtype):
    """uint16 bits -> float64 with library decoders (numpy, torch)."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    if dtype == "f16":
        return bits.view(np.float16).astype(np.float64)
    t = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16)
    return t.double().numpy()


def round_bf16(x):
    """fp64 -> nearest bf16 value (as fp64), via torch's conversions."""
    return torch.from_numpy(np.asarray(x, np.float64)).to(torch.bfloat16).double().numpy()


def ulp_bf16(x):
    """Spacing of bf16 numbers at |x| (normal range; 2^-133 floor)."""
    ax = np.maximum(np.abs(np.asarray(x, np.float64)), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(ax)) - 7)


def compare(o_bits, lse, o_ref, lse_ref, dtype):
    """Check GPU output (bits) and LSE against the oracle. Returns a stats dict
    with 'pass' and the reasons for a failure."""
    o = decode(o_bits, dtype).reshape(o_ref.shape)
    err = np.abs(o - o_ref)
    finite = bool(np.all(np.isfinite(o)))
    st = {"n": int(o.size), "max_abs": float(err.max()) if err.size else 0.0,
          "mean_abs": float(err.mean()) if err.size else 0.0, "finite": finite}
    max_tol, mean_tol = TOL[dtype]
    reasons = []
    if not finite:
        reasons.append("non-finite output")
    if dtype == "f16":
        if st["max_abs"] > max_tol:
            reasons.append(f"max_abs {st['max_abs']:.3g} > {max_tol}")
        if st["mean_abs"] > mean_tol:
            reasons.append(f"mean_abs {st['mean_abs']:.3g} > {mean_tol}")
    else:
        rref = round_bf16(o_ref)
        err_r = np.abs(o - rref)
        bound = np.maximum(max_tol, ulp_bf16(rref))
        worst = float((err_r / bound).max()) if err.size else 0.0
        st["max_err_over_bound"] = worst
        if worst > 1.0:
            reasons.append(f"element error {worst:.3g}x its bound")
        mean_r = float(err_r.mean()) if err.size else 0.0
        st["mean_abs_vs_rounded_ref"] = mean_r
        st["mean_bound"] = mean_tol
        if mean_r > mean_tol:
            reasons.append(f"mean_abs vs rounded ref {mean_r:.3g} > {mean_tol:.3g}")
    if lse is not None and lse_ref is not None:
        lerr = np.abs(np.asarray(lse, np.float64).reshape(lse_ref.shape) - lse_ref)
        st["lse_max_abs"] = float(lerr.max()) if lerr.size else 0.0
        if not np.all(np.isfinite(lse)):
            reasons.append("non-finite lse")
        elif st["lse_max_abs"] > LSE_TOL:
            reasons.append(f"lse_max_abs {st['lse_max_abs']:.3g} > {LSE_TOL}")
    st["pass"] = not reasons
    st["reasons"] = reasons
    return st


def sample_rows(B, H, S, n, seed, extra_i=()):
    """Flat row indices: ``n`` random rows plus, for a few heads, the rows at
    tile edges and the ``extra_i`` positions."""
    rng = np.random.default_rng(seed)
    total = B * H * S
    rows = set(rng.choice(total, size=min(n, total), replace=False).tolist())
    edges = {0, 1, 31, 32, 63, 64, 65, 127, 128, 129, S // 2, S - 129, S - 128, S - 65,
             S - 64, S - 2, S - 1, *extra_i}
    heads = {0, B * H - 1, int(rng.integers(B * H))}
    for bh in heads:
        for i in edges:
            if 0 <= i < S:
                rows.add(bh * S + i)
    return np.array(sorted(rows), dtype=np.int64)
