"""fa_decode_noalloc (the cache entry point that allocates nothing and keeps its
split partials in the library's per-GPU scratch array) against fa_decode with
a caller workspace, through the C ABI (needs a gfx950 GPU). Two calls in a
row, the second smaller, so the second reads a scratch array that still holds
the first call's partials."""
import sys

import numpy as np
import pytest
import torch

import synth
import tiled_attention_11_amd as fa
from parity import compare, to_bits, to_device

pytestmark = pytest.mark.gpu

_MCODE = {"full": 0, "causal": 1, "window": 2}


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


CALLS = [  # B, H, Sq, Sk, D, dtype, mask, window, seed
    (2, 4, 8, 3000, 128, "bf16", "causal", (-1, -1), 901),
    (1, 2, 3, 700, 64, "f16", "window", (300, 0), 902),
]


def test_noalloc_matches_workspace_entry_point(orc):
    for (B, H, Sq, Sk, D, dtype, mask, window, seed) in CALLS:
        need = fa.fa_decode_workspace_bytes(B, H, Sq, Sk, D, _MCODE[mask], *window)
        say("decode_noalloc", (B, H, Sq, Sk, D), dtype, mask, window, "seed", seed,
            "partials", need)
        assert need > 0  # the split path, which uses the scratch array
        q, _, _ = synth.make_qkv(B, H, Sq, D, dtype, seed)
        _, k, v = synth.make_qkv(B, H, Sk, D, dtype, seed + 1)
        tq, tk, tv = (to_device(x, dtype) for x in (q, k, v))
        o_ref_gpu, l_ref_gpu = fa.decode(tq, tk, tv, mask=mask, window=window)
        out = torch.empty_like(tq)
        lse = torch.empty((B, H, Sq), dtype=torch.float32, device="cuda")
        o, l = fa.decode_noalloc(tq, tk, tv, mask=mask, window=window, out=out, lse=lse)
        torch.cuda.synchronize()
        assert o.data_ptr() == out.data_ptr() and l.data_ptr() == lse.data_ptr()
        # same kernels, same split plan: bit for bit the workspace entry point's result
        assert torch.equal(o.view(torch.int16), o_ref_gpu.view(torch.int16))
        assert torch.equal(l.view(torch.int32), l_ref_gpu.view(torch.int32))
        o_ref, lse_ref = orc.attention_kv(q, k, v, dtype, 1.0 / np.sqrt(D), mask, window)
        st = compare(to_bits(o), l.cpu().numpy(), o_ref, lse_ref, dtype)
        say("stats", st)
        assert st["pass"], st


def test_noalloc_single_split_and_empty():
    """One split (no partials) and an empty problem need no scratch at all."""
    say("decode_noalloc single split / empty")
    B, H, Sq, Sk, D = 2, 1, 7, 7, 128
    assert fa.fa_decode_workspace_bytes(B, H, Sq, Sk, D, 1) == 0
    q, _, _ = synth.make_qkv(B, H, Sq, D, "f16", 903)
    _, k, v = synth.make_qkv(B, H, Sk, D, "f16", 904)
    tq, tk, tv = (to_device(x, "f16") for x in (q, k, v))
    a, la = fa.decode(tq, tk, tv, mask="causal")
    b, lb = fa.decode_noalloc(tq, tk, tv, mask="causal")
    e, le = fa.decode_noalloc(tq[:, :, :0], tk, tv, mask="causal")
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert torch.equal(la.view(torch.int32), lb.view(torch.int32))
    assert e.numel() == 0 and le.numel() == 0
