"""The release library against the conservative-synchronisation build
(libfa_sync.so: every DMA and LDS phase waited for, a barrier between the
halves of every key step). Same arithmetic, so every output must be bit for bit
the same; a difference means the release build's hand-ordered DMA / LDS traffic
let a read see a tile that was not there yet or was already being replaced.
Needs a gfx950 GPU; every case prints its name and shape first."""
import ctypes
import math
import os
import sys

import pytest
import torch

import synth
import tiled_attention_11_amd as fa
from parity import to_device

pytestmark = pytest.mark.gpu

_SYNC = os.path.join(os.path.dirname(fa.lib_path()), "libfa_sync.so")
_MCODE = {"full": 0, "causal": 1, "window": 2}


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def sync_lib():
    if not os.path.exists(_SYNC):
        raise FileNotFoundError(f"{_SYNC} is not built (tiled_attention_11_amd._build.build())")
    return fa.load_library(_SYNC)


def _fwd(lib, q, k, v, scale, mask, window):
    B, H, S, D = q.shape
    o = torch.empty_like(q)
    lse = torch.empty((B, H, S), dtype=torch.float32, device=q.device)
    dt = 0 if q.dtype == torch.float16 else 1
    st = lib.fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H,
                    S, D, ctypes.c_float(scale), _MCODE[mask], window[0], window[1], dt,
                    torch.cuda.current_stream().cuda_stream)
    assert st == 0, st
    return o, lse


CASES = [  # B, H, S, D, dtype, mask, window
    (2, 3, 1000, 128, "f16", "causal", (-1, -1)),
    (2, 3, 1000, 128, "bf16", "window", (100, 0)),
    (1, 4, 777, 64, "f16", "full", (-1, -1)),
    (1, 4, 777, 64, "bf16", "window", (37, 50)),
    (4, 64, 512, 128, "f16", "causal", (-1, -1)),     # several items per workgroup
    (2, 64, 640, 64, "f16", "window", (100, 0)),
    (4, 16, 2048, 128, "f16", "window", (1000, 0)),
    (1, 8, 4096, 128, "bf16", "causal", (-1, -1)),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c[:5])) + f"-{c[5]}{c[6]}")
def test_forward_bit_identical(sync_lib, case):
    B, H, S, D, dtype, mask, window = case
    say("sync variant fwd", case)
    q, k, v = (to_device(x, dtype) for x in synth.make_qkv(B, H, S, D, dtype, seed=S + D))
    scale = 1.0 / math.sqrt(D)
    o1, l1 = _fwd(fa.library(), q, k, v, scale, mask, window)
    o2, l2 = _fwd(sync_lib, q, k, v, scale, mask, window)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32))


def test_varlen_bit_identical(sync_lib):
    say("sync variant varlen")
    lengths = [1, 300, 0, 777, 256, 1000, 65]
    cu = synth.cu_seqlens_of(lengths)
    T, H, D = int(cu[-1]), 16, 128
    q, k, v = (to_device(x, "f16") for x in synth.make_qkv(1, T, H, D, "f16", seed=77))
    q, k, v = (x.view(T, H, D) for x in (q, k, v))
    tcu = torch.from_numpy(cu).cuda()
    outs = []
    for lib in (fa.library(), sync_lib):
        o = torch.empty_like(q)
        lse = torch.empty((T, H), dtype=torch.float32, device="cuda")
        st = lib.fa_fwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                               lse.data_ptr(), tcu.data_ptr(), len(lengths), max(lengths), T, H,
                               D, ctypes.c_float(0.09), 1, -1, -1, 0,
                               torch.cuda.current_stream().cuda_stream)
        assert st == 0, st
        outs.append((o, lse))
    torch.cuda.synchronize()
    (o1, l1), (o2, l2) = outs
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32))


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_decode_bit_identical(sync_lib, dtype):
    B, H, Sq, Sk, D = 2, 4, 8, 3000, 128
    say("sync variant decode", dtype, (B, H, Sq, Sk, D))
    q, _, _ = synth.make_qkv(B, H, Sq, D, dtype, seed=81)
    _, k, v = synth.make_qkv(B, H, Sk, D, dtype, seed=82)
    tq, tk, tv = (to_device(x, dtype) for x in (q, k, v))
    need = fa.fa_decode_workspace_bytes(B, H, Sq, Sk, D, 1)
    assert need > 0
    outs = []
    for lib in (fa.library(), sync_lib):
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        o = torch.empty_like(tq)
        lse = torch.empty((B, H, Sq), dtype=torch.float32, device="cuda")
        st = lib.fa_decode(tq.data_ptr(), tk.data_ptr(), tv.data_ptr(), o.data_ptr(),
                           lse.data_ptr(), B, H, Sq, Sk, D, ctypes.c_float(0.1), 1, -1, -1,
                           0 if dtype == "f16" else 1, ws.data_ptr(), need,
                           torch.cuda.current_stream().cuda_stream)
        assert st == 0, st
        outs.append((o, lse))
    torch.cuda.synchronize()
    (o1, l1), (o2, l2) = outs
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32))
