"""The C ABI on the host: the library loads, exports every function that
include/*.h declares, validates every argument before touching the GPU, and
counts visible pairs and FLOPs the way the oracle's enumeration does.
No GPU is needed: every call here returns before any HIP call."""
import glob
import math
import os
import re

import pytest

import tiled_attention_11_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

OK, INVALID, UNSUPPORTED, ALIGNMENT, TOO_LARGE = 0, -1, -2, -3, -4

# Fake, well-aligned, non-overlapping device addresses: validation must reject
# the bad argument before anything dereferences them.
Q, K, V, O, L = 1 << 40, 2 << 40, 3 << 40, 4 << 40, 5 << 40


def _declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names.update(re.findall(r"\b(fa_\w+)\s*\(", text))
    return sorted(names)


def test_header_declares_the_abi():
    assert {"fa_fwd", "fa_fwd_flops", "fa_visible_pairs", "fa_strerror", "fa_decode",
            "fa_decode_workspace_bytes", "fa_decode_flops"} <= set(
        _declared_functions())


@pytest.mark.parametrize("name", _declared_functions())
def test_every_declared_symbol_is_exported(name):
    assert hasattr(fa.library(), name), name


def call(q=Q, k=K, v=V, o=O, lse=L, B=2, H=3, S=100, D=128, scale=0.1, mask=1, wl=-1,
         wr=-1, dtype=0):
    return fa.fa_fwd(q, k, v, o, lse, B, H, S, D, scale, mask, wl, wr, dtype, None)


@pytest.mark.parametrize("kw,code", [
    (dict(B=-1), INVALID), (dict(H=-2), INVALID), (dict(S=-5), INVALID),
    (dict(dtype=2), INVALID), (dict(dtype=-1), INVALID),
    (dict(mask=3), INVALID), (dict(mask=-1), INVALID),
    (dict(scale=float("nan")), INVALID), (dict(scale=float("inf")), INVALID),
    (dict(scale=-float("inf")), INVALID),
    (dict(D=32), UNSUPPORTED), (dict(D=96), UNSUPPORTED), (dict(D=256), UNSUPPORTED),
    (dict(D=0), UNSUPPORTED),
    (dict(q=None), INVALID), (dict(k=None), INVALID), (dict(v=None), INVALID),
    (dict(o=None), INVALID),
    (dict(q=Q + 8), ALIGNMENT), (dict(k=K + 2), ALIGNMENT), (dict(v=V + 4), ALIGNMENT),
    (dict(o=O + 1), ALIGNMENT), (dict(lse=L + 2), ALIGNMENT),
    (dict(o=Q), INVALID), (dict(o=K + 1024), INVALID), (dict(o=V - 1024), INVALID),
    (dict(lse=O + 4096), INVALID), (dict(lse=Q), INVALID),
    (dict(S=1 << 23, D=128), TOO_LARGE),              # one head = 2 GiB
    (dict(B=1 << 16, H=1 << 16, S=128), TOO_LARGE),   # grid over 2^31 workgroups
])
def test_rejected_before_launch(kw, code):
    assert call(**kw) == code


@pytest.mark.parametrize("kw", [dict(B=0), dict(H=0), dict(S=0),
                                dict(B=0, q=None, k=None, v=None, o=None, lse=None)])
def test_empty_problem_is_a_no_op(kw):
    assert call(**kw) == OK


def test_strerror():
    for code in (OK, INVALID, UNSUPPORTED, ALIGNMENT, TOO_LARGE, -5):
        assert fa.fa_strerror(code)
    assert fa.fa_strerror(OK) == "success"
    assert "unknown" in fa.fa_strerror(-99)


MASKS = [(0, -1, -1), (1, -1, -1), (2, 0, 0), (2, 1024, 0), (2, 1000, 0), (2, 5, 7),
         (2, -1, 3), (2, 9, -1), (2, -1, -1), (2, -1, 0), (2, 1 << 30, 0), (2, 3, 1 << 30)]
_NAMES = {0: "full", 1: "causal", 2: "window"}


@pytest.mark.parametrize("S", [0, 1, 2, 63, 64, 65, 127, 129, 300, 1000])
@pytest.mark.parametrize("m,wl,wr", MASKS)
def test_visible_pairs_match_oracle_enumeration(orc, S, m, wl, wr):
    assert fa.fa_visible_pairs(S, m, wl, wr) == orc.pair_count(S, _NAMES[m], (wl, wr))


def test_visible_pairs_headline_counts():
    S = 4096
    assert fa.fa_visible_pairs(S, 0) == S * S
    assert fa.fa_visible_pairs(S, 1) == S * (S + 1) // 2
    assert fa.fa_visible_pairs(S, 2, 1024, 0) == 1024 * 1025 // 2 + (S - 1024) * 1025
    assert fa.fa_visible_pairs(S, 2, 1000, 0) == 1000 * 1001 // 2 + (S - 1000) * 1001


def test_flops():
    assert fa.fa_fwd_flops(4, 32, 4096, 128, 1) == 549_890_031_616
    assert fa.fa_fwd_flops(4, 32, 4096, 128, 0) == 4 * 128 * 4 * 32 * 4096 ** 2
    assert fa.fa_fwd_flops(1, 32, 2048, 64, 1) == 4 * 64 * 32 * 2048 * 2049 // 2
    assert fa.fa_fwd_flops(0, 32, 2048, 64, 1) == 0
    assert fa.fa_fwd_flops(-1, 1, 1, 64, 0) == INVALID
    assert fa.fa_fwd_flops(1, 1, 1, 64, 7) == INVALID
    assert fa.fa_fwd_flops(1 << 30, 1 << 30, 1 << 20, 128, 0) == TOO_LARGE


def test_forward_rejects_bad_tensors_on_cpu():
    torch = pytest.importorskip("torch")
    x = torch.zeros(1, 1, 8, 64, dtype=torch.float16)
    with pytest.raises(ValueError):
        fa.forward(x, x, x)          # not on a GPU
    with pytest.raises(ValueError):
        fa.forward(x, x, x[..., :32])
    with pytest.raises(ValueError):
        fa.forward(x.float(), x.float(), x.float())
    assert math.isclose(1 / math.sqrt(64), 0.125)


def test_one_hip_runtime_in_process():
    """libfa binds to the HIP runtime torch loaded, never to a second copy."""
    maps = open("/proc/self/maps").read()
    libs = {line.split()[-1] for line in maps.splitlines() if "libamdhip64" in line}
    assert len(libs) == 1, libs
