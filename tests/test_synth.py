"""The seeded input generator: determinism, rounding, outlier rows (CPU only)."""
import numpy as np
import torch

import synth


def test_same_seed_same_bytes():
    a = synth.make_qkv(1, 2, 77, 64, "f16", seed=4)
    b = synth.make_qkv(1, 2, 77, 64, "f16", seed=4)
    c = synth.make_qkv(1, 2, 77, 64, "f16", seed=5)
    assert synth.digest(*a) == synth.digest(*b)
    assert synth.digest(*a) != synth.digest(*c)
    for x in a:
        assert x.dtype == np.uint16 and x.shape == (1, 2, 77, 64) and x.flags.c_contiguous


def test_f16_rounding_matches_torch():
    x = np.random.default_rng(0).standard_normal(100000, dtype=np.float32) * 300
    got = synth.f32_to_bits(x, "f16")
    ref = torch.from_numpy(x).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref)


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(1)
    x = rng.standard_normal(200000, dtype=np.float32) * 50
    # exact ties: low 16 bits 0x8000, with even and odd kept halves
    ties = (rng.integers(0, 1 << 6, 1000, dtype=np.uint32) << np.uint32(17)) | np.uint32(0x3F808000)
    ties2 = ties | np.uint32(0x10000)
    x = np.concatenate([x, ties.view(np.float32), ties2.view(np.float32),
                        np.array([0.0, -0.0, 1e-40, -3.4e38], np.float32)])
    got = synth.f32_to_bits(x, "bf16")
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref)


def test_outlier_rows():
    S = 300
    base = synth.make_qkv(2, 3, S, 16, "bf16", seed=9)
    out = synth.make_qkv(2, 3, S, 16, "bf16", seed=9, outlier_frac=0.01, outlier_scale=20.0)
    assert np.array_equal(base[0], out[0]) and np.array_equal(base[2], out[2])
    changed = np.any(base[1] != out[1], axis=-1)          # [B, H, S]
    assert np.all(changed.sum(axis=-1) == 3)              # round(0.01 * 300)
    kb = torch.from_numpy(base[1].view(np.int16).copy()).view(torch.bfloat16).float()
    ko = torch.from_numpy(out[1].view(np.int16).copy()).view(torch.bfloat16).float()
    ratio = (ko[torch.from_numpy(changed)] / kb[torch.from_numpy(changed)]).numpy()
    assert np.all(np.abs(ratio - 20.0) < 0.2)


def test_workload_table():
    for name, w in synth.WORKLOADS.items():
        assert w["dtype"] in ("f16", "bf16") and w["D"] in (64, 128), name
        assert w["mask"] in ("full", "causal", "window"), name
    h = synth.WORKLOADS[synth.HEADLINE]
    assert (h["B"], h["H"], h["S"], h["D"], h["mask"]) == (4, 32, 4096, 128, "causal")
