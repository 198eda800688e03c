"""Generator determinism and structure of the seeded synthetic inputs (CPU)."""
import json
import os

import numpy as np

import workloads

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "input_sha256.json")


def test_input_bytes_are_stable():
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "make_input_hashes", os.path.join(os.path.dirname(GOLDEN), "make_input_hashes.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    with open(GOLDEN) as f:
        assert mod.hashes() == json.load(f)


def test_trmm_input_structure():
    w = workloads.TrmmWorkload("t", 300, 40, 1.0, 256, 4)
    A_cm, B_cm = workloads.trmm_inputs(w)
    A = A_cm.T                     # logical [row, col]
    assert np.all(np.triu(A, 1) == 0)
    d = np.diag(A).astype(np.float64)
    assert d.min() >= 0.5 and d.max() <= 1.5
    low = A[np.tril_indices(300, -1)].astype(np.float64)
    assert low.min() >= -1 and low.max() <= 1 and np.abs(low).mean() > 0.4
    assert B_cm.shape == (40, 300)


def test_gemm_inputs_beta_zero_C_is_nan():
    A, Bt, C = workloads.gemm_inputs(workloads.WORKLOADS["hgemm_256"])
    assert A.dtype == np.float16 and Bt.shape == (256, 256) and np.isnan(C).all()
    A, Bt, C = workloads.gemm_inputs(workloads.WORKLOADS["hgemm_1000_ragged"])
    assert C.dtype == np.float16 and np.isfinite(C).all()


def test_sample_indices_include_corners():
    ri, cj = workloads.sample_indices(3, 8192, 8192)
    assert ri.size == 1024
    assert set(zip(ri[-4:].tolist(), cj[-4:].tolist())) == {(0, 0), (0, 8191), (8191, 0), (8191, 8191)}


def test_bf16_rounding_matches_torch():
    """The generator's bf16 rounding (nearest even on the dropped bits) agrees
    with torch's float32 -> bfloat16 conversion, ties and specials included."""
    import torch
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.uniform(-3, 3, 20000).astype(np.float32),
                        np.array([1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 0.0, -0.0,
                                  np.inf, -np.inf, 3e38, 1e-40], np.float32)])
    ours = workloads.to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert workloads.to_bf16_bits(np.array([1 + 2 ** -8], np.float32))[0] == 0x3F80   # tie to even
    nanbits = workloads.to_bf16_bits(np.array([np.nan], np.float32))[0]
    assert (nanbits & 0x7F80) == 0x7F80 and (nanbits & 0x7F) != 0
