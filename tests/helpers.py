"""Helpers shared by the GPU parity tests (device transfer, tolerance rule, verify parity)."""
import numpy as np
import torch

from strided_verify_propose_amd import synth

DEV = "cuda:0"
RTOL = {"bf16": 2e-2, "f32": 1e-5}


def to_dev(a, dtype=None):
    """NumPy -> device tensor.  uint16 arrays are bf16 bit patterns."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(DEV)
    t = torch.from_numpy(a)
    return t.to(DEV) if dtype is None else t.to(DEV, dtype)


def to_np(t):
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def as_f64(a):
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return synth.bf16_bits_to_f32(a).astype(np.float64)
    return a.astype(np.float64)


def assert_close(gpu, ref, rtol, what=""):
    """|gpu - ref| <= rtol |ref| + rtol RMS(ref), elementwise."""
    gpu = as_f64(gpu)
    ref = np.asarray(ref, np.float64)
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    err = np.abs(gpu - ref)
    bound = rtol * np.abs(ref) + rtol * rms
    bad = err > bound
    assert not bad.any(), (f"{what}: {int(bad.sum())}/{bad.size} outside tolerance; worst "
                           f"err {err.max():.3e} (rms ref {rms:.3e})")
    return float((err / (np.abs(ref) + rms + 1e-300)).max()) if ref.size else 0.0


def verify_parity(gpu: dict, ref: dict, N: int):
    """Bit-exact comparison of decisions and ids, skipping draws the oracle flags as
    within 1e-6 of a threshold and everything after them in the same request.
    Returns (number of compared decisions/ids, number excluded)."""
    B = ref["n_accept"].shape[0]
    g = {k: to_np(v) for k, v in gpu.items()}
    compared = excluded = 0
    assert np.array_equal(g["argmax_ids"], ref["argmax_ids"]), "argmax ids differ"
    for b in range(B):
        n_ref = int(ref["n_accept"][b])
        evaluated = min(n_ref + 1, N - 1)
        flagged = [i for i in range(evaluated) if ref["accept_flag"][b, i]]
        upto = flagged[0] if flagged else evaluated
        assert np.array_equal(g["accept"][b, :upto], ref["accept"][b, :upto]), f"accept bits, request {b}"
        compared += upto
        if flagged:
            excluded += 1
        else:
            assert np.array_equal(g["accept"][b], ref["accept"][b]), f"accept bits, request {b}"
            assert int(g["n_accept"][b]) == n_ref, f"n_accept, request {b}"
            compared += 1
            if ref["residual_flag"][b]:
                excluded += 1
            else:
                assert int(g["next_token"][b]) == int(ref["next_token"][b]), f"next_token, request {b}"
                compared += 1
        for j in range(N):
            if ref["sample_flag"][b, j]:
                excluded += 1
            else:
                assert int(g["sampled_ids"][b, j]) == int(ref["sampled_ids"][b, j]), \
                    f"sampled id, request {b} row {j}"
                compared += 1
    return compared, excluded
