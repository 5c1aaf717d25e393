"""Shared test helpers: moving seeded inputs onto the device and comparing the HIP
verifier's outputs with the oracle's, slot by slot, allowing differences only where
either side flags a near-tie."""
import numpy as np

import oracle

TIE_MASK = oracle.TIE_MASK
OVERFLOW = 64


def to_device(arr, device):
    import torch
    arr = np.ascontiguousarray(arr)
    if arr.dtype == np.uint16:
        return torch.from_numpy(arr.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(arr).to(device)


def dtype_name(arr):
    return "bf16" if arr.dtype == np.uint16 else "f32"


def compare_verify(gpu, ref, b, seqs=None, allow_overflow=False):
    """gpu: dict of numpy arrays from the HIP path; ref: oracle dict for the same
    sequences (rows of ref correspond to `seqs` rows of gpu). Returns stats dict."""
    S = ref["accept_len"].shape[0]
    seqs = list(range(S)) if seqs is None else list(seqs)
    near = 0
    exact = 0
    for a, s in enumerate(seqs):
        gflags = gpu["diag"][s, :, 3].astype(np.int64)
        rflags = ref["diag"][a, :, 3].astype(np.int64)
        if not allow_overflow:
            assert not np.any(gflags & OVERFLOW), (s, gflags)
        # uniforms are bit-identical (Philox on both sides); ratios agree to fp64 rounding
        np.testing.assert_array_equal(gpu["diag"][s, :, 0], ref["diag"][a, :, 0].astype(np.float32))
        np.testing.assert_array_equal(gpu["diag"][s, :, 2], ref["diag"][a, :, 2].astype(np.float32))
        tie_seen = False
        ok_seq = True
        for i in range(b):
            tie = bool((gflags[i] | rflags[i]) & TIE_MASK)
            if gpu["slot_accept"][s, i] != ref["slot_accept"][a, i]:
                assert tie, (s, i, "accept decision differs without a near-tie")
                tie_seen = True
                ok_seq = False
                break
            np.testing.assert_allclose(gpu["diag"][s, i, 1], np.float32(ref["diag"][a, i, 1]),
                                       rtol=1e-6, atol=0)
            if tie:
                tie_seen = True
        if tie_seen:
            near += 1
        if ok_seq and not tie_seen:
            assert gpu["accept_len"][s] == ref["accept_len"][a], (s, gpu["accept_len"][s], ref["accept_len"][a])
            np.testing.assert_array_equal(gpu["out_tokens"][s], ref["out_tokens"][a], err_msg=f"seq {s}")
            assert gpu["resampled"][s] == ref["resampled"][a], s
            exact += 1
    return dict(exact=exact, near_tie=near)
