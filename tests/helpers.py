"""Shared test helpers: moving seeded inputs onto the device and comparing the HIP
verifier's outputs with the oracle's, slot by slot, allowing differences only where
either side flags a near-tie on a decision that matters."""
import numpy as np

import oracle

TIE_MASK = oracle.TIE_MASK
# A near-tie of these kinds can change the slot's accept decision: the accept test
# itself, or a top-p boundary that changes a filtered set and with it the ratio.
DECISION_TIES = oracle.TIE_ACCEPT | oracle.TIE_TOPP_P | oracle.TIE_TOPP_Q
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
    """Compare the HIP verifier's outputs with the oracle's.

    gpu: dict of numpy arrays from the HIP path; ref: the oracle's dict for the same
    sequences (row a of ref is row seqs[a] of gpu).

    Rules (a mismatch is allowed only where a near-tie decides it):
      * the uniforms of every slot are bit-identical;
      * every slot whose decision neither side flags (accept tie or top-p tie) has the
        same raw accept decision and a ratio within 1e-6 relative, whatever its
        position in the block;
      * the decisive slots of a sequence are slot 0, the oracle's accepted slots and
        its first rejected slot. If none of them carries a near-tie flag on either
        side, accept_len, every output token and the resample are equal. Otherwise,
        let f be the first flagged decisive slot: the tokens before f are equal, the
        HIP accept_len is at least f, and the sequence is counted as excused.
    Flags on slots after the first rejection decide nothing and excuse nothing.

    Returns dict(exact, excused, flagged_slots, excused_at) where excused_at lists
    (sequence, slot, flag bits) of every excused sequence.
    """
    S = ref["accept_len"].shape[0]
    seqs = list(range(S)) if seqs is None else list(seqs)
    exact = 0
    excused_at = []
    flagged_slots = 0
    for a, s in enumerate(seqs):
        gflags = gpu["diag"][s, :, 3].astype(np.int64)
        rflags = ref["diag"][a, :, 3].astype(np.int64)
        if not allow_overflow:
            assert not np.any(gflags & OVERFLOW), (s, gflags)
        # uniforms are bit-identical (Philox on both sides)
        np.testing.assert_array_equal(gpu["diag"][s, :, 0], ref["diag"][a, :, 0].astype(np.float32))
        np.testing.assert_array_equal(gpu["diag"][s, :, 2], ref["diag"][a, :, 2].astype(np.float32))
        both = gflags | rflags
        flagged_slots += int(np.count_nonzero(both & TIE_MASK))
        for i in range(b):
            if both[i] & DECISION_TIES:
                continue
            assert gpu["slot_accept"][s, i] == ref["slot_accept"][a, i], \
                (s, i, "accept decision differs without a near-tie")
            np.testing.assert_allclose(gpu["diag"][s, i, 1], np.float32(ref["diag"][a, i, 1]),
                                       rtol=1e-6, atol=0, err_msg=f"ratio of seq {s} slot {i}")
        n_ref = int(ref["accept_len"][a])
        decisive = range(min(n_ref, b - 1) + 1)
        f = next((i for i in decisive if both[i] & TIE_MASK), None)
        if f is None:
            assert gpu["accept_len"][s] == ref["accept_len"][a], (s, gpu["accept_len"][s], n_ref)
            np.testing.assert_array_equal(gpu["out_tokens"][s], ref["out_tokens"][a], err_msg=f"seq {s}")
            assert gpu["resampled"][s] == ref["resampled"][a], s
            exact += 1
        else:
            np.testing.assert_array_equal(gpu["out_tokens"][s, :f], ref["out_tokens"][a, :f],
                                          err_msg=f"seq {s} before its near-tie at slot {f}")
            assert gpu["accept_len"][s] >= f, (s, f, gpu["accept_len"][s])
            excused_at.append((int(s), int(f), int(both[f])))
    return dict(exact=exact, excused=len(excused_at), flagged_slots=flagged_slots, excused_at=excused_at)


def assert_mostly_exact(st, S, max_excused=1):
    """Every sequence compared exactly, except at most `max_excused` excused by a
    near-tie on a decisive slot (each one listed in the message)."""
    assert st["exact"] + st["excused"] == S, st
    assert st["excused"] <= max_excused, st
