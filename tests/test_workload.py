"""CPU tests of the input generator: its bf16 rounding of drawn values is torch's."""
import numpy as np

from chunked_prefill_paged_ca_amd.workload import make_config, round_to_storage


def test_round_to_storage_matches_torch():
    """The numpy bit-pattern rounding gives exactly torch's float32 -> bfloat16 values on random
    data of several magnitudes, on every exact tie between two bf16 neighbours of one binade
    range, on the largest finite values (some round to infinity), subnormals and signed zeros,
    and with a NaN present (the torch path)."""
    import torch
    rng = np.random.default_rng(7)
    cases = [rng.standard_normal(1 << 18, dtype=np.float32) * np.float32(s) for s in (1e-30, 1.0, 1e30)]
    ties = (np.arange(1, 1 << 16, dtype=np.uint32) << np.uint32(16) | np.uint32(0x8000)).view(np.float32)
    cases.append(ties[np.isfinite(ties)])
    cases.append(np.array([3.3e38, 3.4e38, -3.4e38, 1e-40, -1e-40, 0.0, -0.0], np.float32))
    cases.append(np.array([1.0, np.nan, -2.5], np.float32))
    for a in cases:
        ref = torch.from_numpy(a).to(torch.bfloat16).to(torch.float32).numpy()
        got = round_to_storage(a, "bf16")
        assert np.array_equal(ref.view(np.uint32), got.view(np.uint32))
    assert round_to_storage(cases[1], "fp32") is not None


def test_history_is_seeded_and_rounded():
    wl = make_config(2)
    k1, v1 = wl.history(3)
    k2, v2 = wl.history(3)
    assert np.array_equal(k1, k2) and np.array_equal(v1, v2)
    assert k1.shape == (int(wl.num_computed[3]), 8, 128)
    assert np.all((k1.view(np.uint32) & np.uint32(0xFFFF)) == 0)
