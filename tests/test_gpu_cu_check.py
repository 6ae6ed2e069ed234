"""The device-side check of cu_seqlens contents (cdr_check_cu_seqlens), on a GPU."""
import pytest
import torch

import chunked_gated_delta_chunk_amd as cdr

pytestmark = pytest.mark.gpu

# label, offsets, T, expected result (0 = valid, else first bad index + 1)
CASES = [
    ("valid", [0, 400, 1024, 2024, 4072, 8168], 8168, 0),
    ("valid_empty_sequences", [0, 0, 5, 5, 9], 9, 0),
    ("valid_one_sequence", [0, 7], 7, 0),
    ("valid_all_empty", [0, 0, 0], 0, 0),
    ("first_not_zero", [1, 5, 9], 9, 1),
    ("decreasing", [0, 5, 3, 9], 9, 3),
    ("last_not_T", [0, 5, 8], 9, 3),
    ("beyond_T", [0, 12, 9], 9, 2),
    ("negative", [0, -2, 9], 9, 2),
    ("first_of_several", [0, 6, 4, 2, 9], 9, 3),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_cu_seqlens_check(case):
    label, cu, T, expected = case
    print(f"[cu check] {label}", flush=True)
    t = torch.tensor(cu, dtype=torch.int32, device="cuda:0")
    assert cdr.check_cu_seqlens(t, T) == expected


def test_cu_seqlens_check_many_sequences():
    """More offsets than threads in the check's workgroup: the first failure wins."""
    n = 3000
    cu = torch.arange(n + 1, dtype=torch.int32) * 2
    T = int(cu[-1])
    dev = cu.to("cuda:0")
    assert cdr.check_cu_seqlens(dev, T) == 0
    bad = cu.clone()
    bad[2500] = bad[2499] - 1     # decreasing at 2500
    bad[2900] = bad[2899] - 1     # and later again
    assert cdr.check_cu_seqlens(bad.to("cuda:0"), T) == 2501
    assert cdr.check_cu_seqlens(dev, T + 1) == n + 1
