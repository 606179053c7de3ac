"""GPU parity of moe_permute on its own (top-k modes), bit for bit against the
oracle's dispatch.

The permutation has two launch plans: up to 8192 assignments (T*k) a single
launch in which every workgroup counts all assignments itself; above that a
counting launch followed by the scan + scatter.  The cases sit on both sides
of that limit, with skewed expert choices, with and without capacity
dropping, and with up to 256 experts and 16 slots per token.  x_perm rows
must be exact copies of the token rows.
"""
import numpy as np
import pytest
import torch

import oracle
from mixture_experts_layer_topkrouter_amd import moe
from mixture_experts_layer_topkrouter_amd import workloads as W

CASES = [  # T, k, E, capacity factor (0 = dropless), d
    (4096, 2, 8, 0.0, 64),      # 8192 assignments: single launch, dropless
    (8192, 1, 64, 1.0, 32),     # 8192: single launch, drops
    (8193, 1, 8, 0.0, 32),      # 8193: counting launch + scan/scatter
    (2731, 3, 256, 1.25, 64),   # 8193, 256 experts, drops
    (1000, 16, 37, 0.5, 40),    # 16 slots per token, heavy drops, single launch
    (3, 2, 4, 0.0, 8),          # fewer tokens than one workgroup takes
    (12000, 4, 256, 1.25, 8),   # [blocks x E] table past LDS: count, scan, scatter launches; drops
    (9000, 6, 200, 0.0, 520),   # the same path dropless, 2-KB rows
    (100, 1, 4, 1.2, 8),        # cf * T * k / E = 30 exactly; 1.2 has no exact float32 value
    (1000, 1, 4, 1.1, 16),      # 275 exactly; likewise for 1.1
]


def skewed_choices(rng, T, k, E):
    """k distinct experts per token, drawn with Zipf-like weights so that a few
    experts receive most assignments."""
    p = 1.0 / np.arange(1, E + 1) ** 1.1
    p /= p.sum()
    return np.stack([rng.choice(E, size=k, replace=False, p=p) for _ in range(T)]).astype(np.int32)


@pytest.mark.gpu
@pytest.mark.parametrize("T,k,E,cf,d", CASES)
def test_permute_matches_oracle_dispatch(T, k, E, cf, d):
    rng = np.random.default_rng(T * 7 + k * 131 + E)
    idx = skewed_choices(rng, T, k, E)
    x = rng.standard_normal((T, d)).astype(np.float32)
    cfg = moe.MoeConfig(T, d, E, k, 8, 0, cf, 0, W.F32, W.GELU, W.SOFTMAX_ALL)
    rows = moe.max_rows(cfg)
    dev = torch.device("cuda")
    d_x = torch.from_numpy(x).to(dev)
    d_idx = torch.from_numpy(idx).to(dev)
    x_perm = torch.full((rows, d), float("nan"), device=dev)
    row_token = torch.full((rows,), -7, dtype=torch.int32, device=dev)
    slot_row = torch.full((T, k), -7, dtype=torch.int32, device=dev)
    cnt = torch.empty(E, dtype=torch.int32, device=dev)
    load = torch.empty(E, dtype=torch.int32, device=dev)
    off = torch.empty(E + 1, dtype=torch.int32, device=dev)
    nb = moe.permute_scratch_bytes(cfg)
    scratch = torch.empty(max(nb, 256), dtype=torch.uint8, device=dev)
    moe.permute(cfg, d_x, x_perm, row_token, slot_row, cnt, load, off, topk_idx=d_idx, scratch=scratch)
    torch.cuda.synchronize()

    ref = oracle.dispatch_topk(idx, E, oracle.capacity(cf, T, k, E))
    n = ref.n_rows
    assert np.array_equal(off.cpu().numpy(), ref.expert_offset)
    assert np.array_equal(cnt.cpu().numpy(), ref.expert_count)
    assert np.array_equal(load.cpu().numpy(), ref.expert_load)
    assert np.array_equal(slot_row.cpu().numpy(), ref.slot_row)
    rt = row_token.cpu().numpy()
    assert np.array_equal(rt[:n], ref.row_token)
    assert np.array_equal(x_perm[:n].cpu().numpy(), x[ref.row_token])
    if cf > 0:
        assert (ref.slot_row < 0).any(), "the case was meant to drop assignments"
