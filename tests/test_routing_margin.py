"""Near-tie report for grouped routing (reading S9 of the design notes).

Expert and group choices compare logits, which the oracle and the device
read identically.  The one place where a transcendental decides an integer
is the mode-1 group key: the sum of a group's two largest scores, each
evaluated in double and rounded to float32 on both sides.  A device
exponential that differs from the host's in the last double bit can move a
score by one float32 ulp only where the double value lies within one
double ulp of a float32 rounding boundary; that changes a group choice only
where two groups' keys at the k_group boundary are within a few float32 ulps
of each other.  This test measures that margin on the seeded logits of every
grouped workload: exact ties are harmless (both sides compute the same bits
and break them toward the lower group index), and a gap below 1e-9
(relative) other than an exact tie cannot occur between float32 keys.  It
reports the tokens within 4 float32 ulps of a tie (expected: none or a
handful per workload)."""
import numpy as np
import pytest

import oracle
from mixture_experts_ffn_router_amd import workloads as W

FP32_ULP = 2.0 ** -23


def boundary_gaps(keys: np.ndarray, k_group: int) -> np.ndarray:
    """Per token: (k-th largest key - (k+1)-th largest) / k-th largest,
    the relative margin of the last chosen group over the first left out."""
    s = -np.sort(-keys.astype(np.float64), axis=1)
    return (s[:, k_group - 1] - s[:, k_group]) / np.abs(s[:, k_group - 1])


def margin_report(logits, cfg) -> dict:
    keys = oracle.group_keys(logits, cfg.group_count, cfg.group_select_mode,
                             scoring=cfg.scoring)
    gaps = boundary_gaps(keys, cfg.k_group)
    near = (gaps > 0) & (gaps < 4 * FP32_ULP)
    rep = {"tokens": int(gaps.size), "exact_ties": int((gaps == 0).sum()),
           "near_ties": int(near.sum()),
           "min_nonzero_gap": float(gaps[gaps > 0].min()) if (gaps > 0).any() else None}
    print(f"[margin] {cfg.name}: {rep}", flush=True)
    return rep


GROUPED = [(W.DEEPSEEK_GROUPED, 1000 + W.CONFIGS.index(W.DEEPSEEK_GROUPED)),
           (W.EP8_SHARD, 1100 + W.EXTRA.index(W.EP8_SHARD)),
           (W.DEEPSEEK_GROUPED.scaled(name="deepseek_small", M=64, H=256, I=128, E=64), 61),
           (W.MIXTRAL_PREFILL.scaled(name="e256_grouped", M=1300, H=32, I=32, E=256, top_k=8,
                                     scoring="sigmoid", renormalize=False, group_count=8,
                                     k_group=4, group_select_mode=1), 2006)]


@pytest.mark.parametrize("cfg,seed", GROUPED, ids=[c.name for c, _ in GROUPED])
def test_group_boundary_margin(cfg, seed):
    logits = W.make_logits(cfg, seed)
    rep = margin_report(logits, cfg)
    gaps = boundary_gaps(oracle.group_keys(logits, cfg.group_count, cfg.group_select_mode,
                                           scoring=cfg.scoring), cfg.k_group)
    # between float32 keys a nonzero gap is at least one ulp of the larger
    assert not ((gaps > 0) & (gaps < 1e-9)).any()
    assert rep["near_ties"] <= max(2, rep["tokens"] // 1000), rep
