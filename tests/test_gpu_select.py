"""The persistent stack kernel's own expert selection (per-wave ranking or
per-wave picks, the candidate merge and the routing weights), run through its
test export on the same logits the oracle gets: 4000 tie-heavy sets per
(E, k) for E in {32, 128, 256, 320, 1024} and k in {1, 4, 8, 12, 16} (k <= E).
The sets draw their values from a few levels (so most experts tie), and
include all-equal sets, duplicated pairs, +0/-0 mixes, NaN (ranked as -inf),
-inf and +inf.  The ids must equal the oracle's top-k bit for bit; the
weights (softmax over the selected logits) and the shared-expert gate
(sigmoid of logit E) must be within 2e-3 of the oracle's wherever the
oracle's are finite.  For E <= 256 and k <= 8 the export also runs the
one-barrier form of the merge (each wave finding the expert of a rank from
the candidates, and the candidates' copied logits) and reports ids of -1 if
it disagrees with the two-barrier form in any id or selected logit bit."""
import numpy as np
import pytest
import torch

import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    import quantized_router_expert_amd as q
    assert torch.cuda.is_available()
    return q


def tie_heavy_sets(E, n, seed):
    rng = np.random.default_rng(seed)
    L = np.zeros((n, E + 1), np.float32)
    for t in range(n):
        levels = rng.standard_normal(int(rng.integers(1, 6))).astype(np.float32)
        L[t, :E] = levels[rng.integers(0, levels.size, E)]
        if t % 5 == 0:
            L[t, rng.integers(0, E, 3)] = rng.standard_normal(3).astype(np.float32)
        if t % 97 == 0:
            L[t, :E] = 0.0                                         # all equal
        if t % 89 == 0:
            L[t, :E] = np.repeat(rng.standard_normal((E + 1) // 2).astype(np.float32), 2)[:E]
        if t % 53 == 0:                                            # +0 and -0 tie
            z = rng.integers(0, E, max(1, E // 3))
            L[t, z] = np.where(rng.random(z.size) < 0.5, np.float32(0.0), np.float32(-0.0))
        if t % 61 == 0:                                            # NaN ranks as -inf
            L[t, rng.integers(0, E, max(1, E // 8))] = np.nan
        if t % 67 == 0:
            L[t, rng.integers(0, E, max(1, E // 8))] = -np.inf
        if t % 71 == 0:
            L[t, rng.integers(0, E, 2)] = np.inf
        if t % 400 == 7:                                           # every logit NaN or -inf
            L[t, :E] = np.where(rng.random(E) < 0.5, np.float32(np.nan), np.float32(-np.inf))
        L[t, E] = rng.standard_normal() * 3.0                      # the shared-gate logit
    return L


CASES = [(E, k) for E in (32, 128, 256, 320, 1024) for k in (1, 4, 8, 12, 16) if k <= E]


@pytest.mark.parametrize("E,k", CASES)
def test_stack_selection_tie_heavy(q, orc, E, k):
    gu.banner(f"persistent-kernel selection E {E} k {k}: 4000 tie-heavy sets")
    n = 4000
    L = tie_heavy_sets(E, n, E * 1000 + k)
    with_gate = (E + k) % 2 == 0
    ids = torch.full((n, k), -2, dtype=torch.int32, device="cuda")
    wts = torch.zeros(n, k, dtype=torch.float32, device="cuda")
    gate = torch.zeros(n, dtype=torch.float32, device="cuda")
    q.moe_test_stack_select(gu.dev(L), n, E, k, with_gate, ids, wts, gate if with_gate else None)
    torch.cuda.synchronize()
    g_ids, g_w, g_g = gu.host(ids), gu.host(wts), gu.host(gate)
    for t in range(n):
        o_ids = orc.topk(L[t, :E], k)
        assert np.array_equal(g_ids[t], o_ids), (t, g_ids[t], o_ids)
        o_w = orc.softmax_selected(L[t, :E], o_ids)
        if np.all(np.isfinite(o_w)):
            gu.assert_f32_within(g_w[t], o_w, f"weights set {t}")
    if with_gate:
        z = L[:, E].astype(np.float64)
        gu.assert_f32_within(g_g, (1.0 / (1.0 + np.exp(-z))).astype(np.float32), "gate")
