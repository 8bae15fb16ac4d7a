"""Host-side pieces of the Stage-2 module (no GPU): the rank-agreement
statistics used by the step-count ablation."""
import numpy as np

from fp4_quantized_diffusion_amd import stage2


def test_rank_stats_hand_case():
    """Identical orders give rho = tau = 1 and full overlaps; a reversed
    order gives -1 and none."""
    a = np.array([0.3, 1.0, -2.0, 0.5, 4.0])
    s = stage2.rank_stats(a, a * 2 + 1, 2)
    assert s == {"spearman": 1.0, "kendall_tau": 1.0, "top_overlap": 2, "bottom_overlap": 2, "k": 2}
    s = stage2.rank_stats(a, -a, 2)
    assert s["spearman"] == -1.0 and s["kendall_tau"] == -1.0 and s["top_overlap"] == 0 and s["bottom_overlap"] == 0


def test_kendall_tau_brute_force():
    """tau over all pairs, against an explicit double loop with one swap."""
    a = np.array([3.0, 1.0, 2.0, 5.0, 4.0])
    b = np.array([3.0, 2.0, 1.0, 5.0, 4.0])  # one discordant pair (1, 2)
    s = stage2.rank_stats(a, b, 1)
    assert s["kendall_tau"] == round((10 - 2) / 10, 4)
