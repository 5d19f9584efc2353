"""Statistics helpers for the oracle's distribution tests."""
import numpy as np
from scipy import stats


def chi2_pvalue(counts, probs, min_expected=5.0):
    """Pearson chi-square goodness of fit of `counts` to cell probabilities
    `probs`, pooling cells whose expected count is below `min_expected` into
    one cell.  Cells with zero probability must have zero counts (checked)."""
    counts = np.asarray(counts, dtype=np.float64).ravel()
    probs = np.asarray(probs, dtype=np.float64).ravel()
    assert counts.shape == probs.shape
    assert abs(probs.sum() - 1.0) < 1e-9, probs.sum()
    impossible = probs <= 0.0
    assert counts[impossible].sum() == 0, "an outcome of probability zero occurred"
    n = counts.sum()
    exp = probs * n
    small = (exp < min_expected) & ~impossible
    big = ~small & ~impossible
    obs_cells = list(counts[big])
    exp_cells = list(exp[big])
    if small.any():
        obs_cells.append(counts[small].sum())
        exp_cells.append(exp[small].sum())
    obs_cells = np.array(obs_cells)
    exp_cells = np.array(exp_cells)
    chi2 = float(((obs_cells - exp_cells) ** 2 / exp_cells).sum())
    dof = len(obs_cells) - 1
    return chi2, float(stats.chi2.sf(chi2, dof)), dof


def total_variation(freq, probs):
    return 0.5 * float(np.abs(np.asarray(freq) - np.asarray(probs)).sum())
