"""Structure checks of the seeded synthetic workloads (CPU)."""
import numpy as np
import pytest

from edge_aware_graph_amd import workloads as W


def _is_connected(adj):
    n = adj.shape[0]
    seen = np.zeros(n, bool)
    stack = [0]
    seen[0] = True
    while stack:
        u = stack.pop()
        for v in np.flatnonzero(adj[u]):
            if not seen[v]:
                seen[v] = True
                stack.append(v)
    return seen.all()


def test_delaunay_planar_bounds():
    rng = np.random.default_rng(0)
    for _ in range(5):
        a = W.delaunay_adjacency(rng, 64)
        assert np.array_equal(a, a.T) and not a.diagonal().any()
        m = a.sum() // 2
        assert 64 - 1 <= m <= 3 * 64 - 6
        assert _is_connected(a)


def test_prufer_is_tree():
    rng = np.random.default_rng(1)
    for nb in (2, 3, 10, 64):
        a = W.prufer_tree_adjacency(rng, nb)
        assert np.array_equal(a, a.T) and not a.diagonal().any()
        assert a.sum() // 2 == nb - 1
        assert _is_connected(a)


def test_sbm_densities():
    rng = np.random.default_rng(2)
    a = W.sbm_adjacency(rng, 2000, 2, 0.3, 0.005)
    assert np.array_equal(a, a.T) and not a.diagonal().any()
    # two communities of ~1000: about half the pairs are intra-community
    dens = a.sum() / (2000 * 1999)
    assert 0.5 * (0.3 + 0.005) * 0.9 < dens < 0.5 * (0.3 + 0.005) * 1.1


def test_rgg_mean_degree():
    r = W.rgg_radius(1024, 8.0)
    assert 0.045 < r < 0.056
    rng = np.random.default_rng(3)
    degs = [W.rgg_adjacency(rng, 1024, r).sum(1).mean() for _ in range(4)]
    assert abs(np.mean(degs) - 8.0) < 0.5


@pytest.mark.parametrize("name", ["tiny", "planar", "tree", "sbm"])
def test_batches(name):
    b = W.make_batch(name)
    dims = W.CONFIGS[name].dims
    assert b["X"].shape == (dims.B, dims.n, dims.d)
    assert b["E"].shape == (dims.B, dims.n, dims.n, dims.de)
    assert b["y"].shape == (dims.B, dims.dy)
    assert b["w_e"].shape == (dims.de, dims.H)
    for g in range(dims.B):
        k = int(b["n_real"][g])
        assert np.all(b["mask"][g, :k] == 1) and np.all(b["mask"][g, k:] == 0)
    pm = b["mask"][:, :, None].astype(bool) & b["mask"][:, None, :].astype(bool)
    assert np.all(b["E"][~pm] == 0) and np.all(b["X"][b["mask"] == 0] == 0)
    if dims.dtype == "bf16":
        for k in ("X", "E", "y", "w_q", "w_e"):
            assert np.array_equal(W.bf16_round_array(b[k]), b[k])
    if name == "tiny":
        assert list(b["n_real"]) == [12, 9]
    if name == "sbm":
        assert b["n_real"].min() >= 44 and b["n_real"].max() <= 187
    if name == "tree":
        assert np.all(b["adj"].sum((1, 2)) // 2 == 63)


def test_seeded_determinism():
    a, b = W.make_batch("tiny"), W.make_batch("tiny")
    for k in a:
        assert np.array_equal(a[k], b[k])
    c = W.make_batch("tiny", seed=99)
    assert not np.array_equal(a["X"], c["X"])
