"""Seeded synthetic inputs for draft-tree construction.

This module is shared by the tests, the benchmark and the smoke check. It
holds input generation only: Gaussian draft-logit rows, bf16 rounding, and
the target-token draws that stand in for the target model's argmax. It
computes nothing that the tree builder computes (no normaliser, no ranking,
no prefix selection), and it imports neither the oracle nor the HIP binding.

Shapes follow the pages' workloads: L = 15 draft positions and a ~152k
vocabulary (SparklingTree post, "Step 1: Sorting the DFlash marginals"),
node budgets 64/128/256 (DDTree explainer, section 7 "Experiments": budget
trade-off). The value distributions (per-row sigma ~ U[lo, hi] Gaussian,
optional planted peak) are synthetic stand-ins for drafter rows; the pages
give none.

Every request b of configuration c with seed s draws from its own stream
``numpy.random.default_rng(SeedSequence([c, s, b]))``; target draws use the
stream ``SeedSequence([c, s, b, 1])``. Requests are therefore independent
of the batch size they are generated in.
"""

from __future__ import annotations

import numpy as np

DTYPE_BF16 = 0
DTYPE_F32 = 1

# name -> parameters. V=151936 is the Qwen3 vocabulary of the pages' targets.
CONFIGS = {
    1: dict(batch=1, L=15, V=1024, B=32, dtype=DTYPE_F32, sigma=(1.0, 6.0),
            peak=False, targets="fresh_argmax"),
    2: dict(batch=1, L=15, V=151936, B=64, dtype=DTYPE_BF16, sigma=(1.0, 6.0),
            peak=True, targets="drafter"),
    3: dict(batch=64, L=15, V=151936, B=128, dtype=DTYPE_BF16, sigma=(1.0, 6.0),
            peak=True, targets="drafter"),
    5: dict(batch=256, L=15, V=151936, B=256, dtype=DTYPE_BF16, sigma=(0.5, 8.0),
            peak=False, targets="drafter"),
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 with round-to-nearest-even; returns uint16 bits.

    Finite inputs only (the generators never produce inf/NaN).
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _rng(cfg_id: int, seed: int, b: int, stream: int | None = None) -> np.random.Generator:
    key = [int(cfg_id), int(seed), int(b)] + ([] if stream is None else [int(stream)])
    return np.random.default_rng(np.random.SeedSequence(key))


def request_rows(cfg_id: int, seed: int, b: int, *, L: int, V: int, sigma, peak: bool,
                 dtype: int) -> np.ndarray:
    """Draft logits of one request, shape [L, V]: uint16 bf16 bits or float32."""
    rng = _rng(cfg_id, seed, b)
    lo, hi = sigma
    s = rng.uniform(lo, hi, L).astype(np.float32)
    g = rng.standard_normal((L, V), dtype=np.float32)
    x = (s[:, None] * g).astype(np.float32)
    if peak:
        # Planted peak: one token per row sits U[2,10] above the row's Gaussian max.
        pid = rng.integers(0, V, L)
        off = rng.uniform(2.0, 10.0, L).astype(np.float32)
        rowmax = x.max(axis=1)
        x[np.arange(L), pid] = (rowmax + off).astype(np.float32)
    if dtype == DTYPE_BF16:
        return f32_to_bf16_bits(x)
    return x


def make_logits(cfg_id: int, seed: int = 0, *, batch: int | None = None, first: int = 0,
                L: int | None = None, V: int | None = None) -> np.ndarray:
    """Logits [batch, L, V] for requests first .. first+batch-1 of a configuration."""
    c = CONFIGS[cfg_id]
    batch = c["batch"] if batch is None else batch
    L = c["L"] if L is None else L
    V = c["V"] if V is None else V
    dt = np.uint16 if c["dtype"] == DTYPE_BF16 else np.float32
    out = np.empty((batch, L, V), dtype=dt)
    for i in range(batch):
        out[i] = request_rows(cfg_id, seed, first + i, L=L, V=V, sigma=c["sigma"],
                              peak=c["peak"], dtype=c["dtype"])
    return out


def logits_as_f64(logits: np.ndarray, dtype: int) -> np.ndarray:
    """Exact float64 values of generated logits (bf16 bits or float32)."""
    if dtype == DTYPE_BF16:
        return bf16_bits_to_f32(logits).astype(np.float64)
    return np.asarray(logits, dtype=np.float32).astype(np.float64)


def drafter_draws(cfg_id: int, seed: int, logits: np.ndarray, dtype: int, *,
                  first: int = 0) -> np.ndarray:
    """One sequence Y ~ Q per request, shape [batch, L+1] int32.

    Y_d for d = 1..L is drawn from softmax(x_d) by the Gumbel-max rule
    (argmax of x_d[v] + G_v with G_v standard Gumbel, in float64); Y_{L+1}
    is uniform over the vocabulary. A tree node at depth d then receives the
    target token Y_{d+1} (root: Y_1), so a node is reached by the greedy walk
    exactly when the draft agrees with Y along its path, which happens with
    probability equal to the node's prefix probability under the drafter's
    factorised distribution (DDTree explainer, section 2 and Proposition 1).
    """
    batch, L, V = logits.shape
    out = np.empty((batch, L + 1), dtype=np.int32)
    for i in range(batch):
        rng = _rng(cfg_id, seed, first + i, stream=1)
        x = logits_as_f64(logits[i], dtype)
        u = rng.random((L, V))
        # Gumbel(0,1) = -log(-log U); U in (0,1) with probability one.
        g = -np.log(-np.log(np.clip(u, 1e-300, None)))
        out[i, :L] = np.argmax(x + g, axis=1).astype(np.int32)
        out[i, L] = int(rng.integers(0, V))
    return out


def node_targets_from_depths(Y: np.ndarray, depths: np.ndarray, num_nodes: np.ndarray,
                             B: int) -> np.ndarray:
    """Per-node target tokens [batch, B+1]: root gets Y_1, a depth-d node Y_{d+1}.

    Stand-in for the target model's argmax at each tree position. Entries past
    num_nodes are unused by the walk and set to 0.
    """
    batch = Y.shape[0]
    out = np.zeros((batch, B + 1), dtype=np.int32)
    for i in range(batch):
        n = int(num_nodes[i])
        out[i, 0] = Y[i, 0]
        if n:
            out[i, 1:n + 1] = Y[i, np.asarray(depths[i, :n], dtype=np.int64)]
    return out


def fresh_argmax_targets(cfg_id: int, seed: int, batch: int, B: int, V: int, *,
                         first: int = 0) -> np.ndarray:
    """Targets independent of the tree: argmax of fresh 4*N(0,1) logits per node.

    Shape [batch, B+1]; ties go to the lowest index (numpy.argmax).
    """
    out = np.empty((batch, B + 1), dtype=np.int32)
    for i in range(batch):
        rng = _rng(cfg_id, seed, first + i, stream=1)
        g = 4.0 * rng.standard_normal((B + 1, V))
        out[i] = np.argmax(g, axis=1).astype(np.int32)
    return out


# ---------------------------------------------------------------------------
# TreeSpark parent-conditioned expansion (TreeSpark README, item 1: one
# backbone pass gives per-depth vocabulary logits l_d; a first-order Markov
# head adds W . e(t_u) for parent token t_u; k = 4, 7 depths, N = 32 packed
# non-root nodes; the model width 2560 is Qwen3-4B's hidden size).
TREESPARK = dict(batch=32, D=7, V=151936, H=2560, k=4, F=4, N=32, sigma=(1.0, 6.0), wscale=0.02)
CFG_TREESPARK = 4


def treespark_backbone(seed: int, b: int, *, D: int, V: int, sigma=(1.0, 6.0)) -> np.ndarray:
    """Backbone logits of one request, [D, V] bf16 bits: per-depth sigma ~ U[lo, hi] Gaussian."""
    rng = _rng(CFG_TREESPARK, seed, b)
    lo, hi = sigma
    s = rng.uniform(lo, hi, D).astype(np.float32)
    g = rng.standard_normal((D, V), dtype=np.float32)
    return f32_to_bf16_bits((s[:, None] * g).astype(np.float32))


def treespark_matrix(seed: int, which: int, *, V: int, H: int, wscale: float = 0.02) -> np.ndarray:
    """Head weight (which = 2) or embedding table (which = 3): [V, H] bf16 bits, N(0, wscale^2)."""
    assert which in (2, 3)
    rng = _rng(CFG_TREESPARK, seed, 0, stream=which)
    out = np.empty((V, H), dtype=np.uint16)
    step = 8192  # generate in row blocks to bound the float32 temporary
    for r0 in range(0, V, step):
        r1 = min(V, r0 + step)
        out[r0:r1] = f32_to_bf16_bits(
            (rng.standard_normal((r1 - r0, H), dtype=np.float32) * np.float32(wscale)).astype(np.float32))
    return out


def treespark_anchor(seed: int, b: int, *, V: int) -> int:
    """The anchor (root) token of request b."""
    return int(_rng(CFG_TREESPARK, seed, b, stream=4).integers(0, V))


def treespark_inputs(seed: int = 0, *, batch: int | None = None, first: int = 0, D: int | None = None,
                     V: int | None = None, H: int | None = None, sigma=None, wscale: float | None = None):
    """(backbone [batch, D, V] bf16 bits, W [V, H] bf16 bits, E [V, H] bf16 bits, anchor [batch] int32)."""
    c = TREESPARK
    batch = c["batch"] if batch is None else batch
    D = c["D"] if D is None else D
    V = c["V"] if V is None else V
    H = c["H"] if H is None else H
    sigma = c["sigma"] if sigma is None else sigma
    wscale = c["wscale"] if wscale is None else wscale
    bb = np.stack([treespark_backbone(seed, first + b, D=D, V=V, sigma=sigma) for b in range(batch)])
    W = treespark_matrix(seed, 2, V=V, H=H, wscale=wscale)
    E = treespark_matrix(seed, 3, V=V, H=H, wscale=wscale)
    anchor = np.array([treespark_anchor(seed, first + b, V=V) for b in range(batch)], dtype=np.int32)
    return bb, W, E, anchor


# SparklingTree (SparklingTree post): the batch-64 drafter rows, a top-C
# pre-filter of C = 128 and a node budget of 64 (the post's reported setting),
# and a first-order Markov head in low-rank form: delta(p, v) = W1[p] . W2t[v]
# with rank R = 256 (extraction W1 and projection W2, the latter stored
# transposed). No trained head exists here: the factors are random with
# std(delta) ~ 0.5, a bias small beside the logits' spread.
SPARKLING = dict(batch=64, L=15, V=151936, B=64, C=128, R=256, wscale=0.177)
CFG_SPARKLING = 6


def sparkling_factor(seed: int, which: int, *, V: int, R: int, wscale: float) -> np.ndarray:
    """W1 (which = 1) or W2t (which = 2): [V, R] bf16 bits, N(0, wscale^2)."""
    assert which in (1, 2)
    rng = _rng(CFG_SPARKLING, seed, 0, stream=which)
    out = np.empty((V, R), dtype=np.uint16)
    step = 16384
    for r0 in range(0, V, step):
        r1 = min(V, r0 + step)
        out[r0:r1] = f32_to_bf16_bits(
            (rng.standard_normal((r1 - r0, R), dtype=np.float32) * np.float32(wscale)).astype(np.float32))
    return out


def sparkling_inputs(seed: int = 0, *, batch: int | None = None, first: int = 0, L: int | None = None,
                     V: int | None = None, R: int | None = None, wscale: float | None = None):
    """(logits [batch, L, V] bf16 bits (the batch-64 workload's rows), W1 [V, R], W2t [V, R] bf16 bits)."""
    c = SPARKLING
    batch = c["batch"] if batch is None else batch
    L = c["L"] if L is None else L
    V = c["V"] if V is None else V
    R = c["R"] if R is None else R
    wscale = c["wscale"] if wscale is None else wscale
    c3 = CONFIGS[3]
    x = np.stack([request_rows(CFG_SPARKLING, seed, first + b, L=L, V=V, sigma=c3["sigma"],
                               peak=c3["peak"], dtype=c3["dtype"]) for b in range(batch)])
    return x, sparkling_factor(seed, 1, V=V, R=R, wscale=wscale), sparkling_factor(seed, 2, V=V, R=R,
                                                                                 wscale=wscale)


# DSpark budget workload: 256 active requests with blocks of 16 guesses (the
# long end of the 4-16 token blocks the pages report), and the DSpark guide's
# made-up step cost of 25 ms plus 0.1 ms per verified token.
DSPARK = dict(batch=256, P=16, c0=25.0, c1=0.1)
CFG_DSPARK = 7


def dspark_inputs(seed: int = 0, *, batch: int | None = None, P: int | None = None,
                  c0: float | None = None, c1: float | None = None):
    """(conf [batch, P] float32, cost [batch * (P + 1) + 1] float32 ms).

    conf[b][p] = clip(u_b - delta_b * p + N(0, 0.05^2), 0.01, 0.999) with a
    per-request level u_b ~ U[0.35, 0.98] and decay delta_b ~ U[0, 0.06]:
    confident and unsure requests side by side, each falling along its block.
    cost[T] = c0 + c1 * T.
    """
    c = DSPARK
    batch = c["batch"] if batch is None else batch
    P = c["P"] if P is None else P
    c0 = c["c0"] if c0 is None else c0
    c1 = c["c1"] if c1 is None else c1
    rng = _rng(CFG_DSPARK, seed, 0)
    u = rng.uniform(0.35, 0.98, (batch, 1))
    dl = rng.uniform(0.0, 0.06, (batch, 1))
    conf = u - dl * np.arange(P)[None, :] + rng.normal(0.0, 0.05, (batch, P))
    conf = np.clip(conf, 0.01, 0.999).astype(np.float32)
    T = np.arange(batch * (P + 1) + 1, dtype=np.float64)
    cost = (c0 + c1 * T).astype(np.float32)
    return conf, cost
