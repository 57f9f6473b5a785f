"""Seeded synthetic inputs for the verify step.

Draws the logits, draft tokens, uniforms, temperatures and token trees that
both the HIP path and the oracle consume, with the shapes and value
distributions of the five standard workloads.  Nothing here performs any part
of the verify arithmetic: the random numbers the method consumes (accept and
draw uniforms) are drawn here and passed in as inputs.

Draft tokens are drawn from the draft's own temperature distribution with the
Gumbel-max construction, argmax_x (z(x)/T + G(x)) with i.i.d. standard Gumbel
G, applied to the stored (possibly bf16-rounded) draft logits, so the tokens
follow q exactly as the verify step will compute it.

Every generator is a pure function of its seed: numpy SeedSequence streams
are spawned per component, and large tensors are filled in fixed row blocks
(each with its own spawned stream), so the result does not depend on the
number of worker threads.
"""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

# Uniforms lie on the grid k / 2^24, k in [0, 2^24): exact in fp32 and fp64, in [0, 1).
UNIFORM_GRID = 1 << 24

# Draft-noise sigma of the Zipf workload, chosen so that the mean per-position
# acceptance rate alpha = sum_x min(p(x), q(x)) is about 0.7.  The value comes
# from oracle/calibrate_zipf_sigma.py (bisection on a calibration draw).
ZIPF_DRAFT_SIGMA = 0.75

_THREADS = max(1, min(16, len(os.sched_getaffinity(0))))


# ----------------------------------------------------------------------------- bf16 storage

def bf16_bits(x):
    """fp32 -> bf16 bit patterns (uint16), rounding to nearest, ties to even (finite inputs)."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    return ((b + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_value(bits):
    """bf16 bit patterns -> the fp32 numbers they denote."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def stored_value(a, dtype):
    """Stored logits as fp32 numbers (fp32 as is; bf16 patterns widened)."""
    return bf16_value(a) if dtype == "bf16" else np.asarray(a, dtype=np.float32)


# ----------------------------------------------------------------------------- batches

@dataclass
class ChainBatch:
    """One batch of chain-verify inputs.

    target [B, gamma+1, V] and draft [B, gamma, V] hold fp32 numbers or bf16
    bit patterns (uint16); draft_tokens int32 [B, gamma]; uniforms fp32
    [B, gamma+1] (columns 0..gamma-1 drive the accept tests, column gamma the
    draw); temperature fp32 [B].
    """
    name: str
    dtype: str
    target: np.ndarray
    draft: np.ndarray
    draft_tokens: np.ndarray
    uniforms: np.ndarray
    temperature: np.ndarray
    meta: dict = field(default_factory=dict)

    @property
    def B(self):
        return self.target.shape[0]

    @property
    def gamma(self):
        return self.draft.shape[1]

    @property
    def V(self):
        return self.target.shape[2]

    @property
    def rows(self):
        """Logit rows consumed: gamma+1 target rows and gamma draft rows per sequence."""
        return self.B * (2 * self.gamma + 1)

    @property
    def logit_bytes(self):
        return self.target.nbytes + self.draft.nbytes


@dataclass
class TreeBatch:
    """One batch of token-tree inputs.

    logits [n_trees, n_nodes, V] (fp32 or bf16 bit patterns), row u scoring the
    children of node u; parents int32 [n_trees, n_nodes] with parents[t][0] = -1
    and parents[t][i] < i; node_tokens int32 [n_trees, n_nodes] (node 0 holds the
    last committed token).
    """
    name: str
    dtype: str
    logits: np.ndarray
    parents: np.ndarray
    node_tokens: np.ndarray
    meta: dict = field(default_factory=dict)

    @property
    def n_trees(self):
        return self.logits.shape[0]

    @property
    def n_nodes(self):
        return self.logits.shape[1]

    @property
    def V(self):
        return self.logits.shape[2]

    @property
    def rows(self):
        return self.n_trees * self.n_nodes

    @property
    def logit_bytes(self):
        return self.logits.nbytes


# ----------------------------------------------------------------------------- helpers

def _streams(seed, n):
    ss = seed if isinstance(seed, np.random.SeedSequence) else np.random.SeedSequence(seed)
    return ss.spawn(n)


def _row_blocks(n_rows, block):
    return [(s, min(n_rows, s + block)) for s in range(0, n_rows, block)]


def _fill_rows(seq, n_rows, block, fill):
    """Call fill(generator, r0, r1) for fixed row blocks, one spawned stream per block."""
    blocks = _row_blocks(n_rows, block)
    subs = seq.spawn(len(blocks))
    jobs = [(np.random.default_rng(s), r0, r1) for s, (r0, r1) in zip(subs, blocks)]
    if len(jobs) == 1 or _THREADS == 1:
        for g, r0, r1 in jobs:
            fill(g, r0, r1)
        return
    with ThreadPoolExecutor(_THREADS) as ex:
        list(ex.map(lambda j: fill(*j), jobs))


def uniforms(gen, shape):
    """U[0, 1) on the 2^-24 grid, as fp32."""
    k = gen.integers(0, UNIFORM_GRID, size=shape, dtype=np.int64)
    return (k.astype(np.float64) / UNIFORM_GRID).astype(np.float32)


def draft_tokens_gumbel(seq, z_rows, temp_rows, block=64):
    """One token per row drawn from softmax(z/T) by Gumbel-max; z_rows [R, V] fp32, temp_rows [R]."""
    R = z_rows.shape[0]
    out = np.empty(R, dtype=np.int32)

    def fill(g, r0, r1):
        z = z_rows[r0:r1].astype(np.float64) / temp_rows[r0:r1, None].astype(np.float64)
        z += g.gumbel(size=z.shape)
        out[r0:r1] = np.argmax(z, axis=1)

    _fill_rows(seq, R, block, fill)
    return out


def _store(x, dtype):
    return bf16_bits(x) if dtype == "bf16" else np.ascontiguousarray(x, dtype=np.float32)


def _finish_chain(name, dtype, t32, d32, temperature, seq_tok, seq_u, meta):
    """Round to the storage dtype, draw draft tokens from q of the stored draft, draw uniforms."""
    B, g1, V = t32.shape
    gamma = g1 - 1
    target = _store(t32, dtype)
    draft = _store(d32, dtype)
    dz = stored_value(draft, dtype).reshape(B * gamma, V)
    toks = draft_tokens_gumbel(seq_tok, dz, np.repeat(temperature, gamma)).reshape(B, gamma)
    u = uniforms(np.random.default_rng(seq_u), (B, gamma + 1))
    return ChainBatch(name, dtype, target, draft, toks, u, temperature.astype(np.float32), meta)


# ----------------------------------------------------------------------------- chain workloads

def chain_gaussian(seed, B, gamma, V, dtype, sigma_t, sigma_d, temperature, draft_scale=1.0,
                   name=None):
    """Gaussian chain workload: z_t ~ N(0, sigma_t^2) i.i.d.; z_d = draft_scale*z_t + N(0, sigma_d^2).

    temperature is a scalar or a length-B array.
    """
    s_t, s_d, s_tok, s_u = _streams(seed, 4)
    t32 = np.empty((B, gamma + 1, V), dtype=np.float32)
    d32 = np.empty((B, gamma, V), dtype=np.float32)
    tv = t32.reshape(B * (gamma + 1), V)
    block = max(1, (1 << 22) // max(V, 1))

    def fill_t(g, r0, r1):
        tv[r0:r1] = g.standard_normal((r1 - r0, V), dtype=np.float32) * np.float32(sigma_t)

    _fill_rows(s_t, B * (gamma + 1), block, fill_t)

    def fill_d(g, b0, b1):
        noise = g.standard_normal((b1 - b0, gamma, V), dtype=np.float32) * np.float32(sigma_d)
        d32[b0:b1] = np.float32(draft_scale) * t32[b0:b1, :gamma] + noise

    _fill_rows(s_d, B, max(1, block // max(gamma, 1)), fill_d)
    temp = np.broadcast_to(np.asarray(temperature, dtype=np.float32), (B,)).copy()
    meta = {"sigma_t": sigma_t, "sigma_d": sigma_d, "draft_scale": draft_scale}
    return _finish_chain(name or f"gaussian_B{B}_g{gamma}_V{V}_{dtype}", dtype, t32, d32, temp,
                         s_tok, s_u, meta)


def chain_b1_v1000(seed=1):
    """B=1, gamma=4, V=1000, fp32, T=1.0; z_t ~ N(0, 2^2); z_d = z_t + N(0, 0.5^2)."""
    return chain_gaussian(seed, 1, 4, 1000, "f32", 2.0, 0.5, 1.0, name="gauss_b1_g4_v1000_f32")


def chain_b1_v32000(seed=2, gamma=4):
    """B=1, gamma in {4..7}, V=32000, bf16, T=0.8; z_t ~ N(0, 3^2); z_d = z_t + N(0, 1^2)."""
    return chain_gaussian(seed, 1, gamma, 32000, "bf16", 3.0, 1.0, 0.8, name=f"gauss_b1_g{gamma}_v32000_bf16")


def chain_b256_v152064(seed=4):
    """B=256, gamma=7, V=152064, fp32, T in {0.6, 1.0} per sequence;
    z_t ~ N(0, 2.5^2); z_d = 0.8 z_t + N(0, 1.5^2)."""
    s_main, s_temp = _streams(seed, 2)
    temp = np.where(np.random.default_rng(s_temp).random(256) < 0.5, 0.6, 1.0).astype(np.float32)
    return chain_gaussian(s_main, 256, 7, 152064, "f32", 2.5, 1.5, temp, draft_scale=0.8,
                          name="gauss_b256_g7_v152064_f32")


def chain_zipf(seed, B, gamma, V, dtype, sigma_d, temperature=1.0, name=None):
    """Zipf-shaped workload: the token at rank r (1-based) of a fresh random permutation per
    (sequence, position) row gets logit -1.1 ln r + N(0, 0.3^2); the draft row at the same
    position adds N(0, sigma_d^2) to the target row."""
    s_t, s_d, s_tok, s_u = _streams(seed, 4)
    t32 = np.empty((B, gamma + 1, V), dtype=np.float32)
    d32 = np.empty((B, gamma, V), dtype=np.float32)
    tv = t32.reshape(B * (gamma + 1), V)
    base = (-1.1 * np.log(np.arange(1, V + 1, dtype=np.float64))).astype(np.float32)

    def fill_t(g, r0, r1):
        for r in range(r0, r1):
            perm = g.permutation(V)
            row = base + g.standard_normal(V, dtype=np.float32) * np.float32(0.3)
            tv[r, perm] = row

    _fill_rows(s_t, B * (gamma + 1), 16, fill_t)

    def fill_d(g, b0, b1):
        noise = g.standard_normal((b1 - b0, gamma, V), dtype=np.float32) * np.float32(sigma_d)
        d32[b0:b1] = t32[b0:b1, :gamma] + noise

    _fill_rows(s_d, B, 4, fill_d)
    temp = np.full(B, temperature, dtype=np.float32)
    meta = {"sigma_d": sigma_d, "seed": seed}
    return _finish_chain(name or f"zipf_B{B}_g{gamma}_V{V}_{dtype}", dtype, t32, d32, temp,
                         s_tok, s_u, meta)


def chain_zipf_b64_v128256(seed=3, sigma_d=ZIPF_DRAFT_SIGMA):
    """B=64, gamma=4, V=128256, bf16, T=1.0, Zipf-shaped logits, mean alpha about 0.7."""
    return chain_zipf(seed, 64, 4, 128256, "bf16", sigma_d, 1.0, name="zipf_b64_g4_v128256_bf16")


def chain_from_logits(seed, target32, draft32, temperature, dtype="f32", name="custom"):
    """Chain batch from given fp32 logits: rounds to dtype, draws draft tokens and uniforms."""
    _, _, s_tok, s_u = _streams(seed, 4)
    target32 = np.asarray(target32, dtype=np.float32)
    B = target32.shape[0]
    temp = np.broadcast_to(np.asarray(temperature, dtype=np.float32), (B,)).copy()
    return _finish_chain(name, dtype, target32, np.asarray(draft32, dtype=np.float32), temp,
                         s_tok, s_u, {"seed": seed})


# ----------------------------------------------------------------------------- greedy chains

@dataclass
class GreedyBatch:
    """One batch of greedy chain inputs: target logits [B, gamma+1, V] (fp32 or bf16 bit
    patterns) and draft tokens int32 [B, gamma]; no draft logits or random numbers."""
    name: str
    dtype: str
    target: np.ndarray
    draft_tokens: np.ndarray
    meta: dict = field(default_factory=dict)

    @property
    def B(self):
        return self.target.shape[0]

    @property
    def gamma(self):
        return self.target.shape[1] - 1

    @property
    def V(self):
        return self.target.shape[2]

    @property
    def rows(self):
        return self.B * (self.gamma + 1)

    @property
    def logit_bytes(self):
        return self.target.nbytes


def chain_greedy_planted(seed, B, gamma, V, dtype, sigma=2.0, boost=16.0, match_prob=0.8,
                         name=None):
    """Greedy chain workload: target logits ~ N(0, sigma^2); in every row one token, chosen
    uniformly, gets +boost (fp32, before rounding to the storage dtype); draft token i is row i's
    planted token with probability match_prob, else a uniform token.  With the default boost the
    planted token all but surely holds the row's maximum, so accepted runs are long; which token
    actually holds the maximum is for the verify step to find."""
    s_t, s_plant, s_tok = _streams(seed, 3)
    t32 = np.empty((B, gamma + 1, V), dtype=np.float32)
    tv = t32.reshape(B * (gamma + 1), V)

    def fill_t(g, r0, r1):
        tv[r0:r1] = g.standard_normal((r1 - r0, V), dtype=np.float32) * np.float32(sigma)

    _fill_rows(s_t, B * (gamma + 1), max(1, (1 << 22) // max(V, 1)), fill_t)
    gp = np.random.default_rng(s_plant)
    plant = gp.integers(0, V, size=(B, gamma + 1))
    tv[np.arange(B * (gamma + 1)), plant.reshape(-1)] += np.float32(boost)
    gk = np.random.default_rng(s_tok)
    other = gk.integers(0, V, size=(B, gamma))
    toks = np.where(gk.random((B, gamma)) < match_prob, plant[:, :gamma], other).astype(np.int32)
    meta = {"sigma": sigma, "boost": boost, "match_prob": match_prob, "seed": seed}
    return GreedyBatch(name or f"greedy_B{B}_g{gamma}_V{V}_{dtype}", dtype, _store(t32, dtype),
                       toks, meta)


def chain_greedy_b256_v152064(seed=6):
    """Greedy chain at the shape of the largest chain workload: B=256, gamma=7, V=152064, fp32."""
    return chain_greedy_planted(seed, 256, 7, 152064, "f32", name="greedy_b256_g7_v152064_f32")


def chain_greedy_b64_v128256(seed=7):
    """Greedy chain at the shape of the Zipf workload: B=64, gamma=4, V=128256, bf16."""
    return chain_greedy_planted(seed, 64, 4, 128256, "bf16", name="greedy_b64_g4_v128256_bf16")


# ----------------------------------------------------------------------------- sampler rows

@dataclass
class SampleBatch:
    """One batch of sampler inputs: logits [rows, V] (fp32 or bf16 bit patterns), a temperature
    and a uniform per row."""
    name: str
    dtype: str
    logits: np.ndarray
    temperature: np.ndarray
    uniforms: np.ndarray
    meta: dict = field(default_factory=dict)

    @property
    def rows(self):
        return self.logits.shape[0]

    @property
    def V(self):
        return self.logits.shape[1]

    @property
    def logit_bytes(self):
        return self.logits.nbytes


def sample_gaussian(seed, rows, V, dtype, sigma, temperature, name=None):
    """Sampler workload: logits ~ N(0, sigma^2) i.i.d.; temperature a scalar or per-row array;
    uniforms on the 2^-24 grid."""
    s_z, s_u = _streams(seed, 2)
    z = np.empty((rows, V), dtype=np.float32)

    def fill(g, r0, r1):
        z[r0:r1] = g.standard_normal((r1 - r0, V), dtype=np.float32) * np.float32(sigma)

    _fill_rows(s_z, rows, max(1, (1 << 22) // max(V, 1)), fill)
    temp = np.broadcast_to(np.asarray(temperature, dtype=np.float32), (rows,)).copy()
    u = uniforms(np.random.default_rng(s_u), (rows,))
    return SampleBatch(name or f"sample_R{rows}_V{V}_{dtype}", dtype, _store(z, dtype), temp, u,
                       {"sigma": sigma, "seed": seed})


def sample_b256_v152064(seed=8):
    """One draft token for each of 256 sequences, V=152064, fp32, T in {0.6, 1.0} per row."""
    s_main, s_temp = _streams(seed, 2)
    temp = np.where(np.random.default_rng(s_temp).random(256) < 0.5, 0.6, 1.0)
    return sample_gaussian(s_main, 256, 152064, "f32", 2.5, temp, name="sample_b256_v152064_f32")


def sample_b64_v128256(seed=9):
    """One draft token for each of 64 sequences, V=128256, bf16, T=1."""
    return sample_gaussian(seed, 64, 128256, "bf16", 2.5, 1.0, name="sample_b64_v128256_bf16")


# ----------------------------------------------------------------------------- KV blocks

@dataclass
class KvBatch:
    """One batch of KV-compaction inputs: speculative KV blocks src [n, src_rows, row_bytes]
    (uint8), the initial caches dst_init [n, dst_rows, row_bytes], accepted paths [n, path_len]
    (node ids, -1 padded; None for chains), accepted counts and destination start rows."""
    name: str
    src: np.ndarray
    dst_init: np.ndarray
    paths: object
    num_accepted: np.ndarray
    dst_start: np.ndarray
    meta: dict = field(default_factory=dict)

    @property
    def n(self):
        return self.src.shape[0]

    @property
    def row_bytes(self):
        return self.src.shape[2]

    @property
    def moved_rows(self):
        return int((self.num_accepted.astype(np.int64) + 1).sum())


def _random_bytes(seq, shape):
    out = np.empty(shape, dtype=np.uint8)
    flat = out.reshape(shape[0] * shape[1], shape[2])

    def fill(g, r0, r1):
        flat[r0:r1] = g.integers(0, 256, size=(r1 - r0, shape[2]), dtype=np.uint8)

    _fill_rows(seq, shape[0] * shape[1], max(1, (1 << 24) // max(shape[2], 1)), fill)
    return out


def kv_tree_paths(seed, n_trees, n_nodes, row_bytes, dst_rows=96, max_branch=4, max_depth=8,
                  stop_prob=0.25, name=None):
    """Tree KV workload: random BFS trees (as the tree workloads), and for each a synthetic
    accepted path that starts at the root and moves to a uniformly chosen child until it reaches
    a leaf or stops (probability stop_prob per step); random KV bytes; the cache's destination
    starts at a random row leaving room for the path."""
    s_tree, s_walk, s_src, s_dst = _streams(seed, 4)
    gt = np.random.default_rng(s_tree)
    gw = np.random.default_rng(s_walk)
    paths = np.full((n_trees, n_nodes), -1, dtype=np.int32)
    k = np.empty(n_trees, dtype=np.int32)
    start = np.empty(n_trees, dtype=np.int32)
    for t in range(n_trees):
        parents, _ = random_tree(gt, n_nodes, 1000, max_branch, max_depth)
        u, path = 0, [0]
        while True:
            kids = np.flatnonzero(parents == u)
            if len(kids) == 0 or gw.random() < stop_prob:
                break
            u = int(kids[int(gw.integers(0, len(kids)))])
            path.append(u)
        paths[t, :len(path)] = path
        k[t] = len(path) - 1
        start[t] = int(gw.integers(0, dst_rows - len(path) + 1))
    src = _random_bytes(s_src, (n_trees, n_nodes, row_bytes))
    dst = _random_bytes(s_dst, (n_trees, dst_rows, row_bytes))
    return KvBatch(name or f"kv_tree_{n_trees}x{n_nodes}_W{row_bytes}", src, dst, paths, k, start,
                   {"seed": seed})


def kv_chain(seed, B, gamma, row_bytes, dst_rows=64, name=None):
    """Chain KV workload: gamma + 1 KV rows per sequence, a uniform accepted count in [0, gamma],
    random KV bytes and destination start rows."""
    s_k, s_src, s_dst = _streams(seed, 3)
    g = np.random.default_rng(s_k)
    k = g.integers(0, gamma + 1, size=B).astype(np.int32)
    start = np.array([g.integers(0, dst_rows - kk) for kk in k], dtype=np.int32)
    src = _random_bytes(s_src, (B, gamma + 1, row_bytes))
    dst = _random_bytes(s_dst, (B, dst_rows, row_bytes))
    return KvBatch(name or f"kv_chain_B{B}_g{gamma}_W{row_bytes}", src, dst, None, k, start,
                   {"seed": seed})


# Bytes of one token's KV row for a 32-layer model with 8 KV heads of dimension 128 in bf16
# (keys and values): 32 * 2 * 8 * 128 * 2.
KV_ROW_BYTES = 131072


def kv_tree_16x64():
    """KV rows of the 16 x 64-node token trees, 128 KiB per row, synthetic accepted paths."""
    return kv_tree_paths(10, 16, 64, KV_ROW_BYTES, name="kv_tree_16x64_w131072")


def kv_chain_b256_g7():
    """KV rows of 256 chains of gamma = 7, 128 KiB per row, uniform accepted counts."""
    return kv_chain(11, 256, 7, KV_ROW_BYTES, dst_rows=16, name="kv_chain_b256_g7_w131072")


# ----------------------------------------------------------------------------- token trees

def random_tree(gen, n_nodes, vocab, max_branch=4, max_depth=8, max_draws=10000):
    """Breadth-first token tree: each expanded node gets a uniform number of children in
    [1, max_branch] (nodes at max_depth are not expanded), truncated at n_nodes nodes.
    Child tokens are uniform on [0, vocab) and distinct among siblings.  A draw that runs
    out of nodes to expand before n_nodes is discarded and drawn again, at most max_draws
    times; a shape that no tree of that branching and depth can reach raises ValueError."""
    b = min(max_branch, vocab)
    capacity, level = 1, 1
    for _ in range(max_depth):
        if capacity >= n_nodes:
            break
        level *= b
        capacity += level
    if capacity < n_nodes:
        raise ValueError(f"no tree of {n_nodes} nodes has branching <= {b} and depth <= {max_depth}")
    for _ in range(max_draws):
        parents = [-1]
        depth = [0]
        tokens = [int(gen.integers(0, vocab))]
        head = 0
        while len(parents) < n_nodes and head < len(parents):
            u = head
            head += 1
            if depth[u] >= max_depth:
                continue
            nb = int(gen.integers(1, max_branch + 1))
            nb = min(nb, n_nodes - len(parents))
            toks = gen.choice(vocab, size=nb, replace=False) if nb <= vocab else None
            if toks is None:
                break
            for t in toks:
                parents.append(u)
                depth.append(depth[u] + 1)
                tokens.append(int(t))
        if len(parents) == n_nodes:
            return np.array(parents, dtype=np.int32), np.array(tokens, dtype=np.int32)
    raise ValueError(f"no {n_nodes}-node tree drawn in {max_draws} draws (branching <= "
                     f"{max_branch}, depth <= {max_depth})")


def tree_random(seed, n_trees, n_nodes, V, dtype, sigma=2.0, boost=4.0, boost_prob=0.6,
                max_branch=4, max_depth=8, name=None):
    """Token-tree workload: logits ~ N(0, sigma^2); for each node with children, with
    probability boost_prob one child is picked uniformly and the node's logit at that
    child's token is raised by boost (in fp32, before rounding to the storage dtype)."""
    s_tree, s_logit, s_boost = _streams(seed, 3)
    gt = np.random.default_rng(s_tree)
    parents = np.empty((n_trees, n_nodes), dtype=np.int32)
    tokens = np.empty((n_trees, n_nodes), dtype=np.int32)
    for t in range(n_trees):
        parents[t], tokens[t] = random_tree(gt, n_nodes, V, max_branch, max_depth)
    z = np.empty((n_trees, n_nodes, V), dtype=np.float32)
    zv = z.reshape(n_trees * n_nodes, V)

    def fill(g, r0, r1):
        zv[r0:r1] = g.standard_normal((r1 - r0, V), dtype=np.float32) * np.float32(sigma)

    _fill_rows(s_logit, n_trees * n_nodes, max(1, (1 << 22) // max(V, 1)), fill)
    gb = np.random.default_rng(s_boost)
    for t in range(n_trees):
        for u in range(n_nodes):
            kids = np.flatnonzero(parents[t] == u)
            if len(kids) == 0:
                continue
            if gb.random() < boost_prob:
                c = kids[int(gb.integers(0, len(kids)))]
                z[t, u, tokens[t, c]] += np.float32(boost)
    meta = {"sigma": sigma, "boost": boost, "boost_prob": boost_prob, "seed": seed}
    return TreeBatch(name or f"tree_{n_trees}x{n_nodes}_V{V}_{dtype}", dtype, _store(z, dtype),
                     parents, tokens, meta)


def tree_16x64_v32000(seed=5):
    """16 trees x 64 nodes, depth <= 8, branching 1..4, V=32000, bf16, N(0, 2^2) logits with
    the +4 boost applied with probability 0.6."""
    return tree_random(seed, 16, 64, 32000, "bf16", name="tree_16x64_v32000_bf16")


# ----------------------------------------------------------------------------- registry

CHAIN_WORKLOADS = {
    "gauss_b1_g4_v1000_f32": chain_b1_v1000,
    "gauss_b1_g4_v32000_bf16": lambda: chain_b1_v32000(gamma=4),
    "gauss_b1_g5_v32000_bf16": lambda: chain_b1_v32000(gamma=5),
    "gauss_b1_g6_v32000_bf16": lambda: chain_b1_v32000(gamma=6),
    "gauss_b1_g7_v32000_bf16": lambda: chain_b1_v32000(gamma=7),
    "zipf_b64_g4_v128256_bf16": chain_zipf_b64_v128256,
    "gauss_b256_g7_v152064_f32": chain_b256_v152064,
}
TREE_WORKLOADS = {"tree_16x64_v32000_bf16": tree_16x64_v32000}
SAMPLE_WORKLOADS = {
    "sample_b256_v152064_f32": sample_b256_v152064,
    "sample_b64_v128256_bf16": sample_b64_v128256,
}
KV_WORKLOADS = {
    "kv_tree_16x64_w131072": kv_tree_16x64,
    "kv_chain_b256_g7_w131072": kv_chain_b256_g7,
}
GREEDY_WORKLOADS = {
    "greedy_b256_g7_v152064_f32": chain_greedy_b256_v152064,
    "greedy_b64_g4_v128256_bf16": chain_greedy_b64_v128256,
}
