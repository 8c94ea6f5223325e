"""Seeded synthetic inputs for draft-token verification.

This module only makes inputs: logits rows, draft tokens, uniforms, d2t maps
and draft-tree topologies, shaped like the workloads the pages describe.  It
holds none of the verification arithmetic (no softmax, no top-p, no accept
rule, no residual); the draft tokens come from a Gumbel-max draw over the
draft logits (a draft-side sampler, upstream of verification), or, for the
greedy workloads, from NumPy's argmax as each workload's recipe states.

Every array is host NumPy.  bfloat16 tensors are carried as uint16 bit
patterns (round-to-nearest-even of the float32 value); `bf16_to_f32` widens
them exactly.  Uniforms are k / 2**24 with k uniform in [0, 2**24), so the
float32 value is exact and every consumer sees the same number.

Workloads (sizes are parameters; the defaults are the full sizes):
  sample_plain   B=1,  gamma=3, V=49152, fp32 target ~N(0, 2^2), draft = target + N(0, 0.5^2),
                 T=1, no top-p.  The tutorial's generate() defaults aside, the vocabulary
                 size is the one of the 2.16x blog's SmolLM2 model.
  sample_topp    B=64, gamma=5, V=151936, bf16 target ~N(0, 3^2) with 1% of the ids of
                 every row raised by +8, draft = target + N(0, 1^2), T=0.8, top-p 0.9
                 (the tutorial's generate() defaults).
  greedy         B=128, gamma=6, V=128256, bf16 ~N(0, 2^2); draft token i equals the row's
                 argmax with probability 0.7, else a uniform other id (the SSD guide's
                 temperature-0, k=6 benchmark run).
  eagle_d2t      B=32, gamma=7, Vt=128256, Vd=32000; d2t = sorted random 32000 target ids;
                 draft fp32 ~N(0, 2^2); target bf16 = mapped draft + N(0, 1^2), unmapped
                 ~N(-4, 1^2); the bonus row is built the same way from a fresh draft-like
                 row; T=1 (the SSD guide's EAGLE3 k=7 run).
  tree           B=16, N=32 nodes, depth <= 5, <= 8 children, V=49152, bf16 ~N(0, 2^2);
                 node token = argmax of its parent's row with probability 0.6 (the 2.16x
                 blog's 32-node, depth-5, top-k-8 tree).
  draft          B=64 rows, V=151936, bf16, shaped like sample_topp's rows; T=0.8,
                 top-p 0.9, top-k 50 (the draft-side sampler).
  fanout         B=64, gamma=7, f=3 candidates per accepted length, L=8 drafts per
                 branch (the SSD fan-out lookup).
  trim           2^24 token ids over Vt=128256 from a bounded Zipf law (s = 1.1) at
                 random ids, P = 0.95 (the vocabulary trim; no corpus is used).
  lmhead         hidden [128, 7, 4096] and W [128256, 4096] bfloat16 with a planted
                 token per row (the fused lm_head -> greedy verification).
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "bf16_bits", "bf16_to_f32", "uniforms", "gumbel_draw",
    "sample_plain", "sample_topp", "greedy", "eagle_d2t", "tree", "WORKLOADS",
]


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest, ties to even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float32, exact."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def uniforms(rng: np.random.Generator, shape) -> np.ndarray:
    """Uniforms in [0, 1) of the form k / 2**24, as float32 (exact)."""
    return (rng.integers(0, 1 << 24, size=shape, dtype=np.int64).astype(np.float64)
            / float(1 << 24)).astype(np.float32)


def _normal(rng, shape, sigma, mean=0.0):
    return (rng.standard_normal(size=shape, dtype=np.float32) * np.float32(sigma)
            + np.float32(mean))


def gumbel_draw(rng: np.random.Generator, logits_f32: np.ndarray, temperature: float) -> np.ndarray:
    """One draw per row of a [..., V] array by the Gumbel-max trick on logits/T.

    A stand-in for the draft model's own sampler; it is not part of
    verification.  Rows are drawn one by one to bound memory."""
    flat = logits_f32.reshape(-1, logits_f32.shape[-1])
    out = np.empty(flat.shape[0], np.int32)
    for r in range(flat.shape[0]):
        g = rng.gumbel(size=flat.shape[1])
        out[r] = int(np.argmax(flat[r].astype(np.float64) / temperature + g))
    return out.reshape(logits_f32.shape[:-1])


def _other_id(rng, V, avoid):
    """A uniform id in [0, V) different from `avoid` (element-wise); with
    V = 1 there is no other id and `avoid` itself is returned."""
    if V == 1:
        return np.zeros(np.shape(avoid), np.int32)
    r = rng.integers(0, V - 1, size=np.shape(avoid))
    return (r + (r >= avoid)).astype(np.int32)


def sample_plain(seed: int, B: int = 1, gamma: int = 3, V: int = 49152) -> dict:
    rng = np.random.default_rng(seed)
    zt = _normal(rng, (B, gamma + 1, V), 2.0)
    zd = (zt[:, :gamma] + _normal(rng, (B, gamma, V), 0.5)).astype(np.float32)
    return dict(kind="sample", target=zt, draft=zd,
                tokens=gumbel_draw(rng, zd, 1.0) if gamma > 0 else np.zeros((B, 0), np.int32),
                u_accept=uniforms(rng, (B, gamma)), u_sample=uniforms(rng, (B,)),
                d2t=None, temperature=1.0, top_p=1.0)


def sample_topp(seed: int, B: int = 64, gamma: int = 5, V: int = 151936,
                spike_frac: float = 0.01, temperature: float = 0.8, top_p: float = 0.9) -> dict:
    rng = np.random.default_rng(seed)
    zt = _normal(rng, (B, gamma + 1, V), 3.0)
    n_spike = max(1, int(round(spike_frac * V)))
    for b in range(B):
        for i in range(gamma + 1):
            zt[b, i, rng.choice(V, n_spike, replace=False)] += np.float32(8.0)
    zd = (zt[:, :gamma] + _normal(rng, (B, gamma, V), 1.0)).astype(np.float32)
    tb, db = bf16_bits(zt), bf16_bits(zd)
    return dict(kind="sample", target=tb, draft=db,
                tokens=(gumbel_draw(rng, bf16_to_f32(db), temperature) if gamma > 0
                        else np.zeros((B, 0), np.int32)),
                u_accept=uniforms(rng, (B, gamma)), u_sample=uniforms(rng, (B,)),
                d2t=None, temperature=temperature, top_p=top_p)


def greedy(seed: int, B: int = 128, gamma: int = 6, V: int = 128256, p_match: float = 0.7) -> dict:
    rng = np.random.default_rng(seed)
    zb = bf16_bits(_normal(rng, (B, gamma + 1, V), 2.0))
    am = np.argmax(bf16_to_f32(zb[:, :gamma]), axis=-1).astype(np.int32)
    match = rng.random(size=(B, gamma)) < p_match
    tokens = np.where(match, am, _other_id(rng, V, am)).astype(np.int32)
    return dict(kind="greedy", target=zb, tokens=tokens)


def eagle_d2t(seed: int, B: int = 32, gamma: int = 7, Vt: int = 128256, Vd: int = 32000,
              temperature: float = 1.0) -> dict:
    rng = np.random.default_rng(seed)
    d2t = np.sort(rng.choice(Vt, Vd, replace=False)).astype(np.int32)
    zd = _normal(rng, (B, gamma, Vd), 2.0)
    aux = _normal(rng, (B, 1, Vd), 2.0)                 # stands in for a draft row at the bonus position
    src = np.concatenate([zd, aux], axis=1)
    zt = _normal(rng, (B, gamma + 1, Vt), 1.0, mean=-4.0)
    zt[:, :, d2t] = src + _normal(rng, (B, gamma + 1, Vd), 1.0)
    j = gumbel_draw(rng, zd, temperature) if gamma > 0 else np.zeros((B, 0), np.int32)
    return dict(kind="sample", target=bf16_bits(zt), draft=zd.astype(np.float32),
                tokens=d2t[j].astype(np.int32), u_accept=uniforms(rng, (B, gamma)),
                u_sample=uniforms(rng, (B,)), d2t=d2t, temperature=temperature, top_p=1.0)


def draft(seed: int, B: int = 64, V: int = 151936, spike_frac: float = 0.01, temperature: float = 0.8,
          top_p: float = 0.9, top_k: int = 50, bf16: bool = True) -> dict:
    """Draft-side sampler input: B rows shaped like the sampling workload's
    (N(0, 3^2), 1% of the ids of every row raised by +8), one uniform per row."""
    rng = np.random.default_rng(seed)
    z = _normal(rng, (B, V), 3.0)
    n_spike = max(1, int(round(spike_frac * V)))
    for b in range(B):
        z[b, rng.choice(V, n_spike, replace=False)] += np.float32(8.0)
    return dict(kind="draft", logits=bf16_bits(z) if bf16 else z, u=uniforms(rng, (B,)),
                temperature=temperature, top_p=top_p, top_k=top_k, d2t=None)


def fanout(seed: int, B: int = 64, gamma: int = 7, f: int = 3, L: int = 8, V: int = 128256,
           p_hit: float = 0.6) -> dict:
    """SSD fan-out lookup input: verification outputs (accepted lengths and
    emitted tokens), f candidate tokens per accepted length (the emitted one
    among them with probability p_hit) and L pre-drafted tokens per branch
    (the SSD guide's EAGLE run: k = 7, f = 3)."""
    rng = np.random.default_rng(seed)
    n = rng.integers(0, gamma + 1, B).astype(np.int32)
    ot = np.full((B, gamma + 1), -1, np.int32)
    emitted = rng.integers(0, V, B).astype(np.int32)
    for b in range(B):
        ot[b, :n[b]] = rng.integers(0, V, n[b])
        ot[b, n[b]] = emitted[b]
    cand = rng.integers(0, V, (B, gamma + 1, f)).astype(np.int32)
    hit = rng.random(B) < p_hit
    cand[np.flatnonzero(hit), n[hit], rng.integers(0, f, hit.sum())] = emitted[hit]
    drafts = rng.integers(0, V, (B, (gamma + 1) * f, L)).astype(np.int32)
    return dict(kind="fanout", out_tokens=ot, accept_len=n, cand=cand, drafts=drafts)


def token_stream(seed: int, N: int = 1 << 24, Vt: int = 128256, s: float = 1.1, invalid_frac: float = 0.0) -> dict:
    """A corpus stand-in for the vocabulary trim: N token ids drawn from a
    bounded Zipf law (p(rank r) proportional to r^-s over Vt ranks) with the
    ranks placed at random ids, optionally with a fraction of ids outside
    [0, Vt)."""
    rng = np.random.default_rng(seed)
    w = np.arange(1, Vt + 1, dtype=np.float64) ** -s
    cdf = np.cumsum(w)
    cdf /= cdf[-1]
    ranks = np.minimum(np.searchsorted(cdf, rng.random(N)), Vt - 1)
    ids = rng.permutation(Vt).astype(np.int32)[ranks]
    if invalid_frac > 0:
        bad = rng.random(N) < invalid_frac
        ids[bad] = Vt + rng.integers(0, 100, bad.sum())
    return dict(kind="trim", tokens=ids, Vt=Vt, P=0.95)


def _bf16_rows(rng, shape, scale, block=1 << 22):
    """Normal(0, scale^2) bfloat16 bits of the given 2-D shape, made in row
    blocks of about `block` elements (bounded host memory)."""
    rows, cols = shape
    out = np.empty(shape, np.uint16)
    step = max(1, block // max(cols, 1))
    for r0 in range(0, rows, step):
        r1 = min(rows, r0 + step)
        out[r0:r1] = bf16_bits(_normal(rng, (r1 - r0, cols), scale))
    return out


def lmhead(seed: int, B: int = 128, R: int = 7, d: int = 4096, V: int = 128256, alpha: float = 4.2,
           noise: float = 0.8, p_match: float = 0.7, tree: bool = False, max_depth: int = 5,
           max_children: int = 8) -> dict:
    """Fused lm_head input: W [V, d] ~ N(0, 2.5^2 / d) and, for every row, a
    planted token g whose unit weight row the hidden state follows:
    h = alpha u_g + N(0, noise^2) per component (so g's logit is about
    2.5 alpha, the others about N(0, (2.5 noise)^2)).  Chain: draft token i is
    g of row i with probability p_match, else another id.  Tree (R = N nodes):
    a random parent array and node token = g of the parent's row with
    probability p_match.  All bfloat16; the defaults are a Llama-3-8B-sized
    lm_head (d = 4096, V = 128256) over the greedy batch (B = 128, gamma = 6)."""
    rng = np.random.default_rng(seed)
    W = _bf16_rows(rng, (V, d), 2.5 / np.sqrt(d))
    g = rng.integers(0, V, (B, R)).astype(np.int32)
    Wg = bf16_to_f32(W[g.reshape(-1)]).astype(np.float64)
    u = Wg / np.maximum(np.linalg.norm(Wg, axis=1, keepdims=True), 1e-30)
    h = (alpha * u + rng.standard_normal(u.shape) * noise).astype(np.float32)
    hidden = bf16_bits(h).reshape(B, R, d)
    w = dict(kind="lmhead", hidden=hidden, W=W, planted=g, tree=tree)
    if not tree:
        gam = R - 1
        match = rng.random((B, gam)) < p_match
        w["tokens"] = np.where(match, g[:, :gam], _other_id(rng, V, g[:, :gam])).astype(np.int32)
    else:
        parents = np.stack([tree_topology(rng, R, max_depth, max_children) for _ in range(B)])
        tokens = np.zeros((B, R), np.int32)
        for b in range(B):
            for k in range(1, R):
                pg = g[b, parents[b, k]]
                tokens[b, k] = pg if rng.random() < p_match else _other_id(rng, V, pg)
        w["tokens"], w["parents"] = tokens, parents
    return w


def tree_topology(rng: np.random.Generator, N: int = 32, max_depth: int = 5, max_children: int = 8):
    """Random parent array: node 0 is the root; node k picks a parent uniformly
    among earlier nodes with depth < max_depth and fewer than max_children children."""
    parents = np.full(N, -1, np.int32)
    depth = np.zeros(N, np.int32)
    kids = np.zeros(N, np.int32)
    for k in range(1, N):
        ok = np.flatnonzero((depth[:k] < max_depth) & (kids[:k] < max_children))
        p = int(ok[rng.integers(0, len(ok))])
        parents[k] = p
        depth[k] = depth[p] + 1
        kids[p] += 1
    return parents


def tree(seed: int, B: int = 16, N: int = 32, V: int = 49152, max_depth: int = 5,
         max_children: int = 8, p_match: float = 0.6) -> dict:
    rng = np.random.default_rng(seed)
    zb = bf16_bits(_normal(rng, (B, N, V), 2.0))
    am = np.argmax(bf16_to_f32(zb), axis=-1).astype(np.int32)      # [B, N]
    parents = np.stack([tree_topology(rng, N, max_depth, max_children) for _ in range(B)])
    tokens = np.zeros((B, N), np.int32)
    for b in range(B):
        for k in range(1, N):
            g = am[b, parents[b, k]]
            tokens[b, k] = g if rng.random() < p_match else _other_id(rng, V, g)
    return dict(kind="tree", target=zb, tokens=tokens, parents=parents)


WORKLOADS = {
    "sample_plain": sample_plain,
    "sample_topp": sample_topp,
    "greedy": greedy,
    "eagle_d2t": eagle_d2t,
    "tree": tree,
    "draft": draft,
    "fanout": fanout,
    "trim": token_stream,
    "lmhead": lmhead,
}
