"""Seeded synthetic inputs for the verification path.

This module only draws random logits, per-request parameters and (for the branch tree)
draft tokens with the shapes and value distributions of the workloads the pages describe.
It holds none of the verification arithmetic (no processing of distributions, no acceptance
test, no residual, no cache), so the GPU path and the CPU oracle can both be fed from it.

Workloads (the logit recipes are stand-ins for real model logits, which are not available):

* ``vanilla``  - fp32, target logits iid N(0, 2^2), draft = target + N(0, 0.5^2),
  temperature 1, no truncation (B independent rounds batched as B requests).
* ``llama``    - bf16, V = 128256, Zipf-shaped target rows (the logit of the token at
  sorted rank r is -1.1 ln(r+1) + N(0,1), ranks placed by a fresh random permutation per
  row), draft = target + N(0, 0.8^2), temperature 1, top-p 0.8.
* ``saguaro``  - bf16, B = 16, K = 5, V = 128256, Zipf target rows, per-row draft noise
  sigma ~ U[0.3, 1.2], per-request temperature U[0.6, 1.0], top-p 0.95, downweight of the
  top F = 4 draft tokens by C = 0.3.  One extra draft row (position K) is drawn for the
  outcome cache (budget 32, a = 0.7, r = 1).
* ``tree``     - bf16, 64 requests x 8 branches of depth 7 (512 chains), V = 151936,
  temperature 0.8, top-k 50.  Branch j >= 1 shares rows and tokens with branch 0 up to
  depth j-2, takes at depth j-1 the highest-logit draft token other than branch 0's, and
  continues with rows and tokens of its own.  Draft tokens are proposals of a stand-in
  drafter: a Gumbel-max draw over the 50 largest raw draft logits scaled by 1/T.
* ``mirror``   - bf16 early-exit rows (B = 64, V = 151936, Zipf-shaped) for the signposts, and
  per request a draft tree in parent-first order: kappa = 8 root tokens, each expanded to a
  chain of depth gamma = 7, with extra siblings forking off internal nodes (each fork
  continues to depth gamma), padded to N nodes with token -1.  The verified path is root 0's
  chain; k is a truncated geometric draw (per-token acceptance 0.7) and t* is, with
  probability 1/2, the token of a fork off the accepted prefix, else a random token.
* ``pyramid``  - bf16, V = 128256, three models of one family with an entropy gradient (the
  smaller the model, the flatter its rows).  Stage 1 verifies l_D = 12 drafted tokens against
  the qualifier (tau_Q = 0.4): qualifier rows 0.8 t + N(0, 1), drafter rows
  0.55 t + N(0, s^2) with s ~ U[0.8, 1.6] per row.  Stage 2 verifies l_Q = 25 tokens against
  the target (tau_T = 0.5): target rows t, qualifier rows 0.8 t + N(0, s^2), s ~ U[1, 3] per
  row.  t is Zipf-shaped; temperature 1, no truncation, B = 16; the drafted tokens of both
  stages are drawn by the path from the drafting rows.  The per-row noise spreads the
  divergences across the thresholds.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

DATA_SEED_BASE = 0x5EED0000
VERIFY_SEED_BASE = 0xC0FFEE00

FP32 = 0
BF16 = 1


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even); returns uint16 bits."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    nan = (b & 0x7FFFFFFF) > 0x7F800000
    r = ((b + np.uint32(0x7FFF) + ((b >> 16) & np.uint32(1))) >> 16).astype(np.uint16)
    r[nan] = np.uint16(0x7FC0)
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def zipf_rows(rng: np.random.Generator, n: int, V: int, slope: float = 1.1,
              jitter: float = 1.0) -> np.ndarray:
    """n rows whose token at sorted rank r has logit -slope*ln(r+1) + N(0, jitter^2)."""
    base = (-slope * np.log1p(np.arange(V, dtype=np.float64))).astype(np.float32)
    out = np.empty((n, V), dtype=np.float32)
    step = max(1, (1 << 24) // max(V, 1))
    for lo in range(0, n, step):
        hi = min(n, lo + step)
        perm = rng.permuted(np.tile(np.arange(V, dtype=np.int64), (hi - lo, 1)), axis=1)
        vals = base[None, :] + jitter * rng.standard_normal((hi - lo, V), dtype=np.float32)
        np.put_along_axis(out[lo:hi], perm, vals, axis=1)
    return out


@dataclass
class Workload:
    """One batch of verification inputs.

    draft: [B][Kd][V] (uint16 bf16 bits or float32), Kd = K, or K + 1 when the cache row is present
    target: [B][K+1][V]
    temperature/top_k/top_p: per request, applied to draft and target alike
    tokens: [B][K] int32 draft tokens, or None when they are to be sampled by the path itself
    """
    name: str
    dtype: int
    B: int
    K: int
    V: int
    draft: np.ndarray
    target: np.ndarray
    temperature: np.ndarray
    top_k: np.ndarray
    top_p: np.ndarray
    F: int = 0
    C: float = 1.0
    seed: int = 0
    round: int = 0
    tokens: Optional[np.ndarray] = None
    budget: int = 0
    a: float = 0.0
    r: float = 0.0
    kappa: int = 0
    gamma: int = 0
    meta: dict = field(default_factory=dict)

    @property
    def draft_rows(self) -> int:
        return int(self.draft.shape[1])

    def logit_bytes(self) -> int:
        return int(self.draft.nbytes + self.target.nbytes)

    def params(self) -> np.ndarray:
        """Per-request parameters packed as the C struct {float T; int32 top_k; float top_p}."""
        rec = np.zeros(self.B, dtype=np.dtype([("t", "<f4"), ("k", "<i4"), ("p", "<f4")]))
        rec["t"] = self.temperature
        rec["k"] = self.top_k
        rec["p"] = self.top_p
        return rec

    def without_cache_row(self) -> "Workload":
        if self.draft_rows == self.K:
            return self
        w = Workload(**{**self.__dict__})
        w.draft = np.ascontiguousarray(self.draft[:, : self.K])
        return w


def _params(B, T, k, p):
    return (np.full(B, T, np.float32) if np.isscalar(T) else np.asarray(T, np.float32),
            np.full(B, k, np.int32) if np.isscalar(k) else np.asarray(k, np.int32),
            np.full(B, p, np.float32) if np.isscalar(p) else np.asarray(p, np.float32))


def vanilla(B: int = 10000, K: int = 4, V: int = 1024, cfg: int = 1) -> Workload:
    rng = np.random.default_rng(DATA_SEED_BASE + cfg)
    target = (2.0 * rng.standard_normal((B, K + 1, V), dtype=np.float32)).astype(np.float32)
    draft = (target[:, :K] + 0.5 * rng.standard_normal((B, K, V), dtype=np.float32)).astype(np.float32)
    T, k, p = _params(B, 1.0, 0, 1.0)
    return Workload("vanilla", FP32, B, K, V, np.ascontiguousarray(draft), target, T, k, p,
                    seed=VERIFY_SEED_BASE + cfg)


def llama(B: int = 1000, K: int = 5, V: int = 128256, cfg: int = 2) -> Workload:
    rng = np.random.default_rng(DATA_SEED_BASE + cfg)
    target = zipf_rows(rng, B * (K + 1), V).reshape(B, K + 1, V)
    draft = target[:, :K] + 0.8 * rng.standard_normal((B, K, V), dtype=np.float32)
    T, k, p = _params(B, 1.0, 0, 0.8)
    return Workload("llama", BF16, B, K, V, f32_to_bf16_bits(draft), f32_to_bf16_bits(target),
                    T, k, p, seed=VERIFY_SEED_BASE + cfg)


def saguaro(B: int = 16, K: int = 5, V: int = 128256, cache_row: bool = True, cfg: int = 3,
            F: int = 4, C: float = 0.3, top_p: float = 0.95) -> Workload:
    """Batched verify + Saguaro sampling; with ``cache_row`` also the row for position K."""
    rng = np.random.default_rng(DATA_SEED_BASE + 3)
    target = zipf_rows(rng, B * (K + 1), V).reshape(B, K + 1, V)
    sigma = rng.uniform(0.3, 1.2, size=(B, K + 1)).astype(np.float32)
    draft = target + sigma[:, :, None] * rng.standard_normal((B, K + 1, V), dtype=np.float32)
    temp = rng.uniform(0.6, 1.0, size=B).astype(np.float32)
    T, k, p = _params(B, temp, 0, top_p)
    d = draft if cache_row else draft[:, :K]
    w = Workload("saguaro", BF16, B, K, V, f32_to_bf16_bits(np.ascontiguousarray(d)),
                 f32_to_bf16_bits(target), T, k, p, F=F, C=C, seed=VERIFY_SEED_BASE + cfg,
                 budget=32, a=0.7, r=1.0)
    w.meta["sigma"] = sigma
    return w


def _gumbel_topk_token(rng, logits: np.ndarray, T: float, top_k: int) -> int:
    idx = np.argpartition(-logits, top_k - 1)[:top_k]
    g = -np.log(-np.log(rng.uniform(np.finfo(np.float64).tiny, 1.0, size=top_k)))
    return int(idx[np.argmax(logits[idx].astype(np.float64) / T + g)])


def tree(n_req: int = 64, kappa: int = 8, gamma: int = 7, V: int = 151936, T: float = 0.8,
         top_k: int = 50, cfg: int = 5) -> Workload:
    """Branch-complete trees verified as n_req*kappa independent chains of depth gamma."""
    assert 1 <= kappa - 1 <= gamma
    rng = np.random.default_rng(DATA_SEED_BASE + cfg)
    B = n_req * kappa
    draft = np.empty((B, gamma, V), dtype=np.uint16)
    target = np.empty((B, gamma + 1, V), dtype=np.uint16)
    tokens = np.empty((B, gamma), dtype=np.int32)
    for r in range(n_req):
        b0 = r * kappa
        t0 = zipf_rows(rng, gamma + 1, V)
        d0 = t0[:gamma] + 0.8 * rng.standard_normal((gamma, V), dtype=np.float32)
        target[b0] = f32_to_bf16_bits(t0)
        draft[b0] = f32_to_bf16_bits(d0)
        d0q = bf16_bits_to_f32(draft[b0])
        for d in range(gamma):
            tokens[b0, d] = _gumbel_topk_token(rng, d0q[d], T, top_k)
        for j in range(1, kappa):
            b = b0 + j
            split = j - 1                      # depth at which branch j leaves branch 0
            target[b, : split + 1] = target[b0, : split + 1]
            draft[b, : split + 1] = draft[b0, : split + 1]
            tokens[b, :split] = tokens[b0, :split]
            row = d0q[split].copy()
            row[tokens[b0, split]] = -np.inf
            tokens[b, split] = int(np.argmax(row))   # highest raw logit, lowest id on ties
            n_new = gamma - split - 1
            if n_new > 0:
                tn = zipf_rows(rng, n_new + 1, V)
                dn = tn[:n_new] + 0.8 * rng.standard_normal((n_new, V), dtype=np.float32)
                target[b, split + 1:] = f32_to_bf16_bits(tn)
                draft[b, split + 1:] = f32_to_bf16_bits(dn)
                dnq = bf16_bits_to_f32(draft[b, split + 1:])
                for d in range(n_new):
                    tokens[b, split + 1 + d] = _gumbel_topk_token(rng, dnq[d], T, top_k)
            else:
                tn = zipf_rows(rng, 1, V)
                target[b, gamma] = f32_to_bf16_bits(tn)[0]
    Tv, kv, pv = _params(B, T, top_k, 1.0)
    return Workload("tree", BF16, B, gamma, V, draft, target, Tv, kv, pv, seed=VERIFY_SEED_BASE + cfg,
                    tokens=tokens, kappa=kappa, gamma=gamma)


def random_rows(rng: np.random.Generator, B: int, K: int, V: int, dtype: int, draft_rows: Optional[int] = None,
                scale: float = 2.0, noise: float = 0.7) -> tuple[np.ndarray, np.ndarray]:
    """Small gaussian draft/target logits for fuzz shapes (dtype FP32 -> float32, BF16 -> bits)."""
    Kd = K if draft_rows is None else draft_rows
    target = (scale * rng.standard_normal((B, K + 1, V))).astype(np.float32)
    extra = Kd - K
    base = np.concatenate([target[:, :K], target[:, K:K + extra]], axis=1) if extra else target[:, :K]
    draft = (base + noise * rng.standard_normal((B, Kd, V))).astype(np.float32)
    if dtype == BF16:
        return f32_to_bf16_bits(draft), f32_to_bf16_bits(target)
    return draft, target


@dataclass
class MirrorWorkload:
    """Early-exit rows [B][V] (bf16 bits) and per-request draft trees [B][N] (parent-first)."""
    B: int
    V: int
    kappa: int
    gamma: int
    logits: np.ndarray
    tokens: np.ndarray
    parents: np.ndarray
    path: np.ndarray
    k: np.ndarray
    tstar: np.ndarray


def mirror(B: int = 64, V: int = 151936, kappa: int = 8, gamma: int = 7, N: int = 128, p_fork: float = 0.25,
           cfg: int = 6) -> MirrorWorkload:
    rng = np.random.default_rng(DATA_SEED_BASE + cfg)
    logits = f32_to_bf16_bits(zipf_rows(rng, B, V))
    tok = np.full((B, N), -1, np.int32)
    par = np.full((B, N), -1, np.int32)
    path = np.zeros((B, gamma), np.int32)
    kk = np.zeros(B, np.int32)
    tt = np.zeros(B, np.int32)
    for b in range(B):
        nodes = []                                   # (token, parent)

        def chain(parent, depth):                    # nodes from `depth` (1-based) to gamma
            ids = []
            for _ in range(depth, gamma + 1):
                nodes.append((int(rng.integers(0, V)), parent))
                parent = len(nodes) - 1
                ids.append(parent)
            return ids

        roots = rng.choice(V, kappa, replace=False)
        main = []
        for j in range(kappa):
            nodes.append((int(roots[j]), -1))
        for j in range(kappa):
            ids = [j] + chain(j, 2)
            if j == 0:
                main = ids
            for d in range(1, gamma):                # forks below internal nodes
                if rng.random() < p_fork and len(nodes) + gamma - d <= N:
                    chain(ids[d - 1], d + 1)
        nodes = nodes[:N]
        for n, (t_, p_) in enumerate(nodes):
            tok[b, n], par[b, n] = t_, p_
        path[b] = [nodes[i][0] for i in main]
        k = 0
        while k < gamma and rng.random() < 0.7:
            k += 1
        kk[b] = k
        if k < gamma:
            parent = main[k - 1] if k > 0 else -1
            # a rejected draft token is never the correction: forks of the prefix only
            kids = [n for n, (_, p_) in enumerate(nodes) if p_ == parent and n != main[k]]
            tt[b] = nodes[int(rng.choice(kids))][0] if kids and rng.random() < 0.5 else int(rng.integers(0, V))
        else:
            tt[b] = int(rng.integers(0, V))
    return MirrorWorkload(B, V, kappa, gamma, logits, tok, par, path, kk, tt)


@dataclass
class PyramidStage:
    """One fuzzy verification stage: drafter rows [B][K][V] against verifier rows [B][K+1][V]."""
    name: str
    B: int
    K: int
    V: int
    draft: np.ndarray
    verifier: np.ndarray
    tau: np.ndarray
    tokens: Optional[np.ndarray]
    seed: int


def pyramid(B: int = 16, l_d: int = 12, l_q: int = 25, V: int = 128256, tau_q: float = 0.4, tau_t: float = 0.5,
            cfg: int = 7) -> tuple[PyramidStage, PyramidStage]:
    rng = np.random.default_rng(DATA_SEED_BASE + cfg)
    # stage 1: qualifier rows 0.8 t + N(0, 1), drafter rows 0.55 t + N(0, s^2), s ~ U[0.8, 1.6] per row
    t = zipf_rows(rng, B * (l_d + 1), V).reshape(B, l_d + 1, V)
    q1 = 0.8 * t + rng.standard_normal(t.shape, dtype=np.float32)
    s_d = rng.uniform(0.8, 1.6, size=(B, l_d, 1)).astype(np.float32)
    d1 = 0.55 * t[:, :l_d] + s_d * rng.standard_normal((B, l_d, V), dtype=np.float32)
    s1 = PyramidStage("draft->qualifier", B, l_d, V, f32_to_bf16_bits(d1), f32_to_bf16_bits(q1),
                      np.full(B, tau_q, np.float32), None, VERIFY_SEED_BASE + cfg)
    del t, q1, d1
    # stage 2: target rows t, qualifier rows 0.8 t + N(0, s^2), s ~ U[1, 3] per row
    t2 = zipf_rows(rng, B * (l_q + 1), V).reshape(B, l_q + 1, V)
    s_q = rng.uniform(1.0, 3.0, size=(B, l_q, 1)).astype(np.float32)
    q2 = 0.8 * t2[:, :l_q] + s_q * rng.standard_normal((B, l_q, V), dtype=np.float32)
    s2 = PyramidStage("qualifier->target", B, l_q, V, f32_to_bf16_bits(q2), f32_to_bf16_bits(t2),
                      np.full(B, tau_t, np.float32), None, VERIFY_SEED_BASE + cfg + 1)
    return s1, s2
