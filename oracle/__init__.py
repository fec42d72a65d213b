"""CPU oracle of the verification path - TEST INFRASTRUCTURE ONLY.

ctypes binding over ``oracle/liboracle.so`` (built from ``oracle/oracle.cpp`` by
``oracle.build_oracle()``, or by the repository's build entry point).  Only tests, the smoke check and the
bench's CPU-baseline leg use it; the product package never imports it.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")
SRC_PATH = os.path.join(_HERE, "oracle.cpp")

ST_EMPTY_RESIDUAL = 8
ST_OUTSIDE_DRAFT_SUPPORT = 16
ST_BAD_LOGIT = 32
ST_BAD_TOKEN = 64
ST_DEGENERATE_DOWNWEIGHT = 128
ST_BAD_PARAM = 256
FL_NEAR_ACCEPT = 1
FL_NEAR_CDF = 2
FL_NEAR_NUCLEUS = 4
FL_NEAR_FUZZY = 8

FP32 = 0
BF16 = 1

PARAMS_DTYPE = np.dtype([("t", "<f4"), ("k", "<i4"), ("p", "<f4")])


def build_oracle() -> str:
    cmd = ["g++", "-O2", "-std=c++17", "-Wall", "-shared", "-fPIC", SRC_PATH, "-o", LIB_PATH, "-lpthread"]
    subprocess.run(cmd, check=True)
    return LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH) or os.path.getmtime(LIB_PATH) < os.path.getmtime(SRC_PATH):
            build_oracle()
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        i32, u64, f32, f64 = ctypes.c_int, ctypes.c_uint64, ctypes.c_float, ctypes.c_double
        L.orc_philox4x64_10.argtypes = [P, P, P]
        L.orc_uniforms.argtypes = [u64, u64, i32, i32, P]
        L.orc_process_row_f64.argtypes = [P, i32, f32, ctypes.c_int32, f32, P, P, P]
        L.orc_process_row_f64.restype = i32
        L.orc_downweight_probs_f64.argtypes = [P, P, i32, i32, f64, P, P]
        L.orc_downweight_probs_f64.restype = f64
        L.orc_downweight.argtypes = [P, i32, i32, i32, i32, i32, P, i32, f64, P, P, P, P, i32]
        L.orc_verify_u.argtypes = [P, i32, P, i32, i32, i32, i32, P, i32, f64, P, i32, P, P, P, P, P, P, i32, i32,
                                   P, i32, P]
        L.orc_verify.argtypes = [P, i32, P, i32, i32, i32, i32, P, i32, f64, P, i32, u64, u64, P, P, P, P, P, i32,
                                 i32, P, i32, P]
        L.orc_jsd_bits.argtypes = [P, P, i32]
        L.orc_jsd_bits.restype = f64
        L.orc_uniform_tokens.argtypes = [P, i32, i32, P]
        L.orc_backup_plan.argtypes = [i32, P, i32, i32, P, P]
        L.orc_fanout.argtypes = [i32, i32, f64, f64, P, P]
        L.orc_cache_build.argtypes = [P, i32, i32, i32, i32, P, P, P, i32]
        L.orc_cache_lookup.argtypes = [i32, P, P, i32, i32, P, P, P, P, P]
        L.orc_threads_used.argtypes = [i32]
        L.orc_signposts.argtypes = [P, i32, i32, i32, i32, P, P, P, i32]
        L.orc_tree_lookup.argtypes = [P, P, i32, i32, i32, P, P, P, P, P, P]
        for fn in ("orc_downweight", "orc_verify_u", "orc_verify", "orc_fanout", "orc_cache_build",
                   "orc_cache_lookup", "orc_threads_used", "orc_signposts", "orc_tree_lookup"):
            getattr(L, fn).restype = i32
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data


def threads_used(nthreads: int = 0) -> int:
    return lib().orc_threads_used(nthreads)


def philox4x64_10(ctr, key) -> np.ndarray:
    c = np.ascontiguousarray(ctr, dtype=np.uint64)
    k = np.ascontiguousarray(key, dtype=np.uint64)
    out = np.zeros(4, dtype=np.uint64)
    lib().orc_philox4x64_10(_p(c), _p(k), _p(out))
    return out


def uniforms(seed: int, round_: int, B: int, K: int) -> np.ndarray:
    """U[B][K+1][3]: lanes 0 (acceptance), 1 (residual/bonus), 2 (draft sampling)."""
    U = np.zeros((B, K + 1, 3), dtype=np.float64)
    lib().orc_uniforms(seed, round_, B, K, _p(U))
    return U


def process_row(z, temperature=1.0, top_k=0, top_p=1.0):
    """Processed distribution of one fp64 logit row. Returns (p, bad, near_cut, n_kept)."""
    z = np.ascontiguousarray(z, dtype=np.float64)
    p = np.zeros(z.shape[0], dtype=np.float64)
    near = ctypes.c_int(0)
    nk = ctypes.c_int(0)
    bad = lib().orc_process_row_f64(_p(z), z.shape[0], temperature, top_k, top_p, _p(p),
                                    ctypes.byref(near), ctypes.byref(nk))
    return p, bool(bad), bool(near.value), nk.value


def downweight_probs(z, p, F, C):
    """sigma_{F,C} on a processed row p (order taken from logits z). Returns (p', Z, ids, degenerate)."""
    z = np.ascontiguousarray(z, dtype=np.float64)
    pp = np.array(p, dtype=np.float64, copy=True)
    ids = np.full(max(F, 1), -1, dtype=np.int32)
    deg = ctypes.c_int(0)
    Z = lib().orc_downweight_probs_f64(_p(z), _p(pp), z.shape[0], F, C, _p(ids), ctypes.byref(deg))
    return pp, Z, ids[:F], bool(deg.value)


def params_array(temperature, top_k, top_p, B=None):
    if B is None:
        B = len(np.atleast_1d(temperature))
    rec = np.zeros(B, dtype=PARAMS_DTYPE)
    rec["t"] = temperature
    rec["k"] = top_k
    rec["p"] = top_p
    return rec


@dataclass
class VerifyResult:
    k: np.ndarray
    t: np.ndarray
    W: np.ndarray
    status: np.ndarray
    flags: np.ndarray
    tokens: np.ndarray
    div: Optional[np.ndarray] = None


def _check(rc, name):
    if rc != 0:
        raise ValueError(f"oracle {name} rejected its arguments (rc={rc})")


def verify(draft, target, dtype, K, params, F=0, C=1.0, tokens=None, seed=0, round_=0, U=None,
           nthreads=0, uniform_draft=False, tau=None, assisted=False) -> VerifyResult:
    """draft [B][Kd][V], target [B][K+1][V] (float32 or uint16 bf16 bits).

    ``tokens`` None => the draft tokens are sampled from the processed draft (lane 2).
    ``U`` given => explicit uniforms [B][K+1][3] instead of the Philox stream.
    ``uniform_draft`` => the draft distribution is uniform on [0, V) (``draft`` may be None).
    ``tau`` [B] => fuzzy acceptance (PyramidSD) with these thresholds; ``assisted`` => the
    correction is drawn from q; the result's ``div`` holds the divergences [B][K].
    """
    target = np.ascontiguousarray(target)
    if draft is None:
        assert uniform_draft
        B, _, V = target.shape
        Kd = K
    else:
        draft = np.ascontiguousarray(draft)
        B, Kd, V = draft.shape
    params = np.ascontiguousarray(params, dtype=PARAMS_DTYPE)
    sample = tokens is None
    tok = np.zeros((B, K), dtype=np.int32) if sample else np.array(tokens, dtype=np.int32, copy=True)
    k = np.zeros(B, np.int32)
    t = np.zeros(B, np.int32)
    W = np.zeros(B, np.float64)
    st = np.zeros(B, np.uint32)
    fl = np.zeros(B, np.uint32)
    tau_a = None if tau is None else np.ascontiguousarray(np.broadcast_to(np.asarray(tau, np.float64), (B,)))
    div = None if tau is None else np.zeros((B, K), np.float64)
    fz = (_p(tau_a), int(assisted), _p(div))
    if U is None:
        rc = lib().orc_verify(_p(draft), Kd, _p(target), dtype, B, K, V, _p(params), F, C, _p(tok), int(sample),
                              seed, round_, _p(k), _p(t), _p(W), _p(st), _p(fl), nthreads, int(uniform_draft), *fz)
    else:
        U = np.ascontiguousarray(U, dtype=np.float64)
        assert U.shape == (B, K + 1, 3)
        rc = lib().orc_verify_u(_p(draft), Kd, _p(target), dtype, B, K, V, _p(params), F, C, _p(tok), int(sample),
                                _p(U), _p(k), _p(t), _p(W), _p(st), _p(fl), nthreads, int(uniform_draft), *fz)
    _check(rc, "verify")
    return VerifyResult(k, t, W, st, fl, tok, div)


def downweight(draft, dtype, K, params, F, C, want_probs=False, nthreads=0):
    draft = np.ascontiguousarray(draft)
    B, Kd, V = draft.shape
    params = np.ascontiguousarray(params, dtype=PARAMS_DTYPE)
    ids = np.zeros((B, K, max(F, 1)), np.int32)
    Z = np.zeros((B, K), np.float64)
    st = np.zeros((B, K), np.uint32)
    probs = np.zeros((B, K, V), np.float64) if want_probs else None
    rc = lib().orc_downweight(_p(draft), Kd, dtype, B, K, V, _p(params), F, C, _p(ids), _p(Z), _p(probs), _p(st),
                              nthreads)
    _check(rc, "downweight")
    return ids[:, :, :F], Z, probs, st


def fanout(K, budget, a, r):
    real = np.zeros(K + 1, np.float64)
    ints = np.zeros(K + 1, np.int32)
    _check(lib().orc_fanout(K, budget, a, r, _p(real), _p(ints)), "fanout")
    return real, ints


def cache_build(draft, dtype, K, tokens, fan, nthreads=0):
    draft = np.ascontiguousarray(draft)
    B, Kd, V = draft.shape
    assert Kd == K + 1
    tokens = np.ascontiguousarray(tokens, dtype=np.int32)
    fan = np.ascontiguousarray(fan, dtype=np.int32)
    out = np.zeros((B, int(fan.sum())), np.int32)
    _check(lib().orc_cache_build(_p(draft), dtype, B, K, V, _p(tokens), _p(fan), _p(out), nthreads), "cache_build")
    return out


def cache_lookup(mode, cache, fan_or_shape, K, B, k, t):
    cache = np.ascontiguousarray(cache, dtype=np.int32)
    fs = np.ascontiguousarray(fan_or_shape, dtype=np.int32)
    k = np.ascontiguousarray(k, dtype=np.int32)
    t = np.ascontiguousarray(t, dtype=np.int32)
    slot = np.zeros(B, np.int32)
    hit = np.zeros(B, np.uint8)
    batch = np.zeros(2, np.int32)
    _check(lib().orc_cache_lookup(mode, _p(cache), _p(fs), K, B, _p(k), _p(t), _p(slot), _p(hit), _p(batch)),
           "cache_lookup")
    return slot, hit, batch


def uniform_tokens(u, V):
    """floor(u * V) for uniforms u from the Philox stream (exact)."""
    u = np.ascontiguousarray(u, dtype=np.float64)
    out = np.zeros(u.shape, np.int32)
    lib().orc_uniform_tokens(_p(u), u.size, V, _p(out))
    return out


def backup_plan(B, hit, all_hit, b_star):
    """(use_backup[B], switch): the batch-aware random-token fallback."""
    hit = np.ascontiguousarray(hit, dtype=np.uint8)
    use = np.zeros(B, np.int32)
    sw = np.zeros(1, np.int32)
    lib().orc_backup_plan(B, _p(hit), int(all_hit), b_star, _p(use), _p(sw))
    return use, int(sw[0])


def signposts(logits, dtype, kappa, nthreads=0):
    """Mirror-SD signposts of early-exit logits [B][V]: (ids [B][kappa], log p~ [B][kappa], status [B])."""
    logits = np.ascontiguousarray(logits)
    B, V = logits.shape
    ids = np.zeros((B, kappa), np.int32)
    lp = np.zeros((B, kappa), np.float64)
    st = np.zeros(B, np.uint32)
    _check(lib().orc_signposts(_p(logits), dtype, B, V, kappa, _p(ids), _p(lp), _p(st), nthreads), "signposts")
    return ids, lp, st


def tree_lookup(tokens, parents, path, k, t):
    """Reuse of the committed prefix against draft trees [B][N]: (node [B], hit [B], batch [2])."""
    tokens = np.ascontiguousarray(tokens, dtype=np.int32)
    parents = np.ascontiguousarray(parents, dtype=np.int32)
    path = np.ascontiguousarray(path, dtype=np.int32)
    k = np.ascontiguousarray(k, dtype=np.int32)
    t = np.ascontiguousarray(t, dtype=np.int32)
    B, N = tokens.shape
    gamma = path.shape[1]
    node = np.zeros(B, np.int32)
    hit = np.zeros(B, np.uint8)
    batch = np.zeros(2, np.int32)
    _check(lib().orc_tree_lookup(_p(tokens), _p(parents), B, N, gamma, _p(path), _p(k), _p(t), _p(node), _p(hit),
                                 _p(batch)), "tree_lookup")
    return node, hit, batch


def jsd_bits(p, q):
    """Jensen-Shannon divergence in bits of two distributions (the oracle's own routine)."""
    p = np.ascontiguousarray(p, dtype=np.float64)
    q = np.ascontiguousarray(q, dtype=np.float64)
    return float(lib().orc_jsd_bits(_p(p), _p(q), len(p)))
