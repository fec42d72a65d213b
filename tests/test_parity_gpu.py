"""GPU <-> oracle parity through the C ABI (needs an MI355X).

Integers (k, t*, sampled draft tokens, status bits, downweighted sets, cache token sets, hit
flags, slots, branch reuse) must be equal on every request the oracle does not flag as a near
tie (a uniform within 1e-6 relative of an acceptance boundary, a CDF or nucleus target within
1e-9 of the total mass); floats within 1e-5
relative (fp32 inputs) or 2e-3 (bf16 inputs).  Flagged requests are counted and reported.
"""
import numpy as np
import pytest
import torch

import oracle
from flagbound import bound_flagged
from lossless_speculative_sampling_amd import capi, synth

pytestmark = pytest.mark.gpu

RTOL = {synth.FP32: 1e-5, synth.BF16: 2e-3}


def dev(a: np.ndarray) -> torch.Tensor:
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def say(msg):
    print(msg, flush=True)


def run_gpu(w, tokens=None, seed=None, round_=0):
    sample = tokens is None
    prm = capi.params_tensor(w.temperature, w.top_k, w.top_p)
    tok = torch.zeros((w.B, w.K), dtype=torch.int32, device="cuda") if sample else dev(np.asarray(tokens, np.int32))
    out = capi.spec_verify(dev(w.draft), dev(w.target), w.K, prm, tok, F=w.F, C=w.C,
                           seed=w.seed if seed is None else seed, round_=round_,
                           flags=capi.SPEC_SAMPLE_DRAFT if sample else 0)
    torch.cuda.synchronize()
    return (out.k.cpu().numpy(), out.tstar.cpu().numpy(), out.resid_mass.cpu().numpy(),
            out.status.cpu().numpy().astype(np.uint32), out.tokens.cpu().numpy())


def run_oracle(w, tokens=None, seed=None, round_=0):
    return oracle.verify(w.draft, w.target, w.dtype, w.K, w.params(), F=w.F, C=float(np.float32(w.C)),
                         tokens=tokens, seed=w.seed if seed is None else seed, round_=round_)


def check_verify(w, tokens=None, seed=None, round_=0, label="", allow_flags=None):
    say(f"[parity] {label} {w.name} B={w.B} K={w.K} V={w.V} dtype={w.dtype} sample={tokens is None}")
    o = run_oracle(w, tokens, seed, round_)
    bound_flagged(o.flags, f"{label} {w.name}", allow_flags)
    k, t, W, st, tok = run_gpu(w, tokens, seed, round_)
    ok = o.flags == 0
    bad = np.flatnonzero(ok & ((k != o.k) | (t != o.t) | (st != o.status)))
    assert len(bad) == 0, (f"{len(bad)} mismatches, first {bad[:5]}: gpu k={k[bad[:5]]} t={t[bad[:5]]} "
                           f"st={st[bad[:5]]} | oracle k={o.k[bad[:5]]} t={o.t[bad[:5]]} st={o.status[bad[:5]]}")
    if tokens is None:
        good = ok & ((o.status & (oracle.ST_BAD_LOGIT | oracle.ST_BAD_PARAM)) == 0)
        assert (tok[good] == o.tokens[good]).all()
    np.testing.assert_allclose(W[ok], o.W[ok], rtol=RTOL[w.dtype], atol=1e-6)
    say(f"[parity] {label} ok: flagged {int((~ok).sum())} of {w.B}; mean k {k.mean():.3f}")
    return o, int((~ok).sum())


def test_vanilla_fp32_ten_thousand_rounds():
    check_verify(synth.vanilla(B=10000), label="vanilla")


def test_llama_vocab_bf16_nucleus():
    check_verify(synth.llama(B=12), label="llama")


def test_saguaro_full_size_sampled_and_given_tokens():
    w = synth.saguaro(B=16, K=5, V=128256, cache_row=False)
    o, _ = check_verify(w, label="saguaro-sampled")
    check_verify(w, tokens=o.tokens, label="saguaro-given")
    # also with the cache row present in the draft tensor
    w4 = synth.saguaro(B=16, K=5, V=128256, cache_row=True)
    check_verify(w4, tokens=o.tokens, label="saguaro-cache-row")


def test_deterministic_repeat():
    w = synth.saguaro(B=16, K=5, V=128256, cache_row=False)
    a = run_gpu(w)
    b = run_gpu(w)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_downweight_parity():
    w = synth.saguaro(B=16, K=5, V=128256, cache_row=False)
    say("[parity] downweight B=16 K=5 V=128256")
    prm = capi.params_tensor(w.temperature, w.top_k, w.top_p)
    ids, Z, probs, st = capi.saguaro_downweight(dev(w.draft), w.K, prm, w.F, w.C, want_probs=True)
    torch.cuda.synchronize()
    oids, oZ, oprobs, ost = oracle.downweight(w.draft, w.dtype, w.K, w.params(), w.F, float(np.float32(w.C)),
                                              want_probs=True)
    assert (ids.cpu().numpy() == oids).all()
    assert (st.cpu().numpy().astype(np.uint32) == ost).all()
    np.testing.assert_allclose(Z.cpu().numpy(), oZ, rtol=1e-6)
    np.testing.assert_allclose(probs.cpu().numpy(), oprobs, rtol=2e-6, atol=1e-12)


def test_cache_build_and_lookup():
    w = synth.saguaro(B=16, K=5, V=128256, cache_row=True)
    say("[parity] cache build + lookup B=16 K=5 V=128256 budget=32")
    o = run_oracle(w.without_cache_row())
    cache, fan = capi.saguaro_cache_build(dev(w.draft), w.K, dev(o.tokens), w.budget, w.a, w.r)
    torch.cuda.synchronize()
    assert fan == [7, 6, 5, 4, 4, 6]
    ocache = oracle.cache_build(w.draft, w.dtype, w.K, o.tokens, np.array(fan, np.int32))
    assert (cache.cpu().numpy() == ocache).all()
    slot, hit, batch = capi.saguaro_cache_lookup(0, cache, fan, w.K, w.B, dev(o.k), dev(o.t))
    torch.cuda.synchronize()
    oslot, ohit, obatch = oracle.cache_lookup(0, ocache, fan, w.K, w.B, o.k, o.t)
    assert (slot.cpu().numpy() == oslot).all() and (hit.cpu().numpy() == ohit).all()
    assert (batch.cpu().numpy() == obatch).all()
    say(f"[parity] cache ok: hits {int(obatch[0])}/{w.B}")


def _check_fused(w, tokens=None, label="", allow_flags=None, round_=0):
    """saguaro_verify_cache against the oracle's verify and cache build on the same inputs."""
    say(f"[parity] fused verify+cache {label} B={w.B} K={w.K} V={w.V} budget={w.budget} sample={tokens is None}")
    sample = tokens is None
    o = run_oracle(w, tokens, round_=round_)
    bound_flagged(o.flags, f"fused {label}", allow_flags)
    prm = capi.params_tensor(w.temperature, w.top_k, w.top_p)
    tok = torch.zeros((w.B, w.K), dtype=torch.int32, device="cuda") if sample else dev(np.asarray(tokens, np.int32))
    out, cache, fan = capi.saguaro_verify_cache(dev(w.draft), dev(w.target), w.K, prm, tok, w.budget, w.a, w.r,
                                                F=w.F, C=w.C, seed=w.seed, round_=round_,
                                                flags=capi.SPEC_SAMPLE_DRAFT if sample else 0)
    torch.cuda.synchronize()
    k, t = out.k.cpu().numpy(), out.tstar.cpu().numpy()
    st, tk = out.status.cpu().numpy().astype(np.uint32), out.tokens.cpu().numpy()
    ok = o.flags == 0
    bad = np.flatnonzero(ok & ((k != o.k) | (t != o.t) | (st != o.status)))
    assert len(bad) == 0, f"{len(bad)} verify mismatches, first {bad[:5]}"
    if sample:
        good = ok & ((o.status & (oracle.ST_BAD_LOGIT | oracle.ST_BAD_PARAM)) == 0)
        assert (tk[good] == o.tokens[good]).all()
    np.testing.assert_allclose(out.resid_mass.cpu().numpy()[ok], o.W[ok], rtol=RTOL[w.dtype], atol=1e-6)
    # the cache depends only on the draft rows and the drafted tokens the call used
    ocache = oracle.cache_build(w.draft, w.dtype, w.K, tk, np.array(fan, np.int32))
    gcache = cache.cpu().numpy()
    rows = np.flatnonzero((gcache != ocache).any(axis=1))
    assert len(rows) == 0, f"cache mismatch in requests {rows[:5]}: gpu {gcache[rows[0]]} oracle {ocache[rows[0]]}"
    say(f"[parity] fused {label} ok: flagged {int((~ok).sum())} of {w.B}")
    return o


def test_fused_verify_and_cache_full_size():
    w = synth.saguaro(B=16, K=5, V=128256, cache_row=True)
    o = _check_fused(w, label="sampled")
    _check_fused(w, tokens=o.tokens, label="given")
    for seed_off in (1, 2):
        w2 = synth.saguaro(B=16, K=5, V=128256, cache_row=True)
        w2.seed += seed_off
        _check_fused(w2, label=f"seed+{seed_off}")


def test_fused_verify_and_cache_special_rows():
    rng = np.random.default_rng(11)
    B, K, V = 10, 3, 20480
    d, t = synth.random_rows(rng, B, K, V, synth.BF16, draft_rows=K + 1)
    # ties at the top of a cache row, a NaN and a +inf draft row, -inf spread, tiny values
    d[0, 1, :50] = d[0, 1].max()
    d[1, 0, 7] = synth.f32_to_bf16_bits(np.array([np.nan], np.float32))[0]
    d[2, K, 100] = synth.f32_to_bf16_bits(np.array([np.inf], np.float32))[0]
    d[3, 2, ::3] = synth.f32_to_bf16_bits(np.array([-np.inf], np.float32))[0]
    d[4, 0, :300] = synth.f32_to_bf16_bits(np.array([1e-5], np.float32))[0]
    w = _work(d, t, synth.BF16, K, rng.choice([0.0, 0.7, 1.0], B), rng.choice([0, 3, 40, 200], B),
              rng.choice([0.5, 0.95, 1.0], B), F=3, C=0.5)
    w.budget, w.a, w.r = 24, 0.6, 1.0
    _check_fused(w, tokens=rng.integers(0, V, (B, K)), label="special rows")
    _check_fused(w, label="special rows sampled")


def test_tree_chains_and_branch_reuse():
    w = synth.tree(n_req=4)
    say(f"[parity] tree chains B={w.B} gamma={w.K} V={w.V} top-k 50")
    o, _ = check_verify(w, tokens=w.tokens, label="tree")
    shape = [w.kappa, w.gamma]
    n_req = w.B // w.kappa
    br = dev(w.tokens)
    slot, hit, batch = capi.saguaro_cache_lookup(1, br, shape, 0, n_req, dev(o.k), dev(o.t))
    torch.cuda.synchronize()
    oslot, ohit, obatch = oracle.cache_lookup(1, w.tokens, shape, 0, n_req, o.k, o.t)
    assert (slot.cpu().numpy() == oslot).all() and (batch.cpu().numpy() == obatch).all()


# ------------------------------------------------------------------------------------------
# edge cases
# ------------------------------------------------------------------------------------------
def _work(draft, target, dtype, K, T, tk, tp, F=0, C=1.0, seed=99):
    B, _, V = target.shape
    Tv, kv, pv = (np.broadcast_to(np.asarray(x), (B,)).copy() for x in (T, tk, tp))
    draft = None if draft is None else np.ascontiguousarray(draft)
    return synth.Workload("edge", dtype, B, K, V, draft, np.ascontiguousarray(target),
                          Tv.astype(np.float32), kv.astype(np.int32), pv.astype(np.float32), F=F, C=C, seed=seed)


@pytest.mark.parametrize("dtype", [synth.FP32, synth.BF16])
@pytest.mark.parametrize("V", [1, 2, 63, 1000, 4097])
def test_shapes_and_parameter_mix(dtype, V):
    rng = np.random.default_rng(V * 7 + dtype)
    B, K = 24, 3
    d, t = synth.random_rows(rng, B, K, V, dtype)
    T = rng.choice([0.0, 0.5, 1.0, 1.7], B)
    tk = rng.choice([0, 1, 2, 5, V, V + 3], B)
    tp = rng.choice([0.01, 0.3, 0.9, 1.0, 1.5], B)
    w = _work(d, t, dtype, K, T, tk, tp, F=2, C=0.4)
    check_verify(w, label=f"mix V={V}")
    check_verify(w, tokens=rng.integers(0, V, (B, K)), label=f"mix-given V={V}")


def test_special_rows_and_bad_inputs():
    rng = np.random.default_rng(5)
    B, K, V = 12, 2, 300
    d, t = synth.random_rows(rng, B, K, V, synth.FP32)
    d[0] = -np.inf
    d[0, :, 17] = 1.0                 # one finite draft logit per row
    t[1, 1, 5] = np.nan               # NaN -> bad logit
    t[2, 0] = -np.inf                 # a target row with no finite logit
    d[3] *= 1e4                       # masses underflow to exactly 0
    t[3] *= 1e4
    d[4] = np.round(d[4])             # heavy ties
    t[4] = np.round(t[4])
    T = np.ones(B, np.float32)
    T[5] = -1.0                       # bad parameter
    tp = np.full(B, 0.9, np.float32)
    tp[6] = 0.0                       # bad parameter
    tk = np.zeros(B, np.int32)
    tk[7] = 2                         # with F = 4, C = 0: the set holds all mass -> degenerate
    w = _work(d, t, synth.FP32, K, T, tk, tp, F=4, C=0.0)
    check_verify(w, label="special-sampled")
    tok = rng.integers(0, V, (B, K)).astype(np.int32)
    tok[8, 1] = V                     # bad token
    tok[9, 0] = -1
    check_verify(w, tokens=tok, label="special-given")


def test_vocabulary_of_one():
    d = np.zeros((2, 1, 1), np.float32)
    t = np.zeros((2, 2, 1), np.float32)
    w = _work(d, t, synth.FP32, 1, [1.0, 0.0], 0, 1.0)
    o, _ = check_verify(w, label="V=1")
    assert (o.k == 1).all() and (o.t == 0).all()


# ------------------------------------------------------------------------------------------
# bf16 rows with V a multiple of 8 and given draft tokens take the register-resident path
# ------------------------------------------------------------------------------------------
def _zipf_work(rng, B, K, V, T, tk, tp, F=0, C=1.0, noise=0.8, seed=1234):
    target = synth.zipf_rows(rng, B * (K + 1), V).reshape(B, K + 1, V)
    draft = target[:, :K] + noise * rng.standard_normal((B, K, V), dtype=np.float32)
    w = _work(synth.f32_to_bf16_bits(draft), synth.f32_to_bf16_bits(target), synth.BF16, K, T, tk, tp, F=F, C=C,
              seed=seed)
    return w


def _oracle_tokens(w):
    return run_oracle(w).tokens


def test_fast_llama_given_tokens():
    w = synth.llama(B=24)
    check_verify(w, tokens=_oracle_tokens(w), label="fast-llama")


@pytest.mark.parametrize("V", [2048, 4096, 16392, 40000, 151936])
def test_fast_parameter_mix(V):
    rng = np.random.default_rng(V)
    B, K = 24, 3
    T = rng.choice([0.0, 0.6, 1.0, 1.5], B)
    tk = rng.choice([0, 1, 5, 64, 65, 200, 3000], B)
    tp = rng.choice([0.05, 0.5, 0.9, 0.99, 1.0], B)
    w = _zipf_work(rng, B, K, V, T, tk, tp, F=4, C=0.3)
    check_verify(w, tokens=_oracle_tokens(w), label=f"fast-mix V={V}")
    check_verify(w, tokens=rng.integers(0, V, (B, K)), label=f"fast-mix-random V={V}")


# The register-resident path's largest vocabulary: 16 slices of 16384 columns, whose candidate
# lists of 64 (top-k 64) fill the 1024-entry merge buffer exactly; 8 columns more and the call
# takes the general path (one workgroup per position)
@pytest.mark.parametrize("V", [262144, 262152])
def test_fast_path_vocabulary_limit(V):
    rng = np.random.default_rng(V % 1000)
    B, K = 6, 2
    T = np.array([1.0, 0.7, 1.0, 0.0, 1.3, 1.0])
    tk = np.array([64, 64, 0, 0, 65, 50])
    tp = np.array([1.0, 0.9, 0.95, 1.0, 1.0, 0.5])
    w = _zipf_work(rng, B, K, V, T, tk, tp, F=4, C=0.3)
    check_verify(w, tokens=_oracle_tokens(w), label=f"fast-limit V={V}")


def test_fast_ties_and_large_sets():
    rng = np.random.default_rng(77)
    B, K, V = 16, 2, 20000
    t = np.round(rng.normal(0, 2, (B, K + 1, V))).astype(np.float32)  # ~15 distinct values
    d = np.round(t[:, :K] + rng.normal(0, 1, (B, K, V))).astype(np.float32)
    T = rng.choice([0.5, 1.0, 2.0], B)
    tk = rng.choice([0, 30, 64, 500, 15000], B)
    tp = rng.choice([0.3, 0.8, 1.0], B)
    w = _work(synth.f32_to_bf16_bits(d), synth.f32_to_bf16_bits(t), synth.BF16, K, T, tk, tp, F=64, C=0.2)
    check_verify(w, tokens=_oracle_tokens(w), label="fast-ties")


# Rows whose values spread over most of the bf16 bins: ~1,500-2,000 distinct values per slice row,
# so a slice lists more (bin, count) entries than one batch of the settle's merge covers and more
# than the resolve kernel's first two entries per thread (the loops over the remaining entries)
@pytest.mark.parametrize("V", [40000, 131072])
def test_fast_wide_value_spread(V):
    rng = np.random.default_rng(4242 + V)
    B, K = 12, 3
    t = rng.uniform(-30, 30, (B, K + 1, V)).astype(np.float32)
    t[B // 2:] = 8 * rng.standard_normal((B - B // 2, K + 1, V), dtype=np.float32)
    d = t[:, :K] + 1.5 * rng.standard_normal((B, K, V), dtype=np.float32)
    T = rng.choice([0.6, 1.0, 3.0, 20.0], B)
    tk = rng.choice([0, 700, 5000], B)
    tp = rng.choice([0.5, 0.95, 1.0], B)
    w = _work(synth.f32_to_bf16_bits(d), synth.f32_to_bf16_bits(t), synth.BF16, K, T, tk, tp, F=4, C=0.3)
    o, _ = check_verify(w, tokens=_oracle_tokens(w), label=f"fast-wide V={V}")
    assert (o.k < K).sum() >= 3  # the residual pass runs for several requests
    check_verify(w, tokens=rng.integers(0, V, (B, K)), label=f"fast-wide-random V={V}")


def test_fast_cut_on_signed_zeros():
    # most of each row is +0 or -0, so the nucleus (and the downweighted set) end inside the
    # zero key, whose elements the owner slice orders one by one
    rng = np.random.default_rng(79)
    B, K, V = 8, 2, 40000
    t = np.where(rng.random((B, K + 1, V)) < 0.5, 0.0, -0.0).astype(np.float32)
    d = np.where(rng.random((B, K, V)) < 0.5, -0.0, 0.0).astype(np.float32)
    for arr in (t, d):
        idx = rng.integers(0, V, (arr.shape[0], arr.shape[1], 12))
        np.put_along_axis(arr, idx, 1.0, axis=2)
        idx = rng.integers(0, V, (arr.shape[0], arr.shape[1], 3000))
        np.put_along_axis(arr, idx, -1.0, axis=2)
    T = np.full(B, 1.0, np.float32)
    tk = rng.choice([0, 20000], B)
    tp = rng.choice([0.3, 0.6, 0.9], B)
    w = _work(synth.f32_to_bf16_bits(d), synth.f32_to_bf16_bits(t), synth.BF16, K, T, tk, tp, F=20, C=0.5)
    check_verify(w, tokens=_oracle_tokens(w), label="fast-zero-cut")
    check_verify(w, tokens=rng.integers(0, V, (B, K)), label="fast-zero-cut-random")


def test_fast_shifted_rows_have_empty_residual():
    # draft logits = target logits + 3 exactly: both rows process to the same distribution, so
    # every rejection (a token outside the kept set) leaves the residual exactly empty
    rng = np.random.default_rng(80)
    B, K, V = 16, 3, 20000
    t = np.clip(np.round(rng.normal(-4, 2, (B, K + 1, V))), -12, 4).astype(np.float32)
    d = (t[:, :K] + 3.0).astype(np.float32)
    T = rng.choice([0.5, 1.0], B)
    tk = rng.choice([0, 1, 50, 3000], B)
    tp = rng.choice([0.2, 0.9, 1.0], B)
    w = _work(synth.f32_to_bf16_bits(d), synth.f32_to_bf16_bits(t), synth.BF16, K, T, tk, tp)
    o, _ = check_verify(w, tokens=rng.integers(0, V, (B, K)), label="fast-shifted")
    assert (o.status & capi.ST_EMPTY_RESIDUAL).sum() > 0


def test_fast_special_values_and_fallback():
    rng = np.random.default_rng(78)
    B, K, V = 12, 2, 32768
    target = synth.zipf_rows(rng, B * (K + 1), V).reshape(B, K + 1, V)
    draft = target[:, :K] + 0.7 * rng.standard_normal((B, K, V), dtype=np.float32)
    # values outside the exact bins: tiny, zero, huge; masked tokens
    for arr in (target, draft):
        idx = rng.integers(0, V, (arr.shape[0], arr.shape[1], 20))
        vals = rng.choice([1e-3, -1e-3, 0.0, -0.0, 40.0, -40.0, 1e4, -1e4, 5e-5], idx.shape).astype(np.float32)
        np.put_along_axis(arr, idx, vals, axis=2)
        mask = rng.integers(0, V, (arr.shape[0], arr.shape[1], 50))
        np.put_along_axis(arr, mask, -np.inf, axis=2)
    target[3, 1, :400] = 2e-4   # > 64 finite specials in one slice: general path for that unit
    draft[5, 0, 100:300] = -100.0
    target[7, 2, 11] = 60.0     # a huge maximum
    T = np.full(B, 1.0, np.float32)
    tk = rng.choice([0, 3, 100], B)
    tp = rng.choice([0.9, 0.999, 1.0], B)
    w = _work(synth.f32_to_bf16_bits(draft), synth.f32_to_bf16_bits(target), synth.BF16, K, T, tk, tp, F=4, C=0.3)
    check_verify(w, tokens=_oracle_tokens(w), label="fast-specials")
    check_verify(w, tokens=rng.integers(0, V, (B, K)), label="fast-specials-random")


def test_fast_workspace_reuse_and_determinism():
    w = synth.saguaro(B=16, K=5, V=128256, cache_row=True)
    tok = dev(_oracle_tokens(w.without_cache_row()))
    prm = capi.params_tensor(w.temperature, w.top_k, w.top_p)
    ws = capi.new_workspace(w.B, w.K, w.V)
    outs = []
    for rnd in (0, 1, 0):
        o = capi.spec_verify(dev(w.draft), dev(w.target), w.K, prm, tok, F=w.F, C=w.C, seed=w.seed, round_=rnd,
                             workspace=ws)
        torch.cuda.synchronize()
        outs.append((o.k.cpu().numpy().copy(), o.tstar.cpu().numpy().copy(), o.status.cpu().numpy().copy()))
    assert all(np.array_equal(x, y) for x, y in zip(outs[0], outs[2]))
    o1 = run_oracle(w.without_cache_row(), tokens=tok.cpu().numpy(), round_=1)
    bound_flagged(o1.flags, "workspace reuse, round 1")
    ok = o1.flags == 0
    assert (outs[1][0][ok] == o1.k[ok]).all() and (outs[1][1][ok] == o1.t[ok]).all()


# ------------------------------------------------------------------------------------------
# random-token backup speculation: the draft distribution is uniform on the vocabulary
# ------------------------------------------------------------------------------------------
def check_uniform(w, tokens=None, label="", allow_flags=None):
    """Uniform-draft verification (SPEC_UNIFORM_DRAFT, no draft logits) against the oracle."""
    sample = tokens is None
    say(f"[parity] uniform {label} B={w.B} K={w.K} V={w.V} dtype={w.dtype} sample={sample}")
    o = oracle.verify(None, w.target, w.dtype, w.K, w.params(), tokens=tokens, seed=w.seed, uniform_draft=True)
    bound_flagged(o.flags, f"uniform {label}", allow_flags)
    prm = capi.params_tensor(w.temperature, w.top_k, w.top_p)
    tok = torch.zeros((w.B, w.K), dtype=torch.int32, device="cuda") if sample else dev(np.asarray(tokens, np.int32))
    flags = capi.SPEC_UNIFORM_DRAFT | (capi.SPEC_SAMPLE_DRAFT if sample else 0)
    out = capi.spec_verify(None, dev(w.target), w.K, prm, tok, seed=w.seed, flags=flags)
    torch.cuda.synchronize()
    k, t, W = out.k.cpu().numpy(), out.tstar.cpu().numpy(), out.resid_mass.cpu().numpy()
    st, gtok = out.status.cpu().numpy().astype(np.uint32), out.tokens.cpu().numpy()
    ok = o.flags == 0
    bad = np.flatnonzero(ok & ((k != o.k) | (t != o.t) | (st != o.status)))
    assert len(bad) == 0, (f"{len(bad)} mismatches, first {bad[:5]}: gpu k={k[bad[:5]]} t={t[bad[:5]]} "
                           f"st={st[bad[:5]]} | oracle k={o.k[bad[:5]]} t={o.t[bad[:5]]} st={o.status[bad[:5]]}")
    if sample:
        # the drafted tokens are uniform draws, independent of the logits: equal on every request
        assert (gtok == o.tokens).all()
    np.testing.assert_allclose(W[ok], o.W[ok], rtol=RTOL[w.dtype], atol=1e-6)
    say(f"[parity] uniform {label} ok: flagged {int((~ok).sum())} of {w.B}; mean k {k.mean():.3f}")
    return o


def test_uniform_draft_full_size():
    w = synth.saguaro(B=16, K=5, V=128256)
    o = check_uniform(w, label="saguaro-size")
    rng = np.random.default_rng(5)
    check_uniform(w, tokens=rng.integers(0, w.V, (w.B, w.K)), label="saguaro-size-given")
    # a flat target accepts almost every uniform draft token
    flat = synth.f32_to_bf16_bits(np.zeros((w.B, w.K + 1, w.V), np.float32))
    wf = _work(None, flat, synth.BF16, w.K, 1.0, 0, 1.0, seed=7)
    of = check_uniform(wf, label="flat-target")
    assert (of.k == w.K).all()
    assert o.k.mean() < of.k.mean()


@pytest.mark.parametrize("V", [2048, 16392, 151936])
def test_uniform_draft_fast_parameter_mix(V):
    rng = np.random.default_rng(V + 1)
    B, K = 24, 3
    T = rng.choice([0.0, 0.6, 1.0, 1.5], B)
    tk = rng.choice([0, 1, 5, 64, 200, 3000], B)
    tp = rng.choice([0.05, 0.5, 0.9, 1.0], B)
    target = synth.zipf_rows(rng, B * (K + 1), V, slope=0.6).reshape(B, K + 1, V)
    w = _work(None, synth.f32_to_bf16_bits(target), synth.BF16, K, T, tk, tp, seed=31)
    check_uniform(w, label=f"fast-mix V={V}")
    check_uniform(w, tokens=rng.integers(0, V, (B, K)), label=f"fast-mix-given V={V}")


@pytest.mark.parametrize("dtype", [synth.FP32, synth.BF16])
@pytest.mark.parametrize("V", [1, 2, 63, 1000, 4097])
def test_uniform_draft_generic_shapes(dtype, V):
    rng = np.random.default_rng(V * 3 + dtype)
    B, K = 40, 4
    t = rng.normal(0, 1.5, (B, K + 1, V)).astype(np.float32)
    if dtype == synth.BF16:
        t = synth.f32_to_bf16_bits(t)
    T = rng.choice([0.0, 0.5, 1.0, 2.0], B)
    tk = rng.choice([0, 1, 3, 50], B)
    tp = rng.choice([0.2, 0.9, 1.0], B)
    w = _work(None, t, dtype, K, T, tk, tp, seed=3)
    check_uniform(w, label=f"generic V={V}")
    check_uniform(w, tokens=rng.integers(0, V, (B, K)), label=f"generic-given V={V}")


def test_backup_plan():
    rng = np.random.default_rng(11)
    for B in (1, 7, 64, 1000):
        for p_hit in (0.0, 0.5, 0.97, 1.0):
            hit = (rng.random(B) < p_hit).astype(np.uint8)
            batch = np.array([hit.sum(), int(hit.all())], np.int32)
            for b_star in (1, 8, 64, 5000):
                use, sw = capi.saguaro_backup_plan(dev(hit), dev(batch), b_star)
                o_use, o_sw = oracle.backup_plan(B, hit, int(batch[1]), b_star)
                assert int(sw.cpu()[0]) == o_sw, (B, p_hit, b_star)
                assert (use.cpu().numpy() == o_use).all(), (B, p_hit, b_star)
    say("[parity] backup plan ok")


# ------------------------------------------------------------------------------------------
# long drafts (more than 8 positions: the per-unit request rendezvous instead of the packed
# 64-bit one) and large batches on the bf16 path
# ------------------------------------------------------------------------------------------
@pytest.mark.parametrize("K", [8, 12, 25])
def test_fast_long_drafts(K):
    rng = np.random.default_rng(100 + K)
    B, V = 12, 16392
    T = rng.choice([0.0, 0.7, 1.0], B)
    tk = rng.choice([0, 20, 500], B)
    tp = rng.choice([0.8, 0.95, 1.0], B)
    w = _zipf_work(rng, B, K, V, T, tk, tp, F=3, C=0.5, noise=0.3)
    o, _ = check_verify(w, tokens=_oracle_tokens(w), label=f"fast-long K={K}")
    assert o.k.max() > 7 or K == 8
    check_verify(w, tokens=rng.integers(0, V, (B, K)), label=f"fast-long-random K={K}")


def test_fast_large_batch():
    rng = np.random.default_rng(300)
    B, K, V = 600, 3, 2048
    T = rng.choice([0.0, 0.5, 1.0], B)
    tk = rng.choice([0, 1, 8, 100], B)
    tp = rng.choice([0.5, 0.9, 1.0], B)
    w = _zipf_work(rng, B, K, V, T, tk, tp, F=2, C=0.2)
    check_verify(w, tokens=_oracle_tokens(w), label="fast-large-batch")


@pytest.mark.parametrize("K", [63, 64, 100])
def test_drafts_at_the_wave_limit(K):
    """K + 1 = 64 positions is the bf16 count path's limit (one request decision wave); K = 64 and
    K = 100 take the general path.  Request 0 accepts every position (draft rows equal the target
    rows), request 1 is rejected at position K - 3 (the drafted token's target logit is -inf
    there, its draft logit finite: past position 63 for K = 100), request 2 has a NaN in its
    bonus row K, request 3 a +inf in its bonus row."""
    rng = np.random.default_rng(700 + K)
    B, V = 4, 2048
    zt = synth.f32_to_bf16_bits(rng.normal(0, 2.0, (B, K + 1, V)).astype(np.float32))
    zd = zt[:, :K].copy()
    tok = rng.integers(0, V, (B, K)).astype(np.int32)
    jr = K - 3
    zt[1, jr, tok[1, jr]] = 0xFF80  # -inf in the target only: q(s) = 0 < p(s)
    zt[2, K, 5] = 0x7FC0            # NaN
    zt[3, K, 9] = 0x7F80            # +inf
    w = _work(zd, zt, synth.BF16, K, 1.0, 0, 1.0)
    o, _ = check_verify(w, tokens=tok, label=f"wave-limit K={K}")
    assert o.k[0] == K and o.k[1] == jr
    assert o.status[2] == oracle.ST_BAD_LOGIT and o.status[3] == oracle.ST_BAD_LOGIT


def test_fused_given_tokens_twenty_rounds():
    """The benchmark's call at full size (B = 16, K = 5, V = 128256 with the cache row, given
    drafted tokens) over the twenty rounds the benchmark times: every round draws its own
    uniforms from the Philox counter."""
    w = synth.saguaro(B=16, K=5, V=128256, cache_row=True)
    tok = _oracle_tokens(w.without_cache_row())
    for rnd in range(20):
        _check_fused(w, tokens=tok, label=f"given round {rnd}", round_=rnd)


def test_tree_chains_full_size():
    """Config 5 at full size: 64 requests x 8 branches = 512 chains, gamma = 7, V = 151936, top-k 50."""
    w = synth.tree(n_req=64)
    o, _ = check_verify(w, tokens=w.tokens, label="tree-full")
    shape = [w.kappa, w.gamma]
    n_req = w.B // w.kappa
    slot, hit, batch = capi.saguaro_cache_lookup(1, dev(w.tokens), shape, 0, n_req, dev(o.k), dev(o.t))
    torch.cuda.synchronize()
    oslot, ohit, obatch = oracle.cache_lookup(1, w.tokens, shape, 0, n_req, o.k, o.t)
    assert (slot.cpu().numpy() == oslot).all() and (batch.cpu().numpy() == obatch).all()


def test_llama_two_hundred_rounds_given_tokens():
    """Config 2 (B = 1, K = 5, V = 128256, top-p 0.8): 200 rounds batched as 200 requests, then
    twenty single-request calls that step the round counter."""
    w = synth.llama(B=200)
    tok = _oracle_tokens(w)
    check_verify(w, tokens=tok, label="llama-200")
    for rnd in range(20):
        b = rnd * 7
        one = _work(w.draft[b:b + 1], w.target[b:b + 1], w.dtype, w.K, w.temperature[b], w.top_k[b], w.top_p[b],
                    seed=w.seed)
        check_verify(one, tokens=tok[b:b + 1], round_=rnd, label=f"llama round {rnd}")


def test_placement_status_stays_clear():
    """The bf16 path's rendezvous assume that every workgroup of a unit (count kernel) and of a
    request (resolve kernel) runs on one XCD; a unit or request that saw more than one XCD
    reports SPEC_ST_PLACEMENT.  The bit stays clear at the headline size (fused call, ten
    rounds) and at the branch-tree size (512 chains, five rounds)."""
    rng = np.random.default_rng(7)
    w = synth.saguaro(B=16, K=5, V=128256, cache_row=True)
    prm = capi.params_tensor(w.temperature, w.top_k, w.top_p)
    tok = dev(rng.integers(0, w.V, size=(w.B, w.K)).astype(np.int32))
    d, t = dev(w.draft), dev(w.target)
    for rnd in range(10):
        out, _, _ = capi.saguaro_verify_cache(d, t, w.K, prm, tok, w.budget, w.a, w.r, F=w.F, C=w.C, seed=w.seed,
                                              round_=rnd)
        st = out.status.cpu().numpy().astype(np.uint32)
        assert ((st & capi.ST_PLACEMENT) == 0).all(), f"placement status in round {rnd}: {st}"
    tw = synth.tree(n_req=64)
    tprm = capi.params_tensor(tw.temperature, tw.top_k, tw.top_p)
    dd, tt, tk = dev(tw.draft), dev(tw.target), dev(tw.tokens.astype(np.int32))
    for rnd in range(5):
        out = capi.spec_verify(dd, tt, tw.K, tprm, tk, F=tw.F, C=tw.C, seed=tw.seed, round_=rnd)
        st = out.status.cpu().numpy().astype(np.uint32)
        assert ((st & capi.ST_PLACEMENT) == 0).all(), f"placement status in tree round {rnd}"
    say("[placement] clear: 10 headline rounds, 5 branch-tree rounds")


def _fused_lookup_case(w, tok, rnd, C=None):
    """saguaro_verify_cache_lookup against saguaro_verify_cache + saguaro_cache_lookup (mode 0)."""
    C = w.C if C is None else C
    d, t = dev(w.draft), dev(w.target)
    prm = capi.params_tensor(w.temperature, w.top_k, w.top_p)
    ref, ref_cache, fan = capi.saguaro_verify_cache(d, t, w.K, prm, tok, w.budget, w.a, w.r, F=w.F, C=C, seed=w.seed,
                                                    round_=rnd)
    rslot, rhit, rbatch = capi.saguaro_cache_lookup(0, ref_cache.contiguous(), fan, w.K, w.B, ref.k, ref.tstar)
    out, cache, fan2, slot, hit, batch = capi.saguaro_verify_cache_lookup(d, t, w.K, prm, tok, w.budget, w.a, w.r,
                                                                          F=w.F, C=C, seed=w.seed, round_=rnd)
    torch.cuda.synchronize()
    assert fan2 == fan
    for name in ("k", "tstar", "status"):
        assert torch.equal(getattr(out, name), getattr(ref, name)), name
    assert torch.equal(out.resid_mass, ref.resid_mass)
    assert torch.equal(cache, ref_cache)
    assert torch.equal(slot, rslot) and torch.equal(hit, rhit) and torch.equal(batch, rbatch), \
        f"lookup differs: {slot.cpu().numpy()} vs {rslot.cpu().numpy()}, batch {batch.cpu().numpy()} {rbatch.cpu().numpy()}"
    return out, cache, fan, slot, hit, batch


def test_fused_lookup_matches_the_two_calls():
    """The lookup fused into the verification call equals the separate lookup: the headline shape over
    six rounds at C = 0.3 and C = 1, a small bf16 shape, a shape whose drafts outnumber the residual's
    workgroups (two-call path inside) and the general path; one round also against the oracle."""
    rng = np.random.default_rng(11)
    w = synth.saguaro(B=16, K=5, V=128256, cache_row=True)
    tok = dev(rng.integers(0, w.V, size=(w.B, w.K)).astype(np.int32))
    tok[:, 0] = dev(synth.bf16_bits_to_f32(w.draft[:, 0]).argmax(axis=1).astype(np.int32))  # often accepted
    for rnd in range(6):
        out, cache, fan, slot, hit, batch = _fused_lookup_case(w, tok, rnd, C=(w.C if rnd % 2 == 0 else 1.0))
    oslot, ohit, obatch = oracle.cache_lookup(0, cache.cpu().numpy(), np.array(fan, np.int32), w.K, w.B,
                                              out.k.cpu().numpy(), out.tstar.cpu().numpy())
    assert (slot.cpu().numpy() == oslot).all() and (batch.cpu().numpy() == obatch).all()
    for shape in ((4, 3, 16392), (3, 7, 16392), (3, 2, 4099)):
        B, K, V = shape
        w2 = synth.saguaro(B=B, K=K, V=V, cache_row=True)
        tok2 = dev(rng.integers(0, V, size=(B, K)).astype(np.int32))
        _fused_lookup_case(w2, tok2, 2)
    say("[fused lookup] equal to the two calls on every case")
