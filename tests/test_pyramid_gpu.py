"""PyramidSD fuzzy acceptance (pyramid_verify): GPU <-> oracle parity through the C ABI.

Integers (k, t*, status, sampled tokens) are equal on every request the oracle does not flag
(near acceptance, CDF, nucleus or fuzzy-threshold ties); the residual mass within 1e-5 (fp32)
/ 2e-3 (bf16) relative; the divergences within 1e-6 absolute (fp64 sums stored as fp32).
"""
import numpy as np
import pytest
import torch

import oracle
from flagbound import bound_flagged
from lossless_speculative_sampling_amd import capi, synth

pytestmark = pytest.mark.gpu

RTOL = {synth.FP32: 1e-5, synth.BF16: 2e-3}
BAD = oracle.ST_BAD_LOGIT | oracle.ST_BAD_PARAM | oracle.ST_BAD_TOKEN


def say(msg):
    print(msg, flush=True)


def dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


def check_pyramid(draft, verifier, dtype, K, prm, tau, tokens=None, F=0, C=1.0, seed=5, assisted=False,
                  uniform=False, label="", allow_flags=None):
    B, _, V = verifier.shape
    sample = tokens is None
    say(f"[pyramid] {label} B={B} K={K} V={V} dtype={dtype} sample={sample} assisted={assisted}")
    o = oracle.verify(None if uniform else draft, verifier, dtype, K, prm, F=F, C=float(np.float32(C)),
                      tokens=tokens, seed=seed, uniform_draft=uniform, tau=np.asarray(tau, np.float64),
                      assisted=assisted)
    bound_flagged(o.flags, f"pyramid {label}", allow_flags)
    flags = (capi.SPEC_SAMPLE_DRAFT if sample else 0) | (capi.SPEC_ASSISTED if assisted else 0) | \
        (capi.SPEC_UNIFORM_DRAFT if uniform else 0)
    tok = torch.zeros((B, K), dtype=torch.int32, device="cuda") if sample else dev(np.asarray(tokens, np.int32))
    prm_t = capi.params_tensor(prm["t"], prm["k"], prm["p"])
    out, div = capi.pyramid_verify(None if uniform else dev(draft), dev(verifier), K, prm_t,
                                   dev(np.asarray(tau, np.float32)), tok, F=F, C=C, seed=seed, flags=flags,
                                   want_div=True)
    torch.cuda.synchronize()
    k, t, W = out.k.cpu().numpy(), out.tstar.cpu().numpy(), out.resid_mass.cpu().numpy()
    st, gtok, gdiv = out.status.cpu().numpy().astype(np.uint32), out.tokens.cpu().numpy(), div.cpu().numpy()
    ok = o.flags == 0
    bad = np.flatnonzero(ok & ((k != o.k) | (t != o.t) | (st != o.status)))
    assert len(bad) == 0, (f"{len(bad)} mismatches, first {bad[:5]}: gpu k={k[bad[:5]]} t={t[bad[:5]]} "
                           f"st={st[bad[:5]]} | oracle k={o.k[bad[:5]]} t={o.t[bad[:5]]} st={o.status[bad[:5]]}")
    valid = ok & ((o.status & BAD) == 0)
    if sample:
        assert (gtok[valid] == o.tokens[valid]).all()
    np.testing.assert_allclose(W[ok], o.W[ok], rtol=RTOL[dtype], atol=1e-6)
    np.testing.assert_allclose(gdiv[valid], o.div[valid], rtol=0, atol=1e-6)
    say(f"[pyramid] {label} ok: flagged {int((~ok).sum())} of {B}; mean k {k.mean():.3f}; "
        f"mean div {o.div[valid].mean() if valid.any() else 0:.3f}")
    return o


@pytest.mark.parametrize("dtype", [synth.FP32, synth.BF16])
@pytest.mark.parametrize("V", [1, 2, 63, 1000, 4097])
def test_pyramid_shapes_and_parameter_mix(dtype, V):
    rng = np.random.default_rng(V * 11 + dtype)
    B, K = 24, 3
    zt = rng.normal(0, 1.5, (B, K + 1, V)).astype(np.float32)
    zd = (0.7 * zt[:, :K] + rng.normal(0, 1.0, (B, K, V))).astype(np.float32)
    if dtype == synth.BF16:
        zt, zd = synth.f32_to_bf16_bits(zt), synth.f32_to_bf16_bits(zd)
    T = rng.choice([0.0, 0.6, 1.0, 1.5], B).astype(np.float32)
    tk = rng.choice([0, 1, 5, 50], B).astype(np.int32)
    tp = rng.choice([0.3, 0.9, 1.0], B).astype(np.float32)
    prm = oracle.params_array(T, tk, tp)
    tau = rng.choice([-1.0, 0.05, 0.2, 0.5, 1.0], B).astype(np.float32)
    # tau = 1 meets rows whose processed supports are disjoint (top-k 1, greedy): their divergence
    # is exactly 1, on the threshold, and the oracle flags them (up to 4 of these 24 requests)
    for assisted in (False, True):
        check_pyramid(zd, zt, dtype, K, prm, tau, F=2, C=0.4, assisted=assisted, label=f"mix V={V}", allow_flags=4)
        check_pyramid(zd, zt, dtype, K, prm, tau, tokens=rng.integers(0, V, (B, K)), F=2, C=0.4,
                      assisted=assisted, label=f"mix-given V={V}", allow_flags=4)
    check_pyramid(None, zt, dtype, K, prm, tau, uniform=True, label=f"uniform V={V}")


def test_pyramid_two_stages_full_size():
    s1, s2 = synth.pyramid()
    prm = oracle.params_array(1.0, 0, 1.0, B=s1.B)
    o1 = check_pyramid(s1.draft, s1.verifier, synth.BF16, s1.K, prm, s1.tau, seed=s1.seed, label=s1.name)
    o2 = check_pyramid(s2.draft, s2.verifier, synth.BF16, s2.K, prm, s2.tau, seed=s2.seed, label=s2.name)
    check_pyramid(s2.draft, s2.verifier, synth.BF16, s2.K, prm, s2.tau, tokens=o2.tokens, seed=s2.seed,
                  assisted=True, label=s2.name + " assisted")
    # both branches of the rule occur, and a threshold never shortens the accepted run
    for o, s in ((o1, s1), (o2, s2)):
        assert (o.div <= s.tau[:, None]).any() and (o.div > s.tau[:, None]).any()
    o2l = oracle.verify(s2.draft, s2.verifier, synth.BF16, s2.K, prm, tokens=o2.tokens, seed=s2.seed)
    assert (o2.k >= o2l.k).all()


def test_pyramid_negative_threshold_is_spec_verify():
    rng = np.random.default_rng(4)
    B, K, V = 16, 4, 3000
    zt = rng.normal(0, 2, (B, K + 1, V)).astype(np.float32)
    zd = (zt[:, :K] + rng.normal(0, 1, (B, K, V))).astype(np.float32)
    prm = oracle.params_array(0.8, 0, 0.95, B=B)
    tok = rng.integers(0, V, (B, K)).astype(np.int32)
    prm_t = capi.params_tensor(prm["t"], prm["k"], prm["p"])
    a, _ = capi.pyramid_verify(dev(zd), dev(zt), K, prm_t, dev(np.full(B, -1.0, np.float32)), dev(tok), seed=9)
    b = capi.spec_verify(dev(zd), dev(zt), K, prm_t, dev(tok), seed=9)
    torch.cuda.synchronize()
    for x, y in zip((a.k, a.tstar, a.status), (b.k, b.tstar, b.status)):
        assert torch.equal(x, y)


# bf16 rows (V a multiple of 8, at least 2048) with given tokens take the register-resident
# path: the count kernel defers the decision, a divergence pass sums every position's
# divergence from the exact per-element values, and the resolve kernel draws the residual
@pytest.mark.parametrize("V", [2048, 16392, 128256])
def test_pyramid_fast_path(V):
    rng = np.random.default_rng(V + 5)
    B, K = 16, 6
    zt = synth.zipf_rows(rng, B * (K + 1), V).reshape(B, K + 1, V)
    s = rng.uniform(0.3, 2.0, size=(B, K, 1)).astype(np.float32)
    zd = (0.8 * zt[:, :K] + s * rng.standard_normal((B, K, V), dtype=np.float32)).astype(np.float32)
    zt, zd = synth.f32_to_bf16_bits(zt), synth.f32_to_bf16_bits(zd)
    T = rng.choice([0.0, 0.6, 1.0, 1.3], B).astype(np.float32)
    tk = rng.choice([0, 1, 20, 3000], B).astype(np.int32)
    tp = rng.choice([0.5, 0.95, 1.0], B).astype(np.float32)
    prm = oracle.params_array(T, tk, tp)
    probe = oracle.verify(zd, zt, synth.BF16, K, prm, F=2, C=0.4, seed=5, tau=np.full(B, -1.0))
    tau = np.median(probe.div, axis=1).astype(np.float32)     # about half the positions pass
    tau[::5] = -1.0
    tau[1::7] = 1.0
    tau[(T == 0.0) | (tk == 1)] = 0.5                          # one-hot rows diverge by exactly 0 or 1
    for tokens, label in ((probe.tokens, "drafted"), (rng.integers(0, V, (B, K)), "random")):
        check_pyramid(zd, zt, synth.BF16, K, prm, tau, tokens=tokens, F=2, C=0.4, label=f"fast {label} V={V}")
    check_pyramid(None, zt, synth.BF16, K, prm, tau, tokens=rng.integers(0, V, (B, K)), uniform=True,
                  label=f"fast uniform V={V}")


# Logits near zero (|z| < 2^-6) or of magnitude 32 and more fall outside the exact bins: the
# divergence pass lists them for the whole workgroup, or, past the list's capacity (1024
# elements per slice), takes the slice element by element.  Scales from 0.002 (every element
# outside) to 12 (the far tails outside); the second slice of V = 16392 holds 8 columns.
def test_pyramid_fast_path_outside_bins():
    rng = np.random.default_rng(77)
    B, K, V = 8, 4, 16392
    scale = np.array([0.002, 0.02, 0.3, 1.0, 2.0, 12.0, 0.05, 0.6], np.float32)[:, None, None]
    zt = scale * rng.standard_normal((B, K + 1, V), dtype=np.float32)
    zd = 0.8 * zt[:, :K] + 0.5 * scale * rng.standard_normal((B, K, V), dtype=np.float32)
    zt, zd = synth.f32_to_bf16_bits(zt.astype(np.float32)), synth.f32_to_bf16_bits(zd.astype(np.float32))
    prm = oracle.params_array(np.full(B, 1.0, np.float32), np.array([0, 0, 50, 0, 5000, 0, 0, 3], np.int32),
                              np.array([1.0, 0.9, 1.0, 1.0, 0.95, 1.0, 0.9, 1.0], np.float32))
    probe = oracle.verify(zd, zt, synth.BF16, K, prm, seed=5, tau=np.full(B, -1.0))
    tau = np.median(probe.div, axis=1).astype(np.float32)
    # the threshold is each request's own median divergence: the flattest rows (scale 0.002) diverge
    # by ~2e-7 with gaps of ~1e-9, and the top-3 row repeats a divergence, so up to two requests sit
    # within the oracle's 1e-9 band of their threshold
    o = check_pyramid(zd, zt, synth.BF16, K, prm, tau, tokens=probe.tokens, label="fast outside bins", allow_flags=2)
    assert (o.div <= tau[:, None]).any() and (o.div > tau[:, None]).any()


# Long drafts on the bf16 path: 40 drafted positions (one divergence arrival per position, the
# request's arrival counting to K), mixed thresholds, drafted and random tokens
def test_pyramid_fast_path_long_draft():
    rng = np.random.default_rng(40)
    B, K, V = 3, 40, 16392
    zt = synth.zipf_rows(rng, B * (K + 1), V).reshape(B, K + 1, V)
    zd = (0.8 * zt[:, :K] + rng.uniform(0.3, 1.5, (B, K, 1)).astype(np.float32)
          * rng.standard_normal((B, K, V), dtype=np.float32)).astype(np.float32)
    zt, zd = synth.f32_to_bf16_bits(zt), synth.f32_to_bf16_bits(zd)
    prm = oracle.params_array(np.array([1.0, 0.7, 1.2], np.float32), np.array([0, 100, 0], np.int32),
                              np.array([1.0, 1.0, 0.9], np.float32))
    probe = oracle.verify(zd, zt, synth.BF16, K, prm, seed=5, tau=np.full(B, -1.0))
    tau = np.quantile(probe.div, 0.8, axis=1).astype(np.float32)  # most positions pass
    for tokens, label in ((probe.tokens, "drafted"), (rng.integers(0, V, (B, K)), "random")):
        check_pyramid(zd, zt, synth.BF16, K, prm, tau, tokens=tokens, label=f"fast long {label}")


# The bf16 fuzzy path's longest draft (K = 63: the request's positions in one wave) and one
# past it (K = 64, general path)
@pytest.mark.parametrize("K", [63, 64])
def test_pyramid_draft_length_limit(K):
    rng = np.random.default_rng(K)
    B, V = 2, 2048
    zt = synth.zipf_rows(rng, B * (K + 1), V).reshape(B, K + 1, V)
    zd = (0.8 * zt[:, :K] + 0.6 * rng.standard_normal((B, K, V), dtype=np.float32)).astype(np.float32)
    zt, zd = synth.f32_to_bf16_bits(zt), synth.f32_to_bf16_bits(zd)
    prm = oracle.params_array(np.array([1.0, 0.8], np.float32), np.array([0, 40], np.int32),
                              np.array([1.0, 0.95], np.float32))
    probe = oracle.verify(zd, zt, synth.BF16, K, prm, seed=5, tau=np.full(B, -1.0))
    tau = np.quantile(probe.div, 0.9, axis=1).astype(np.float32)
    check_pyramid(zd, zt, synth.BF16, K, prm, tau, tokens=probe.tokens, label=f"draft limit K={K}")


def test_pyramid_fast_path_full_size_stages():
    s1, s2 = synth.pyramid()
    prm = oracle.params_array(1.0, 0, 1.0, B=s1.B)
    for s in (s1, s2):
        drafted = oracle.verify(s.draft, s.verifier, synth.BF16, s.K, prm, seed=s.seed, tau=s.tau).tokens
        o = check_pyramid(s.draft, s.verifier, synth.BF16, s.K, prm, s.tau, tokens=drafted, seed=s.seed,
                          label=s.name + " given tokens")
        assert (o.div <= s.tau[:, None]).any() and (o.div > s.tau[:, None]).any()
