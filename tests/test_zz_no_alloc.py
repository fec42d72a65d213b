"""saguaro_verify_cache_noalloc (the library's static scratch, no workspace) against
saguaro_verify_cache (a caller workspace) through the C-ABI, on the same inputs: calls in a row
on one GPU, each smaller than the one before (the scratch keeps the previous call's contents),
and a shape too large for the scratch."""
import numpy as np
import pytest
import torch

from lossless_speculative_sampling_amd import capi, synth

pytestmark = pytest.mark.gpu


def dev(a):
    a = np.ascontiguousarray(a)
    return torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).cuda()


def _compare(w, rnd):
    """Both entry points on workload w (drafted tokens sampled once from the draft rows)."""
    d, t = dev(w.draft), dev(w.target)
    prm = capi.params_tensor(w.temperature, w.top_k, w.top_p)
    tok = torch.zeros((w.B, w.K), dtype=torch.int32, device="cuda")
    capi.spec_verify(d, t, w.K, prm, tok, F=w.F, C=w.C, seed=w.seed, flags=capi.SPEC_SAMPLE_DRAFT)
    ref, ref_cache, ref_fan = capi.saguaro_verify_cache(d, t, w.K, prm, tok, w.budget, w.a, w.r, F=w.F, C=w.C,
                                                        seed=w.seed, round_=rnd)
    out = capi.VerifyOut(torch.full((w.B,), -7, dtype=torch.int32, device="cuda"),
                         torch.full((w.B,), -7, dtype=torch.int32, device="cuda"),
                         torch.full((w.B,), -7.0, dtype=torch.float32, device="cuda"),
                         torch.full((w.B,), -7, dtype=torch.int32, device="cuda"), tok)
    cache = torch.full((w.B, w.budget), -7, dtype=torch.int32, device="cuda")
    fan = capi.saguaro_verify_cache_noalloc(d, t, w.K, prm, tok, w.budget, w.a, w.r, out, cache, F=w.F, C=w.C,
                                            seed=w.seed, round_=rnd)
    torch.cuda.synchronize()
    assert fan == ref_fan
    for name in ("k", "tstar", "status"):
        a, b = getattr(out, name).cpu().numpy(), getattr(ref, name).cpu().numpy()
        assert (a == b).all(), f"{name} differs: {a} vs {b}"
    np.testing.assert_allclose(out.resid_mass.cpu().numpy(), ref.resid_mass.cpu().numpy(), rtol=1e-6, atol=1e-7)
    assert torch.equal(cache, ref_cache), "cache differs"
    print(f"[noalloc] B={w.B} K={w.K} V={w.V} round {rnd}: equal (k {out.k.cpu().numpy().tolist()})", flush=True)


def test_noalloc_matches_the_workspace_call():
    # the headline shape, then two smaller shapes (bf16 path, then the general path: V % 8 != 0)
    _compare(synth.saguaro(B=16, K=5, V=128256, cache_row=True), 3)
    _compare(synth.saguaro(B=4, K=3, V=16392, cache_row=True), 4)
    _compare(synth.saguaro(B=3, K=2, V=4099, cache_row=True), 5)


def test_noalloc_rejects_shapes_beyond_the_scratch():
    big_B = 32  # 32 requests at K = 5, V = 128256 need 37 MiB
    assert capi.spec_workspace_bytes(big_B, 5, 128256) > capi.SPEC_NOALLOC_SCRATCH_BYTES
    L = capi.load().cdll
    x = torch.zeros(16, dtype=torch.int32, device="cuda")
    p = x.data_ptr()
    rc = L.saguaro_verify_cache_noalloc(p, p, capi.SPEC_BF16, big_B, 5, 128256, p, 0, 1.0, p, 0, 0, 0, 32, 0.7, 1.0,
                                        None, p, p, None, None, p, None)
    assert rc == capi.SPEC_EWORKSPACE
