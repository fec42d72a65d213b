"""Streams and HIP graphs through the C ABI (needs an MI355X).

The entry points take the caller's stream, allocate nothing and leave their workspace's arrival
counters at zero (each is reset by its last arriver; no memset is issued), so they
run on non-default streams, concurrently on two streams with two workspaces, and inside
captured HIP graphs.  Every result here must equal the eager default-stream result bit for bit.
"""
import numpy as np
import pytest
import torch

from lossless_speculative_sampling_amd import capi, synth

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)


def dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


def _fused_inputs(B=8, V=40000):
    w = synth.saguaro(B=B, K=5, V=V)
    prm = capi.params_tensor(w.temperature, w.top_k, w.top_p)
    d, t = dev(w.draft), dev(w.target)
    tok = torch.zeros((w.B, w.K), dtype=torch.int32, device="cuda")
    capi.spec_verify(d[:, :w.K].contiguous(), t, w.K, prm, tok, F=w.F, C=w.C, seed=w.seed,
                     flags=capi.SPEC_SAMPLE_DRAFT)
    torch.cuda.synchronize()
    return w, prm, d, t, tok


def _fused(w, prm, d, t, tok, round_, ws, out, cache):
    o, c, fan = capi.saguaro_verify_cache(d, t, w.K, prm, tok, w.budget, w.a, w.r, F=w.F, C=w.C, seed=w.seed,
                                          round_=round_, workspace=ws, out=out, cache=cache)
    slot, hit, batch = capi.saguaro_cache_lookup(0, c, fan, w.K, w.B, o.k, o.tstar)
    return o, c, slot, hit, batch


def _snap(o, c, slot, hit, batch):
    return [x.clone() for x in (o.k, o.tstar, o.resid_mass, o.status, c, slot, hit, batch)]


def _new_out(w):
    return (capi.VerifyOut(*(torch.empty(w.B, dtype=dt, device="cuda")
                             for dt in (torch.int32, torch.int32, torch.float32, torch.int32)), None),
            torch.empty((w.B, w.budget), dtype=torch.int32, device="cuda"))


def test_side_streams_and_concurrent_calls():
    w, prm, d, t, tok = _fused_inputs()
    ref = {}
    for r in (3, 4):
        ws = capi.new_workspace(w.B, w.K, w.V)
        o, c = _new_out(w)
        ref[r] = _snap(*_fused(w, prm, d, t, tok, r, ws, o, c))
    torch.cuda.synchronize()
    say("[streams] eager references done")
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    got = {}
    wss = {3: capi.new_workspace(w.B, w.K, w.V), 4: capi.new_workspace(w.B, w.K, w.V)}
    torch.cuda.synchronize()
    for rep in range(3):
        for r, s in ((3, s1), (4, s2)):
            with torch.cuda.stream(s):
                o, c = _new_out(w)
                got[r] = _fused(w, prm, d, t, tok, r, wss[r], o, c)
        torch.cuda.synchronize()
        # (equal results on every repetition also show that each call left its workspace's
        # arrival counters at zero for the next one)
        for r in (3, 4):
            for x, y in zip(_snap(*got[r]), ref[r]):
                assert torch.equal(x, y), (rep, r)
    say("[streams] two streams, three repetitions ok")


def test_graph_replays_of_the_fused_call():
    w, prm, d, t, tok = _fused_inputs()
    ws_eager = capi.new_workspace(w.B, w.K, w.V)
    refs = {}
    for r in (7, 8):
        o, c = _new_out(w)
        refs[r] = _snap(*_fused(w, prm, d, t, tok, r, ws_eager, o, c))
    torch.cuda.synchronize()
    ws = capi.new_workspace(w.B, w.K, w.V)
    o, c = _new_out(w)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _fused(w, prm, d, t, tok, 7, ws, o, c)           # warm-up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        res = _fused(w, prm, d, t, tok, 7, ws, o, c)
    torch.cuda.synchronize()
    for rep in range(4):
        g.replay()
        torch.cuda.synchronize()
        for x, y in zip(_snap(*res), refs[7]):
            assert torch.equal(x, y), rep
        # eager work between the replays, on the same workspace
        o2, c2 = _new_out(w)
        for x, y in zip(_snap(*_fused(w, prm, d, t, tok, 8, ws, o2, c2)), refs[8]):
            assert torch.equal(x, y), rep
        torch.cuda.synchronize()
    say("[graphs] fused call: four replays equal the eager call")


def test_graph_replays_of_signposts_and_tree_lookup():
    m = synth.mirror(B=16, V=50000)
    logits = dev(m.logits)
    ws = capi.new_signpost_workspace(m.B, m.V, m.kappa)
    tree = [dev(x) for x in (m.tokens, m.parents, m.path, m.k, m.tstar)]
    ref_sp = [x.clone() for x in capi.mirror_signposts(logits, m.kappa, want_bf16=True)]
    ref_tr = [x.clone() for x in capi.mirror_tree_lookup(*tree)]
    torch.cuda.synchronize()
    out = tuple(torch.empty_like(x) for x in ref_sp)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        capi.mirror_signposts(logits, m.kappa, workspace=ws, out=out)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        capi.mirror_signposts(logits, m.kappa, workspace=ws, out=out)
        tr = capi.mirror_tree_lookup(*tree)
    torch.cuda.synchronize()
    for rep in range(4):
        for x in out:
            x.zero_()
        g.replay()
        torch.cuda.synchronize()
        for x, y in zip(out, ref_sp):
            assert torch.equal(x, y), rep
        for x, y in zip(tr, ref_tr):
            assert torch.equal(x, y), rep
        capi.mirror_signposts(logits, m.kappa, workspace=ws)   # eager use of the same workspace
        torch.cuda.synchronize()
    say("[graphs] signposts + tree lookup: four replays equal the eager calls")
