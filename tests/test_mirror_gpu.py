"""Mirror-SD signposts and draft-tree reuse: GPU <-> oracle parity through the C ABI.

Signpost ids are equal on every row (integer work on exact order keys).  log p~ agrees within
2e-5 + 1e-5 |log p~| (the GPU sums fp32 exponentials in fp64; the oracle is fp64 throughout);
its bf16 form is the round-to-nearest-even of the fp32 value, within 2e-5 + 4e-3 |log p~| of
the oracle's value.
Tree reuse (node, hit, batch) is equal everywhere.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from lossless_speculative_sampling_amd import capi, synth

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def say(msg):
    print(msg, flush=True)


def dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


def _bf16_of(x):
    u = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    r[nan] = 0x7FC0
    return r


def check_signposts(logits, dtype, kappa, label="", gpu_logits=None):
    B, V = logits.shape
    say(f"[mirror] signposts {label} B={B} V={V} kappa={kappa} dtype={dtype}")
    g = dev(logits) if gpu_logits is None else gpu_logits
    ids, lp, lp16, st = capi.mirror_signposts(g, kappa, want_bf16=True)
    torch.cuda.synchronize()
    ids, lp, st = ids.cpu().numpy(), lp.cpu().numpy(), st.cpu().numpy().astype(np.uint32)
    lp16 = lp16.cpu().numpy().view(np.uint16)
    o_ids, o_lp, o_st = oracle.signposts(logits, dtype, kappa)
    assert (st == o_st).all(), np.flatnonzero(st != o_st)[:5]
    bad = np.flatnonzero((ids != o_ids).any(axis=1))
    assert len(bad) == 0, f"rows {bad[:5]}: gpu {ids[bad[0]]} oracle {o_ids[bad[0]]}"
    fin = np.isfinite(o_lp)
    assert ((np.isnan(lp) == np.isnan(o_lp)) & (np.isneginf(lp) == np.isneginf(o_lp))).all()
    err = np.abs(lp[fin] - o_lp[fin])
    assert (err <= 2e-5 + 1e-5 * np.abs(o_lp[fin])).all(), err.max()
    # the bf16 form is the round-to-nearest-even of the fp32 value, and within bf16 precision
    # of the oracle's value
    assert (lp16 == _bf16_of(lp)).all()
    dec = (lp16.astype(np.uint32) << 16).view(np.float32)
    assert (np.abs(dec[fin] - o_lp[fin]) <= 2e-5 + 4e-3 * np.abs(o_lp[fin])).all()
    say(f"[mirror] signposts {label} ok: max |d log p| {err.max() if err.size else 0:.2e}")
    return ids, lp


def test_signposts_full_size():
    w = synth.mirror()
    ids, lp = check_signposts(w.logits, synth.BF16, w.kappa, label="early-exit rows")
    assert (np.diff(lp, axis=1) <= 0).all()


@pytest.mark.parametrize("dtype", [synth.FP32, synth.BF16])
@pytest.mark.parametrize("V", [1, 2, 7, 63, 2047, 2048, 2049, 8191, 8192, 8193, 40000, 128256])
def test_signposts_shapes(dtype, V):
    rng = np.random.default_rng(V * 7 + dtype)
    B = 12
    z = rng.normal(0, 3, (B, V)).astype(np.float32)
    z[1] = np.round(z[1])                                 # heavy ties
    z[2] = 0.0                                            # flat row
    z[2, rng.random(V) < 0.5] = -0.0                      # signed zeros tie
    z[3] = -np.inf
    z[3, V // 2] = 1.5                                    # one finite logit
    z[4, rng.random(V) < 0.3] = -np.inf
    if V > 5:
        z[5] = np.nan if V % 2 else np.inf                 # a bad row
        z[5, :V // 2] = 0.5
    z[6] = -np.inf                                        # no finite logit
    z[7] = z[7] * 40.0 + 300.0                            # large magnitudes
    arr = synth.f32_to_bf16_bits(z) if dtype == synth.BF16 else z
    for kappa in (1, 3, 8, 16):
        check_signposts(arr, dtype, kappa, label=f"V={V} kappa={kappa}")


def test_signposts_unaligned_rows_and_zipf():
    rng = np.random.default_rng(5)
    z = synth.zipf_rows(rng, 9, 100003)                   # odd V: element loads
    check_signposts(synth.f32_to_bf16_bits(z), synth.BF16, 8, label="odd V")
    full = synth.f32_to_bf16_bits(synth.zipf_rows(rng, 5, 32768 + 8))
    buf = dev(np.concatenate([np.zeros(1, np.uint16), full.ravel()]))
    view = buf[1:].view(full.shape)                       # 2-byte aligned base: element loads
    check_signposts(full, synth.BF16, 8, label="unaligned base", gpu_logits=view)


def test_signposts_workspace_reuse_and_determinism():
    w = synth.mirror(B=16, V=50000)
    g = dev(w.logits)
    ws = capi.new_signpost_workspace(16, 50000, 8)
    a = capi.mirror_signposts(g, 8, workspace=ws)
    torch.cuda.synchronize()
    assert int(ws[:16 * 128].sum()) == 0                  # arrival counters back at zero
    b = capi.mirror_signposts(g, 8, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def check_tree(tokens, parents, path, k, t, label=""):
    say(f"[mirror] tree {label} B={tokens.shape[0]} N={tokens.shape[1]} gamma={path.shape[1]}")
    node, hit, batch = capi.mirror_tree_lookup(dev(tokens.astype(np.int32)), dev(parents.astype(np.int32)),
                                               dev(path.astype(np.int32)), dev(np.asarray(k, np.int32)),
                                               dev(np.asarray(t, np.int32)))
    torch.cuda.synchronize()
    o_node, o_hit, o_batch = oracle.tree_lookup(tokens, parents, path, k, t)
    assert (node.cpu().numpy() == o_node).all()
    assert (hit.cpu().numpy() == o_hit).all()
    assert (batch.cpu().numpy() == o_batch).all()
    say(f"[mirror] tree {label} ok: hits {int(o_batch[0])} of {tokens.shape[0]}")
    return o_node


def test_tree_full_size():
    w = synth.mirror()
    check_tree(w.tokens, w.parents, w.path, w.k, w.tstar, label="mirror trees")


def test_tree_random_and_large():
    rng = np.random.default_rng(99)
    for N, B, alphabet in ((1, 8, 2), (37, 50, 3), (300, 40, 4), (5000, 6, 3)):
        gamma = 6
        tok = rng.integers(0, alphabet, (B, N)).astype(np.int32)
        par = np.array([[int(rng.integers(-1, n)) if n else -1 for n in range(N)] for _ in range(B)], np.int32)
        tok[rng.random((B, N)) < 0.05] = -1
        par[rng.random((B, N)) < 0.02] = N + 1
        path = rng.integers(0, alphabet, (B, gamma)).astype(np.int32)
        k = rng.integers(-1, gamma + 2, B).astype(np.int32)
        t = rng.integers(-1, alphabet, B).astype(np.int32)
        check_tree(tok, par, path, k, t, label=f"random N={N}")


def test_tree_worked_example_and_comb():
    ex = json.load(open(os.path.join(GOLDEN, "mirror_reuse_example.json")))
    names = {}
    for lab in list(ex["roots"]) + list(ex["verified_path"]) + ["zhong1", "shang4"]:
        names.setdefault(lab, len(names))
    # the example's fork with the correction among its children: a hit at depth 3
    gamma = len(ex["verified_path"])
    tok = [names[r] for r in ex["roots"]]
    par = [-1] * len(tok)
    prev = 0
    for name in ex["verified_path"][1:]:
        tok.append(names[name]); par.append(prev); prev = len(tok) - 1
    fork = 8  # the depth-2 node of the first branch
    for name in ex["cases"][0]["fork_children"]:
        tok.append(names[name]); par.append(fork)
    path = np.array([[names[x] for x in ex["verified_path"]]], np.int32)
    node = check_tree(np.array([tok], np.int32), np.array([par], np.int32), path, [2], [names["zhong1"]],
                      label="worked example")
    assert node[0] >= 0 and tok[node[0]] == names["zhong1"]
    # a comb is the branch-complete tree of the branch-reuse lookup
    rng = np.random.default_rng(3)
    B, kappa, gamma = 64, 8, 7
    br = rng.integers(0, 3, (B, kappa, gamma)).astype(np.int32)
    combp = np.tile(np.array([-1 if d == 0 else j * gamma + d - 1 for j in range(kappa) for d in range(gamma)],
                             np.int32), (B, 1))
    k = rng.integers(0, gamma + 1, B).astype(np.int32)
    t = rng.integers(0, 3, B).astype(np.int32)
    check_tree(br.reshape(B, -1), combp, br[:, 0], k, t, label="comb")


def test_signposts_size_limits():
    rng = np.random.default_rng(17)
    z = synth.zipf_rows(rng, 3, 1 << 19)                  # the largest vocabulary (256 lists per row)
    check_signposts(synth.f32_to_bf16_bits(z), synth.BF16, capi.SPEC_MAX_KAPPA, label="V=2^19")
    w = synth.mirror(B=16)
    check_signposts(w.logits, synth.BF16, capi.SPEC_MAX_KAPPA, label="kappa=16 early-exit rows")
