// Register-resident bf16 verification path: see fastpath.h for the structure.
//
// What is computed is the same as the general path (generic.hip): temperature, top-k, softmax
// and nucleus processing of draft and target rows (DeepMind speculative-sampling page, section
// 6), Saguaro sigma_{F,C} on the draft (SSD reading notes, section 4.4; hyper.ai summary,
// Method), the min(1, q/p) acceptance test with first-rejection cutoff and the residual /
// bonus sampling (DeepMind page, sections 1 and 3; SSD reading notes, section 2.2).
//
// How it is computed differs: bf16 logits take few distinct values, so a row's processed
// distribution is fixed by the count of every distinct value.  Counting replaces the
// per-element exp: masses are count * exp((z - m)/T) in fp64, one exp per distinct value.
#include "fast_common.h"

namespace sv {
namespace fast {

// ------------------------------------------------------------------------------------------
// Host side
// ------------------------------------------------------------------------------------------
FastPlan fast_plan(int B, int K, int V) {
    FastPlan p;
    p.nS = (V + kSliceCols - 1) / kSliceCols;
    p.units = B * (K + 1);
    const int reqs_per_xcd = (B + kXcd - 1) / kXcd;
    p.grid = kXcd * reqs_per_xcd * (K + 1) * p.nS;
    // two workgroups per slice of the residual when they all fit on the device at once (the
    // residual pass's latency halves); beyond one round of workgroups, one per slice (half as many
    // fixed phases).  Two also whenever a request has more cache rows than slices, so that every
    // workgroup writing a cache row is one of the residual's (the fused lookup's rendezvous).
    const int two_grid = kXcd * reqs_per_xcd * max(2 * p.nS, K + 1);
    p.halves = (two_grid <= resolve_resident() || K + 1 > p.nS) ? 2 : 1;
    p.grid_resolve = p.halves == 2 ? two_grid : kXcd * reqs_per_xcd * max(p.nS, K + 1);
    p.grid_diverge = kXcd * reqs_per_xcd * p.nS * K;               // one per slice of every drafted position
    p.slice_prio = p.grid <= count_resident() ? 1 : 0;
    p.ws_bytes = layout(B, p.units, p.nS).total;
    return p;
}

bool fast_path_applies(const VerifyArgs& a) {
    // drafted tokens are sampled here only from the uniform draft (random-token backup)
    if (a.dtype != SPEC_BF16 || ((a.flags & SPEC_SAMPLE_DRAFT) && !(a.flags & SPEC_UNIFORM_DRAFT))) return false;
    if (a.V % 8 != 0 || a.V < 2048) return false;
    // the request decision reads one unit per lane of a single wave: K + 1 <= 64 positions
    if (a.K + 1 > kWave) return false;
    if ((reinterpret_cast<uintptr_t>(a.draft) & 15) || (reinterpret_cast<uintptr_t>(a.target) & 15)) return false;
    const int nS = (a.V + kSliceCols - 1) / kSliceCols;
    return nS * kTop <= kMergeCap;  // every slice's candidate list fits the merge buffer
}

bool fast_fuzzy_applies(const VerifyArgs& a) {
    return fast_path_applies(a) && !(a.flags & SPEC_ASSISTED) && a.K < kWave;
}

static int launch_fast(const VerifyArgs& a, const CacheArgs* c, void* ws, size_t ws_bytes, hipStream_t stream,
                       const LookupOut* lk = nullptr, const CountEvents* ev = nullptr) {
    const FastPlan p = fast_plan(a.B, a.K, a.V);
    if (ws_bytes < p.ws_bytes) return SPEC_EWORKSPACE;
    FastArgs f;
    f.a = a;
    f.nS = p.nS;
    f.halves = p.halves;
    f.slice_prio = p.slice_prio;
    f.units = p.units;
    f.ws = static_cast<char*>(ws);
    f.L = layout(a.B, p.units, p.nS);
    f.cache = c ? 1 : 0;
    f.uniform = (a.flags & SPEC_UNIFORM_DRAFT) ? 1 : 0;
    f.budget = c ? c->budget : 0;
    f.out_cache = c ? c->out_cache : nullptr;
    if (c) f.fan = c->fanout;
    else f.fan = Fanout{};
    f.lookup = lk ? 1 : 0;
    f.out_slot = lk ? lk->slot : nullptr;
    f.out_hit = lk ? lk->hit : nullptr;
    f.out_batch = lk ? lk->batch : nullptr;
    launch_count(f, p.grid, stream, ev ? ev->before : nullptr, ev ? ev->after : nullptr);
    if (a.tau) launch_diverge(f, p.grid_diverge, stream);
    launch_resolve(f, p.grid_resolve, stream);
    return hipGetLastError() == hipSuccess ? SPEC_OK : SPEC_EHIP;
}

int fast_verify(const VerifyArgs& a, void* ws, size_t ws_bytes, hipStream_t stream) {
    return launch_fast(a, nullptr, ws, ws_bytes, stream);
}

bool fast_cache_applies(const VerifyArgs& a, const CacheArgs& c) {
    if (!fast_path_applies(a) || a.draft_rows != a.K + 1 || c.budget < 1) return false;
    for (int k = 0; k <= a.K; ++k)
        if (c.fanout.f[k] + (k < a.K ? 1 : 0) > kTop) return false;  // a slice lists at most kTop
    return true;
}

int fast_verify_cache(const VerifyArgs& a, const CacheArgs& c, void* ws, size_t ws_bytes, hipStream_t stream) {
    return launch_fast(a, &c, ws, ws_bytes, stream);
}

// Every workgroup that writes a request's cache rows in the resolve kernel (unit w <= K) meets
// the request's others at its arrival counter: needs K + 1 <= 2 nS (the residual's workgroups).
bool fast_lookup_fuses(const VerifyArgs& a) {
    const int nS = (a.V + kSliceCols - 1) / kSliceCols;
    return a.K + 1 <= 2 * nS && !a.tau;
}

int fast_verify_cache_lookup(const VerifyArgs& a, const CacheArgs& c, const LookupOut& l, void* ws, size_t ws_bytes,
                             hipStream_t stream, const CountEvents* ev) {
    return launch_fast(a, &c, ws, ws_bytes, stream, &l, ev);
}

}  // namespace fast
}  // namespace sv
