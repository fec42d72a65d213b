"""Thin ctypes binding of libspecverify.so (include/specverify.h), same names as the C ABI.

Argument marshalling only: torch tensors supply device pointers and the current HIP stream;
every step of the path runs in the library's kernels.  There is no CPU fallback - a missing
or unloadable library raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libspecverify.so")

SPEC_OK, SPEC_EINVAL, SPEC_EDTYPE, SPEC_EWORKSPACE, SPEC_EHIP = 0, -1, -2, -3, -4
SPEC_FP32, SPEC_BF16 = 0, 1
SPEC_SAMPLE_DRAFT = 1
SPEC_UNIFORM_DRAFT = 2
SPEC_ASSISTED = 4
SPEC_MAX_F = 64
SPEC_MAX_KAPPA = 16
SPEC_NOALLOC_SCRATCH_BYTES = 32 << 20
ST_EMPTY_RESIDUAL = 8
ST_OUTSIDE_DRAFT_SUPPORT = 16
ST_BAD_LOGIT = 32
ST_BAD_TOKEN = 64
ST_DEGENERATE_DOWNWEIGHT = 128
ST_BAD_PARAM = 256
ST_PLACEMENT = 512

EXPORTS = ("spec_workspace_bytes", "spec_verify", "saguaro_downweight", "saguaro_fanout", "saguaro_cache_build",
           "saguaro_cache_lookup", "saguaro_verify_cache", "saguaro_backup_plan", "mirror_signpost_workspace_bytes",
           "mirror_signposts", "mirror_tree_lookup", "pyramid_verify", "spec_read_ceiling",
           "saguaro_verify_cache_noalloc", "saguaro_verify_cache_lookup", "saguaro_verify_cache_lookup_timed")

_P = ctypes.c_void_p
_I = ctypes.c_int
_U64 = ctypes.c_uint64
_D = ctypes.c_double


class SpecError(RuntimeError):
    def __init__(self, fn: str, rc: int):
        names = {SPEC_EINVAL: "SPEC_EINVAL", SPEC_EDTYPE: "SPEC_EDTYPE", SPEC_EWORKSPACE: "SPEC_EWORKSPACE",
                 SPEC_EHIP: "SPEC_EHIP"}
        super().__init__(f"{fn} returned {names.get(rc, rc)}")
        self.rc = rc


class Lib:
    def __init__(self, path: str = LIB_PATH):
        if not os.path.exists(path):
            raise RuntimeError(f"HIP library {path} is not built (python -m lossless_speculative_sampling_amd.build)")
        self.cdll = L = ctypes.CDLL(path)
        L.spec_workspace_bytes.argtypes = [_I, _I, _I]
        L.spec_workspace_bytes.restype = ctypes.c_size_t
        L.spec_verify.argtypes = [_P, _I, _P, _I, _I, _I, _I, _P, _I, ctypes.c_float, _P, _U64, _U64, ctypes.c_uint32,
                                  _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
        L.saguaro_downweight.argtypes = [_P, _I, _I, _I, _I, _I, _P, _I, ctypes.c_float, _P, _P, _P, _P, _P]
        L.saguaro_fanout.argtypes = [_I, _I, _D, _D, _P]
        L.saguaro_cache_build.argtypes = [_P, _I, _I, _I, _I, _P, _I, _D, _D, _P, _P, _P]
        L.saguaro_cache_lookup.argtypes = [_I, _P, _P, _I, _I, _P, _P, _P, _P, _P, _P]
        L.saguaro_backup_plan.argtypes = [_I, _P, _P, _I, _P, _P, _P]
        L.mirror_signpost_workspace_bytes.argtypes = [_I, _I, _I]
        L.mirror_signpost_workspace_bytes.restype = ctypes.c_size_t
        L.mirror_signposts.argtypes = [_P, _I, _I, _I, _I, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
        L.mirror_tree_lookup.argtypes = [_P, _P, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P]
        L.pyramid_verify.argtypes = [_P, _I, _P, _I, _I, _I, _I, _P, _I, ctypes.c_float, _P, _P, ctypes.c_uint64,
                                     ctypes.c_uint64, ctypes.c_uint32, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
        L.saguaro_verify_cache.argtypes = [_P, _P, _I, _I, _I, _I, _P, _I, ctypes.c_float, _P, _U64, _U64,
                                           ctypes.c_uint32, _I, _D, _D, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t,
                                           _P]
        L.spec_read_ceiling.argtypes = [_P, ctypes.c_size_t, _P, _P]
        L.saguaro_verify_cache_lookup.argtypes = [_P, _P, _I, _I, _I, _I, _P, _I, ctypes.c_float, _P, _U64, _U64,
                                                  ctypes.c_uint32, _I, _D, _D, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                                  ctypes.c_size_t, _P]
        L.saguaro_verify_cache_lookup_timed.argtypes = L.saguaro_verify_cache_lookup.argtypes + [_P, _P]
        L.saguaro_verify_cache_noalloc.argtypes = [_P, _P, _I, _I, _I, _I, _P, _I, ctypes.c_float, _P, _U64, _U64,
                                                   ctypes.c_uint32, _I, _D, _D, _P, _P, _P, _P, _P, _P, _P]
        for fn in EXPORTS[1:]:
            getattr(L, fn).restype = _I


_lib: Optional[Lib] = None


def load(path: str = LIB_PATH) -> Lib:
    global _lib
    if _lib is None:
        _lib = Lib(path)
    return _lib


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("device tensor expected")
    if not t.is_contiguous():
        raise ValueError("contiguous tensor expected")
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _check(fn: str, rc: int):
    if rc != SPEC_OK:
        raise SpecError(fn, rc)


def dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return SPEC_FP32
    if t.dtype in (torch.bfloat16, torch.int16, torch.uint16):
        return SPEC_BF16
    raise ValueError(f"unsupported logit dtype {t.dtype}")


# ---- argument checks: every shape and dtype the C ABI assumes, so that a wrong tensor raises here
# instead of being read past its end by the library ----
def _need(cond: bool, msg: str):
    if not cond:
        raise ValueError(msg)


def _int32(name: str, t: Optional[torch.Tensor], shape: tuple):
    _need(t is not None, f"{name} is required")
    _need(t.dtype == torch.int32, f"{name} must be int32, got {t.dtype}")
    _need(tuple(t.shape) == tuple(shape), f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _params(params: torch.Tensor, B: int):
    _int32("params", params, (B, 3))


def _logits(name: str, t: torch.Tensor, dims: int = 3) -> int:
    _need(t.dim() == dims, f"{name} must be {dims}-D, got shape {tuple(t.shape)}")
    _need(all(n > 0 for n in t.shape), f"{name} has an empty dimension: {tuple(t.shape)}")
    return dtype_code(t)


def _verify_inputs(draft: Optional[torch.Tensor], target: torch.Tensor, K: int, params: torch.Tensor,
                   tokens: torch.Tensor, draft_rows=None) -> int:
    code = _logits("target", target)
    B, rows, V = target.shape
    _need(K >= 1 and rows == K + 1, f"target must hold K + 1 = {K + 1} rows per request, got {rows}")
    if draft is not None:
        _need(_logits("draft", draft) == code, "draft and target must have the same dtype")
        _need(draft.shape[0] == B and draft.shape[2] == V, f"draft {tuple(draft.shape)} does not match target "
                                                           f"{tuple(target.shape)}")
        allowed = (K, K + 1) if draft_rows is None else (draft_rows,)
        _need(draft.shape[1] in allowed, f"draft must hold {' or '.join(map(str, allowed))} rows, got {draft.shape[1]}")
    _params(params, B)
    _int32("tokens", tokens, (B, K))
    return code


def _verify_out(out, B: int):
    for name in ("k", "tstar", "status"):
        _int32(f"out.{name}", getattr(out, name), (B,))
    _need(out.resid_mass.dtype == torch.float32 and tuple(out.resid_mass.shape) == (B,), "out.resid_mass must be float32 [B]")


def _workspace(ws: torch.Tensor):
    _need(ws.dtype == torch.uint8 and ws.dim() == 1, "workspace must be a 1-D uint8 tensor")


def spec_workspace_bytes(B: int, K: int, V: int) -> int:
    return int(load().cdll.spec_workspace_bytes(B, K, V))


def params_tensor(temperature, top_k, top_p, device="cuda") -> torch.Tensor:
    """[B] spec_params packed as int32 words {float T, int32 top_k, float top_p}."""
    T = torch.as_tensor(temperature, dtype=torch.float32).reshape(-1)
    k = torch.as_tensor(top_k, dtype=torch.int32).reshape(-1)
    p = torch.as_tensor(top_p, dtype=torch.float32).reshape(-1)
    B = max(T.numel(), k.numel(), p.numel())
    T, k, p = T.expand(B), k.expand(B), p.expand(B)
    rec = torch.stack([T.view(torch.int32), k, p.view(torch.int32)], dim=1).contiguous()
    return rec.to(device)


def new_workspace(B: int, K: int, V: int, device="cuda") -> torch.Tensor:
    """Zero-filled spec_verify workspace (the library leaves it zero-filled after every call)."""
    return torch.zeros(max(spec_workspace_bytes(B, K, V), 1), dtype=torch.uint8, device=device)


@dataclass
class VerifyOut:
    k: torch.Tensor
    tstar: torch.Tensor
    resid_mass: torch.Tensor
    status: torch.Tensor
    tokens: torch.Tensor


def spec_verify(draft: Optional[torch.Tensor], target: torch.Tensor, K: int, params: torch.Tensor,
                tokens: torch.Tensor, F: int = 0, C: float = 1.0, seed: int = 0, round_: int = 0, flags: int = 0,
                workspace: Optional[torch.Tensor] = None, out: Optional[VerifyOut] = None, stream=None) -> VerifyOut:
    """draft [B][Kd][V] and target [B][K+1][V] device logits; tokens [B][K] int32 (in, or out under
    SPEC_SAMPLE_DRAFT).  With SPEC_UNIFORM_DRAFT draft may be None.  Returns the outputs (allocated
    here unless `out` is given)."""
    _need(draft is not None or bool(flags & SPEC_UNIFORM_DRAFT), "draft logits are required without SPEC_UNIFORM_DRAFT")
    code = _verify_inputs(draft, target, K, params, tokens)
    B, _, V = target.shape
    Kd = draft.shape[1] if draft is not None else K
    dev = target.device
    if out is None:
        out = VerifyOut(torch.empty(B, dtype=torch.int32, device=dev), torch.empty(B, dtype=torch.int32, device=dev),
                        torch.empty(B, dtype=torch.float32, device=dev), torch.empty(B, dtype=torch.int32, device=dev),
                        tokens)
    _verify_out(out, B)
    if workspace is None:
        workspace = new_workspace(B, K, V, dev)
    _workspace(workspace)
    rc = load().cdll.spec_verify(_ptr(draft), Kd, _ptr(target), code, B, K, V, _ptr(params), F,
                                 ctypes.c_float(C), _ptr(tokens), seed, round_, flags, _ptr(out.k), _ptr(out.tstar),
                                 _ptr(out.resid_mass), _ptr(out.status), _ptr(workspace), workspace.numel(),
                                 _stream(stream))
    _check("spec_verify", rc)
    out.tokens = tokens
    return out


def saguaro_downweight(draft: torch.Tensor, K: int, params: torch.Tensor, F: int, C: float, want_probs=False,
                       stream=None):
    _logits("draft", draft)
    B, Kd, V = draft.shape
    _need(1 <= K <= Kd, f"K = {K} must lie in [1, {Kd}] (draft rows)")
    _params(params, B)
    dev = draft.device
    ids = torch.empty((B, K, max(F, 1)), dtype=torch.int32, device=dev)
    Z = torch.empty((B, K), dtype=torch.float32, device=dev)
    st = torch.empty((B, K), dtype=torch.int32, device=dev)
    probs = torch.empty((B, K, V), dtype=torch.float32, device=dev) if want_probs else None
    rc = load().cdll.saguaro_downweight(_ptr(draft), Kd, dtype_code(draft), B, K, V, _ptr(params), F,
                                        ctypes.c_float(C), _ptr(ids), _ptr(Z), _ptr(probs), _ptr(st), _stream(stream))
    _check("saguaro_downweight", rc)
    return ids[:, :, :F], Z, probs, st


def saguaro_fanout(K: int, budget: int, a: float, r: float) -> list[int]:
    buf = (ctypes.c_int32 * (K + 1))()
    _check("saguaro_fanout", load().cdll.saguaro_fanout(K, budget, a, r, ctypes.cast(buf, _P)))
    return list(buf)


def saguaro_cache_build(draft: torch.Tensor, K: int, tokens: torch.Tensor, budget: int, a: float, r: float,
                        stream=None):
    _logits("draft", draft)
    B, Kd, V = draft.shape
    _need(K >= 1 and Kd == K + 1, f"draft must hold K + 1 = {K + 1} rows per request, got {Kd}")
    _int32("tokens", tokens, (B, K))
    fan = (ctypes.c_int32 * (K + 1))()
    cache = torch.empty((B, max(budget, 1)), dtype=torch.int32, device=draft.device)
    rc = load().cdll.saguaro_cache_build(_ptr(draft), dtype_code(draft), B, K, V, _ptr(tokens), budget, a, r,
                                         ctypes.cast(fan, _P), _ptr(cache), _stream(stream))
    _check("saguaro_cache_build", rc)
    return cache[:, :budget], list(fan)


def saguaro_verify_cache(draft: torch.Tensor, target: torch.Tensor, K: int, params: torch.Tensor, tokens: torch.Tensor,
                         budget: int, a: float, r: float, F: int = 0, C: float = 1.0, seed: int = 0, round_: int = 0,
                         flags: int = 0, workspace: Optional[torch.Tensor] = None, out: Optional[VerifyOut] = None,
                         cache: Optional[torch.Tensor] = None, stream=None):
    """spec_verify + saguaro_cache_build in one pass; draft [B][K+1][V].  Returns (VerifyOut,
    cache [B][budget], fan-out list)."""
    code = _verify_inputs(draft, target, K, params, tokens, draft_rows=K + 1)
    B, Kd, V = draft.shape
    dev = draft.device
    if out is None:
        out = VerifyOut(torch.empty(B, dtype=torch.int32, device=dev), torch.empty(B, dtype=torch.int32, device=dev),
                        torch.empty(B, dtype=torch.float32, device=dev), torch.empty(B, dtype=torch.int32, device=dev),
                        tokens)
    _verify_out(out, B)
    if workspace is None:
        workspace = new_workspace(B, K, V, dev)
    _workspace(workspace)
    if cache is None:
        cache = torch.empty((B, max(budget, 1)), dtype=torch.int32, device=dev)
    _need(cache.dtype == torch.int32 and cache.dim() == 2 and cache.shape[0] == B and cache.shape[1] >= budget,
          f"cache must be int32 [{B}][>= {budget}]")
    fan = (ctypes.c_int32 * (K + 1))()
    rc = load().cdll.saguaro_verify_cache(_ptr(draft), _ptr(target), code, B, K, V, _ptr(params), F,
                                          ctypes.c_float(C), _ptr(tokens), seed, round_, flags, budget, a, r,
                                          ctypes.cast(fan, _P), _ptr(out.k), _ptr(out.tstar), _ptr(out.resid_mass),
                                          _ptr(out.status), _ptr(cache), _ptr(workspace), workspace.numel(),
                                          _stream(stream))
    _check("saguaro_verify_cache", rc)
    out.tokens = tokens
    return out, cache[:, :budget], list(fan)


def saguaro_verify_cache_lookup(draft: torch.Tensor, target: torch.Tensor, K: int, params: torch.Tensor,
                                tokens: torch.Tensor, budget: int, a: float, r: float, F: int = 0, C: float = 1.0,
                                seed: int = 0, round_: int = 0, flags: int = 0, workspace: Optional[torch.Tensor] = None,
                                out: Optional[VerifyOut] = None, cache: Optional[torch.Tensor] = None, stream=None):
    """saguaro_verify_cache and the mode-0 lookup of its outcomes in one call.  Returns (VerifyOut,
    cache [B][budget], fan-out list, slot [B] int32, hit [B] uint8, batch [2] int32)."""
    code = _verify_inputs(draft, target, K, params, tokens, draft_rows=K + 1)
    B, Kd, V = draft.shape
    dev = draft.device
    if out is None:
        out = VerifyOut(torch.empty(B, dtype=torch.int32, device=dev), torch.empty(B, dtype=torch.int32, device=dev),
                        torch.empty(B, dtype=torch.float32, device=dev), torch.empty(B, dtype=torch.int32, device=dev),
                        tokens)
    _verify_out(out, B)
    if workspace is None:
        workspace = new_workspace(B, K, V, dev)
    _workspace(workspace)
    if cache is None:
        cache = torch.empty((B, max(budget, 1)), dtype=torch.int32, device=dev)
    _need(cache.dtype == torch.int32 and cache.dim() == 2 and cache.shape[0] == B and cache.shape[1] >= budget,
          f"cache must be int32 [{B}][>= {budget}]")
    slot = torch.empty(B, dtype=torch.int32, device=dev)
    hit = torch.empty(B, dtype=torch.uint8, device=dev)
    batch = torch.empty(2, dtype=torch.int32, device=dev)
    fan = (ctypes.c_int32 * (K + 1))()
    rc = load().cdll.saguaro_verify_cache_lookup(_ptr(draft), _ptr(target), code, B, K, V, _ptr(params), F,
                                                 ctypes.c_float(C), _ptr(tokens), seed, round_, flags, budget, a, r,
                                                 ctypes.cast(fan, _P), _ptr(out.k), _ptr(out.tstar),
                                                 _ptr(out.resid_mass), _ptr(out.status), _ptr(cache), _ptr(slot),
                                                 _ptr(hit), _ptr(batch), _ptr(workspace), workspace.numel(),
                                                 _stream(stream))
    _check("saguaro_verify_cache_lookup", rc)
    out.tokens = tokens
    return out, cache[:, :budget], list(fan), slot, hit, batch


def saguaro_verify_cache_noalloc(draft: torch.Tensor, target: torch.Tensor, K: int, params: torch.Tensor,
                                 tokens: torch.Tensor, budget: int, a: float, r: float, out: VerifyOut,
                                 cache: torch.Tensor, F: int = 0, C: float = 1.0, seed: int = 0, round_: int = 0,
                                 flags: int = 0, stream=None):
    """saguaro_verify_cache on the library's static scratch (no workspace); the caller passes the
    outputs (out, cache [B][>= budget]).  Returns the fan-out list."""
    code = _verify_inputs(draft, target, K, params, tokens, draft_rows=K + 1)
    B, Kd, V = draft.shape
    _verify_out(out, B)
    _need(cache.dtype == torch.int32 and cache.dim() == 2 and cache.shape[0] == B and cache.shape[1] >= budget,
          f"cache must be int32 [{B}][>= {budget}]")
    fan = (ctypes.c_int32 * (K + 1))()
    rc = load().cdll.saguaro_verify_cache_noalloc(_ptr(draft), _ptr(target), code, B, K, V, _ptr(params), F,
                                                  ctypes.c_float(C), _ptr(tokens), seed, round_, flags, budget, a, r,
                                                  ctypes.cast(fan, _P), _ptr(out.k), _ptr(out.tstar),
                                                  _ptr(out.resid_mass), _ptr(out.status), _ptr(cache),
                                                  _stream(stream))
    _check("saguaro_verify_cache_noalloc", rc)
    return list(fan)


def saguaro_cache_lookup(mode: int, cache: torch.Tensor, fanout_or_shape, K: int, B: int, k: torch.Tensor,
                         tstar: torch.Tensor, stream=None):
    dev = cache.device
    fs_list = [int(x) for x in fanout_or_shape]
    _need(cache.dtype == torch.int32, "cache must be int32")
    if mode == 0:
        _need(len(fs_list) == K + 1, f"mode 0 takes K + 1 = {K + 1} fan-out entries, got {len(fs_list)}")
        _need(cache.dim() == 2 and cache.shape[0] == B, f"cache must be [{B}][budget]")
        _need(cache.shape[1] >= sum(fs_list), f"cache holds {cache.shape[1]} slots, the fan-out needs {sum(fs_list)}")
        per = 1
    elif mode == 1:
        _need(len(fs_list) == 2, "mode 1 takes {kappa, gamma}")
        _need(cache.numel() == B * fs_list[0] * fs_list[1], "branches must hold B * kappa * gamma tokens")
        per = fs_list[0]  # k and t* of every chain
    else:
        raise ValueError(f"unknown lookup mode {mode}")
    _need(k.numel() == B * per, f"k must hold {B * per} entries")
    _need(tstar.numel() == B * per, f"tstar must hold {B * per} entries")
    _need(k.dtype == torch.int32, "k must be int32")
    _need(tstar.dtype == torch.int32, "tstar must be int32")
    fs = (ctypes.c_int32 * len(fs_list))(*fs_list)
    slot = torch.empty(B, dtype=torch.int32, device=dev)
    hit = torch.empty(B, dtype=torch.uint8, device=dev)
    batch = torch.empty(2, dtype=torch.int32, device=dev)
    rc = load().cdll.saguaro_cache_lookup(mode, _ptr(cache), ctypes.cast(fs, _P), K, B, _ptr(k), _ptr(tstar),
                                          _ptr(slot), _ptr(hit), _ptr(batch), _stream(stream))
    _check("saguaro_cache_lookup", rc)
    return slot, hit, batch


def saguaro_backup_plan(hit: torch.Tensor, batch: torch.Tensor, b_star: int, stream=None):
    """(use_backup [B] int32, switch [1] int32) on the device: the batch-aware random-token fallback."""
    B = hit.shape[0]
    _need(hit.dtype == torch.uint8 and hit.dim() == 1, "hit must be uint8 [B]")
    _int32("batch", batch, (2,))
    use = torch.empty(B, dtype=torch.int32, device=hit.device)
    sw = torch.empty(1, dtype=torch.int32, device=hit.device)
    rc = load().cdll.saguaro_backup_plan(B, _ptr(hit), _ptr(batch), b_star, _ptr(use), _ptr(sw), _stream(stream))
    _check("saguaro_backup_plan", rc)
    return use, sw



def mirror_signpost_workspace_bytes(B: int, V: int, kappa: int) -> int:
    return int(load().cdll.mirror_signpost_workspace_bytes(B, V, kappa))


def new_signpost_workspace(B: int, V: int, kappa: int, device="cuda") -> torch.Tensor:
    n = mirror_signpost_workspace_bytes(B, V, kappa)
    if n == 0:
        raise SpecError("mirror_signpost_workspace_bytes", SPEC_EINVAL)
    return torch.zeros(n, dtype=torch.uint8, device=device)


def mirror_signposts(logits: torch.Tensor, kappa: int, want_bf16: bool = False,
                     workspace: Optional[torch.Tensor] = None, out=None, stream=None):
    """Early-exit signposts of logits [B][V]: (ids [B][kappa] int32, log p~ [B][kappa] float32,
    log p~ as bf16 bits [B][kappa] int16 or None, status [B] int32)."""
    code = _logits("logits", logits, dims=2)
    B, V = logits.shape
    dev = logits.device
    if workspace is None:
        workspace = new_signpost_workspace(B, V, kappa, dev)
    _workspace(workspace)
    if out is None:
        out = (torch.empty((B, kappa), dtype=torch.int32, device=dev),
               torch.empty((B, kappa), dtype=torch.float32, device=dev),
               torch.empty((B, kappa), dtype=torch.int16, device=dev) if want_bf16 else None,
               torch.empty(B, dtype=torch.int32, device=dev))
    ids, lp, lp16, st = out
    rc = load().cdll.mirror_signposts(_ptr(logits), code, B, V, kappa, _ptr(ids), _ptr(lp), _ptr(lp16),
                                      _ptr(st), _ptr(workspace), workspace.numel(), _stream(stream))
    _check("mirror_signposts", rc)
    return out


def mirror_tree_lookup(tokens: torch.Tensor, parents: torch.Tensor, path: torch.Tensor, k: torch.Tensor,
                       tstar: torch.Tensor, stream=None):
    """Reuse node of the committed prefix in each request's draft tree [B][N]: (node [B], hit [B], batch [2])."""
    _need(tokens.dim() == 2, "tokens must be [B][N]")
    B, N = tokens.shape
    _int32("tokens", tokens, (B, N))
    _int32("parents", parents, (B, N))
    _need(path.dim() == 2 and path.shape[0] == B, "path must be [B][gamma]")
    gamma = path.shape[1]
    _int32("path", path, (B, gamma))
    _int32("k", k, (B,))
    _int32("tstar", tstar, (B,))
    dev = tokens.device
    node = torch.empty(B, dtype=torch.int32, device=dev)
    hit = torch.empty(B, dtype=torch.uint8, device=dev)
    batch = torch.empty(2, dtype=torch.int32, device=dev)
    rc = load().cdll.mirror_tree_lookup(_ptr(tokens), _ptr(parents), B, N, gamma, _ptr(path), _ptr(k), _ptr(tstar),
                                        _ptr(node), _ptr(hit), _ptr(batch), _stream(stream))
    _check("mirror_tree_lookup", rc)
    return node, hit, batch


def pyramid_verify(draft: Optional[torch.Tensor], verifier: torch.Tensor, K: int, params: torch.Tensor,
                   tau: torch.Tensor, tokens: torch.Tensor, F: int = 0, C: float = 1.0, seed: int = 0, round_: int = 0,
                   flags: int = 0, want_div: bool = False, workspace: Optional[torch.Tensor] = None, stream=None):
    """Fuzzy (PyramidSD) verification of one stage: (VerifyOut, divergences [B][K] or None)."""
    _need(draft is not None or bool(flags & SPEC_UNIFORM_DRAFT), "draft logits are required without SPEC_UNIFORM_DRAFT")
    code = _verify_inputs(draft, verifier, K, params, tokens)
    B, _, V = verifier.shape
    _need(tau.dtype == torch.float32 and tuple(tau.shape) == (B,), "tau must be float32 [B]")
    Kd = draft.shape[1] if draft is not None else K
    dev = verifier.device
    if workspace is None:
        workspace = new_workspace(B, K, V, dev)
    _workspace(workspace)
    out = VerifyOut(torch.empty(B, dtype=torch.int32, device=dev), torch.empty(B, dtype=torch.int32, device=dev),
                    torch.empty(B, dtype=torch.float32, device=dev), torch.empty(B, dtype=torch.int32, device=dev),
                    tokens)
    div = torch.zeros((B, K), dtype=torch.float32, device=dev) if want_div else None
    rc = load().cdll.pyramid_verify(_ptr(draft), Kd, _ptr(verifier), code, B, K, V, _ptr(params), F,
                                    ctypes.c_float(C), _ptr(tau), _ptr(tokens), seed, round_, flags, _ptr(out.k),
                                    _ptr(out.tstar), _ptr(out.resid_mass), _ptr(out.status), _ptr(div),
                                    _ptr(workspace), workspace.numel(), _stream(stream))
    _check("pyramid_verify", rc)
    return out, div


def spec_read_ceiling(data: torch.Tensor, sink: torch.Tensor, stream: Optional[int] = None) -> None:
    """One plain streaming read of every byte of `data` (contiguous, 16-byte aligned, a multiple
    of 16 bytes): the bandwidth ceiling a call reading as many bytes is set against."""
    _need(data.is_contiguous(), "data must be contiguous")
    _need(sink.dtype == torch.int32 and sink.numel() >= 1, "sink must hold one int32")
    nbytes = data.numel() * data.element_size()
    rc = load().cdll.spec_read_ceiling(_ptr(data), nbytes, _ptr(sink), _stream(stream))
    _check("spec_read_ceiling", rc)
