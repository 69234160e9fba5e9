"""KDA forward prefill and decode on MI355X (gfx950): Python binding of libkda.so.

Argument marshalling only: every step runs in the library's HIP kernels,
reached through the C ABI of include/kda.h. PyTorch provides device memory and
the current HIP stream. There is no fallback: if the library is not built,
every entry point raises.

    import kda_chunked_delta_amd as kda
    o, s = kda.prefill(q, k, v, g, beta, cu_seqlens=cu, initial_state=s0,
                       output_final_state=True, use_intracard_cp="auto")
    o_t = kda.decode(q_t, k_t, v_t, g_t, beta_t, s)   # one token each, s in place

The interface follows the FLA-compatible prefill of "feat(kda/sm90): FlashKDA
prefill port + intracard-CP prefill" (cuLA pull request #103, description:
varlen packing, initial/final state, use_intracard_cp = "auto" | True | False,
default off) and the in-place state update exercised by "fix(cake_kda):
support non-aligned recurrent prefill head counts" (FlashInfer pull request
#4351, description).
"""
from __future__ import annotations

import atexit
import collections
import ctypes
import os
import threading

__all__ = ["prefill", "decode", "plan", "plan_host", "plan_segments", "Plan", "Context", "context",
           "KDAError", "lib", "LIB_PATH", "CP_OFF", "CP_ON", "CP_AUTO"]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkda.so")
D = 128
CP_OFF, CP_ON, CP_AUTO = 0, 1, 2


class KDAError(RuntimeError):
    """A libkda call returned an error status."""

    def __init__(self, status, message):
        super().__init__("%s (status %d)" % (message, status))
        self.status = status


class PlanInfo(ctypes.Structure):
    _fields_ = [("n_seqs", ctypes.c_int32), ("H", ctypes.c_int32), ("dk", ctypes.c_int32),
                ("dv", ctypes.c_int32), ("total_tokens", ctypes.c_int64),
                ("total_chunks", ctypes.c_int32), ("uses_cp", ctypes.c_int32),
                ("n_units", ctypes.c_int32), ("n_cp_seqs", ctypes.c_int32),
                ("n_prescan", ctypes.c_int32), ("n_carry_slots", ctypes.c_int32),
                ("max_unit_chunks", ctypes.c_int32), ("n_cus", ctypes.c_int32),
                ("workspace_bytes", ctypes.c_size_t), ("est_serial_us", ctypes.c_double),
                ("est_cp_us", ctypes.c_double), ("k1_materialized", ctypes.c_int32),
                ("n_split_seqs", ctypes.c_int32), ("split_warm_chunks", ctypes.c_int32),
                ("est_split_us", ctypes.c_double), ("warm_cp", ctypes.c_int32),
                ("warm_cp_seg_chunks", ctypes.c_int32), ("n_warm_segments", ctypes.c_int32),
                ("est_warm_cp_us", ctypes.c_double), ("speculation_off", ctypes.c_int32),
                ("split_warm_work", ctypes.c_int32)]

    def as_dict(self):
        return {name: getattr(self, name) for name, _ in self._fields_}


class PrefillOpts(ctypes.Structure):
    _fields_ = [("qk_heads", ctypes.c_int32), ("beta_bf16", ctypes.c_int32), ("state_bf16", ctypes.c_int32)]


class UnitInfo(ctypes.Structure):
    _fields_ = [("seq", ctypes.c_int32), ("chunk0", ctypes.c_int32), ("n_chunks", ctypes.c_int32),
                ("segment", ctypes.c_int32), ("n_segments", ctypes.c_int32),
                ("warm_chunks", ctypes.c_int32)]


_lib = None
_lib_lock = threading.Lock()


def lib():
    """The loaded libkda.so (raises if it has not been built)."""
    global _lib
    with _lib_lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise ImportError("libkda.so is not built (%s); run `python -m kda_chunked_delta_amd.build`"
                                  % LIB_PATH)
            L = ctypes.CDLL(LIB_PATH)
            P, I32, I64, F32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
            PP = ctypes.POINTER(ctypes.c_void_p)
            sig = {
                "kda_create": (ctypes.c_int, [ctypes.c_int, PP]),
                "kda_destroy": (None, [P]),
                "kda_last_error": (ctypes.c_char_p, []),
                "kda_version": (ctypes.c_char_p, []),
                "kda_plan_prefill": (ctypes.c_int, [P, P, I32, I32, I32, I32, ctypes.c_int, PP]),
                "kda_plan_prefill_host": (ctypes.c_int, [I32, P, I32, I32, I32, I32, ctypes.c_int, PP]),
                "kda_plan_prefill_segments": (ctypes.c_int, [P, P, I32, I32, I32, I32, I32, PP]),
                "kda_plan_prefill_split": (ctypes.c_int, [P, P, I32, I32, I32, I32, P, I32, PP]),
                "kda_plan_prefill_warm_cp": (ctypes.c_int, [P, P, I32, I32, I32, I32, I32, I32, PP]),
                "kda_plan_destroy": (None, [P]),
                "kda_plan_get_info": (ctypes.c_int, [P, ctypes.POINTER(PlanInfo)]),
                "kda_plan_workspace_bytes": (ctypes.c_size_t, [P]),
                "kda_plan_get_units": (ctypes.c_int, [P, ctypes.POINTER(UnitInfo), I32]),
                "kda_prefill_validate": (ctypes.c_int, [P, P, P, P, P, P, P, F32, P, P, P]),
                "kda_prefill": (ctypes.c_int, [P, P, P, P, P, P, P, P, F32, P, P, P, P]),
                "kda_debug_k1_records": (ctypes.c_int, [P, P, P, P, P, P, P, P, P, P]),
                "kda_prefill_ex": (ctypes.c_int, [P, P, ctypes.POINTER(PrefillOpts), P, P, P, P, P, P, F32, P, P,
                                                  P, P]),
                "kda_prefill_ex_validate": (ctypes.c_int, [P, ctypes.POINTER(PrefillOpts), P, P, P, P, P, P, F32,
                                                           P, P, P]),
                "kda_prefill_noalloc": (ctypes.c_int, [P, P, ctypes.POINTER(PrefillOpts), P, P, P, P, P, P, F32, P,
                                                       P, P, P]),
                "kda_noalloc_scratch_bytes": (ctypes.c_size_t, []),
                "kda_decode": (ctypes.c_int, [P, I32, I32, I32, I32, I32, P, P, P, P, P, F32, P, P, P]),
                "kda_decode_validate": (ctypes.c_int, [I32, I32, I32, I32, I32, P, P, P, P, P, F32, P, P]),
                "kda_decode_slots": (ctypes.c_int, [P, I32, I32, I32, I32, I32, P, P, P, P, P, F32, P, I32, P, P, P]),
                "kda_decode_slots_validate": (ctypes.c_int, [I32, I32, I32, I32, I32, P, P, P, P, P, F32, P, I32, P,
                                                             P]),
                "kda_set_timing": (ctypes.c_int, [P, ctypes.c_int]),
                "kda_get_timing": (I32, [P, ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(ctypes.c_double),
                                         ctypes.POINTER(I32), I32]),
            }
            for name, (res, args) in sig.items():
                fn = getattr(L, name)
                fn.restype = res
                fn.argtypes = args
            _lib = L
        return _lib


def _check(status, what):
    if status != 0:
        raise KDAError(status, "%s: %s" % (what, lib().kda_last_error().decode()))


def _cp_mode(use_intracard_cp):
    if use_intracard_cp is False or use_intracard_cp is None or use_intracard_cp == CP_OFF:
        return CP_OFF
    if use_intracard_cp is True or use_intracard_cp == CP_ON:
        return CP_ON
    if use_intracard_cp == "auto" or use_intracard_cp == CP_AUTO:
        return CP_AUTO
    raise ValueError("use_intracard_cp must be 'auto', True or False (got %r)" % (use_intracard_cp,))


def _cu_array(cu):
    cu = [int(x) for x in cu]
    return (ctypes.c_int32 * len(cu))(*cu), len(cu) - 1


class Context:
    """A libkda context on one device (device properties cached once)."""

    def __init__(self, device_index):
        self.device = int(device_index)
        h = ctypes.c_void_p()
        _check(lib().kda_create(self.device, ctypes.byref(h)), "kda_create")
        self.handle = h

    def close(self):
        if self.handle:
            lib().kda_destroy(self.handle)
            self.handle = None

    def set_timing(self, enable=True):
        _check(lib().kda_set_timing(self.handle, int(bool(enable))), "kda_set_timing")

    def timing(self):
        """{kernel name: (total ms, launches)} of the prefill calls since the
        last read (waits for them; clears the log)."""
        names = (ctypes.c_char_p * 16)()
        ms = (ctypes.c_double * 16)()
        cnt = (ctypes.c_int32 * 16)()
        n = lib().kda_get_timing(self.handle, names, ms, cnt, 16)
        if n < 0:
            raise KDAError(5, "kda_get_timing: " + lib().kda_last_error().decode())
        return {names[i].decode(): (ms[i], cnt[i]) for i in range(n)}


_contexts = {}
_ctx_lock = threading.Lock()


def context(device=None):
    """The shared Context of a torch device (default: the current device)."""
    import torch
    idx = torch.cuda.current_device() if device is None else torch.device(device).index
    if idx is None:
        idx = torch.cuda.current_device()
    with _ctx_lock:
        ctx = _contexts.get(idx)
        if ctx is None:
            ctx = _contexts[idx] = Context(idx)
        return ctx


_shutting_down = False


@atexit.register
def _close_contexts():
    global _shutting_down
    _plan_cache.clear()
    _shutting_down = True
    for ctx in list(_contexts.values()):
        try:
            ctx.close()
        except Exception:
            pass
    _contexts.clear()


class Plan:
    """A libkda plan (chunk table, work units, CP segments)."""

    def __init__(self, handle, cu_host, device=None):
        self.handle = handle
        self.cu_host = [int(x) for x in cu_host]
        self.device = device
        self._cu_dev = None
        self._shape = None

    def __del__(self):
        try:
            if self.handle and _lib is not None and not _shutting_down:
                _lib.kda_plan_destroy(self.handle)
        except Exception:
            pass
        self.handle = None

    def info(self):
        pi = PlanInfo()
        _check(lib().kda_plan_get_info(self.handle, ctypes.byref(pi)), "kda_plan_get_info")
        return pi.as_dict()

    def shape(self):
        """(H, total tokens, sequences) the plan was built for (cached)."""
        if self._shape is None:
            i = self.info()
            self._shape = (i["H"], i["total_tokens"], i["n_seqs"])
        return self._shape

    def units(self):
        n = self.info()["n_units"]
        arr = (UnitInfo * max(n, 1))()
        _check(lib().kda_plan_get_units(self.handle, arr, n), "kda_plan_get_units")
        return [dict(seq=u.seq, chunk0=u.chunk0, n_chunks=u.n_chunks, segment=u.segment,
                     n_segments=u.n_segments, warm_chunks=u.warm_chunks) for u in arr[:n]]

    def cu_device(self):
        import torch
        if self._cu_dev is None:
            self._cu_dev = torch.tensor(self.cu_host, dtype=torch.int32, device="cuda:%d" % self.device)
        return self._cu_dev


def plan_host(cu_seqlens, H, n_cus, use_intracard_cp=False):
    """Host-only plan for an explicit CU count (inspection; no GPU needed)."""
    arr, n = _cu_array(cu_seqlens)
    h = ctypes.c_void_p()
    _check(lib().kda_plan_prefill_host(int(n_cus), arr, n, int(H), D, D, _cp_mode(use_intracard_cp),
                                       ctypes.byref(h)), "kda_plan_prefill_host")
    return Plan(h, cu_seqlens)


def plan(cu_seqlens, H, use_intracard_cp=False, device=None):
    """Executable plan on a device (tables uploaded to it)."""
    ctx = context(device)
    arr, n = _cu_array(cu_seqlens)
    h = ctypes.c_void_p()
    _check(lib().kda_plan_prefill(ctx.handle, arr, n, int(H), D, D, _cp_mode(use_intracard_cp),
                                  ctypes.byref(h)), "kda_plan_prefill")
    return Plan(h, cu_seqlens, ctx.device)


def plan_segments(cu_seqlens, H, seg_chunks, device=None):
    """Executable CP plan with a forced segment length (in 16-token chunks)."""
    ctx = context(device)
    arr, n = _cu_array(cu_seqlens)
    h = ctypes.c_void_p()
    _check(lib().kda_plan_prefill_segments(ctx.handle, arr, n, int(H), D, D, int(seg_chunks),
                                           ctypes.byref(h)), "kda_plan_prefill_segments")
    return Plan(h, cu_seqlens, ctx.device)


def plan_split(cu_seqlens, H, split_chunk, warm_chunks, device=None):
    """Executable plan with forced warm-start splits: sequence i is split at
    chunk split_chunk[i] (0: not split)."""
    ctx = context(device)
    arr, n = _cu_array(cu_seqlens)
    if len(split_chunk) != n:
        raise ValueError("split_chunk needs one entry per sequence (%d), got %d" % (n, len(split_chunk)))
    sp = (ctypes.c_int32 * max(n, 1))(*[int(x) for x in split_chunk])
    h = ctypes.c_void_p()
    _check(lib().kda_plan_prefill_split(ctx.handle, arr, n, int(H), D, D, sp, int(warm_chunks),
                                        ctypes.byref(h)), "kda_plan_prefill_split")
    return Plan(h, cu_seqlens, ctx.device)


def plan_warm_cp(cu_seqlens, H, seg_chunks, warm_chunks, device=None):
    """Executable warm-start CP plan with a forced segment length (chunks)."""
    ctx = context(device)
    arr, n = _cu_array(cu_seqlens)
    h = ctypes.c_void_p()
    _check(lib().kda_plan_prefill_warm_cp(ctx.handle, arr, n, int(H), D, D, int(seg_chunks), int(warm_chunks),
                                          ctypes.byref(h)), "kda_plan_prefill_warm_cp")
    return Plan(h, cu_seqlens, ctx.device)


_plan_cache = collections.OrderedDict()
_PLAN_CACHE_MAX = 64
# Plans used by a call captured into a graph: the graph holds their device
# tables, and may be replayed at any later time, so they are never released.
_captured_plans = []


def _cached_plan(cu_host, H, mode, device):
    key = (device, tuple(cu_host), H, mode)
    p = _plan_cache.get(key)
    if p is None:
        p = plan(cu_host, H, mode, device="cuda:%d" % device)
        _plan_cache[key] = p
        if len(_plan_cache) > _PLAN_CACHE_MAX:
            _plan_cache.popitem(last=False)
    else:
        _plan_cache.move_to_end(key)
    return p


def k1_records(q, k, v, g, beta, plan):
    """Run K1 alone and return its chunk records as a uint8 tensor
    [H, total_chunks, RECORD_BYTES] (layout documented in include/kda.h)."""
    import torch
    info = plan.info()
    rec = torch.empty(info["H"], info["total_chunks"], RECORD_BYTES, dtype=torch.uint8, device=q.device)
    ctx = context(q.device)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    _check(lib().kda_debug_k1_records(ctx.handle, plan.handle, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                      _ptr(plan.cu_device()), _ptr(rec), ctypes.c_void_p(stream)),
           "kda_debug_k1_records")
    return rec


RECORD_BYTES = 14336


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def prefill(q, k, v, g, beta, cu_seqlens=None, initial_state=None, output_final_state=False,
            use_intracard_cp=False, scale=1.0, final_state=None, out=None, plan=None,
            cu_seqlens_host=None, state_dtype=None, no_alloc=False):
    """KDA forward prefill.

    q, k, v: bf16 [Tt, H, 128] packed, or [B, T, H, 128] (B equal-length
    sequences when cu_seqlens is None); g: fp32 log-decay, same shape;
    beta: fp32 or bf16 [Tt, H] (or [B, T, H]). q and k may have fewer heads
    Hk than v (grouped value heads, H a multiple of Hk: value head h reads
    q/k head h // (H // Hk)). cu_seqlens: int32 [N + 1] (device
    tensor, host list, or None). initial_state: [N, H, 128, 128] or None.
    final_state: a tensor to write the final state into (may be
    initial_state: in-place update); with output_final_state=True and no
    final_state, a new one is allocated. States are fp32, or all bf16
    (state_dtype, default: the dtype of the given state, else fp32).
    no_alloc=True runs kda_prefill_noalloc: the library then allocates
    nothing and uses its static per-device scratch (pass out, and
    final_state if wanted, so that this wrapper allocates nothing either).
    Returns (o, final_state or None).
    """
    import torch
    if q.dim() == 4:
        B, T = q.shape[0], q.shape[1]
        if cu_seqlens is None and cu_seqlens_host is None:
            cu_seqlens_host = [i * T for i in range(B + 1)]
        elif B != 1:
            raise ValueError("4-D inputs with cu_seqlens must have batch size 1")
        flat = lambda x: x.reshape(B * T, *x.shape[2:])
        o, s = prefill(flat(q), flat(k), flat(v), flat(g), flat(beta), cu_seqlens, initial_state,
                       output_final_state, use_intracard_cp, scale, final_state,
                       None if out is None else flat(out), plan, cu_seqlens_host, state_dtype)
        return o.view(v.shape), s
    if q.dim() != 3 or q.shape[-1] != D or v.dim() != 3:
        raise ValueError("q must be [Tt, H, 128] or [B, T, H, 128], got %s" % (tuple(q.shape),))
    Tt, Hk, H = q.shape[0], q.shape[1], v.shape[1]
    if H % Hk:
        raise ValueError("v has %d heads, not a multiple of the %d q/k heads" % (H, Hk))
    beta16 = beta.dtype == torch.bfloat16
    for name, t, dt, shape in (("q", q, torch.bfloat16, (Tt, Hk, D)), ("k", k, torch.bfloat16, (Tt, Hk, D)),
                               ("v", v, torch.bfloat16, (Tt, H, D)), ("g", g, torch.float32, (Tt, H, D)),
                               ("beta", beta, torch.bfloat16 if beta16 else torch.float32, (Tt, H))):
        if t.dtype != dt or tuple(t.shape) != shape or not t.is_contiguous() or not t.is_cuda:
            raise ValueError("%s must be a contiguous %s CUDA tensor of shape %s (got %s %s)"
                             % (name, dt, shape, t.dtype, tuple(t.shape)))
    dev = q.device.index
    if cu_seqlens_host is None:
        if cu_seqlens is None:
            cu_seqlens_host = [0, Tt]
        elif isinstance(cu_seqlens, (list, tuple)):
            cu_seqlens_host = list(cu_seqlens)
        else:
            cu_seqlens_host = cu_seqlens.tolist()  # host copy for the planner (synchronises)
    cu_seqlens_host = [int(x) for x in cu_seqlens_host]
    N = len(cu_seqlens_host) - 1
    # the library sizes every buffer from the plan, so the table must describe
    # exactly the packed tokens the tensors hold
    if (N < 1 or cu_seqlens_host[0] != 0 or cu_seqlens_host[-1] != Tt
            or any(b < a for a, b in zip(cu_seqlens_host, cu_seqlens_host[1:]))):
        raise ValueError("cu_seqlens must start at 0, never decrease and end at the %d packed tokens (got %d "
                         "entries from %s to %s)" % (Tt, N + 1, cu_seqlens_host[0] if N >= 0 else None,
                                                    cu_seqlens_host[-1] if N >= 0 else None))
    if plan is None:
        plan = _cached_plan(cu_seqlens_host, H, _cp_mode(use_intracard_cp), dev)
    else:
        if plan.device != dev:
            raise ValueError("the plan is for device %s, the tensors are on device %d" % (plan.device, dev))
        if plan.shape() != (H, Tt, N) or plan.cu_host != cu_seqlens_host:
            raise ValueError("the plan was built for H=%d, %d tokens, %d sequences (cu_seqlens %s...); the call "
                             "has H=%d, %d tokens, %d sequences" % (*plan.shape(), plan.cu_host[:4], H, Tt, N))
    if cu_seqlens is None or isinstance(cu_seqlens, (list, tuple)):
        cu_dev = plan.cu_device()
    else:
        cu_dev = cu_seqlens
        if cu_dev.dtype != torch.int32 or not cu_dev.is_cuda or cu_dev.numel() != N + 1:
            raise ValueError("cu_seqlens must be an int32 CUDA tensor of %d entries" % (N + 1))
    if state_dtype is None:
        given = initial_state if initial_state is not None else final_state
        state_dtype = given.dtype if given is not None else torch.float32
    if state_dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("states must be fp32 or bf16, got %s" % (state_dtype,))
    for name, t in (("initial_state", initial_state), ("final_state", final_state)):
        if t is not None and (t.dtype != state_dtype or tuple(t.shape) != (N, H, D, D)
                              or not t.is_contiguous() or not t.is_cuda):
            raise ValueError("%s must be a contiguous %s CUDA tensor of shape %s"
                             % (name, state_dtype, (N, H, D, D)))
    if out is None:
        out = torch.empty_like(v)
    if final_state is None and output_final_state:
        final_state = torch.empty(N, H, D, D, dtype=state_dtype, device=q.device)
    ctx = context(q.device)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    if torch.cuda.is_current_stream_capturing() and not any(p is plan for p in _captured_plans):
        _captured_plans.append(plan)
    opts = PrefillOpts(Hk, int(beta16), int(state_dtype == torch.bfloat16))
    entry = lib().kda_prefill_noalloc if no_alloc else lib().kda_prefill_ex
    _check(entry(ctx.handle, plan.handle, ctypes.byref(opts), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                 _ptr(cu_dev), float(scale), _ptr(initial_state), _ptr(final_state), _ptr(out),
                 ctypes.c_void_p(stream)), "kda_prefill_noalloc" if no_alloc else "kda_prefill")
    return out, final_state


def decode(q, k, v, g, beta, state, scale=1.0, out=None, slots=None):
    """KDA decode step: one new token per sequence, state advanced in place.

    q, k, v: bf16 [N, H, 128] (or [N, 1, H, 128]); g: fp32 log-decay, same
    shape as v; beta: fp32 [N, H] (or [N, 1, H]); state: fp32 [N, H, 128, 128],
    overwritten with the advanced state. q and k may have fewer heads than v
    (grouped value heads, as in prefill). With slots (int32 CUDA tensor [N]),
    state is a pool [n_slots, H, 128, 128] and sequence n uses slot slots[n];
    a slot outside the pool skips that sequence (zero output). Returns o,
    shaped like v.
    """
    import torch
    shape = v.shape
    if q.dim() == 4:
        if q.shape[1] != 1:
            raise ValueError("4-D decode inputs must have one token per sequence, got %s" % (tuple(q.shape),))
        sq = lambda x: x.reshape(x.shape[0], *x.shape[2:])
        q, k, v, g, beta = sq(q), sq(k), sq(v), sq(g), sq(beta)
        if out is not None:
            out = sq(out)
    if q.dim() != 3 or q.shape[-1] != D:
        raise ValueError("q must be [N, H, 128] or [N, 1, H, 128], got %s" % (tuple(shape),))
    N, Hk, H = q.shape[0], q.shape[1], v.shape[1]
    if H % Hk:
        raise ValueError("v has %d heads, not a multiple of the %d q/k heads" % (H, Hk))
    for name, t, dt, shp in (("q", q, torch.bfloat16, (N, Hk, D)), ("k", k, torch.bfloat16, (N, Hk, D)),
                             ("v", v, torch.bfloat16, (N, H, D)), ("g", g, torch.float32, (N, H, D)),
                             ("beta", beta, torch.float32, (N, H)),
                             ("state", state, torch.float32, (state.shape[0] if slots is not None else N, H, D, D))):
        if t.dtype != dt or tuple(t.shape) != shp or not t.is_contiguous() or not t.is_cuda:
            raise ValueError("%s must be a contiguous %s CUDA tensor of shape %s (got %s %s)"
                             % (name, dt, shp, t.dtype, tuple(t.shape)))
    if out is None:
        out = torch.empty_like(v)
    ctx = context(q.device)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    if slots is not None:
        if slots.dtype != torch.int32 or tuple(slots.shape) != (N,) or not slots.is_contiguous() or not slots.is_cuda:
            raise ValueError("slots must be a contiguous int32 CUDA tensor of shape (%d,)" % N)
        _check(lib().kda_decode_slots(ctx.handle, N, H, Hk, D, D, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                      float(scale), _ptr(state), state.shape[0], _ptr(slots), _ptr(out),
                                      ctypes.c_void_p(stream)), "kda_decode_slots")
        return out.view(shape)
    _check(lib().kda_decode(ctx.handle, N, H, Hk, D, D, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                            float(scale), _ptr(state), _ptr(out), ctypes.c_void_p(stream)), "kda_decode")
    return out.view(shape)
