"""Python binding of libh2o.so (include/h2o.h): argument marshalling only.

Every step of the decode path runs in the HIP library; this module checks
shapes and dtypes of torch device tensors, passes their pointers and the
current HIP stream, and turns status codes into exceptions.  It fails loudly
when the library has not been built: there is no fallback.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

from .build import LIB

# a test may point the binding at another build of the same sources (a sanitizer build)
LIB = os.environ.get("H2O_LIB") or LIB

H2O_OK, H2O_EINVAL, H2O_ENOMEM, H2O_EDEVICE, H2O_ESTATE = 0, -1, -2, -3, -4
SEL_H2O, SEL_RANDOM, SEL_BLOCK = 0, 1, 2
_SELECTORS = {"h2o": SEL_H2O, "random": SEL_RANDOM, "block": SEL_BLOCK}
F32, BF16, F64, I8, F16 = 0, 1, 2, 3, 4
_STATUS = {H2O_EINVAL: "H2O_EINVAL", H2O_ENOMEM: "H2O_ENOMEM", H2O_EDEVICE: "H2O_EDEVICE",
           H2O_ESTATE: "H2O_ESTATE"}

# Every symbol include/h2o.h declares.
SYMBOLS = ("h2o_workspace_size", "h2o_pool_pages", "h2o_init", "h2o_step", "h2o_compact", "h2o_step_compact", "h2o_read_indices",
           "h2o_info", "h2o_read_kv", "h2o_destroy", "h2o_prefill_scores", "h2o_snapkv_select",
           "h2o_snapkv_select_noalloc", "h2o_last_error")


class H2OConfig(C.Structure):
    _fields_ = [("batch", C.c_int32), ("n_q_heads", C.c_int32), ("n_kv_heads", C.c_int32),
                ("head_dim", C.c_int32), ("kv_dtype", C.c_int32), ("score_dtype", C.c_int32),
                ("scale", C.c_float), ("selector", C.c_int32), ("n_sink", C.c_int32),
                ("budget_fixed", C.c_int32), ("hh_fixed", C.c_int32), ("budget_num", C.c_int32),
                ("budget_den", C.c_int32), ("rand_k", C.c_int32), ("rand_r", C.c_int32),
                ("seed", C.c_uint64), ("page_size", C.c_int32), ("max_pages", C.c_int32),
                ("max_len", C.c_int32), ("workspace", C.c_void_p), ("workspace_bytes", C.c_uint64),
                ("score_decay", C.c_float)]


class H2OError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{_STATUS.get(code, code)}: {msg}")
        self.code = code


_lib = None


def load_library(path: str = LIB):
    """Load libh2o.so (built in-tree by build.py / __graft_entry__.build())."""
    global _lib
    if _lib is not None:
        return _lib
    try:  # load torch's HIP runtime first so the library binds to that same runtime
        import torch  # noqa: F401
    except ImportError:
        pass
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build the HIP library first "
                           "(python -c 'import __graft_entry__ as g; g.build()')")
    lib = C.CDLL(path)
    vp, i32p, f64p = C.c_void_p, C.POINTER(C.c_int32), C.POINTER(C.c_double)
    lib.h2o_workspace_size.restype = C.c_int
    lib.h2o_workspace_size.argtypes = [C.POINTER(H2OConfig), i32p, C.POINTER(C.c_uint64)]
    lib.h2o_pool_pages.restype = C.c_int
    lib.h2o_pool_pages.argtypes = [C.POINTER(H2OConfig), i32p, C.c_int32, i32p]
    lib.h2o_init.restype = C.c_int
    lib.h2o_init.argtypes = [C.POINTER(vp), C.POINTER(H2OConfig), i32p, vp, vp, vp, vp]
    for name in ("h2o_step", "h2o_step_compact"):
        f = getattr(lib, name)
        f.restype = C.c_int
        f.argtypes = [vp, vp, vp, vp, vp, vp]
    lib.h2o_compact.restype = C.c_int
    lib.h2o_compact.argtypes = [vp, vp]
    lib.h2o_read_indices.restype = C.c_int
    lib.h2o_read_indices.argtypes = [vp, i32p, i32p, f64p, f64p, C.c_size_t, vp]
    lib.h2o_read_kv.restype = C.c_int
    lib.h2o_read_kv.argtypes = [vp, vp, vp, vp, vp, C.c_size_t, vp]
    lib.h2o_info.restype = C.c_int
    lib.h2o_info.argtypes = [vp, i32p, i32p, i32p]
    lib.h2o_destroy.restype = None
    lib.h2o_destroy.argtypes = [vp]
    lib.h2o_prefill_scores.restype = C.c_int
    lib.h2o_prefill_scores.argtypes = [C.POINTER(H2OConfig), i32p, vp, vp, vp, vp]
    for name in ("h2o_snapkv_select", "h2o_snapkv_select_noalloc"):
        f = getattr(lib, name)
        f.restype = C.c_int
        f.argtypes = [C.POINTER(H2OConfig), i32p, C.c_int32, C.c_int32, C.c_int32, vp, vp, vp, vp, vp, C.c_int32,
                      vp]
    lib.h2o_last_error.restype = C.c_char_p
    lib.h2o_last_error.argtypes = [vp]
    _lib = lib
    return lib


def make_config(*, batch, n_q_heads, n_kv_heads, head_dim, kv_dtype="bf16", score_dtype="f32",
                scale=0.0, selector="h2o", n_sink=4, budget_fixed=0, hh_fixed=0, budget_num=1,
                budget_den=5, rand_k=0, rand_r=0, seed=0, page_size=0, max_pages=0,
                max_len, score_decay=0.0) -> H2OConfig:
    dt = {"f32": F32, "bf16": BF16, "f64": F64, "i8": I8, "f16": F16}
    return H2OConfig(batch, n_q_heads, n_kv_heads, head_dim, dt[kv_dtype], dt[score_dtype],
                     float(scale), _SELECTORS[selector], n_sink,
                     budget_fixed, hh_fixed, budget_num, budget_den, rand_k, rand_r,
                     int(seed) & 0xFFFFFFFFFFFFFFFF, page_size, max_pages, max_len, None, 0,
                     float(score_decay))


def config_from_workload(w, *, max_len, max_pages=0, **over) -> H2OConfig:
    """Library configuration of a workload (see workloads.Workload)."""
    kw = dict(batch=w.batch, n_q_heads=w.n_q_heads, n_kv_heads=w.n_kv_heads,
              head_dim=w.head_dim, kv_dtype=w.kv_dtype, score_dtype=w.score_dtype,
              selector=w.selector, n_sink=w.n_sink, budget_fixed=w.budget_fixed,
              hh_fixed=w.hh_fixed, budget_num=w.budget_num, budget_den=w.budget_den,
              rand_k=w.rand_k, rand_r=w.rand_r, seed=w.recipe.seed, page_size=w.page_size,
              max_pages=max_pages, max_len=max_len, score_decay=w.score_decay)
    kw.update(over)
    return make_config(**kw)


def pages_needed(prompt_lens, steps: int, cfg: H2OConfig) -> int:
    """Page pool that covers the prompts and `steps` decode steps (h2o_pool_pages)."""
    lib = load_library()
    lens = np.ascontiguousarray(prompt_lens, dtype=np.int32)
    if lens.shape != (cfg.batch,):
        raise ValueError("prompt_lens must have one entry per sequence")
    n = C.c_int32()
    rc = lib.h2o_pool_pages(C.byref(cfg), lens.ctypes.data_as(C.POINTER(C.c_int32)), int(steps), C.byref(n))
    if rc != H2O_OK:
        raise H2OError(rc, lib.h2o_last_error(None).decode(errors="replace"))
    return int(n.value)


def prefill_scores(cfg: H2OConfig, prompt_lens, prompt_q, prompt_k, out=None, stream=None):
    """Prefill-scored initial scores (h2o_prefill_scores): returns out, a cuda float64
    tensor [sum P_b][Hkv] usable as H2OCache's init_scores."""
    import torch
    lib = load_library()
    lens = np.ascontiguousarray(prompt_lens, dtype=np.int32)
    if lens.shape != (cfg.batch,):
        raise ValueError("prompt_lens must have one entry per sequence")
    total = int(lens.sum())
    kv = torch.bfloat16 if cfg.kv_dtype in (BF16, I8) else torch.float32
    H2OCache._check_tensor("prompt_q", prompt_q, (total, cfg.n_q_heads, cfg.head_dim), torch.float32)
    H2OCache._check_tensor("prompt_k", prompt_k, (total, cfg.n_kv_heads, cfg.head_dim), kv)
    if out is None:
        out = torch.empty((total, cfg.n_kv_heads), dtype=torch.float64, device=prompt_q.device)
    H2OCache._check_tensor("out", out, (total, cfg.n_kv_heads), torch.float64)
    rc = lib.h2o_prefill_scores(C.byref(cfg), lens.ctypes.data_as(C.POINTER(C.c_int32)), _ptr(prompt_q),
                                _ptr(prompt_k), _ptr(out), _stream_handle(stream))
    if rc != H2O_OK:
        raise H2OError(rc, lib.h2o_last_error(None).decode(errors="replace"))
    return out


def snapkv_select(cfg: H2OConfig, prompt_lens, prompt_q, prompt_k, window: int, pool: int, keep: int,
                  stream=None):
    """SnapKV's prompt selection (h2o_snapkv_select): returns (kept [B][Hkv][cap] int32
    cuda, ascending, -1 after the count; kept_count [B][Hkv]; votes [sum P][Hq] fp64)."""
    import torch
    lib = load_library()
    lens = np.ascontiguousarray(prompt_lens, dtype=np.int32)
    if lens.shape != (cfg.batch,):
        raise ValueError("prompt_lens must have one entry per sequence")
    total = int(lens.sum())
    kv = torch.bfloat16 if cfg.kv_dtype in (BF16, I8) else torch.float32
    H2OCache._check_tensor("prompt_q", prompt_q, (total, cfg.n_q_heads, cfg.head_dim), torch.float32)
    H2OCache._check_tensor("prompt_k", prompt_k, (total, cfg.n_kv_heads, cfg.head_dim), kv)
    G = cfg.n_q_heads // cfg.n_kv_heads
    cap = max(1, max(min(P, min(window, P) + G * min(keep, P - min(window, P))) for P in lens))
    dev = prompt_q.device
    votes = torch.empty((total, cfg.n_q_heads), dtype=torch.float64, device=dev)
    kept = torch.empty((cfg.batch, cfg.n_kv_heads, cap), dtype=torch.int32, device=dev)
    count = torch.empty((cfg.batch, cfg.n_kv_heads), dtype=torch.int32, device=dev)
    rc = lib.h2o_snapkv_select(C.byref(cfg), lens.ctypes.data_as(C.POINTER(C.c_int32)), int(window),
                               int(pool), int(keep), _ptr(prompt_q), _ptr(prompt_k), _ptr(votes),
                               _ptr(kept), _ptr(count), int(cap), _stream_handle(stream))
    if rc != H2O_OK:
        raise H2OError(rc, lib.h2o_last_error(None).decode(errors="replace"))
    return kept, count, votes


def workspace_size(cfg: H2OConfig, prompt_lens) -> int:
    """Device bytes a context keeps for its state (h2o_workspace_size): the size of
    a caller-provided workspace (see H2OCache's `workspace`)."""
    lib = load_library()
    lens = np.ascontiguousarray(prompt_lens, dtype=np.int32)
    if lens.shape != (cfg.batch,):
        raise ValueError("prompt_lens must have one entry per sequence")
    n = C.c_uint64()
    rc = lib.h2o_workspace_size(C.byref(cfg), lens.ctypes.data_as(C.POINTER(C.c_int32)), C.byref(n))
    if rc != H2O_OK:
        raise H2OError(rc, lib.h2o_last_error(None).decode(errors="replace"))
    return int(n.value)


def _stream_handle(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return C.c_void_p(s.cuda_stream)


def _check(lib, ctx, rc):
    if rc != H2O_OK:
        raise H2OError(rc, lib.h2o_last_error(ctx).decode(errors="replace"))


def _ptr(t):
    return C.c_void_p(t.data_ptr())


class H2OCache:
    """One decode-step context: retained K/V, cumulative scores, positions.

    prompt_k / prompt_v: cuda tensors [sum P_b][Hkv][D] (bfloat16 or float32);
    init_scores: optional cuda float64 [sum P_b][Hkv];
    workspace: optional contiguous cuda uint8 tensor of at least workspace_size(cfg,
    prompt_lens) bytes holding the context's state (kept alive by the cache).
    """

    def __init__(self, cfg: H2OConfig, prompt_lens, prompt_k, prompt_v, init_scores=None,
                 stream=None, workspace=None):
        import torch
        self.lib = load_library()
        self.cfg = cfg
        self.B, self.Hq, self.Hkv, self.D = cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
        self.kv_torch = torch.bfloat16 if cfg.kv_dtype in (BF16, I8) else torch.float32  # inputs
        lens = np.ascontiguousarray(prompt_lens, dtype=np.int32)
        if lens.shape != (self.B,):
            raise ValueError("prompt_lens must have one entry per sequence")
        total = int(lens.sum())
        for name, t in (("prompt_k", prompt_k), ("prompt_v", prompt_v)):
            self._check_tensor(name, t, (total, self.Hkv, self.D), self.kv_torch)
        if init_scores is not None:
            self._check_tensor("init_scores", init_scores, (total, self.Hkv), torch.float64)
        self._ws = None
        if workspace is not None:
            if not (workspace.is_cuda and workspace.dtype == torch.uint8 and workspace.is_contiguous()):
                raise ValueError("workspace: expected a contiguous cuda uint8 tensor")
            cfg = H2OConfig.from_buffer_copy(cfg)
            cfg.workspace = workspace.data_ptr()
            cfg.workspace_bytes = workspace.numel()
            self.cfg = cfg
            self._ws = workspace
        self.ctx = C.c_void_p()
        rc = self.lib.h2o_init(C.byref(self.ctx), C.byref(cfg),
                               lens.ctypes.data_as(C.POINTER(C.c_int32)), _ptr(prompt_k),
                               _ptr(prompt_v), _ptr(init_scores) if init_scores is not None else None,
                               _stream_handle(stream))
        if rc != H2O_OK:
            raise H2OError(rc, self.lib.h2o_last_error(None).decode(errors="replace"))
        self.prompt_lens = lens

    @staticmethod
    def _check_tensor(name, t, shape, dtype):
        if not (t.is_cuda and t.dtype == dtype and tuple(t.shape) == tuple(shape)
                and t.is_contiguous()):
            raise ValueError(f"{name}: expected contiguous cuda {dtype} {tuple(shape)}, got "
                             f"{t.device} {t.dtype} {tuple(t.shape)}")

    def _step_args(self, q, k_new, v_new, out):
        import torch
        self._check_tensor("q", q, (self.B, self.Hq, self.D), torch.float32)
        self._check_tensor("k_new", k_new, (self.B, self.Hkv, self.D), self.kv_torch)
        self._check_tensor("v_new", v_new, (self.B, self.Hkv, self.D), self.kv_torch)
        self._check_tensor("out", out, (self.B, self.Hq, self.D), torch.float32)
        return _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(out)

    def step(self, q, k_new, v_new, out, stream=None):
        """a1-a6; h2o_compact must follow."""
        _check(self.lib, self.ctx, self.lib.h2o_step(self.ctx, *self._step_args(q, k_new, v_new, out),
                                                     _stream_handle(stream)))

    def compact(self, stream=None):
        _check(self.lib, self.ctx, self.lib.h2o_compact(self.ctx, _stream_handle(stream)))

    def step_compact(self, q, k_new, v_new, out, stream=None):
        """a1-a7 in one launch where possible (same result as step + compact)."""
        _check(self.lib, self.ctx,
               self.lib.h2o_step_compact(self.ctx, *self._step_args(q, k_new, v_new, out),
                                         _stream_handle(stream)))

    def info(self):
        cap, steps, pages = C.c_int32(), C.c_int32(), C.c_int32()
        _check(self.lib, self.ctx, self.lib.h2o_info(self.ctx, C.byref(cap), C.byref(steps),
                                                     C.byref(pages)))
        return cap.value, steps.value, pages.value

    def read_indices(self, cap=None, stream=None):
        """(pos [B][Hkv][cap] ascending, count [B], scores [B][Hkv][cap], evicted_mass [B][Hkv])."""
        if cap is None:
            cap = self.info()[0]
        pos = np.empty((self.B, self.Hkv, cap), dtype=np.int32)
        cnt = np.empty(self.B, dtype=np.int32)
        sc = np.empty((self.B, self.Hkv, cap), dtype=np.float64)
        em = np.empty((self.B, self.Hkv), dtype=np.float64)
        rc = self.lib.h2o_read_indices(self.ctx, pos.ctypes.data_as(C.POINTER(C.c_int32)),
                                       cnt.ctypes.data_as(C.POINTER(C.c_int32)),
                                       sc.ctypes.data_as(C.POINTER(C.c_double)),
                                       em.ctypes.data_as(C.POINTER(C.c_double)), cap,
                                       _stream_handle(stream))
        _check(self.lib, self.ctx, rc)
        return pos, cnt, sc, em

    def read_kv(self, cap=None, stream=None):
        """Stored rows of the retained tokens, ascending positions: (K rows, V rows,
        K scales, V scales); rows [B][Hkv][cap][D] as uint16 bf16 bits, float32, or
        int8 codes; scales [B][Hkv][cap] float32 for int8 storage, else None."""
        if cap is None:
            cap = self.info()[0]
        i8 = self.cfg.kv_dtype == I8
        rb = 128 if i8 else 256
        kr = np.empty((self.B, self.Hkv, cap, rb), dtype=np.uint8)
        vr = np.empty_like(kr)
        ks = np.empty((self.B, self.Hkv, cap), dtype=np.float32) if i8 else None
        vs = np.empty_like(ks) if i8 else None
        rc = self.lib.h2o_read_kv(self.ctx, kr.ctypes.data, vr.ctypes.data,
                                  ks.ctypes.data if i8 else None, vs.ctypes.data if i8 else None, cap,
                                  _stream_handle(stream))
        _check(self.lib, self.ctx, rc)
        view = np.int8 if i8 else (np.uint16 if self.cfg.kv_dtype == BF16 else np.float32)
        return kr.view(view), vr.view(view), ks, vs

    def close(self):
        if getattr(self, "ctx", None) and self.ctx.value:
            self.lib.h2o_destroy(self.ctx)
            self.ctx = C.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
