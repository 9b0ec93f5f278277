"""ctypes binding of libsegmla (include/segmla.h): argument marshalling only.

Functions carry the C names. Host arrays are numpy arrays; device buffers are torch
tensors on the GPU (PyTorch provides device memory and streams only). Every call
raises SegmlaError on a non-OK status; nothing here computes any part of the method.
The library must be built (__graft_entry__.build()); loading fails loudly otherwise.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsegmla.so")

SEGMLA_OK = 0
SEGMLA_E_NULL, SEGMLA_E_GEOMETRY, SEGMLA_E_SHAPE, SEGMLA_E_DTYPE = -1, -2, -3, -4
SEGMLA_E_PROTECT, SEGMLA_E_WORKSPACE, SEGMLA_E_HIP, SEGMLA_E_UNSUPPORTED, SEGMLA_E_STATE = (
    -5, -6, -7, -8, -9)
SEGMLA_SEG_PREFIX, SEGMLA_SEG_DOC, SEGMLA_SEG_NEW = 0, 1, 2
SEGMLA_F32, SEGMLA_BF16, SEGMLA_E4M3_B128 = 0, 1, 2

EXPORTED = [
    "segmla_plan_create", "segmla_plan_workspace_bytes", "segmla_plan_rows", "segmla_plan_build",
    "segmla_forward", "segmla_copy_protected", "segmla_copy_geometry", "segmla_lse_merge",
    "segmla_plan_pairs", "segmla_ledger", "segmla_plan_destroy", "segmla_status_string",
    "segmla_abi_version", "segmla_profile_enable", "segmla_profile_read",
    "segmla_plan_create_range", "segmla_plan_create_paged", "segmla_plan_get_info",
    "segmla_forward_noalloc", "segmla_plan_set_window", "segmla_prefetcher_create",
    "segmla_prefetch", "segmla_prefetch_wait", "segmla_prefetch_elapsed",
    "segmla_prefetcher_destroy", "segmla_dual_create", "segmla_dual_sizes", "segmla_dual_build",
    "segmla_dual_forward", "segmla_dual_destroy",
]

NOALLOC_MAX_BYTES = 96 << 20  # SEGMLA_NOALLOC_MAX_BYTES


class SegmlaError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__("%s: %s (status %d)" % (what, _status_string(status), status))


class Pages(ctypes.Structure):
    _fields_ = [("page_rows", ctypes.c_int32), ("n_entries", ctypes.c_int64),
                ("page_start", ctypes.POINTER(ctypes.c_int64)),
                ("page_table", ctypes.POINTER(ctypes.c_int64))]


class Geometry(ctypes.Structure):
    _fields_ = [("n_seg", ctypes.c_int32), ("pool_row", ctypes.POINTER(ctypes.c_int64)),
                ("len", ctypes.POINTER(ctypes.c_int32)), ("offset", ctypes.POINTER(ctypes.c_int64)),
                ("kind", ctypes.POINTER(ctypes.c_uint8))]


class Layer(ctypes.Structure):
    _fields_ = [("n_heads", ctypes.c_int32), ("d_nope", ctypes.c_int32), ("d_rope", ctypes.c_int32),
                ("d_state", ctypes.c_int32), ("v_has_rope", ctypes.c_int32),
                ("head_is_global", ctypes.POINTER(ctypes.c_uint8)), ("rope_base", ctypes.c_double),
                ("softmax_scale", ctypes.c_float), ("kv_dtype", ctypes.c_int32),
                ("io_dtype", ctypes.c_int32), ("split_keys", ctypes.c_int32),
                ("group_heads", ctypes.c_int32), ("n_sink", ctypes.c_int32),
                ("window", ctypes.c_int32), ("z_e4m3", ctypes.c_int32)]


class Protect(ctypes.Structure):
    _fields_ = [("edge_rows", ctypes.c_int32), ("tail_rows", ctypes.c_int32),
                ("budget_permille", ctypes.c_int32), ("n_dirty", ctypes.c_int32),
                ("dirty_rows", ctypes.POINTER(ctypes.c_int32))]


class Tensors(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("kv", ctypes.c_void_p), ("kv_scale", ctypes.c_void_p),
                ("kv_rope", ctypes.c_void_p), ("w", ctypes.c_void_p), ("z_cached", ctypes.c_void_p),
                ("out", ctypes.c_void_p), ("z", ctypes.c_void_p), ("lse", ctypes.c_void_p),
                ("z_scale", ctypes.c_void_p)]


class CopyRange(ctypes.Structure):
    _fields_ = [("src", ctypes.c_void_p), ("dst", ctypes.c_void_p), ("rows", ctypes.c_int64),
                ("row_bytes", ctypes.c_int64), ("src_stride", ctypes.c_int64),
                ("dst_stride", ctypes.c_int64)]


class DualPool(ctypes.Structure):
    _fields_ = [("ratio", ctypes.c_int32), ("window", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("n_cpool", ctypes.c_int64), ("cpool_row", ctypes.c_void_p)]


class DualTensors(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("q", "kv", "ckv", "cidx", "clen", "out", "lse")]


class PlanInfo(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("q_begin", ctypes.c_int64), ("q_end", ctypes.c_int64),
                ("n_pool", ctypes.c_int64), ("n_protected", ctypes.c_int64),
                ("workspace_bytes", ctypes.c_int64), ("n_heads", ctypes.c_int32),
                ("n_global", ctypes.c_int32), ("n_local", ctypes.c_int32),
                ("n_window", ctypes.c_int32),
                ("d_nope", ctypes.c_int32), ("d_rope", ctypes.c_int32), ("d_v", ctypes.c_int32),
                ("d_state", ctypes.c_int32), ("z_slots", ctypes.c_int32),
                ("zc_slots", ctypes.c_int32), ("kv_dtype", ctypes.c_int32),
                ("io_dtype", ctypes.c_int32), ("n_split", ctypes.c_int32),
                ("z_e4m3", ctypes.c_int32)]


_lib = None


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libsegmla.so is not built at %s; run __graft_entry__.build()" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        i32, i64, dbl = ctypes.c_int32, ctypes.c_int64, ctypes.c_double
        sig = {
            "segmla_plan_create": (i32, [ctypes.POINTER(Geometry), ctypes.POINTER(Layer),
                                         ctypes.POINTER(Protect), i64, ctypes.POINTER(P)]),
            "segmla_plan_create_range": (i32, [ctypes.POINTER(Geometry), ctypes.POINTER(Layer),
                                               ctypes.POINTER(Protect), i64, i64, i64,
                                               ctypes.POINTER(P)]),
            "segmla_plan_create_paged": (i32, [ctypes.POINTER(Geometry), ctypes.POINTER(Pages),
                                               ctypes.POINTER(Layer), ctypes.POINTER(Protect), i64,
                                               i64, i64, ctypes.POINTER(P)]),
            "segmla_plan_workspace_bytes": (i32, [P, ctypes.POINTER(ctypes.c_size_t)]),
            "segmla_plan_rows": (i32, [P, ctypes.POINTER(i64), ctypes.POINTER(i64)]),
            "segmla_plan_get_info": (i32, [P, ctypes.POINTER(PlanInfo)]),
            "segmla_plan_set_window": (i32, [P, i64, i64, P]),
            "segmla_prefetcher_create": (i32, [ctypes.POINTER(P)]),
            "segmla_prefetch": (i32, [P, ctypes.POINTER(CopyRange), i32, P]),
            "segmla_prefetch_wait": (i32, [P, P]),
            "segmla_prefetch_elapsed": (i32, [P, ctypes.POINTER(ctypes.c_float)]),
            "segmla_prefetcher_destroy": (None, [P]),
            "segmla_plan_build": (i32, [P, P, ctypes.c_size_t, P, P]),
            "segmla_forward": (i32, [P, ctypes.POINTER(Tensors), P]),
            "segmla_forward_noalloc": (i32, [P, P, ctypes.POINTER(Tensors), P]),
            "segmla_copy_protected": (i32, [P, ctypes.POINTER(i32), i64, P]),
            "segmla_copy_geometry": (i32, [P, ctypes.POINTER(i32), ctypes.POINTER(i64), i64, P]),
            "segmla_lse_merge": (i32, [P, P, i32, i64, i32, P, i32, P, P]),
            "segmla_plan_pairs": (i32, [P, ctypes.POINTER(dbl), P]),
            "segmla_ledger": (i32, [i32, i32, i32, i32, i32, i64, i64, dbl, dbl, ctypes.POINTER(dbl)]),
            "segmla_plan_destroy": (None, [P]),
            "segmla_status_string": (ctypes.c_char_p, [i32]),
            "segmla_abi_version": (i32, []),
            "segmla_profile_enable": (i32, [P, i32]),
            "segmla_profile_read": (i32, [P, ctypes.POINTER(dbl), ctypes.POINTER(i64),
                                          ctypes.POINTER(i64)]),
            "segmla_dual_create": (i32, [P, ctypes.POINTER(DualPool), ctypes.POINTER(P)]),
            "segmla_dual_sizes": (i32, [P, ctypes.POINTER(ctypes.c_size_t), ctypes.POINTER(i64)]),
            "segmla_dual_build": (i32, [P, P, ctypes.c_size_t, P]),
            "segmla_dual_forward": (i32, [P, ctypes.POINTER(DualTensors), P]),
            "segmla_dual_destroy": (None, [P]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _status_string(status):
    try:
        return lib().segmla_status_string(int(status)).decode()
    except Exception:  # library missing while formatting an error
        return "status"


def _check(status, what):
    if status != SEGMLA_OK:
        raise SegmlaError(status, what)


def _ptr(t):
    """Device (or host) address of a torch tensor, or None."""
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        import torch
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return ctypes.c_void_p(int(stream))


def _arr(a, dtype):
    return np.ascontiguousarray(np.asarray(a, dtype=dtype))


def _torch_dtypes(code):
    """torch dtypes a tensor of segmla_dtype `code` may have (E4M3 codes: bytes)."""
    import torch
    return {SEGMLA_F32: (torch.float32,), SEGMLA_BF16: (torch.bfloat16,),
            SEGMLA_E4M3_B128: (torch.uint8, torch.float8_e4m3fn)}[code]


def _check_tensors(specs):
    """specs: (name, tensor, dtypes, numel, required). Raise ValueError unless every given
    tensor is a contiguous GPU tensor of one of its dtypes with at least `numel` elements. The
    C ABI sees only raw addresses, so this is the last place where a host tensor, a wrong dtype
    or an undersized buffer can be caught before a kernel reads or writes past it. Types,
    dtypes and sizes of all tensors are checked before any device."""
    import torch
    given = []
    for name, t, dtypes, numel, required in specs:
        if t is None:
            if required:
                raise ValueError("%s is required" % name)
            continue
        if not torch.is_tensor(t):
            raise ValueError("%s must be a torch tensor, got %s" % (name, type(t).__name__))
        if t.dtype not in dtypes:
            raise ValueError("%s has dtype %s, expected %s"
                             % (name, t.dtype, " or ".join(map(str, dtypes))))
        if not t.is_contiguous():
            raise ValueError("%s must be contiguous" % name)
        if t.numel() < numel:
            raise ValueError("%s holds %d elements, the plan needs %d" % (name, t.numel(), numel))
        given.append((name, t))
    for name, t in given:
        if t.device.type != "cuda":
            raise ValueError("%s must be on the GPU, got device %s" % (name, t.device))


# ------------------------------------------------------------------- C entry points
def segmla_abi_version():
    return int(lib().segmla_abi_version())


def segmla_status_string(status):
    return _status_string(status)


def segmla_plan_create(kinds, lens, offsets, pool_rows, n_pool, n_heads, head_is_global, d_nope,
                       d_rope, d_state, v_has_rope=1, rope_base=10000.0, softmax_scale=1.0,
                       kv_dtype=SEGMLA_BF16, io_dtype=SEGMLA_BF16, split_keys=0, edge_rows=0,
                       tail_rows=0, budget_permille=0, dirty_rows=(), q_range=None, pages=None,
                       group_heads=0, n_sink=0, window=0, z_e4m3=0):
    """Validate and size a plan; returns the plan handle. q_range = (q_begin, q_end): a plan
    for that window of request rows (segmla_plan_create_range); None: the whole request.
    pages = dict(page_rows, page_start, page_table): a paged latent pool
    (segmla_plan_create_paged; pool_rows is then ignored)."""
    keep = dict(kind=_arr(kinds, np.uint8), len=_arr(lens, np.int32), offset=_arr(offsets, np.int64),
                pool=_arr(pool_rows, np.int64), glob=_arr(head_is_global, np.uint8),
                dirty=_arr(list(dirty_rows), np.int32))
    g = Geometry(len(keep["kind"]), keep["pool"].ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                 keep["len"].ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                 keep["offset"].ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                 keep["kind"].ctypes.data_as(ctypes.POINTER(ctypes.c_uint8)))
    L = Layer(n_heads, d_nope, d_rope, d_state, v_has_rope,
              keep["glob"].ctypes.data_as(ctypes.POINTER(ctypes.c_uint8)), rope_base, softmax_scale,
              kv_dtype, io_dtype, split_keys, group_heads, n_sink, window, z_e4m3)
    pr = Protect(edge_rows, tail_rows, budget_permille, len(keep["dirty"]),
                 keep["dirty"].ctypes.data_as(ctypes.POINTER(ctypes.c_int32)) if len(keep["dirty"])
                 else None)
    h = ctypes.c_void_p()
    if pages is not None:
        keep["pstart"] = _arr(pages["page_start"], np.int64)
        keep["ptable"] = _arr(pages["page_table"], np.int64)
        pg = Pages(int(pages["page_rows"]), len(keep["ptable"]),
                   keep["pstart"].ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                   keep["ptable"].ctypes.data_as(ctypes.POINTER(ctypes.c_int64)))
        q0, q1 = (0, -1) if q_range is None else (int(q_range[0]), int(q_range[1]))
        _check(lib().segmla_plan_create_paged(ctypes.byref(g), ctypes.byref(pg), ctypes.byref(L),
                                              ctypes.byref(pr), int(n_pool), q0, q1,
                                              ctypes.byref(h)), "segmla_plan_create_paged")
    elif q_range is None:
        _check(lib().segmla_plan_create(ctypes.byref(g), ctypes.byref(L), ctypes.byref(pr),
                                        int(n_pool), ctypes.byref(h)), "segmla_plan_create")
    else:
        _check(lib().segmla_plan_create_range(ctypes.byref(g), ctypes.byref(L), ctypes.byref(pr),
                                              int(n_pool), int(q_range[0]), int(q_range[1]),
                                              ctypes.byref(h)), "segmla_plan_create_range")
    return h


def segmla_plan_workspace_bytes(plan):
    n = ctypes.c_size_t()
    _check(lib().segmla_plan_workspace_bytes(plan, ctypes.byref(n)), "segmla_plan_workspace_bytes")
    return int(n.value)


def segmla_plan_rows(plan):
    T, nA = ctypes.c_int64(), ctypes.c_int64()
    _check(lib().segmla_plan_rows(plan, ctypes.byref(T), ctypes.byref(nA)), "segmla_plan_rows")
    return int(T.value), int(nA.value)


def segmla_plan_get_info(plan):
    """The plan's shapes (segmla_plan_info) as a dict."""
    info = PlanInfo()
    _check(lib().segmla_plan_get_info(plan, ctypes.byref(info)), "segmla_plan_get_info")
    return {name: int(getattr(info, name)) for name, _ in PlanInfo._fields_}


def segmla_plan_set_window(plan, q_begin, q_end, stream=None):
    _check(lib().segmla_plan_set_window(plan, int(q_begin), int(q_end), _stream(stream)),
           "segmla_plan_set_window")


def segmla_plan_build(plan, workspace, indexer_score=None, stream=None):
    import torch
    info = segmla_plan_get_info(plan)
    _check_tensors([("workspace", workspace, (torch.uint8,), info["workspace_bytes"], True),
                    ("indexer_score", indexer_score, (torch.int32, torch.uint32), info["T"], False)])
    nbytes = workspace.numel() * workspace.element_size()
    _check(lib().segmla_plan_build(plan, _ptr(workspace), nbytes, _ptr(indexer_score),
                                   _stream(stream)), "segmla_plan_build")


def check_forward_tensors(info, q, kv, w, out, z, z_cached=None, kv_scale=None, kv_rope=None,
                          lse=None, z_scale=None):
    """Validate the tensors of one forward against a plan's shapes (segmla_plan_get_info)."""
    import torch
    io = _torch_dtypes(info["io_dtype"])
    nq = info["q_end"] - info["q_begin"]
    H, dn, dr, dv, ds = (info[k] for k in ("n_heads", "d_nope", "d_rope", "d_v", "d_state"))
    n_pool = info["n_pool"]
    specs = [("q", q, io, nq * H * (dn + dr), True)]
    if info["kv_dtype"] == SEGMLA_E4M3_B128:
        specs += [("kv", kv, _torch_dtypes(SEGMLA_E4M3_B128), n_pool * dn, True),
                  ("kv_scale", kv_scale, (torch.float32,), n_pool * (dn // 128), True),
                  ("kv_rope", kv_rope, (torch.bfloat16,), n_pool * dr, True)]
    else:
        specs += [("kv", kv, _torch_dtypes(info["kv_dtype"]), n_pool * (dn + dr), True)]
    specs += [("w", w, io, H * ds * dv, True),
              ("z_cached", z_cached, io, n_pool * info["zc_slots"] * ds, info["n_local"] > 0),
              ("out", out, io, nq * H * dv, True),
              ("z", z, (torch.uint8,) if info["z_e4m3"] else io, nq * info["z_slots"] * ds, True),
              ("lse", lse, (torch.float32,), nq * H, False)]
    if info["z_e4m3"]:
        specs.append(("z_scale", z_scale, (torch.float32,), nq * info["z_slots"] * (ds // 128), True))
    elif z_scale is not None:
        raise ValueError("z_scale is given but the plan's z is not E4M3")
    _check_tensors(specs)


def segmla_forward(plan, q, kv, w, out, z, z_cached=None, kv_scale=None, kv_rope=None, lse=None,
                   stream=None, z_scale=None):
    check_forward_tensors(segmla_plan_get_info(plan), q, kv, w, out, z, z_cached, kv_scale,
                          kv_rope, lse, z_scale)
    t = Tensors(_ptr(q), _ptr(kv), _ptr(kv_scale), _ptr(kv_rope), _ptr(w), _ptr(z_cached), _ptr(out),
                _ptr(z), _ptr(lse), _ptr(z_scale))
    _check(lib().segmla_forward(plan, ctypes.byref(t), _stream(stream)), "segmla_forward")


def segmla_forward_noalloc(plan, indexer_score, q, kv, w, out, z, z_cached=None, kv_scale=None,
                           kv_rope=None, lse=None, stream=None, z_scale=None):
    """Plan build + forward with the workspace in the library's own device array (no device
    memory allocated anywhere in the call)."""
    import torch
    info = segmla_plan_get_info(plan)
    _check_tensors([("indexer_score", indexer_score, (torch.int32, torch.uint32), info["T"], False)])
    check_forward_tensors(info, q, kv, w, out, z, z_cached, kv_scale, kv_rope, lse, z_scale)
    t = Tensors(_ptr(q), _ptr(kv), _ptr(kv_scale), _ptr(kv_rope), _ptr(w), _ptr(z_cached), _ptr(out),
                _ptr(z), _ptr(lse), _ptr(z_scale))
    _check(lib().segmla_forward_noalloc(plan, _ptr(indexer_score), ctypes.byref(t), _stream(stream)),
           "segmla_forward_noalloc")


def segmla_copy_protected(plan, n_protected, stream=None):
    buf = np.empty(max(1, n_protected), dtype=np.int32)
    _check(lib().segmla_copy_protected(plan, buf.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                       len(buf), _stream(stream)), "segmla_copy_protected")
    return buf[:n_protected]


def segmla_copy_geometry(plan, T, stream=None):
    seg = np.empty(T, dtype=np.int32)
    pool = np.empty(T, dtype=np.int64)
    _check(lib().segmla_copy_geometry(plan, seg.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                      pool.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), T,
                                      _stream(stream)), "segmla_copy_geometry")
    return seg, pool


def segmla_lse_merge(partial_o, partial_ml, out, lse=None, stream=None):
    """partial_o fp32 [n_split, n_vec, d], partial_ml fp32 [n_split, n_vec, 2] (device tensors)."""
    import torch
    if not torch.is_tensor(partial_o) or partial_o.dim() != 3:
        raise ValueError("partial_o must be a [n_split, n_vec, d] tensor")
    n_split, n_vec, d = partial_o.shape
    _check_tensors([("partial_o", partial_o, (torch.float32,), n_split * n_vec * d, True),
                    ("partial_ml", partial_ml, (torch.float32,), n_split * n_vec * 2, True),
                    ("out", out, (torch.float32, torch.bfloat16), n_vec * d, True),
                    ("lse", lse, (torch.float32,), n_vec, False)])
    dt = SEGMLA_F32 if out.dtype == torch.float32 else SEGMLA_BF16
    _check(lib().segmla_lse_merge(_ptr(partial_o), _ptr(partial_ml), n_split, n_vec, d, _ptr(out), dt,
                                  _ptr(lse), _stream(stream)), "segmla_lse_merge")


def segmla_plan_pairs(plan, stream=None):
    """(Global, Local, sink + window) counts of computed (row, head, key) triples."""
    out = (ctypes.c_double * 3)()
    _check(lib().segmla_plan_pairs(plan, out, _stream(stream)), "segmla_plan_pairs")
    return float(out[0]), float(out[1]), float(out[2])


def segmla_ledger(f_front, r, f_back, h, h_local, T, n_protected, global_pairs=-1.0,
                  local_pairs=-1.0):
    out = (ctypes.c_double * 3)()
    _check(lib().segmla_ledger(f_front, r, f_back, h, h_local, T, n_protected, global_pairs,
                               local_pairs, out), "segmla_ledger")
    return tuple(float(x) for x in out)


def segmla_profile_enable(plan, enable=True):
    _check(lib().segmla_profile_enable(plan, 1 if enable else 0), "segmla_profile_enable")


def segmla_profile_read(plan):
    """Accumulated ms per stage: (attention, split merge, epilogue, build), n_forward, n_build."""
    ms = (ctypes.c_double * 4)()
    nf, nb = ctypes.c_int64(), ctypes.c_int64()
    _check(lib().segmla_profile_read(plan, ms, ctypes.byref(nf), ctypes.byref(nb)),
           "segmla_profile_read")
    return tuple(float(x) for x in ms), int(nf.value), int(nb.value)


def segmla_plan_destroy(plan):
    if plan:
        lib().segmla_plan_destroy(plan)


class Prefetcher:
    """Staging of a later layer's artifact rows on the library's own stream (segmla_prefetch*).

    prefetch(pairs): each pair (src, dst) of tensors of one dtype and shape, rows along dim 0,
    each row contiguous; src on the GPU or in pinned host memory, dst on the GPU. The transfers
    start after the work already enqueued on `after_stream` (default: torch's current stream)
    and run beside what is enqueued there next; wait(stream) orders `stream` after them."""

    def __init__(self):
        h = ctypes.c_void_p()
        _check(lib().segmla_prefetcher_create(ctypes.byref(h)), "segmla_prefetcher_create")
        self.handle = h
        self._keep = None

    @staticmethod
    def _range(src, dst):
        import torch
        if not (torch.is_tensor(src) and torch.is_tensor(dst)):
            raise ValueError("prefetch pairs are (src, dst) tensors")
        if src.dtype != dst.dtype or src.shape != dst.shape or src.dim() < 1:
            raise ValueError("src and dst must share dtype and shape, got %s %s and %s %s"
                             % (src.dtype, tuple(src.shape), dst.dtype, tuple(dst.shape)))
        if dst.device.type != "cuda":
            raise ValueError("dst must be on the GPU")
        if src.device.type != "cuda" and not src.is_pinned():
            raise ValueError("src must be on the GPU or in pinned host memory")
        rows = src.shape[0]
        if rows and not (src[0].is_contiguous() and dst[0].is_contiguous()):
            raise ValueError("each row must be contiguous")
        es = src.element_size()
        row_bytes = max(1, src[0].numel() * es) if rows else 1
        return CopyRange(src.data_ptr(), dst.data_ptr(), rows, row_bytes,
                         src.stride(0) * es if rows > 1 else row_bytes,
                         dst.stride(0) * es if rows > 1 else row_bytes)

    def prefetch(self, pairs, after_stream=None):
        ranges = [self._range(s, d) for s, d in pairs]
        arr = (CopyRange * max(1, len(ranges)))(*ranges)
        self._keep = (pairs, arr)  # the tensors stay alive until the next prefetch
        _check(lib().segmla_prefetch(self.handle, arr, len(ranges), _stream(after_stream)),
               "segmla_prefetch")

    def wait(self, stream=None):
        _check(lib().segmla_prefetch_wait(self.handle, _stream(stream)), "segmla_prefetch_wait")

    def elapsed_ms(self):
        ms = ctypes.c_float()
        _check(lib().segmla_prefetch_elapsed(self.handle, ctypes.byref(ms)), "segmla_prefetch_elapsed")
        return float(ms.value)

    def close(self):
        if self.handle:
            lib().segmla_prefetcher_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def segmla_dual_create(plan, ratio, window, top_k, cpool_rows, n_cpool):
    rows = _arr(cpool_rows, np.int64)
    dp = DualPool(int(ratio), int(window), int(top_k), int(n_cpool),
                  rows.ctypes.data_as(ctypes.c_void_p))
    h = ctypes.c_void_p()
    _check(lib().segmla_dual_create(plan, ctypes.byref(dp), ctypes.byref(h)), "segmla_dual_create")
    return h


def segmla_dual_sizes(dual):
    nb, ne = ctypes.c_size_t(), ctypes.c_int64()
    _check(lib().segmla_dual_sizes(dual, ctypes.byref(nb), ctypes.byref(ne)), "segmla_dual_sizes")
    return int(nb.value), int(ne.value)


def segmla_dual_build(dual, workspace, stream=None):
    import torch
    need, _ = segmla_dual_sizes(dual)
    _check_tensors([("workspace", workspace, (torch.uint8,), need, True)])
    _check(lib().segmla_dual_build(dual, _ptr(workspace), workspace.numel(), _stream(stream)),
           "segmla_dual_build")


def check_dual_tensors(info, top_k, n_cpool, q, kv, ckv, out, cidx=None, clen=None, lse=None):
    """Validate the tensors of one dual-pool forward against the plan's shapes."""
    import torch
    nq = info["q_end"] - info["q_begin"]
    H, dqk, dv = info["n_heads"], info["d_nope"] + info["d_rope"], info["d_v"]
    bf = (torch.bfloat16,)
    specs = [("q", q, bf, nq * H * dqk, True), ("kv", kv, bf, info["n_pool"] * dqk, True),
             ("ckv", ckv, bf, n_cpool * dqk, True), ("out", out, bf, nq * H * dv, True),
             ("lse", lse, (torch.float32,), nq * H, False)]
    if top_k > 0:
        specs += [("cidx", cidx, (torch.int32,), nq * top_k, True),
                  ("clen", clen, (torch.int32,), nq, True)]
    elif cidx is not None or clen is not None:
        raise ValueError("cidx / clen are given but the layer takes every available entry (top_k = 0)")
    _check_tensors(specs)


def segmla_dual_forward(dual, info, top_k, n_cpool, q, kv, ckv, out, cidx=None, clen=None,
                        lse=None, stream=None):
    check_dual_tensors(info, top_k, n_cpool, q, kv, ckv, out, cidx, clen, lse)
    t = DualTensors(_ptr(q), _ptr(kv), _ptr(ckv), _ptr(cidx), _ptr(clen), _ptr(out), _ptr(lse))
    _check(lib().segmla_dual_forward(dual, ctypes.byref(t), _stream(stream)), "segmla_dual_forward")


def segmla_dual_destroy(dual):
    if dual:
        lib().segmla_dual_destroy(dual)


class Dual:
    """Compressed-history (dual-pool) attention on a plan (segmla_dual_*), with the workspace
    of its entry tables (torch uint8 tensor on the current GPU). The plan must outlive it."""

    def __init__(self, plan, ratio, window, top_k, cpool_rows, n_cpool):
        self.plan, self.top_k, self.n_cpool = plan, int(top_k), int(n_cpool)
        self.handle = segmla_dual_create(plan.handle, ratio, window, top_k, cpool_rows, n_cpool)
        self.ws_bytes, self.n_entries = segmla_dual_sizes(self.handle)
        self.workspace = None

    def build(self, stream=None):
        import torch
        self.workspace = torch.empty(max(256, self.ws_bytes), dtype=torch.uint8, device="cuda")
        segmla_dual_build(self.handle, self.workspace, stream)

    def forward(self, q, kv, ckv, out, cidx=None, clen=None, lse=None, stream=None):
        """q, out, lse, cidx and clen: the rows of the plan's window."""
        segmla_dual_forward(self.handle, segmla_plan_get_info(self.plan.handle), self.top_k,
                            self.n_cpool, q, kv, ckv, out, cidx, clen, lse, stream)

    def close(self):
        if self.handle:
            segmla_dual_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @classmethod
    def for_inputs(cls, plan, dual_inp):
        return cls(plan, dual_inp["ratio"], dual_inp["window"], dual_inp["top_k"],
                   dual_inp["cpool_rows"], dual_inp["n_cpool"])


# ------------------------------------------------------------------ convenience
_DT = {"f32": SEGMLA_F32, "bf16": SEGMLA_BF16, "e4m3": SEGMLA_E4M3_B128}


class Plan:
    """A plan plus its device workspace (torch uint8 tensor on the current GPU)."""

    def __init__(self, cfg, kinds, lens, offsets, pool_rows, n_pool, head_is_global, split_keys=0,
                 dirty_rows=(), q_range=None, pages=None):
        d_v = cfg["d_nope"] + cfg["d_rope"] if cfg["v_has_rope"] else cfg["d_nope"]
        self.cfg, self.d_v = cfg, d_v
        self.handle = segmla_plan_create(
            kinds, lens, offsets, pool_rows, n_pool, cfg["n_heads"], head_is_global, cfg["d_nope"],
            cfg["d_rope"], cfg["d_state"], cfg["v_has_rope"], cfg["rope_base"], cfg["softmax_scale"],
            _DT[cfg["kv_dtype"]], _DT[cfg["dtype"]], split_keys, cfg["edge_rows"], cfg["tail_rows"],
            cfg["budget_permille"], dirty_rows, q_range, pages, cfg.get("group_heads", 0),
            cfg.get("n_sink", 0), cfg.get("window", 0), cfg.get("z_e4m3", 0))
        self.T, self.n_protected = segmla_plan_rows(self.handle)
        # computed window: q, out, z and lse hold rows q0 .. q1 - 1
        self.q0, self.q1 = (0, self.T) if q_range is None else (int(q_range[0]), int(q_range[1]))
        self.workspace = None

    def build(self, scores=None, stream=None, min_bytes=0):
        """Build into a workspace of at least the plan's need, or of min_bytes when larger (room
        for the larger windows that set_window may move the plan to)."""
        import torch
        nbytes = max(segmla_plan_workspace_bytes(self.handle), int(min_bytes))
        if self.workspace is None or self.workspace.numel() < nbytes:
            self.workspace = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        segmla_plan_build(self.handle, self.workspace, scores, stream)

    def forward(self, inp, out, z, lse=None, stream=None, z_scale=None):
        """out, z, lse (and z_scale for an E4M3 state): the window's rows. inp["q"] may hold
        the whole request (its window rows are passed, a view) or the window only."""
        q = inp["q"]
        if q.shape[0] != self.q1 - self.q0:
            q = q[self.q0:self.q1]
        segmla_forward(self.handle, q, inp["kv"], inp["w"], out, z, inp.get("z_cached"),
                       inp.get("kv_scale"), inp.get("kv_rope"), lse, stream, z_scale)

    def set_window(self, q_begin, q_end, stream=None):
        """Another window of the same request on the built plan (segmla_plan_set_window)."""
        segmla_plan_set_window(self.handle, q_begin, q_end, stream)
        self.q0, self.q1 = int(q_begin), int(self.T if q_end == -1 else q_end)

    def protected(self):
        return segmla_copy_protected(self.handle, self.n_protected)

    def geometry(self):
        return segmla_copy_geometry(self.handle, self.T)

    def pairs(self):
        return segmla_plan_pairs(self.handle)

    def close(self):
        if self.handle:
            segmla_plan_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @classmethod
    def for_inputs(cls, inp, split_keys=0, q_range=None):
        return cls(inp["cfg"], inp["kinds"], inp["lens"], inp["offsets"], inp["pool_rows"],
                   inp["n_pool"], inp["head_is_global"], split_keys, inp["cfg"].get("dirty_rows", ()),
                   q_range, inp.get("pages"))
