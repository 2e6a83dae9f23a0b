"""ctypes binding of ``include/wf.h``: same names, argument marshalling only.

Every step of a round runs in ``libwf.so`` (HIP kernels for gfx950); this
module only converts Python values and torch tensors to C arguments.  There
is no fallback: if the library is missing, importing raises.
"""

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
# WF_LIBRARY selects another build of the same library (the sanitizer build
# of the CPU ABI tests); by default the in-tree libwf.so.
LIB_PATH = os.environ.get("WF_LIBRARY") or os.path.join(_PKG, "libwf.so")

WF_MAX_STAGES = 8
WF_MAX_GROUPS = WF_MAX_STAGES + 1
WF_MAX_PAGES = 48

WF_OK, WF_EINVAL, WF_ERANGE, WF_EORDER, WF_ESMALL, WF_EDEVICE, WF_EUNSUPPORTED = 0, -1, -2, -3, -4, -5, -6
WF_F32, WF_BF16, WF_FP8, WF_FP8K = 0, 1, 2, 3
WF_MASK_WAVE, WF_MASK_ROLLING = 0, 1
WF_SPLIT_AUTO, WF_SPLIT_OFF, WF_SPLIT_FORCE = 0, 1, 2
WF_KIND_ANCHOR, WF_KIND_HISTORY, WF_KIND_STORE, WF_KIND_DENOISE = 0, 1, 2, 3

i32, i64, u64, f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64, ctypes.c_double


class wf_config(ctypes.Structure):
    _fields_ = [("S", i32), ("W", i32), ("W_store", i32), ("anchor", i32), ("n_chunk", i32),
                ("F", i32), ("Hh", i32), ("Ww", i32), ("n_heads", i32), ("head_dim", i32),
                ("n_layers", i32), ("dtype", i32), ("mask", i32), ("max_frames", i32),
                ("rope_theta", f64), ("softmax_scale", f64)]


class wf_cell(ctypes.Structure):
    _fields_ = [("stage", i32), ("chunk", i32), ("active", i32), ("slot", i32), ("frame0", i32)]


class wf_group(ctypes.Structure):
    _fields_ = [("stage", i32), ("n_pages", i32), ("slot", i32 * WF_MAX_PAGES),
                ("chunk", i32 * WF_MAX_PAGES), ("kind", i32 * WF_MAX_PAGES)]


class wf_anchor(ctypes.Structure):
    _fields_ = [("present", i32), ("slot", i32), ("frame0", i32), ("capture", i32)]


class wf_plan(ctypes.Structure):
    _fields_ = [("k", i64), ("config_hash", u64), ("S", i32), ("n_active", i32),
                ("cells", wf_cell * WF_MAX_GROUPS), ("groups", wf_group * WF_MAX_GROUPS),
                ("anchor", wf_anchor), ("evict_chunk", i32), ("reserved", i32),
                ("kv_tokens", i64), ("flops", f64), ("publish_bytes", f64)]


class wf_layout(ctypes.Structure):
    _fields_ = [(n, i64) for n in
                ("n_slots", "page_bytes", "pool_bytes", "anchor_page_bytes", "anchor_bytes",
                 "tokens", "tokens_padded", "tiles", "vt_offset", "codes_offset", "table_bytes",
                 "split_scratch_offset", "split_scratch_bytes")]


class wf_dit_config(ctypes.Structure):
    _fields_ = [("ffn_dim", i32), ("reserved", i32), ("eps", f64)]


class wf_dit_weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("w_qkv", "b_qkv", "g_q", "g_k", "w_o", "b_o", "w_1", "b_1", "w_2", "b_2")]


class WfError(RuntimeError):
    def __init__(self, status, detail):
        super().__init__(f"{_strerror(status)} ({status}): {detail}")
        self.status = status
        self.detail = detail


def _load():
    # torch ships its own HIP runtime; it must be the one in the process
    # before libwf.so is loaded, or the library's libamdhip64 dependency binds
    # the system copy first and torch then finds no usable device.
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
    lib = ctypes.CDLL(LIB_PATH)
    vp, cvp, sz = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t
    H = ctypes.c_void_p  # opaque wf_handle*
    sig = {
        "wf_strerror": (ctypes.c_char_p, [i32]),
        "wf_last_error": (ctypes.c_char_p, []),
        "wf_create": (i32, [ctypes.POINTER(wf_config), ctypes.POINTER(H)]),
        "wf_destroy": (None, [H]),
        "wf_pool_bytes": (i32, [ctypes.POINTER(wf_config), ctypes.POINTER(sz),
                                ctypes.POINTER(sz), ctypes.POINTER(sz)]),
        "wf_page_layout": (i32, [ctypes.POINTER(wf_config), ctypes.POINTER(wf_layout)]),
        "wf_bind": (i32, [H, vp, sz, vp, sz, vp, sz]),
        "wf_round_plan": (i32, [H, i64, ctypes.POINTER(wf_plan)]),
        "wf_next_round": (i32, [H, ctypes.POINTER(i64)]),
        "wf_reset": (i32, [H]),
        "wf_finish_stream": (i32, [H, i64]),
        "wf_kv_publish": (i32, [H, ctypes.POINTER(wf_plan), i32, cvp, cvp, cvp, vp, vp]),
        "wf_wave_attention": (i32, [H, ctypes.POINTER(wf_plan), i32, cvp, vp, vp]),
        "wf_wave_attention_noalloc": (i32, [H, ctypes.POINTER(wf_plan), i32, cvp, vp, vp]),
        "wf_set_attention_split": (i32, [H, i32]),
        "wf_attention_split_choice": (i32, [H, ctypes.POINTER(wf_plan), ctypes.POINTER(i32),
                                            ctypes.POINTER(i32), ctypes.POINTER(i32)]),
        "wf_round_commit": (i32, [H, ctypes.POINTER(wf_plan)]),
        "wf_round": (i32, [H, ctypes.POINTER(wf_plan), cvp, cvp, cvp, vp, vp, vp]),
        "wf_dit_workspace_bytes": (i32, [H, ctypes.POINTER(wf_dit_config), ctypes.POINTER(sz)]),
        "wf_dit_layer": (i32, [H, ctypes.POINTER(wf_plan), i32, ctypes.POINTER(wf_dit_config),
                               ctypes.POINTER(wf_dit_weights), cvp, vp, vp, sz, vp]),
        "wf_dit_tune": (i32, [H, ctypes.POINTER(wf_dit_config), ctypes.POINTER(wf_dit_weights), vp, sz,
                              vp]),
        "wf_dit_round": (i32, [H, ctypes.POINTER(wf_plan), ctypes.POINTER(wf_dit_config),
                               ctypes.POINTER(wf_dit_weights), cvp, vp, vp, sz, vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()


def _strerror(status):
    return _lib.wf_strerror(status).decode()


def _check(status):
    if status != WF_OK:
        raise WfError(status, _lib.wf_last_error().decode())


def _ptr(t):
    """Device pointer of a tensor (or an int address, or None)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    """hipStream_t handle: a torch stream, an int handle, or torch's current stream."""
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def make_config(S, W, n_chunk, F, Hh, Ww, n_heads, head_dim, n_layers, *, W_store=-1,
                anchor=1, dtype=WF_BF16, mask=WF_MASK_WAVE, rope_theta=0.0, softmax_scale=0.0,
                max_frames=0):
    return wf_config(S=S, W=W, W_store=W_store, anchor=anchor, n_chunk=n_chunk, F=F, Hh=Hh,
                     Ww=Ww, n_heads=n_heads, head_dim=head_dim, n_layers=n_layers, dtype=dtype,
                     mask=mask, max_frames=max_frames, rope_theta=rope_theta,
                     softmax_scale=softmax_scale)


def wf_strerror(status):
    return _strerror(status)


def wf_last_error():
    return _lib.wf_last_error().decode()


def wf_create(cfg):
    h = ctypes.c_void_p()
    _check(_lib.wf_create(ctypes.byref(cfg), ctypes.byref(h)))
    return h


def wf_destroy(h):
    _lib.wf_destroy(h)


def wf_pool_bytes(cfg):
    p, a, t = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    _check(_lib.wf_pool_bytes(ctypes.byref(cfg), ctypes.byref(p), ctypes.byref(a), ctypes.byref(t)))
    return p.value, a.value, t.value


def wf_page_layout(cfg):
    out = wf_layout()
    _check(_lib.wf_page_layout(ctypes.byref(cfg), ctypes.byref(out)))
    return out


def wf_bind(h, pool, pool_bytes, anchor_raw, anchor_bytes, tables, table_bytes):
    _check(_lib.wf_bind(h, _ptr(pool), pool_bytes, _ptr(anchor_raw), anchor_bytes,
                        _ptr(tables), table_bytes))


def wf_round_plan(h, k):
    p = wf_plan()
    _check(_lib.wf_round_plan(h, k, ctypes.byref(p)))
    return p


def wf_next_round(h):
    k = ctypes.c_int64()
    _check(_lib.wf_next_round(h, ctypes.byref(k)))
    return k.value


def wf_reset(h):
    _check(_lib.wf_reset(h))


def wf_finish_stream(h, n_chunk):
    _check(_lib.wf_finish_stream(h, n_chunk))


def wf_kv_publish(h, plan, layer, q, k, v, q_rot, stream=None):
    _check(_lib.wf_kv_publish(h, ctypes.byref(plan), layer, _ptr(q), _ptr(k), _ptr(v),
                              _ptr(q_rot), _stream(stream)))


def wf_wave_attention(h, plan, layer, q_rot, out, stream=None):
    _check(_lib.wf_wave_attention(h, ctypes.byref(plan), layer, _ptr(q_rot), _ptr(out),
                                  _stream(stream)))


def wf_wave_attention_noalloc(h, plan, layer, q_rot, out, stream=None):
    _check(_lib.wf_wave_attention_noalloc(h, ctypes.byref(plan), layer, _ptr(q_rot), _ptr(out),
                                          _stream(stream)))


WF_STATIC_SCRATCH_BYTES = 128 << 20


def wf_set_attention_split(h, mode):
    _check(_lib.wf_set_attention_split(h, mode))


WF_MAX_SPLIT = 2


def wf_attention_split_choice(h, plan):
    """[(stage, at), ...]: the groups wf_wave_attention splits for `plan`
    (pages [0, at) and [at, n) of the group's context)."""
    n = i32()
    stage = (i32 * WF_MAX_SPLIT)()
    at = (i32 * WF_MAX_SPLIT)()
    _check(_lib.wf_attention_split_choice(h, ctypes.byref(plan), ctypes.byref(n), stage, at))
    return [(stage[i], at[i]) for i in range(n.value)]


def wf_round_commit(h, plan):
    _check(_lib.wf_round_commit(h, ctypes.byref(plan)))


def wf_round(h, plan, q, k, v, q_rot, out, stream=None):
    _check(_lib.wf_round(h, ctypes.byref(plan), _ptr(q), _ptr(k), _ptr(v), _ptr(q_rot),
                         _ptr(out), _stream(stream)))


def make_dit_config(ffn_dim, eps=0.0):
    return wf_dit_config(ffn_dim=ffn_dim, reserved=0, eps=eps)


def make_dit_weights(layers):
    """Array of wf_dit_weights from dicts of tensors (one dict per layer)."""
    arr = (wf_dit_weights * len(layers))()
    for i, d in enumerate(layers):
        for n, _ in wf_dit_weights._fields_:
            setattr(arr[i], n, _ptr(d[n]))
    return arr


def wf_dit_workspace_bytes(h, dc):
    b = ctypes.c_size_t()
    _check(_lib.wf_dit_workspace_bytes(h, ctypes.byref(dc), ctypes.byref(b)))
    return b.value


def wf_dit_layer(h, plan, layer, dc, weights, mod, x, work, work_bytes, stream=None):
    """``weights``: a wf_dit_weights (or an array whose element ``layer`` is used)."""
    w = weights[layer] if isinstance(weights, ctypes.Array) else weights
    _check(_lib.wf_dit_layer(h, ctypes.byref(plan), layer, ctypes.byref(dc), ctypes.byref(w),
                             _ptr(mod), _ptr(x), _ptr(work), work_bytes, _stream(stream)))


def wf_dit_tune(h, dc, weights, work, work_bytes, stream=None):
    """``weights``: an array of wf_dit_weights (element 0 is used)."""
    _check(_lib.wf_dit_tune(h, ctypes.byref(dc), weights, _ptr(work), work_bytes, _stream(stream)))


def wf_dit_round(h, plan, dc, weights, mod, x, work, work_bytes, stream=None):
    """``weights``: an array of wf_dit_weights, one per layer."""
    _check(_lib.wf_dit_round(h, ctypes.byref(plan), ctypes.byref(dc), weights, _ptr(mod),
                             _ptr(x), _ptr(work), work_bytes, _stream(stream)))


def status_of(fn, *args, **kw):
    """Call a binding function and return its status code instead of raising."""
    try:
        fn(*args, **kw)
        return WF_OK
    except WfError as e:
        return e.status


def plan_to_dict(p):
    """Plain-Python view of a wf_plan, in the same shape the tests compare."""
    S = p.S
    cells = [dict(stage=c.stage, chunk=c.chunk, active=bool(c.active), slot=c.slot,
                  frame0=c.frame0) for c in p.cells[:S + 1]]
    groups = [dict(stage=g.stage, entries=[(g.kind[i], g.chunk[i], g.slot[i])
                                           for i in range(g.n_pages)]) for g in p.groups[:S + 1]]
    return dict(k=p.k, cells=cells, groups=groups,
                anchor=dict(present=bool(p.anchor.present), slot=p.anchor.slot,
                            frame0=p.anchor.frame0, capture=bool(p.anchor.capture)),
                evict=p.evict_chunk, flops=p.flops, kv_tokens=p.kv_tokens,
                n_active=p.n_active)
