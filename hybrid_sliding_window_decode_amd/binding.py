"""ctypes binding of libhswd.so: argument marshalling only.

Each function takes torch tensors on the GPU, checks dtype, shape and
contiguity, and passes raw device pointers and torch's current stream to the
C entry point of the same name (include/hswd.h).  No arithmetic happens here.
A missing library raises HswdUnavailable on the first call; there is no
fallback path.
"""
import ctypes
import os

import torch

from . import build as _build

F32, F16, BF16, FP8 = 0, 1, 2, 3
_TORCH_CODE = {torch.float32: F32, torch.float16: F16, torch.bfloat16: BF16,
               torch.float8_e4m3fn: FP8}

STATUS = {0: "ok", -1: "invalid argument", -2: "pointer not 16-byte aligned",
          -3: "workspace missing or too small", -4: "position does not fit the cache",
          -5: "HIP runtime error", -6: "unsupported configuration"}
FLAG_CAPACITY, FLAG_MAX_POS, FLAG_NEG_POS = 1, 2, 4


class HswdError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__("%s failed: %s (%d)" % (fn, STATUS.get(status, "unknown"), status))


class HswdUnavailable(ImportError):
    pass


class AttnDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("n_slots", ctypes.c_int32), ("kv_dtype", ctypes.c_int32),
                ("scale", ctypes.c_float), ("keys_per_split", ctypes.c_int32),
                ("chunks_per_workgroup", ctypes.c_int32), ("kv_scale", ctypes.c_void_p)]


_P, _I, _Z, _D = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.c_double
_DP = ctypes.POINTER(AttnDesc)
SIGNATURES = {
    "hswd_version": ([], _I),
    "hswd_status_string": ([_I], ctypes.c_char_p),
    "hswd_workspace_bytes": ([_DP, _I, _I], _Z),
    "hswd_workspace_init": ([_P, _Z, _P], _I),
    "hswd_num_splits": ([_DP, _I, _I], _I),
    "hswd_ring_mask": ([_P, _P, _P, _I, _I, _I, _P], _I),
    "hswd_rope_apply": ([_P, _P, _P, _I, _I, _I, _I, _I, _D, _P], _I),
    "hswd_kv_slot_write": ([_P, _P, _P, _P, _P, _DP, _I, _P, _P, _P], _I),
    "hswd_decode_attn_sliding": ([_P, _P, _P, _P, _P, _P, _P, _DP, _P, _Z, _P], _I),
    "hswd_decode_attn_full": ([_P, _P, _P, _P, _P, _P, _P, _I, _DP, _P, _Z, _P], _I),
    "hswd_decode_attn_partials": ([_P, _P, _P, _P, _P, _P, _I, _I, _DP, _P], _I),
    "hswd_lse_merge": ([_P, _P, _P, _I, _I, _I, _I, _P], _I),
    "hswd_head_gate": ([_P, _P, _P, _I, _I, _I, _P], _I),
    "hswd_layer_step": ([_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _D, _I, _DP, _P, _Z, _P], _I),
    "hswd_layer_step_noalloc": ([_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _D, _I, _DP, _P, _P],
                                _I),
    "hswd_check_errors": ([_P, ctypes.POINTER(ctypes.c_int32), _P], _I),
    "hswd_gate_proj": ([_P, _P, _P, _I, _I, _I, _P], _I),
    "hswd_layer_step_gproj": ([_P, _P, _P, _P, _P, _P, _I, _P, _P, _P, _I, _I, _D, _I, _DP, _P,
                               _Z, _P], _I),
}

# include/hswd_measure.h, the measurement library beside libhswd.so
MEASURE_SIGNATURES = {
    "hswd_measure_stream_read": ([_P, _Z, _P, _I, _P], _I),
}

_lib = None
_measure_lib = None


def library_path():
    return os.environ.get("HSWD_LIBRARY", _build.LIB)


def measure_library_path():
    """libhswd_measure.so beside the loaded libhswd.so."""
    return os.path.join(os.path.dirname(os.path.abspath(library_path())),
                        os.path.basename(_build.MEASURE_LIB))


def lib():
    """The loaded libhswd.so (loaded once)."""
    global _lib
    if _lib is None:
        path = library_path()
        if not os.path.exists(path):
            raise HswdUnavailable("libhswd.so is not built (%s); run "
                                  "python -m hybrid_sliding_window_decode_amd.build" % path)
        L = ctypes.CDLL(path)
        for name, (args, res) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def measure_lib():
    """The loaded libhswd_measure.so (loaded once)."""
    global _measure_lib
    if _measure_lib is None:
        path = measure_library_path()
        if not os.path.exists(path):
            raise HswdUnavailable("libhswd_measure.so is not built (%s); run "
                                  "python -m hybrid_sliding_window_decode_amd.build" % path)
        L = ctypes.CDLL(path)
        for name, (args, res) in MEASURE_SIGNATURES.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _measure_lib = L
    return _measure_lib


def _check(fn, status):
    if status != 0:
        raise HswdError(fn, status)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _need(t, name, dtype=None, shape=None):
    if not t.is_cuda:
        raise ValueError("%s must be a CUDA (HIP) tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise ValueError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))


def make_desc(k_cache, n_heads=None, scale=None, keys_per_split=0, chunks_per_workgroup=0,
              kv_scale=None):
    """Descriptor of a layer from its cache tensor [B, Hkv, n_slots, D].

    kv_scale: for a float8_e4m3fn cache, a float32 device tensor [2, Hkv] of
    per-head K and V scales (the caller keeps it alive while the descriptor
    is in use)."""
    B, Hkv, S, D = k_cache.shape
    if k_cache.dtype not in _TORCH_CODE:
        raise ValueError("cache dtype must be float32, float16, bfloat16 or float8_e4m3fn")
    H = Hkv if n_heads is None else n_heads
    sc = (1.0 / D ** 0.5) if scale is None else float(scale)
    ptr = None
    if kv_scale is not None:
        _need(kv_scale, "kv_scale", torch.float32, (2, Hkv))
        ptr = kv_scale.data_ptr()
    return AttnDesc(B, H, Hkv, D, S, _TORCH_CODE[k_cache.dtype], sc, keys_per_split,
                    chunks_per_workgroup, ptr)


def version():
    return lib().hswd_version()


def status_string(status):
    return lib().hswd_status_string(status).decode()


def workspace_bytes(desc, ring, max_pos=0):
    return lib().hswd_workspace_bytes(ctypes.byref(desc), int(ring), int(max_pos))


def num_splits(desc, ring, max_pos=0):
    n = lib().hswd_num_splits(ctypes.byref(desc), int(ring), int(max_pos))
    _check("hswd_num_splits", n if n < 0 else 0)
    return n


def workspace(desc, ring, max_pos=0, device="cuda"):
    """A zeroed workspace tensor (uint8) sized for this layer."""
    n = workspace_bytes(desc, ring, max_pos)
    if n == 0:
        raise HswdError("hswd_workspace_bytes", -1)
    ws = torch.empty(n, dtype=torch.uint8, device=device)
    workspace_init(ws)
    return ws


def workspace_init(ws):
    _need(ws, "ws")
    _check("hswd_workspace_init", lib().hswd_workspace_init(_ptr(ws), ws.numel(), _stream()))


def ring_mask(pos, n_slots, ring):
    """(mask uint8 [B, n_slots], slot int32 [B]) of positions `pos`."""
    _need(pos, "pos", torch.int32)
    B = pos.numel()
    mask = torch.empty(B, n_slots, dtype=torch.uint8, device=pos.device)
    slot = torch.empty(B, dtype=torch.int32, device=pos.device)
    _check("hswd_ring_mask", lib().hswd_ring_mask(_ptr(mask), _ptr(slot), _ptr(pos), B, n_slots,
                                                  int(ring), _stream()))
    return mask, slot


def rope_apply(q, k, pos, rot_dim, theta):
    """RoPE in place on q [B,H,D] and k [B,Hkv,D] (k may be None)."""
    _need(q, "q", torch.float32)
    _need(pos, "pos", torch.int32)
    B, H, D = q.shape
    Hkv = 0
    if k is not None:
        _need(k, "k", torch.float32)
        if k.shape[0] != B or k.shape[2] != D:
            raise ValueError("k shape %s does not match q %s" % (tuple(k.shape), tuple(q.shape)))
        Hkv = k.shape[1]
    if pos.numel() != B:
        raise ValueError("pos must have B entries")
    _check("hswd_rope_apply", lib().hswd_rope_apply(_ptr(q), _ptr(k), _ptr(pos), B, H, Hkv, D,
                                                    int(rot_dim), float(theta), _stream()))
    return q, k


def _cache_pair(k_cache, v_cache):
    _need(k_cache, "k_cache")
    _need(v_cache, "v_cache", k_cache.dtype, k_cache.shape)


def check_desc(desc, k_cache, n_heads):
    """A caller-supplied descriptor must describe the tensors passed with it:
    the library addresses every cache row, query and output from the
    descriptor alone, so a stale one (another batch, cache or head count)
    would read and write outside the tensors."""
    if k_cache.dim() != 4:
        raise ValueError("k_cache must be [B, Hkv, n_slots, D], got %s" % (tuple(k_cache.shape),))
    B, Hkv, S, D = k_cache.shape
    code = _TORCH_CODE.get(k_cache.dtype)
    want = dict(batch=B, n_heads=n_heads, n_kv_heads=Hkv, head_dim=D, n_slots=S, kv_dtype=code)
    for name, value in want.items():
        if getattr(desc, name) != value:
            raise ValueError("desc.%s = %d does not match the tensors (%s)"
                             % (name, getattr(desc, name), value))


def kv_slot_write(k_cache, v_cache, k_rot, v, pos, ring, ws, slot_out=None, desc=None):
    if desc is not None:
        check_desc(desc, k_cache, desc.n_heads)
    _cache_pair(k_cache, v_cache)
    B, Hkv, S, D = k_cache.shape
    _need(k_rot, "k_rot", torch.float32, (B, Hkv, D))
    _need(v, "v", torch.float32, (B, Hkv, D))
    _need(pos, "pos", torch.int32, (B,))
    if slot_out is not None:
        _need(slot_out, "slot_out", torch.int32, (B,))
    d = desc or make_desc(k_cache)
    _check("hswd_kv_slot_write", lib().hswd_kv_slot_write(
        _ptr(k_cache), _ptr(v_cache), _ptr(k_rot), _ptr(v), _ptr(pos), ctypes.byref(d),
        int(ring), _ptr(slot_out), _ptr(ws), _stream()))
    return slot_out


def _attn_args(q, k, v, k_cache, v_cache, pos, desc):
    if desc is not None:
        check_desc(desc, k_cache, q.shape[1])
    _cache_pair(k_cache, v_cache)
    B, Hkv, S, D = k_cache.shape
    H = q.shape[1]
    _need(q, "q", torch.float32, (B, H, D))
    _need(k, "k", torch.float32, (B, Hkv, D))
    _need(v, "v", torch.float32, (B, Hkv, D))
    _need(pos, "pos", torch.int32, (B,))
    return desc or make_desc(k_cache, n_heads=H)


def decode_attn_sliding(q_rot, k_rot, v, k_ring, v_ring, pos, ws, out=None, desc=None):
    d = _attn_args(q_rot, k_rot, v, k_ring, v_ring, pos, desc)
    out = torch.empty_like(q_rot) if out is None else out
    _need(out, "out", torch.float32, q_rot.shape)
    _need(ws, "ws")
    _check("hswd_decode_attn_sliding", lib().hswd_decode_attn_sliding(
        _ptr(out), _ptr(q_rot), _ptr(k_rot), _ptr(v), _ptr(k_ring), _ptr(v_ring), _ptr(pos),
        ctypes.byref(d), _ptr(ws), ws.numel(), _stream()))
    return out


def decode_attn_full(q_rot, k_rot, v, k_cache, v_cache, pos, max_pos, ws, out=None, desc=None):
    d = _attn_args(q_rot, k_rot, v, k_cache, v_cache, pos, desc)
    out = torch.empty_like(q_rot) if out is None else out
    _need(out, "out", torch.float32, q_rot.shape)
    _need(ws, "ws")
    _check("hswd_decode_attn_full", lib().hswd_decode_attn_full(
        _ptr(out), _ptr(q_rot), _ptr(k_rot), _ptr(v), _ptr(k_cache), _ptr(v_cache), _ptr(pos),
        int(max_pos), ctypes.byref(d), _ptr(ws), ws.numel(), _stream()))
    return out


def decode_attn_partials(q_rot, k_cache, v_cache, pos, ring, max_pos=0, desc=None):
    """(part_o [B,H,n,D], part_ml [B,H,n,2]) of the cached keys alone."""
    if desc is not None:
        check_desc(desc, k_cache, q_rot.shape[1])
    _cache_pair(k_cache, v_cache)
    B, Hkv, S, D = k_cache.shape
    H = q_rot.shape[1]
    _need(q_rot, "q_rot", torch.float32, (B, H, D))
    _need(pos, "pos", torch.int32, (B,))
    d = desc or make_desc(k_cache, n_heads=H)
    n = num_splits(d, ring, max_pos)
    part_o = torch.empty(B, H, n, D, dtype=torch.float32, device=q_rot.device)
    part_ml = torch.empty(B, H, n, 2, dtype=torch.float32, device=q_rot.device)
    _check("hswd_decode_attn_partials", lib().hswd_decode_attn_partials(
        _ptr(part_o), _ptr(part_ml), _ptr(q_rot), _ptr(k_cache), _ptr(v_cache), _ptr(pos),
        int(ring), int(max_pos), ctypes.byref(d), _stream()))
    return part_o, part_ml


def lse_merge(part_o, part_ml, out=None):
    _need(part_o, "part_o", torch.float32)
    B, H, n, D = part_o.shape
    _need(part_ml, "part_ml", torch.float32, (B, H, n, 2))
    out = torch.empty(B, H, D, dtype=torch.float32, device=part_o.device) if out is None else out
    _need(out, "out", torch.float32, (B, H, D))
    _check("hswd_lse_merge", lib().hswd_lse_merge(_ptr(out), _ptr(part_o), _ptr(part_ml), B, H, D,
                                                  n, _stream()))
    return out


def head_gate(o, gate, out=None):
    _need(o, "o", torch.float32)
    B, H, D = o.shape
    _need(gate, "gate", torch.float32, (B, H))
    out = torch.empty_like(o) if out is None else out
    _need(out, "out", torch.float32, o.shape)
    _check("hswd_head_gate", lib().hswd_head_gate(_ptr(out), _ptr(o), _ptr(gate), B, H, D,
                                                  _stream()))
    return out


class BoundCall:
    """One library entry point with its arguments marshalled once: calling it
    launches on the stream that was current when it was bound and returns the
    output tensor.  For loops that issue the same launch many times (a decode
    step per layer), so each launch costs one foreign call.  It holds
    references to the tensors and the descriptor it was bound with, so their
    memory stays valid while it exists; their contents are read at each
    launch."""

    def __init__(self, name, fn, args, out, keep=()):
        self.name, self._fn, self._args, self.out = name, fn, args, out
        self._keep = tuple(keep)

    def __call__(self):
        status = self._fn(*self._args)
        if status != 0:
            raise HswdError(self.name, status)
        return self.out


def _layer_step_args(q, k, v, gate, k_cache, v_cache, pos, ring, rot_dim, theta, ws, max_pos,
                     out, desc):
    d = _attn_args(q, k, v, k_cache, v_cache, pos, desc)
    if gate is not None:
        _need(gate, "gate", torch.float32, (q.shape[0], q.shape[1]))
    out = torch.empty_like(q) if out is None else out
    _need(out, "out", torch.float32, q.shape)
    _need(ws, "ws")
    return out, (_ptr(out), _ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(k_cache),
                 _ptr(v_cache), _ptr(pos), int(ring), int(rot_dim), float(theta), int(max_pos),
                 ctypes.byref(d), _ptr(ws), ws.numel(), _stream())


def layer_step(q, k, v, gate, k_cache, v_cache, pos, ring, rot_dim, theta, ws, max_pos=0,
               out=None, desc=None):
    """Whole layer step in one launch; returns the gated output [B,H,D]."""
    out, args = _layer_step_args(q, k, v, gate, k_cache, v_cache, pos, ring, rot_dim, theta,
                                 ws, max_pos, out, desc)
    _check("hswd_layer_step", lib().hswd_layer_step(*args))
    return out


NOALLOC_SCRATCH_BYTES = 32 << 20       # HSWD_NOALLOC_SCRATCH_BYTES


def layer_step_noalloc(q, k, v, gate, k_cache, v_cache, pos, ring, rot_dim, theta, max_pos=0,
                       out=None, desc=None, err=None):
    """layer_step with the library's own per-GPU workspace (no workspace
    argument; the call allocates nothing when `out` is given).  err: an
    optional int32 device tensor of one element into which the error flags
    are OR-ed (read with check_errors(err)).  Calls that overlap in time on
    one GPU share that workspace and must be serialised."""
    d = _attn_args(q, k, v, k_cache, v_cache, pos, desc)
    if gate is not None:
        _need(gate, "gate", torch.float32, (q.shape[0], q.shape[1]))
    if err is not None:
        _need(err, "err", torch.int32)
    out = torch.empty_like(q) if out is None else out
    _need(out, "out", torch.float32, q.shape)
    _check("hswd_layer_step_noalloc", lib().hswd_layer_step_noalloc(
        _ptr(out), _ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(k_cache), _ptr(v_cache),
        _ptr(pos), int(ring), int(rot_dim), float(theta), int(max_pos), ctypes.byref(d),
        _ptr(err), _stream()))
    return out


def bind_layer_step(q, k, v, gate, k_cache, v_cache, pos, ring, rot_dim, theta, ws, max_pos=0,
                    out=None, desc=None):
    """layer_step with its arguments checked and marshalled once (BoundCall)."""
    out, args = _layer_step_args(q, k, v, gate, k_cache, v_cache, pos, ring, rot_dim, theta,
                                 ws, max_pos, out, desc)
    return BoundCall("hswd_layer_step", lib().hswd_layer_step, args, out,
                     keep=(q, k, v, gate, k_cache, v_cache, pos, ws, desc))


def gate_proj(x, w_g, out=None):
    """Gate logits [B, H] = x [B, hidden] @ w_g[H, hidden].T (float32)."""
    _need(x, "x", torch.float32)
    B, hidden = x.shape
    _need(w_g, "w_g", torch.float32)
    if w_g.dim() != 2 or w_g.shape[1] != hidden:
        raise ValueError("w_g must be [H, hidden]")
    H = w_g.shape[0]
    out = torch.empty(B, H, dtype=torch.float32, device=x.device) if out is None else out
    _need(out, "out", torch.float32, (B, H))
    _check("hswd_gate_proj", lib().hswd_gate_proj(_ptr(out), _ptr(x), _ptr(w_g), B, hidden, H,
                                                  _stream()))
    return out


def _layer_step_gproj_args(q, k, v, x, w_g, k_cache, v_cache, pos, ring, rot_dim, theta, ws,
                           max_pos, out, desc):
    d = _attn_args(q, k, v, k_cache, v_cache, pos, desc)
    B, H = q.shape[0], q.shape[1]
    _need(x, "x", torch.float32)
    hidden = x.shape[1]
    _need(x, "x", torch.float32, (B, hidden))
    _need(w_g, "w_g", torch.float32, (H, hidden))
    out = torch.empty_like(q) if out is None else out
    _need(out, "out", torch.float32, q.shape)
    _need(ws, "ws")
    return out, (_ptr(out), _ptr(q), _ptr(k), _ptr(v), _ptr(x), _ptr(w_g), hidden,
                 _ptr(k_cache), _ptr(v_cache), _ptr(pos), int(ring), int(rot_dim), float(theta),
                 int(max_pos), ctypes.byref(d), _ptr(ws), ws.numel(), _stream())


def layer_step_gproj(q, k, v, x, w_g, k_cache, v_cache, pos, ring, rot_dim, theta, ws,
                     max_pos=0, out=None, desc=None):
    """Layer step with the gate logits projected from x [B, hidden] by w_g [H, hidden]."""
    out, args = _layer_step_gproj_args(q, k, v, x, w_g, k_cache, v_cache, pos, ring, rot_dim,
                                       theta, ws, max_pos, out, desc)
    _check("hswd_layer_step_gproj", lib().hswd_layer_step_gproj(*args))
    return out


def bind_layer_step_gproj(q, k, v, x, w_g, k_cache, v_cache, pos, ring, rot_dim, theta, ws,
                          max_pos=0, out=None, desc=None):
    """layer_step_gproj with its arguments checked and marshalled once (BoundCall)."""
    out, args = _layer_step_gproj_args(q, k, v, x, w_g, k_cache, v_cache, pos, ring, rot_dim,
                                       theta, ws, max_pos, out, desc)
    return BoundCall("hswd_layer_step_gproj", lib().hswd_layer_step_gproj, args, out,
                     keep=(q, k, v, x, w_g, k_cache, v_cache, pos, ws, desc))


def check_errors(ws):
    """Synchronise and return the workspace's HSWD_FLAG_* bits."""
    flags = ctypes.c_int32(0)
    st = lib().hswd_check_errors(_ptr(ws), ctypes.byref(flags), _stream())
    if st not in (0, -4):
        raise HswdError("hswd_check_errors", st)
    return flags.value


def stream_read(buf, workgroups=2048, sink=None):
    """Read a device buffer once (the measurement library's
    hswd_measure_stream_read).  Returns the sink tensor [workgroups] int32
    (never written in practice)."""
    _need(buf, "buf")
    nbytes = buf.numel() * buf.element_size()
    if sink is None:
        sink = torch.zeros(workgroups, dtype=torch.int32, device=buf.device)
    _need(sink, "sink", torch.int32)
    if sink.numel() < workgroups:
        raise ValueError("sink must hold at least `workgroups` int32 values")
    _check("hswd_measure_stream_read",
           measure_lib().hswd_measure_stream_read(_ptr(buf), nbytes, _ptr(sink),
                                                  int(workgroups), _stream()))
    return sink
