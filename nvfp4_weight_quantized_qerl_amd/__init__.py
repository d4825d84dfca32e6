"""NVFP4 weight-only linear layer with LoRA and AQN noise for MI355X.

Python binding of libqerl.so (C ABI: include/qerl.h).  Each function has
the name of the C call it wraps and does argument marshalling only: it
checks devices, dtypes and shapes (the C ABI receives raw pointers and
cannot), allocates outputs with torch, passes raw device pointers and
torch's current HIP stream, and raises QerlError on a non-zero status.
Every step of the computation runs in the HIP kernels.

`bind_linear` marshals the arguments of one linear call once and returns a
callable that re-issues it, for callers that repeat the same call many times
(every layer of every decode step).
"""
import ctypes

import torch

from . import _lib

lib = _lib.load()

QERL_OK = 0


class QerlError(RuntimeError):
    def __init__(self, status, call):
        self.status = int(status)
        msg = lib.qerl_status_string(self.status).decode()
        super().__init__(f"{call}: {msg}")


def _check(status, call):
    if status != QERL_OK:
        raise QerlError(status, call)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _bits16(t, name):
    """bf16 tensor (or its uint16/int16 bit view) -> int16 view, contiguous."""
    if t.dtype == torch.bfloat16:
        t = t.view(torch.int16)
    elif t.dtype not in (torch.int16, torch.uint16):
        raise TypeError(f"{name} must be bfloat16 (or its 16-bit pattern)")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    return t.contiguous()


def _need(t, name, dtype, shape, device):
    """Check a tensor argument that goes to the library as a raw pointer."""
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    dts = dtype if isinstance(dtype, tuple) else (dtype,)
    if t.dtype not in dts:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {' or '.join(map(str, dts))}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


_BF16 = (torch.bfloat16, torch.int16, torch.uint16)


def _check_linear_args(m, n, k, r, dev, codes, scales, gscale, lora_a=None, lora_b=None, z=None,
                       y=None):
    _need(codes, "codes", torch.uint8, (n, k // 2), dev)      # None: checked by the caller
    _need(scales, "scales", torch.uint8, (n, k // 16), dev)
    if not isinstance(gscale, torch.Tensor) or gscale.dtype != torch.float32 or \
            gscale.numel() < 1 or gscale.device != dev:
        raise TypeError("gscale must be a float32 device tensor with at least one element")
    if lora_a is not None:
        _need(lora_a, "lora_a", _BF16, (r, k), dev)
    if lora_b is not None:
        _need(lora_b, "lora_b", _BF16, (n, r), dev)
    _need(z, "z", torch.float32, (k,), dev)
    _need(y, "y", _BF16, (m, n), dev)


def qerl_abi_version():
    return lib.qerl_abi_version()


def qerl_quantize_nvfp4(w):
    """bf16 W [n, k] -> (codes uint8 [n, k/2], scales uint8 [n, k/16],
    gscale float32 [1], nonfinite int32 [1]) on W's device."""
    w = _bits16(w, "w")
    n, k = w.shape
    dev = w.device
    codes = torch.empty((n, k // 2), dtype=torch.uint8, device=dev)
    scales = torch.empty((n, k // 16), dtype=torch.uint8, device=dev)
    gscale = torch.empty(1, dtype=torch.float32, device=dev)
    flag = torch.empty(1, dtype=torch.int32, device=dev)
    _check(lib.qerl_quantize_nvfp4(_ptr(w), n, k, _ptr(codes), _ptr(scales), _ptr(gscale),
                                   _ptr(flag), _stream(dev)), "qerl_quantize_nvfp4")
    return codes, scales, gscale, flag


def _quantize_batch_args(ws, outs):
    """Host pointer arrays of qerl_quantize_nvfp4_batch for the bf16 weights
    `ws` and their outputs `outs` [(codes, scales, gscale, flag or None)]."""
    if not ws or len(ws) != len(outs):
        raise ValueError("qerl_quantize_nvfp4_batch: one output tuple per weight, at least one")
    cnt = len(ws)
    ws = [_bits16(w, "w") for w in ws]
    dev = ws[0].device
    for w, (codes, scales, gscale, flag) in zip(ws, outs):
        n, k = w.shape
        if w.device != dev:
            raise ValueError("qerl_quantize_nvfp4_batch: every tensor on one device")
        _need(codes, "codes", torch.uint8, (n, k // 2), dev)
        _need(scales, "scales", torch.uint8, (n, k // 16), dev)
        _need(gscale, "gscale", torch.float32, (1,), dev)
        _need(flag, "flag", torch.int32, (1,), dev)
    ptrs = lambda ts: (ctypes.c_void_p * cnt)(*[None if t is None else t.data_ptr() for t in ts])
    arrays = (ptrs(ws), (ctypes.c_int64 * cnt)(*[w.shape[0] for w in ws]),
              (ctypes.c_int64 * cnt)(*[w.shape[1] for w in ws]),
              ptrs([o[0] for o in outs]), ptrs([o[1] for o in outs]), ptrs([o[2] for o in outs]),
              ptrs([o[3] for o in outs]))
    args = (cnt,) + tuple(ctypes.cast(a, ctypes.c_void_p) for a in arrays) + (_stream(dev),)
    return args, (ws, outs, arrays)


def qerl_quantize_nvfp4_batch(ws):
    """qerl_quantize_nvfp4 of every bf16 weight in the list `ws` in one call
    (count + 2 launches); returns [(codes, scales, gscale, nonfinite)]."""
    outs = []
    for w in ws:
        n, k = w.shape
        dev = w.device
        outs.append((torch.empty((n, k // 2), dtype=torch.uint8, device=dev),
                     torch.empty((n, k // 16), dtype=torch.uint8, device=dev),
                     torch.empty(1, dtype=torch.float32, device=dev),
                     torch.empty(1, dtype=torch.int32, device=dev)))
    args, keep = _quantize_batch_args(ws, outs)
    _check(lib.qerl_quantize_nvfp4_batch(*args), "qerl_quantize_nvfp4_batch")
    return outs


def bind_quantize_nvfp4_batch(ws, outs):
    """A BoundCall of qerl_quantize_nvfp4_batch into preallocated outputs
    [(codes, scales, gscale, flag or None)], one tuple per weight in `ws`."""
    args, keep = _quantize_batch_args(ws, outs)
    return BoundCall("qerl_quantize_nvfp4_batch", args, keep, outs)


def bind_quantize_nvfp4(w, codes, scales, gscale, flag=None):
    """A BoundCall of qerl_quantize_nvfp4 into preallocated outputs (codes
    uint8 [n, k/2], scales uint8 [n, k/16], gscale float32 [1], flag int32 [1]
    or None); its result is (codes, scales, gscale, flag)."""
    w = _bits16(w, "w")
    n, k = w.shape
    dev = w.device
    _need(codes, "codes", torch.uint8, (n, k // 2), dev)
    _need(scales, "scales", torch.uint8, (n, k // 16), dev)
    _need(gscale, "gscale", torch.float32, (1,), dev)
    _need(flag, "flag", torch.int32, (1,), dev)
    args = (_ptr(w), n, k, _ptr(codes), _ptr(scales), _ptr(gscale), _ptr(flag), _stream(dev))
    return BoundCall("qerl_quantize_nvfp4", args, (w, codes, scales, gscale, flag),
                     (codes, scales, gscale, flag))


def qerl_aqn_sigma(sigma_start, sigma_end, num_stages, stage):
    out = ctypes.c_double(0.0)
    _check(lib.qerl_aqn_sigma(sigma_start, sigma_end, num_stages, stage, ctypes.byref(out)),
           "qerl_aqn_sigma")
    return out.value


SCHEDULES = {"exponential": 0, "linear": 1, "cosine": 2, "logarithmic": 3}


def qerl_aqn_sigma_schedule(mode, sigma_start, sigma_end, num_stages, stage):
    """sigma at stage k of K under the named decay schedule (host)."""
    out = ctypes.c_double()
    _check(lib.qerl_aqn_sigma_schedule(SCHEDULES[mode], sigma_start, sigma_end, num_stages,
                                       stage, ctypes.byref(out)), "qerl_aqn_sigma_schedule")
    return out.value


def qerl_aqn_sample(seed, stream_id, call_id, sigma, d, device="cuda", out=None, stream=None):
    """stream: a torch.cuda.Stream to enqueue on (default: the current one)."""
    z = out if out is not None else torch.empty(d, dtype=torch.float32, device=device)
    hs = _stream(z.device) if stream is None else ctypes.c_void_p(stream.cuda_stream)
    _check(lib.qerl_aqn_sample(seed, stream_id, call_id, sigma, d, _ptr(z), hs),
           "qerl_aqn_sample")
    return z


def qerl_aqn_sample_batch(seed, stream_id, call_id0, call_stride, count, sigma, d,
                          device="cuda", out=None):
    """z [count, d]: row i is qerl_aqn_sample(seed, stream_id,
    call_id0 + i * call_stride, sigma, d)."""
    z = out if out is not None else torch.empty((count, d), dtype=torch.float32, device=device)
    _check(lib.qerl_aqn_sample_batch(seed, stream_id, call_id0, call_stride, count, sigma, d,
                                     _ptr(z), _stream(z.device)), "qerl_aqn_sample_batch")
    return z


def qerl_aqn_sample_rows(seed, stream_id, call_id, sigma, m, d, device="cuda", out=None):
    """z [m, d], one noise row per token; row 0 is qerl_aqn_sample's vector."""
    z = out if out is not None else torch.empty((m, d), dtype=torch.float32, device=device)
    _check(lib.qerl_aqn_sample_rows(seed, stream_id, call_id, sigma, m, d, _ptr(z),
                                    _stream(z.device)), "qerl_aqn_sample_rows")
    return z


def qerl_attention_stub(qkv, n_q_heads, n_kv_heads, head_dim, out=None):
    """Attention over a context of one position: each query head outputs the
    value of its key/value head, out [m, n_q_heads * head_dim]."""
    qkv = _bits16(qkv, "qkv")
    m, width = qkv.shape
    if width != (n_q_heads + 2 * n_kv_heads) * head_dim:
        raise ValueError("qkv width must be (n_q_heads + 2 n_kv_heads) head_dim")
    if out is None:
        out = torch.empty((m, n_q_heads * head_dim), dtype=torch.bfloat16, device=qkv.device)
    _need(out, "out", _BF16, (m, n_q_heads * head_dim), qkv.device)
    _check(lib.qerl_attention_stub(_ptr(qkv), m, n_q_heads, n_kv_heads, head_dim, _ptr(out),
                                   _stream(qkv.device)), "qerl_attention_stub")
    return out


def qerl_rmsnorm_noisy(x, w, z=None, delta=1e-6, out=None):
    """y = bf16((w + z) * x / sqrt(mean(x^2) + delta)) per row of x [m, d]."""
    x = _bits16(x, "x")
    w = _bits16(w, "w")
    m, d = x.shape
    if out is None:
        out = torch.empty((m, d), dtype=torch.bfloat16, device=x.device)
    _check(lib.qerl_rmsnorm_noisy(_ptr(x), m, d, _ptr(w), _ptr(z), float(delta), _ptr(out),
                                  _stream(x.device)), "qerl_rmsnorm_noisy")
    return out


def qerl_swiglu(gate_up, out=None):
    """bf16(SiLU(gate) * up) from the fused gate/up output [m, 2 d]."""
    gu = _bits16(gate_up, "gate_up")
    m, d2 = gu.shape
    if d2 % 2:
        raise ValueError("gate_up must have an even number of columns")
    if out is None:
        out = torch.empty((m, d2 // 2), dtype=torch.bfloat16, device=gu.device)
    _check(lib.qerl_swiglu(_ptr(gu), m, d2 // 2, _ptr(out), _stream(gu.device)), "qerl_swiglu")
    return out


def qerl_linear_workspace_bytes(m, n, k, r):
    return int(lib.qerl_linear_workspace_bytes(m, n, k, r))


def workspace(m, n, k, r, device="cuda"):
    """A device workspace of the size qerl_linear_workspace_bytes asks for."""
    nbytes = qerl_linear_workspace_bytes(m, n, k, r)
    if nbytes == 0:
        raise ValueError("invalid linear sizes")
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def _linear_args(fn_name, x, codes, scales, gscale, lora_a, lora_b, lora_scale, z, ws, y,
                 gate_up=False, z_rows=False):
    """Checked C arguments of a whole linear call (and its output y)."""
    x = _bits16(x, "x")
    if x.dim() != 2:
        raise ValueError("x must be 2-D [m, k]")
    m, k = x.shape
    if gate_up:
        if k % 2:
            raise ValueError("gate_up needs an even number of columns")
        k //= 2
    n = codes.shape[0]
    r = 0 if lora_a is None else int(lora_a.shape[0])
    la = None if lora_a is None else _bits16(lora_a, "lora_a")
    lb = None if lora_b is None else _bits16(lora_b, "lora_b")
    if (la is None) != (lb is None):
        raise ValueError("lora_a and lora_b go together")
    if y is None:
        y = torch.empty((m, n), dtype=torch.bfloat16, device=x.device)
    if z_rows:
        _need(z, "z", torch.float32, (m, k), x.device)
        _check_linear_args(m, n, k, r, x.device, codes, scales, gscale, la, lb, None, y)
    else:
        _check_linear_args(m, n, k, r, x.device, codes, scales, gscale, la, lb, z, y)
    if ws is None:
        ws = workspace(m, n, k, r, x.device)
    _need(ws, "workspace", torch.uint8, (ws.numel(),), x.device)
    args = (_ptr(x), m, _ptr(codes), _ptr(scales), _ptr(gscale), n, k, _ptr(la), _ptr(lb), r,
            float(lora_scale), _ptr(z), _ptr(y), _ptr(ws), ws.numel(), _stream(x.device))
    # the tensors stay referenced as long as the arguments are
    return args, y, (x, codes, scales, gscale, la, lb, z, ws)


def _linear(fn_name, x, codes, scales, gscale, lora_a, lora_b, lora_scale, z, ws, y,
            gate_up=False, z_rows=False):
    args, y, _ = _linear_args(fn_name, x, codes, scales, gscale, lora_a, lora_b, lora_scale, z,
                              ws, y, gate_up, z_rows)
    _check(getattr(lib, fn_name)(*args), fn_name)
    return y


class BoundCall:
    """One library call whose arguments were checked and marshalled once;
    each call of the object enqueues it again (on the stream that was
    current when it was bound).  It keeps its tensors alive."""

    def __init__(self, fn_name, args, keep, out):
        self.fn_name = fn_name
        self.fn = getattr(lib, fn_name)
        self.args = args
        self.keep = keep
        self.out = out

    def __call__(self):
        status = self.fn(*self.args)
        if status != QERL_OK:
            raise QerlError(status, self.fn_name)
        return self.out


def bind_linear(x, codes, scales, gscale, lora_a=None, lora_b=None, lora_scale=0.0, z=None,
                workspace=None, y=None, entry="decode"):
    """A BoundCall of qerl_linear_<entry> (entry: decode, prefill, decode_swiglu,
    decode_mxfp4, decode_rownoise or prefill_rownoise) with these arguments;
    its result is y."""
    fn_name = "qerl_linear_" + entry
    args, y, keep = _linear_args(fn_name, x, codes, scales, gscale, lora_a, lora_b, lora_scale,
                                 z, workspace, y, gate_up=(entry == "decode_swiglu"),
                                 z_rows=entry.endswith("rownoise"))
    return BoundCall(fn_name, args, keep, y)


def qerl_linear_decode(x, codes, scales, gscale, lora_a=None, lora_b=None, lora_scale=0.0,
                       z=None, workspace=None, y=None):
    """y = bf16(x_t W_hat^T + s (x_t A^T) B^T), x_t = x (1 + z); tuned for small m."""
    return _linear("qerl_linear_decode", x, codes, scales, gscale, lora_a, lora_b,
                   lora_scale, z, workspace, y)


def qerl_linear_decode_noalloc(x, codes, scales, gscale, lora_a=None, lora_b=None,
                               lora_scale=0.0, z=None, y=None):
    """qerl_linear_decode with the library's own per-GPU scratch (no
    workspace; calls overlapping on one GPU race)."""
    x = _bits16(x, "x")
    m, k = x.shape
    n = codes.shape[0]
    r = 0 if lora_a is None else int(lora_a.shape[0])
    la = None if lora_a is None else _bits16(lora_a, "lora_a")
    lb = None if lora_b is None else _bits16(lora_b, "lora_b")
    if y is None:
        y = torch.empty((m, n), dtype=torch.bfloat16, device=x.device)
    _check_linear_args(m, n, k, r, x.device, codes, scales, gscale, la, lb, z, y)
    _check(lib.qerl_linear_decode_noalloc(_ptr(x), m, _ptr(codes), _ptr(scales), _ptr(gscale), n,
                                          k, _ptr(la), _ptr(lb), r, float(lora_scale), _ptr(z),
                                          _ptr(y), _stream(x.device)),
           "qerl_linear_decode_noalloc")
    return y


def qerl_linear_decode_swiglu(gate_up, codes, scales, gscale, lora_a=None, lora_b=None,
                              lora_scale=0.0, z=None, workspace=None, y=None):
    """qerl_linear_decode of x = bf16(SiLU(gate) * up) from the fused gate/up
    output [m, 2k] (gate first), without writing x."""
    return _linear("qerl_linear_decode_swiglu", gate_up, codes, scales, gscale, lora_a, lora_b,
                   lora_scale, z, workspace, y, gate_up=True)


def qerl_linear_decode_rownoise(x, codes, scales, gscale, lora_a=None, lora_b=None,
                                lora_scale=0.0, z_rows=None, workspace=None, y=None):
    """qerl_linear_decode with one noise row per token (z_rows [m, k])."""
    return _linear("qerl_linear_decode_rownoise", x, codes, scales, gscale, lora_a, lora_b,
                   lora_scale, z_rows, workspace, y, z_rows=True)


def qerl_linear_prefill_rownoise(x, codes, scales, gscale, lora_a=None, lora_b=None,
                                 lora_scale=0.0, z_rows=None, workspace=None, y=None):
    """qerl_linear_prefill with one noise row per token (z_rows [m, k])."""
    return _linear("qerl_linear_prefill_rownoise", x, codes, scales, gscale, lora_a, lora_b,
                   lora_scale, z_rows, workspace, y, z_rows=True)


def qerl_linear_prefill(x, codes, scales, gscale, lora_a=None, lora_b=None, lora_scale=0.0,
                        z=None, workspace=None, y=None):
    """Same as qerl_linear_decode, tuned for large m."""
    return _linear("qerl_linear_prefill", x, codes, scales, gscale, lora_a, lora_b,
                   lora_scale, z, workspace, y)


def bind_linear_prepare(x, n, lora_a, lora_scale, z, workspace):
    """A BoundCall of qerl_linear_prepare (the first half of a linear call)."""
    x = _bits16(x, "x")
    m, k = x.shape
    r = 0 if lora_a is None else int(lora_a.shape[0])
    la = None if lora_a is None else _bits16(lora_a, "lora_a")
    _need(la, "lora_a", _BF16, (r, k), x.device)
    _need(z, "z", torch.float32, (k,), x.device)
    _need(workspace, "workspace", torch.uint8, (workspace.numel(),), x.device)
    args = (_ptr(x), m, n, k, _ptr(la), r, float(lora_scale), _ptr(z), _ptr(workspace),
            workspace.numel(), _stream(x.device))
    return BoundCall("qerl_linear_prepare", args, (x, la, z, workspace), workspace)


def qerl_linear_prepare(x, n, lora_a, lora_scale, z, workspace):
    x = _bits16(x, "x")
    m, k = x.shape
    r = 0 if lora_a is None else int(lora_a.shape[0])
    la = None if lora_a is None else _bits16(lora_a, "lora_a")
    _need(la, "lora_a", _BF16, (r, k), x.device)
    _need(z, "z", torch.float32, (k,), x.device)
    _need(workspace, "workspace", torch.uint8, (workspace.numel(),), x.device)
    _check(lib.qerl_linear_prepare(_ptr(x), m, n, k, _ptr(la), r, float(lora_scale), _ptr(z),
                                   _ptr(workspace), workspace.numel(), _stream(x.device)),
           "qerl_linear_prepare")


def _prepared(fn_name, m, codes, scales, gscale, k, lora_b, y, workspace):
    n = codes.shape[0]
    r = 0 if lora_b is None else int(lora_b.shape[1])
    lb = None if lora_b is None else _bits16(lora_b, "lora_b")
    _check_linear_args(m, n, k, r, codes.device, codes, scales, gscale, None, lb, None, y)
    _need(workspace, "workspace", torch.uint8, (workspace.numel(),), codes.device)
    fn = getattr(lib, fn_name)
    _check(fn(m, _ptr(codes), _ptr(scales), _ptr(gscale), n, k, _ptr(lb), r, _ptr(y),
              _ptr(workspace), workspace.numel(), _stream(y.device)), fn_name)
    return y


def bind_linear_prepared(m, codes, scales, gscale, k, lora_b, y, workspace, entry="decode"):
    """A BoundCall of qerl_linear_<entry>_prepared (entry: decode, prefill or
    decode_mxfp4 for qerl_linear_decode_prepared_mxfp4)."""
    fn_name = ("qerl_linear_decode_prepared_mxfp4" if entry == "decode_mxfp4"
               else f"qerl_linear_{entry}_prepared")
    n = codes.shape[0]
    r = 0 if lora_b is None else int(lora_b.shape[1])
    lb = None if lora_b is None else _bits16(lora_b, "lora_b")
    _check_linear_args(m, n, k, r, codes.device, codes, scales, gscale, None, lb, None, y)
    _need(workspace, "workspace", torch.uint8, (workspace.numel(),), codes.device)
    args = (m, _ptr(codes), _ptr(scales), _ptr(gscale), n, k, _ptr(lb), r, _ptr(y),
            _ptr(workspace), workspace.numel(), _stream(y.device))
    return BoundCall(fn_name, args, (codes, scales, gscale, lb, y, workspace), y)


def qerl_linear_decode_prepared(m, codes, scales, gscale, k, lora_b, y, workspace):
    """Contraction half of qerl_linear_decode from a workspace that
    qerl_linear_prepare filled for the same (m, n, k, r)."""
    return _prepared("qerl_linear_decode_prepared", m, codes, scales, gscale, k, lora_b, y,
                     workspace)


def qerl_linear_prefill_prepared(m, codes, scales, gscale, k, lora_b, y, workspace):
    """Contraction half of qerl_linear_prefill from a prepared workspace."""
    return _prepared("qerl_linear_prefill_prepared", m, codes, scales, gscale, k, lora_b, y,
                     workspace)


def qerl_linear_backward(dy, x, codes, scales, gscale, lora_a=None, lora_b=None,
                         lora_scale=0.0, z=None, want_lora_grads=True, workspace=None):
    """(dx, dA, dB) of the layer through the frozen NVFP4 weight; dA and dB
    are fp32 (None without a LoRA branch or when not wanted)."""
    dy = _bits16(dy, "dy")
    x = _bits16(x, "x")
    m, n = dy.shape
    k = x.shape[1]
    r = 0 if lora_a is None else int(lora_a.shape[0])
    la = None if lora_a is None else _bits16(lora_a, "lora_a")
    lb = None if lora_b is None else _bits16(lora_b, "lora_b")
    if x.shape[0] != m:
        raise ValueError("dy and x must have the same number of rows")
    _check_linear_args(m, n, k, r, dy.device, codes, scales, gscale, la, lb, z)
    nbytes = lib.qerl_linear_backward_workspace_bytes(m, n, k, r)
    if nbytes == 0:
        raise ValueError("invalid backward sizes")
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=dy.device)
    dx = torch.empty((m, k), dtype=torch.bfloat16, device=dy.device)
    da = db = None
    if r and want_lora_grads:
        da = torch.empty((r, k), dtype=torch.float32, device=dy.device)
        db = torch.empty((n, r), dtype=torch.float32, device=dy.device)
    _check(lib.qerl_linear_backward(_ptr(dy), m, _ptr(codes), _ptr(scales), _ptr(gscale), n, k,
                                    _ptr(x), _ptr(la), _ptr(lb), r, float(lora_scale), _ptr(z),
                                    _ptr(dx), _ptr(da), _ptr(db), _ptr(workspace),
                                    workspace.numel(), _stream(dy.device)),
           "qerl_linear_backward")
    return dx, da, db


def qerl_quantize_mxfp4(w):
    """bf16 W [n, k] -> (codes uint8 [n, k/2], E8M0 scales uint8 [n, k/32],
    nonfinite flag int32 [1]) on W's device."""
    w = _bits16(w, "w")
    n, k = w.shape
    codes = torch.empty((n, k // 2), dtype=torch.uint8, device=w.device)
    scales = torch.empty((n, k // 32), dtype=torch.uint8, device=w.device)
    flag = torch.empty(1, dtype=torch.int32, device=w.device)
    _check(lib.qerl_quantize_mxfp4(_ptr(w), n, k, _ptr(codes), _ptr(scales), _ptr(flag),
                                   _stream(w.device)), "qerl_quantize_mxfp4")
    return codes, scales, flag


def qerl_mxfp4_to_nvfp4(codes, scales_e8m0):
    """(E4M3 scales [n, k/16], gscale [1], range flag [1]) expressing the MXFP4
    weight in the NVFP4 layout the linear calls take (with the same codes)."""
    n, k = codes.shape[0], codes.shape[1] * 2
    s4 = torch.empty((n, k // 16), dtype=torch.uint8, device=codes.device)
    g = torch.empty(1, dtype=torch.float32, device=codes.device)
    flag = torch.empty(1, dtype=torch.int32, device=codes.device)
    _check(lib.qerl_mxfp4_to_nvfp4(_ptr(codes), _ptr(scales_e8m0), n, k, _ptr(s4), _ptr(g),
                                   _ptr(flag), _stream(codes.device)), "qerl_mxfp4_to_nvfp4")
    return s4, g, flag


def qerl_nvfp4_check_pow2_scales(scales, k):
    """int32 [1] flag on the device: 1 if any block scale of the NVFP4 weight
    (E4M3 bytes [n, k/16]) is neither zero nor a power of two (the weight then
    must not run through qerl_linear_decode_mxfp4), else 0."""
    n = scales.shape[0]
    _need(scales, "scales", torch.uint8, (n, k // 16), scales.device)
    flag = torch.empty(1, dtype=torch.int32, device=scales.device)
    _check(lib.qerl_nvfp4_check_pow2_scales(_ptr(scales), n, k, _ptr(flag), _stream(scales.device)),
           "qerl_nvfp4_check_pow2_scales")
    return flag


def qerl_linear_decode_mxfp4(x, codes, scales, gscale, lora_a=None, lora_b=None, lora_scale=0.0,
                             z=None, workspace=None, y=None):
    """qerl_linear_decode for an MXFP4 weight in the NVFP4 layout (power-of-two
    block scales, from qerl_mxfp4_to_nvfp4)."""
    return _linear("qerl_linear_decode_mxfp4", x, codes, scales, gscale, lora_a, lora_b,
                   lora_scale, z, workspace, y)


def qerl_linear_decode_prepared_mxfp4(m, codes, scales, gscale, k, lora_b, y, workspace):
    """qerl_linear_decode_prepared for power-of-two block scales."""
    return _prepared("qerl_linear_decode_prepared_mxfp4", m, codes, scales, gscale, k, lora_b, y,
                     workspace)


# ------------------------------------------------------- tiled weight layout
def qerl_nvfp4_tile128_bytes(n, k):
    return int(lib.qerl_nvfp4_tile128_bytes(n, k))


def qerl_nvfp4_tile128(codes, scales):
    """The NVFP4 weight (codes [n, k/2], scales [n, k/16]) re-laid in the
    tiled layout of the 128-token decode kernel (uint8 [ceil(n/32), k/128,
    2304]); n and k are needed again by the tiled linear calls."""
    n, k = codes.shape[0], codes.shape[1] * 2
    _need(scales, "scales", torch.uint8, (n, k // 16), codes.device)
    if not codes.is_contiguous() or codes.dtype != torch.uint8:
        raise TypeError("codes must be a contiguous uint8 tensor")
    nbytes = qerl_nvfp4_tile128_bytes(n, k)
    if nbytes == 0:
        raise ValueError("the tiled layout needs k to be a multiple of 128")
    out = torch.empty(((n + 31) // 32, k // 128, 2304), dtype=torch.uint8, device=codes.device)
    _check(lib.qerl_nvfp4_tile128(_ptr(codes), _ptr(scales), n, k, _ptr(out),
                                  _stream(codes.device)), "qerl_nvfp4_tile128")
    return out


def qerl_linear_tiled_workspace_bytes(m, n, k, r):
    return int(lib.qerl_linear_tiled_workspace_bytes(m, n, k, r))


def tiled_workspace(m, n, k, r, device="cuda"):
    nbytes = qerl_linear_tiled_workspace_bytes(m, n, k, r)
    if nbytes == 0:
        raise ValueError("invalid tiled linear sizes")
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def _tiled_args(x, tiled, gscale, n, lora_a, lora_b, lora_scale, z, ws, y):
    x = _bits16(x, "x")
    m, k = x.shape
    r = 0 if lora_a is None else int(lora_a.shape[0])
    la = None if lora_a is None else _bits16(lora_a, "lora_a")
    lb = None if lora_b is None else _bits16(lora_b, "lora_b")
    if (la is None) != (lb is None):
        raise ValueError("lora_a and lora_b go together")
    _need(tiled, "tiled", torch.uint8, ((n + 31) // 32, k // 128, 2304), x.device)
    if y is None:
        y = torch.empty((m, n), dtype=torch.bfloat16, device=x.device)
    _check_linear_args(m, n, k, r, x.device, None, None, gscale, la, lb, z, y)
    if ws is None:
        ws = tiled_workspace(m, n, k, r, x.device)
    _need(ws, "workspace", torch.uint8, (ws.numel(),), x.device)
    args = (_ptr(x), m, _ptr(tiled), _ptr(gscale), n, k, _ptr(la), _ptr(lb), r,
            float(lora_scale), _ptr(z), _ptr(y), _ptr(ws), ws.numel(), _stream(x.device))
    return args, y, (x, tiled, gscale, la, lb, z, ws)


def qerl_linear_decode_tiled(x, tiled, gscale, n, lora_a=None, lora_b=None, lora_scale=0.0,
                             z=None, workspace=None, y=None):
    """qerl_linear_decode with the weight in the tiled layout."""
    args, y, _ = _tiled_args(x, tiled, gscale, n, lora_a, lora_b, lora_scale, z, workspace, y)
    _check(lib.qerl_linear_decode_tiled(*args), "qerl_linear_decode_tiled")
    return y


def bind_linear_tiled(x, tiled, gscale, n, lora_a=None, lora_b=None, lora_scale=0.0, z=None,
                      workspace=None, y=None):
    """A BoundCall of qerl_linear_decode_tiled; its result is y."""
    args, y, keep = _tiled_args(x, tiled, gscale, n, lora_a, lora_b, lora_scale, z, workspace, y)
    return BoundCall("qerl_linear_decode_tiled", args, keep, y)


def qerl_linear_decode_tiled_prepared(m, tiled, gscale, n, k, lora_b, y, workspace):
    """Contraction half of qerl_linear_decode_tiled from a prepared workspace."""
    r = 0 if lora_b is None else int(lora_b.shape[1])
    lb = None if lora_b is None else _bits16(lora_b, "lora_b")
    _need(tiled, "tiled", torch.uint8, ((n + 31) // 32, k // 128, 2304), tiled.device)
    _check_linear_args(m, n, k, r, tiled.device, None, None, gscale, None, lb, None, y)
    _check(lib.qerl_linear_decode_tiled_prepared(m, _ptr(tiled), _ptr(gscale), n, k, _ptr(lb), r,
                                                 _ptr(y), _ptr(workspace), workspace.numel(),
                                                 _stream(tiled.device)),
           "qerl_linear_decode_tiled_prepared")
    return y


def bind_linear_tiled_prepared(m, tiled, gscale, n, k, lora_b, y, workspace):
    """A BoundCall of qerl_linear_decode_tiled_prepared."""
    r = 0 if lora_b is None else int(lora_b.shape[1])
    lb = None if lora_b is None else _bits16(lora_b, "lora_b")
    _need(tiled, "tiled", torch.uint8, ((n + 31) // 32, k // 128, 2304), tiled.device)
    _check_linear_args(m, n, k, r, tiled.device, None, None, gscale, None, lb, None, y)
    args = (m, _ptr(tiled), _ptr(gscale), n, k, _ptr(lb), r, _ptr(y), _ptr(workspace),
            workspace.numel(), _stream(tiled.device))
    return BoundCall("qerl_linear_decode_tiled_prepared", args, (tiled, gscale, lb, y, workspace),
                     y)
