"""QLoRA NF4 hot path on MI355X (gfx950): thin Python binding over the C ABI.

The functions here have the names of the C entry points in
``include/qlora_nf4.h`` and only marshal arguments: they check that tensors
are contiguous device tensors of the right dtype and size, allocate outputs
with torch when the caller passes none, and call the library on torch's
current stream.  Every step of the computation runs in the HIP kernels of
``lib/libqlora_nf4.so``; there is no other code path.  If the library is not
built, every call raises.

The library is loaded lazily so that ``bit_nf4_quantized_22_amd.synth`` can
be imported without it.
"""

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "lib", "libqlora_nf4.so")

QN_OK, QN_ERR_NULL, QN_ERR_SHAPE, QN_ERR_ALIGN = 0, -1, -2, -3
QN_ERR_UNSUPPORTED, QN_ERR_WORKSPACE, QN_ERR_HIP = -4, -5, -6
QN_F32, QN_BF16 = 0, 1
QN_OP_FWD, QN_OP_BWD_DX, QN_OP_LORA_GRADS, QN_OP_BWD_DX_DROPOUT = 0, 1, 2, 3
BLOCKSIZE, GROUP = 64, 256

EXPORTS = ("qn_status_string", "nf4_codebook", "nf4_quantize", "dq_quantize_scales",
           "nf4_dequant", "qn_workspace_bytes", "qlora_linear_fwd", "qlora_linear_bwd_dx",
           "lora_grads", "qlora_merge", "lora_adamw_step", "lora_dropout",
           "qlora_linear_fwd_dropout", "qlora_linear_bwd_dx_dropout", "fp4_codebook",
           "fp4_quantize", "dq_quantize_scales_fp8", "qlora_linear_fwd_noalloc",
           "dq_quantize_scales_centred", "nf4_quantize_dq", "nf4_quantize_dq_batch",
           "qn_hbm_read_probe")


class QnError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__(f"{fn} failed: status {status} ({msg})")
        self.status = status


class qn_weight(ctypes.Structure):
    _fields_ = [("packed", ctypes.c_void_p), ("qscale", ctypes.c_void_p),
                ("gscale", ctypes.c_void_p), ("absmax", ctypes.c_void_p),
                ("N", ctypes.c_int64), ("K", ctypes.c_int64),
                ("blocksize", ctypes.c_int32), ("group", ctypes.c_int32),
                ("quant_type", ctypes.c_int32), ("scale_type", ctypes.c_int32),
                ("offset", ctypes.c_void_p)]


_lib = None


def load_library():
    """Load lib/libqlora_nf4.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"HIP library not built: {LIB_PATH} is missing "
                           "(run python -m bit_nf4_quantized_22_amd.build)")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, f32, sz, u64 = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                                  ctypes.c_float, ctypes.c_size_t, ctypes.c_uint64)
    wp = ctypes.POINTER(qn_weight)
    sig = {
        "qn_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "nf4_codebook": (ctypes.c_int, [ctypes.POINTER(ctypes.c_float)]),
        "fp4_codebook": (ctypes.c_int, [ctypes.POINTER(ctypes.c_float)]),
        "nf4_quantize": (ctypes.c_int, [vp, i32, i64, i32, vp, vp, vp]),
        "fp4_quantize": (ctypes.c_int, [vp, i32, i64, i32, vp, vp, vp]),
        "dq_quantize_scales": (ctypes.c_int, [vp, i64, i32, vp, vp, vp]),
        "dq_quantize_scales_fp8": (ctypes.c_int, [vp, i64, i32, vp, vp, vp]),
        "dq_quantize_scales_centred": (ctypes.c_int, [vp, i64, i32, vp, vp, vp, vp]),
        "nf4_quantize_dq": (ctypes.c_int, [vp, i32, i64, i32, i32, i32, i32, vp, vp, vp, vp, vp]),
        "nf4_quantize_dq_batch": (ctypes.c_int, [i32, vp, vp, i32, i32, i32, i32, i32, vp, vp, vp,
                                                 vp, vp]),
        "qn_hbm_read_probe": (ctypes.c_int, [vp, i64, vp, vp]),
        "nf4_dequant": (ctypes.c_int, [wp, i32, vp, vp]),
        "qn_workspace_bytes": (sz, [i32, i64, i64, i64, i32]),
        "qlora_linear_fwd": (ctypes.c_int, [wp, vp, i64, vp, vp, i32, f32, vp, vp, vp, sz, vp]),
        "qlora_linear_bwd_dx": (ctypes.c_int, [wp, vp, i64, vp, vp, i32, f32, vp, vp, vp, sz, vp]),
        "lora_grads": (ctypes.c_int, [vp, vp, vp, vp, vp, vp, i64, i64, i64, i32, f32, vp, vp,
                                      vp, sz, vp]),
        "qlora_merge": (ctypes.c_int, [wp, vp, vp, i32, f32, vp, vp]),
        "lora_adamw_step": (ctypes.c_int, [vp, vp, vp, vp, vp, i64, f32, f32, f32, f32, f32, i32,
                                           vp]),
        "lora_dropout": (ctypes.c_int, [vp, i64, i64, f32, u64, vp, vp]),
        "qlora_linear_fwd_noalloc": (ctypes.c_int, [wp, vp, i64, vp, vp, i32, f32, vp, vp, vp]),
        "qlora_linear_fwd_dropout": (ctypes.c_int, [wp, vp, vp, i64, vp, vp, i32, f32, vp, vp, vp,
                                                    sz, vp]),
        "qlora_linear_bwd_dx_dropout": (ctypes.c_int, [wp, vp, i64, vp, vp, i32, f32, f32, u64, vp,
                                                       vp, vp, sz, vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(fn, status):
    if status != QN_OK:
        msg = load_library().qn_status_string(status).decode()
        raise QnError(fn, status, msg)


def _torch():
    import torch
    return torch


def _stream(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev(t, dtype, numel=None, name="tensor"):
    torch = _torch()
    if t is None:
        return None
    if not t.is_cuda or not t.is_contiguous() or t.dtype != dtype:
        raise ValueError(f"{name}: need a contiguous {dtype} device tensor")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name}: expected {numel} elements, got {t.numel()}")
    return t


QN_NF4, QN_FP4 = 0, 1
QN_SCALE_U8, QN_SCALE_FP8, QN_SCALE_CENTRED = 0, 1, 2
_QUANT_TYPES = {"nf4": QN_NF4, "fp4": QN_FP4}
_SCALE_TYPES = {"u8": QN_SCALE_U8, "fp8": QN_SCALE_FP8, "centred": QN_SCALE_CENTRED}


class QuantWeight:
    """Device tensors of a 4-bit weight W[N, K] (+ double-quantised constants).

    packed uint8[N*K/2]; qscale uint8[N*K/64] and gscale fp32[ceil(N*K/64/256)]
    when double-quantised, else absmax fp32[N*K/64].  quant_type "nf4" or
    "fp4" (the code table), scale_type "u8", "fp8" or "centred" (the level-2
    code; "centred" also carries offset, fp32[1], the subtracted mean).
    """

    def __init__(self, packed, N, K, qscale=None, gscale=None, absmax=None, quant_type="nf4",
                 scale_type="u8", offset=None):
        self.packed, self.qscale, self.gscale, self.absmax = packed, qscale, gscale, absmax
        self.N, self.K = int(N), int(K)
        self.quant_type, self.scale_type = quant_type, scale_type
        self.offset = offset

    def c_struct(self):
        return qn_weight(self.packed.data_ptr(),
                         None if self.qscale is None else self.qscale.data_ptr(),
                         None if self.gscale is None else self.gscale.data_ptr(),
                         None if self.absmax is None else self.absmax.data_ptr(),
                         self.N, self.K, BLOCKSIZE, GROUP, _QUANT_TYPES[self.quant_type],
                         _SCALE_TYPES[self.scale_type],
                         None if self.offset is None else self.offset.data_ptr())


def nf4_codebook():
    """The 16 fp32 NF4 code points (host call), as a list of floats."""
    out = (ctypes.c_float * 16)()
    _check("nf4_codebook", load_library().nf4_codebook(out))
    return list(out)


def fp4_codebook():
    """The 16 fp32 FP4 code points (host call), as a list of floats."""
    out = (ctypes.c_float * 16)()
    _check("fp4_codebook", load_library().fp4_codebook(out))
    return list(out)


def nf4_quantize(w, packed=None, absmax=None, stream=None):
    """Blockwise NF4 quantisation of a fp32 or bf16 device tensor (flattened).

    Returns (packed uint8[numel/2], absmax fp32[ceil(numel/64)]).
    """
    return _quantize("nf4_quantize", w, packed, absmax, stream)


def fp4_quantize(w, packed=None, absmax=None, stream=None):
    """nf4_quantize with the FP4 code table."""
    return _quantize("fp4_quantize", w, packed, absmax, stream)


def nf4_quantize_dq(w, quant_type="nf4", scale_type="u8", packed=None, qscale=None, gscale=None,
                    absmax=None, stream=None):
    """Quantisation and double quantisation in one launch: returns (packed,
    qscale, gscale); the block constants are written to absmax only when a
    tensor is given for them."""
    torch = _torch()
    lib = load_library()
    if quant_type not in _QUANT_TYPES or scale_type not in ("u8", "fp8"):
        raise ValueError("quant_type must be 'nf4' or 'fp4', scale_type 'u8' or 'fp8'")
    if w.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("nf4_quantize_dq: weights must be float32 or bfloat16")
    _dev(w, w.dtype, name="w")
    n = w.numel()
    nb = -(-n // BLOCKSIZE)
    ng = -(-nb // GROUP)
    dev = w.device
    packed = torch.empty(n // 2, dtype=torch.uint8, device=dev) if packed is None else packed
    qscale = torch.empty(nb, dtype=torch.uint8, device=dev) if qscale is None else qscale
    gscale = torch.empty(ng, dtype=torch.float32, device=dev) if gscale is None else gscale
    _dev(packed, torch.uint8, n // 2, "packed")
    _dev(qscale, torch.uint8, nb, "qscale")
    _dev(gscale, torch.float32, ng, "gscale")
    _dev(absmax, torch.float32, nb, "absmax")
    dt = QN_F32 if w.dtype == torch.float32 else QN_BF16
    _check("nf4_quantize_dq", lib.nf4_quantize_dq(
        _ptr(w), dt, n, BLOCKSIZE, GROUP, _QUANT_TYPES[quant_type], _SCALE_TYPES[scale_type],
        _ptr(packed), _ptr(absmax), _ptr(qscale), _ptr(gscale), _stream(stream)))
    return packed, qscale, gscale


def nf4_quantize_dq_batch(ws, quant_type="nf4", scale_type="u8", outs=None, absmax=None,
                          stream=None):
    """nf4_quantize_dq over up to 8 weights of one dtype in one launch:
    returns a list of (packed, qscale, gscale), one per weight.  outs, if
    given, holds such triples to write into; absmax, if given, a list of
    fp32 tensors (or None entries) for the block constants."""
    torch = _torch()
    lib = load_library()
    if quant_type not in _QUANT_TYPES or scale_type not in ("u8", "fp8"):
        raise ValueError("quant_type must be 'nf4' or 'fp4', scale_type 'u8' or 'fp8'")
    n = len(ws)
    if n == 0:
        return []
    dtypes = {w.dtype for w in ws}
    if len(dtypes) != 1 or dtypes.pop() not in (torch.float32, torch.bfloat16):
        raise ValueError("nf4_quantize_dq_batch: weights must all be float32 or all bfloat16")
    res = []
    for i, w in enumerate(ws):
        _dev(w, w.dtype, name="w")
        m = w.numel()
        nb = -(-m // BLOCKSIZE)
        ng = -(-nb // GROUP)
        dev = w.device
        if outs is not None:
            packed, qscale, gscale = outs[i]
        else:
            packed = torch.empty(m // 2, dtype=torch.uint8, device=dev)
            qscale = torch.empty(nb, dtype=torch.uint8, device=dev)
            gscale = torch.empty(ng, dtype=torch.float32, device=dev)
        _dev(packed, torch.uint8, m // 2, "packed")
        _dev(qscale, torch.uint8, nb, "qscale")
        _dev(gscale, torch.float32, ng, "gscale")
        if absmax is not None:
            _dev(absmax[i], torch.float32, nb, "absmax")
        res.append((packed, qscale, gscale))
    vpa = ctypes.c_void_p * n
    wa = vpa(*[_ptr(w) for w in ws])
    na = (ctypes.c_int64 * n)(*[w.numel() for w in ws])
    pa = vpa(*[_ptr(r[0]) for r in res])
    qa = vpa(*[_ptr(r[1]) for r in res])
    ga = vpa(*[_ptr(r[2]) for r in res])
    aa = vpa(*[_ptr(a) for a in absmax]) if absmax is not None else None
    dt = QN_F32 if ws[0].dtype == torch.float32 else QN_BF16
    _check("nf4_quantize_dq_batch", lib.nf4_quantize_dq_batch(
        n, wa, na, dt, BLOCKSIZE, GROUP, _QUANT_TYPES[quant_type], _SCALE_TYPES[scale_type],
        pa, aa, qa, ga, _stream(stream)))
    return res


def quantize_weights(ws, stream=None, quant_type="nf4", scale_type="u8"):
    """Double-quantised QuantWeight of each [N, K] tensor in ws (one dtype),
    at most 8 per launch (nf4_quantize_dq_batch)."""
    out = []
    for i in range(0, len(ws), 8):
        part = ws[i:i + 8]
        for w, (packed, qscale, gscale) in zip(part, nf4_quantize_dq_batch(
                part, quant_type, scale_type, stream=stream)):
            out.append(QuantWeight(packed, w.shape[0], w.shape[1], qscale=qscale, gscale=gscale,
                                   quant_type=quant_type, scale_type=scale_type))
    return out


def _quantize(fn, w, packed, absmax, stream):
    torch = _torch()
    lib = load_library()
    if w.dtype == torch.float32:
        dt = QN_F32
    elif w.dtype == torch.bfloat16:
        dt = QN_BF16
    else:
        raise ValueError(f"{fn}: weights must be float32 or bfloat16")
    _dev(w, w.dtype, name="w")
    n = w.numel()
    nb = -(-n // BLOCKSIZE)
    if packed is None:
        packed = torch.empty(n // 2, dtype=torch.uint8, device=w.device)
    if absmax is None:
        absmax = torch.empty(nb, dtype=torch.float32, device=w.device)
    _dev(packed, torch.uint8, n // 2, "packed")
    _dev(absmax, torch.float32, nb, "absmax")
    _check(fn, getattr(lib, fn)(_ptr(w), dt, n, BLOCKSIZE, _ptr(packed), _ptr(absmax),
                                _stream(stream)))
    return packed, absmax


def dq_quantize_scales(absmax, qscale=None, gscale=None, stream=None, fp8=False):
    """Double quantisation: returns (qscale uint8[nb], gscale fp32[ceil(nb/256)]);
    fp8 selects the E4M3 level-2 code (dq_quantize_scales_fp8)."""
    torch = _torch()
    lib = load_library()
    _dev(absmax, torch.float32, name="absmax")
    nb = absmax.numel()
    ng = -(-nb // GROUP)
    if qscale is None:
        qscale = torch.empty(nb, dtype=torch.uint8, device=absmax.device)
    if gscale is None:
        gscale = torch.empty(ng, dtype=torch.float32, device=absmax.device)
    _dev(qscale, torch.uint8, nb, "qscale")
    _dev(gscale, torch.float32, ng, "gscale")
    fn = "dq_quantize_scales_fp8" if fp8 else "dq_quantize_scales"
    _check(fn, getattr(lib, fn)(_ptr(absmax), nb, GROUP, _ptr(qscale), _ptr(gscale),
                                _stream(stream)))
    return qscale, gscale


def dq_quantize_scales_centred(absmax, qscale=None, gscale=None, offset=None, stream=None):
    """Mean-centred double quantisation: returns (qscale uint8[nb] (signed
    codes), gscale fp32[ceil(nb/256)], offset fp32[1])."""
    torch = _torch()
    lib = load_library()
    _dev(absmax, torch.float32, name="absmax")
    nb = absmax.numel()
    ng = -(-nb // GROUP)
    dev = absmax.device
    qscale = torch.empty(nb, dtype=torch.uint8, device=dev) if qscale is None else qscale
    gscale = torch.empty(ng, dtype=torch.float32, device=dev) if gscale is None else gscale
    offset = torch.empty(1, dtype=torch.float32, device=dev) if offset is None else offset
    _dev(qscale, torch.uint8, nb, "qscale")
    _dev(gscale, torch.float32, ng, "gscale")
    _dev(offset, torch.float32, 1, "offset")
    _check("dq_quantize_scales_centred", lib.dq_quantize_scales_centred(
        _ptr(absmax), nb, GROUP, _ptr(qscale), _ptr(gscale), _ptr(offset), _stream(stream)))
    return qscale, gscale, offset


def quantize_weight(w, double_quant=True, stream=None, quant_type="nf4", scale_type="u8"):
    """4-bit quantisation (+ double quantisation) of a [N, K] tensor -> QuantWeight.

    quant_type "nf4" (nf4_quantize) or "fp4" (fp4_quantize); scale_type "u8"
    (dq_quantize_scales), "fp8" (dq_quantize_scales_fp8) or "centred"
    (dq_quantize_scales_centred)."""
    if quant_type not in _QUANT_TYPES or scale_type not in _SCALE_TYPES:
        raise ValueError("quant_type must be 'nf4' or 'fp4', scale_type 'u8', 'fp8' or "
                         "'centred'")
    N, K = w.shape
    if double_quant and scale_type != "centred":
        packed, qscale, gscale = nf4_quantize_dq(w, quant_type, scale_type, stream=stream)
        return QuantWeight(packed, N, K, qscale=qscale, gscale=gscale, quant_type=quant_type,
                           scale_type=scale_type)
    quant = fp4_quantize if quant_type == "fp4" else nf4_quantize
    packed, absmax = quant(w, stream=stream)
    if not double_quant:
        return QuantWeight(packed, N, K, absmax=absmax, quant_type=quant_type)
    qscale, gscale, offset = dq_quantize_scales_centred(absmax, stream=stream)
    return QuantWeight(packed, N, K, qscale=qscale, gscale=gscale, quant_type=quant_type,
                       scale_type=scale_type, offset=offset)


def nf4_dequant(qw, out_dtype=None, out=None, stream=None):
    """Materialise W[N, K] as fp32 or bf16."""
    torch = _torch()
    lib = load_library()
    out_dtype = out_dtype or torch.bfloat16
    dt = QN_BF16 if out_dtype == torch.bfloat16 else QN_F32
    if out is None:
        out = torch.empty((qw.N, qw.K), dtype=out_dtype, device=qw.packed.device)
    _dev(out, out_dtype, qw.N * qw.K, "out")
    cw = qw.c_struct()
    _check("nf4_dequant", lib.nf4_dequant(ctypes.byref(cw), dt, _ptr(out), _stream(stream)))
    return out


def qn_workspace_bytes(op, M, N, K, r):
    return int(load_library().qn_workspace_bytes(op, M, N, K, r))


def workspace(nbytes, device):
    """A uint8 device workspace of nbytes for the linear ops."""
    return _torch().empty(nbytes, dtype=_torch().uint8, device=device)


def _workspace(op, M, N, K, r, ws, device):
    need = qn_workspace_bytes(op, M, N, K, r)
    if ws is None and need > 0:
        ws = workspace(need, device)
    return ws, (0 if ws is None else ws.numel())


def qlora_linear_fwd(qw, x, A, B, r, alpha, y=None, u_out=None, ws=None, stream=None):
    """y = x W^T + (alpha/r) (x A^T) B^T  (bf16 in/out)."""
    return _fwd(qw, x, None, A, B, r, alpha, y, u_out, ws, stream)


def qlora_linear_fwd_dropout(qw, x, x_drop, A, B, r, alpha, y=None, u_out=None, ws=None,
                             stream=None):
    """y = x W^T + (alpha/r) (x_drop A^T) B^T, x_drop from lora_dropout."""
    return _fwd(qw, x, x_drop, A, B, r, alpha, y, u_out, ws, stream)


def hbm_read_probe(buf, sink, stream=None):
    """Streaming read of a contiguous device tensor (a measurement aid);
    sink is a device tensor of at least 4 bytes."""
    if not buf.is_cuda or not buf.is_contiguous() or not sink.is_cuda:
        raise ValueError("hbm_read_probe: contiguous device tensors required")
    nbytes = buf.numel() * buf.element_size()
    _check("qn_hbm_read_probe", load_library().qn_hbm_read_probe(
        _ptr(buf), nbytes - nbytes % 16, _ptr(sink), _stream(stream)))


def qlora_linear_fwd_noalloc(qw, x, A, B, r, alpha, y, u_out=None, stream=None):
    """qlora_linear_fwd on the library's own scratch array: y (and u_out)
    must be given; the call allocates nothing."""
    torch = _torch()
    lib = load_library()
    M = x.shape[0]
    _dev(x, torch.bfloat16, M * qw.K, "x")
    if r:
        _dev(A, torch.bfloat16, r * qw.K, "A")
        _dev(B, torch.bfloat16, qw.N * r, "B")
    if y is None:
        raise ValueError("y: the allocation-free forward writes into a given tensor")
    _dev(y, torch.bfloat16, M * qw.N, "y")
    _dev(u_out, torch.bfloat16, M * r, "u_out")
    cw = qw.c_struct()
    a, b = (_ptr(A), _ptr(B)) if r else (None, None)
    _check("qlora_linear_fwd_noalloc", lib.qlora_linear_fwd_noalloc(
        ctypes.byref(cw), _ptr(x), M, a, b, r, float(alpha), _ptr(y), _ptr(u_out),
        _stream(stream)))
    return y


def _fwd(qw, x, x_drop, A, B, r, alpha, y, u_out, ws, stream):
    torch = _torch()
    lib = load_library()
    M = x.shape[0]
    _dev(x, torch.bfloat16, M * qw.K, "x")
    _dev(x_drop, torch.bfloat16, M * qw.K, "x_drop")
    if r:
        _dev(A, torch.bfloat16, r * qw.K, "A")
        _dev(B, torch.bfloat16, qw.N * r, "B")
    if y is None:
        y = torch.empty((M, qw.N), dtype=torch.bfloat16, device=x.device)
    _dev(y, torch.bfloat16, M * qw.N, "y")
    _dev(u_out, torch.bfloat16, M * r, "u_out")
    ws, wsb = _workspace(QN_OP_FWD, M, qw.N, qw.K, r, ws, x.device)
    cw = qw.c_struct()
    a, b = (_ptr(A), _ptr(B)) if r else (None, None)
    if x_drop is None:
        _check("qlora_linear_fwd", lib.qlora_linear_fwd(
            ctypes.byref(cw), _ptr(x), M, a, b, r, float(alpha), _ptr(y), _ptr(u_out), _ptr(ws),
            wsb, _stream(stream)))
    else:
        _check("qlora_linear_fwd_dropout", lib.qlora_linear_fwd_dropout(
            ctypes.byref(cw), _ptr(x), _ptr(x_drop), M, a, b, r, float(alpha), _ptr(y),
            _ptr(u_out), _ptr(ws), wsb, _stream(stream)))
    return y


def qlora_linear_bwd_dx(qw, dy, A, B, r, alpha, dx=None, t_out=None, ws=None, stream=None):
    """dx = dy W + (alpha/r) (dy B) A  (bf16 in/out)."""
    return _bwd(qw, dy, A, B, r, alpha, None, 0, dx, t_out, ws, stream)


def qlora_linear_bwd_dx_dropout(qw, dy, A, B, r, alpha, p, seed, dx=None, t_out=None, ws=None,
                                stream=None):
    """dx = dy W + keep/(1-p) * ((alpha/r) (dy B) A), the mask of lora_dropout(p, seed)."""
    return _bwd(qw, dy, A, B, r, alpha, p, seed, dx, t_out, ws, stream)


def _bwd(qw, dy, A, B, r, alpha, p, seed, dx, t_out, ws, stream):
    torch = _torch()
    lib = load_library()
    M = dy.shape[0]
    _dev(dy, torch.bfloat16, M * qw.N, "dy")
    if r:
        _dev(A, torch.bfloat16, r * qw.K, "A")
        _dev(B, torch.bfloat16, qw.N * r, "B")
    if dx is None:
        dx = torch.empty((M, qw.K), dtype=torch.bfloat16, device=dy.device)
    _dev(dx, torch.bfloat16, M * qw.K, "dx")
    _dev(t_out, torch.bfloat16, M * r, "t_out")
    ws, wsb = _workspace(QN_OP_BWD_DX if p is None else QN_OP_BWD_DX_DROPOUT, M, qw.N, qw.K, r,
                         ws, dy.device)
    cw = qw.c_struct()
    a, b = (_ptr(A), _ptr(B)) if r else (None, None)
    if p is None:
        _check("qlora_linear_bwd_dx", lib.qlora_linear_bwd_dx(
            ctypes.byref(cw), _ptr(dy), M, a, b, r, float(alpha), _ptr(dx), _ptr(t_out),
            _ptr(ws), wsb, _stream(stream)))
    else:
        _check("qlora_linear_bwd_dx_dropout", lib.qlora_linear_bwd_dx_dropout(
            ctypes.byref(cw), _ptr(dy), M, a, b, r, float(alpha), float(p), int(seed), _ptr(dx),
            _ptr(t_out), _ptr(ws), wsb, _stream(stream)))
    return dx


def lora_dropout(x, p, seed, out=None, stream=None):
    """The LoRA branch's dropped input bf16[M, K]: x * keep / (1 - p), Philox mask."""
    torch = _torch()
    lib = load_library()
    M, K = x.shape
    _dev(x, torch.bfloat16, M * K, "x")
    if out is None:
        out = torch.empty_like(x)
    _dev(out, torch.bfloat16, M * K, "out")
    _check("lora_dropout", lib.lora_dropout(_ptr(x), M, K, float(p), int(seed), _ptr(out),
                                            _stream(stream)))
    return out


def lora_grads(x, dy, A, B, r, alpha, u=None, t=None, dA=None, dB=None, ws=None, stream=None):
    """(dA fp32[r, K], dB fp32[N, r]) = ((alpha/r) (dy B)^T x, (alpha/r) dy^T (x A^T))."""
    torch = _torch()
    lib = load_library()
    M, K = x.shape
    N = dy.shape[1]
    _dev(x, torch.bfloat16, M * K, "x")
    _dev(dy, torch.bfloat16, M * N, "dy")
    _dev(A, torch.bfloat16, r * K, "A")
    _dev(B, torch.bfloat16, N * r, "B")
    _dev(u, torch.bfloat16, M * r, "u")
    _dev(t, torch.bfloat16, M * r, "t")
    if dA is None:
        dA = torch.empty((r, K), dtype=torch.float32, device=x.device)
    if dB is None:
        dB = torch.empty((N, r), dtype=torch.float32, device=x.device)
    _dev(dA, torch.float32, r * K, "dA")
    _dev(dB, torch.float32, N * r, "dB")
    ws, wsb = _workspace(QN_OP_LORA_GRADS, M, N, K, r, ws, x.device)
    _check("lora_grads", lib.lora_grads(
        _ptr(x), _ptr(dy), _ptr(u), _ptr(t), _ptr(A), _ptr(B), M, N, K, r, float(alpha),
        _ptr(dA), _ptr(dB), _ptr(ws), wsb, _stream(stream)))
    return dA, dB


def qlora_merge(qw, A, B, r, alpha, out=None, stream=None):
    """Merged 16-bit weight bf16[N, K] = bf16(dequant(W) + (alpha/r) B A)."""
    torch = _torch()
    lib = load_library()
    N, K = qw.N, qw.K
    if r:
        _dev(A, torch.bfloat16, r * K, "A")
        _dev(B, torch.bfloat16, N * r, "B")
    if out is None:
        out = torch.empty((N, K), dtype=torch.bfloat16, device=qw.packed.device)
    _dev(out, torch.bfloat16, N * K, "out")
    cw = qw.c_struct()
    _check("qlora_merge", lib.qlora_merge(ctypes.byref(cw), _ptr(A) if r else None,
                                          _ptr(B) if r else None, r, float(alpha), _ptr(out),
                                          _stream(stream)))
    return out


def lora_adamw_step(p, g, m, v, step, lr=2e-4, betas=(0.9, 0.999), eps=1e-8, weight_decay=0.0,
                    p_bf16=None, stream=None):
    """In-place AdamW step on fp32 p, m, v with gradient g; optionally writes
    bf16(p) to p_bf16.  Returns p."""
    torch = _torch()
    lib = load_library()
    n = p.numel()
    for t, name in ((p, "p"), (g, "g"), (m, "m"), (v, "v")):
        _dev(t, torch.float32, n, name)
    if p_bf16 is not None:
        _dev(p_bf16, torch.bfloat16, n, "p_bf16")
    _check("lora_adamw_step", lib.lora_adamw_step(
        _ptr(p), _ptr(g), _ptr(m), _ptr(v), _ptr(p_bf16), n, float(lr), float(betas[0]),
        float(betas[1]), float(eps), float(weight_decay), int(step), _stream(stream)))
    return p
