"""MI355X (gfx950) linear layer over packed trellis-coded weights.

A thin ctypes binding over libtrellis.so (include/trellis.h).  The functions
keep the C names without the ``trellis_`` prefix and only marshal
arguments: shapes and dtypes are checked, outputs and workspaces are
allocated with PyTorch on the input's device, and the call is enqueued on
the current PyTorch stream.  Every arithmetic step runs in the HIP library;
if libtrellis.so is missing the functions raise instead of computing
anything another way.

Tensor conventions (all CUDA/HIP device tensors, contiguous):
  codes  int32/uint32 [rows, cols*k/32]  packed code words
  scales float16 [rows]
  x      bfloat16 [M, in_features]
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtrellis.so")

OK, EINVAL, EUNSUPPORTED, EWORKSPACE, EHIP = 0, -1, -2, -3, -4
OUT_BF16, OUT_F32 = 0, 1
PREFILL_FUSED, PREFILL_EXPAND_GEMM, PREFILL_AUTO = 0, 1, 2
MATVEC_MAX_M = 4
GROUP_MAX = 4

# every symbol include/trellis.h declares
EXPORTS = (
    "trellis_matvec_axis1_workspace_bytes", "trellis_matvec_axis1", "trellis_matvec_axis1_group",
    "trellis_gateup_swiglu_workspace_bytes", "trellis_gateup_swiglu",
    "trellis_matvec_axis0_workspace_bytes", "trellis_matvec_axis0", "trellis_matvec_axis0_noalloc",
    "trellis_mlp_decode_workspace_bytes", "trellis_mlp_decode",
    "trellis_matvec_axis0_il", "trellis_expand_bf16_il",
    "trellis_expand_bf16", "trellis_prefill_workspace_bytes", "trellis_prefill",
    "trellis_prefill_axis0_workspace_bytes", "trellis_prefill_axis0", "trellis_prefill_axis0_il",
    "trellis_prefill_tune", "trellis_prefill_axis0_tune",
    "trellis_probe_decode_only", "trellis_probe_gateup_decode_free",
    "trellis_decode_states", "trellis_last_error", "trellis_version",
)


class TrellisError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"[status {status}] {msg}")
        self.status = status


_lib = None
_vp, _i64, _int, _sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t


def load_library():
    """Load libtrellis.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} not built; run trellis_coded_quantized_amd._build.build()")
    lib = ctypes.CDLL(LIB_PATH)
    sig = {
        "trellis_matvec_axis1_workspace_bytes": (_sz, [_i64, _i64, _int, _int, _int, _int]),
        "trellis_matvec_axis1": (_int, [_vp, _vp, _vp, _vp, _int, _i64, _i64, _int, _int, _int, _int,
                                        _vp, _sz, _vp]),
        "trellis_matvec_axis1_group": (_int, [_vp, _vp, _vp, _vp, _int, _vp, _int, _i64, _int, _int, _int, _int,
                                              _vp]),
        "trellis_gateup_swiglu_workspace_bytes": (_sz, [_i64, _i64, _int, _int, _int, _int]),
        "trellis_gateup_swiglu": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _int,
                                         _int, _int, _int, _vp, _sz, _vp]),
        "trellis_matvec_axis0_workspace_bytes": (_sz, [_i64, _i64, _int, _int, _int, _int]),
        "trellis_matvec_axis0": (_int, [_vp, _vp, _vp, _vp, _int, _i64, _i64, _int, _int, _int, _int,
                                        _vp, _sz, _vp]),
        "trellis_matvec_axis0_noalloc": (_int, [_vp, _vp, _vp, _vp, _int, _i64, _i64, _int, _int, _int, _int,
                                                _vp]),
        "trellis_mlp_decode_workspace_bytes": (_sz, [_i64, _i64, _i64, _int, _int, _int, _int, _int]),
        "trellis_mlp_decode": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _int,
                                      _int, _int, _int, _int, _vp, _sz, _vp]),
        "trellis_expand_bf16": (_int, [_vp, _vp, _vp, _i64, _i64, _int, _int, _int, _vp]),
        "trellis_matvec_axis0_il": (_int, [_vp, _vp, _vp, _vp, _int, _i64, _i64, _int, _int, _int, _int,
                                           _vp, _sz, _vp]),
        "trellis_expand_bf16_il": (_int, [_vp, _vp, _vp, _i64, _i64, _int, _int, _int, _vp]),
        "trellis_prefill_workspace_bytes": (_sz, [_i64, _i64, _i64, _int, _int, _int, _int]),
        "trellis_prefill": (_int, [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _int, _int, _int, _int,
                                   _vp, _sz, _vp]),
        "trellis_prefill_axis0_workspace_bytes": (_sz, [_i64, _i64, _i64, _int, _int, _int, _int]),
        "trellis_prefill_axis0": (_int, [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _int, _int, _int, _int,
                                         _vp, _sz, _vp]),
        "trellis_prefill_axis0_il": (_int, [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _int, _int, _int, _int,
                                            _vp, _sz, _vp]),
        "trellis_prefill_tune": (_int, [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _int, _int, _int, _vp, _sz, _vp]),
        "trellis_prefill_axis0_tune": (_int, [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _int, _int, _int, _vp, _sz,
                                              _vp]),
        "trellis_probe_decode_only": (_int, [_vp, _vp, _int, _int, _int, _vp]),
        "trellis_probe_gateup_decode_free": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _int, _int, _int,
                                                    _int, _vp]),
        "trellis_decode_states": (_int, [_vp, _i64, _i64, _int, _int, _int, _vp, _vp, _vp, _vp]),
        "trellis_last_error": (ctypes.c_char_p, []),
        "trellis_version": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def version() -> str:
    return load_library().trellis_version().decode()


def _check(status: int):
    if status != OK:
        raise TrellisError(status, load_library().trellis_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t, name, dtypes, ndim):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype} not in {dtypes}")
    if t.dim() != ndim:
        raise ValueError(f"{name}: expected {ndim} dims, got shape {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")


_CODES = (torch.int32, torch.uint32)


def _geometry(codes, k):
    rows, words = codes.shape
    if (words * 32) % k:
        raise ValueError(f"{words} words are not a whole number of {k}-bit symbols")
    return rows, words * 32 // k


def _axis0_geometry(codes, k):
    """(rows, cols, interleaved) of axis-0 codes: row-major [R, C*k/32], or the
    block-interleaved k = 3 layout [C/512, R, 48] (identified by its shape)."""
    if codes.dim() == 3:
        groups, rows, words = codes.shape
        if k != 3 or words != 48:
            raise ValueError(f"interleaved codes must be k = 3 with 48 words per row pair, got k={k}, {words}")
        return rows, groups * 512, True
    rows, cols = _geometry(codes, k)
    return rows, cols, False


def _workspace(nbytes, device, workspace):
    if nbytes == 0:
        return None, 0
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)
    elif not (isinstance(workspace, torch.Tensor) and workspace.device.type == "cuda" and workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous device tensor")
    return workspace, workspace.numel() * workspace.element_size()


def _rows(scales, n, name="scales"):
    if scales.numel() != n:
        raise ValueError(f"{name} has {scales.numel()} entries, the matrix has {n} stored rows")


def _out(t, name, shape, dtypes, device):
    """A caller's output buffer (exactly `shape`, contiguous, on the device), or a new one."""
    if t is None:
        return torch.empty(shape, dtype=dtypes[0], device=device)
    _need(t, name, dtypes, len(shape))
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t


_F = (torch.bfloat16, torch.float32)


def _odt(out_dtype):
    """output dtypes a matvec accepts, the requested one first"""
    if out_dtype not in _F:
        raise ValueError(f"out_dtype {out_dtype} not in {_F}")
    return (out_dtype,) + _F


def matvec_axis1(codes, scales, x, k, L=12, T=256, out_dtype=torch.bfloat16, out=None,
                 workspace=None):
    """y[m, r] = sum_c w(r, c) x[m, c]; codes [R, C*k/32] coded along inputs."""
    _need(codes, "codes", _CODES, 2)
    _need(scales, "scales", (torch.float16,), 1)
    _need(x, "x", (torch.bfloat16,), 2)
    R, C = _geometry(codes, k)
    _rows(scales, R)
    M = x.shape[0]
    if x.shape[1] != C:
        raise ValueError(f"x has {x.shape[1]} features, codes encode {C}")
    out = _out(out, "out", (M, R), _odt(out_dtype), x.device)
    od = OUT_F32 if out.dtype == torch.float32 else OUT_BF16
    lib = load_library()
    ws, wsb = _workspace(lib.trellis_matvec_axis1_workspace_bytes(R, C, M, k, L, T), x.device, workspace)
    _check(lib.trellis_matvec_axis1(_ptr(codes), _ptr(scales), _ptr(x), _ptr(out), od, R, C, M, k, L,
                                    T, _ptr(ws), wsb, _stream(x.device)))
    return out


def matvec_axis1_group(codes, scales, x, k, L=12, T=256, out_dtype=torch.bfloat16, outs=None):
    """matvec_axis1 of every matrix in `codes` (same C and k, same x) in one launch;
    returns the list of outputs [M, R_j]."""
    n = len(codes)
    if n != len(scales) or not 1 <= n <= GROUP_MAX:
        raise ValueError(f"{n} code tensors, {len(scales)} scale tensors (1..{GROUP_MAX} matrices)")
    _need(x, "x", (torch.bfloat16,), 2)
    Rs = []
    for c, s in zip(codes, scales):
        _need(c, "codes", _CODES, 2)
        _need(s, "scales", (torch.float16,), 1)
        R, C = _geometry(c, k)
        _rows(s, R)
        if x.shape[1] != C:
            raise ValueError(f"x has {x.shape[1]} features, codes encode {C}")
        Rs.append(R)
    M = x.shape[0]
    if outs is None:
        outs = [None] * n
    if len(outs) != n:
        raise ValueError(f"{len(outs)} outputs for {n} matrices")
    outs = [_out(o, f"outs[{j}]", (M, R), _odt(out_dtype), x.device) for j, (o, R) in enumerate(zip(outs, Rs))]
    od = OUT_F32 if outs[0].dtype == torch.float32 else OUT_BF16
    if any(o.dtype != outs[0].dtype for o in outs):
        raise ValueError("outputs of one grouped call share a dtype")
    P = ctypes.c_void_p * n
    _check(load_library().trellis_matvec_axis1_group(
        P(*[c.data_ptr() for c in codes]), P(*[s.data_ptr() for s in scales]), P(*[o.data_ptr() for o in outs]),
        (ctypes.c_int64 * n)(*Rs), n, _ptr(x), od, x.shape[1], M, k, L, T, _stream(x.device)))
    return outs


def gateup_swiglu(gcodes, gscales, ucodes, uscales, x, k, L=12, T=256, out=None,
                  gate_f32=None, up_f32=None, workspace=None):
    """bf16 silu(gate(x)) * up(x) with the bf16 cast chain; returns out [M, R]."""
    for t, n in ((gcodes, "gcodes"), (ucodes, "ucodes")):
        _need(t, n, _CODES, 2)
    for t, n in ((gscales, "gscales"), (uscales, "uscales")):
        _need(t, n, (torch.float16,), 1)
    _need(x, "x", (torch.bfloat16,), 2)
    if gcodes.shape != ucodes.shape:
        raise ValueError("gate and up codes differ in shape")
    R, C = _geometry(gcodes, k)
    _rows(gscales, R, "gscales")
    _rows(uscales, R, "uscales")
    M = x.shape[0]
    if x.shape[1] != C:
        raise ValueError(f"x has {x.shape[1]} features, codes encode {C}")
    out = _out(out, "out", (M, R), (torch.bfloat16,), x.device)
    if gate_f32 is not None:
        _out(gate_f32, "gate_f32", (M, R), (torch.float32,), x.device)
    if up_f32 is not None:
        _out(up_f32, "up_f32", (M, R), (torch.float32,), x.device)
    lib = load_library()
    ws, wsb = _workspace(lib.trellis_gateup_swiglu_workspace_bytes(R, C, M, k, L, T), x.device,
                         workspace)
    _check(lib.trellis_gateup_swiglu(_ptr(gcodes), _ptr(gscales), _ptr(ucodes), _ptr(uscales),
                                     _ptr(x), _ptr(out), _ptr(gate_f32), _ptr(up_f32), R, C, M, k, L,
                                     T, _ptr(ws), wsb, _stream(x.device)))
    return out


def matvec_axis0(codes_t, scales, x, k, L=12, T=256, out_dtype=torch.bfloat16, out=None,
                 workspace=None):
    """y[m, c] = sum_r w(r, c) x[m, r]; codes_t is the stored W^T [R_in, C_out*k/32],
    or for k = 3 the block-interleaved [C_out/512, R_in, 48]."""
    _need(codes_t, "codes", _CODES, codes_t.dim() if codes_t.dim() == 3 else 2)
    _need(scales, "scales", (torch.float16,), 1)
    _need(x, "x", (torch.bfloat16,), 2)
    R, C, il = _axis0_geometry(codes_t, k)
    _rows(scales, R)
    M = x.shape[0]
    if x.shape[1] != R:
        raise ValueError(f"x has {x.shape[1]} features, stored rows are {R}")
    out = _out(out, "out", (M, C), _odt(out_dtype), x.device)
    od = OUT_F32 if out.dtype == torch.float32 else OUT_BF16
    lib = load_library()
    ws, wsb = _workspace(lib.trellis_matvec_axis0_workspace_bytes(R, C, M, k, L, T), x.device,
                         workspace)
    fn = lib.trellis_matvec_axis0_il if il else lib.trellis_matvec_axis0
    _check(fn(_ptr(codes_t), _ptr(scales), _ptr(x), _ptr(out), od, R, C, M, k, L, T, _ptr(ws), wsb,
              _stream(x.device)))
    return out


def mlp_decode(gcodes, gscales, ucodes, uscales, dcodes_t, dscales, x, k_gu, k_down, L=12, T=256,
               hidden=None, out=None, workspace=None):
    """down(silu(gate(x)) * up(x)) for M <= 4 rows: the gate/up SwiGLU kernel,
    then the axis-0 down projection (dcodes_t is the stored W_down^T
    [R, C_out*k_down/32]).  `hidden` (bf16 [M, R]) receives the hidden
    vectors if given."""
    for t, n in ((gcodes, "gcodes"), (ucodes, "ucodes"), (dcodes_t, "dcodes")):
        _need(t, n, _CODES, 2)
    for t, n in ((gscales, "gscales"), (uscales, "uscales"), (dscales, "dscales")):
        _need(t, n, (torch.float16,), 1)
    _need(x, "x", (torch.bfloat16,), 2)
    R, C = _geometry(gcodes, k_gu)
    if _geometry(ucodes, k_gu) != (R, C):
        raise ValueError("gate and up codes differ in shape")
    Rd, C_out = _geometry(dcodes_t, k_down)
    if Rd != R:
        raise ValueError(f"down projection has {Rd} stored rows, the hidden width is {R}")
    M = x.shape[0]
    if x.shape[1] != C:
        raise ValueError(f"x has {x.shape[1]} features, gate/up take {C}")
    _rows(gscales, R, "gscales")
    _rows(uscales, R, "uscales")
    _rows(dscales, Rd, "dscales")
    out = _out(out, "out", (M, C_out), (torch.bfloat16,), x.device)
    if hidden is not None:
        _out(hidden, "hidden", (M, R), (torch.bfloat16,), x.device)
    lib = load_library()
    ws, wsb = _workspace(lib.trellis_mlp_decode_workspace_bytes(R, C, C_out, M, k_gu, k_down, L, T), x.device,
                         workspace)
    _check(lib.trellis_mlp_decode(_ptr(gcodes), _ptr(gscales), _ptr(ucodes), _ptr(uscales), _ptr(dcodes_t),
                                  _ptr(dscales), _ptr(x), _ptr(hidden), _ptr(out),
                                  R, C, C_out, M, k_gu, k_down, L, T, _ptr(ws), wsb, _stream(x.device)))
    return out


def expand_bf16(codes, scales, k, L=12, T=256, out=None):
    """bf16 [R, C] decode of the stored matrix (stored orientation); codes
    [R, C*k/32], or for k = 3 the block-interleaved axis-0 layout [C/512, R, 48]."""
    _need(codes, "codes", _CODES, codes.dim() if codes.dim() == 3 else 2)
    _need(scales, "scales", (torch.float16,), 1)
    R, C, il = _axis0_geometry(codes, k)
    _rows(scales, R)
    out = _out(out, "out", (R, C), (torch.bfloat16,), codes.device)
    lib = load_library()
    fn = lib.trellis_expand_bf16_il if il else lib.trellis_expand_bf16
    _check(fn(_ptr(codes), _ptr(scales), _ptr(out), R, C, k, L, T, _stream(codes.device)))
    return out


def prefill(codes, scales, x, k, L=12, T=256, algo=PREFILL_FUSED, out=None, workspace=None, tune=False):
    """bf16 [M, R] = x [M, C] times the bf16 expansion of the axis-1 codes.
    tune=True runs trellis_prefill_tune (expand + GEMM after timing the GEMM
    candidates; synchronises the host) instead of trellis_prefill."""
    _need(codes, "codes", _CODES, 2)
    _need(scales, "scales", (torch.float16,), 1)
    _need(x, "x", (torch.bfloat16,), 2)
    R, C = _geometry(codes, k)
    _rows(scales, R)
    M = x.shape[0]
    if x.shape[1] != C:
        raise ValueError(f"x has {x.shape[1]} features, codes encode {C}")
    out = _out(out, "out", (M, R), (torch.bfloat16,), x.device)
    lib = load_library()
    if tune:
        algo = PREFILL_EXPAND_GEMM
    ws, wsb = _workspace(lib.trellis_prefill_workspace_bytes(R, C, M, k, L, T, algo), x.device,
                         workspace)
    if tune:
        _check(lib.trellis_prefill_tune(_ptr(codes), _ptr(scales), _ptr(x), _ptr(out), R, C, M, k, L, T,
                                        _ptr(ws), wsb, _stream(x.device)))
    else:
        _check(lib.trellis_prefill(_ptr(codes), _ptr(scales), _ptr(x), _ptr(out), R, C, M, k, L, T, algo,
                                   _ptr(ws), wsb, _stream(x.device)))
    return out


def prefill_axis0(codes_t, scales, x, k, L=12, T=256, algo=PREFILL_EXPAND_GEMM, out=None, workspace=None,
                  tune=False):
    """out[m, c] = bf16(sum_r wb(r, c) x[m, r]) for a matrix stored transposed
    (axis 0): codes_t [R_in, C_out*k/32] (or for k = 3 the block-interleaved
    [C_out/512, R_in, 48]), x bf16 [M, R_in]; expand + GEMM, or the fused
    decode-to-LDS MFMA kernel (R_in a multiple of 128).  tune=True runs
    trellis_prefill_axis0_tune (row-major codes; synchronises the host)."""
    _need(codes_t, "codes", _CODES, codes_t.dim() if codes_t.dim() == 3 else 2)
    _need(scales, "scales", (torch.float16,), 1)
    _need(x, "x", (torch.bfloat16,), 2)
    R, C, il = _axis0_geometry(codes_t, k)
    _rows(scales, R)
    M = x.shape[0]
    if x.shape[1] != R:
        raise ValueError(f"x has {x.shape[1]} features, stored rows are {R}")
    out = _out(out, "out", (M, C), (torch.bfloat16,), x.device)
    lib = load_library()
    if tune:
        if il:
            raise ValueError("tune takes row-major codes (the GEMM it tunes is the same for both layouts)")
        algo = PREFILL_EXPAND_GEMM
    ws, wsb = _workspace(lib.trellis_prefill_axis0_workspace_bytes(R, C, M, k, L, T, algo), x.device, workspace)
    if tune:
        _check(lib.trellis_prefill_axis0_tune(_ptr(codes_t), _ptr(scales), _ptr(x), _ptr(out), R, C, M, k, L, T,
                                              _ptr(ws), wsb, _stream(x.device)))
        return out
    fn = lib.trellis_prefill_axis0_il if il else lib.trellis_prefill_axis0
    _check(fn(_ptr(codes_t), _ptr(scales), _ptr(x), _ptr(out), R, C, M, k, L, T, algo, _ptr(ws), wsb,
              _stream(x.device)))
    return out


def prefill_workspace_bytes(R, C, M, k, algo, L=12, T=256) -> int:
    return int(load_library().trellis_prefill_workspace_bytes(R, C, M, k, L, T, algo))


def decode_states(codes, k, L=12, T=256):
    """(states int16-bits [R, C], y int16 [R, C], value f32 [R, C]) from the GPU decoder."""
    _need(codes, "codes", _CODES, 2)
    R, C = _geometry(codes, k)
    dev = codes.device
    st = torch.empty((R, C), dtype=torch.int16, device=dev)
    ys = torch.empty((R, C), dtype=torch.int16, device=dev)
    vals = torch.empty((R, C), dtype=torch.float32, device=dev)
    _check(load_library().trellis_decode_states(_ptr(codes), R, C, k, L, T, _ptr(st), _ptr(ys),
                                                _ptr(vals), _stream(dev)))
    return st, ys, vals


PROBE_THREADS = 512


def probe_decode_only(runs, k, iters, blocks=None):
    """Measurement probe: decode the runs held in `runs` (int32/uint32
    [blocks * 512, k + 1]) `iters` times each; returns the per-wave sums
    (f32 [blocks * 8], 16 times the sum of the codes each wave decoded)."""
    _need(runs, "runs", _CODES, 2)
    n, words = runs.shape
    if words != k + 1 or n % PROBE_THREADS:
        raise ValueError(f"runs must be [blocks * {PROBE_THREADS}, k + 1], got {tuple(runs.shape)}")
    blocks = n // PROBE_THREADS if blocks is None else blocks
    out = torch.empty(blocks * PROBE_THREADS // 64, dtype=torch.float32, device=runs.device)
    _check(load_library().trellis_probe_decode_only(_ptr(runs), _ptr(out), blocks, iters, k, _stream(runs.device)))
    return out


def probe_gateup_decode_free(gcodes, gscales, ucodes, uscales, x, k, L=12, T=256, out=None):
    """Measurement probe: the gate/up kernel with no decode (timing floor; the
    output values are meaningless)."""
    R, C = _geometry(gcodes, k)
    M = x.shape[0]
    out = _out(out, "out", (M, R), (torch.bfloat16,), x.device)
    _check(load_library().trellis_probe_gateup_decode_free(_ptr(gcodes), _ptr(gscales), _ptr(ucodes), _ptr(uscales),
                                                           _ptr(x), _ptr(out), R, C, M, k, L, T, _stream(x.device)))
    return out
