"""ctypes binding of libseed.so (argument marshalling only).

The functions carry the C names. Tensors are torch tensors used only as device memory: their
data pointers and the current HIP stream are handed to the library, and every step of the
computation runs in the library's gfx950 kernels. There is no CPU fallback: if libseed.so is
missing, importing this module raises.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libseed.so")

SEED_OK, SEED_ERR_ARG, SEED_ERR_UNSUPPORTED, SEED_ERR_WORKSPACE, SEED_ERR_HIP = 0, -1, -2, -3, -4
SEED_GDN, SEED_KDA, SEED_MAMBA2 = 0, 1, 2
SEED_F32, SEED_BF16, SEED_F16 = 0, 1, 2
SEED_ROUND_NEAREST, SEED_ROUND_STOCHASTIC = 0, 1
SEED_OP_COMPRESS, SEED_OP_FROM_DENSE = 0, 1

EXPORTS = [
    "seed_state_bytes", "seed_scale_len", "seed_workspace_bytes", "seed_state_from_dense",
    "seed_from_dense_iterations", "seed_decode_step", "seed_decode_step_ragged", "seed_compress",
    "seed_compress_ragged", "seed_state_energy", "seed_dense_decode_step", "seed_decode_chunk",
    "seed_chunk_max_tokens", "seed_decode_chunk_ragged", "seed_state_spectrum", "seed_compress_units",
    "seed_stream_create_cu_masked", "seed_stream_destroy", "seed_decode_step_normed",
    "seed_decode_step_ragged_normed", "seed_status_string", "seed_version",
]

SEED_SPECTRUM_LEN = 33


class seed_shape(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("batch", ctypes.c_int32), ("heads", ctypes.c_int32),
                ("d_k", ctypes.c_int32), ("d_v", ctypes.c_int32), ("rank", ctypes.c_int32),
                ("period", ctypes.c_int32), ("factor_dtype", ctypes.c_int32),
                ("io_dtype", ctypes.c_int32), ("rounding", ctypes.c_int32),
                ("rng_key", ctypes.c_uint32)]

    @property
    def units(self) -> int:
        return self.batch * self.heads

    @property
    def slots(self) -> int:
        return self.rank + self.period


class seed_head_norm(ctypes.Structure):
    _fields_ = [("weight", ctypes.c_void_p), ("gate", ctypes.c_void_p), ("eps", ctypes.c_float),
                ("gate_first", ctypes.c_int32)]


class seed_state(ctypes.Structure):
    _fields_ = [("a", ctypes.c_void_p), ("U", ctypes.c_void_p), ("V", ctypes.c_void_p),
                ("scale", ctypes.c_void_p)]


class SeedError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn}: {seed_status_string(status)} (status {status})")
        self.status = status


def hip_runtimes_mapped() -> list:
    """Paths of the HIP runtime libraries (libamdhip64) mapped into this process."""
    found = set()
    try:
        with open("/proc/self/maps") as f:
            for line in f:
                parts = line.split()
                if len(parts) >= 6 and "libamdhip64" in os.path.basename(parts[-1]):
                    found.add(os.path.realpath(parts[-1]))
    except OSError:
        pass
    return sorted(found)


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built: run `python -m rank_recurrent_state_amd.build`")
    # libseed binds to whichever HIP runtime the process already holds. Torch's wheel bundles
    # its own copy, and the tensors handed to the library are torch's: torch is imported first,
    # so that libseed's libamdhip64 dependency resolves to that copy. Loaded first, libseed would
    # pull in the system runtime, torch would then map its own, and every launch would fail
    # with tensors of one runtime handed to the other.
    import torch  # noqa: F401

    lib = ctypes.CDLL(LIB_PATH)
    # Two copies would give two sets of streams and device state, and a stream of one handed to
    # the other: refuse that outright.
    rts = hip_runtimes_mapped()
    if len(rts) > 1:
        raise ImportError(f"more than one HIP runtime is mapped into this process: {rts}")
    P = ctypes.c_void_p
    Sp = ctypes.POINTER(seed_shape)
    Stp = ctypes.POINTER(seed_state)
    sig = {
        "seed_state_bytes": (ctypes.c_size_t, [Sp]),
        "seed_scale_len": (ctypes.c_int32, [Sp]),
        "seed_workspace_bytes": (ctypes.c_size_t, [Sp, ctypes.c_int32]),
        "seed_state_from_dense": (ctypes.c_int, [Sp, P, P, Stp, P, ctypes.c_size_t, P]),
        "seed_from_dense_iterations": (ctypes.c_int32, []),
        "seed_decode_step": (ctypes.c_int, [Sp, Stp, ctypes.c_int32, P, P, P, P, P, P, P, P]),
        "seed_decode_step_ragged": (ctypes.c_int, [Sp, Stp, P, P, P, P, P, P, P, P, P]),
        "seed_compress": (ctypes.c_int, [Sp, Stp, ctypes.c_int32, P, ctypes.c_size_t, P]),
        "seed_compress_ragged": (ctypes.c_int, [Sp, Stp, ctypes.c_int32, P, ctypes.c_size_t, P]),
        "seed_state_energy": (ctypes.c_int, [Sp, Stp, P, P, P]),
        "seed_dense_decode_step": (ctypes.c_int, [Sp, P, P, P, P, P, P, P, P]),
        "seed_decode_chunk": (ctypes.c_int, [Sp, Stp, ctypes.c_int32, ctypes.c_int32, P, P, P, P, P, P,
                                             P, P]),
        "seed_chunk_max_tokens": (ctypes.c_int32, []),
        "seed_compress_units": (ctypes.c_int, [Sp, Stp, P, ctypes.c_int32, P, ctypes.c_size_t, P]),
        "seed_decode_chunk_ragged": (ctypes.c_int, [Sp, Stp, P, ctypes.c_int32, P, P, P, P, P, P, P, P]),
        "seed_state_spectrum": (ctypes.c_int, [Sp, Stp, P, P]),
        "seed_stream_create_cu_masked": (ctypes.c_int, [ctypes.c_uint32, P, ctypes.POINTER(ctypes.c_void_p)]),
        "seed_stream_destroy": (ctypes.c_int, [P]),
        "seed_decode_step_normed": (ctypes.c_int, [Sp, Stp, ctypes.c_int32, P, P, P, P, P, P,
                                                   ctypes.POINTER(seed_head_norm), P, P]),
        "seed_decode_step_ragged_normed": (ctypes.c_int, [Sp, Stp, P, P, P, P, P, P, P,
                                                          ctypes.POINTER(seed_head_norm), P, P]),
        "seed_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "seed_version": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


LIB = _load()


def make_shape(kind: int, batch: int, heads: int, d_k: int, d_v: int, rank: int, period: int,
               factor_dtype: int = SEED_F32, io_dtype: int | None = None,
               rounding: int = SEED_ROUND_NEAREST, rng_key: int = 0) -> seed_shape:
    """A seed_shape; io_dtype defaults to the factor dtype (bf16 for fp16 factors, the one
    input format compiled with them)."""
    if io_dtype is None:
        io_dtype = SEED_BF16 if factor_dtype == SEED_F16 else factor_dtype
    return seed_shape(kind, batch, heads, d_k, d_v, rank, period, factor_dtype, io_dtype, rounding,
                      rng_key & 0xFFFFFFFF)


def _stream_ptr(stream):
    if stream is None:
        import torch
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(fn: str, status: int):
    if status != SEED_OK:
        raise SeedError(fn, status)


def seed_status_string(status: int) -> str:
    return LIB.seed_status_string(status).decode()


def seed_version() -> str:
    return LIB.seed_version().decode()


def seed_state_bytes(shape: seed_shape) -> int:
    return int(LIB.seed_state_bytes(ctypes.byref(shape)))


def seed_scale_len(shape: seed_shape) -> int:
    return int(LIB.seed_scale_len(ctypes.byref(shape)))


def seed_workspace_bytes(shape: seed_shape, op: int) -> int:
    return int(LIB.seed_workspace_bytes(ctypes.byref(shape), op))


def seed_from_dense_iterations() -> int:
    return int(LIB.seed_from_dense_iterations())


class State:
    """Device buffers of a factored state (torch tensors used as memory only)."""

    def __init__(self, a, U, V, scale):
        self.a, self.U, self.V, self.scale = a, U, V, scale
        self.c = seed_state(a.data_ptr(), U.data_ptr(), V.data_ptr(), scale.data_ptr())

    @classmethod
    def empty(cls, shape: seed_shape, device="cuda"):
        import torch
        fdt = _torch_dt(shape.factor_dtype)
        n = shape.units
        a = torch.zeros((n, shape.d_k), dtype=torch.float32, device=device)
        U = torch.zeros((n, shape.slots, shape.d_k), dtype=fdt, device=device)
        V = torch.zeros((n, shape.slots, shape.d_v), dtype=fdt, device=device)
        scale = torch.ones((n, seed_scale_len(shape)), dtype=torch.float32, device=device)
        scale[:, seed_scale_len(shape) - shape.period - 2:] = 0.0  # coefficients, window and column counts
        return cls(a, U, V, scale)

    def tensors(self):
        return self.a, self.U, self.V, self.scale


def _state_c(state):
    return ctypes.byref(state if isinstance(state, seed_state) else state.c)


def _torch_dt(code):
    import torch
    return {SEED_F32: torch.float32, SEED_BF16: torch.bfloat16, SEED_F16: torch.float16}[code]


def _expect(name, t, numel, code=None):
    """Marshalling check of a torch tensor: on a GPU, contiguous, right size and dtype.

    Keeps a wrong buffer from ever reaching a kernel; objects that are not torch tensors (raw
    pointer holders) are passed through unchecked.
    """
    if t is None or not hasattr(t, "is_cuda"):
        return
    if not t.is_cuda:
        raise ValueError(f"{name}: expected a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous tensor")
    if t.numel() != numel:
        raise ValueError(f"{name}: expected {numel} elements, got {t.numel()}")
    if code is not None and t.dtype != _torch_dt(code):
        raise ValueError(f"{name}: expected dtype {_torch_dt(code)}, got {t.dtype}")


def _expect_state(shape, state):
    if isinstance(state, State):
        n = shape.units
        _expect("state.a", state.a, n * shape.d_k, SEED_F32)
        _expect("state.U", state.U, n * shape.slots * shape.d_k, shape.factor_dtype)
        _expect("state.V", state.V, n * shape.slots * shape.d_v, shape.factor_dtype)
        _expect("state.scale", state.scale, n * seed_scale_len(shape), SEED_F32)


def _expect_io(shape, q, k, v, beta, g, o):
    n = shape.units
    _expect("q", q, n * shape.d_k, shape.io_dtype)
    _expect("k", k, n * shape.d_k, shape.io_dtype)
    _expect("v", v, n * shape.d_v, shape.io_dtype)
    _expect("beta", beta, n, SEED_F32)
    _expect("g", g, n * (shape.d_k if shape.kind == SEED_KDA else 1), SEED_F32)
    _expect("o", o, n * shape.d_v, shape.io_dtype)


class CUMaskedStream:
    """A HIP stream restricted to a set of compute units, made and destroyed by libseed (so it
    belongs to the runtime that launches the kernels). `.torch` is a torch ExternalStream view of
    it for use with torch's stream and event API; close() (or the context manager) destroys the
    stream after synchronising it."""

    def __init__(self, cu_mask_words):
        words = list(cu_mask_words)
        arr = (ctypes.c_uint32 * len(words))(*words)
        h = ctypes.c_void_p()
        _check("seed_stream_create_cu_masked", LIB.seed_stream_create_cu_masked(len(words), arr, ctypes.byref(h)))
        self.handle = h.value
        import torch
        self.torch = torch.cuda.ExternalStream(self.handle)

    def close(self):
        if self.handle:
            self.torch.synchronize()
            _check("seed_stream_destroy", LIB.seed_stream_destroy(ctypes.c_void_p(self.handle)))
            self.handle = None
            self.torch = None

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def seed_state_from_dense(shape: seed_shape, S, vbar, state, ws=None, stream=None) -> None:
    _expect("S", S, shape.units * shape.d_k * shape.d_v, SEED_F32)
    _expect("vbar", vbar, shape.heads * shape.d_v, SEED_F32)
    _expect_state(shape, state)
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check("seed_state_from_dense", LIB.seed_state_from_dense(
        ctypes.byref(shape), _ptr(S), _ptr(vbar), _state_c(state), _ptr(ws), ws_bytes,
        _stream_ptr(stream)))


def seed_decode_step(shape: seed_shape, state, m: int, q, k, v, beta, g, vbar, o,
                     stream=None) -> None:
    _expect_state(shape, state)
    _expect_io(shape, q, k, v, beta, g, o)
    _expect("vbar", vbar, shape.heads * shape.d_v, SEED_F32)
    _check("seed_decode_step", LIB.seed_decode_step(
        ctypes.byref(shape), _state_c(state), m, _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(g),
        _ptr(vbar), _ptr(o), _stream_ptr(stream)))


def _head_norm(shape, weight, gate, eps, gate_first):
    _expect("norm weight", weight, shape.heads * shape.d_v, SEED_F32)
    _expect("norm gate", gate, shape.units * shape.d_v, shape.io_dtype)
    return seed_head_norm(None if weight is None else weight.data_ptr(),
                          None if gate is None else gate.data_ptr(), float(eps), int(gate_first))


def seed_decode_step_normed(shape: seed_shape, state, m: int, q, k, v, beta, g, vbar, o, weight,
                            gate=None, eps: float = 1e-6, gate_first: bool = False, stream=None) -> None:
    """seed_decode_step with the head normalisation fused into its epilogue: o receives
    weight[h] * x / sqrt(mean(x^2) + eps) (times silu(gate) after, or x = o * silu(gate) first)."""
    _expect_state(shape, state)
    _expect_io(shape, q, k, v, beta, g, o)
    _expect("vbar", vbar, shape.heads * shape.d_v, SEED_F32)
    nrm = _head_norm(shape, weight, gate, eps, gate_first)
    _check("seed_decode_step_normed", LIB.seed_decode_step_normed(
        ctypes.byref(shape), _state_c(state), m, _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(g),
        _ptr(vbar), ctypes.byref(nrm), _ptr(o), _stream_ptr(stream)))


def seed_decode_step_ragged_normed(shape: seed_shape, state, q, k, v, beta, g, vbar, o, weight,
                                   gate=None, eps: float = 1e-6, gate_first: bool = False, active=None,
                                   stream=None) -> None:
    """seed_decode_step_ragged with the head normalisation of seed_decode_step_normed."""
    import torch
    _expect_state(shape, state)
    _expect_io(shape, q, k, v, beta, g, o)
    _expect("vbar", vbar, shape.heads * shape.d_v, SEED_F32)
    if active is not None and hasattr(active, "is_cuda"):
        _expect("active", active, shape.units)
        if active.dtype != torch.uint8:
            raise ValueError(f"active: expected dtype torch.uint8, got {active.dtype}")
    nrm = _head_norm(shape, weight, gate, eps, gate_first)
    _check("seed_decode_step_ragged_normed", LIB.seed_decode_step_ragged_normed(
        ctypes.byref(shape), _state_c(state), _ptr(active), _ptr(q), _ptr(k), _ptr(v), _ptr(beta),
        _ptr(g), _ptr(vbar), ctypes.byref(nrm), _ptr(o), _stream_ptr(stream)))


def seed_decode_step_ragged(shape: seed_shape, state, q, k, v, beta, g, vbar, o, active=None,
                            stream=None) -> None:
    """Every unit steps from its own column count (kept in the state); active (uint8 [units] on
    the device, or None for all) masks units out."""
    import torch
    _expect_state(shape, state)
    _expect_io(shape, q, k, v, beta, g, o)
    _expect("vbar", vbar, shape.heads * shape.d_v, SEED_F32)
    if active is not None and hasattr(active, "is_cuda"):
        _expect("active", active, shape.units)
        if active.dtype != torch.uint8:
            raise ValueError(f"active: expected dtype torch.uint8, got {active.dtype}")
    _check("seed_decode_step_ragged", LIB.seed_decode_step_ragged(
        ctypes.byref(shape), _state_c(state), _ptr(active), _ptr(q), _ptr(k), _ptr(v), _ptr(beta),
        _ptr(g), _ptr(vbar), _ptr(o), _stream_ptr(stream)))


def seed_state_spectrum(shape: seed_shape, state, out=None, stream=None):
    """Per unit the 32 largest squared singular values of the content U V^T, then |U V^T|^2,
    as a float32 [units, 33] device tensor."""
    import torch
    _expect_state(shape, state)
    if out is None:
        out = torch.empty((shape.units, SEED_SPECTRUM_LEN), dtype=torch.float32, device=state.a.device)
    _expect("out", out, shape.units * SEED_SPECTRUM_LEN, SEED_F32)
    _check("seed_state_spectrum", LIB.seed_state_spectrum(ctypes.byref(shape), _state_c(state), _ptr(out),
                                                          _stream_ptr(stream)))
    return out


def seed_chunk_max_tokens() -> int:
    return int(LIB.seed_chunk_max_tokens())


def _expect_chunk_io(shape, length, q, k, v, beta, g, o):
    n = shape.units * length
    _expect("q", q, n * shape.d_k, shape.io_dtype)
    _expect("k", k, n * shape.d_k, shape.io_dtype)
    _expect("v", v, n * shape.d_v, shape.io_dtype)
    _expect("beta", beta, n, SEED_F32)
    _expect("g", g, n * (shape.d_k if shape.kind == SEED_KDA else 1), SEED_F32)
    _expect("o", o, n * shape.d_v, shape.io_dtype)


def seed_decode_chunk_ragged(shape: seed_shape, state, length: int, q, k, v, beta, g, vbar, o,
                             active=None, stream=None) -> None:
    """The chunk of seed_decode_chunk for every unit from its own column count (kept in the
    state); active (uint8 [units] on the device, or None for all) masks units out, and units
    without room for the chunk are skipped."""
    import torch
    _expect_state(shape, state)
    _expect_chunk_io(shape, length, q, k, v, beta, g, o)
    _expect("vbar", vbar, shape.heads * shape.d_v, SEED_F32)
    if active is not None and hasattr(active, "is_cuda"):
        _expect("active", active, shape.units)
        if active.dtype != torch.uint8:
            raise ValueError(f"active: expected dtype torch.uint8, got {active.dtype}")
    _check("seed_decode_chunk_ragged", LIB.seed_decode_chunk_ragged(
        ctypes.byref(shape), _state_c(state), _ptr(active), length, _ptr(q), _ptr(k), _ptr(v), _ptr(beta),
        _ptr(g), _ptr(vbar), _ptr(o), _stream_ptr(stream)))


def seed_decode_chunk(shape: seed_shape, state, m: int, length: int, q, k, v, beta, g, vbar, o,
                      stream=None) -> None:
    """`length` tokens of every unit in one call: q, k [batch, length, heads, d_k], v and o
    [batch, length, heads, d_v], beta [batch, length, heads] and g [batch, length, heads]
    (KDA: [batch, length, heads, d_k]), float32."""
    _expect_state(shape, state)
    _expect_chunk_io(shape, length, q, k, v, beta, g, o)
    _expect("vbar", vbar, shape.heads * shape.d_v, SEED_F32)
    _check("seed_decode_chunk", LIB.seed_decode_chunk(
        ctypes.byref(shape), _state_c(state), m, length, _ptr(q), _ptr(k), _ptr(v), _ptr(beta),
        _ptr(g), _ptr(vbar), _ptr(o), _stream_ptr(stream)))


def seed_compress_units(shape: seed_shape, state, units, ws=None, stream=None) -> None:
    """Compress the listed units (int32 device tensor of unit indices, each listed once), each
    at its own column count."""
    import torch
    _expect_state(shape, state)
    count = 0
    if units is not None and hasattr(units, "is_cuda"):
        if not units.is_cuda or not units.is_contiguous() or units.dtype != torch.int32:
            raise ValueError("units: expected a contiguous int32 device tensor")
        count = units.numel()
    elif units is not None:
        raise ValueError("units: expected a torch tensor")
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check("seed_compress_units", LIB.seed_compress_units(
        ctypes.byref(shape), _state_c(state), _ptr(units), count, _ptr(ws), ws_bytes, _stream_ptr(stream)))


def seed_compress_ragged(shape: seed_shape, state, min_m: int, ws=None, stream=None) -> None:
    """Compress the units whose own column count is >= min_m (min_m = r + T: the full ones)."""
    _expect_state(shape, state)
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check("seed_compress_ragged", LIB.seed_compress_ragged(
        ctypes.byref(shape), _state_c(state), min_m, _ptr(ws), ws_bytes, _stream_ptr(stream)))


def seed_state_energy(shape: seed_shape, state, vbar, out=None, stream=None):
    """Per unit (|S~|^2, |a vbar^T|^2, |U V^T|^2) as a float32 [units, 3] device tensor."""
    import torch
    _expect_state(shape, state)
    _expect("vbar", vbar, shape.heads * shape.d_v, SEED_F32)
    if out is None:
        out = torch.empty((shape.units, 3), dtype=torch.float32, device=state.a.device)
    _expect("out", out, shape.units * 3, SEED_F32)
    _check("seed_state_energy", LIB.seed_state_energy(
        ctypes.byref(shape), _state_c(state), _ptr(vbar), _ptr(out), _stream_ptr(stream)))
    return out


def column_counts(shape: seed_shape, state):
    """Every unit's column count m, read from its state (a host-side int64 tensor)."""
    import torch
    return state.scale[:, seed_scale_len(shape) - 1].contiguous().view(torch.int32).long().cpu()


def seed_compress(shape: seed_shape, state, m: int, ws=None, stream=None) -> None:
    _expect_state(shape, state)
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check("seed_compress", LIB.seed_compress(
        ctypes.byref(shape), _state_c(state), m, _ptr(ws), ws_bytes, _stream_ptr(stream)))


def seed_dense_decode_step(shape: seed_shape, S, q, k, v, beta, g, o, stream=None) -> None:
    _expect("S", S, shape.units * shape.d_k * shape.d_v, SEED_F32)
    _expect_io(shape, q, k, v, beta, g, o)
    _check("seed_dense_decode_step", LIB.seed_dense_decode_step(
        ctypes.byref(shape), _ptr(S), _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(g), _ptr(o),
        _stream_ptr(stream)))
