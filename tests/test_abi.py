"""Host-side checks of the C ABI (no GPU needed): the library loads, exports every function
include/seed.h declares, answers size queries, and rejects bad arguments before launching."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "seed.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(seed_[a-z_]+)\s*\(", text)))


def _lib():
    rrs = pytest.importorskip("rank_recurrent_state_amd._lib",
                              reason="libseed.so not built (python -m rank_recurrent_state_amd.build)")
    return rrs


def test_every_declared_symbol_is_exported():
    rrs = _lib()
    names = _declared()
    assert names, "no declarations parsed"
    lib = ctypes.CDLL(rrs.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in seed.h but not exported"
    assert set(names) == set(rrs.EXPORTS)


def test_size_queries():
    rrs = _lib()
    sh = rrs.make_shape(rrs.SEED_GDN, 64, 16, 128, 128, 16, 16, rrs.SEED_BF16)
    # a (4 d_k) + U, V (2 bytes x 32 slots x (128 + 128)) + scale (4 ((1 + T) + T + 2): decay
    # scales, the sink coefficients, the compression-window and column counts)
    assert rrs.seed_state_bytes(sh) == 4 * 128 + 2 * 32 * 256 + 4 * 35
    assert rrs.seed_scale_len(sh) == 35
    kda = rrs.make_shape(rrs.SEED_KDA, 2, 2, 128, 128, 32, 32, rrs.SEED_F32)
    assert rrs.seed_scale_len(kda) == 128 + 32 + 2
    assert rrs.seed_state_bytes(kda) == 4 * 128 + 4 * 64 * 256 + 4 * 162
    # fp16 factors take the bytes of bf16 ones; their default inputs are bf16
    f16 = rrs.make_shape(rrs.SEED_GDN, 64, 16, 128, 128, 16, 16, rrs.SEED_F16)
    assert f16.io_dtype == rrs.SEED_BF16
    assert rrs.seed_state_bytes(f16) == rrs.seed_state_bytes(sh)
    assert rrs.seed_workspace_bytes(sh, rrs.SEED_OP_COMPRESS) == 0
    assert rrs.seed_workspace_bytes(sh, rrs.SEED_OP_FROM_DENSE) == 0
    assert rrs.seed_from_dense_iterations() >= 1
    bad = rrs.make_shape(rrs.SEED_GDN, 1, 1, 96, 128, 16, 16)
    assert rrs.seed_state_bytes(bad) == 0
    assert "libseed" in rrs.seed_version()


class _FakeState:
    def __init__(self, rrs):
        self.c = rrs.seed_state(8, 8, 8, 8)


class _Fake:
    """A stand-in tensor whose pointer is never dereferenced (validation fails first)."""

    def __init__(self, p=8):
        self.p = p

    def data_ptr(self):
        return self.p

    def numel(self):
        return 0

    def element_size(self):
        return 1


def _codes(rrs):
    f = _Fake()
    st = _FakeState(rrs)

    def decode(sh, m, **kw):
        args = dict(q=f, k=f, v=f, beta=f, g=f, vbar=f, o=f)
        args.update(kw)
        try:
            rrs.seed_decode_step(sh, st, m, args["q"], args["k"], args["v"], args["beta"],
                                 args["g"], args["vbar"], args["o"], stream=0)
        except rrs.SeedError as e:
            return e.status
        return 0

    return decode


def test_invalid_arguments_are_rejected_on_the_host():
    rrs = _lib()
    decode = _codes(rrs)
    sh = rrs.make_shape(rrs.SEED_GDN, 4, 2, 128, 128, 16, 16, rrs.SEED_BF16)
    assert decode(sh, 15) == rrs.SEED_ERR_ARG           # m < r
    assert decode(sh, 32) == rrs.SEED_ERR_ARG           # m >= r + T: no free column slot
    assert decode(sh, 16, q=_Fake(0)) == rrs.SEED_ERR_ARG
    assert decode(rrs.make_shape(rrs.SEED_GDN, 4, 2, 96, 128, 16, 16), 16) == rrs.SEED_ERR_UNSUPPORTED
    assert decode(rrs.make_shape(rrs.SEED_GDN, 4, 2, 128, 128, 48, 32), 48) == rrs.SEED_ERR_UNSUPPORTED
    assert decode(rrs.make_shape(7, 4, 2, 128, 128, 16, 16), 16) == rrs.SEED_ERR_ARG
    assert decode(rrs.make_shape(rrs.SEED_GDN, 0, 2, 128, 128, 16, 16), 16) == rrs.SEED_ERR_ARG
    assert decode(rrs.make_shape(rrs.SEED_GDN, 4, 2, 128, 128, 0, 16), 16) == rrs.SEED_ERR_ARG
    # mixed factor / io dtypes are not compiled for the decode step
    mixed = rrs.make_shape(rrs.SEED_GDN, 4, 2, 128, 128, 16, 16, rrs.SEED_BF16, rrs.SEED_F32)
    assert decode(mixed, 16) == rrs.SEED_ERR_UNSUPPORTED
    # fp16 is a factor format: fp16 inputs, and fp16 factors with fp32 inputs, are not compiled
    f16_io = rrs.make_shape(rrs.SEED_GDN, 4, 2, 128, 128, 16, 16, rrs.SEED_BF16, rrs.SEED_F16)
    assert decode(f16_io, 16) == rrs.SEED_ERR_UNSUPPORTED
    f16_f32 = rrs.make_shape(rrs.SEED_GDN, 4, 2, 128, 128, 16, 16, rrs.SEED_F16, rrs.SEED_F32)
    assert decode(f16_f32, 16) == rrs.SEED_ERR_UNSUPPORTED
    assert decode(rrs.make_shape(rrs.SEED_GDN, 4, 2, 128, 128, 16, 16, 3, 3), 16) == rrs.SEED_ERR_ARG
    # rounding: an unknown mode, or stochastic rounding of fp32 factors, is an argument error
    assert decode(rrs.make_shape(rrs.SEED_GDN, 4, 2, 128, 128, 16, 16, rrs.SEED_BF16, rounding=2), 16) == rrs.SEED_ERR_ARG
    assert decode(rrs.make_shape(rrs.SEED_GDN, 4, 2, 128, 128, 16, 16, rrs.SEED_F32,
                                 rounding=rrs.SEED_ROUND_STOCHASTIC), 16) == rrs.SEED_ERR_ARG
    st = _FakeState(rrs)
    with pytest.raises(rrs.SeedError) as e:
        rrs.seed_compress(sh, st, 33, stream=0)
    assert e.value.status == rrs.SEED_ERR_ARG
    # compress with m <= r is a no-op that touches nothing
    rrs.seed_compress(sh, st, 16, stream=0)
    # ragged compression: min_m must lie in (r, r + T]
    for bad in (16, 33, 0):
        with pytest.raises(rrs.SeedError) as e:
            rrs.seed_compress_ragged(sh, st, bad, stream=0)
        assert e.value.status == rrs.SEED_ERR_ARG
    f = _Fake()
    with pytest.raises(rrs.SeedError) as e:
        rrs.seed_decode_step_ragged(sh, st, f, f, f, f, f, _Fake(0), f, stream=0)
    assert e.value.status == rrs.SEED_ERR_ARG
    with pytest.raises(rrs.SeedError) as e:
        rrs.seed_state_from_dense(sh, _Fake(0), _Fake(), st, stream=0)
    assert e.value.status == rrs.SEED_ERR_ARG
    with pytest.raises(rrs.SeedError) as e:
        rrs.seed_dense_decode_step(sh, _Fake(), _Fake(), _Fake(), _Fake(0), _Fake(), _Fake(), _Fake(), stream=0)
    assert e.value.status == rrs.SEED_ERR_ARG
    # chunked update: 1 <= len <= 32, r <= m and m + len <= r + T; KDA and stochastic rounding
    # are not compiled for it
    assert rrs.seed_chunk_max_tokens() == 32

    def chunk(shape, m, length, q=None):
        with pytest.raises(rrs.SeedError) as e:
            rrs.seed_decode_chunk(shape, st, m, length, q if q is not None else f, f, f, f, f, f, f, stream=0)
        return e.value.status

    assert chunk(sh, 16, 0) == rrs.SEED_ERR_ARG
    assert chunk(sh, 16, 33) == rrs.SEED_ERR_ARG
    assert chunk(sh, 15, 4) == rrs.SEED_ERR_ARG          # m < r
    assert chunk(sh, 30, 3) == rrs.SEED_ERR_ARG          # 30 + 3 > r + T
    assert chunk(sh, 16, 4, q=_Fake(0)) == rrs.SEED_ERR_ARG
    kda = rrs.make_shape(rrs.SEED_KDA, 4, 2, 128, 128, 16, 32, rrs.SEED_BF16)
    assert chunk(kda, 16, 17) == rrs.SEED_ERR_UNSUPPORTED   # KDA: up to 16 tokens per call
    srd = rrs.make_shape(rrs.SEED_GDN, 4, 2, 128, 128, 16, 16, rrs.SEED_BF16,
                         rounding=rrs.SEED_ROUND_STOCHASTIC)
    assert chunk(srd, 16, 4, q=_Fake(0)) == rrs.SEED_ERR_ARG   # stochastic rounding is compiled
    # listed compression: a negative count is an argument error, an empty list does nothing
    assert rrs.LIB.seed_compress_units(ctypes.byref(sh), ctypes.byref(st.c), None, -1,
                                       None, 0, None) == rrs.SEED_ERR_ARG
    assert rrs.LIB.seed_compress_units(ctypes.byref(sh), ctypes.byref(st.c), None, 0,
                                       None, 0, None) == rrs.SEED_OK
    # ragged chunk: len > period cannot fit any unit
    with pytest.raises(rrs.SeedError) as e:
        rrs.seed_decode_chunk_ragged(sh, st, 17, f, f, f, f, f, f, f, stream=0)
    assert e.value.status == rrs.SEED_ERR_ARG
    for code in (0, -1, -2, -3, -4, 5):
        assert isinstance(rrs.seed_status_string(code), str)


def test_stream_helpers_reject_bad_arguments_on_the_host():
    # validation happens before any HIP call: no GPU is needed for these
    rrs = _lib()
    lib = rrs.LIB
    h = ctypes.c_void_p()
    one = (ctypes.c_uint32 * 1)(1)
    zero = (ctypes.c_uint32 * 1)(0)
    assert lib.seed_stream_create_cu_masked(1, None, ctypes.byref(h)) == rrs.SEED_ERR_ARG
    assert lib.seed_stream_create_cu_masked(0, one, ctypes.byref(h)) == rrs.SEED_ERR_ARG
    assert lib.seed_stream_create_cu_masked(65, one, ctypes.byref(h)) == rrs.SEED_ERR_ARG
    assert lib.seed_stream_create_cu_masked(1, zero, ctypes.byref(h)) == rrs.SEED_ERR_ARG
    assert lib.seed_stream_create_cu_masked(1, one, None) == rrs.SEED_ERR_ARG
    assert lib.seed_stream_destroy(None) == rrs.SEED_ERR_ARG


def test_one_hip_runtime_is_mapped():
    # libseed binds to the HIP runtime the process already holds; the binding refuses to load
    # beside a second copy
    rrs = _lib()
    assert len(rrs.hip_runtimes_mapped()) <= 1


def test_one_hip_runtime_when_the_package_is_imported_before_torch():
    # the binding hands torch tensors to libseed, so libseed must bind to torch's HIP runtime
    # even when the package is loaded first (in a fresh process: torch not yet imported)
    import subprocess
    import sys

    _lib()
    code = ("import rank_recurrent_state_amd as rrs\n"
            "rrs.seed_version()\n"
            "import torch\n"
            "from rank_recurrent_state_amd import _lib\n"
            "print(len(_lib.hip_runtimes_mapped()))\n")
    out = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True,
                         timeout=300)
    assert out.returncode == 0, out.stderr
    assert out.stdout.strip().splitlines()[-1] == "1"


def test_normed_step_rejects_bad_norm_on_the_host():
    rrs = _lib()
    f = _Fake()
    st = _FakeState(rrs)
    sh = rrs.make_shape(rrs.SEED_GDN, 4, 2, 128, 128, 16, 16, rrs.SEED_BF16)
    lib = rrs.LIB
    P = ctypes.c_void_p

    def call(norm):
        return lib.seed_decode_step_normed(ctypes.byref(sh), ctypes.byref(st.c), 16, P(8), P(8), P(8), P(8), P(8),
                                           P(8), norm, P(8), None)

    assert call(None) == rrs.SEED_ERR_ARG
    assert call(ctypes.byref(rrs.seed_head_norm(None, None, 1e-6, 0))) == rrs.SEED_ERR_ARG
    assert call(ctypes.byref(rrs.seed_head_norm(8, None, -1.0, 0))) == rrs.SEED_ERR_ARG
    assert call(ctypes.byref(rrs.seed_head_norm(8, None, float("nan"), 0))) == rrs.SEED_ERR_ARG
    assert call(ctypes.byref(rrs.seed_head_norm(8, None, float("inf"), 0))) == rrs.SEED_ERR_ARG
    assert call(ctypes.byref(rrs.seed_head_norm(8, None, 1e-6, 2))) == rrs.SEED_ERR_ARG
    _ = f
