"""The C ABI on the CPU: the library loads, exports every symbol the header
declares, its chunk partition matches the oracle bit for bit, and every
validation error is reported before any GPU work (no device needed)."""

import ctypes
import os
import re
import subprocess

import pytest

import oracle
from context_attention_diffusion_ringattn_amd import _lib
from context_attention_diffusion_ringattn_amd._lib import Shape

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ringattn.h")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ringattn_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    return _lib.lib()


def test_header_symbols_exported(L):
    names = header_functions()
    assert names, "no declarations found in the header"
    assert sorted(_lib.EXPORTED_SYMBOLS) == names
    for n in names:
        assert hasattr(L, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True).stdout
    dyn = set(re.findall(r"\bT (ringattn_[a-z0-9_]+)", out))
    assert set(names) <= dyn


def test_abi_version_and_status_strings(L):
    assert L.ringattn_abi_version() == 6
    assert _lib.status_string(0) == "RINGATTN_OK"
    assert _lib.status_string(-1) == "RINGATTN_EINVAL"
    assert _lib.status_string(-2) == "RINGATTN_EUNSUPPORTED"
    assert _lib.status_string(-3) == "RINGATTN_EWORKSPACE"
    assert _lib.status_string(-4) == "RINGATTN_EHIP"
    assert _lib.status_string(7) == "RINGATTN_UNKNOWN_STATUS"


def _lib_offsets(L, S, N, ra):
    arr = (ctypes.c_int64 * (N + 1))()
    st = L.ringattn_chunk_offsets(S, N, ra, arr)
    return st, list(arr)


def test_offsets_bit_exact_vs_oracle(L):
    for S in range(0, 301):
        for N in range(1, 17):
            st, offs = _lib_offsets(L, S, N, 1)
            assert st == 0 and offs == oracle.chunk_offsets(S, N, ring_anything=True), (S, N)
            st, offs = _lib_offsets(L, S, N, 0)
            if S % N == 0:
                assert st == 0 and offs == oracle.chunk_offsets(S, N), (S, N)
            else:
                assert st == _lib.RINGATTN_EINVAL
                assert "divide" in _lib.last_error()


def test_offsets_workloads_and_limits(L):
    for S, N, ra in ((256, 2, 0), (4608, 4, 0), (4611, 8, 1), (16384, 1, 0), (65536, 8, 0), (4481, 4, 1),
                     (10**12 + 7, 128, 1)):
        st, offs = _lib_offsets(L, S, N, ra)
        assert st == 0 and offs == oracle.chunk_offsets(S, N, ring_anything=bool(ra))
    assert _lib_offsets(L, 10, 0, 1)[0] == _lib.RINGATTN_EINVAL
    assert _lib_offsets(L, 10, 129, 1)[0] == _lib.RINGATTN_EINVAL
    assert _lib_offsets(L, -1, 2, 1)[0] == _lib.RINGATTN_EINVAL
    assert L.ringattn_chunk_offsets(10, 2, 0, None) == _lib.RINGATTN_EINVAL


# Fake but aligned device addresses: every call below must fail validation
# before it could touch them.
P = ctypes.c_void_p(1 << 20)
P_MISALIGNED = ctypes.c_void_p((1 << 20) + 8)


def shape(B=1, H=2, D=64, Sq=128, Skv=256, reserved=0):
    return Shape(batch=B, heads=H, head_dim=D, reserved=reserved, q_len=Sq, kv_len=Skv)


@pytest.mark.parametrize("bad,code", [
    (dict(B=0), _lib.RINGATTN_EINVAL),
    (dict(H=0), _lib.RINGATTN_EINVAL),
    (dict(Sq=0), _lib.RINGATTN_EINVAL),
    (dict(Skv=-1), _lib.RINGATTN_EINVAL),
    (dict(reserved=1), _lib.RINGATTN_EINVAL),
    (dict(D=96), _lib.RINGATTN_EUNSUPPORTED),
    (dict(D=256), _lib.RINGATTN_EUNSUPPORTED),
])
def test_step_shape_errors(L, bad, code):
    s = shape(**bad)
    st = L.ringattn_step(P, P, P, P, P, ctypes.c_float(0.125), ctypes.byref(s), None)
    assert st == code
    assert _lib.last_error()


def test_step_pointer_errors(L):
    s = shape()
    f = ctypes.c_float(0.125)
    assert L.ringattn_step(None, P, P, P, P, f, ctypes.byref(s), None) == _lib.RINGATTN_EINVAL
    assert L.ringattn_step(P, None, P, P, P, f, ctypes.byref(s), None) == _lib.RINGATTN_EINVAL
    assert L.ringattn_step(P, P, None, P, P, f, ctypes.byref(s), None) == _lib.RINGATTN_EINVAL
    assert L.ringattn_step(P, P, P, None, P, f, ctypes.byref(s), None) == _lib.RINGATTN_EINVAL
    assert L.ringattn_step(P, P, P, P, None, f, ctypes.byref(s), None) == _lib.RINGATTN_EINVAL
    assert L.ringattn_step(P_MISALIGNED, P, P, P, P, f, ctypes.byref(s), None) == _lib.RINGATTN_EINVAL
    assert "aligned" in _lib.last_error()
    for bad_scale in (float("inf"), float("nan"), 0.0, -0.125):
        assert L.ringattn_step(P, P, P, P, P, ctypes.c_float(bad_scale), ctypes.byref(s), None) == \
            _lib.RINGATTN_EINVAL
    assert L.ringattn_step(P, P, P, P, P, f, None, None) == _lib.RINGATTN_EINVAL


def test_step_empty_chunk_is_noop(L):
    """kv_len = 0: nothing to attend to; the call succeeds without touching
    any buffer (null K/V are accepted)."""
    s = shape(Skv=0)
    assert L.ringattn_step(P, None, None, P, P, ctypes.c_float(0.125), ctypes.byref(s), None) == 0


def _fwd(L, offs, s, stride=0, splits=0, block_m=0, ws=None, ws_bytes=0, q=P, k=P, v=P, out=P, lse=P, scale=0.125):
    arr = _lib.offsets_array(offs) if offs is not None else None
    plan = _lib.Plan(n_splits=splits, block_m=block_m, workspace_bytes=0)
    return L.ringattn_forward(q, k, v, arr, (len(offs) - 1) if offs is not None else 1, stride, out, lse,
                              ctypes.c_float(scale), ctypes.byref(s), ctypes.byref(plan), ws, ws_bytes, None)


def _plan(L, s, offs, splits=0, block_m=0, stride=0):
    plan = _lib.Plan(n_splits=splits, block_m=block_m, workspace_bytes=0)
    st = L.ringattn_forward_plan(ctypes.byref(s), _lib.offsets_array(offs), len(offs) - 1, stride, ctypes.byref(plan))
    return st, plan


def test_forward_offset_errors(L):
    s = shape(Skv=256)
    assert _fwd(L, None, s) == _lib.RINGATTN_EINVAL
    assert _fwd(L, [1, 128, 256], s) == _lib.RINGATTN_EINVAL            # does not start at 0
    assert _fwd(L, [0, 128, 255], s) == _lib.RINGATTN_EINVAL            # does not end at kv_len
    assert _fwd(L, [0, 200, 100, 256], s) == _lib.RINGATTN_EINVAL       # decreasing
    assert _fwd(L, [0] + [2] * 129 + [256], s) == _lib.RINGATTN_EINVAL  # too many chunks
    assert _fwd(L, [0, 128, 256], s, stride=100) == _lib.RINGATTN_EINVAL  # chunk longer than the stride
    assert _fwd(L, [0, 128, 256], s, stride=-1) == _lib.RINGATTN_EINVAL
    assert _fwd(L, [0, 128, 256], s, splits=-1) == _lib.RINGATTN_EINVAL
    assert _fwd(L, [0, 128, 256], s, block_m=64) == _lib.RINGATTN_EINVAL
    assert _fwd(L, [0, 128, 256], s, out=P_MISALIGNED) == _lib.RINGATTN_EINVAL
    assert _fwd(L, [0, 128, 256], s, q=None) == _lib.RINGATTN_EINVAL
    assert _fwd(L, [0, 128, 256], s, scale=float("nan")) == _lib.RINGATTN_EINVAL
    assert _fwd(L, [0, 128, 256], s, scale=0.0) == _lib.RINGATTN_EINVAL
    assert _fwd(L, [0, 128, 256], s, scale=-0.125) == _lib.RINGATTN_EINVAL
    assert _fwd(L, [0, 128, 256], shape(D=80)) == _lib.RINGATTN_EUNSUPPORTED


def _sweep(L, offs, s, stride=0, q=P, out=P, lse=P, scale=0.125):
    arr = _lib.offsets_array(offs) if offs is not None else None
    return L.ringattn_ring_sweep(q, P, P, arr, len(offs) - 1 if offs else 0, stride, out, lse, scale,
                                 ctypes.byref(s), None)


def test_ring_sweep_errors(L):
    """The sweep validates like ringattn_forward, and needs q_len == kv_len
    (q holds every rank's rows)."""
    s = shape(Sq=256, Skv=256)
    assert _sweep(L, None, s) == _lib.RINGATTN_EINVAL
    assert _sweep(L, [0, 128, 256], shape(Sq=128, Skv=256)) == _lib.RINGATTN_EINVAL
    assert _sweep(L, [1, 128, 256], s) == _lib.RINGATTN_EINVAL
    assert _sweep(L, [0, 128, 255], s) == _lib.RINGATTN_EINVAL
    assert _sweep(L, [0, 200, 100, 256], s) == _lib.RINGATTN_EINVAL
    assert _sweep(L, [0, 128, 256], s, stride=100) == _lib.RINGATTN_EINVAL
    assert _sweep(L, [0, 128, 256], s, out=P_MISALIGNED) == _lib.RINGATTN_EINVAL
    assert _sweep(L, [0, 128, 256], s, q=None) == _lib.RINGATTN_EINVAL
    assert _sweep(L, [0, 128, 256], s, scale=0.0) == _lib.RINGATTN_EINVAL
    assert _sweep(L, [0, 128, 256], shape(D=80, Sq=256, Skv=256)) == _lib.RINGATTN_EUNSUPPORTED


def test_forward_workspace_error(L):
    """A plan with several splits and no (or too small a) workspace is refused."""
    s = shape(B=1, H=2, D=128, Sq=128, Skv=4096)
    for bm in (128, 256):
        st, plan = _plan(L, s, [0, 4096], splits=4, block_m=bm)
        assert st == 0
        assert plan.n_splits == 4 and plan.block_m == bm
        assert plan.workspace_bytes >= 4 * (128 * 2 * 128 + 2 * 128) * 4
        ws = plan.workspace_bytes
        assert _fwd(L, [0, 4096], s, splits=4, block_m=bm) == _lib.RINGATTN_EWORKSPACE
        assert _fwd(L, [0, 4096], s, splits=4, block_m=bm, ws=P, ws_bytes=ws - 1) == _lib.RINGATTN_EWORKSPACE
        assert _fwd(L, [0, 4096], s, splits=4, block_m=bm, ws=P_MISALIGNED, ws_bytes=ws) == _lib.RINGATTN_EINVAL
    assert L.ringattn_forward_plan(ctypes.byref(s), _lib.offsets_array([0, 4096]), 1, 0, None) == \
        _lib.RINGATTN_EINVAL


def test_forward_plan_properties(L):
    """Plans: a single split needs no workspace; splits never exceed the number
    of K/V tiles of the chosen kernel (64 keys for block_m 256, 32 for 128;
    packed chunks form one key range, padded chunks are tiled one by one);
    block_m is 128 or 256; the plan is deterministic and a
    request for either block size is honoured."""
    for (B, H, D, Sq, offs, stride) in ((1, 24, 128, 8192, oracle.chunk_offsets(65536, 8), 0),
                                        (1, 24, 128, 1152, oracle.chunk_offsets(4608, 4), 0),
                                        (1, 24, 128, 577, oracle.chunk_offsets(4611, 8, True), 0),
                                        (1, 24, 128, 577, oracle.chunk_offsets(4611, 8, True), 577),
                                        (1, 6, 128, 16384, [0, 16384], 0),
                                        (1, 2, 64, 128, [0, 128, 256], 0),
                                        (1, 1, 64, 1, [0, 1], 0)):
        s = shape(B=B, H=H, D=D, Sq=Sq, Skv=offs[-1])
        st, plan = _plan(L, s, offs, stride=stride)
        assert st == 0
        n = 64 if plan.block_m == 256 else 32  # keys per tile of the chosen kernel
        if stride:
            tiles = sum(-(-(b - a) // n) for a, b in zip(offs, offs[1:]))
        else:
            tiles = -(-offs[-1] // n)
        assert 1 <= plan.n_splits <= max(1, tiles)
        assert plan.block_m in (128, 256)
        assert (plan.workspace_bytes == 0) == (plan.n_splits == 1)
        st2, plan2 = _plan(L, s, offs, stride=stride)
        assert (plan2.n_splits, plan2.block_m, plan2.workspace_bytes) == \
            (plan.n_splits, plan.block_m, plan.workspace_bytes)
        for bm in (128, 256):
            st3, plan3 = _plan(L, s, offs, block_m=bm, stride=stride)
            assert st3 == 0 and plan3.block_m == bm


def test_merge_and_init_errors(L):
    s = shape()
    assert L.ringattn_merge(None, P, P, P, ctypes.byref(s), None) == _lib.RINGATTN_EINVAL
    assert L.ringattn_merge(P, P, P_MISALIGNED, P, ctypes.byref(s), None) == _lib.RINGATTN_EINVAL
    assert L.ringattn_merge(P, P, P, P, ctypes.byref(shape(D=32)), None) == _lib.RINGATTN_EUNSUPPORTED
    assert L.ringattn_acc_init(P, None, ctypes.byref(s), None) == _lib.RINGATTN_EINVAL
    assert L.ringattn_acc_init(P, P, ctypes.byref(shape(Sq=0)), None) == _lib.RINGATTN_EINVAL


def test_python_config_rules():
    from context_attention_diffusion_ringattn_amd import RingConfig
    RingConfig(ring_degree=8)
    RingConfig(ring_degree=8, ring_anything=True)
    with pytest.raises(ValueError):
        RingConfig(ring_degree=1, ring_anything=True)
    with pytest.raises(ValueError):
        RingConfig(ring_degree=2, ulysses_degree=2, ring_anything=True)
    with pytest.raises(ValueError):
        RingConfig(ring_degree=2, convert_to_fp32=False)
    with pytest.raises(ValueError):
        RingConfig(ring_degree=2, rotate_method="alltoall")
    with pytest.raises(ValueError):
        RingConfig(ring_degree=0)
    cfg = RingConfig(ulysses_degree=4, ulysses_anything=True)
    assert cfg.share(4481, 24, 3) == {"ring_index": 0, "ulysses_index": 3, "token_begin": 3361,
                                      "token_end": 4481, "q_begin": 0, "q_end": 4481,
                                      "head_begin": 18, "head_end": 24}
    with pytest.raises(ValueError):
        RingConfig(ring_degree=2, ulysses_degree=2, ulysses_anything=True)
    with pytest.raises(ValueError):
        RingConfig(ulysses_degree=1, ulysses_anything=True)


def test_python_offsets_wrapper():
    from context_attention_diffusion_ringattn_amd import RingAttnError, chunk_offsets
    assert chunk_offsets(4611, 8, ring_anything=True) == oracle.chunk_offsets(4611, 8, ring_anything=True)
    with pytest.raises(RingAttnError):
        chunk_offsets(4481, 4)


def test_bf16_state_calls_validate(L):
    """ringattn_step_bf16 and ringattn_acc_init_bf16 validate like their float32
    counterparts before any launch; an empty chunk is a no-op."""
    s = shape()
    f = ctypes.c_float(0.125)
    for args in ((None, P, P, P, P), (P, None, P, P, P), (P, P, None, P, P), (P, P, P, None, P), (P, P, P, P, None),
                 (P_MISALIGNED, P, P, P, P)):
        assert L.ringattn_step_bf16(*args, f, ctypes.byref(s), None) == _lib.RINGATTN_EINVAL
    for bad_scale in (float("inf"), float("nan"), 0.0, -1.0):
        assert L.ringattn_step_bf16(P, P, P, P, P, ctypes.c_float(bad_scale), ctypes.byref(s), None) == \
            _lib.RINGATTN_EINVAL
    assert L.ringattn_step_bf16(P, P, P, P, P, f, ctypes.byref(shape(D=96)), None) == _lib.RINGATTN_EUNSUPPORTED
    assert L.ringattn_step_bf16(P, P, P, P, P, f, None, None) == _lib.RINGATTN_EINVAL
    assert L.ringattn_step_bf16(P, None, None, P, P, f, ctypes.byref(shape(Skv=0)), None) == 0
    assert L.ringattn_acc_init_bf16(None, P, ctypes.byref(s), None) == _lib.RINGATTN_EINVAL
    assert L.ringattn_acc_init_bf16(P, None, ctypes.byref(s), None) == _lib.RINGATTN_EINVAL
    assert L.ringattn_acc_init_bf16(P, P, ctypes.byref(shape(Sq=0)), None) == _lib.RINGATTN_EINVAL
    assert L.ringattn_acc_init_bf16(P, P, ctypes.byref(shape(D=80)), None) == _lib.RINGATTN_EUNSUPPORTED


def _step_split(L, s, splits=0, block_m=0, ws=None, ws_bytes=0, q=P, k=P, v=P, out=P, lse=P, scale=0.125):
    plan = _lib.Plan(n_splits=splits, block_m=block_m, workspace_bytes=0)
    return L.ringattn_step_split(q, k, v, out, lse, ctypes.c_float(scale), ctypes.byref(s), ctypes.byref(plan), ws,
                                 ws_bytes, None)


def test_step_split_validation(L):
    """The split ring step checks its plan and workspace like forward does,
    before any launch; its workspace is the one-chunk forward plan's."""
    s = shape(B=1, H=2, D=128, Sq=128, Skv=4096)
    st, plan = _plan(L, s, [0, 4096], splits=4, block_m=256)
    assert st == 0 and plan.n_splits == 4 and plan.workspace_bytes > 0
    ws = plan.workspace_bytes
    assert _step_split(L, s, splits=4, block_m=256) == _lib.RINGATTN_EWORKSPACE
    assert _step_split(L, s, splits=4, block_m=256, ws=P, ws_bytes=ws - 1) == _lib.RINGATTN_EWORKSPACE
    assert _step_split(L, s, splits=4, block_m=256, ws=P_MISALIGNED, ws_bytes=ws) == _lib.RINGATTN_EINVAL
    assert _step_split(L, s, splits=4, block_m=100, ws=P, ws_bytes=ws) == _lib.RINGATTN_EINVAL
    assert _step_split(L, s, splits=-1) == _lib.RINGATTN_EINVAL
    assert _step_split(L, s, splits=1, block_m=256, q=None) == _lib.RINGATTN_EINVAL
    assert _step_split(L, s, splits=1, block_m=256, scale=float("nan")) == _lib.RINGATTN_EINVAL
    assert _step_split(L, shape(D=96, Sq=128, Skv=128), splits=1) == _lib.RINGATTN_EUNSUPPORTED
    # an empty chunk is the merge identity: nothing to launch, no workspace needed
    assert _step_split(L, shape(B=1, H=2, D=128, Sq=128, Skv=0), splits=4, k=None, v=None) == _lib.RINGATTN_OK


def test_workspace_layout(L):
    """A split plan's workspace holds the float32 output slots of every split,
    then their LSE slots, 16-byte aligned -- nothing else."""
    a16 = lambda x: (x + 15) // 16 * 16
    for (B, H, D, Sq, Skv, splits, bm) in ((1, 24, 128, 577, 4611, 3, 256), (2, 3, 64, 300, 5000, 5, 128)):
        st, plan = _plan(L, shape(B=B, H=H, D=D, Sq=Sq, Skv=Skv), [0, Skv], splits=splits, block_m=bm)
        assert st == 0 and plan.n_splits == splits
        lse_off = a16(splits * B * Sq * H * D * 4)
        assert plan.workspace_bytes == a16(lse_off + splits * B * H * Sq * 4)


def _noalloc(L, offs, s, splits=0, block_m=0, q=P, k=P, v=P, out=P, lse=P, scale=0.125, stride=0):
    arr = _lib.offsets_array(offs)
    plan = _lib.Plan(n_splits=splits, block_m=block_m, workspace_bytes=0)
    return L.ringattn_forward_noalloc(q, k, v, arr, len(offs) - 1, stride, out, lse, ctypes.c_float(scale),
                                      ctypes.byref(s), ctypes.byref(plan), None)


def test_forward_noalloc_validation(L):
    """The no-allocation forward validates like ringattn_forward before any
    HIP call, and rejects a requested plan whose workspace exceeds its fixed
    64 MiB scratch array with RINGATTN_EWORKSPACE and a message saying so."""
    s = shape(B=1, H=24, D=128, Sq=16384, Skv=16384)
    st, plan = _plan(L, s, [0, 16384], splits=4, block_m=256)
    assert st == 0 and plan.workspace_bytes > (64 << 20)
    assert _noalloc(L, [0, 16384], s, splits=4, block_m=256) == _lib.RINGATTN_EWORKSPACE
    assert "workspace" in _lib.last_error()
    assert _noalloc(L, [0, 16384], s, q=None) == _lib.RINGATTN_EINVAL
    assert _noalloc(L, [0, 16384], s, scale=-1.0) == _lib.RINGATTN_EINVAL
    assert _noalloc(L, [0, 100], s) == _lib.RINGATTN_EINVAL
    assert _noalloc(L, [0, 16384], shape(D=32, Sq=16384, Skv=16384)) == _lib.RINGATTN_EUNSUPPORTED
