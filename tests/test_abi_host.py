"""Host-side checks of the C ABI (no GPU needed).

The library must load, export every function ``include/streamkl.h``
declares, and reject bad arguments with the documented status before it
enqueues anything.  Pointers passed here are fake (never dereferenced): every
call below returns during validation, or -- on a host without a GPU -- at the
launch, with STREAMKL_ERR_HIP.
"""
import os
import re

import pytest

from attention_distillation_kl_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "streamkl.h")

A = 0x10000       # fake 16-byte aligned device addresses
A2, A3, A4 = 0x20000, 0x30000, 0x40000
O1, O2, O3 = 0x50000, 0x60000, 0x70000


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+char\s*\*|size_t|int|streamkl_status)\s*\**\s*(streamkl_\w+)\s*\(",
                                 text, flags=re.M)))


def test_header_declares_the_abi():
    assert declared_functions() == sorted(_lib.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_version_and_status_strings(lib):
    assert _lib.abi_version() == 1
    names = ["STREAMKL_OK", "STREAMKL_ERR_INVALID_ARGUMENT", "STREAMKL_ERR_UNSUPPORTED",
             "STREAMKL_ERR_WORKSPACE", "STREAMKL_ERR_HIP"]
    for code, name in enumerate(names):
        assert _lib.status_str(code) == name
        assert name in open(HEADER).read()
    assert _lib.status_str(99) == "STREAMKL_ERR_UNKNOWN"


def fwd(**kw):
    a = dict(q1=A, k1=A2, q2=A3, k2=A4, B=1, H=2, NQ=64, NK=64, d=128, scale=0.125, causal=1,
             dtype=_lib.BF16, kl=O1, lse1=O2, lse2=O3, stream=None)
    a.update(kw)
    return _lib.fwd(a["q1"], a["k1"], a["q2"], a["k2"], a["B"], a["H"], a["NQ"], a["NK"], a["d"],
                    a["scale"], a["causal"], a["dtype"], a["kl"], a["lse1"], a["lse2"], a["stream"])


def bwd(**kw):
    a = dict(q1=A, k1=A2, q2=A3, k2=A4, kl=O1, lse1=O2, lse2=O3, dkl=None, B=1, H=2, NQ=64, NK=64,
             d=128, scale=0.125, causal=1, dtype=_lib.BF16, mask=3, dq1=0x80000, dk1=0x90000,
             dq2=0xA0000, dk2=0xB0000, ws=None, wsb=None, stream=None)
    a.update(kw)
    if a["wsb"] is None:  # the declared workspace, at a fake address when there is one
        a["wsb"] = _lib.bwd_workspace_size(a["B"], a["H"], a["NQ"], a["NK"], a["d"], a["causal"], a["dtype"],
                                           a["mask"])
        if a["wsb"] and a["ws"] is None:
            a["ws"] = 0xC0000
    return _lib.bwd(a["q1"], a["k1"], a["q2"], a["k2"], a["kl"], a["lse1"], a["lse2"], a["dkl"],
                    a["B"], a["H"], a["NQ"], a["NK"], a["d"], a["scale"], a["causal"], a["dtype"],
                    a["mask"], a["dq1"], a["dk1"], a["dq2"], a["dk2"], a["ws"], a["wsb"], a["stream"])


INV, UNS = _lib.ERR_INVALID_ARGUMENT, _lib.ERR_UNSUPPORTED


@pytest.mark.parametrize("kw,status", [
    (dict(d=96), UNS), (dict(d=256), UNS), (dict(dtype=7), UNS),
    (dict(scale=0.0), INV), (dict(scale=-1.0), INV), (dict(scale=float("inf")), INV),
    (dict(scale=float("nan")), INV),
    (dict(B=-1), INV), (dict(NQ=-3), INV), (dict(NK=-1), INV), (dict(d=-64), INV),
    (dict(NQ=65, NK=64), INV),            # causal with more queries than keys
    (dict(NK=0), INV),                    # rows with no keys
    (dict(causal=2), INV),
    (dict(q1=None), INV), (dict(k2=None), INV), (dict(kl=None), INV), (dict(lse2=None), INV),
    (dict(q2=A3 + 8), INV), (dict(lse1=O2 + 4), INV),
])
def test_fwd_rejects_bad_arguments(lib, kw, status):
    assert fwd(**kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(mask=0), INV), (dict(mask=4), INV),
    (dict(mask=1, dq1=None), INV), (dict(mask=1, dk1=None), INV),
    (dict(mask=2, dq2=None), INV), (dict(mask=2, dk2=None), INV),
    (dict(lse1=None), INV), (dict(dkl=O1 + 4), INV), (dict(dk2=0xB0008), INV),
    (dict(d=32), UNS), (dict(scale=0.0), INV), (dict(NQ=70, NK=64), INV),
])
def test_bwd_rejects_bad_arguments(lib, kw, status):
    assert bwd(**kw) == status


def test_empty_problems_are_noops(lib):
    # Nothing to do: returns OK without touching the GPU.
    assert fwd(B=0) == _lib.OK
    assert fwd(NQ=0, kl=None, lse1=None, lse2=None, q1=None, q2=None) == _lib.OK
    assert fwd(H=0, NK=0) == _lib.OK
    assert bwd(B=0) == _lib.OK
    assert bwd(NQ=0, NK=0, q1=None, k1=None, q2=None, k2=None, kl=None, lse1=None, lse2=None,
               dq1=None, dk1=None, dq2=None, dk2=None) == _lib.OK


def fwd_splitk(**kw):
    a = dict(q1=A, k1=A2, q2=A3, k2=A4, B=1, H=2, NQ=64, NK=4096, d=128, scale=0.125, causal=0,
             dtype=_lib.BF16, splits=4, kl=O1, lse1=O2, lse2=O3, ws=0xC0000, wsb=None, stream=None)
    a.update(kw)
    if a["wsb"] is None:
        a["wsb"] = _lib.fwd_workspace_size(a["B"], a["H"], a["NQ"], a["NK"], a["d"], a["causal"], a["dtype"],
                                           a["splits"])
    return _lib.fwd_splitk(a["q1"], a["k1"], a["q2"], a["k2"], a["B"], a["H"], a["NQ"], a["NK"], a["d"],
                           a["scale"], a["causal"], a["dtype"], a["splits"], a["kl"], a["lse1"], a["lse2"],
                           a["ws"], a["wsb"], a["stream"])


def test_splitk_workspace_size_is_five_states_per_row_and_partition(lib):
    assert _lib.fwd_workspace_size(2, 3, 100, 5000, 128, 0, _lib.BF16, 7) == 5 * 7 * 2 * 3 * 100 * 4
    assert _lib.fwd_workspace_size(2, 3, 100, 5000, 128, 0, _lib.BF16, 1) == 0
    assert _lib.fwd_workspace_size(2, 3, 0, 5000, 128, 0, _lib.BF16, 7) == 0


@pytest.mark.parametrize("kw,status", [
    (dict(splits=0), INV), (dict(splits=-2), INV), (dict(splits=1025), INV),
    (dict(ws=None), _lib.ERR_WORKSPACE), (dict(wsb=16), _lib.ERR_WORKSPACE),
    (dict(ws=0xC0004), _lib.ERR_WORKSPACE),
    (dict(d=96), UNS), (dict(scale=0.0), INV), (dict(kl=None), INV), (dict(NQ=65, NK=64, causal=1), INV),
])
def test_fwd_splitk_rejects_bad_arguments(lib, kw, status):
    assert fwd_splitk(**kw) == status


def test_fwd_splitk_single_partition_needs_no_workspace(lib, no_gpu):
    assert fwd_splitk(splits=1, ws=None, wsb=0) == _lib.ERR_HIP


def fwd_splitk_noalloc(**kw):
    a = dict(q1=A, k1=A2, q2=A3, k2=A4, B=1, H=2, NQ=64, NK=4096, d=128, scale=0.125, causal=0,
             dtype=_lib.BF16, splits=4, kl=O1, lse1=O2, lse2=O3, stream=None)
    a.update(kw)
    return _lib.fwd_splitk_noalloc(a["q1"], a["k1"], a["q2"], a["k2"], a["B"], a["H"], a["NQ"], a["NK"], a["d"],
                                   a["scale"], a["causal"], a["dtype"], a["splits"], a["kl"], a["lse1"],
                                   a["lse2"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(splits=0), INV), (dict(splits=1025), INV), (dict(d=96), UNS), (dict(scale=0.0), INV),
    (dict(kl=None), INV), (dict(NQ=65, NK=64, causal=1), INV),
    # 5 * 64 * 32 * 2048 floats = 80 MiB of partition states: beyond the fixed scratch
    (dict(H=32, NQ=2048, NK=65536, splits=64), _lib.ERR_WORKSPACE),
])
def test_fwd_splitk_noalloc_rejects_bad_arguments(lib, kw, status):
    assert fwd_splitk_noalloc(**kw) == status


def test_fwd_splitk_noalloc_scratch_limit(lib, no_gpu):
    """The largest problem whose partition states fit the fixed scratch array
    passes validation (and, with no GPU here, fails at the device lookup);
    one more query row per head does not fit."""
    per_row = 5 * 4 * 4                       # five fp32 states, four partitions
    nq = _lib.NOALLOC_SCRATCH_BYTES // per_row // 2
    assert fwd_splitk_noalloc(NQ=nq) == _lib.ERR_HIP
    assert fwd_splitk_noalloc(NQ=nq + 1) == _lib.ERR_WORKSPACE
    assert fwd_splitk_noalloc(NQ=0) == _lib.OK          # nothing to do


def test_default_split_choice(lib):
    # short query block over long keys: split; a grid that fills the GPU: not
    assert _lib.fwd_splits(1, 32, 2048, 65536, 128, 0, _lib.BF16) > 1
    assert _lib.fwd_splits(1, 32, 32768, 32768, 128, 1, _lib.BF16) == 1
    # causal grids of more than one round whose heads fit the XCD ranges
    # balance by order, unsplit (32 x 8K: 1024 workgroups of 32 blocks a
    # head; 64 x 4K); within one round (32 x 4K, 16 x 8K: 512 workgroups)
    # key partitions still balance them
    assert _lib.fwd_splits(1, 32, 8192, 8192, 128, 1, _lib.BF16) == 1
    assert _lib.fwd_splits(1, 64, 4096, 4096, 128, 1, _lib.BF16) == 1
    assert _lib.fwd_splits(1, 32, 4096, 4096, 128, 1, _lib.BF16) == 4
    assert _lib.fwd_splits(1, 16, 8192, 8192, 128, 1, _lib.BF16) == 4
    # 12 heads x 8K: 384 workgroups, within one round
    assert _lib.fwd_splits(1, 12, 8192, 8192, 128, 1, _lib.BF16) > 1
    assert _lib.fwd_splits(1, 1, 1, 64, 128, 0, _lib.BF16) == 1      # one key tile: nothing to split
    assert _lib.fwd_splits(0, 1, 1, 64, 128, 0, _lib.BF16) == 1      # invalid sizes
    for nq, nk in ((1, 65536), (1, 1 << 20), (64, 4096)):
        s = _lib.fwd_splits(1, 8, nq, nk, 128, 0, _lib.BF16)
        assert 1 <= s <= 1024 and (nk + 63) // 64 >= 4 * s


def test_backward_workspace_query(lib):
    # query-gradient grids that fill the GPU: no workspace
    for mask in (1, 2, 3):
        assert _lib.bwd_workspace_size(2, 32, 8192, 8192, 128, 1, _lib.BF16, mask) == 0
    # short query blocks: key partitions, splits * B*H*N_Q*d floats per requested gradient
    for mask, ngrad in ((1, 1), (2, 1), (3, 2)):
        ws = _lib.bwd_workspace_size(1, 4, 100, 8192, 128, 1, _lib.BF16, mask)
        assert ws > 0 and ws % (4 * 100 * 128 * 4 * ngrad) == 0
        splits = ws // (4 * 100 * 128 * 4 * ngrad)
        assert 2 <= splits <= 256 and (8192 // 64) >= 4 * splits
    assert _lib.bwd_workspace_size(1, 4, 100, 128, 128, 1, _lib.BF16, 3) == 0   # too few key tiles
    assert _lib.bwd_workspace_size(1, 4, 64, 8192, 96, 1, _lib.BF16, 3) == 0    # invalid sizes


def test_fused_backward_selection_and_workspace(lib):
    """streamkl_bwd takes the fused form for bf16 with at most 64 queries per
    head (one query tile) while the fp32 query-gradient buffer fits the 32
    MiB of L2; its workspace is then at least one [B, H, N_Q, d] fp32 array
    per requested gradient (and still at least what the partitioned query
    half needs)."""
    sel = _lib.bwd_fused_selected
    for nq in (1, 17, 64):
        assert sel(1, 32, nq, 65536, 128, 1, _lib.BF16, 3) == 1
        assert sel(1, 32, nq, 65536, 64, 0, _lib.BF16, 1) == 1
    assert sel(1, 32, 65, 65536, 64, 0, _lib.BF16, 1) == 0        # a second query tile
    assert sel(1, 32, 65, 65536, 128, 1, _lib.BF16, 3) == 0
    assert sel(1, 32, 64, 65536, 128, 1, _lib.F32, 3) == 0        # bf16 only
    assert sel(1, 32, 0, 65536, 128, 1, _lib.BF16, 3) == 0        # nothing to add
    # 1024 heads of 64 queries: 64 MiB of fp32 sums for both gradients, 32 MiB for one
    assert sel(1, 1024, 64, 4096, 128, 0, _lib.BF16, 3) == 0
    assert sel(1, 1024, 64, 4096, 128, 0, _lib.BF16, 1) == 1
    assert sel(1, 1025, 64, 4096, 128, 0, _lib.BF16, 1) == 0
    assert sel(1, 2, 64, 32, 128, 1, _lib.BF16, 3) == 0           # causal with more queries than keys
    for mask, ngrad in ((1, 1), (2, 1), (3, 2)):
        fused = _lib.bwd_fused_workspace_size(1, 4, 64, 8192, 128, 1, _lib.BF16, mask)
        assert fused == 4 * 64 * 128 * 4 * ngrad
        assert _lib.bwd_workspace_size(1, 4, 64, 8192, 128, 1, _lib.BF16, mask) >= fused
    assert _lib.bwd_workspace_size(1, 4, 64, 128, 128, 1, _lib.BF16, 3) == 4 * 64 * 128 * 4 * 2
    assert _lib.bwd_fused_workspace_size(1, 4, 64, 8192, 128, 1, _lib.F32, 3) == 0


def test_fused_backward_rejects_bad_arguments(lib):
    def call(**kw):
        a = dict(q1=A, k1=A2, q2=A3, k2=A4, kl=O1, lse1=O2, lse2=O3, dkl=None, B=1, H=2, NQ=64, NK=8192,
                 d=128, scale=0.125, causal=1, dtype=_lib.BF16, mask=3, dq1=0x80000, dk1=0x90000,
                 dq2=0xA0000, dk2=0xB0000, ws=0xC0000, wsb=None, stream=None)
        a.update(kw)
        if a["wsb"] is None:
            a["wsb"] = _lib.bwd_fused_workspace_size(a["B"], a["H"], a["NQ"], a["NK"], a["d"], a["causal"],
                                                     a["dtype"], a["mask"])
        return _lib.bwd_fused(a["q1"], a["k1"], a["q2"], a["k2"], a["kl"], a["lse1"], a["lse2"], a["dkl"],
                              a["B"], a["H"], a["NQ"], a["NK"], a["d"], a["scale"], a["causal"], a["dtype"],
                              a["mask"], a["dq1"], a["dk1"], a["dq2"], a["dk2"], a["ws"], a["wsb"], a["stream"])
    assert call(dtype=_lib.F32, wsb=1 << 20) == UNS
    assert call(ws=None, wsb=0) == _lib.ERR_WORKSPACE
    assert call(wsb=16) == _lib.ERR_WORKSPACE
    assert call(ws=0xC0004) == _lib.ERR_WORKSPACE
    assert call(d=96) == UNS
    assert call(mask=0) == INV
    assert call(dq1=None) == INV
    assert call(NQ=65, NK=64) == INV
    assert call(B=0) == _lib.OK


def test_bwd_rejects_short_or_misaligned_workspace(lib):
    for nq in (64, 100):   # the fused and the partitioned form
        need = _lib.bwd_workspace_size(1, 2, nq, 8192, 128, 1, _lib.BF16, 3)
        assert need > 0
        kw = dict(NQ=nq, NK=8192)
        assert bwd(ws=None, wsb=0, **kw) == _lib.ERR_WORKSPACE
        assert bwd(ws=0xC0004, wsb=need, **kw) == _lib.ERR_WORKSPACE
    need = _lib.bwd_workspace_size(1, 2, 100, 8192, 128, 1, _lib.BF16, 3)
    kw = dict(NQ=100, NK=8192)
    assert bwd(ws=None, wsb=0, **kw) == _lib.ERR_WORKSPACE
    assert bwd(ws=0xC0000, wsb=need - 16, **kw) == _lib.ERR_WORKSPACE
    assert bwd(ws=0xC0004, wsb=need, **kw) == _lib.ERR_WORKSPACE


def bwd_dq_ws(**kw):
    a = dict(q1=A, k1=A2, q2=A3, k2=A4, kl=O1, lse1=O2, lse2=O3, dkl=None, B=1, H=2, NQ=64, NK=8192,
             d=128, scale=0.125, causal=1, dtype=_lib.BF16, mask=3, dq1=0x80000, dq2=0xA0000,
             ws=0xC0000, wsb=None, stream=None)
    a.update(kw)
    if a["wsb"] is None:
        a["wsb"] = _lib.bwd_workspace_size(a["B"], a["H"], a["NQ"], a["NK"], a["d"], a["causal"], a["dtype"],
                                           a["mask"])
    return _lib.bwd_dq_ws(a["q1"], a["k1"], a["q2"], a["k2"], a["kl"], a["lse1"], a["lse2"], a["dkl"],
                          a["B"], a["H"], a["NQ"], a["NK"], a["d"], a["scale"], a["causal"], a["dtype"],
                          a["mask"], a["dq1"], a["dq2"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(ws=None, wsb=0), _lib.ERR_WORKSPACE), (dict(wsb=16), _lib.ERR_WORKSPACE),
    (dict(ws=0xC0004), _lib.ERR_WORKSPACE),
    (dict(mask=0), INV), (dict(mask=1, dq1=None), INV), (dict(mask=2, dq2=None), INV),
    (dict(kl=None), INV), (dict(dq2=0xA0008), INV), (dict(d=96), UNS), (dict(NQ=8193), INV),
])
def test_bwd_dq_ws_rejects_bad_arguments(lib, kw, status):
    assert bwd_dq_ws(**kw) == status


def test_bwd_dq_ws_needs_workspace_only_where_the_query_grid_is_short(lib, no_gpu):
    assert _lib.bwd_workspace_size(1, 2, 64, 8192, 128, 1, _lib.BF16, 3) > 0
    assert bwd_dq_ws() == _lib.ERR_HIP                                   # partitioned: reaches the launch
    assert _lib.bwd_workspace_size(2, 32, 8192, 8192, 128, 1, _lib.BF16, 3) == 0
    assert bwd_dq_ws(B=2, H=32, NQ=8192, ws=None, wsb=0) == _lib.ERR_HIP  # unpartitioned: none needed
    assert bwd_dq_ws(B=0, ws=None, wsb=0) == _lib.OK                    # nothing to do


def test_unrequested_gradients_may_be_null(lib, no_gpu):
    assert bwd(mask=1, dq2=None, dk2=None) == _lib.ERR_HIP
    assert bwd(mask=2, dq1=None, dk1=None) == _lib.ERR_HIP


@pytest.fixture
def no_gpu():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present: the no-device path cannot be exercised")


def test_valid_call_without_gpu_reports_hip_error(lib, no_gpu):
    assert fwd() == _lib.ERR_HIP
    assert fwd(dtype=_lib.F32, d=64, causal=0, NQ=100, NK=37) == _lib.ERR_HIP
    assert bwd() == _lib.ERR_HIP
    assert bwd(NQ=0, q1=None, q2=None, kl=None, lse1=None, lse2=None, dq1=None, dq2=None) == _lib.ERR_HIP


def test_python_binding_refuses_cpu_tensors():
    import torch
    from attention_distillation_kl_amd import ops
    x = torch.zeros(1, 1, 4, 64)
    with pytest.raises(ValueError, match="GPU"):
        ops.streamkl_fwd(x, x, x, x)
