"""Every kernel path through the bounds-checked debug build.

libstreamkl_debug.so runs the same sources with every global-memory access,
and the LDS accesses of the tile loops, checked against its buffer's extent;
an access out of range is not made, and streamkl_debug_take reports the
first one.  Each case below runs the forward (library partition count,
explicit partitions, the no-alloc form), the selected backward, its two
halves with their workspace and, for bf16, the fused backward through the
debug build, and requires:
  * no out-of-range access (streamkl_debug_take() == 0);
  * the results of the release build, bit for bit (the checks change no
    arithmetic); query gradients added by atomics in a varying order (the
    fused backward's, and the selected backward's where it is the fused
    one) to the bf16 tolerance;
  * on the small cases, the fp64 oracle at the stated tolerances.
The cases reach every kernel instantiation family: bf16/fp32, d = 64/128,
causal or not, ragged sizes, decoding rows (the row-major split-K kernel),
partitioned query and key gradients, paired and unpaired key-gradient
layouts, the fused backward's one-tile and tiled forms, and the causal
grid orders (longest-first, rank-major).
"""
import pytest
import torch

from attention_distillation_kl_amd import _lib, make_inputs, ops
from attention_distillation_kl_amd.inputs import upstream_grad
from parity_util import check_grad, check_rows, log, oracle_heads, to64

pytestmark = pytest.mark.gpu

DEV = "cuda"

#      B, H,  NQ,    NK,    d,   dtype,          causal, mask, g,     splits, oracle
CASES = [
    (1, 2, 300, 517, 128, torch.bfloat16, True, 3, True, None, True),
    (2, 1, 100, 70, 64, torch.float32, False, 3, False, None, True),
    (1, 3, 129, 900, 64, torch.bfloat16, True, 1, True, 5, True),
    (1, 2, 77, 333, 128, torch.float32, True, 2, False, 3, True),
    (1, 4, 17, 3000, 128, torch.bfloat16, False, 3, True, 16, True),     # decoding-row kernel
    (1, 8, 1, 9000, 128, torch.bfloat16, True, 3, False, None, False),  # one query row
    (1, 2, 40, 5000, 128, torch.bfloat16, True, 3, True, None, True),   # fused one-tile form
    (1, 32, 512, 4096, 128, torch.bfloat16, True, 3, False, None, False),  # partitioned dQ, longest-first
    (1, 1, 8192, 8192, 128, torch.bfloat16, True, 3, True, None, False),   # partitioned dK
    (1, 16, 8192, 8192, 128, torch.bfloat16, True, 3, False, None, False),  # unpaired dK
    (1, 4, 32768, 32768, 128, torch.bfloat16, True, 3, False, None, False),  # rank-major orders
    (1, 32, 4096, 4096, 64, torch.bfloat16, True, 2, True, None, False),  # longest-first, d = 64
]


def _run(q1, k1, q2, k2, scale, causal, mask, g, splits):
    out = {}
    kl, l1, l2 = ops.streamkl_fwd(q1, k1, q2, k2, scale, causal, splits=splits)
    out.update(kl=kl, lse1=l1, lse2=l2)
    grads = ops.streamkl_bwd(q1, k1, q2, k2, kl, l1, l2, g, scale, causal, mask)
    out.update({f"bwd_{n}": t for n, t in zip(("dq1", "dk1", "dq2", "dk2"), grads) if t is not None})
    ws = ops.streamkl_bwd_workspace(q1, k1, causal, mask)
    dk = ops.streamkl_bwd_half("dk", q1, k1, q2, k2, kl, l1, l2, g, scale, causal, mask, workspace=ws)
    dq = ops.streamkl_bwd_half("dq", q1, k1, q2, k2, kl, l1, l2, g, scale, causal, mask, workspace=ws)
    out.update({f"half_{n}": t for n, t in zip(("dk1", "dk2"), dk) if t is not None})
    out.update({f"half_{n}": t for n, t in zip(("dq1", "dq2"), dq) if t is not None})
    if q1.dtype == torch.bfloat16:
        fused = ops.streamkl_bwd_fused(q1, k1, q2, k2, kl, l1, l2, g, scale, causal, mask)
        out.update({f"fused_{n}": t for n, t in zip(("dq1", "dk1", "dq2", "dk2"), fused) if t is not None})
    B, H, NQ, d = q1.shape
    sp = splits if splits and splits > 1 else 4
    if NQ * B * H * 5 * sp * 4 <= _lib.NOALLOC_SCRATCH_BYTES:
        kl2 = torch.empty_like(kl)
        a2, b2 = torch.empty_like(kl), torch.empty_like(kl)
        dt = _lib.BF16 if q1.dtype == torch.bfloat16 else _lib.F32
        st = _lib.fwd_splitk_noalloc(q1.data_ptr(), k1.data_ptr(), q2.data_ptr(), k2.data_ptr(), B, H, NQ,
                                     k1.shape[2], d, scale, int(causal), dt, sp, kl2.data_ptr(), a2.data_ptr(),
                                     b2.data_ptr(), torch.cuda.current_stream().cuda_stream)
        assert st == _lib.OK, _lib.status_str(st)
        out.update(noalloc_kl=kl2, noalloc_lse1=a2, noalloc_lse2=b2)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("case", range(len(CASES)))
def test_debug_build_has_no_out_of_range_access(case, monkeypatch):
    B, H, NQ, NK, d, dt, causal, mask, use_g, splits, with_oracle = CASES[case]
    tag = f"debug case {case}: B={B} H={H} NQ={NQ} NK={NK} d={d} {dt} causal={causal} mask={mask} g={use_g} splits={splits}"
    log(tag)
    dbg = _lib.load(_lib.DEBUG_LIB_PATH)
    assert _lib.debug_take(dbg) == 0, "a record left over from an earlier call"
    q1, k1, q2, k2 = make_inputs(B, H, NQ, NK, d, dt, "student", 0.3, seed=900 + case, device=DEV)
    g = upstream_grad(B, H, NQ, seed=case, device=DEV) if use_g else None
    scale = d ** -0.5
    rel = _run(q1, k1, q2, k2, scale, causal, mask, g, splits)
    with monkeypatch.context() as m:
        m.setattr(_lib, "load", lambda path=None: dbg)
        got = _run(q1, k1, q2, k2, scale, causal, mask, g, splits)
    site = _lib.debug_take(dbg)
    assert site == 0, f"{tag}: out-of-range access at {_lib.debug_site(site)}"
    assert got.keys() == rel.keys()
    # Query gradients added by atomics in a varying order: the fused
    # backward's, and streamkl_bwd's where it selects the fused form.
    fused_sel = dt == torch.bfloat16 and _lib.bwd_fused_selected(B, H, NQ, NK, d, int(causal), _lib.BF16, mask)
    unordered = ("fused_dq", "bwd_dq") if fused_sel else ("fused_dq",)
    differ = []
    for name, t in got.items():
        if torch.equal(t, rel[name]):
            continue
        differ.append(name)
        if name.startswith(unordered):
            for hh in range(B * H):
                b, h = divmod(hh, H)
                check_grad(to64(t[b, h]), to64(rel[name][b, h]), dt, f"{tag} {name} head {hh}")
        else:
            raise AssertionError(f"{tag}: {name} differs from the release build")
    log(f"{tag}: no out-of-range access; bitwise equal to the release build except {differ or 'nothing'}")
    if not with_oracle:
        return
    heads = list(range(B * H))
    ref = oracle_heads(q1, k1, q2, k2, scale, causal, heads, g=g, grads=True)
    for hh in heads:
        b, h = divmod(hh, H)
        for name, t in got.items():
            base = name.rsplit("_", 1)[-1]
            if base in ("kl", "lse1", "lse2"):
                check_rows(to64(t[b, h]), ref[hh][base], dt, f"{tag} head {hh} {name}")
            else:
                check_grad(to64(t[b, h]), ref[hh][base], dt, f"{tag} head {hh} {name}")
