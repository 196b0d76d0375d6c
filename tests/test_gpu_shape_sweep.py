"""GPU parity over head shapes the configurations do not reach: rotation widths and GQA group sizes.

Rotation widths, on prefill, decode (bf16 and fp8 caches), chunked extend and the multi-token
extend: no rotated dim, 16 and 48 (half-widths 8 and 24: a dim's partner sits in the other half of
the wave), two thirds of the head and every dim.

The kernels find the partner of a rotated dim in different places depending on the width (another
lane, another chunk of the same lane, a table row), and the decode kernel compiles a separate
variant for widths beyond 64, so each path is run at each width.  Inputs are the workloads' own:
q, k, v ~ N(0,1) at full scale and each kind's theta (1e4 sliding, 5e6 global).  Besides the
fixed bound, prefill and decode are held to the rounding model (tests/rounding_model.py): every
rotated dim is one more bf16 rounding of an operand, so the error grows with the width, and the
kernel's L2 error must stay within a small factor of what ideal bf16 arithmetic gives at that
width.  Seeds: 7000 + width + kind (+ path offset).
"""
import pytest

from tests import rounding_model
from tests.gpu_helpers import assert_close, assert_near_model
from tests.test_gpu_extend import run_extend_case
from tests.test_gpu_fp8 import _check_key_codes, _decode8_case, _np8, run_prefill_fp8_chain
from tests.test_gpu_parity import _decode_case, _f32, _note, _oparams, _run_prefill, _wl

pytestmark = pytest.mark.gpu

WIDTHS = [0, 16, 48, 128, 192]


@pytest.mark.parametrize("kind", [0, 1])
@pytest.mark.parametrize("r", WIDTHS)
def test_prefill_rope_widths(kind, r):
    # GQA group 4: the sliding kind takes its grouped kernel (cos/sin table of the rows)
    w = _wl(kind=kind, B=2, S=150, Hq=8, Hkv=2, sinks=kind == 1, r=r)
    _note(f"prefill kind={kind} r={r}")
    q, k, v, s, out, ref, _, _, pos = _run_prefill(w, seed=7000 + r + kind, starts=[0, 517])
    bound = rounding_model.prefill_bound(_oparams(w), _f32(q), _f32(k), _f32(v), pos, _f32(s))
    assert_close(out, ref, what=f"prefill kind={kind} r={r}", bound=bound)
    model = rounding_model.prefill(_oparams(w), _f32(q), _f32(k), _f32(v), pos, _f32(s))
    assert_near_model(out, ref, model, what=f"prefill kind={kind} r={r}")


@pytest.mark.parametrize("kind", [0, 1])
@pytest.mark.parametrize("r", WIDTHS)
def test_decode_rope_widths(kind, r):
    positions = [0, 130, 3000]
    w = _wl(kind=kind, B=len(positions), S=1, Hq=8, Hkv=2, sinks=kind == 1, r=r)
    _note(f"decode kind={kind} r={r} positions {positions}")
    out, ref, model = _decode_case(w, positions, seed=7100 + r + kind, with_model=True)
    assert_close(out, ref, what=f"decode kind={kind} r={r}")
    assert_near_model(out, ref, model, what=f"decode kind={kind} r={r}")


@pytest.mark.parametrize("kind", [0, 1])
@pytest.mark.parametrize("r", WIDTHS)
def test_decode_fp8_rope_widths(kind, r):
    # fp8 caches: the query's dims are taken in the order one 16-byte load of key codes splits
    # into, and the appended key is coded after its rotation
    positions = [0, 130, 3000]
    w = _wl(kind=kind, B=len(positions), S=1, Hq=8, Hkv=2, sinks=kind == 1, r=r)
    _note(f"fp8 decode kind={kind} r={r} positions {positions}")
    out, ref, krot, _, vcode, kc8, vc8, _, _ = _decode8_case(w, positions, 7500 + r + kind)
    assert_close(out, ref, what=f"fp8 decode kind={kind} r={r}")
    kc1, vc1 = _np8(kc8), _np8(vc8)
    for b, p in enumerate(positions):
        slot = p % w.window if kind == 1 else p
        assert (vc1[b, :, slot] == vcode[b]).all(), f"seq {b}: value codes"
        _check_key_codes(kc1[b, :, slot], krot[b], f"seq {b} r={r}")


@pytest.mark.parametrize("kind", [0, 1])
@pytest.mark.parametrize("r", [0, 192])
def test_prefill_fp8_caches_rope_widths(kind, r):
    # prefill coding the rotated keys it stores, then a decode step over those codes
    run_prefill_fp8_chain(kind, seed=7600 + r + kind, r=r)


@pytest.mark.parametrize("S", [40, 4])
@pytest.mark.parametrize("kind", [0, 1])
@pytest.mark.parametrize("r", WIDTHS)
def test_extend_rope_widths(kind, r, S):
    # S = 40: the chunked path (prefill kernel on the cache); S = 4: the multi-token tile kernel
    case = dict(kind=kind, B=2, S=S, Hq=8, Hkv=2, sinks=kind == 1, starts=[3, 700], r=r)
    run_extend_case(case, 7200 + r + kind + S)


# ----------------------------------------------------------------------------- GQA group sizes
# The decode kernel packs a group's query heads as the 16 columns of its products and the
# multi-token kernel packs (head, token) pairs as columns, so group sizes from 1 to 16 (and, for
# extend, token counts that fill a column block exactly or leave it ragged) are run on both kinds.

@pytest.mark.parametrize("kind", [0, 1])
@pytest.mark.parametrize("Hq,Hkv", [(8, 8), (8, 4), (16, 1)])
def test_decode_group_sizes(kind, Hq, Hkv):
    positions = [7, 129, 2500]
    w = _wl(kind=kind, B=len(positions), S=1, Hq=Hq, Hkv=Hkv, sinks=kind == 1)
    _note(f"decode kind={kind} Hq={Hq} Hkv={Hkv}")
    out, ref, *_ = _decode_case(w, positions, seed=7300 + Hq + Hkv + kind)
    assert_close(out, ref, what=f"decode kind={kind} group {Hq // Hkv}")


@pytest.mark.parametrize("S", [1, 3, 16])
@pytest.mark.parametrize("kind", [0, 1])
@pytest.mark.parametrize("Hq,Hkv", [(8, 8), (8, 4), (16, 1)])
def test_extend_group_sizes(kind, Hq, Hkv, S):
    case = dict(kind=kind, B=2, S=S, Hq=Hq, Hkv=Hkv, sinks=kind == 1, starts=[0, 301])
    run_extend_case(case, 7400 + Hq + Hkv + kind + S)
