"""Host-side checks of the several-readers entry points (readyPrepSize,
readyStatePrepare, readyStateApply): sizes, and every argument error, which
the library finds before it launches anything (no GPU needed)."""
import ctypes

import pytest

import hla_recurrent_state_amd as R
from tests.test_abi import _lib, _shape, _Fake


def _plan(shape, layer_ids=(0, 1)):
    _lib()
    st, plan = R.readyPlanCreate(shape, list(layer_ids))
    assert st == R.READY_OK
    return plan


def test_prep_size_closed_form():
    B, L_sel, H, r = 3, 2, 4, 8
    plan = _plan(_shape(B=B, L_sel=L_sel, H=H, r=r))
    M = L_sel * H
    up = lambda x: (x + 255) // 256 * 256
    for n_inj in (1, 3, 8):
        st, n = R.readyPrepSize(plan, n_inj)
        assert st == R.READY_OK
        assert n == up(4 * n_inj * B * M * r * r) + up(4 * B * M) + up(4 * B)
    R.readyPlanDestroy(plan)


def test_prep_size_rejects_injection_counts():
    plan = _plan(_shape())
    for n_inj in (0, -1, R.READY_MAX_INJ + 1):
        assert R.readyPrepSize(plan, n_inj)[0] == R.READY_ERR_BAD_SHAPE
    R.readyPlanDestroy(plan)


@pytest.mark.parametrize("kw", [dict(state_dtype="f32"), dict(weight_dtype="f32"), dict(act_dtype="f32"),
                                dict(r=64)])
def test_multi_reader_needs_the_single_kernel_path(kw):
    plan = _plan(_shape(**kw))
    assert R.readyPrepSize(plan, 2)[0] == R.READY_ERR_UNSUPPORTED
    R.readyPlanDestroy(plan)


def _prep_args(shape, n_inj=3, layer_ids=(0, 1)):
    plan = _plan(shape, layer_ids)
    _, ws_bytes = R.readyWorkspaceSize(plan)
    _, prep_bytes = R.readyPrepSize(plan, n_inj)
    f = _Fake(shape)
    B, P, L, H = shape.B, shape.P, shape.L_tot, shape.H
    M = shape.L_sel * H
    tile = 128 * 128
    states = R.readyStates(base=f.alloc(B * P * L * H * tile * 2), stride_b=P * L * H * tile,
                           stride_p=L * H * tile, stride_l=H * tile, stride_h=tile)
    ws = (R.readyWeights * n_inj)(*[R.readyWeights(u=f.alloc(M * shape.r * 128 * 2), v=f.alloc(M * shape.r * 128 * 2))
                                   for _ in range(n_inj)])
    return dict(plan=plan, states=states, accept_idx=f.alloc(4 * max(B, 1)), n_inj=n_inj, inj_weights=ws,
                gathered=f.alloc(B * M * tile * 2), logrms=None, dev_status=None, prep=f.alloc(prep_bytes),
                prep_bytes=prep_bytes, workspace=f.alloc(ws_bytes), workspace_bytes=ws_bytes, stream=None)


def _prepare(shape, mutate=None, **kw):
    a = _prep_args(shape, **kw)
    if mutate:
        mutate(a)
    code = R.readyStatePrepare(**a)
    R.readyPlanDestroy(a["plan"])
    return code


def test_prepare_zero_batch_is_ok():
    assert _prepare(_shape(B=0)) == R.READY_OK


def test_prepare_argument_errors():
    def set_(k, v):
        def f(a):
            a[k] = v
        return f

    def null_u(a):
        a["inj_weights"][1].u = None

    def null_states(a):
        a["states"].base = None
    for m in (set_("accept_idx", None), set_("gathered", None), set_("prep", None), set_("workspace", None),
              null_u, null_states):
        assert _prepare(_shape(), mutate=m) == R.READY_ERR_NULL_POINTER
    assert _prepare(_shape(), mutate=set_("n_inj", 0)) == R.READY_ERR_BAD_SHAPE
    assert _prepare(_shape(), mutate=set_("n_inj", R.READY_MAX_INJ + 1)) == R.READY_ERR_BAD_SHAPE

    def small_prep(a):
        a["prep_bytes"] -= 256

    def small_ws(a):
        a["workspace_bytes"] -= 256
    assert _prepare(_shape(), mutate=small_prep) == R.READY_ERR_WORKSPACE_TOO_SMALL
    assert _prepare(_shape(), mutate=small_ws) == R.READY_ERR_WORKSPACE_TOO_SMALL

    def mis_prep(a):
        a["prep"] += 16

    def mis_v(a):
        a["inj_weights"][2].v += 2

    def mis_stride(a):
        a["states"].stride_h += 3
    for m in (mis_prep, mis_v, mis_stride):
        assert _prepare(_shape(), mutate=m) == R.READY_ERR_MISALIGNED

    def prep_on_u(a):
        a["prep"] = a["inj_weights"][2].u

    def gathered_in_states(a):
        a["gathered"] = a["states"].base + 128 * 128 * 2

    def prep_on_ws(a):
        a["prep"] = a["workspace"]
    for m in (prep_on_u, gathered_in_states, prep_on_ws):
        assert _prepare(_shape(), mutate=m) == R.READY_ERR_ALIASING


def _apply_args(shape, n_inj=3, inj=1):
    plan = _plan(shape)
    _, ws_bytes = R.readyWorkspaceSize(plan)
    _, prep_bytes = R.readyPrepSize(plan, n_inj)
    f = _Fake(shape)
    B, n, d, r, Hm = shape.B, shape.n, shape.d, shape.r, shape.Hm
    M = shape.L_sel * shape.H
    F = M * (r + 1)
    w = R.readyWeights(wq=f.alloc(M * r * d * 2), w1=f.alloc(Hm * F * 2), w2=f.alloc(d * Hm * 2))
    o = R.readyOutputs(out=f.alloc(B * n * d * 2))
    return dict(plan=plan, prep=f.alloc(prep_bytes), prep_bytes=prep_bytes, n_inj=n_inj, inj=inj,
                h=f.alloc(B * n * d * 2), weights=w, outputs=o, workspace=f.alloc(ws_bytes), workspace_bytes=ws_bytes,
                stream=None)


def _apply(shape, mutate=None, **kw):
    a = _apply_args(shape, **kw)
    if mutate:
        mutate(a)
    code = R.readyStateApply(**a)
    R.readyPlanDestroy(a["plan"])
    return code


def test_apply_zero_batch_and_in_place_are_ok():
    def in_place(a):
        a["outputs"].out = a["h"]
    assert _apply(_shape(B=0)) == R.READY_OK
    assert _apply(_shape(B=0), mutate=in_place) == R.READY_OK


def test_apply_argument_errors():
    def set_(k, v):
        def f(a):
            a[k] = v
        return f

    def null_w1(a):
        a["weights"].w1 = None

    def null_out(a):
        a["outputs"].out = None
    for m in (set_("prep", None), set_("h", None), set_("workspace", None), null_w1, null_out):
        assert _apply(_shape(), mutate=m) == R.READY_ERR_NULL_POINTER
    for m in (set_("inj", 3), set_("inj", -1), set_("n_inj", 0), set_("n_inj", R.READY_MAX_INJ + 1)):
        assert _apply(_shape(), mutate=m) == R.READY_ERR_BAD_SHAPE
    assert _apply(_shape(), mutate=set_("workspace_bytes", 256)) == R.READY_ERR_WORKSPACE_TOO_SMALL
    assert _apply(_shape(), mutate=set_("prep_bytes", 256)) == R.READY_ERR_WORKSPACE_TOO_SMALL

    def mis_h(a):
        a["h"] += 2

    def mis_prep(a):
        a["prep"] += 64
    for m in (mis_h, mis_prep):
        assert _apply(_shape(), mutate=m) == R.READY_ERR_MISALIGNED

    def out_on_prep(a):
        a["outputs"].out = a["prep"]

    def out_overlaps_h(a):
        a["outputs"].out = a["h"] + 64

    def delta_on_h(a):
        a["outputs"].delta = a["h"]
    for m in (out_on_prep, out_overlaps_h, delta_on_h):
        assert _apply(_shape(), mutate=m) == R.READY_ERR_ALIASING


def test_apply_unsupported_plan():
    assert _apply(_shape(state_dtype="f32")) == R.READY_ERR_UNSUPPORTED
