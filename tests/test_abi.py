"""Host-side tests of the C ABI (CPU only, no GPU needed).

The library must load, export every symbol include/ready.h declares, and
reject every malformed argument before touching the HIP runtime.  No test
here lets a call reach a kernel launch: each either fails validation or has
B = 0 (a valid no-op).
"""
import ctypes
import os
import re

import pytest

import hla_recurrent_state_amd as R

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _lib():
    try:
        return R.load()
    except R.ReadyError:
        import __graft_entry__
        __graft_entry__.build_library()
        return R.load()


def test_exports_every_declared_symbol():
    lib = _lib()
    header = open(os.path.join(ROOT, "include", "ready.h")).read()
    declared = set(re.findall(r"^\s*(?:readyStatus|const char\*|int32_t)\s+(ready\w+)\s*\(", header, re.M))
    assert declared == set(R.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name
    assert R.readyVersion() == 100


def test_status_strings():
    _lib()
    for code, name in [(0, "READY_OK"), (6, "READY_ERR_ALIASING"), (9, "READY_ERR_ACCEPT_IDX")]:
        assert R.readyStatusString(code) == name
    assert R.readyStatusString(999) == "READY_ERR_UNKNOWN"


def _shape(**kw):
    base = dict(B=2, P=8, n=7, L_tot=3, L_sel=2, H=4, r=8, d=512, Hm=64)
    base.update(kw)
    return R.make_shape(**base)


@pytest.mark.parametrize("kw,code", [
    (dict(B=-1), R.READY_ERR_BAD_SHAPE),
    (dict(P=0), R.READY_ERR_BAD_SHAPE),
    (dict(P=65), R.READY_ERR_BAD_SHAPE),
    (dict(n=0), R.READY_ERR_BAD_SHAPE),
    (dict(n=17), R.READY_ERR_BAD_SHAPE),
    (dict(H=0), R.READY_ERR_BAD_SHAPE),
    (dict(r=12), R.READY_ERR_BAD_SHAPE),
    (dict(r=136), R.READY_ERR_BAD_SHAPE),
    (dict(d=100), R.READY_ERR_BAD_SHAPE),
    (dict(Hm=0), R.READY_ERR_BAD_SHAPE),
    (dict(d_k=64), R.READY_ERR_BAD_SHAPE),
    (dict(state_eps=-1.0), R.READY_ERR_BAD_SHAPE),
    (dict(B=1 << 19, n=4), R.READY_ERR_BAD_SHAPE),
])
def test_plan_rejects_bad_shapes(kw, code):
    _lib()
    st, plan = R.readyPlanCreate(_shape(**kw), [0, 1])
    assert st == code
    assert not plan.value


def test_plan_path_selector():
    _lib()
    st, _ = R.readyPlanCreate(_shape(path="fused"), [0, 1])
    assert st == R.READY_OK
    bad = _shape()
    bad.path = 2
    assert R.readyPlanCreate(bad, [0, 1])[0] == R.READY_ERR_BAD_SHAPE
    # the unfused path never takes the single kernel, so the shared-gather
    # entry points (which need it) report it as unsupported
    st, plan = R.readyPlanCreate(_shape(path="unfused"), [0, 1])
    assert st == R.READY_OK and R.readyPrepSize(plan, 2)[0] == R.READY_ERR_UNSUPPORTED
    st, plan = R.readyPlanCreate(_shape(path="fused"), [0, 1])
    assert st == R.READY_OK and R.readyPrepSize(plan, 2)[0] == R.READY_OK


def test_plan_rejects_bad_dtype_and_activation():
    _lib()
    s = _shape()
    s.state_dtype = 7
    assert R.readyPlanCreate(s, [0, 1])[0] == R.READY_ERR_UNSUPPORTED_DTYPE
    s = _shape()
    s.act = 9
    assert R.readyPlanCreate(s, [0, 1])[0] == R.READY_ERR_UNSUPPORTED_DTYPE


def test_plan_rejects_layer_ids_out_of_range():
    _lib()
    assert R.readyPlanCreate(_shape(), [0, 3])[0] == R.READY_ERR_LAYER_ID_RANGE
    assert R.readyPlanCreate(_shape(), [-1, 0])[0] == R.READY_ERR_LAYER_ID_RANGE
    st, plan = R.readyPlanCreate(_shape(), [2, 2])      # repeats are allowed
    assert st == R.READY_OK
    R.readyPlanDestroy(plan)


def test_null_arguments():
    lib = _lib()
    assert lib.readyPlanCreate(None, None, None) == R.READY_ERR_NULL_POINTER
    assert lib.readyWorkspaceSize(None, None) == R.READY_ERR_NULL_POINTER
    assert lib.readyPlanDestroy(None) == R.READY_OK


def test_workspace_size_grows_with_batch():
    _lib()
    sizes = []
    for B in (0, 1, 64):
        st, plan = R.readyPlanCreate(_shape(B=B), [0, 1])
        assert st == R.READY_OK
        st, n = R.readyWorkspaceSize(plan)
        assert st == R.READY_OK and n % 256 == 0
        sizes.append(n)
        R.readyPlanDestroy(plan)
    assert sizes[0] <= sizes[1] < sizes[2]


class _Fake:
    """Host-side fake device addresses (never dereferenced: every call below
    fails validation or is a B = 0 no-op)."""

    def __init__(self, shape):
        self.s = shape
        self.next = 1 << 40

    def alloc(self, nbytes):
        p = self.next
        self.next += (nbytes + 4095) // 4096 * 4096 + 4096
        return p


def _call(shape, layer_ids=(0, 1), mutate=None, static=False):
    _lib()
    st, plan = R.readyPlanCreate(shape, list(layer_ids))
    assert st == R.READY_OK
    _, ws_bytes = R.readyWorkspaceSize(plan)
    f = _Fake(shape)
    B, P, L, H, n, d, r, Hm = shape.B, shape.P, shape.L_tot, shape.H, shape.n, shape.d, shape.r, shape.Hm
    M = shape.L_sel * H
    F = M * (r + 1)
    es = 2
    tile = 128 * 128
    states = R.readyStates(base=f.alloc(B * P * L * H * tile * es), stride_b=P * L * H * tile,
                           stride_p=L * H * tile, stride_l=H * tile, stride_h=tile)
    w = R.readyWeights(wq=f.alloc(M * r * d * es), u=f.alloc(M * r * 128 * es), v=f.alloc(M * r * 128 * es),
                       h_gamma=None, w1=f.alloc(Hm * F * es), b1=None, w2=f.alloc(d * Hm * es), b2=None)
    o = R.readyOutputs(gathered=f.alloc(B * M * tile * es), out=f.alloc(B * n * d * es), logrms=None,
                       delta=None, feat=None, dev_status=None)
    args = dict(plan=plan, states=states, accept_idx=f.alloc(4 * max(B, 1)), h=f.alloc(B * n * d * es),
                weights=w, outputs=o, workspace=f.alloc(ws_bytes), workspace_bytes=ws_bytes, stream=None)
    if mutate:
        mutate(args)
    if static:
        code = R.readyStateReaderStatic(args["plan"], args["states"], args["accept_idx"], args["h"],
                                        args["weights"], args["outputs"], args["stream"])
    else:
        code = R.readyStateReader(**args)
    R.readyPlanDestroy(plan)
    return code


def test_zero_batch_valid_call_is_ok():
    assert _call(_shape(B=0)) == R.READY_OK


def test_reader_null_pointers():
    def m(field):
        def f(a):
            if field == "states":
                a["states"].base = None
            elif field.startswith("w."):
                setattr(a["weights"], field[2:], None)
            elif field.startswith("o."):
                setattr(a["outputs"], field[2:], None)
            else:
                a[field] = None
        return f
    for field in ("states", "accept_idx", "h", "workspace", "w.wq", "w.u", "w.v", "w.w1", "w.w2",
                  "o.gathered", "o.out"):
        assert _call(_shape(), mutate=m(field)) == R.READY_ERR_NULL_POINTER, field


def test_reader_workspace_too_small():
    def m(a):
        a["workspace_bytes"] -= 256
    assert _call(_shape(), mutate=m) == R.READY_ERR_WORKSPACE_TOO_SMALL


def test_reader_misaligned_pointers_and_strides():
    for what in ("h", "wq", "gathered", "states", "workspace"):
        def m(a, what=what):
            if what == "h":
                a["h"] += 2
            elif what == "wq":
                a["weights"].wq += 8
            elif what == "gathered":
                a["outputs"].gathered += 4
            elif what == "states":
                a["states"].base += 2
            else:
                a["workspace"] += 16
        assert _call(_shape(), mutate=m) == R.READY_ERR_MISALIGNED, what

    def stride(a):
        a["states"].stride_h += 3          # 6 bytes: tiles no longer 16-byte aligned
    assert _call(_shape(), mutate=stride) == R.READY_ERR_MISALIGNED

    def negative(a):
        a["states"].stride_p = -a["states"].stride_p
    assert _call(_shape(), mutate=negative) == R.READY_ERR_BAD_SHAPE


def test_reader_aliasing_rules():
    def gathered_in_states(a):
        a["outputs"].gathered = a["states"].base + 128 * 128 * 2
    assert _call(_shape(), mutate=gathered_in_states) == R.READY_ERR_ALIASING

    def out_overlaps_h(a):
        a["outputs"].out = a["h"] + 64            # partial overlap
    assert _call(_shape(), mutate=out_overlaps_h) == R.READY_ERR_ALIASING

    def out_on_weights(a):
        a["outputs"].out = a["weights"].w2
    assert _call(_shape(), mutate=out_on_weights) == R.READY_ERR_ALIASING

    def ws_on_gathered(a):
        a["workspace"] = a["outputs"].gathered
    assert _call(_shape(), mutate=ws_on_gathered) == R.READY_ERR_ALIASING

    def delta_on_feat(a):
        p = a["workspace"] + (1 << 30)
        a["outputs"].delta = p
        a["outputs"].feat = p + 16
    assert _call(_shape(), mutate=delta_on_feat) == R.READY_ERR_ALIASING

    def in_place_b0(a):
        a["outputs"].out = a["h"]                 # exactly in place is allowed
    assert _call(_shape(B=0), mutate=in_place_b0) == R.READY_OK


def test_python_binding_raises_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(R, "_lib", None)
    monkeypatch.setattr(R, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(R.ReadyError):
        R.load()


def test_workspace_init_validation():
    """readyWorkspaceInit rejects bad arguments on the host, before any launch."""
    _lib()
    st, plan = R.readyPlanCreate(_shape(), [0, 1])
    assert st == R.READY_OK
    _, n = R.readyWorkspaceSize(plan)
    assert R.readyWorkspaceInit(None, 1 << 40, n, None) == R.READY_ERR_NULL_POINTER
    assert R.readyWorkspaceInit(plan, None, n, None) == R.READY_ERR_NULL_POINTER
    assert R.readyWorkspaceInit(plan, (1 << 40) + 16, n, None) == R.READY_ERR_MISALIGNED
    assert R.readyWorkspaceInit(plan, 1 << 40, n - 1, None) == R.READY_ERR_WORKSPACE_TOO_SMALL
    R.readyPlanDestroy(plan)
    # the general path (fp32 at 21 rows) keeps no counters: nothing to
    # prepare, nothing launched
    st, plan = R.readyPlanCreate(_shape(B=3, state_dtype="f32", act_dtype="f32", weight_dtype="f32"), [0, 1])
    assert R.readyPlanLaunches(plan) == (R.READY_OK, 4)
    _, n = R.readyWorkspaceSize(plan)
    assert R.readyWorkspaceInit(plan, 1 << 40, n, None) == R.READY_OK
    R.readyPlanDestroy(plan)


# ------------------------------------------------------------ readyVerifyStates

def _verify_call(B=2, P=8, L=2, H=4, sdt=R.READY_BF16, kdt=R.READY_BF16, mutate=None):
    """Arguments of a well-formed call on fake, disjoint, aligned addresses;
    `mutate` breaks one of them.  A call that passed validation would launch,
    so every case here must be rejected (or have B = 0)."""
    lib = _lib()
    M = L * H
    base = 1 << 40
    es = 2 if sdt == R.READY_BF16 else 4
    a = {"state_t": base, "k": base + (1 << 34), "v": base + (2 << 34), "alpha": base + (3 << 34),
         "beta": base + (4 << 34)}
    tile = 128 * 128
    out = R.readyVerifyBuffer(base=base + (5 << 34), stride_b=P * L * H * tile, stride_p=L * H * tile,
                              stride_l=H * tile, stride_h=tile)
    a["out"] = out
    a["B"], a["P"], a["L"], a["H"], a["sdt"], a["kdt"] = B, P, L, H, sdt, kdt
    if mutate:
        mutate(a)
    return lib.readyVerifyStates(a["B"], a["P"], a["L"], a["H"], a["sdt"], a["kdt"], a["state_t"], a["k"], a["v"],
                                 a["alpha"], a["beta"], ctypes.byref(a["out"]) if a["out"] is not None else None,
                                 None)


def test_verify_zero_batch_is_ok():
    assert _verify_call(B=0) == R.READY_OK


@pytest.mark.parametrize("kw", [dict(P=0), dict(P=65), dict(L=0), dict(H=0), dict(L=64, H=65), dict(B=-1)])
def test_verify_rejects_bad_shapes(kw):
    assert _verify_call(**kw) == R.READY_ERR_BAD_SHAPE


def test_verify_rejects_bad_dtype():
    assert _verify_call(sdt=7) == R.READY_ERR_UNSUPPORTED_DTYPE
    assert _verify_call(kdt=-1) == R.READY_ERR_UNSUPPORTED_DTYPE


def test_verify_null_pointers():
    for field in ("state_t", "k", "v", "alpha", "beta", "out"):
        def m(a, field=field):
            a[field] = None
        assert _verify_call(mutate=m) == R.READY_ERR_NULL_POINTER, field

    def m(a):
        a["out"].base = None
    assert _verify_call(mutate=m) == R.READY_ERR_NULL_POINTER


def test_verify_misaligned():
    for field in ("state_t", "k", "v"):
        def m(a, field=field):
            a[field] += 2
        assert _verify_call(mutate=m) == R.READY_ERR_MISALIGNED, field

    def stride(a):
        a["out"].stride_h += 3
    assert _verify_call(mutate=stride) == R.READY_ERR_MISALIGNED

    def negative(a):
        a["out"].stride_p = -a["out"].stride_p
    assert _verify_call(mutate=negative) == R.READY_ERR_BAD_SHAPE


def test_verify_aliasing():
    for field in ("state_t", "k", "alpha"):
        def m(a, field=field):
            a["out"].base = a[field]
        assert _verify_call(mutate=m) == R.READY_ERR_ALIASING, field

    def inside(a):
        a["state_t"] = a["out"].base + 7 * 128 * 128 * 2   # an input inside the buffer's span
    assert _verify_call(mutate=inside) == R.READY_ERR_ALIASING


# ---------------------------------------------------------------- step 1 alone (readyGather)

def _gather_call(shape, mutate=None):
    _lib()
    st, plan = R.readyPlanCreate(shape, [0, 1])
    assert st == R.READY_OK
    f = _Fake(shape)
    B, P, L, H = shape.B, shape.P, shape.L_tot, shape.H
    M = shape.L_sel * H
    tile = 128 * 128
    es = 2 if shape.state_dtype == R.READY_BF16 else 4
    args = dict(plan=plan,
                states=R.readyStates(base=f.alloc(max(B, 1) * P * L * H * tile * es), stride_b=P * L * H * tile,
                                     stride_p=L * H * tile, stride_l=H * tile, stride_h=tile),
                accept_idx=f.alloc(4 * max(B, 1)), gathered=f.alloc(max(B, 1) * M * tile * es),
                dev_status=f.alloc(4), stream=None)
    if mutate:
        mutate(args)
    code = R.readyGather(**args)
    R.readyPlanDestroy(plan)
    return code


def test_gather_validation():
    assert _gather_call(_shape(B=0)) == R.READY_OK

    def set_(k, v):
        def f(a):
            a[k] = v
        return f

    def null_states(a):
        a["states"].base = None

    for m in (set_("accept_idx", None), set_("gathered", None), null_states):
        assert _gather_call(_shape(), mutate=m) == R.READY_ERR_NULL_POINTER

    def mis_gathered(a):
        a["gathered"] += 8

    def mis_stride(a):
        a["states"].stride_l += 1

    def neg_stride(a):
        a["states"].stride_b = -a["states"].stride_b
    assert _gather_call(_shape(), mutate=mis_gathered) == R.READY_ERR_MISALIGNED
    assert _gather_call(_shape(), mutate=mis_stride) == R.READY_ERR_MISALIGNED
    assert _gather_call(_shape(), mutate=neg_stride) == R.READY_ERR_BAD_SHAPE

    def gathered_in_states(a):
        a["gathered"] = a["states"].base + 4 * 128 * 128 * 2

    def status_in_gathered(a):
        a["dev_status"] = a["gathered"] + 64
    assert _gather_call(_shape(), mutate=gathered_in_states) == R.READY_ERR_ALIASING
    assert _gather_call(_shape(), mutate=status_in_gathered) == R.READY_ERR_ALIASING


# ------------------------------------------------------------ readyStateReaderStatic (no workspace)

def test_static_entry_validates_before_touching_the_device():
    """The no-workspace form checks its arguments like readyStateReader; no
    case here reaches the device lookup (B = 0 is a valid no-op)."""
    assert _call(_shape(B=0), static=True) == R.READY_OK

    def null(field):
        def f(a):
            if field.startswith("o."):
                setattr(a["outputs"], field[2:], None)
            else:
                a[field] = None
        return f
    for field in ("accept_idx", "h", "o.gathered", "o.out"):
        assert _call(_shape(), mutate=null(field), static=True) == R.READY_ERR_NULL_POINTER, field

    def mis(a):
        a["h"] += 2
    assert _call(_shape(), mutate=mis, static=True) == R.READY_ERR_MISALIGNED

    def alias(a):
        a["outputs"].out = a["weights"].w2
    assert _call(_shape(), mutate=alias, static=True) == R.READY_ERR_ALIASING
    _lib()
    assert R.load().readyStateReaderStatic(None, None, None, None, None, None, None) == R.READY_ERR_NULL_POINTER


def test_static_entry_rejects_plans_beyond_the_array():
    """Plans whose scratch exceeds the static array are refused with their
    own status, before any argument is looked at; plans that fit are not."""
    _lib()
    big = R.make_shape(B=256, P=8, n=7, L_tot=3, L_sel=3, H=16, r=128, d=5120, Hm=256)
    st, plan = R.readyPlanCreate(big, [0, 1, 2])
    assert st == R.READY_OK
    assert R.readyWorkspaceSize(plan)[1] > R.READY_STATIC_SCRATCH_BYTES
    assert R.load().readyStateReaderStatic(plan, None, None, None, None, None, None) == \
        R.READY_ERR_STATIC_SCRATCH_TOO_SMALL
    R.readyPlanDestroy(plan)
    batched = R.make_shape(B=64, P=8, n=7, L_tot=2, L_sel=2, H=16, r=8, d=5120, Hm=256)
    st, plan = R.readyPlanCreate(batched, [0, 1])
    assert R.readyWorkspaceSize(plan)[1] <= R.READY_STATIC_SCRATCH_BYTES - R.READY_STATIC_COUNTER_BYTES
    assert R.load().readyStateReaderStatic(plan, None, None, None, None, None, None) == R.READY_ERR_NULL_POINTER
    R.readyPlanDestroy(plan)
    assert R.readyStatusString(R.READY_ERR_STATIC_SCRATCH_TOO_SMALL) == "READY_ERR_STATIC_SCRATCH_TOO_SMALL"


@pytest.mark.parametrize("kw,launches", [
    (dict(), 1),                                                    # bf16, r = 8: k_reader
    (dict(r=32), 1),
    (dict(r=64), 4),                                                # bf16 general path
    (dict(path="unfused"), 4),
    (dict(B=1, state_dtype="f32", act_dtype="f32", weight_dtype="f32"), 1),   # k_reader_f32
    (dict(B=2, n=8, r=16, state_dtype="f32", act_dtype="f32", weight_dtype="f32"), 1),
    (dict(B=1, state_dtype="f32", act_dtype="f32", weight_dtype="f32", path="unfused"), 4),
    (dict(B=3, state_dtype="f32", act_dtype="f32", weight_dtype="f32"), 4),   # 21 rows
    (dict(B=1, r=24, state_dtype="f32", act_dtype="f32", weight_dtype="f32"), 4),
    (dict(B=1, Hm=66, state_dtype="f32", act_dtype="f32", weight_dtype="f32"), 4),
    (dict(B=1, state_dtype="f32", act_dtype="f32", weight_dtype="bf16"), 4),
])
def test_plan_launch_count(kw, launches):
    """Which shapes run as one kernel: all-bf16 with r <= 32, and all-fp32 at
    most 16 rows with r <= 16 and Hm a multiple of 4; the rest as the
    general path's four launches."""
    _lib()
    st, plan = R.readyPlanCreate(_shape(**kw), [0, 1])
    assert st == R.READY_OK
    assert R.readyPlanLaunches(plan) == (R.READY_OK, launches)
    R.readyPlanDestroy(plan)


def test_plan_launch_count_null_arguments():
    lib = _lib()
    st, plan = R.readyPlanCreate(_shape(), [0, 1])
    assert lib.readyPlanLaunches(None, None) == R.READY_ERR_NULL_POINTER
    assert lib.readyPlanLaunches(plan, None) == R.READY_ERR_NULL_POINTER
    R.readyPlanDestroy(plan)
