"""Python binding of the ready.h C ABI (libready.so, gfx950).

Argument marshalling only: every step of the state reader runs in the HIP
kernels of libready.so.  If the library is missing, loading raises
ReadyError -- there is no fallback path.

Low-level names mirror the C functions (readyPlanCreate, readyWorkspaceSize,
readyPlanLaunches, readyStateReader, readyGather, readyPrepSize, readyStatePrepare, readyStateApply,
readyVerifyStates, readyPlanDestroy, readyStatusString, readyVersion) and the C structs (readyShape, readyStates, readyWeights,
readyOutputs, readyVerifyBuffer), plus readyStateReaderStatic, the form with
no workspace argument for callers that cannot allocate.  StateReader and verify_states wrap them for
torch tensors: they forward data_ptr() values and the current HIP stream
(StateReader.prepare / StateReader.apply for several readers sharing one
gather).
"""
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libready.so")
SRC_DIR = os.path.join(_HERE, "csrc")
INCLUDE_DIR = os.path.join(os.path.dirname(_HERE), "include")

READY_OK = 0
READY_ERR_NULL_POINTER = 1
READY_ERR_BAD_SHAPE = 2
READY_ERR_UNSUPPORTED_DTYPE = 3
READY_ERR_MISALIGNED = 4
READY_ERR_WORKSPACE_TOO_SMALL = 5
READY_ERR_ALIASING = 6
READY_ERR_LAYER_ID_RANGE = 7
READY_ERR_HIP = 8
READY_ERR_ACCEPT_IDX = 9
READY_ERR_OUT_OF_HOST_MEMORY = 10
READY_ERR_SYNC_TIMEOUT = 11
READY_ERR_WORKSPACE_UNINIT = 12
READY_ERR_UNSUPPORTED = 13
READY_ERR_STATIC_SCRATCH_TOO_SMALL = 14
READY_STATIC_SCRATCH_BYTES = 16 << 20
READY_STATIC_COUNTER_BYTES = 64 << 10
READY_MAX_INJ = 8

READY_F32 = 0
READY_BF16 = 1
READY_ACT_SILU = 0
READY_ACT_GELU_TANH = 1
READY_ACT_RELU = 2

DTYPES = {"f32": READY_F32, "bf16": READY_BF16}
ACTS = {"silu": READY_ACT_SILU, "gelu_tanh": READY_ACT_GELU_TANH, "relu": READY_ACT_RELU}
READY_PATH_FUSED = 0
READY_PATH_UNFUSED = 1
PATHS = {"fused": READY_PATH_FUSED, "unfused": READY_PATH_UNFUSED}

# Every symbol include/ready.h declares.
EXPORTS = ("readyPlanCreate", "readyPlanDestroy", "readyWorkspaceSize", "readyPlanLaunches", "readyWorkspaceInit",
           "readyStateReader", "readyStateReaderProfiled", "readyStateReaderStatic", "readyGather", "readyPrepSize", "readyStatePrepare",
           "readyStateApply", "readyVerifyStates", "readyStatusString", "readyVersion")
READY_STAGES = 4


class ReadyError(RuntimeError):
    def __init__(self, code, what=""):
        self.code = code
        name = readyStatusString(code) if _lib is not None else str(code)
        super().__init__("%s%s" % (name, (": " + what) if what else ""))


class readyShape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("B", "P", "n", "L_tot", "L_sel", "H", "d_k", "d_v", "r", "d", "Hm",
                 "state_dtype", "act_dtype", "weight_dtype", "act", "shared_params")] + \
               [("state_eps", ctypes.c_float), ("h_eps", ctypes.c_float), ("path", ctypes.c_int32)]


class readyStates(ctypes.Structure):
    _fields_ = [("base", ctypes.c_void_p), ("stride_b", ctypes.c_int64), ("stride_p", ctypes.c_int64),
                ("stride_l", ctypes.c_int64), ("stride_h", ctypes.c_int64)]


class readyVerifyBuffer(ctypes.Structure):
    _fields_ = [("base", ctypes.c_void_p), ("stride_b", ctypes.c_int64), ("stride_p", ctypes.c_int64),
                ("stride_l", ctypes.c_int64), ("stride_h", ctypes.c_int64)]


class readyWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("wq", "u", "v", "h_gamma", "w1", "b1", "w2", "b2")]


class readyOutputs(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("gathered", "out", "logrms", "delta", "feat", "dev_status")]


_lib = None


def load():
    """Load libready.so (raises ReadyError if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ReadyError(-1, "libready.so not built; run __graft_entry__.build()")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER
    lib.readyPlanCreate.argtypes = [P(readyShape), P(ctypes.c_int32), P(ctypes.c_void_p)]
    lib.readyPlanCreate.restype = ctypes.c_int
    lib.readyPlanDestroy.argtypes = [ctypes.c_void_p]
    lib.readyPlanDestroy.restype = ctypes.c_int
    lib.readyWorkspaceSize.argtypes = [ctypes.c_void_p, P(ctypes.c_size_t)]
    lib.readyWorkspaceSize.restype = ctypes.c_int
    lib.readyPlanLaunches.argtypes = [ctypes.c_void_p, P(ctypes.c_int32)]
    lib.readyPlanLaunches.restype = ctypes.c_int
    lib.readyWorkspaceInit.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.readyWorkspaceInit.restype = ctypes.c_int
    lib.readyStateReader.argtypes = [ctypes.c_void_p, P(readyStates), ctypes.c_void_p, ctypes.c_void_p,
                                     P(readyWeights), P(readyOutputs), ctypes.c_void_p, ctypes.c_size_t,
                                     ctypes.c_void_p]
    lib.readyStateReader.restype = ctypes.c_int
    lib.readyStateReaderProfiled.argtypes = lib.readyStateReader.argtypes + [P(ctypes.c_void_p)]
    lib.readyStateReaderProfiled.restype = ctypes.c_int
    lib.readyStateReaderStatic.argtypes = [ctypes.c_void_p, P(readyStates), ctypes.c_void_p, ctypes.c_void_p,
                                           P(readyWeights), P(readyOutputs), ctypes.c_void_p]
    lib.readyStateReaderStatic.restype = ctypes.c_int
    lib.readyGather.argtypes = [ctypes.c_void_p, P(readyStates), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                ctypes.c_void_p]
    lib.readyGather.restype = ctypes.c_int
    lib.readyPrepSize.argtypes = [ctypes.c_void_p, ctypes.c_int32, P(ctypes.c_size_t)]
    lib.readyPrepSize.restype = ctypes.c_int
    lib.readyStatePrepare.argtypes = [ctypes.c_void_p, P(readyStates), ctypes.c_void_p, ctypes.c_int32,
                                      P(readyWeights), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                      ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_size_t,
                                      ctypes.c_void_p]
    lib.readyStatePrepare.restype = ctypes.c_int
    lib.readyStateApply.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32,
                                    ctypes.c_int32, ctypes.c_void_p, P(readyWeights), P(readyOutputs),
                                    ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.readyStateApply.restype = ctypes.c_int
    lib.readyVerifyStates.argtypes = [ctypes.c_int32] * 6 + [ctypes.c_void_p] * 5 + [P(readyVerifyBuffer),
                                                                      ctypes.c_void_p]
    lib.readyVerifyStates.restype = ctypes.c_int
    lib.readyStatusString.argtypes = [ctypes.c_int]
    lib.readyStatusString.restype = ctypes.c_char_p
    lib.readyVersion.argtypes = []
    lib.readyVersion.restype = ctypes.c_int32
    _lib = lib
    return lib


# ------------------------------------------------------------ C-named calls

def readyStatusString(code):
    return load().readyStatusString(int(code)).decode()


def readyVersion():
    return load().readyVersion()


def readyPlanCreate(shape, layer_ids):
    """shape: readyShape; layer_ids: sequence of ints.  Returns (status, plan)."""
    ids = (ctypes.c_int32 * max(1, len(layer_ids)))(*layer_ids)
    plan = ctypes.c_void_p()
    st = load().readyPlanCreate(ctypes.byref(shape), ids, ctypes.byref(plan))
    return st, plan


def readyPlanDestroy(plan):
    return load().readyPlanDestroy(plan)


def readyWorkspaceSize(plan):
    """Returns (status, bytes)."""
    n = ctypes.c_size_t()
    st = load().readyWorkspaceSize(plan, ctypes.byref(n))
    return st, n.value


def readyPlanLaunches(plan):
    """Returns (status, kernel launches per readyStateReader call)."""
    n = ctypes.c_int32()
    st = load().readyPlanLaunches(plan, ctypes.byref(n))
    return st, n.value


def readyWorkspaceInit(plan, workspace, workspace_bytes, stream):
    """Enqueue the preparation of a workspace for `plan`.  Returns status."""
    return load().readyWorkspaceInit(plan, workspace, workspace_bytes, stream)


def readyStateReader(plan, states, accept_idx, h, weights, outputs, workspace, workspace_bytes, stream):
    """Raw call: pointers are ints, structs are the ctypes mirrors.  Returns status."""
    return load().readyStateReader(plan, ctypes.byref(states), accept_idx, h, ctypes.byref(weights),
                                   ctypes.byref(outputs), workspace, workspace_bytes, stream)


def readyStateReaderProfiled(plan, states, accept_idx, h, weights, outputs, workspace, workspace_bytes,
                             stream, events):
    """As readyStateReader; `events` is a sequence of 2 * READY_STAGES
    hipEvent_t handles (ints) or None entries: start and end of each stage's
    kernel (on the bf16 path the single kernel is stage 1)."""
    ev = (ctypes.c_void_p * (2 * READY_STAGES))(*[e for e in events])
    return load().readyStateReaderProfiled(plan, ctypes.byref(states), accept_idx, h, ctypes.byref(weights),
                                           ctypes.byref(outputs), workspace, workspace_bytes, stream, ev)


def readyStateReaderStatic(plan, states, accept_idx, h, weights, outputs, stream):
    """Raw call of the form with the library's static scratch (no workspace)."""
    return load().readyStateReaderStatic(plan, ctypes.byref(states), accept_idx, h, ctypes.byref(weights),
                                         ctypes.byref(outputs), stream)


def readyGather(plan, states, accept_idx, gathered, dev_status, stream):
    """Raw call of step 1 alone.  Returns status."""
    return load().readyGather(plan, ctypes.byref(states), accept_idx, gathered, dev_status, stream)


def readyPrepSize(plan, n_inj):
    """Returns (status, bytes) of the prepared-state buffer for n_inj readers."""
    n = ctypes.c_size_t()
    st = load().readyPrepSize(plan, n_inj, ctypes.byref(n))
    return st, n.value


def readyStatePrepare(plan, states, accept_idx, n_inj, inj_weights, gathered, logrms, dev_status, prep,
                      prep_bytes, workspace, workspace_bytes, stream):
    """Raw call; `inj_weights` is a ctypes array of n_inj readyWeights."""
    return load().readyStatePrepare(plan, ctypes.byref(states), accept_idx, n_inj, inj_weights, gathered,
                                    logrms, dev_status, prep, prep_bytes, workspace, workspace_bytes, stream)


def readyStateApply(plan, prep, prep_bytes, n_inj, inj, h, weights, outputs, workspace, workspace_bytes, stream):
    return load().readyStateApply(plan, prep, prep_bytes, n_inj, inj, h, ctypes.byref(weights),
                                  ctypes.byref(outputs), workspace, workspace_bytes, stream)


# ------------------------------------------------------------ torch wrapper

def readyVerifyStates(B, P, L, H, state_dtype, kv_dtype, state_t, k, v, alpha, beta, out, stream):
    return load().readyVerifyStates(B, P, L, H, state_dtype, kv_dtype, state_t, k, v, alpha, beta,
                                    ctypes.byref(out), stream)


def verify_states(state_t, k, v, alpha, beta, out, H, stream=None):
    """Write the verify block's per-position states into `out` (torch tensors).

    state_t [B][L*H][128][128]; k, v [B][P-1][L*H][128]; alpha, beta fp32
    [B][P-1][L*H]; out [B][P][L][H][128][128] (any outer strides), the same
    dtype as state_t.  P = out.shape[1]; L = out.shape[2] layers are written.
    """
    import torch
    if out.dim() != 6 or state_t.dim() != 4:
        raise ReadyError(READY_ERR_BAD_SHAPE, "out must be [B][P][L][H][128][128], state_t [B][L*H][128][128]")
    B, P, L = out.shape[0], out.shape[1], out.shape[2]
    dt = {torch.float32: READY_F32, torch.bfloat16: READY_BF16}
    if out.dtype != state_t.dtype or state_t.dtype not in dt or (P > 1 and k.dtype not in dt):
        raise ReadyError(READY_ERR_UNSUPPORTED_DTYPE, "verify_states dtypes")
    st = out.stride()
    buf = readyVerifyBuffer(base=out.data_ptr(), stride_b=st[0], stride_p=st[1], stride_l=st[2], stride_h=st[3])
    if stream is None:
        stream = torch.cuda.current_stream(out.device).cuda_stream
    kv_dt = dt[k.dtype] if P > 1 else READY_F32
    code = readyVerifyStates(B, P, L, H, dt[state_t.dtype], kv_dt, state_t.data_ptr(), _ptr(k), _ptr(v),
                             _ptr(alpha), _ptr(beta), buf, stream)
    if code != READY_OK:
        raise ReadyError(code, "readyVerifyStates")


def make_shape(B, P, n, L_tot, L_sel, H, r, d, Hm, state_dtype="bf16", act_dtype="bf16",
               weight_dtype="bf16", act="silu", shared=False, state_eps=1e-6, h_eps=1e-6,
               d_k=128, d_v=128, path="fused"):
    return readyShape(B=B, P=P, n=n, L_tot=L_tot, L_sel=L_sel, H=H, d_k=d_k, d_v=d_v, r=r, d=d, Hm=Hm,
                      state_dtype=DTYPES[state_dtype], act_dtype=DTYPES[act_dtype],
                      weight_dtype=DTYPES[weight_dtype], act=ACTS[act], shared_params=int(bool(shared)),
                      state_eps=state_eps, h_eps=h_eps, path=PATHS[path])


def _ptr(t):
    return None if t is None else t.data_ptr()


class StateReader:
    """A plan plus a call that takes torch tensors on the current device.

    reader = StateReader(shape, layer_ids)
    reader(states, accept_idx, h, weights, gathered, out, logrms=None,
           delta=None, feat=None, dev_status=None, workspace=None)
    A workspace passed in must come from new_workspace() (or have been
    prepared with init_workspace()); by default the reader keeps its own, one
    per (device, stream), prepared on that stream: calls on different streams
    never share synchronisation counters.
    `states` is a tensor [B][P][L_tot][H][128][128] (any outer strides with a
    contiguous tile) and `weights` a dict with keys wq, u, v, w1, w2 and
    optionally h_gamma, b1, b2.  Raises ReadyError on a non-zero status.
    """

    def __init__(self, shape, layer_ids):
        self.shape = shape
        self.layer_ids = list(layer_ids)
        st, self.plan = readyPlanCreate(shape, self.layer_ids)
        if st != READY_OK:
            raise ReadyError(st, "readyPlanCreate")
        st, self.workspace_bytes = readyWorkspaceSize(self.plan)
        if st != READY_OK:
            raise ReadyError(st, "readyWorkspaceSize")
        st, self.launches = readyPlanLaunches(self.plan)
        if st != READY_OK:
            raise ReadyError(st, "readyPlanLaunches")
        self._ws = {}

    def close(self):
        if getattr(self, "plan", None):
            readyPlanDestroy(self.plan)
            self.plan = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def new_workspace(self, device, stream=None):
        """A workspace for this plan, prepared by readyWorkspaceInit on the
        current (or given) stream."""
        import torch
        ws = torch.empty(max(self.workspace_bytes, 256), dtype=torch.uint8, device=device)
        self.init_workspace(ws, stream)
        return ws

    def init_workspace(self, ws, stream=None):
        import torch
        if stream is None:
            stream = torch.cuda.current_stream(ws.device).cuda_stream
        code = readyWorkspaceInit(self.plan, ws.data_ptr(), ws.numel() * ws.element_size(), stream)
        if code != READY_OK:
            raise ReadyError(code, "readyWorkspaceInit")

    def workspace(self, device, stream=None):
        """The reader's own workspace for `device` and `stream` (the current
        stream when None), prepared on that stream when first made."""
        import torch
        device = torch.device(device)
        if stream is None:
            stream = torch.cuda.current_stream(device).cuda_stream
        key = (str(device), int(stream or 0))
        ws = self._ws.get(key)
        if ws is None:
            ws = self.new_workspace(device, stream)
            self._ws[key] = ws
        return ws

    def __call__(self, states, accept_idx, h, weights, gathered, out, logrms=None, delta=None,
                 feat=None, dev_status=None, workspace=None, stream=None, events=None):
        import torch
        if states.dim() != 6:
            raise ReadyError(READY_ERR_BAD_SHAPE, "states must be [B][P][L_tot][H][128][128]")
        st = states.stride()
        sd = readyStates(base=states.data_ptr(), stride_b=st[0], stride_p=st[1], stride_l=st[2],
                         stride_h=st[3])
        wd = readyWeights(**{k: _ptr(weights.get(k)) for k in ("wq", "u", "v", "h_gamma", "w1", "b1", "w2", "b2")})
        od = readyOutputs(gathered=_ptr(gathered), out=_ptr(out), logrms=_ptr(logrms), delta=_ptr(delta),
                          feat=_ptr(feat), dev_status=_ptr(dev_status))
        if stream is None:
            stream = torch.cuda.current_stream(h.device).cuda_stream
        if workspace is None:
            workspace = self.workspace(h.device, stream)
        args = (self.plan, sd, accept_idx.data_ptr(), h.data_ptr(), wd, od, workspace.data_ptr(),
                workspace.numel() * workspace.element_size(), stream)
        if events is None:
            code = readyStateReader(*args)
        else:
            code = readyStateReaderProfiled(*args, events)
        if code != READY_OK:
            raise ReadyError(code, "readyStateReader")

    def call_static(self, states, accept_idx, h, weights, gathered, out, logrms=None, delta=None, feat=None,
                    dev_status=None, stream=None):
        """As __call__, through readyStateReaderStatic: no workspace, the
        library's static per-device scratch instead."""
        import torch
        if states.dim() != 6:
            raise ReadyError(READY_ERR_BAD_SHAPE, "states must be [B][P][L_tot][H][128][128]")
        st = states.stride()
        sd = readyStates(base=states.data_ptr(), stride_b=st[0], stride_p=st[1], stride_l=st[2],
                         stride_h=st[3])
        wd = readyWeights(**{k: _ptr(weights.get(k)) for k in ("wq", "u", "v", "h_gamma", "w1", "b1", "w2", "b2")})
        od = readyOutputs(gathered=_ptr(gathered), out=_ptr(out), logrms=_ptr(logrms), delta=_ptr(delta),
                          feat=_ptr(feat), dev_status=_ptr(dev_status))
        if stream is None:
            stream = torch.cuda.current_stream(h.device).cuda_stream
        code = readyStateReaderStatic(self.plan, sd, accept_idx.data_ptr(), h.data_ptr(), wd, od, stream)
        if code != READY_OK:
            raise ReadyError(code, "readyStateReaderStatic")

    def gather(self, states, accept_idx, gathered, dev_status=None, stream=None):
        """Step 1 alone: the committed states into `gathered`."""
        import torch
        if states.dim() != 6:
            raise ReadyError(READY_ERR_BAD_SHAPE, "states must be [B][P][L_tot][H][128][128]")
        st = states.stride()
        sd = readyStates(base=states.data_ptr(), stride_b=st[0], stride_p=st[1], stride_l=st[2],
                         stride_h=st[3])
        if stream is None:
            stream = torch.cuda.current_stream(states.device).cuda_stream
        code = readyGather(self.plan, sd, accept_idx.data_ptr(), gathered.data_ptr(), _ptr(dev_status), stream)
        if code != READY_OK:
            raise ReadyError(code, "readyGather")

    # -------------------------------------------- several readers, one gather

    def prep_size(self, n_inj):
        code, n = readyPrepSize(self.plan, n_inj)
        if code != READY_OK:
            raise ReadyError(code, "readyPrepSize")
        return n

    def new_prep(self, n_inj, device):
        """A prepared-state buffer for n_inj readers."""
        import torch
        return torch.empty(max(self.prep_size(n_inj), 256), dtype=torch.uint8, device=device)

    def prepare(self, states, accept_idx, inj_weights, gathered, prep, logrms=None, dev_status=None,
                workspace=None, stream=None):
        """Steps 1-3 once for len(inj_weights) readers (dicts with at least
        u and v); fills `prep` (from new_prep) for apply()."""
        import torch
        if states.dim() != 6:
            raise ReadyError(READY_ERR_BAD_SHAPE, "states must be [B][P][L_tot][H][128][128]")
        st = states.stride()
        sd = readyStates(base=states.data_ptr(), stride_b=st[0], stride_p=st[1], stride_l=st[2],
                         stride_h=st[3])
        n_inj = len(inj_weights)
        arr = (readyWeights * max(1, n_inj))(*[
            readyWeights(**{k: _ptr(w.get(k)) for k in ("wq", "u", "v", "h_gamma", "w1", "b1", "w2", "b2")})
            for w in inj_weights])
        if stream is None:
            stream = torch.cuda.current_stream(states.device).cuda_stream
        if workspace is None:
            workspace = self.workspace(states.device, stream)
        code = readyStatePrepare(self.plan, sd, accept_idx.data_ptr(), n_inj, arr, gathered.data_ptr(),
                                 _ptr(logrms), _ptr(dev_status), prep.data_ptr(),
                                 prep.numel() * prep.element_size(), workspace.data_ptr(),
                                 workspace.numel() * workspace.element_size(), stream)
        if code != READY_OK:
            raise ReadyError(code, "readyStatePrepare")

    def apply(self, prep, n_inj, inj, h, weights, out, delta=None, feat=None, dev_status=None,
              workspace=None, stream=None):
        """Steps 4-5 of reader `inj` on its own h, from a prepared buffer."""
        import torch
        wd = readyWeights(**{k: _ptr(weights.get(k)) for k in ("wq", "u", "v", "h_gamma", "w1", "b1", "w2", "b2")})
        od = readyOutputs(gathered=None, out=_ptr(out), logrms=None, delta=_ptr(delta), feat=_ptr(feat),
                          dev_status=_ptr(dev_status))
        if stream is None:
            stream = torch.cuda.current_stream(h.device).cuda_stream
        if workspace is None:
            workspace = self.workspace(h.device, stream)
        code = readyStateApply(self.plan, prep.data_ptr(), prep.numel() * prep.element_size(), n_inj, inj,
                               h.data_ptr(), wd, od, workspace.data_ptr(),
                               workspace.numel() * workspace.element_size(), stream)
        if code != READY_OK:
            raise ReadyError(code, "readyStateApply")
