"""Shared helpers of the GPU parity tests and the smoke check.

run_reader       places generated inputs on the device, calls the library
                 through the C ABI and returns every output on the host.
oracle_reference runs the float64 oracle on the same stored inputs (or a
                 sample of sequences).
compare          applies the parity bar: bit-exact gather; normwise
                 relative error of Delta h within 1e-2 (bf16 inputs, fp32
                 accumulation) or 1e-4 (all fp32); out within one bf16 ulp of
                 the rounded oracle sum plus that tolerance; log-RMS within
                 1e-5 (relative, floored at 1).
"""
import numpy as np

from synth.device import to_device, to_numpy_bits, torch_dtype


def tol_for(cfg):
    fp32 = cfg.state_dtype == "f32" and cfg.act_dtype == "f32" and cfg.weight_dtype == "f32"
    return 1e-4 if fp32 else 1e-2


def reader_shape(cfg, B=None, path="fused"):
    from hla_recurrent_state_amd import make_shape
    return make_shape(B=cfg.B if B is None else B, P=cfg.P, n=cfg.n, L_tot=cfg.L_tot, L_sel=cfg.L_sel,
                      H=cfg.H, r=cfg.r, d=cfg.d, Hm=cfg.Hm, state_dtype=cfg.state_dtype,
                      act_dtype=cfg.act_dtype, weight_dtype=cfg.weight_dtype, act=cfg.act,
                      shared=cfg.shared, state_eps=cfg.state_eps, h_eps=cfg.h_eps, path=path)


def alloc_outputs(cfg, device, B=None):
    import torch
    B = cfg.B if B is None else B
    return {
        "gathered": torch.empty((B, cfg.M, cfg.d_v, cfg.d_k), dtype=torch_dtype(cfg.state_dtype), device=device),
        "out": torch.empty((B, cfg.n, cfg.d), dtype=torch_dtype(cfg.act_dtype), device=device),
        "logrms": torch.empty((B, cfg.M), dtype=torch.float32, device=device),
        "delta": torch.empty((B, cfg.n, cfg.d), dtype=torch.float32, device=device),
        "feat": torch.empty((B, cfg.n, cfg.F), dtype=torch.float32, device=device),
        "dev_status": torch.zeros(1, dtype=torch.int32, device=device),
    }


def run_reader(inp, device, dev_inputs=None, inplace=False, path="fused", debug=True):
    """One call; returns host copies of all outputs plus the device status.
    With debug=False the optional logrms, delta and feat outputs are not
    passed (the configuration the benchmark times) and come back as None."""
    import torch
    from hla_recurrent_state_amd import StateReader
    cfg = inp.cfg
    d = dev_inputs if dev_inputs is not None else to_device(inp, device)
    reader = StateReader(reader_shape(cfg, path=path), cfg.slots)
    o = alloc_outputs(cfg, device)
    if inplace:
        o["out"] = d["h"].clone()
        h_arg = o["out"]
    else:
        h_arg = d["h"]
    if debug:
        dbg = dict(logrms=o["logrms"], delta=o["delta"], feat=o["feat"])
    else:
        dbg = dict(logrms=None, delta=None, feat=None)
    reader(d["states"], d["accept_idx"], h_arg, d["weights"], o["gathered"], o["out"],
           dev_status=o["dev_status"], **dbg)
    torch.cuda.synchronize(device)
    res = {
        "gathered": to_numpy_bits(o["gathered"], cfg.state_dtype),
        "out": to_numpy_bits(o["out"], cfg.act_dtype),
        "logrms": o["logrms"].cpu().numpy() if debug else None,
        "delta": o["delta"].cpu().numpy() if debug else None,
        "feat": o["feat"].cpu().numpy() if debug else None,
        "dev_status": int(o["dev_status"].item()),
    }
    reader.close()
    return res


def oracle_reference(inp, seqs=None):
    """float64 oracle on the stored inputs; `seqs` restricts it to a sample."""
    from oracle import reader as orc
    cfg = inp.cfg
    seqs = list(range(cfg.B)) if seqs is None else list(seqs)
    buf = orc.decode(inp.buf[seqs], cfg.state_dtype)
    h = orc.decode(inp.h[seqs], cfg.act_dtype)
    W = {k: (None if getattr(inp, k) is None else orc.decode(getattr(inp, k), cfg.weight_dtype))
         for k in ("wq", "u", "v", "w1", "w2", "gamma", "b1", "b2")}
    ref = orc.state_reader(buf, inp.accept_idx[seqs], list(cfg.slots), cfg.H, h, W["wq"], W["u"], W["v"],
                           W["w1"], W["w2"], gamma=W["gamma"], b1=W["b1"], b2=W["b2"], act=cfg.act,
                           state_eps=cfg.state_eps, h_eps=cfg.h_eps, shared=cfg.shared)
    ref["seqs"] = seqs
    ref["h"] = h
    return ref


def _decode(x, dtype):
    from oracle import reader as orc
    return orc.decode(x, dtype)


def compare(inp, res, ref, tol=None):
    """Parity report of a GPU result against the oracle (on ref['seqs'])."""
    from oracle import reader as orc
    cfg = inp.cfg
    tol = tol_for(cfg) if tol is None else tol
    seqs = ref["seqs"]
    rep = {"tol": tol}
    # 1. gather: bit-exact against direct indexing of the stored buffer and
    #    value-exact against the oracle's gather
    want_bits = np.stack([inp.buf[b, inp.accept_idx[b]][list(cfg.slots)].reshape(cfg.M, cfg.d_v, cfg.d_k)
                          for b in seqs])
    got_bits = res["gathered"][seqs]
    rep["gather_bitexact"] = bool(np.array_equal(got_bits.view(np.uint8), want_bits.view(np.uint8)))
    rep["gather_oracle_equal"] = bool(np.array_equal(_decode(got_bits, cfg.state_dtype), ref["G"]))
    if res["logrms"] is None:
        # the timed configuration: no debug outputs, so only gathered and out
        return _compare_out(cfg, res, ref, rep, tol)
    # 2. log-RMS
    ell = res["logrms"][seqs].astype(np.float64)
    rep["logrms_err"] = float(np.max(np.abs(ell - ref["ell"]) / np.maximum(1.0, np.abs(ref["ell"]))))
    # 3. features f and Delta h (normwise relative)
    f = res["feat"][seqs].astype(np.float64)
    rep["feat_rel"] = float(np.max(np.abs(f - ref["f"])) / max(np.max(np.abs(ref["f"])), 1e-30))
    dh = res["delta"][seqs].astype(np.float64)
    scale = max(np.max(np.abs(ref["dh"])), 1e-30)
    rep["dh_rel"] = float(np.max(np.abs(dh - ref["dh"])) / scale)
    # 4. out = RNE(h + Delta h_ref) within one ulp plus the tolerance
    out = _decode(res["out"][seqs], cfg.act_dtype)
    if cfg.act_dtype == "bf16":
        want = orc.round_to_bf16(ref["h_new"])
        ulp = np.ldexp(1.0, np.frexp(np.abs(want))[1] - 8)
    else:
        want = ref["h_new"]
        ulp = np.ldexp(1.0, np.frexp(np.abs(want))[1] - 24)
    rep["out_excess"] = float(np.max(np.abs(out - want) - ulp - tol * scale))
    rep["dev_status"] = res["dev_status"]
    rep["ok"] = (rep["gather_bitexact"] and rep["gather_oracle_equal"] and rep["logrms_err"] <= 1e-5
                 and rep["feat_rel"] <= tol and rep["dh_rel"] <= tol and rep["out_excess"] <= 0.0
                 and rep["dev_status"] == 0)
    return rep


def _compare_out(cfg, res, ref, rep, tol):
    """gathered (already in rep) and out = RNE(h + Delta h_ref) within one
    ulp plus tol times max|Delta h_ref|."""
    from oracle import reader as orc
    seqs = ref["seqs"]
    scale = max(np.max(np.abs(ref["dh"])), 1e-30)
    out = _decode(res["out"][seqs], cfg.act_dtype)
    if cfg.act_dtype == "bf16":
        want = orc.round_to_bf16(ref["h_new"])
        ulp = np.ldexp(1.0, np.frexp(np.abs(want))[1] - 8)
    else:
        want = ref["h_new"]
        ulp = np.ldexp(1.0, np.frexp(np.abs(want))[1] - 24)
    rep["out_excess"] = float(np.max(np.abs(out - want) - ulp - tol * scale))
    rep["dev_status"] = res["dev_status"]
    rep["ok"] = (rep["gather_bitexact"] and rep["gather_oracle_equal"] and rep["out_excess"] <= 0.0
                 and rep["dev_status"] == 0)
    return rep
