"""GPU checks of step 1 alone (readyGather): bit-exact against direct
indexing of the stored verify buffer at the accept index, for fp32 and bf16
states, strided buffers whose selected layers are not the first slots, and
an out-of-range accept index (reported, that sequence left alone)."""
import sys

import numpy as np
import pytest

import synth
from synth.device import to_device, to_numpy_bits, torch_dtype

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _run(inp):
    from hla_recurrent_state_amd import StateReader
    from tests.gpu_util import reader_shape
    dev = _dev()
    cfg = inp.cfg
    print("gather case", cfg.name, "B", cfg.B, "M", cfg.M, cfg.state_dtype, "slots", cfg.slots, flush=True)
    d = to_device(inp, dev)
    gathered = torch.full((cfg.B, cfg.M, 128, 128), 3.0, dtype=torch_dtype(cfg.state_dtype), device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    sr = StateReader(reader_shape(cfg), cfg.slots)
    sr.gather(d["states"], d["accept_idx"], gathered, dev_status=status)
    torch.cuda.synchronize(dev)
    got = to_numpy_bits(gathered, cfg.state_dtype)
    sr.close()
    return got, int(status.item())


def _want(inp, b):
    cfg = inp.cfg
    return inp.buf[b, inp.accept_idx[b]][list(cfg.slots)].reshape(cfg.M, 128, 128)


@pytest.mark.parametrize("name,kw", [("tiny", {}), ("paper", {}), ("batched", {}),
                                     ("paper", dict(B=3, layer_ids=(62, 30), slots=(3, 1), L_tot=4))])
def test_gather_bit_exact(name, kw):
    inp = synth.make(name, seed=21, **kw)
    got, status = _run(inp)
    assert status == 0
    for b in range(inp.cfg.B):
        assert np.array_equal(got[b].view(np.uint8), _want(inp, b).view(np.uint8)), b


def test_gather_out_of_range_accept_index():
    inp = synth.make("paper", seed=22, B=3)
    inp.accept_idx[2] = -1
    got, status = _run(inp)
    assert status == 9  # READY_ERR_ACCEPT_IDX
    for b in (0, 1):
        assert np.array_equal(got[b].view(np.uint8), _want(inp, b).view(np.uint8))
    from oracle import reader as orc
    assert np.all(orc.decode(got[2], inp.cfg.state_dtype) == 3.0)  # left as it was
