"""The draft-length controller on the GPU (through the C ABI) against the
oracle on seeded serving traces, and chained after a verify call on the same
stream (its accepted counts feed the controller without a host round trip)."""
import dataclasses

import numpy as np
import pytest

import oracle
import workloads as W
from oracle import adaptive as A
from tests.adaptive_sim import make_trace
from tests.gpu_helpers import log, make_verifier, to_device

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


@pytest.mark.parametrize("preset,slots,steps,seed,max_batch", [
    ("window50", 64, 300, 1, None), ("last10", 200, 200, 2, None),
    ("window50", 3000, 40, 3, None), ("window50", 5000, 20, 4, 2500)])
def test_device_controller_matches_oracle(preset, slots, steps, seed, max_batch):
    from rejection_sampling_verify_08_amd import DraftLengthController, adapt_params
    p = {"window50": A.preset_vllm_page, "last10": A.preset_checklist}[preset]()
    log(f"[case] adaptive device {preset} slots={slots} steps={steps} seed={seed}")
    trace = make_trace(p, slots, steps, seed, max_batch)
    ctl = DraftLengthController(slots, adapt_params(preset), device="cuda")
    for t, st in enumerate(trace):
        if st.resets.size:
            ctl.reset(_dev(st.resets))
        nk, ncu = ctl.update(_dev(st.cu), _dev(st.accepted), slots=_dev(st.slots))
        np.testing.assert_array_equal(nk.cpu().numpy(), st.next_k, err_msg=f"step {t}")
        np.testing.assert_array_equal(ncu.cpu().numpy(), st.next_cu, err_msg=f"step {t}")
        assert ctl.totals() == st.totals, t
    assert int(ctl.status.item()) == 0
    log(f"[parity] adaptive device {preset}: {steps} steps bit-exact, "
        f"accept rate {ctl.accept_rate():.4f}")


def test_controller_chained_after_verify():
    from rejection_sampling_verify_08_amd import DraftLengthController, adapt_params
    inp = W.config(3, seed=21, num_seqs=64)
    d = to_device(inp)
    sv = make_verifier(inp)
    ctl = DraftLengthController(inp.num_seqs, adapt_params("window50", min_history=1),
                                device="cuda")
    out = sv(d.cu, d.target, d.draft, d.tokens, d.uniforms, inp.temperature)
    nk, ncu = ctl.update(d.cu, out.num_accepted)         # same stream, no sync between
    torch.cuda.synchronize()
    ora = oracle.verify_inputs(inp)
    bank = A.Bank(dataclasses.replace(A.preset_vllm_page(), min_history=1), inp.num_seqs)
    ek, ecu = bank.step(list(range(inp.num_seqs)), inp.cu_draft, ora.num_accepted)
    assert (ora.flagged & 1 == 0).all()     # no accept test within the tie window
    np.testing.assert_array_equal(nk.cpu().numpy(), ek)
    np.testing.assert_array_equal(ncu.cpu().numpy(), ecu)


def test_empty_batch_writes_zero_offset():
    from rejection_sampling_verify_08_amd import DraftLengthController
    ctl = DraftLengthController(4, device="cuda")
    ncu = torch.full((1,), 7, dtype=torch.int32, device="cuda")
    ctl.update(torch.zeros(1, dtype=torch.int32, device="cuda"),
               torch.zeros(0, dtype=torch.int32, device="cuda"), next_cu=ncu)
    torch.cuda.synchronize()
    assert ncu.item() == 0
