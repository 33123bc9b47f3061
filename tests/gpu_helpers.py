"""Helpers of the GPU tests: move seeded inputs to the device, run the HIP
path through the C ABI, and compare with the oracle by the parity rule.

Parity rule: accepted counts and emitted tokens are bit-exact for every
sequence the oracle does not flag; a flagged sequence (a uniform within 1e-6
of a decision threshold) may differ only at that tie -- the first differing
accept decision must be a flagged test, and a differing final token must have
a CDF interval within 1e-6 of u.  p_i(x_i), q_i(x_i) and the residual sums
agree within 1e-5 relative for f32 logits and 2e-3 for bf16 logits.
"""
from __future__ import annotations

import dataclasses
import sys

import numpy as np

import oracle
import workloads as W

TIE = oracle.TIE_TOL
PROB_RTOL = {"f32": 1e-5, "bf16": 2e-3}
ILL_RESIDUAL = 8   # oracle flag: residual mass below 2^-20


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def torch_logits(arr: np.ndarray, dtype: str, device, ld: int | None = None,
                 offset: int = 0):
    """Host logits -> device tensor [R, V] view with row pitch ld (>= V)
    starting `offset` elements into its allocation."""
    import torch
    R, V = arr.shape
    ld = V if ld is None else ld
    if dtype == "bf16":
        host = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
        tdt = torch.bfloat16
    else:
        host = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32))
        tdt = torch.float32
    buf = torch.zeros(max(R * ld + offset, 1), dtype=tdt, device=device)
    view = buf[offset:offset + R * ld].view(R, ld)[:, :V] if R > 0 else \
        buf[offset:offset].view(0, V)
    if R > 0:
        view.copy_(host.to(device))
    return view


@dataclasses.dataclass
class DeviceInputs:
    cu: "torch.Tensor"
    target: "torch.Tensor"
    draft: "torch.Tensor"
    tokens: "torch.Tensor"
    uniforms: "torch.Tensor"


def to_device(inp: W.VerifyInputs, device="cuda", ld=None, offset=0) -> DeviceInputs:
    import torch
    return DeviceInputs(
        cu=torch.from_numpy(inp.cu_draft.astype(np.int32)).to(device),
        target=torch_logits(inp.target_logits, inp.dtype, device, ld, offset),
        draft=torch_logits(inp.draft_logits, inp.dtype, device, ld, offset),
        tokens=torch.from_numpy(np.ascontiguousarray(inp.draft_tokens, np.int32)).to(device),
        uniforms=torch.from_numpy(np.ascontiguousarray(inp.uniforms, np.float32)).to(device))


def make_verifier(inp: W.VerifyInputs, check=False, max_seqs=None, max_draft_rows=None):
    from rejection_sampling_verify_08_amd import SpecVerifier
    return SpecVerifier(inp.vocab, inp.dtype,
                        max_seqs=max(max_seqs or inp.num_seqs, 1),
                        max_draft_rows=max_draft_rows if max_draft_rows is not None
                        else inp.draft_rows, check=check)


@dataclasses.dataclass
class HostOutput:
    out_tokens: np.ndarray
    num_accepted: np.ndarray
    p_draft: np.ndarray
    q_draft: np.ndarray
    residual_sum: np.ndarray
    status: int


def run_gpu(inp: W.VerifyInputs, sv=None, dev_inputs=None, check=False, mode="sampled",
            **kw) -> HostOutput:
    """Run one entry point on `inp`: mode "sampled" (spec_verify_run),
    "point" (spec_verify_run_point_drafts) or "greedy"
    (spec_verify_run_greedy).  Outputs a mode does not write read back as
    whatever allocate_outputs left there."""
    import torch
    sv = sv or make_verifier(inp, check=check)
    d = dev_inputs or to_device(inp, **kw)
    if mode == "sampled":
        out = sv(d.cu, d.target, d.draft, d.tokens, d.uniforms, inp.temperature,
                 num_seqs=inp.num_seqs, total_draft_rows=inp.draft_rows)
    elif mode == "point":
        out = sv.point_drafts(d.cu, d.target, d.tokens, d.uniforms, inp.temperature,
                              num_seqs=inp.num_seqs)
    elif mode == "greedy":
        out = sv.greedy(d.cu, d.target, d.tokens, num_seqs=inp.num_seqs)
    else:
        raise ValueError(mode)
    torch.cuda.synchronize()
    return HostOutput(out.out_tokens.cpu().numpy(), out.num_accepted.cpu().numpy(),
                      out.p_draft.cpu().numpy().astype(np.float64),
                      out.q_draft.cpu().numpy().astype(np.float64),
                      out.residual_sum.cpu().numpy().astype(np.float64),
                      int(out.status.cpu().numpy()[0]) & 0xFFFFFFFF)


def _final_cdf(inp: W.VerifyInputs, b: int, n: int, point: bool = False):
    """Normalised CDF of the oracle's final-draw weights at position n
    (point: the draft distribution is the point mass at the draft token)."""
    g = int(inp.gammas[b])
    p = oracle.row_softmax(inp.target_logits[inp.target_row(b, n)], inp.temperature, inp.dtype)
    if n < g and point:
        w = p.copy()
        w[int(inp.draft_tokens[inp.draft_row(b, n)])] = 0.0
    elif n < g:
        q = oracle.row_softmax(inp.draft_logits[inp.draft_row(b, n)], inp.temperature,
                               inp.dtype)
        w = np.maximum(p - q, 0.0)
    else:
        w = p
    c = np.cumsum(w)
    return w, c / c[-1]


@dataclasses.dataclass
class ParityReport:
    sequences: int
    flagged: int
    tie_differences: int
    max_prob_rel: float
    max_residual_rel: float


def compare(inp: W.VerifyInputs, gpu: HostOutput, ora, *, label: str = "",
            check_probs: bool = True, point: bool = False) -> ParityReport:
    B = inp.num_seqs
    cu = inp.cu_draft
    bad = []
    flagged = 0
    tie_diffs = 0
    for b in range(B):
        g = int(inp.gammas[b])
        t0 = int(cu[b]) + b
        d0 = int(cu[b])
        gn, on = int(gpu.num_accepted[b]), int(ora.num_accepted[b])
        gt = gpu.out_tokens[t0:t0 + g + 1]
        ot = ora.out_tokens[t0:t0 + g + 1]
        same = gn == on and np.array_equal(gt, ot)
        if ora.flagged[b]:
            flagged += 1
        if same:
            continue
        if not ora.flagged[b]:
            bad.append((b, "unflagged difference", gn, on, gt.tolist(), ot.tolist()))
            continue
        tie_diffs += 1
        if gn != on:
            i = min(gn, on)
            if not (ora.tie_accept[d0 + i] < TIE):
                bad.append((b, "accept decision differs away from a tie", gn, on))
            continue
        # same count, different drawn token: it must sit at the final-draw tie,
        # or the residual's mass is below fp32 resolution (oracle flag bit 3:
        # the draw is not determined at the precision of the inputs)
        k = int(gt[gn])
        if ora.flagged[b] & ILL_RESIDUAL:
            if not 0 <= k < inp.vocab:
                bad.append((b, "final token out of range", k, int(ot[gn])))
            continue
        w, C = _final_cdf(inp, b, gn, point)
        u = float(inp.uniforms[t0 + g])
        lo = C[k - 1] if k > 0 else 0.0
        if not (0 <= k < inp.vocab and w[k] > 0 and lo - TIE <= u <= C[k] + TIE):
            bad.append((b, "final token outside the tie window", k, int(ot[gn])))
    assert not bad, f"{label}: {len(bad)} parity failures, first: {bad[:3]}"

    max_prob_rel = 0.0
    max_res_rel = 0.0
    if check_probs:
        rtol = PROB_RTOL[inp.dtype]
        for name, g_arr, o_arr in (("p_draft", gpu.p_draft, ora.p_draft),
                                   ("q_draft", gpu.q_draft, ora.q_draft)):
            if o_arr.size:
                rel = np.abs(g_arr - o_arr) / np.maximum(np.abs(o_arr), 1e-30)
                rel[np.abs(o_arr) < 1e-30] = 0.0
                max_prob_rel = max(max_prob_rel, float(rel.max()))
                assert rel.max() <= rtol, f"{label}: {name} rel err {rel.max():.3g} > {rtol}"
        # residual sums below fp32 resolution (flag bit 3) carry no relative precision
        same_n = (gpu.num_accepted == ora.num_accepted) & ((ora.flagged & ILL_RESIDUAL) == 0)
        o = ora.residual_sum[same_n]
        g_ = gpu.residual_sum[same_n]
        if o.size:
            rel = np.abs(g_ - o) / np.maximum(np.abs(o), 1e-30)
            rel[o == 0] = np.abs(g_[o == 0])
            max_res_rel = float(rel.max())
            assert rel.max() <= rtol, f"{label}: residual_sum rel err {rel.max():.3g} > {rtol}"
    rep = ParityReport(B, flagged, tie_diffs, max_prob_rel, max_res_rel)
    log(f"[parity] {label}: seqs={B} flagged={flagged} tie_diffs={tie_diffs} "
        f"max_prob_rel={max_prob_rel:.3g} max_residual_rel={max_res_rel:.3g}")
    return rep


def compare_greedy(inp: W.VerifyInputs, gpu: HostOutput, ora, *, label: str = "") -> None:
    """Greedy verification is integer work: bit-exact counts and tokens."""
    R_t = inp.target_rows
    bad = np.nonzero(gpu.num_accepted != ora.num_accepted)[0]
    assert bad.size == 0, f"{label}: num_accepted differs at {bad[:5].tolist()}"
    diff = np.nonzero(gpu.out_tokens[:R_t] != ora.out_tokens[:R_t])[0]
    assert diff.size == 0, (f"{label}: out_tokens differ at rows {diff[:5].tolist()}: "
                            f"{gpu.out_tokens[diff[:5]].tolist()} vs "
                            f"{ora.out_tokens[diff[:5]].tolist()}")
    log(f"[parity] {label}: seqs={inp.num_seqs} greedy bit-exact, "
        f"mean accepted {float(ora.num_accepted.mean()):.3f}")


def oracle_greedy(inp: W.VerifyInputs):
    return oracle.verify_greedy(inp.num_seqs, inp.cu_draft, inp.target_logits,
                                inp.draft_tokens, vocab=inp.vocab, dtype=inp.dtype)


def oracle_point(inp: W.VerifyInputs):
    return oracle.verify_onehot(inp.num_seqs, inp.cu_draft, inp.target_logits,
                                inp.draft_tokens, inp.uniforms, inp.temperature,
                                vocab=inp.vocab, dtype=inp.dtype)
