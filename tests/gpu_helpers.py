"""Helpers of the GPU tests: move seeded inputs to the device, run the HIP
path through the C ABI, and compare with the oracle by the parity rule.

Parity rule: accepted counts and emitted tokens are bit-exact for every
sequence the oracle does not flag as a tie (flag bits 0-2: a uniform within
1e-6 of a decision threshold, the threshold known to within the oracle's own
error bound E, or an empty residual).  A flagged sequence may differ only at
its tie: the first differing accept decision must be a flagged test, and a
differing final token must have a CDF interval within 1e-6 + E of u and a
residual weight that the oracle's bound does not exclude (p_k - q_k above
-E S / 2).  Flag bit 3 alone (E above a tenth of the window: a residual of
near-equal distributions) keeps the exact comparison; such sequences are
counted as "widened".  p_i(x_i), q_i(x_i) agree within 1e-5 relative for f32
logits and 2e-3 for bf16 logits; residual sums within that plus E.
"""
from __future__ import annotations

import dataclasses
import sys

import numpy as np

import oracle
import workloads as W

TIE = oracle.TIE_TOL
PROB_RTOL = {"f32": 1e-5, "bf16": 2e-3}
TIE_BITS = 7       # oracle flags: accept-test tie, final-draw tie, empty residual
WIDENED = 8        # oracle flag: E above a tenth of the tie window
# device status bits a batch with oracle-unresolved residuals may raise
RESIDUAL_STATUS = 64 | 256


def ties(flags):
    """Sequences the parity rule lets differ at their tie."""
    return (np.asarray(flags) & TIE_BITS) != 0


def status_ok(status: int, ora) -> bool:
    """0, or only residual-resolution bits when the oracle itself could not
    resolve some residual (flag bit 3)."""
    if status == 0:
        return True
    return (status & ~RESIDUAL_STATUS) == 0 and bool((np.asarray(ora.flagged) & WIDENED).any())


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
    (spec_verify_run_greedy).  Greedy verification writes no p, q or
    residual sums; those come back empty."""
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
    # greedy verification writes tokens and counts only
    none = np.zeros(0, np.float64)
    return HostOutput(out.out_tokens.cpu().numpy(), out.num_accepted.cpu().numpy(),
                      none if mode == "greedy" else out.p_draft.cpu().numpy().astype(np.float64),
                      none if mode == "greedy" else out.q_draft.cpu().numpy().astype(np.float64),
                      none if mode == "greedy" else
                      out.residual_sum.cpu().numpy().astype(np.float64),
                      int(out.status.cpu().numpy()[0]) & 0xFFFFFFFF)


def _final_cdf(inp: W.VerifyInputs, b: int, n: int, point: bool = False):
    """The oracle's final-draw weights at position n (signed: p - q before
    the clip at 0), their running sum, and p (point: the draft distribution
    is the point mass at the draft token)."""
    g = int(inp.gammas[b])
    p = oracle.row_softmax(inp.target_logits[inp.target_row(b, n)], inp.temperature, inp.dtype)
    if n < g and point:
        w = p.copy()
        w[int(inp.draft_tokens[inp.draft_row(b, n)])] -= 1.0
    elif n < g:
        q = oracle.row_softmax(inp.draft_logits[inp.draft_row(b, n)], inp.temperature,
                               inp.dtype)
        w = p - q
    else:
        w = p
    return w, np.cumsum(np.maximum(w, 0.0)), p


@dataclasses.dataclass
class ParityReport:
    sequences: int
    flagged: int            # tie-flagged sequences (bits 0-2)
    tie_differences: int    # of those, sequences whose outputs differ
    widened: int            # sequences with E above a tenth of the window (bit 3)
    max_prob_rel: float
    max_residual_rel: float
    failures: list          # violations of the parity rule (empty: parity holds)


def parity_check(inp: W.VerifyInputs, gpu: HostOutput, ora, *, check_probs: bool = True,
                 point: bool = False) -> ParityReport:
    """The parity rule of this module's docstring, without asserting:
    every violation is listed in the report's `failures`."""
    B = inp.num_seqs
    cu = inp.cu_draft
    bad = []
    tie = ties(ora.flagged)
    widened = (np.asarray(ora.flagged) & WIDENED) != 0
    tie_diffs = 0
    for b in range(B):
        g = int(inp.gammas[b])
        t0 = int(cu[b]) + b
        d0 = int(cu[b])
        gn, on = int(gpu.num_accepted[b]), int(ora.num_accepted[b])
        gt = gpu.out_tokens[t0:t0 + g + 1]
        ot = ora.out_tokens[t0:t0 + g + 1]
        if gn == on and np.array_equal(gt, ot):
            continue
        if not tie[b]:
            bad.append((b, "difference outside a tie", gn, on, gt.tolist(), ot.tolist()))
            continue
        tie_diffs += 1
        if gn != on:
            i = min(gn, on)
            if not (ora.tie_accept[d0 + i] < TIE):
                bad.append((b, "accept decision differs away from a tie", gn, on))
            continue
        if not np.array_equal(gt[:gn], ot[:gn]) or not np.all(gt[gn + 1:] == -1):
            bad.append((b, "prefix or padding differs", gt.tolist(), ot.tolist()))
            continue
        # same count, different drawn token: it must sit at the final-draw
        # tie (window 1e-6 + E) with a weight the oracle does not exclude
        k = int(gt[gn])
        E = float(ora.final_err[b])
        if not 0 <= k < inp.vocab:
            bad.append((b, "final token out of range", k, int(ot[gn])))
            continue
        w, C, p = _final_cdf(inp, b, gn, point)
        if np.isfinite(E):
            S = float(C[-1])
            in_support = w[k] > -E * S / 2
            Cn = C / S
            u = float(inp.uniforms[t0 + g])
            lo = Cn[k - 1] if k > 0 else 0.0
            in_window = lo - TIE - E <= u <= Cn[k] + TIE + E
        else:                       # the residual is below the oracle's resolution
            in_support = p[k] > 0
            in_window = True
        if not (in_support and in_window):
            bad.append((b, "final token outside the tie window or support", k, int(ot[gn]), E))

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
                if rel.max() > rtol:
                    bad.append((name, f"relative error {rel.max():.3g} > {rtol}"))
        # residual sums where the counts agree; the oracle's own value is
        # known to E / 2 relative (infinite E: not resolved, not compared)
        E = np.asarray(ora.final_err)
        same_n = (gpu.num_accepted == ora.num_accepted) & np.isfinite(E)
        o = ora.residual_sum[same_n]
        g_ = gpu.residual_sum[same_n]
        e = E[same_n]
        if o.size:
            rel = np.abs(g_ - o) / np.maximum(np.abs(o), 1e-300)
            rel[o == 0] = np.abs(g_[o == 0])
            max_res_rel = float(rel.max())
            if (rel - (rtol + e / 2)).max() > 0:
                bad.append(("residual_sum", f"relative error {rel.max():.3g} > {rtol} + E/2"))
    return ParityReport(B, int(tie.sum()), tie_diffs, int(widened.sum()), max_prob_rel,
                        max_res_rel, bad)


def compare(inp: W.VerifyInputs, gpu: HostOutput, ora, *, label: str = "",
            check_probs: bool = True, point: bool = False) -> ParityReport:
    rep = parity_check(inp, gpu, ora, check_probs=check_probs, point=point)
    assert not rep.failures, (f"{label}: {len(rep.failures)} parity failures, "
                              f"first: {rep.failures[:3]}")
    log(f"[parity] {label}: seqs={rep.sequences} tie_flagged={rep.flagged} "
        f"tie_diffs={rep.tie_differences} widened={rep.widened} "
        f"max_prob_rel={rep.max_prob_rel:.3g} max_residual_rel={rep.max_residual_rel:.3g}")
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
