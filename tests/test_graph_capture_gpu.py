"""Every entry point captured in a HIP graph (torch.cuda.CUDAGraph) and
replayed several times, with new inputs copied into the captured buffers
between replays and eager work and synchronisations in between: each replay
must give exactly what an eager call gives on the same inputs (the kernels
clear their own counters, so a replay needs nothing else)."""
import numpy as np
import pytest

import workloads as W
from tests.gpu_helpers import log, make_verifier, to_device

pytestmark = pytest.mark.gpu

REPLAYS = 4


def _inputs(k: int):
    # same shapes for every k (the captured launch has fixed sizes), new values
    return W.build(f"graph {k}", 900 + k, [3, 0, 8, 5, 1, 8, 2, 6], 20000, W.BF16, 0.9,
                   W.boosted_random_ids_rows(3.0, 20, 8.0), 1.0)


def _copy_into(dst, src):
    dst.cu.copy_(src.cu)
    dst.target.copy_(src.target)
    dst.draft.copy_(src.draft)
    dst.tokens.copy_(src.tokens)
    dst.uniforms.copy_(src.uniforms)


def _host(out):
    return {k: getattr(out, k).cpu().numpy().copy()
            for k in ("out_tokens", "num_accepted", "p_draft", "q_draft", "residual_sum")
            if getattr(out, k) is not None}


@pytest.mark.parametrize("mode", ["sampled", "point", "greedy"])
def test_chain_entry_points_replay_in_a_graph(mode):
    import torch
    log(f"[graph] {mode}")
    inps = [_inputs(k) for k in range(REPLAYS)]
    if mode != "sampled":
        inps = [W.with_deterministic_drafts(x) for x in inps]
    sv = make_verifier(inps[0])
    dev_sets = [to_device(x) for x in inps]
    B, R_d, T = inps[0].num_seqs, inps[0].draft_rows, inps[0].temperature

    def call(d, out):
        if mode == "sampled":
            return sv(d.cu, d.target, d.draft, d.tokens, d.uniforms, T, out=out)
        if mode == "point":
            return sv.point_drafts(d.cu, d.target, d.tokens, d.uniforms, T, out=out)
        return sv.greedy(d.cu, d.target, d.tokens, out=out)

    eager = []
    for d in dev_sets:
        out = sv.allocate_outputs(B, R_d)
        call(d, out)
        torch.cuda.synchronize()
        eager.append(_host(out))

    cap_in = to_device(inps[0])
    cap_out = sv.allocate_outputs(B, R_d)
    call(cap_in, cap_out)                       # warm-up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(cap_in, cap_out)
    for rep in range(2 * REPLAYS):
        k = (3 * rep + 1) % REPLAYS
        _copy_into(cap_in, dev_sets[k])
        g.replay()
        torch.cuda.synchronize()
        got = _host(cap_out)
        for key, ref in eager[k].items():
            if mode == "greedy" and key in ("p_draft", "q_draft", "residual_sum"):
                continue
            assert np.array_equal(got[key], ref, equal_nan=True), (mode, rep, k, key)
        # eager work between replays
        tmp = sv.allocate_outputs(B, R_d)
        call(dev_sets[(k + 1) % REPLAYS], tmp)
        torch.cuda.synchronize()
    assert int(cap_out.status.cpu().item()) == 0


@pytest.mark.parametrize("mode", ["tree_greedy", "tree_point"])
def test_tree_entry_points_replay_in_a_graph(mode):
    import torch
    log(f"[graph] {mode}")
    shapes = [W.tree_shape(W.TREE_17)] * 6 + [W.tree_shape([(1, 1)] * 5)]
    trs = [W.build_tree(f"graph tree {k}", 950 + k, shapes, 20000, W.BF16, 1.0,
                        W.boosted_top_rows(2.0, 4, 6.0), 0.6) for k in range(REPLAYS)]
    from rejection_sampling_verify_08_amd import SpecVerifier
    sv = SpecVerifier(trs[0].vocab, "bf16", max_seqs=trs[0].num_seqs,
                      max_draft_rows=trs[0].rows)
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    rows = lambda tr: torch.from_numpy(tr.target_logits.view(np.int16)).view(torch.bfloat16).cuda()
    sets = [(d(t.cu_nodes), d(t.parent), d(t.tokens), rows(t), d(t.uniforms)) for t in trs]

    def call(s, out):
        if mode == "tree_greedy":
            return sv.tree_greedy(s[0], s[1], s[2], s[3], out=out)
        return sv.tree_point(s[0], s[1], s[2], s[3], s[4], 1.0, out=out)

    eager = []
    for s in sets:
        o = call(s, None)
        torch.cuda.synchronize()
        eager.append((o.out_tokens.cpu().numpy().copy(), o.out_path.cpu().numpy().copy(),
                      o.num_accepted.cpu().numpy().copy()))
    cap = tuple(x.clone() for x in sets[0])
    cap_out = call(cap, None)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(cap, cap_out)
    for rep in range(2 * REPLAYS):
        k = (3 * rep + 1) % REPLAYS
        for dst, src in zip(cap, sets[k]):
            dst.copy_(src)
        g.replay()
        torch.cuda.synchronize()
        got = (cap_out.out_tokens.cpu().numpy(), cap_out.out_path.cpu().numpy(),
               cap_out.num_accepted.cpu().numpy())
        for a, b in zip(got, eager[k]):
            assert np.array_equal(a, b), (mode, rep, k)
        call(sets[(k + 1) % REPLAYS], None)
        torch.cuda.synchronize()
    assert int(cap_out.status.cpu().item()) == 0


def test_controller_replays_in_a_graph():
    import torch
    from rejection_sampling_verify_08_amd import DraftLengthController, adapt_params
    log("[graph] adaptive controller")
    B = 40
    rng = np.random.default_rng(12)
    gam = rng.integers(0, 9, size=B).astype(np.int32)
    cu = torch.from_numpy(np.concatenate([[0], np.cumsum(gam)]).astype(np.int32)).cuda()
    acc_sets = [torch.from_numpy((rng.random(B) * (gam + 1)).astype(np.int32).clip(0, gam)).cuda()
                for _ in range(REPLAYS)]
    p = adapt_params("last10")
    eager = DraftLengthController(B, p, device="cuda")
    graphed = DraftLengthController(B, p, device="cuda")
    nk = torch.empty(B, dtype=torch.int32, device="cuda")
    ncu = torch.empty(B + 1, dtype=torch.int32, device="cuda")
    acc = acc_sets[0].clone()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        graphed.update(cu, acc, next_k=nk, next_cu=ncu)
    for rep in range(3 * REPLAYS):
        k = rep % REPLAYS
        acc.copy_(acc_sets[k])
        g.replay()
        ek, ecu = eager.update(cu, acc_sets[k])
        torch.cuda.synchronize()
        assert np.array_equal(nk.cpu().numpy(), ek.cpu().numpy()), rep
        assert np.array_equal(ncu.cpu().numpy(), ecu.cpu().numpy()), rep
    assert graphed.totals() == eager.totals()
