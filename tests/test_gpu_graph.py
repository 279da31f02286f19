"""The fused loss path captured in a HIP graph (torch.cuda.graph over the
library's launches on the capturing stream) and replayed: every replay, with
eager work and synchronisations between replays and the outputs cleared
beforehand, reproduces the eager run bit for bit.  Covers the valid-token
count, the fused kernel on both paths (register and streaming), the row and
chunk statistics and the extra terms' row weights."""

import numpy as np
import pytest
import torch

from gpu_common import DEV, make_chunk
from grpo_token_level_amd import ops
from grpo_token_level_amd._capi import AGG_SEQ_MEAN_TOKEN_MEAN, KL_K3

pytestmark = pytest.mark.gpu


def _setup(ld=None):
    chunks = [make_chunk(64, 1024, torch.float32, seed=s, n_rows=8, ld=ld) for s in range(4)]
    outs = [ops.loss_workspace(64, 8, DEV) for _ in chunks]
    dls = [torch.empty((64, 1024), dtype=torch.float32, device=DEV) for _ in chunks]
    N = torch.empty(1, dtype=torch.int64, device=DEV)
    B = torch.empty(1, dtype=torch.int64, device=DEV)
    w = [torch.empty(8, dtype=torch.float32, device=DEV) for _ in chunks]
    mask_all = torch.cat([c["g"]["mask"] for c in chunks])
    return chunks, outs, dls, N, B, w, mask_all


def _device_work(chunks, outs, dls, N, B, w, mask_all, terms):
    ops.count_valid(mask_all, out=N)
    for c, ws, dl, wr in zip(chunks, outs, dls, w):
        g = c["g"]
        kw = dict(scale=1.0, denom=N)
        if terms:
            ops.count_rows(g["mask"], g["row_off"], out=B)
            ops.row_weights(g["mask"], g["row_off"], AGG_SEQ_MEAN_TOKEN_MEAN, B, out=wr)
            kw = dict(scale=1.0, row_weight=wr, ref_logp=g["old"], ent_coef=0.01, kl_coef=0.05, kl_type=KL_K3)
        ops.loss_fwd_bwd(c["logits"], g["target"], g["mask"], g["old"], g["tok_row"], g["adv_row"], g["row_off"],
                         dlogits=dl, ws=ws, **kw)


KEYS = ("logp", "entropy", "loss_tok", "tok_flags", "row_stats", "chunk_stats")


def _keys(terms):
    # kl_tok is written only when a reference log-prob is given
    return KEYS + ("kl_tok",) if terms else KEYS


def _snapshot(outs, dls, terms):
    snap = [dl.clone() for dl in dls]
    for ws in outs:
        for k in _keys(terms):
            snap.append(ws[k].clone())
    return snap


def _clear(outs, dls, terms):
    for dl in dls:
        dl.fill_(float("nan"))
    for ws in outs:
        for k in _keys(terms):
            ws[k].zero_()


@pytest.mark.parametrize("terms,ld", [(False, None), (True, None), (False, 1029)])
def test_graph_replays_match_the_eager_run(terms, ld):
    state = _setup(ld)
    chunks, outs, dls = state[0], state[1], state[2]
    _device_work(*state, terms)
    torch.cuda.synchronize()
    eager = _snapshot(outs, dls, terms)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        _device_work(*state, terms)
    torch.cuda.synchronize()
    for rep in range(4):
        _clear(outs, dls, terms)
        # unrelated eager work between replays
        x = torch.randn(1 << 20, device=DEV)
        (x * 2).sum().item()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = _snapshot(outs, dls, terms)
        for a, b in zip(eager, got):
            assert torch.equal(a.view(torch.uint8) if a.dtype != torch.uint8 else a,
                               b.view(torch.uint8) if b.dtype != torch.uint8 else b), rep
    assert np.isfinite(ops.stats_to_dicts(outs[0]["chunk_stats"])[0]["loss_sum"])


# The LM head's deferred-dW step under capture (the callers that capture the
# library's launches): two chunks append to a dW window and the flush adds dW,
# captured once (the window's host count ends at zero with the flush, as the
# replays' device counter does) and replayed; each replay, with dW and the
# per-token outputs cleared beforehand and eager work in between, reproduces
# the eager run bit for bit.  With the logits kept for pass 2 as well.
@pytest.mark.parametrize("keep_z", [False, True])
def test_deferred_lmhead_step_replays_match_the_eager_run(keep_z):
    from test_gpu_lmhead import _case
    n, H, V = 300, 128, 5000
    c = _case(n, H, V, seed=21)
    N = max(1, int(c["mask"].sum()))
    Wt = ops.transpose_bf16(c["W"])
    bounds = [(0, 130), (130, n)]
    win = ops.LmheadDwWindow(sum((b - a + 63) // 64 * 64 for a, b in bounds), H, V, device=DEV)
    wsp = torch.empty(ops.lmhead_workspace_bytes(max(b - a for a, b in bounds), H, V, keep_z, True),
                      dtype=torch.uint8, device=DEV)
    outs = [ops.loss_workspace(b - a, 1, DEV) for a, b in bounds]
    dhs = [torch.empty((b - a, H), dtype=torch.float32, device=DEV) for a, b in bounds]
    rows = [torch.zeros(b - a, dtype=torch.int32, device=DEV) for a, b in bounds]
    advs = [c["g"]["adv"][i:i + 1].clone() for i in range(len(bounds))]
    offs = [torch.tensor([0, b - a], dtype=torch.int64, device=DEV) for a, b in bounds]
    dW = torch.zeros((V, H), dtype=torch.float32, device=DEV)
    g = c["g"]

    def work():
        for i, (a, b) in enumerate(bounds):
            ops.lmhead_fwd_bwd(c["h"][a:b], c["W"], Wt, g["target"][a:b], g["mask"][a:b], g["old"][a:b], rows[i],
                               advs[i], offs[i], None, scale=1.0 / N, dh=dhs[i], ws=outs[i], workspace=wsp,
                               keep_z=keep_z, dw_window=win)
        win.flush(dW)

    keys = ("logp", "entropy", "loss_tok", "tok_flags", "row_stats", "chunk_stats")
    work()
    torch.cuda.synchronize()
    eager = [dW.clone()] + [d.clone() for d in dhs] + [ws[k].clone() for ws in outs for k in keys]
    graph = torch.cuda.CUDAGraph()
    dW.zero_()
    with torch.cuda.graph(graph):
        work()
    torch.cuda.synchronize()
    assert win.reserved == 0
    for rep in range(3):
        dW.zero_()
        for d in dhs:
            d.fill_(float("nan"))
        for ws in outs:
            for k in keys:
                ws[k].zero_()
        x = torch.randn(1 << 20, device=DEV)
        (x * 2).sum().item()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [dW] + dhs + [ws[k] for ws in outs for k in keys]
        for a, b in zip(eager, got):
            assert torch.equal(a.view(torch.uint8) if a.dtype != torch.uint8 else a,
                               b.view(torch.uint8) if b.dtype != torch.uint8 else b), rep
