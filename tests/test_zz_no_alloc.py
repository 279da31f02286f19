"""The LM-head entry point that allocates nothing (grpo_lmhead_fwd_bwd_noalloc),
through the C ABI, against the workspace entry point it mirrors and against
the oracle.

Two calls in a row on one GPU share the library's fixed scratch: a large
chunk at the compaction workload's sizes (H 2048, V 151936), then a smaller
one; each is compared with grpo_lmhead_fwd_bwd on the same inputs.  The
per-token outputs and dW come out of the same tiles in both and are equal
bit for bit; dh sums the same bf16 products split another way, so rows agree
to float32 summation order.  The smaller chunk is also checked against the
oracle.  A chunk too large for the scratch is refused before any launch, and
a call leaves the device's free memory unchanged."""

import numpy as np
import pytest
import torch

from gpu_common import DEV, oracle_lmhead_at_kernel_clip, to_f64
from grpo_token_level_amd import ops
from grpo_token_level_amd._capi import LMHEAD_NOALLOC_SCRATCH_BYTES

pytestmark = pytest.mark.gpu


def _case(n, H, V, seed):
    g = torch.Generator(device="cpu").manual_seed(seed)
    h = (torch.randn((n, H), generator=g)).to(torch.bfloat16)
    W = (torch.randn((V, H), generator=g) * 0.02).to(torch.bfloat16)
    rng = np.random.default_rng(seed)
    target = rng.integers(0, V, n).astype(np.int32)
    mask = (rng.random(n) > 0.15).astype(np.uint8)
    row_off = np.array([0, n // 4, n // 2, 3 * n // 4, n], np.int64)
    tok_row = np.repeat(np.arange(4, dtype=np.int32), np.diff(row_off))
    adv = rng.normal(0, 1, 4).astype(np.float32)
    old = rng.normal(-12.0, 0.5, n).astype(np.float32)
    G = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)  # noqa: E731
    return dict(h=h.to(DEV), W=W.to(DEV), h_cpu=h, W_cpu=W, target=target, mask=mask, old=old, adv=adv,
                tok_row=tok_row, row_off=row_off,
                g={k: G(v) for k, v in (("target", target), ("mask", mask), ("old", old), ("adv", adv),
                                        ("tok_row", tok_row), ("row_off", row_off))})


def _outputs(n, H, V):
    ws = ops.loss_workspace(n, 4, torch.device(DEV))
    return ws, torch.empty((n, H), dtype=torch.float32, device=DEV), torch.zeros((V, H), dtype=torch.float32,
                                                                                 device=DEV)


def _call(c, Wt, noalloc, out):
    ws, dh, dW = out
    g = c["g"]
    N = max(1, int(c["mask"].sum()))
    return ops.lmhead_fwd_bwd(c["h"], c["W"], Wt, g["target"], g["mask"], g["old"], g["tok_row"], g["adv"],
                              g["row_off"], dW, scale=1.0 / N, dh=dh, ws=ws, noalloc=noalloc)


def _same_as_workspace_path(c, label):
    n, H = c["h"].shape
    V = c["W"].shape[0]
    Wt = ops.transpose_bf16(c["W"])
    a_out = _outputs(n, H, V)
    b_out = _outputs(n, H, V)
    _call(c, Wt, False, a_out)
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    _call(c, Wt, True, b_out)
    torch.cuda.synchronize()
    assert torch.cuda.mem_get_info()[0] == free0, f"{label}: device memory changed across the call"
    (wa, dha, dWa), (wb, dhb, dWb) = a_out, b_out
    for k in ("logp", "lse", "entropy", "loss_tok", "tok_flags", "row_stats", "chunk_stats"):
        assert torch.equal(wa[k], wb[k]), (label, k)
    assert torch.equal(dWa, dWb), label
    a, b = to_f64(dha), to_f64(dhb)
    err = np.sqrt(np.sum((a - b) ** 2, axis=1))
    assert np.all(err <= 1e-5 * np.sqrt(np.sum(a * a, axis=1)) + 1e-30), (label, float(np.max(err)))
    return b_out


def test_noalloc_matches_the_workspace_entry_point_two_calls_in_a_row():
    print("noalloc: a compaction-size chunk, then a smaller one", flush=True)
    big = _case(2000, 2048, 151936, seed=1)
    _same_as_workspace_path(big, "n=2000 H=2048 V=151936")
    del big
    small = _case(300, 768, 5000, seed=2)
    ws, dh, dW = _same_as_workspace_path(small, "n=300 H=768 V=5000")
    # the smaller call against the oracle (as the workspace path is checked)
    h64, W64 = small["h_cpu"].double().numpy(), small["W_cpu"].double().numpy()
    N = int(small["mask"].sum())
    ref, _ = oracle_lmhead_at_kernel_clip(ws["tok_flags"].cpu().numpy(), h64, W64, small["target"], small["mask"],
                                          small["old"], small["adv"].astype(np.float64)[small["tok_row"]], 1.0 / N)
    v = ref["valid"]
    assert np.max(np.abs(to_f64(ws["logp"])[v] - ref["logp"][v])) <= 1e-4
    bound = 2.0 ** -8 + 2.0 ** -12
    for got, want, mag in ((to_f64(dh), ref["dh"], np.abs(ref["dz"]) @ np.abs(W64)),
                           (to_f64(dW), ref["dW"], np.abs(ref["dz"]).T @ np.abs(h64))):
        err = np.sqrt(np.sum((got - want) ** 2, axis=1))
        assert np.all(err <= bound * np.sqrt(np.sum(mag ** 2, axis=1)))


def test_noalloc_refuses_a_chunk_beyond_its_scratch():
    # 20000 tokens at V = 151936 need ~760 MB of log-softmax slice partials alone
    n, H, V = 20000, 2048, 151936
    assert n * ((V + 63) // 64) * 16 > LMHEAD_NOALLOC_SCRATCH_BYTES
    h = torch.zeros((n, H), dtype=torch.bfloat16, device=DEV)
    W = torch.zeros((V, H), dtype=torch.bfloat16, device=DEV)
    Wt = torch.zeros((H, V), dtype=torch.bfloat16, device=DEV)
    dW = torch.zeros((V, H), dtype=torch.float32, device=DEV)
    z32 = torch.zeros(n, dtype=torch.int32, device=DEV)
    with pytest.raises(ops.GrpoError) as e:
        ops.lmhead_fwd_bwd(h, W, Wt, z32, torch.ones(n, dtype=torch.uint8, device=DEV),
                           torch.zeros(n, dtype=torch.float32, device=DEV), z32,
                           torch.zeros(1, dtype=torch.float32, device=DEV),
                           torch.tensor([0, n], dtype=torch.int64, device=DEV), dW, noalloc=True)
    assert e.value.kind == "ECAPACITY" and "scratch" in str(e.value)
    torch.cuda.synchronize()
    assert not dW.any()
