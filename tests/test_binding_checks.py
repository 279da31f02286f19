"""The Python binding refuses, before any call into libgrpo, a tensor whose
device, element type, layout or length does not fit what the call will touch.

libgrpo receives device addresses only and cannot see a buffer's size, so a
short or mistyped tensor would otherwise be read or written out of bounds by a
kernel.  These run on the CPU: a CPU tensor is wrapped to report itself as a
GPU one, and the library is replaced by a stub that records the calls that get
through (the stub never touches the addresses)."""

import pytest
import torch

from grpo_token_level_amd import ops


class Dev:
    """A CPU tensor presenting itself as a device tensor."""
    is_cuda = True

    def __init__(self, x):
        self._x = x

    def __getattr__(self, k):
        return getattr(self._x, k)

    def __getitem__(self, k):
        return Dev(self._x[k])


class StubLib:
    def __init__(self):
        self.calls = []

    def __getattr__(self, name):
        def f(*args):
            self.calls.append(name)
            return 0
        return f


@pytest.fixture
def stub(monkeypatch):
    lib = StubLib()
    monkeypatch.setattr(ops.C, "lib", lambda: lib)
    monkeypatch.setattr(ops, "_stream", lambda: None)
    return lib


N, V, ROWS = 12, 40, 3


def loss_inputs(n=N, n_src=None, dtype=torch.bfloat16):
    n_src = n if n_src is None else n_src
    f = dict(dtype=torch.float32)
    return {
        "logits": Dev(torch.zeros((n_src, V), dtype=dtype)),
        "target": Dev(torch.zeros(n_src, dtype=torch.int32)),
        "mask": Dev(torch.ones(n_src, dtype=torch.uint8)),
        "old_logp": Dev(torch.zeros(n_src, **f)),
        "tok_row_": Dev(torch.zeros(n, dtype=torch.int32)),
        "adv_row": Dev(torch.zeros(ROWS, **f)),
        "row_off": Dev(torch.tensor([0, 4, 8, n], dtype=torch.int64)),
    }


def workspace(n=N, rows=ROWS):
    f = dict(dtype=torch.float32)
    return {"logp": Dev(torch.zeros(n, **f)), "lse": Dev(torch.zeros(n, **f)), "entropy": Dev(torch.zeros(n, **f)),
            "loss_tok": Dev(torch.zeros(n, **f)), "kl_tok": Dev(torch.zeros(n, **f)),
            "tok_flags": Dev(torch.zeros(n, dtype=torch.uint8)),
            "row_stats": Dev(torch.zeros((rows, ops.STATS_BYTES), dtype=torch.uint8)),
            "chunk_stats": Dev(torch.zeros((1, ops.STATS_BYTES), dtype=torch.uint8))}


def call_loss(over=None, ws_over=None, **kw):
    args = loss_inputs()
    args.update(over or {})
    ws = workspace()
    ws.update(ws_over or {})
    kw.setdefault("dlogits", Dev(torch.zeros((N, V), dtype=torch.bfloat16)))
    return ops.loss_fwd_bwd(args.pop("logits"), *args.values(), ws=ws, **kw)


def test_loss_accepts_fitting_tensors(stub):
    call_loss()
    call_loss(dlogits=None)
    call_loss(over={"mask": Dev(torch.ones(N, dtype=torch.bool))})
    call_loss(ws_over={"lse": None})
    # a padded row stride on both sides
    pad = Dev(torch.zeros((N, V + 8), dtype=torch.bfloat16)[:, :V])
    call_loss(over={"logits": pad}, dlogits=Dev(torch.zeros((N, V + 24), dtype=torch.float32)[:, :V]))
    assert stub.calls == ["grpo_loss_fwd_bwd"] * 5


BAD_LOSS = {
    "target int64": ({"target": Dev(torch.zeros(N, dtype=torch.int64))}, {}, {}),
    "target short": ({"target": Dev(torch.zeros(N - 1, dtype=torch.int32))}, {}, {}),
    "target on the host": ({"target": torch.zeros(N, dtype=torch.int32)}, {}, {}),
    "mask float": ({"mask": Dev(torch.ones(N, dtype=torch.float32))}, {}, {}),
    "old_logp strided": ({"old_logp": Dev(torch.zeros(2 * N))[::2]}, {}, {}),
    "old_logp bf16": ({"old_logp": Dev(torch.zeros(N, dtype=torch.bfloat16))}, {}, {}),
    "tok_row short": ({"tok_row_": Dev(torch.zeros(N - 1, dtype=torch.int32))}, {}, {}),
    "adv_row short": ({"adv_row": Dev(torch.zeros(ROWS - 1))}, {}, {}),
    "row_off int32": ({"row_off": Dev(torch.tensor([0, 4, 8, N], dtype=torch.int32))}, {}, {}),
    "logits int": ({"logits": Dev(torch.zeros((N, V), dtype=torch.int16))}, {}, {}),
    "logits column-strided": ({"logits": Dev(torch.zeros((V, N), dtype=torch.bfloat16).t())}, {}, {}),
    "logp short": ({}, {"logp": Dev(torch.zeros(N - 1))}, {}),
    "entropy missing": ({}, {"entropy": None}, {}),
    "tok_flags int32": ({}, {"tok_flags": Dev(torch.zeros(N, dtype=torch.int32))}, {}),
    "row_stats one row short": ({}, {"row_stats": Dev(torch.zeros((ROWS - 1, ops.STATS_BYTES), dtype=torch.uint8))},
                                {}),
    "chunk_stats short": ({}, {"chunk_stats": Dev(torch.zeros(ops.STATS_BYTES - 1, dtype=torch.uint8))}, {}),
    "dlogits too few rows": ({}, {}, {"dlogits": Dev(torch.zeros((N - 1, V), dtype=torch.bfloat16))}),
    "dlogits other width": ({}, {}, {"dlogits": Dev(torch.zeros((N, V - 1), dtype=torch.bfloat16))}),
    "dlogits fp16": ({}, {}, {"dlogits": Dev(torch.zeros((N, V), dtype=torch.float16))}),
    "denom int32": ({}, {}, {"denom": Dev(torch.ones(1, dtype=torch.int32))}),
    "row_weight short": ({}, {}, {"row_weight": Dev(torch.ones(ROWS - 1))}),
    "ref_logp short": ({}, {}, {"ref_logp": Dev(torch.zeros(N - 1))}),
    "kl_tok missing": ({}, {"kl_tok": None}, {"ref_logp": Dev(torch.zeros(N))}),
}


@pytest.mark.parametrize("case", sorted(BAD_LOSS))
def test_loss_refuses_before_the_call(stub, case):
    over, ws_over, kw = BAD_LOSS[case]
    with pytest.raises(ValueError):
        call_loss(over, ws_over, **kw)
    assert stub.calls == []


def test_loss_tok_src_needs_batch_length_inputs(stub):
    """With tok_src the per-token inputs and dlogits are the batch's (n_src
    tokens) while the outputs and row arrays stay chunk-local (n tokens)."""
    n_src = 20
    args = loss_inputs(N, n_src)
    tok_src = Dev(torch.arange(N, dtype=torch.int64))
    dl = Dev(torch.zeros((n_src, V), dtype=torch.bfloat16))
    ops.loss_fwd_bwd(args.pop("logits"), *args.values(), ws=workspace(), dlogits=dl, tok_src=tok_src)
    assert stub.calls == ["grpo_loss_fwd_bwd"]
    for name, short in (("target", Dev(torch.zeros(N, dtype=torch.int32))),
                        ("mask", Dev(torch.ones(N, dtype=torch.uint8))),
                        ("old_logp", Dev(torch.zeros(N)))):
        args = loss_inputs(N, n_src)
        args[name] = short
        with pytest.raises(ValueError, match=name):
            ops.loss_fwd_bwd(args.pop("logits"), *args.values(), ws=workspace(), dlogits=dl, tok_src=tok_src)
    args = loss_inputs(N, n_src)
    logits = args.pop("logits")
    with pytest.raises(ValueError, match="dlogits"):
        ops.loss_fwd_bwd(logits, *args.values(), ws=workspace(),
                         dlogits=Dev(torch.zeros((N, V), dtype=torch.bfloat16)), tok_src=tok_src)
    with pytest.raises(ValueError, match="tok_src"):
        ops.loss_fwd_bwd(logits, *args.values(), ws=workspace(), dlogits=dl,
                         tok_src=Dev(torch.arange(N, dtype=torch.int32)))
    assert stub.calls == ["grpo_loss_fwd_bwd"]


H, VH = 16, 32


def lmhead_inputs():
    bf = dict(dtype=torch.bfloat16)
    x = loss_inputs()
    del x["logits"]
    return {"h": Dev(torch.zeros((N, H), **bf)), "W": Dev(torch.zeros((VH, H), **bf)),
            "Wt": Dev(torch.zeros((H, VH), **bf)), **x, "dW": Dev(torch.zeros((VH, H)))}


def call_lmhead(over=None, **kw):
    args = lmhead_inputs()
    args.update(over or {})
    kw.setdefault("dh", Dev(torch.zeros((N, H))))
    kw.setdefault("workspace", Dev(torch.zeros(64, dtype=torch.uint8)))
    return ops.lmhead_fwd_bwd(*args.values(), ws=workspace(), **kw)


def test_lmhead_checks(stub):
    call_lmhead()
    assert stub.calls == ["grpo_lmhead_fwd_bwd"]
    bad = [({"W": Dev(torch.zeros((VH, H)))}, {}),
           ({"Wt": Dev(torch.zeros((H + 8, VH), dtype=torch.bfloat16))}, {}),
           ({"Wt": Dev(torch.zeros((VH, H), dtype=torch.bfloat16).t())}, {}),
           ({"h": Dev(torch.zeros((N, H)))}, {}),
           ({"dW": Dev(torch.zeros((VH, H), dtype=torch.bfloat16))}, {}),
           ({"dW": Dev(torch.zeros((VH - 8, H)))}, {}),
           ({"target": Dev(torch.zeros(N - 1, dtype=torch.int32))}, {}),
           ({}, {"dh": Dev(torch.zeros((N - 1, H)))}),
           ({}, {"dh": Dev(torch.zeros((N, 2 * H)))[:, :H]}),
           ({}, {"workspace": torch.zeros(64, dtype=torch.uint8)})]
    for over, kw in bad:
        with pytest.raises(ValueError):
            call_lmhead(over, **kw)
    assert stub.calls == ["grpo_lmhead_fwd_bwd"]


def test_index_helpers_check(stub):
    row_off = Dev(torch.tensor([0, 3, 7], dtype=torch.int64))
    ops.tok_row(row_off, 7, out=Dev(torch.zeros(7, dtype=torch.int32)))
    with pytest.raises(ValueError):
        ops.tok_row(row_off, 7, out=Dev(torch.zeros(6, dtype=torch.int32)))
    with pytest.raises(ValueError):
        ops.tok_row(row_off, 7, out=Dev(torch.zeros(7, dtype=torch.int64)))
    src = Dev(torch.zeros(10))
    idx = Dev(torch.zeros(4, dtype=torch.int64))
    ops.gather(src, idx, out=Dev(torch.zeros(4)))
    with pytest.raises(ValueError):
        ops.gather(src, idx, out=Dev(torch.zeros(3)))
    with pytest.raises(ValueError):
        ops.gather(src, idx, out=Dev(torch.zeros(4, dtype=torch.float64)))
    with pytest.raises(ValueError):
        ops.gather(src, Dev(torch.zeros(4, dtype=torch.int32)), out=Dev(torch.zeros(4)))
    mask = Dev(torch.ones(7, dtype=torch.uint8))
    ops.count_valid(mask, out=Dev(torch.zeros(1, dtype=torch.int64)))
    with pytest.raises(ValueError):
        ops.count_valid(mask, out=Dev(torch.zeros(1, dtype=torch.int32)))
    n_seq = Dev(torch.ones(1, dtype=torch.int64))
    ops.row_weights(mask, row_off, ops.C.AGG_TOKEN_MEAN, n_seq, out=Dev(torch.zeros(2)))
    with pytest.raises(ValueError):
        ops.row_weights(mask, row_off, ops.C.AGG_TOKEN_MEAN, n_seq, out=Dev(torch.zeros(1)))
    rows = Dev(torch.tensor([1, 0], dtype=torch.int64))
    dst_off = Dev(torch.tensor([0, 4, 7], dtype=torch.int64))
    ops.chunk_tok_src(row_off, rows, dst_off, out=Dev(torch.zeros(7, dtype=torch.int64)))
    with pytest.raises(ValueError):
        ops.chunk_tok_src(row_off, rows, Dev(torch.tensor([0, 4], dtype=torch.int64)),
                          out=Dev(torch.zeros(7, dtype=torch.int64)))
    x = Dev(torch.zeros((8, 16), dtype=torch.bfloat16))
    ops.transpose_bf16(x, out=Dev(torch.zeros((16, 8), dtype=torch.bfloat16)))
    with pytest.raises(ValueError):
        ops.transpose_bf16(x, out=Dev(torch.zeros((16, 7), dtype=torch.bfloat16)))
    with pytest.raises(ValueError):
        ops.transpose_bf16(x, out=Dev(torch.zeros((15, 8), dtype=torch.bfloat16)))
    assert stub.calls == ["grpo_tok_row", "grpo_gather", "grpo_count_valid", "grpo_row_weights",
                          "grpo_chunk_tok_src", "grpo_transpose_bf16"]


def test_probe_compare_and_logprob_check(stub):
    n = 9
    mask = Dev(torch.ones(n, dtype=torch.uint8))
    out = Dev(torch.zeros(ops.PROBE_STATS_BYTES, dtype=torch.uint8))
    ops.probe_compare(Dev(torch.zeros(n)), Dev(torch.zeros(n)), mask, out=out)
    with pytest.raises(ValueError):
        ops.probe_compare(Dev(torch.zeros(n - 1)), Dev(torch.zeros(n)), mask, out=out)
    with pytest.raises(ValueError):
        ops.probe_compare(Dev(torch.zeros(n)), Dev(torch.zeros(n)), mask,
                          out=Dev(torch.zeros(ops.PROBE_STATS_BYTES - 1, dtype=torch.uint8)))
    assert stub.calls == ["grpo_probe_compare"]
    logits = Dev(torch.zeros((n, V), dtype=torch.float32))
    with pytest.raises(ValueError):
        ops.logprob_fwd(logits, Dev(torch.zeros(n - 1, dtype=torch.int32)), mask)
    with pytest.raises(ValueError):
        ops.logprob_fwd(logits, Dev(torch.zeros(n, dtype=torch.int32)), Dev(torch.ones(n - 1, dtype=torch.uint8)))
    assert stub.calls == ["grpo_probe_compare"]
