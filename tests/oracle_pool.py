"""The oracle over every token of a full-size batch, on a pool of CPU processes.

Test infrastructure: the parent copies blocks of token rows from the GPU into
shared memory as their raw bits (bf16 or fp32), spawned worker processes read
them back as exact float32 values and run ``oracle.loss_fwd_bwd`` (forward
outputs only, no dlogits) on slices of a block.  The workers never touch the
GPU.  Per-token results come back in token order."""

import os
from multiprocessing import get_context, shared_memory

import numpy as np

import oracle

KEYS = ("logp", "lse", "entropy", "loss_tok", "coef")
FLAGS = ("clipped", "valid", "nonfinite")


def pool_size():
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _forward_task(args):
    name, shape, kind, a, e, target, mask, old, adv, scale, eps = args
    shm = shared_memory.SharedMemory(name=name)
    try:
        raw = np.ndarray(shape, dtype=np.uint16 if kind == "bf16" else np.float32, buffer=shm.buf)[a:e]
        if kind == "bf16":
            z = (raw.astype(np.uint32) << 16).view(np.float32)     # the exact bf16 values
        else:
            z = np.array(raw)
        out = oracle.loss_fwd_bwd(z, target, mask, old, adv, scale, eps[0], eps[1], want_dz=False)
        return a, {k: out[k] for k in KEYS + FLAGS}
    finally:
        shm.close()


def _loss_task(args):
    name, shape, a, e, target, mask, old, adv, scale, eps, cols, rows = args
    shm = shared_memory.SharedMemory(name=name)
    try:
        z = np.array(np.ndarray(shape, dtype=np.float32, buffer=shm.buf)[a:e])
        out = oracle.loss_fwd_bwd(z, target, mask, old, adv, scale, eps[0], eps[1], want_dz=True)
        dz = out["dz"]
        keep = [r for r in rows if a <= r < e]
        return a, {k: out[k] for k in KEYS + FLAGS}, dz[:, cols], {r: dz[r - a] for r in keep}
    finally:
        shm.close()


class OraclePool:
    """``with OraclePool() as P: ref = P.forward(...)``."""

    def __init__(self, processes=None):
        self.n = processes or pool_size()
        self.pool = None

    def __enter__(self):
        self.pool = get_context("spawn").Pool(self.n)
        return self

    def __exit__(self, *exc):
        self.pool.terminate()
        self.pool.join()
        return False

    def forward(self, logits, idx, target, mask, old, adv_tok, scale, eps=(0.2, 0.2), block=4096, task=32,
                progress=None):
        """Oracle forward outputs for the token rows ``idx`` of the GPU matrix
        ``logits`` [n_tok, V] (bf16 or fp32); ``target``, ``mask``, ``old``,
        ``adv_tok`` are host arrays over ``idx``.  Returns a dict of arrays over
        ``idx`` (logp, lse, entropy, loss_tok, coef, clipped, valid, nonfinite)."""
        import torch
        idx = np.asarray(idx, np.int64)
        n = len(idx)
        out = {k: np.zeros(n, np.float64) for k in KEYS}
        out.update({k: np.zeros(n, bool) for k in FLAGS})
        kind = "bf16" if logits.dtype == torch.bfloat16 else "f32"
        for b0 in range(0, n, block):
            sel = idx[b0:b0 + block]
            rows = logits[torch.as_tensor(sel, device=logits.device)]
            host = rows.view(torch.int16 if kind == "bf16" else torch.float32).cpu().numpy()
            del rows
            shm = shared_memory.SharedMemory(create=True, size=max(host.nbytes, 1))
            try:
                np.ndarray(host.shape, dtype=host.dtype, buffer=shm.buf)[:] = host
                sl = slice(b0, b0 + len(sel))
                tg, mk, od, av = target[sl], mask[sl], old[sl], adv_tok[sl]
                tasks = [(shm.name, host.shape, kind, a, min(a + task, len(sel)), tg[a:a + task], mk[a:a + task],
                          od[a:a + task], av[a:a + task], scale, eps) for a in range(0, len(sel), task)]
                for a, res in self.pool.imap_unordered(_forward_task, tasks):
                    for k, v in res.items():
                        out[k][b0 + a:b0 + a + len(v)] = v
            finally:
                shm.close()
                shm.unlink()
            if progress:
                progress(b0 + len(sel), n)
        return out

    def loss_host(self, z, target, mask, old, adv_tok, scale, cols, rows, eps=(0.2, 0.2), task=32):
        """The oracle on a host float32 logit matrix ``z`` [n, V] (exact values
        of a product computed on the host): per-token forward outputs, the
        dlogits columns ``cols`` of every token ([n, len(cols)]) and the whole
        dlogits rows of the tokens ``rows`` (a dict token -> row)."""
        n = z.shape[0]
        out = {k: np.zeros(n, np.float64) for k in KEYS}
        out.update({k: np.zeros(n, bool) for k in FLAGS})
        dz_cols = np.zeros((n, len(cols)), np.float64)
        dz_rows = {}
        shm = shared_memory.SharedMemory(create=True, size=max(z.nbytes, 1))
        try:
            np.ndarray(z.shape, dtype=np.float32, buffer=shm.buf)[:] = z
            rows = sorted(int(r) for r in rows)
            tasks = [(shm.name, z.shape, a, min(a + task, n), target[a:a + task], mask[a:a + task],
                      old[a:a + task], adv_tok[a:a + task], scale, eps, np.asarray(cols),
                      [r for r in rows if a <= r < a + task]) for a in range(0, n, task)]
            for a, res, dc, dr in self.pool.imap_unordered(_loss_task, tasks):
                for k, v in res.items():
                    out[k][a:a + len(v)] = v
                dz_cols[a:a + dc.shape[0]] = dc
                dz_rows.update(dr)
        finally:
            shm.close()
            shm.unlink()
        out["dz_cols"] = dz_cols
        out["dz_rows"] = dz_rows
        return out
