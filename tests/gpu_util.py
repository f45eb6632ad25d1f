"""Shared helpers for the GPU parity tests (inputs on the CPU, same tensors to both sides)."""
import numpy as np
import torch

import oracle
from draft_tree_build_amd import api

DEV = "cuda:0"


def note(msg: str) -> None:
    """Name the case before a GPU step (a fault may leave nothing else behind)."""
    print("[gpu-case] " + msg, flush=True)


def gpu_build(logits_cpu, roots_cpu, K, N, tau, ws=None):
    B, L, V = logits_cpu.shape
    r = api.Round(B, L, V, K, N, DEV)
    if ws is not None:
        r.ws_build = ws
    logits = logits_cpu.to(DEV)
    roots = torch.as_tensor(roots_cpu, dtype=torch.int32).to(DEV)
    r.build(logits, roots, tau)
    torch.cuda.synchronize()
    return dict(tokens=r.tokens.cpu().numpy(), parents=r.parents.cpu().numpy(),
                depths=r.depths.cpu().numpy(), scores=r.scores.cpu().numpy(),
                num_nodes=r.num_nodes.cpu().numpy(),
                mask=r.mask.cpu().numpy().view(np.uint64),
                topk_tok=r.topk_tokens.cpu().numpy(), topk_lp=r.topk_logprobs.cpu().numpy(),
                status=r.status.cpu().numpy()), r


def assert_same_build(g, o, rows_only=False):
    np.testing.assert_array_equal(g["topk_tok"], o["topk_tok"])
    np.testing.assert_array_equal(g["topk_lp"].view(np.uint32), o["topk_lp"].view(np.uint32))
    np.testing.assert_array_equal(g["status"], o["status"])
    if rows_only:
        return
    np.testing.assert_array_equal(g["num_nodes"], o["num_nodes"])
    np.testing.assert_array_equal(g["tokens"], o["tokens"])
    np.testing.assert_array_equal(g["parents"], o["parents"])
    np.testing.assert_array_equal(g["depths"], o["depths"])
    np.testing.assert_array_equal(g["scores"].view(np.uint32), o["scores"].view(np.uint32))
    np.testing.assert_array_equal(g["mask"], o["mask"])


def attn_tol(dtype):
    # bf16: |gpu - ref| <= 1e-3 + 2e-2 |ref|; f32: 1e-5 + 1e-5 |ref|
    return (1e-3, 2e-2) if dtype == torch.bfloat16 else (1e-5, 1e-5)


def check_attn(out_gpu, ref, sel, dtype):
    atol, rtol = attn_tol(dtype)
    got = np.stack([out_gpu[b, i, h].float().numpy() for (b, i, h) in sel]).astype(np.float64)
    err = np.abs(got - ref)
    bad = err > atol + rtol * np.abs(ref)
    assert not bad.any(), "max err %.3g at %s (ref %.4g got %.4g); %d of %d elements" % (
        err.max(), sel[int(np.argwhere(bad)[0][0])], ref[bad][0], got[bad][0], bad.sum(), bad.size)
