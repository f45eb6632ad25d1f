"""Thin Python binding of the C ABI in include/ddtree.h (ctypes + torch tensors).

Argument marshalling only: every function passes device pointers, sizes and
the current HIP stream to the library of the same name; all work runs in the
HIP kernels. The library must be built (``python -m draft_tree_build_amd.build``);
nothing here falls back to another implementation.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libddtree.so")

BF16 = 0
F32 = 1
STATUS_NONFINITE = 1
STATUS_ALL_NEG_INF = 2
STATUS_OUT_NONFINITE = 4
STATUS_BAD_KV = 8
_lib = None


class DDTreeError(RuntimeError):
    def __init__(self, fn: str, code: int):
        super().__init__("%s failed: %d (%s)" % (fn, code, strerror(code)))
        self.code = code


def lib():
    """The loaded libddtree.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libddtree.so is not built; run: python -m draft_tree_build_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, f32, sz = (ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float,
                                 ctypes.c_size_t)
        L.ddtree_version.restype = i32
        L.ddtree_version.argtypes = []
        L.ddtree_strerror.restype = ctypes.c_char_p
        L.ddtree_strerror.argtypes = [i32]
        L.ddtree_build_workspace_size.restype = sz
        L.ddtree_build_workspace_size.argtypes = [i32, i32, i32, i32, i32]
        L.ddtree_build.restype = i32
        L.ddtree_build.argtypes = [vp, i32, vp, i32, i32, i32, i32, i32, f32, vp, vp, vp, vp, vp,
                                   vp, vp, vp, vp, vp, sz, vp]
        L.ddtree_build_noalloc.restype = i32
        L.ddtree_build_noalloc.argtypes = [vp, i32, vp, i32, i32, i32, i32, i32, f32, vp, vp, vp,
                                           vp, vp, vp, vp, vp, vp, vp]
        L.ddtree_mask.restype = i32
        L.ddtree_mask.argtypes = [vp, vp, i32, i32, vp, vp]
        L.ddtree_verify_workspace_size.restype = sz
        L.ddtree_verify_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32, i32]
        L.ddtree_verify_attn.restype = i32
        L.ddtree_verify_attn.argtypes = [vp, vp, vp, i32, vp, vp, vp, vp, i32, i32, i32, i32, i32,
                                         i32, i64, f32, vp, vp, vp, sz, vp]
        L.ddtree_accept_workspace_size.restype = sz
        L.ddtree_accept_workspace_size.argtypes = [i32, i32]
        L.ddtree_accept_sample.restype = i32
        L.ddtree_accept_sample.argtypes = [vp, i32, vp, vp, vp, i32, i32, i32, i32, f32,
                                           ctypes.c_uint64, ctypes.c_uint64, vp, vp, vp, vp, vp,
                                           vp, sz, vp]
        L.ddtree_commit_kv.restype = i32
        L.ddtree_commit_kv.argtypes = [vp, vp, i32, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32,
                                       i64, vp, vp, vp]
        L.ddtree_accept.restype = i32
        L.ddtree_accept.argtypes = [vp, i32, vp, vp, vp, vp, i32, i32, i32, i32, vp, vp, vp, vp,
                                    vp, vp, sz, vp]
        L.ddtree_probe_mfma_bf16.restype = i32
        L.ddtree_probe_mfma_bf16.argtypes = [vp, i32, i32, vp]
        L.ddtree_probe_hbm_read.restype = i32
        L.ddtree_probe_hbm_read.argtypes = [vp, i64, vp, i32, vp]
        _lib = L
    return _lib


def version() -> int:
    return int(lib().ddtree_version())


def strerror(code: int) -> str:
    return lib().ddtree_strerror(int(code)).decode()


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to the C ABI must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise ValueError("expected bfloat16 or float32 data, got %s" % t.dtype)


def _stream(stream, device) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _check(fn: str, code: int) -> None:
    if code != 0:
        raise DDTreeError(fn, code)


# ----------------------------------------------------------------- workspaces
def ddtree_build_workspace_size(batch: int, L: int, V: int, K: int, N: int) -> int:
    return int(lib().ddtree_build_workspace_size(batch, L, V, K, N))


def ddtree_verify_workspace_size(dtype: int, batch: int, T: int, Hq: int, Hkv: int, D: int,
                                 max_prefix_len: int) -> int:
    return int(lib().ddtree_verify_workspace_size(dtype, batch, T, Hq, Hkv, D, max_prefix_len))


def ddtree_accept_workspace_size(batch: int, T: int) -> int:
    return int(lib().ddtree_accept_workspace_size(batch, T))


def new_workspace(nbytes: int, device) -> torch.Tensor:
    """A device byte buffer for a workspace argument (zero-filled for tidiness)."""
    return torch.zeros(max(int(nbytes), 256), dtype=torch.uint8, device=device)


# ----------------------------------------------------------------- the calls
def ddtree_build(logits: torch.Tensor, root_tokens: torch.Tensor, K: int, N: int,
                 draft_temp: float, tokens: torch.Tensor, parents: torch.Tensor,
                 depths: torch.Tensor, scores: torch.Tensor, num_nodes: torch.Tensor,
                 mask: Optional[torch.Tensor], topk_tokens: Optional[torch.Tensor],
                 topk_logprobs: Optional[torch.Tensor], status_flags: Optional[torch.Tensor],
                 workspace: torch.Tensor, stream=None) -> None:
    batch, L, V = logits.shape
    code = lib().ddtree_build(
        _ptr(logits), _dtype_code(logits), _ptr(root_tokens), batch, L, V, K, N,
        float(draft_temp), _ptr(tokens), _ptr(parents), _ptr(depths), _ptr(scores),
        _ptr(num_nodes), _ptr(mask), _ptr(topk_tokens), _ptr(topk_logprobs), _ptr(status_flags),
        _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(stream, logits.device))
    _check("ddtree_build", code)


def ddtree_build_noalloc(logits: torch.Tensor, root_tokens: torch.Tensor, K: int, N: int,
                         draft_temp: float, tokens: torch.Tensor, parents: torch.Tensor,
                         depths: torch.Tensor, scores: torch.Tensor, num_nodes: torch.Tensor,
                         mask: Optional[torch.Tensor], topk_tokens: Optional[torch.Tensor],
                         topk_logprobs: Optional[torch.Tensor],
                         status_flags: Optional[torch.Tensor], stream=None) -> None:
    """ddtree_build with the library's static scratch instead of a workspace."""
    batch, L, V = logits.shape
    code = lib().ddtree_build_noalloc(
        _ptr(logits), _dtype_code(logits), _ptr(root_tokens), batch, L, V, K, N,
        float(draft_temp), _ptr(tokens), _ptr(parents), _ptr(depths), _ptr(scores),
        _ptr(num_nodes), _ptr(mask), _ptr(topk_tokens), _ptr(topk_logprobs), _ptr(status_flags),
        _stream(stream, logits.device))
    _check("ddtree_build_noalloc", code)


def ddtree_mask(parents: torch.Tensor, num_nodes: torch.Tensor, mask: torch.Tensor,
                stream=None) -> None:
    batch, T = parents.shape
    code = lib().ddtree_mask(_ptr(parents), _ptr(num_nodes), batch, T, _ptr(mask),
                             _stream(stream, parents.device))
    _check("ddtree_mask", code)


def ddtree_verify_attn(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                       kv_offsets: torch.Tensor, prefix_lens: torch.Tensor,
                       num_nodes: torch.Tensor, mask: torch.Tensor, max_prefix_len: int,
                       out: torch.Tensor, workspace: torch.Tensor, softmax_scale: float = 0.0,
                       stream=None, status_flags: Optional[torch.Tensor] = None) -> None:
    batch, T, Hq, D = q.shape
    Hkv = k.shape[1]
    code = lib().ddtree_verify_attn(
        _ptr(q), _ptr(k), _ptr(v), _dtype_code(q), _ptr(kv_offsets), _ptr(prefix_lens),
        _ptr(num_nodes), _ptr(mask), batch, T, Hq, Hkv, D, int(max_prefix_len), k.shape[0],
        float(softmax_scale), _ptr(out), _ptr(status_flags), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream, q.device))
    _check("ddtree_verify_attn", code)


def ddtree_accept(target_logits: Optional[torch.Tensor], target_ids: Optional[torch.Tensor],
                  tokens: torch.Tensor, parents: torch.Tensor, num_nodes: torch.Tensor, L: int,
                  accepted: torch.Tensor, accepted_nodes: Optional[torch.Tensor],
                  accept_len: torch.Tensor, bonus: torch.Tensor,
                  target_argmax: Optional[torch.Tensor], workspace: torch.Tensor,
                  stream=None) -> None:
    batch, T = tokens.shape
    if target_logits is not None:
        V, dt = target_logits.shape[-1], _dtype_code(target_logits)
    else:
        V, dt = 0, F32
    code = lib().ddtree_accept(
        _ptr(target_logits), dt, _ptr(target_ids), _ptr(tokens), _ptr(parents), _ptr(num_nodes),
        batch, T, V, L, _ptr(accepted), _ptr(accepted_nodes), _ptr(accept_len), _ptr(bonus),
        _ptr(target_argmax), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(stream, tokens.device))
    _check("ddtree_accept", code)


def ddtree_accept_sample(target_logits: torch.Tensor, tokens: torch.Tensor,
                         parents: torch.Tensor, num_nodes: torch.Tensor, L: int,
                         temperature: float, seed: int, offset: int, accepted: torch.Tensor,
                         accepted_nodes: Optional[torch.Tensor], accept_len: torch.Tensor,
                         bonus: torch.Tensor, target_tokens: Optional[torch.Tensor],
                         workspace: Optional[torch.Tensor], stream=None) -> None:
    batch, T = tokens.shape
    V = target_logits.shape[-1]
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    code = lib().ddtree_accept_sample(
        _ptr(target_logits), _dtype_code(target_logits), _ptr(tokens), _ptr(parents),
        _ptr(num_nodes), batch, T, V, L, float(temperature), int(seed) & (2**64 - 1),
        int(offset) & (2**64 - 1), _ptr(accepted), _ptr(accepted_nodes), _ptr(accept_len),
        _ptr(bonus), _ptr(target_tokens), _ptr(workspace), nbytes,
        _stream(stream, tokens.device))
    _check("ddtree_accept_sample", code)


def ddtree_commit_kv(k_cache: torch.Tensor, v_cache: torch.Tensor, kv_offsets: torch.Tensor,
                     prefix_lens: torch.Tensor, accept_len: torch.Tensor,
                     accepted_nodes: torch.Tensor, bonus: torch.Tensor, T: int,
                     new_prefix_lens: torch.Tensor, next_roots: Optional[torch.Tensor],
                     stream=None) -> None:
    rows, Hkv, D = k_cache.shape
    batch, L = accepted_nodes.shape
    code = lib().ddtree_commit_kv(
        _ptr(k_cache), _ptr(v_cache), _dtype_code(k_cache), _ptr(kv_offsets), _ptr(prefix_lens),
        _ptr(accept_len), _ptr(accepted_nodes), _ptr(bonus), batch, Hkv, D, L, int(T), rows,
        _ptr(new_prefix_lens), _ptr(next_roots), _stream(stream, k_cache.device))
    _check("ddtree_commit_kv", code)


# ----------------------------------------------------------------- convenience
class Round:
    """Preallocated outputs and workspaces for one round of a fixed shape.

    ``build``, ``verify`` and ``accept`` enqueue the three ABI calls on the
    current stream; nothing is allocated after construction.
    """

    def __init__(self, batch: int, L: int, V: int, K: int, N: int, device,
                 Hq: int = 0, Hkv: int = 0, D: int = 0, max_prefix_len: int = 0,
                 dtype=torch.bfloat16):
        dev = torch.device(device)
        T = N + 1
        W = (T + 63) // 64
        i32 = dict(dtype=torch.int32, device=dev)
        self.batch, self.L, self.V, self.K, self.N, self.T = batch, L, V, K, N, T
        self.tokens = torch.empty(batch, T, **i32)
        self.parents = torch.empty(batch, T, **i32)
        self.depths = torch.empty(batch, T, **i32)
        self.scores = torch.empty(batch, T, dtype=torch.float32, device=dev)
        self.num_nodes = torch.empty(batch, **i32)
        self.mask = torch.empty(batch, T, W, dtype=torch.int64, device=dev)
        self.topk_tokens = torch.empty(batch, L, K, **i32)
        self.topk_logprobs = torch.empty(batch, L, K, dtype=torch.float32, device=dev)
        self.status = torch.empty(batch, **i32)
        self.ws_build = new_workspace(ddtree_build_workspace_size(batch, L, V, K, N), dev)
        self.accepted = torch.empty(batch, L, **i32)
        self.accepted_nodes = torch.empty(batch, L, **i32)
        self.accept_len = torch.empty(batch, **i32)
        self.bonus = torch.empty(batch, **i32)
        self.target_argmax = torch.empty(batch, T, **i32)
        self.ws_accept = new_workspace(ddtree_accept_workspace_size(batch, T), dev)
        self.max_prefix_len = max_prefix_len
        if Hq:
            self.out = torch.empty(batch, T, Hq, D, dtype=dtype, device=dev)
            code = BF16 if dtype == torch.bfloat16 else F32
            self.ws_verify = new_workspace(
                ddtree_verify_workspace_size(code, batch, T, Hq, Hkv, D, max_prefix_len), dev)

    def build(self, logits, root_tokens, draft_temp: float = 1.0, stream=None):
        ddtree_build(logits, root_tokens, self.K, self.N, draft_temp, self.tokens, self.parents,
                     self.depths, self.scores, self.num_nodes, self.mask, self.topk_tokens,
                     self.topk_logprobs, self.status, self.ws_build, stream)

    def verify(self, q, k, v, kv_offsets, prefix_lens, stream=None, status_flags=None):
        ddtree_verify_attn(q, k, v, kv_offsets, prefix_lens, self.num_nodes, self.mask,
                           self.max_prefix_len, self.out, self.ws_verify, 0.0, stream,
                           status_flags)

    def accept(self, target_logits, stream=None):
        ddtree_accept(target_logits, None, self.tokens, self.parents, self.num_nodes, self.L,
                      self.accepted, self.accepted_nodes, self.accept_len, self.bonus,
                      self.target_argmax, self.ws_accept, stream)

    def commit(self, k_cache, v_cache, kv_offsets, prefix_lens, stream=None):
        """KV compaction of the last accepted paths; new prefix lengths and
        next roots go to ``new_prefix_lens`` and ``next_roots``."""
        if not hasattr(self, "new_prefix_lens"):
            raise RuntimeError("Round.commit needs buffers: call Round.prepare_commit() first")
        ddtree_commit_kv(k_cache, v_cache, kv_offsets, prefix_lens, self.accept_len,
                         self.accepted_nodes, self.bonus, self.T, self.new_prefix_lens,
                         self.next_roots, stream)

    def prepare_commit(self):
        dev = self.tokens.device
        self.new_prefix_lens = torch.empty(self.batch, dtype=torch.int32, device=dev)
        self.next_roots = torch.empty(self.batch, dtype=torch.int32, device=dev)

    def accept_sample(self, target_logits, temperature: float, seed: int, offset: int,
                      stream=None):
        """Acceptance at target temperature > 0; the sampled token per node
        goes to ``target_argmax`` (the per-node target token buffer)."""
        ddtree_accept_sample(target_logits, self.tokens, self.parents, self.num_nodes, self.L,
                             temperature, seed, offset, self.accepted, self.accepted_nodes,
                             self.accept_len, self.bonus, self.target_argmax, None, stream)


# ---------------------------------------------------------------- calibration
def ddtree_probe_mfma_bf16(out: torch.Tensor, grid: int, iters: int, stream=None) -> None:
    """Dense bf16 MFMA loop (measurement only): grid * 4 * 4 * iters * 32768 flops."""
    _check("ddtree_probe_mfma_bf16", lib().ddtree_probe_mfma_bf16(
        _ptr(out), int(grid), int(iters), _stream(stream, out.device)))


def ddtree_probe_hbm_read(src: torch.Tensor, out: torch.Tensor, grid: int, stream=None) -> None:
    """One streaming read of src (measurement only)."""
    _check("ddtree_probe_hbm_read", lib().ddtree_probe_hbm_read(
        _ptr(src), src.numel() * src.element_size(), _ptr(out), int(grid),
        _stream(stream, src.device)))
