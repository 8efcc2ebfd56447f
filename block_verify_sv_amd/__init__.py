"""Python binding of libspecverify (block verification for speculative decoding, MI355X).

Argument marshalling only: every step of the computation runs in the HIP kernels of
``libspecverify.so``.  PyTorch supplies device memory and the current stream.  There is
no CPU fallback: if the library is not built, every call raises.

    import block_verify_sv_amd as sv
    out, lse = sv.verify_attention(q, k_cache, v_cache, page_table, ctx_lens, max_ctx=...)
    acc, toks, am = sv.accept_greedy(logits, drafts)
    acc, toks = sv.accept_sample(target_logits, draft_logits, drafts, 1.0, seed, offset)
    fhat = sv.latent_compress(queries, feats)

Layouts and semantics are those of ``include/specverify.h``.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

__all__ = [
    "LIB_PATH", "load", "SvError", "AttnDesc", "verify_attention", "verify_attention_into",
    "verify_attention_noalloc_into",
    "attention_workspace_bytes", "mask_array", "accept_greedy", "accept_greedy_tree",
    "accept_sample", "accept_sample_tree", "lm_head_greedy", "lm_head_pack",
    "lm_head_greedy_packed", "latent_compress", "kv_append", "commit", "commit_tree",
    "make_desc", "set_wait_limit", "SV_F32", "SV_BF16", "SV_F16",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libspecverify.so")

SV_F32, SV_BF16, SV_F16 = 0, 1, 2
_DTYPES = {torch.float32: SV_F32, torch.bfloat16: SV_BF16, torch.float16: SV_F16}

c_i32, c_i64, c_u64, c_f32, c_vp, c_sz = (ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64,
                                          ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t)


class SvError(RuntimeError):
    """A libspecverify call returned a nonzero status."""


class AttnDesc(ctypes.Structure):
    """Mirror of ``sv_attn_desc``."""
    _fields_ = [("batch", c_i32), ("block", c_i32), ("num_q_heads", c_i32),
                ("num_kv_heads", c_i32), ("head_dim", c_i32), ("page_size", c_i32),
                ("max_pages_per_seq", c_i32), ("num_pages", c_i32), ("max_ctx", c_i32),
                ("split_keys", c_i32), ("scale", c_f32), ("dtype", c_i32),
                ("sum_ctx_hint", c_i64)]


_LIB = None

_SIGNATURES = {
    "sv_version": (c_i32, []),
    "sv_status_string": (ctypes.c_char_p, [c_i32]),
    "sv_last_error": (ctypes.c_char_p, []),
    "sv_set_wait_limit": (c_i32, [c_i32]),
    "sv_verify_attention_workspace": (c_i32, [ctypes.POINTER(AttnDesc), ctypes.POINTER(c_sz)]),
    "sv_verify_attention": (c_i32, [ctypes.POINTER(AttnDesc), c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                                    c_vp, c_vp, c_vp, c_sz, c_vp]),
    "sv_verify_attention_noalloc": (c_i32, [ctypes.POINTER(AttnDesc), c_vp, c_vp, c_vp, c_vp,
                                            c_vp, c_vp, c_vp, c_vp, c_vp]),
    "sv_accept_greedy_workspace": (c_i32, [c_i32, c_i32, c_i32, ctypes.POINTER(c_sz)]),
    "sv_accept_greedy": (c_i32, [c_i32, c_i32, c_i32, c_i32, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                                 c_sz, c_vp]),
    "sv_accept_sample_workspace": (c_i32, [c_i32, c_i32, c_i32, ctypes.POINTER(c_sz)]),
    "sv_accept_sample": (c_i32, [c_i32, c_i32, c_i32, c_i32, c_vp, c_vp, c_vp, c_f32, c_u64,
                                 c_u64, c_vp, c_vp, c_vp, c_sz, c_vp]),
    "sv_latent_compress_workspace": (c_i32, [c_i32, c_i32, c_i32, c_i32, ctypes.POINTER(c_sz)]),
    "sv_latent_compress": (c_i32, [c_i32, c_i32, c_i32, c_i32, c_i32, c_vp, c_vp, c_vp, c_f32,
                                   c_vp, c_sz, c_vp]),
    "sv_kv_append": (c_i32, [ctypes.POINTER(AttnDesc), c_i32, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                             c_vp]),
    "sv_commit": (c_i32, [c_i32, c_i32, c_vp, c_vp, c_vp, c_vp, c_vp]),
    "sv_accept_greedy_tree": (c_i32, [c_i32, c_i32, c_i32, c_i32, c_vp, c_vp, c_vp, c_vp, c_vp,
                                      c_vp, c_vp, c_vp, c_sz, c_vp]),
    "sv_accept_sample_tree_workspace": (c_i32, [c_i32, c_i32, c_i32, ctypes.POINTER(c_sz)]),
    "sv_accept_sample_tree": (c_i32, [c_i32, c_i32, c_i32, c_i32, c_vp, c_vp, c_vp, c_vp, c_f32,
                                      c_u64, c_u64, c_vp, c_vp, c_vp, c_vp, c_sz, c_vp]),
    "sv_commit_tree": (c_i32, [ctypes.POINTER(AttnDesc), c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                               c_vp, c_vp, c_vp]),
    "sv_lm_head_greedy_workspace": (c_i32, [c_i32, c_i32, c_i32, c_i32, ctypes.POINTER(c_sz)]),
    "sv_lm_head_greedy": (c_i32, [c_i32, c_i32, c_i32, c_i32, c_i32, c_vp, c_vp, c_vp, c_vp,
                                  c_vp, c_vp, c_vp, c_sz, c_vp]),
    "sv_lm_head_pack_bytes": (c_i32, [c_i32, c_i32, ctypes.POINTER(c_sz)]),
    "sv_lm_head_pack": (c_i32, [c_i32, c_i32, c_i32, c_vp, c_vp, c_vp]),
    "sv_lm_head_greedy_packed": (c_i32, [c_i32, c_i32, c_i32, c_i32, c_i32, c_vp, c_vp, c_vp,
                                         c_vp, c_vp, c_vp, c_vp, c_sz, c_vp]),
}


def load():
    """Load libspecverify.so (built in-tree); raises if it is missing."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise SvError(f"{LIB_PATH} is not built: run `python -m block_verify_sv_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = lib
    return _LIB


def _check(status: int, what: str):
    if status != 0:
        lib = load()
        msg = lib.sv_last_error().decode()
        raise SvError(f"{what}: {lib.sv_status_string(status).decode()} ({status}): {msg}")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _on_stream(stream, *tensors):
    """Tell the caching allocator that tensors made on the current stream are used by
    a launch on another stream, so their memory is not reused before that stream gets
    past the launch."""
    if stream is None:
        return
    if stream.cuda_stream == torch.cuda.current_stream(stream.device).cuda_stream:
        return
    for t in tensors:
        if t is not None:
            t.record_stream(stream)


def _require(t: torch.Tensor, name: str, dtype=None):
    if not t.is_cuda:
        raise SvError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise SvError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise SvError(f"{name} must be {dtype} (got {t.dtype})")


# ----------------------------------------------------------------------- workspace cache
_WS: dict = {}


def _workspace(kind: str, nbytes: int, device, zero: bool, stream=None) -> torch.Tensor:
    """A per-(kind, device, stream) workspace grown on demand (the library needs no
    initial contents; ``zero`` only picks a zero-filled first allocation).  Calls on
    different streams get different buffers, since two calls sharing one must not
    overlap in time; a buffer replaced by a larger one is released only after the work
    its stream has queued (record_stream)."""
    s = stream if stream is not None else torch.cuda.current_stream(device)
    key = (kind, str(device), s.cuda_stream)
    ws = _WS.get(key)
    if ws is None or ws.numel() < nbytes:
        n = max(nbytes, 256)
        with torch.cuda.stream(s):
            ws = (torch.zeros if zero else torch.empty)(n, dtype=torch.uint8, device=device)
        _WS[key] = ws
    return ws


# ----------------------------------------------------------------------- attention
def make_desc(q: torch.Tensor, k_cache: torch.Tensor, page_table: torch.Tensor, max_ctx: int,
              scale: float = 0.0, split_keys: int = 0, sum_ctx_hint: int = 0) -> AttnDesc:
    B, K, Hq, D = q.shape
    num_pages, Hkv, P, Dk = k_cache.shape
    if Dk != D:
        raise SvError("q and k_cache head_dim differ")
    if q.dtype not in _DTYPES:
        raise SvError(f"unsupported dtype {q.dtype}")
    return AttnDesc(B, K, Hq, Hkv, D, P, page_table.shape[1], num_pages, int(max_ctx),
                    int(split_keys), float(scale), _DTYPES[q.dtype], int(sum_ctx_hint))


def attention_workspace_bytes(desc: AttnDesc) -> int:
    n = c_sz()
    _check(load().sv_verify_attention_workspace(ctypes.byref(desc), ctypes.byref(n)),
           "sv_verify_attention_workspace")
    return n.value


def verify_attention_into(desc: AttnDesc, q, k_cache, v_cache, page_table, ctx_lens, out,
                          lse=None, block_mask=None, workspace=None, stream=None):
    """Launch into preallocated outputs.  ``block_mask`` is a host ctypes uint64 array
    (or None for causal); ``workspace`` a device uint8 tensor (or None: cached)."""
    nbytes = attention_workspace_bytes(desc)
    if workspace is None:
        workspace = _workspace("attn", nbytes, q.device, zero=False, stream=stream)
    _on_stream(stream, out, lse)
    _check(load().sv_verify_attention(ctypes.byref(desc), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                      _ptr(page_table), _ptr(ctx_lens), block_mask, _ptr(out),
                                      _ptr(lse), _ptr(workspace), workspace.numel(),
                                      _stream(stream)),
           "sv_verify_attention")


def verify_attention_noalloc_into(desc: AttnDesc, q, k_cache, v_cache, page_table, ctx_lens,
                                  out, lse=None, block_mask=None, stream=None):
    """The allocation-free call: as verify_attention_into, with the library's own
    per-GPU scratch array in place of a workspace (calls overlapping on one GPU race)."""
    _on_stream(stream, out, lse)
    _check(load().sv_verify_attention_noalloc(ctypes.byref(desc), _ptr(q), _ptr(k_cache),
                                              _ptr(v_cache), _ptr(page_table), _ptr(ctx_lens),
                                              block_mask, _ptr(out), _ptr(lse), _stream(stream)),
           "sv_verify_attention_noalloc")


def mask_array(mask):
    """Host uint64 row masks as a ctypes array (None stays None = causal)."""
    if mask is None:
        return None
    vals = [int(m) for m in mask]
    return (c_u64 * len(vals))(*vals)


def verify_attention(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                     page_table: torch.Tensor, ctx_lens: torch.Tensor, max_ctx: int,
                     block_mask=None, scale: float = 0.0, want_lse: bool = True,
                     split_keys: int = 0, sum_ctx_hint: int = 0, stream=None):
    """Block-causal GQA of the K block rows over the paged cache.  Returns (out, lse)."""
    for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache)):
        _require(t, name, q.dtype)
    _require(page_table, "page_table", torch.int32)
    _require(ctx_lens, "ctx_lens", torch.int32)
    desc = make_desc(q, k_cache, page_table, max_ctx, scale, split_keys, sum_ctx_hint)
    if tuple(v_cache.shape) != (desc.num_pages, desc.num_kv_heads, desc.head_dim, desc.page_size):
        raise SvError(f"v_cache must be [num_pages][Hkv][d][P], got {tuple(v_cache.shape)}")
    if tuple(page_table.shape)[0] != desc.batch or tuple(ctx_lens.shape) != (desc.batch,):
        raise SvError("page_table / ctx_lens batch mismatch")
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device) if want_lse else None
    verify_attention_into(desc, q, k_cache, v_cache, page_table, ctx_lens, out, lse,
                          mask_array(block_mask), None, stream)
    return out, lse


# ----------------------------------------------------------------------- acceptance
def accept_greedy(logits: torch.Tensor, drafts: torch.Tensor, want_argmax: bool = True,
                  out=None, workspace=None, stream=None):
    """Greedy acceptance.  Returns (accept_len [B], out_tokens [B][K], argmax [B][K] or None)."""
    _require(logits, "logits")
    _require(drafts, "drafts", torch.int32)
    B, K, V = logits.shape
    if logits.dtype not in (torch.float32, torch.bfloat16):
        raise SvError("greedy logits must be float32 or bfloat16")
    if tuple(drafts.shape) != (B, K - 1):
        raise SvError(f"drafts must be [B][K-1] = {(B, K - 1)}, got {tuple(drafts.shape)}")
    lib = load()
    n = c_sz()
    _check(lib.sv_accept_greedy_workspace(B, K, V, ctypes.byref(n)), "sv_accept_greedy_workspace")
    if workspace is None:
        workspace = _workspace("greedy", n.value, logits.device, zero=True, stream=stream)
    if out is None:
        acc = torch.empty(B, dtype=torch.int32, device=logits.device)
        toks = torch.empty(B, K, dtype=torch.int32, device=logits.device)
        am = torch.empty(B, K, dtype=torch.int32, device=logits.device) if want_argmax else None
        _on_stream(stream, acc, toks, am)
    else:
        acc, toks, am = out
    _check(lib.sv_accept_greedy(B, K, V, _DTYPES[logits.dtype], _ptr(logits), _ptr(drafts),
                                _ptr(acc), _ptr(toks), _ptr(am), _ptr(workspace),
                                workspace.numel(), _stream(stream)),
           "sv_accept_greedy")
    return acc, toks, am


def accept_greedy_tree(logits: torch.Tensor, parents: torch.Tensor, tokens: torch.Tensor,
                       want_argmax: bool = True, out=None, workspace=None, stream=None):
    """Greedy acceptance over a draft tree (node 0 = anchor; parents/tokens [B][K-1] of
    nodes 1..K-1).  Returns (accept_len [B], out_tokens [B][K], accept_path [B][K],
    argmax [B][K] or None)."""
    _require(logits, "logits")
    _require(parents, "parents", torch.int32)
    _require(tokens, "tokens", torch.int32)
    B, K, V = logits.shape
    if logits.dtype not in (torch.float32, torch.bfloat16):
        raise SvError("greedy logits must be float32 or bfloat16")
    if tuple(parents.shape) != (B, K - 1) or tuple(tokens.shape) != (B, K - 1):
        raise SvError(f"parents and tokens must be [B][K-1] = {(B, K - 1)}")
    lib = load()
    n = c_sz()
    _check(lib.sv_accept_greedy_workspace(B, K, V, ctypes.byref(n)), "sv_accept_greedy_workspace")
    if workspace is None:
        workspace = _workspace("greedy", n.value, logits.device, zero=True, stream=stream)
    if out is None:
        acc = torch.empty(B, dtype=torch.int32, device=logits.device)
        toks = torch.empty(B, K, dtype=torch.int32, device=logits.device)
        path = torch.empty(B, K, dtype=torch.int32, device=logits.device)
        am = torch.empty(B, K, dtype=torch.int32, device=logits.device) if want_argmax else None
        _on_stream(stream, acc, toks, path, am)
    else:
        acc, toks, path, am = out
    _check(lib.sv_accept_greedy_tree(B, K, V, _DTYPES[logits.dtype], _ptr(logits),
                                     _ptr(parents), _ptr(tokens), _ptr(acc), _ptr(toks),
                                     _ptr(path), _ptr(am), _ptr(workspace), workspace.numel(),
                                     _stream(stream)),
           "sv_accept_greedy_tree")
    return acc, toks, path, am


def lm_head_pack(weight: torch.Tensor, out=None, stream=None) -> torch.Tensor:
    """Rearranges the LM head weight [V][hidden] (bf16 or fp16) once into the packed tile
    layout that lm_head_greedy_packed reads: a flat tensor of ceil(V / 32) * 32 * hidden
    elements of the weight's dtype."""
    _require(weight, "weight")
    if weight.dim() != 2 or weight.dtype not in (torch.bfloat16, torch.float16):
        raise SvError("weight must be a [V][hidden] bfloat16 or float16 tensor")
    V, Hd = weight.shape
    lib = load()
    n = c_sz()
    _check(lib.sv_lm_head_pack_bytes(V, Hd, ctypes.byref(n)), "sv_lm_head_pack_bytes")
    elems = n.value // weight.element_size()
    if out is None:
        out = torch.empty(elems, dtype=weight.dtype, device=weight.device)
        _on_stream(stream, out)
    elif out.dtype != weight.dtype or out.numel() != elems or not out.is_contiguous():
        raise SvError(f"out must be a contiguous {weight.dtype} tensor of {elems} elements")
    _check(lib.sv_lm_head_pack(V, Hd, _DTYPES[weight.dtype], _ptr(weight), _ptr(out),
                               _stream(stream)), "sv_lm_head_pack")
    return out


def lm_head_greedy_packed(hidden_states: torch.Tensor, packed: torch.Tensor, V: int,
                          drafts: torch.Tensor, want_argmax: bool = True, out=None,
                          workspace=None, stream=None):
    """lm_head_greedy over a weight packed by lm_head_pack (V = the weight's row count)."""
    _require(packed, "packed", hidden_states.dtype)
    Hd = hidden_states.shape[-1]
    n = c_sz()
    _check(load().sv_lm_head_pack_bytes(V, Hd, ctypes.byref(n)), "sv_lm_head_pack_bytes")
    if packed.numel() * packed.element_size() != n.value:
        raise SvError(f"packed must hold {n.value} bytes for V={V}, hidden={Hd}")
    return _lm_head(hidden_states, packed, V, drafts, want_argmax, out, workspace, stream, True)


def lm_head_greedy(hidden_states: torch.Tensor, weight: torch.Tensor, drafts: torch.Tensor,
                   want_argmax: bool = True, out=None, workspace=None, stream=None):
    """LM head + greedy acceptance: hidden_states [B][K][hidden], weight [V][hidden] (bf16
    or fp16).  Returns (accept_len [B], out_tokens [B][K], argmax [B][K] or None)."""
    _require(weight, "weight", hidden_states.dtype)
    if weight.dim() != 2 or weight.shape[1] != hidden_states.shape[-1]:
        raise SvError("weight must be [V][hidden]")
    return _lm_head(hidden_states, weight, weight.shape[0], drafts, want_argmax, out, workspace,
                    stream, False)


def _lm_head(hidden_states, weight, V, drafts, want_argmax, out, workspace, stream, packed):
    _require(hidden_states, "hidden_states")
    _require(drafts, "drafts", torch.int32)
    B, K, Hd = hidden_states.shape
    if hidden_states.dtype not in (torch.bfloat16, torch.float16):
        raise SvError("LM head operands must be bfloat16 or float16")
    if tuple(drafts.shape) != (B, K - 1):
        raise SvError("drafts must be [B][K-1]")
    lib = load()
    n = c_sz()
    _check(lib.sv_lm_head_greedy_workspace(B, K, V, Hd, ctypes.byref(n)),
           "sv_lm_head_greedy_workspace")
    if workspace is None:
        workspace = _workspace("lm_head", n.value, weight.device, zero=False, stream=stream)
    if out is None:
        acc = torch.empty(B, dtype=torch.int32, device=weight.device)
        toks = torch.empty(B, K, dtype=torch.int32, device=weight.device)
        am = torch.empty(B, K, dtype=torch.int32, device=weight.device) if want_argmax else None
        _on_stream(stream, acc, toks, am)
    else:
        acc, toks, am = out
    fn, name = ((lib.sv_lm_head_greedy_packed, "sv_lm_head_greedy_packed") if packed
                else (lib.sv_lm_head_greedy, "sv_lm_head_greedy"))
    _check(fn(B, K, V, Hd, _DTYPES[hidden_states.dtype], _ptr(hidden_states), _ptr(weight),
              _ptr(drafts), _ptr(acc), _ptr(toks), _ptr(am), _ptr(workspace), workspace.numel(),
              _stream(stream)), name)
    return acc, toks, am


def accept_sample(target_logits: torch.Tensor, draft_logits: torch.Tensor, drafts: torch.Tensor,
                  temperature: float, seed: int, offset: int, out=None, workspace=None,
                  stream=None):
    """Sampling acceptance.  Returns (accept_len [B], out_tokens [B][K])."""
    _require(target_logits, "target_logits")
    _require(draft_logits, "draft_logits", target_logits.dtype)
    _require(drafts, "drafts", torch.int32)
    B, K, V = target_logits.shape
    if target_logits.dtype not in (torch.float32, torch.bfloat16):
        raise SvError("sampling logits must be float32 or bfloat16")
    if tuple(draft_logits.shape) != (B, K - 1, V) or tuple(drafts.shape) != (B, K - 1):
        raise SvError("draft_logits must be [B][K-1][V] and drafts [B][K-1]")
    lib = load()
    n = c_sz()
    _check(lib.sv_accept_sample_workspace(B, K, V, ctypes.byref(n)), "sv_accept_sample_workspace")
    if workspace is None:
        workspace = _workspace("sample", n.value, target_logits.device, zero=False,
                               stream=stream)
    if out is None:
        acc = torch.empty(B, dtype=torch.int32, device=target_logits.device)
        toks = torch.empty(B, K, dtype=torch.int32, device=target_logits.device)
        _on_stream(stream, acc, toks)
    else:
        acc, toks = out
    _check(lib.sv_accept_sample(B, K, V, _DTYPES[target_logits.dtype], _ptr(target_logits),
                                _ptr(draft_logits), _ptr(drafts), float(temperature),
                                int(seed) & (2**64 - 1), int(offset) & (2**64 - 1), _ptr(acc),
                                _ptr(toks), _ptr(workspace), workspace.numel(), _stream(stream)),
           "sv_accept_sample")
    return acc, toks


def accept_sample_tree(target_logits: torch.Tensor, draft_logits: torch.Tensor, parents,
                       tokens: torch.Tensor, temperature: float, seed: int, offset: int,
                       out=None, workspace=None, stream=None):
    """Sampling acceptance over a draft tree shared by the batch.  parents: host sequence of
    K-1 ints (parent of node i at [i-1]); tokens [B][K-1] device int32.  Returns
    (accept_len [B], out_tokens [B][K], accept_path [B][K])."""
    _require(target_logits, "target_logits")
    _require(draft_logits, "draft_logits", target_logits.dtype)
    _require(tokens, "tokens", torch.int32)
    B, K, V = target_logits.shape
    if target_logits.dtype not in (torch.float32, torch.bfloat16):
        raise SvError("sampling logits must be float32 or bfloat16")
    if tuple(draft_logits.shape) != (B, K - 1, V) or tuple(tokens.shape) != (B, K - 1):
        raise SvError("draft_logits must be [B][K-1][V] and tokens [B][K-1]")
    par = [int(x) for x in parents]
    if len(par) != K - 1:
        raise SvError(f"parents must hold K-1 = {K - 1} entries")
    par_c = (c_i32 * max(1, len(par)))(*par)
    lib = load()
    n = c_sz()
    _check(lib.sv_accept_sample_tree_workspace(B, K, V, ctypes.byref(n)),
           "sv_accept_sample_tree_workspace")
    if workspace is None:
        workspace = _workspace("sample_tree", n.value, target_logits.device, zero=False,
                               stream=stream)
    if out is None:
        dev = target_logits.device
        acc = torch.empty(B, dtype=torch.int32, device=dev)
        toks = torch.empty(B, K, dtype=torch.int32, device=dev)
        path = torch.empty(B, K, dtype=torch.int32, device=dev)
        _on_stream(stream, acc, toks, path)
    else:
        acc, toks, path = out
    _check(lib.sv_accept_sample_tree(B, K, V, _DTYPES[target_logits.dtype], _ptr(target_logits),
                                     _ptr(draft_logits), ctypes.cast(par_c, c_vp), _ptr(tokens),
                                     float(temperature), int(seed) & (2**64 - 1),
                                     int(offset) & (2**64 - 1), _ptr(acc), _ptr(toks), _ptr(path),
                                     _ptr(workspace), workspace.numel(), _stream(stream)),
           "sv_accept_sample_tree")
    return acc, toks, path


# ----------------------------------------------------------------------- compressor
def latent_compress(queries: torch.Tensor, feats: torch.Tensor, scale: float = 1.0, out=None,
                    workspace=None, stream=None):
    """softmax(scale * C . F^T) . F per image.  queries [C][D], feats [B][N][D] (fp16)."""
    _require(queries, "queries", torch.float16)
    _require(feats, "feats", torch.float16)
    C, D = queries.shape
    B, N, D2 = feats.shape
    if D2 != D:
        raise SvError("queries and feats dims differ")
    lib = load()
    n = c_sz()
    _check(lib.sv_latent_compress_workspace(B, C, N, D, ctypes.byref(n)),
           "sv_latent_compress_workspace")
    if workspace is None:
        workspace = _workspace("compress", n.value, feats.device, zero=False, stream=stream)
    if out is None:
        out = torch.empty(B, C, D, dtype=torch.float16, device=feats.device)
        _on_stream(stream, out)
    _check(lib.sv_latent_compress(B, C, N, D, SV_F16, _ptr(queries), _ptr(feats), _ptr(out),
                                  float(scale), _ptr(workspace), workspace.numel(),
                                  _stream(stream)),
           "sv_latent_compress")
    return out


# ----------------------------------------------------------------------- KV append
def kv_append(k_new: torch.Tensor, v_new: torch.Tensor, start: torch.Tensor,
              page_table: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
              stream=None):
    """Write rows [B][n][Hkv][d] into the paged caches at positions start[b] + t."""
    for name, t in (("k_new", k_new), ("v_new", v_new), ("k_cache", k_cache),
                    ("v_cache", v_cache)):
        _require(t, name, k_cache.dtype)
    _require(start, "start", torch.int32)
    _require(page_table, "page_table", torch.int32)
    B, n, Hkv, D = k_new.shape
    num_pages, Hkv2, P, D2 = k_cache.shape
    if (Hkv2, D2) != (Hkv, D) or tuple(v_new.shape) != tuple(k_new.shape):
        raise SvError("kv_append shape mismatch")
    desc = AttnDesc(B, 1, Hkv, Hkv, D, P, page_table.shape[1], num_pages, 0, 0, 0.0,
                    _DTYPES[k_cache.dtype], 0)
    _check(load().sv_kv_append(ctypes.byref(desc), n, _ptr(k_new), _ptr(v_new), _ptr(start),
                               _ptr(page_table), _ptr(k_cache), _ptr(v_cache), _stream(stream)),
           "sv_kv_append")


# ----------------------------------------------------------------------- cycle commit
def set_wait_limit(polls: int) -> None:
    """Polls a waiting workgroup of the sampling calls makes before it gives up and reports
    its sequence as failed (accept_len -1); process-wide, 2**18 by default."""
    _check(load().sv_set_wait_limit(int(polls)), "sv_set_wait_limit")


def commit(accept_len: torch.Tensor, out_tokens: torch.Tensor, ctx_lens: torch.Tensor,
           next_anchor: torch.Tensor = None, stream=None) -> torch.Tensor:
    """Close a cycle on the device: ctx_lens += accept_len + 1 (in place) and return the
    next anchors out_tokens[b][accept_len[b]]."""
    _require(accept_len, "accept_len", torch.int32)
    _require(out_tokens, "out_tokens", torch.int32)
    _require(ctx_lens, "ctx_lens", torch.int32)
    B, K = out_tokens.shape
    if accept_len.numel() != B or ctx_lens.numel() != B:
        raise SvError("commit shape mismatch")
    if next_anchor is None:
        next_anchor = torch.empty(B, dtype=torch.int32, device=out_tokens.device)
        _on_stream(stream, next_anchor)
    _require(next_anchor, "next_anchor", torch.int32)
    _check(load().sv_commit(B, K, _ptr(accept_len), _ptr(out_tokens), _ptr(ctx_lens),
                            _ptr(next_anchor), _stream(stream)),
           "sv_commit")
    return next_anchor


def commit_tree(accept_len: torch.Tensor, out_tokens: torch.Tensor, accept_path: torch.Tensor,
                page_table: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                ctx_lens: torch.Tensor, next_anchor: torch.Tensor = None,
                stream=None) -> torch.Tensor:
    """Close a tree cycle on the device: move the accepted path's K/V rows to
    ctx+1 .. ctx+a, then ctx_lens += accept_len + 1 (in place); returns the next anchors."""
    for name, t in (("accept_len", accept_len), ("out_tokens", out_tokens),
                    ("accept_path", accept_path), ("page_table", page_table),
                    ("ctx_lens", ctx_lens)):
        _require(t, name, torch.int32)
    _require(k_cache, "k_cache")
    _require(v_cache, "v_cache", k_cache.dtype)
    B, K = out_tokens.shape
    num_pages, Hkv, P, D = k_cache.shape
    if (accept_len.numel() != B or ctx_lens.numel() != B or tuple(accept_path.shape) != (B, K)
            or page_table.shape[0] != B or tuple(v_cache.shape) != (num_pages, Hkv, D, P)):
        raise SvError("commit_tree shape mismatch")
    if next_anchor is None:
        next_anchor = torch.empty(B, dtype=torch.int32, device=out_tokens.device)
        _on_stream(stream, next_anchor)
    _require(next_anchor, "next_anchor", torch.int32)
    desc = AttnDesc(B, K, Hkv, Hkv, D, P, page_table.shape[1], num_pages, 0, 0, 0.0,
                    _DTYPES[k_cache.dtype], 0)
    _check(load().sv_commit_tree(ctypes.byref(desc), _ptr(accept_len), _ptr(out_tokens),
                                 _ptr(accept_path), _ptr(page_table), _ptr(k_cache),
                                 _ptr(v_cache), _ptr(ctx_lens), _ptr(next_anchor),
                                 _stream(stream)),
           "sv_commit_tree")
    return next_anchor
