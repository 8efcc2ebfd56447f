"""C-ABI checks that need no GPU: the library loads, exports every symbol the header
declares, and rejects invalid calls on the host before launching anything.

Every call here fails validation, so nothing reaches the device even where one exists.
"""
import ctypes
import os
import re

import pytest

import block_verify_sv_amd as sv

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include",
                      "specverify.h")
OK, INVALID, UNSUPPORTED, WORKSPACE = 0, -1, -2, -3
FAKE = ctypes.c_void_p(0x1000)          # never dereferenced: validation fails first


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(sv.LIB_PATH):
        pytest.fail("libspecverify.so is not built (run python -m block_verify_sv_amd.build)")
    return sv.load()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:sv_status|int|const char\*)\s+(sv_\w+)\s*\(", text, re.M)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert len(names) == 24, names
    for n in names:
        assert hasattr(lib, n), f"missing export {n}"
    assert lib.sv_version() == 1


def test_descriptor_layout_matches_header():
    """ctypes mirror: 12 four-byte fields then one int64 -> 56 bytes, int64 at offset 48."""
    assert ctypes.sizeof(sv.AttnDesc) == 56
    assert sv.AttnDesc.sum_ctx_hint.offset == 48
    text = open(HEADER).read()
    body = re.search(r"typedef struct \{(.*?)\} sv_attn_desc;", text, re.S).group(1)
    fields = re.findall(r"^\s*(?:int32_t|int64_t|float|sv_dtype)\s+(\w+);", body, re.M)
    assert fields == [f[0] for f in sv.AttnDesc._fields_]


def _desc(**kw):
    base = dict(batch=1, block=16, num_q_heads=28, num_kv_heads=4, head_dim=128, page_size=16,
                max_pages_per_seq=1571, num_pages=1571, max_ctx=25119, split_keys=0, scale=0.0,
                dtype=sv.SV_BF16, sum_ctx_hint=25119)
    base.update(kw)
    return sv.AttnDesc(**base)


def _ws(lib, d):
    n = ctypes.c_size_t()
    st = lib.sv_verify_attention_workspace(ctypes.byref(d), ctypes.byref(n))
    return st, n.value


def test_attention_workspace_query(lib):
    st, n = _ws(lib, _desc())
    assert st == OK
    assert n > 0
    # 4 KV heads x 25 splits x (128 padded rows x 128 bf16 partial outputs + 112 rows x (m, l))
    st, n2 = _ws(lib, _desc(split_keys=1024))
    assert st == OK and n2 == 4 * 25 * (128 * 128 * 2 + 112 * 8)


@pytest.mark.parametrize("kw,code", [
    (dict(batch=0), INVALID), (dict(block=0), INVALID), (dict(block=65), INVALID),
    (dict(num_q_heads=30), INVALID), (dict(num_q_heads=28 * 20, block=16), INVALID),
    (dict(head_dim=96), UNSUPPORTED), (dict(dtype=7), UNSUPPORTED), (dict(page_size=24), INVALID),
    (dict(page_size=8), INVALID), (dict(max_ctx=-1), INVALID), (dict(max_pages_per_seq=10), INVALID),
    (dict(split_keys=40), INVALID), (dict(split_keys=16400), INVALID),
    (dict(split_keys=48, page_size=32, max_pages_per_seq=786), INVALID),
    (dict(split_keys=96, page_size=128, max_pages_per_seq=197), INVALID),
    (dict(scale=-1.0), INVALID), (dict(scale=float("nan")), INVALID),
    (dict(sum_ctx_hint=-5), INVALID), (dict(num_pages=0), INVALID),
])
def test_attention_rejects_bad_descriptors(lib, kw, code):
    st, _ = _ws(lib, _desc(**kw))
    assert st == code, lib.sv_last_error()
    assert lib.sv_last_error().decode() != ""
    st = lib.sv_verify_attention(ctypes.byref(_desc(**kw)), FAKE, FAKE, FAKE, FAKE, FAKE, None,
                                 FAKE, None, FAKE, 1 << 40, None)
    assert st == code


def test_attention_rejects_bad_masks_and_buffers(lib):
    d = _desc(block=4, num_q_heads=2, num_kv_heads=1, head_dim=64, max_ctx=512,
              max_pages_per_seq=33, num_pages=33)
    good = (ctypes.c_uint64 * 4)(1, 3, 7, 15)
    no_self = (ctypes.c_uint64 * 4)(1, 1, 7, 15)
    beyond = (ctypes.c_uint64 * 4)(1, 3, 7, 31)
    call = lambda q, mask, ws, nbytes: lib.sv_verify_attention(
        ctypes.byref(d), q, FAKE, FAKE, FAKE, FAKE, mask, FAKE, None, ws, nbytes, None)
    assert call(FAKE, no_self, FAKE, 1 << 40) == INVALID
    assert "own bit" in lib.sv_last_error().decode()
    assert call(FAKE, beyond, FAKE, 1 << 40) == INVALID
    assert call(None, good, FAKE, 1 << 40) == INVALID                 # missing q
    assert call(ctypes.c_void_p(0x1008), good, FAKE, 1 << 40) == INVALID   # misaligned q
    assert call(FAKE, good, None, 1 << 40) == WORKSPACE               # no workspace
    assert call(FAKE, good, FAKE, 16) == WORKSPACE                    # too small
    assert "workspace" in lib.sv_last_error().decode()


def test_greedy_validation(lib):
    n = ctypes.c_size_t()
    assert lib.sv_accept_greedy_workspace(1, 16, 152064, ctypes.byref(n)) == OK
    assert n.value == 16 * 32 * 8        # packed argmax keys of up to 32 chunks per row
    for B, K, V in [(0, 16, 10), (1, 0, 10), (1, 65, 10), (1, 16, 0), (5000, 16, 10)]:
        assert lib.sv_accept_greedy_workspace(B, K, V, ctypes.byref(n)) == INVALID
    args = lambda dt, ws: (1, 16, 1000, dt, FAKE, FAKE, FAKE, FAKE, None, ws, 1 << 20, None)
    assert lib.sv_accept_greedy(*args(sv.SV_F16, FAKE)) == UNSUPPORTED
    assert lib.sv_accept_greedy(*args(sv.SV_BF16, None)) == WORKSPACE
    assert lib.sv_accept_greedy(1, 16, 1000, sv.SV_BF16, None, FAKE, FAKE, FAKE, None, FAKE,
                                1 << 20, None) == INVALID


def test_sample_validation(lib):
    n = ctypes.c_size_t()
    assert lib.sv_accept_sample_workspace(1, 32, 152064, ctypes.byref(n)) == OK
    assert lib.sv_accept_sample_workspace(1, 1, 100, ctypes.byref(n)) == INVALID   # K >= 2
    call = lambda T, ws=FAKE, dt=sv.SV_BF16: lib.sv_accept_sample(
        1, 4, 100, dt, FAKE, FAKE, FAKE, T, 1, 0, FAKE, FAKE, ws, 1 << 30, None)
    assert call(0.0) == INVALID
    assert call(-1.0) == INVALID
    assert call(float("inf")) == INVALID
    assert call(1.0, dt=sv.SV_F16) == UNSUPPORTED
    assert call(1.0, ws=None) == WORKSPACE
    assert call(1.0, ws=ctypes.c_void_p(0x1008)) == INVALID         # misaligned workspace
    odd = ctypes.c_void_p(0x1008)                                   # 8- but not 16-byte aligned
    for tl, dl in ((odd, FAKE), (FAKE, odd)):
        assert lib.sv_accept_sample(1, 4, 100, sv.SV_BF16, tl, dl, FAKE, 1.0, 1, 0, FAKE, FAKE,
                                    FAKE, 1 << 30, None) == INVALID


def test_compress_validation(lib):
    n = ctypes.c_size_t()
    assert lib.sv_latent_compress_workspace(32, 64, 576, 4096, ctypes.byref(n)) == OK
    # two fp32 partial score sets, fp16 weights over 64 padded rows x N rounded up to 32, fp32 row sums
    assert n.value == 2 * 32 * 64 * 576 * 4 + 32 * 64 * 576 * 2 + 32 * 64 * 4
    for B, C, N, D in [(0, 64, 576, 4096), (32, 65, 576, 4096), (32, 64, 0, 4096),
                       (32, 64, 2000, 4096), (32, 64, 576, 100)]:
        assert lib.sv_latent_compress_workspace(B, C, N, D, ctypes.byref(n)) == INVALID
    call = lambda dt, ws: lib.sv_latent_compress(2, 4, 8, 128, dt, FAKE, FAKE, FAKE, 1.0, ws,
                                                 1 << 20, None)
    assert call(sv.SV_BF16, FAKE) == UNSUPPORTED
    assert call(sv.SV_F16, None) == WORKSPACE
    assert call(sv.SV_F16, ctypes.c_void_p(0x1008)) == INVALID      # misaligned workspace


def test_kv_append_validation(lib):
    d = _desc()
    assert lib.sv_kv_append(ctypes.byref(d), 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == INVALID
    assert lib.sv_kv_append(ctypes.byref(d), 16, None, FAKE, FAKE, FAKE, FAKE, FAKE, None) == INVALID
    d2 = _desc(head_dim=80)
    assert lib.sv_kv_append(ctypes.byref(d2), 16, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == UNSUPPORTED


def test_commit_validation(lib):
    assert lib.sv_commit(0, 16, FAKE, FAKE, FAKE, FAKE, None) == INVALID
    assert lib.sv_commit(4, 65, FAKE, FAKE, FAKE, FAKE, None) == INVALID
    assert lib.sv_commit(4, 16, FAKE, None, FAKE, FAKE, None) == INVALID
    assert lib.sv_commit(4, 16, FAKE, FAKE, FAKE, None, None) == INVALID


def test_row_limit(lib):
    """A KV head holds up to 512 query rows (4 groups of 128): Tree-60 at the 7B shape
    (61 nodes x 7 query heads = 427 rows) is accepted, 64 x 9 = 576 rows are not."""
    st, n = _ws(lib, _desc(block=61, max_pages_per_seq=1574, num_pages=1574))
    assert st == OK and n > 0
    st, _ = _ws(lib, _desc(block=64, num_q_heads=36))
    assert st == INVALID and "512" in lib.sv_last_error().decode()


def test_tree_validation(lib):
    call = lambda dt, par, path, ws: lib.sv_accept_greedy_tree(
        1, 61, 1000, dt, FAKE, par, FAKE, FAKE, FAKE, path, None, ws, 1 << 20, None)
    assert call(sv.SV_BF16, None, FAKE, FAKE) == INVALID          # no parents
    assert call(sv.SV_BF16, FAKE, None, FAKE) == INVALID          # no path output
    assert call(sv.SV_F16, FAKE, FAKE, FAKE) == UNSUPPORTED
    assert call(sv.SV_BF16, FAKE, FAKE, None) == WORKSPACE
    assert lib.sv_accept_greedy_tree(1, 65, 1000, sv.SV_BF16, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                      None, FAKE, 1 << 20, None) == INVALID
    d = _desc(block=61, max_pages_per_seq=1574, num_pages=1574)
    arrays = [FAKE] * 8
    assert lib.sv_commit_tree(None, *arrays, None) == INVALID
    assert lib.sv_commit_tree(ctypes.byref(_desc(block=65)), *arrays, None) == INVALID
    assert lib.sv_commit_tree(ctypes.byref(_desc(head_dim=96)), *arrays, None) == UNSUPPORTED
    for i in range(8):
        a = list(arrays)
        a[i] = None
        assert lib.sv_commit_tree(ctypes.byref(d), *a, None) == INVALID


def test_lm_head_validation(lib):
    n = ctypes.c_size_t()
    assert lib.sv_lm_head_greedy_workspace(1, 16, 152064, 3584, ctypes.byref(n)) == OK
    # one key per (row, argmax workgroup), sized for the largest grid: 2,048 workgroups
    # (eight per CU) over the 4,752 units of 32 rows
    assert n.value == 16 * 2048 * 8
    for B, K, V, Hd in [(5, 16, 10, 64), (1, 16, 10, 48), (1, 16, 10, 0), (1, 0, 10, 64),
                        (1, 16, 0, 64)]:
        assert lib.sv_lm_head_greedy_workspace(B, K, V, Hd, ctypes.byref(n)) == INVALID
    call = lambda dt, h, ws, nbytes: lib.sv_lm_head_greedy(
        1, 16, 1000, 64, dt, h, FAKE, FAKE, FAKE, FAKE, None, ws, nbytes, None)
    assert call(sv.SV_F32, FAKE, FAKE, 1 << 20) == UNSUPPORTED
    assert call(sv.SV_BF16, None, FAKE, 1 << 20) == INVALID
    assert call(sv.SV_BF16, ctypes.c_void_p(0x1008), FAKE, 1 << 20) == INVALID
    assert call(sv.SV_BF16, FAKE, FAKE, 8) == WORKSPACE


def test_lm_head_pack_validation(lib):
    """The packed size is ceil(V / 32) * 32 rows of hidden 2-byte elements; the pack and
    the packed LM head reject bad shapes, dtypes and alignments on the host."""
    n = ctypes.c_size_t()
    assert lib.sv_lm_head_pack_bytes(152064, 3584, ctypes.byref(n)) == OK
    assert n.value == 152064 * 3584 * 2
    assert lib.sv_lm_head_pack_bytes(777, 96, ctypes.byref(n)) == OK and n.value == 800 * 96 * 2
    assert lib.sv_lm_head_pack_bytes(1, 32, ctypes.byref(n)) == OK and n.value == 32 * 32 * 2
    for V, Hd in [(0, 64), (10, 48), (10, 0), (-1, 64)]:
        assert lib.sv_lm_head_pack_bytes(V, Hd, ctypes.byref(n)) == INVALID
    assert lib.sv_lm_head_pack_bytes(10, 64, None) == INVALID
    pack = lambda dt, w, out: lib.sv_lm_head_pack(100, 64, dt, w, out, None)
    assert pack(sv.SV_F32, FAKE, FAKE) == UNSUPPORTED
    assert pack(sv.SV_BF16, None, FAKE) == INVALID
    assert pack(sv.SV_BF16, FAKE, None) == INVALID
    assert pack(sv.SV_F16, ctypes.c_void_p(0x1008), FAKE) == INVALID
    assert lib.sv_lm_head_pack(0, 64, sv.SV_BF16, FAKE, FAKE, None) == INVALID
    call = lambda dt, h, ws, nbytes, B=1: lib.sv_lm_head_greedy_packed(
        B, 16, 1000, 64, dt, h, FAKE, FAKE, FAKE, FAKE, None, ws, nbytes, None)
    assert call(sv.SV_F32, FAKE, FAKE, 1 << 20) == UNSUPPORTED
    assert call(sv.SV_BF16, None, FAKE, 1 << 20) == INVALID
    assert call(sv.SV_BF16, ctypes.c_void_p(0x1008), FAKE, 1 << 20) == INVALID
    assert call(sv.SV_BF16, FAKE, FAKE, 8) == WORKSPACE
    assert call(sv.SV_BF16, FAKE, FAKE, 1 << 20, B=5) == INVALID    # B * K > 64


def test_status_strings(lib):
    assert lib.sv_status_string(0) == b"ok"
    assert lib.sv_status_string(-3) == b"workspace too small"


def test_noalloc_validation(lib):
    """The allocation-free attention call validates like sv_verify_attention and rejects,
    before any device call, a descriptor whose partials exceed its scratch array."""
    A = ctypes.c_void_p
    args = lambda d: (ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, None, None)
    assert lib.sv_verify_attention_noalloc(*args(_desc(block=0))) == INVALID
    assert lib.sv_verify_attention_noalloc(*args(_desc(head_dim=96))) == UNSUPPORTED
    big = _desc(batch=64, split_keys=64, sum_ctx_hint=0)
    assert _ws(lib, big)[1] > (32 << 20)
    assert lib.sv_verify_attention_noalloc(*args(big)) == WORKSPACE
    assert b"32" in lib.sv_last_error() or b"33554432" in lib.sv_last_error()


def test_sample_tree_validation(lib):
    n = ctypes.c_size_t()
    assert lib.sv_accept_sample_tree_workspace(1, 61, 152064, ctypes.byref(n)) == OK and n.value > 0
    assert lib.sv_accept_sample_tree_workspace(1, 1, 100, ctypes.byref(n)) == INVALID   # K >= 2
    good = (ctypes.c_int32 * 3)(0, 0, 1)
    call = lambda par, T=1.0, ws=FAKE, dt=sv.SV_BF16, tl=FAKE: lib.sv_accept_sample_tree(
        1, 4, 100, dt, tl, FAKE, par, FAKE, T, 1, 0, FAKE, FAKE, FAKE, ws, 1 << 30, None)
    assert call(good, T=0.0) == INVALID
    assert call(good, dt=sv.SV_F16) == UNSUPPORTED
    assert call(None) == INVALID
    assert call((ctypes.c_int32 * 3)(0, 2, 1)) == INVALID              # parent of node 2 is 2
    assert call((ctypes.c_int32 * 3)(0, 0, -1)) == INVALID
    assert call(good, ws=None) == WORKSPACE
    assert call(good, ws=ctypes.c_void_p(0x1008)) == INVALID
    assert call(good, tl=ctypes.c_void_p(0x1008)) == INVALID


def test_out_of_range_dtype_values(lib):
    """A C caller may pass any int as an sv_dtype: every entry point rejects values outside
    the enumerators as unsupported, before touching anything else."""
    for bad in (7, -1, 1 << 20):
        assert lib.sv_accept_greedy(1, 4, 100, bad, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 20,
                                    None) == UNSUPPORTED
        assert lib.sv_accept_sample(1, 4, 100, bad, FAKE, FAKE, FAKE, 1.0, 1, 0, FAKE, FAKE, FAKE,
                                    1 << 30, None) == UNSUPPORTED
        assert lib.sv_latent_compress(2, 4, 8, 128, bad, FAKE, FAKE, FAKE, 1.0, FAKE, 1 << 20,
                                      None) == UNSUPPORTED
        assert lib.sv_lm_head_greedy(1, 4, 100, 64, bad, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE,
                                     1 << 20, None) == UNSUPPORTED
        assert lib.sv_lm_head_greedy_packed(1, 4, 100, 64, bad, FAKE, FAKE, FAKE, FAKE, FAKE, None,
                                            FAKE, 1 << 20, None) == UNSUPPORTED
        assert lib.sv_lm_head_pack(100, 64, bad, FAKE, FAKE, None) == UNSUPPORTED
        d = _desc(dtype=bad)
        assert lib.sv_kv_append(ctypes.byref(d), 1, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                None) == UNSUPPORTED


def test_wait_limit_validation(lib):
    assert lib.sv_set_wait_limit(0) == INVALID
    assert lib.sv_set_wait_limit(-5) == INVALID
    assert lib.sv_set_wait_limit(1) == OK
    assert lib.sv_set_wait_limit(1 << 18) == OK                 # the default, restored

