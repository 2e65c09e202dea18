"""The C ABI on the host: the library loads, exports every function the
header declares, and rejects bad arguments before any HIP call (so these run
without a GPU: every call here fails validation and enqueues nothing)."""

import ctypes
import os
import re

import pytest

import speculative_decoding_medusa_amd as md

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "medusa.h")

L = md.lib
A = 0x10000          # a 16-byte aligned stand-in address (never dereferenced)
MIS = 0x10004        # misaligned
OK, NULL, SHAPE, DTYPE, VALUE, WS, HIP, ALIGN, ALIAS = 0, -1, -2, -3, -4, -5, -6, -7, -8


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(medusa_[a-z_]+)\s*\(", src)))


def test_header_and_exports_agree():
    names = _declared()
    assert len(names) >= 13
    for n in names:
        assert hasattr(L, n), n
    assert sorted(md.EXPORTED) == names


def test_version_and_strings():
    assert L.medusa_abi_version() == 109
    for code in (OK, NULL, SHAPE, DTYPE, VALUE, WS, HIP, ALIGN, ALIAS):
        assert L.medusa_status_string(code).decode() not in ("", "unknown status")
    assert L.medusa_status_string(-99).decode() == "unknown status"


def heads(dt=1, B=1, H=64, V=100, K=2, k=4, hidden=A, w1=A, b1=A, wlm=A, ids=A, vals=A, logits=None,
          r=None, ws=A, wsb=1 << 30):
    return L.medusa_heads(dt, B, H, V, K, k, hidden, w1, b1, wlm, ids, vals, logits, r, ws, wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dt=7), DTYPE), (dict(B=0), SHAPE), (dict(B=17), SHAPE), (dict(K=0), SHAPE), (dict(K=9), SHAPE),
    (dict(H=12), SHAPE), (dict(dt=0, H=6), SHAPE), (dict(k=0), SHAPE), (dict(k=65), SHAPE),
    (dict(V=3, k=4), SHAPE), (dict(hidden=None), NULL), (dict(wlm=None), NULL), (dict(ws=None), NULL),
    (dict(w1=MIS), ALIGN), (dict(logits=MIS), ALIGN), (dict(r=MIS), ALIGN), (dict(wsb=16), WS),
])
def test_heads_validation(kw, code):
    assert heads(**kw) == code
    assert L.medusa_last_error().decode() != ""


def heads_tree(dt=1, B=1, H=64, V=100, K=2, k=4, hidden=A, w1=A, b1=A, wlm=A, ids=A, vals=A, T=7, tidx=A, dep=A,
               root=A, plen=A, cand=A + 256, pos=A + 512, ws=A, wsb=1 << 30):
    return L.medusa_heads_tree(dt, B, H, V, K, k, hidden, w1, b1, wlm, ids, vals, None, None, T, tidx, dep, root,
                               plen, cand, pos, ws, wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dt=7), DTYPE), (dict(B=17), SHAPE), (dict(K=9), SHAPE), (dict(T=0), SHAPE), (dict(T=257), SHAPE),
    (dict(tidx=None), NULL), (dict(root=None), NULL), (dict(pos=None), NULL), (dict(dep=MIS), ALIGN),
    (dict(cand=A + 512), ALIAS), (dict(cand=A), ALIAS), (dict(pos=A), ALIAS), (dict(ws=None), NULL),
    (dict(wsb=16), WS),
])
def test_heads_tree_validation(kw, code):
    assert heads_tree(**kw) == code
    assert L.medusa_last_error().decode() != ""


def test_lm_head_topk_tree_validation():
    f = L.medusa_lm_head_topk_tree
    args = [1, 1, 64, 100, 2, 4, A, A, A, A, None, 7, A, A, A, A, A + 256, A + 512, A, 1 << 30, None]
    bad = list(args)
    bad[11] = 0
    assert f(*bad) == SHAPE
    bad = list(args)
    bad[12] = None
    assert f(*bad) == NULL
    bad = list(args)
    bad[16] = A
    assert f(*bad) == ALIAS
    bad = list(args)
    bad[19] = 8
    assert f(*bad) == WS


def heads_noalloc(dt=1, B=1, H=64, V=100, K=2, k=4, hidden=A, w1=A, b1=A, wlm=A, ids=A, vals=A, logits=None,
                  r=None):
    return L.medusa_heads_noalloc(dt, B, H, V, K, k, hidden, w1, b1, wlm, ids, vals, logits, r, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dt=7), DTYPE), (dict(B=17), SHAPE), (dict(K=9), SHAPE), (dict(k=65), SHAPE), (dict(hidden=None), NULL),
    (dict(ids=None), NULL), (dict(w1=MIS), ALIGN), (dict(r=MIS), ALIGN),
    # a shape whose workspace exceeds the library's per-GPU scratch
    (dict(B=16, H=8192, V=1 << 20, K=8, k=64), WS),
])
def test_heads_noalloc_validation(kw, code):
    assert heads_noalloc(**kw) == code
    assert L.medusa_last_error().decode() != ""


def test_heads_noalloc_scratch_limit_is_stated():
    # the header's MEDUSA_HEADS_NOALLOC_SCRATCH_BYTES: 16 MiB; the Vicuna-7B
    # and Vicuna-33B batch-8 head shapes fit, the rejected case above does not
    src = open(HEADER).read()
    assert "#define MEDUSA_HEADS_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)" in src
    lim = 16 << 20
    assert md.medusa_heads_workspace(1, 1, 4096, 32000, 5, 10) <= lim
    assert md.medusa_heads_workspace(1, 8, 6656, 32000, 5, 10) <= lim
    assert md.medusa_heads_workspace(1, 16, 8192, 1 << 20, 8, 64) > lim


def test_heads_workspace_sizes():
    assert md.medusa_heads_workspace(1, 1, 4096, 32000, 5, 10) > 0
    assert md.medusa_heads_workspace(1, 0, 4096, 32000, 5, 10) == 0
    assert md.medusa_heads_workspace(9, 1, 4096, 32000, 5, 10) == 0
    small = md.medusa_heads_workspace(1, 1, 4096, 32000, 5, 10)
    big = md.medusa_heads_workspace(1, 8, 6656, 32000, 5, 10)
    assert big > small


def test_resblock_and_lm_validation():
    assert L.medusa_resblock(1, 1, 12, 2, A, A, A, A, None) == SHAPE
    assert L.medusa_resblock(1, 1, 64, 2, A, None, A, A, None) == NULL
    assert L.medusa_lm_head_topk(1, 1, 64, 100, 2, 4, A, A, A, A, None, A, 8, None) == WS
    assert L.medusa_lm_head_topk(1, 1, 64, 100, 2, 4, MIS, A, A, A, None, A, 1 << 30, None) == ALIGN


def tree(B=1, K=2, k=2, N=6, ch=A, p_max=4, status=A, **kw):
    ptrs = [kw.get(n, A) for n in ("ids", "root", "plen", "cand", "tidx", "par", "dep", "pos", "mask",
                                   "ret", "np")]
    return L.medusa_build_tree(B, K, k, N, ch, *ptrs, p_max, status, None)


@pytest.mark.parametrize("kw,code", [
    (dict(B=0), SHAPE), (dict(K=9), SHAPE), (dict(k=65), SHAPE), (dict(N=256), SHAPE), (dict(N=-1), SHAPE),
    (dict(p_max=0), SHAPE), (dict(p_max=257), SHAPE), (dict(ch=None), NULL), (dict(status=None), NULL),
    (dict(mask=MIS), ALIGN), (dict(ret=None), NULL),
])
def test_tree_validation(kw, code):
    assert tree(**kw) == code


def attn(dt=1, B=1, T=15, Hq=4, d=64, S=200, q=A, kc=A, vc=A, plen=A, mask=A, scale=0.125, out=A, ws=A,
         wsb=1 << 30):
    return L.medusa_tree_attention(dt, B, T, Hq, d, S, q, kc, vc, plen, mask, scale, out, ws, wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dt=3), DTYPE), (dict(d=96), SHAPE), (dict(T=0), SHAPE), (dict(T=257), SHAPE), (dict(S=10), SHAPE),
    (dict(B=17), SHAPE), (dict(scale=0.0), VALUE), (dict(scale=-1.0), VALUE), (dict(scale=float("nan")), VALUE),
    (dict(q=None), NULL), (dict(out=MIS), ALIGN), (dict(wsb=8), WS),
])
def test_attention_validation(kw, code):
    assert attn(**kw) == code


def test_attention_workspace_sizes():
    assert md.medusa_tree_attention_workspace(1, 1, 64, 32, 128, 2112) > 0
    assert md.medusa_tree_attention_workspace(1, 1, 64, 32, 96, 2112) == 0


def post(B=1, T=15, V=1000, p_max=8, D=4, temp=0.7, eps=0.09, delta=0.3, logits=A, ws=A, wsb=1 << 30, **kw):
    return L.medusa_evaluate_posterior(B, T, V, p_max, D, logits, kw.get("cand", A), kw.get("ret", A),
                                       kw.get("np", A), temp, eps, delta, kw.get("best", A), kw.get("acc", A),
                                       kw.get("nxt", A), ws, wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(T=257), SHAPE), (dict(V=0), SHAPE), (dict(D=10), SHAPE), (dict(p_max=0), SHAPE),
    (dict(temp=-0.1), VALUE), (dict(temp=float("nan")), VALUE), (dict(eps=0.0), VALUE),
    (dict(delta=-1.0), VALUE), (dict(logits=None), NULL), (dict(best=MIS), ALIGN), (dict(wsb=4), WS),
])
def test_posterior_validation(kw, code):
    assert post(**kw) == code


def test_posterior_greedy_ignores_eps_delta():
    # with temperature 0, eps/delta are unused: validation passes them; the
    # first failing check is then the deliberately missing logits pointer
    assert post(temp=0.0, eps=0.0, delta=0.0, logits=None) == NULL


def commit(dt=1, B=1, nl=2, H=4, d=128, S=100, kc=A, vc=A + 0x100000, plen=A, ret=A, p_max=4, D=4, best=A,
           acc=A, newlen=A + 0x200):
    return L.medusa_commit_kv(dt, B, nl, H, d, S, kc, vc, plen, ret, p_max, D, best, acc, newlen, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dt=5), DTYPE), (dict(d=96), SHAPE), (dict(D=10), SHAPE), (dict(nl=0), SHAPE),
    (dict(newlen=A), ALIAS), (dict(vc=A), ALIAS), (dict(kc=None), NULL), (dict(best=MIS), ALIGN),
])
def test_commit_validation(kw, code):
    assert commit(**kw) == code


def base(dt=1, M=64, H=4096, V=32000, hidden=A, w=A, logits=A, packed=0):
    return L.medusa_base_lm_head(dt, M, H, V, hidden, w, packed, logits, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dt=0), DTYPE), (dict(dt=5), DTYPE), (dict(M=0), SHAPE), (dict(M=4097), SHAPE), (dict(H=0), SHAPE),
    (dict(H=12), SHAPE), (dict(H=1 << 17), SHAPE), (dict(V=0), SHAPE), (dict(hidden=None), NULL),
    (dict(w=None), NULL), (dict(logits=None), NULL), (dict(hidden=MIS), ALIGN), (dict(logits=MIS), ALIGN),
])
def test_base_lm_head_validation(kw, code):
    assert base(**kw) == code
    assert L.medusa_last_error().decode() != ""


def test_base_lm_head_pack_validation_and_sizes():
    # one KB per (16-row tile, 32-element k step), partial tiles and steps padded
    assert L.medusa_base_lm_head_packed_bytes(4096, 32000) == 2000 * 128 * 1024
    assert L.medusa_base_lm_head_packed_bytes(40, 17) == 2 * 2 * 1024
    assert L.medusa_base_lm_head_packed_bytes(40, 33) == 4 * 2 * 1024   # three tiles padded to four
    assert L.medusa_base_lm_head_packed_bytes(12, 17) == 0
    assert L.medusa_base_lm_head_packed_bytes(4096, 0) == 0
    assert L.medusa_base_lm_head_pack(0, 64, 100, A, A + 4096, None) == DTYPE
    assert L.medusa_base_lm_head_pack(1, 60, 100, A, A + 4096, None) == SHAPE
    assert L.medusa_base_lm_head_pack(1, 64, 100, None, A, None) == NULL
    assert L.medusa_base_lm_head_pack(1, 64, 100, A, MIS, None) == ALIGN
    assert L.medusa_base_lm_head_pack(1, 64, 100, A, A, None) == ALIAS


def bpost(B=1, T=64, H=4096, V=32000, p_max=64, D=6, hidden=A, w=A, packed=1, cand=A, ret=A, npaths=A,
          temp=0.7, eps=0.09, delta=0.3, best=A, acc=A, nxt=A, ws=A, wsb=1 << 30):
    return L.medusa_base_posterior(B, T, H, V, p_max, D, hidden, w, packed, cand, ret, npaths, temp, eps, delta,
                                   best, acc, nxt, ws, wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(B=0), SHAPE), (dict(T=257), SHAPE), (dict(H=12), SHAPE), (dict(V=131073), SHAPE), (dict(D=10), SHAPE),
    (dict(p_max=0), SHAPE), (dict(temp=-1.0), VALUE), (dict(eps=0.0), VALUE), (dict(hidden=None), NULL),
    (dict(cand=None), NULL), (dict(ws=None), NULL), (dict(w=MIS), ALIGN), (dict(wsb=16), WS),
])
def test_base_posterior_validation(kw, code):
    assert bpost(**kw) == code
    assert L.medusa_last_error().decode() != ""


def test_base_posterior_workspace_sizes():
    assert L.medusa_base_posterior_workspace(1, 64, 4096, 32000) > 0
    assert L.medusa_base_posterior_workspace(1, 64, 4096, 131072) > 0
    assert L.medusa_base_posterior_workspace(1, 64, 4096, 131073) == 0
    assert L.medusa_base_posterior_workspace(0, 64, 4096, 32000) == 0
    assert L.medusa_base_posterior_workspace(1, 64, 12, 32000) == 0


def nuc(B=1, T=64, V=32000, p_max=64, D=6, logits=A, cand=A, ret=A, npaths=A, temp=0.7, top_p=0.8, u=A, best=A,
        acc=A, nxt=A, samples=None, ws=A, wsb=1 << 20):
    return L.medusa_evaluate_posterior_nucleus(B, T, V, p_max, D, logits, cand, ret, npaths, temp, top_p, u, best,
                                               acc, nxt, samples, ws, wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(B=0), SHAPE), (dict(B=17), SHAPE), (dict(T=257), SHAPE), (dict(V=0), SHAPE), (dict(V=262145), SHAPE),
    (dict(D=10), SHAPE), (dict(p_max=0), SHAPE), (dict(temp=0.0), VALUE), (dict(temp=float("inf")), VALUE),
    (dict(temp=float("nan")), VALUE), (dict(top_p=0.0), VALUE), (dict(top_p=1.01), VALUE),
    (dict(top_p=float("nan")), VALUE), (dict(logits=None), NULL), (dict(u=None), NULL), (dict(ws=None), NULL),
    (dict(u=MIS), ALIGN), (dict(samples=MIS), ALIGN), (dict(wsb=16), WS),
])
def test_nucleus_validation(kw, code):
    assert nuc(**kw) == code
    assert L.medusa_last_error().decode() != ""


def test_nucleus_workspace_sizes():
    assert L.medusa_posterior_nucleus_workspace(1, 64) == 1280
    assert L.medusa_posterior_nucleus_workspace(16, 256) == 16 * 256 * 20
    assert L.medusa_posterior_nucleus_workspace(0, 64) == 0
    assert L.medusa_posterior_nucleus_workspace(1, 257) == 0


@pytest.mark.parametrize("call,code", [
    (lambda: L.medusa_embed(0, 64, 10, A, A, A, None), SHAPE),
    (lambda: L.medusa_embed(4, 60, 10, A, A, A, None), SHAPE),
    (lambda: L.medusa_embed(4, 64, 10, None, A, A, None), NULL),
    (lambda: L.medusa_embed(4, 64, 10, A, A, MIS, None), ALIGN),
    (lambda: L.medusa_add_rmsnorm(0, 64, A, None, A, 1e-6, A, None), SHAPE),
    (lambda: L.medusa_add_rmsnorm(4, 12, A, None, A, 1e-6, A, None), SHAPE),
    (lambda: L.medusa_add_rmsnorm(4, 64, A, None, A, -1.0, A, None), VALUE),
    (lambda: L.medusa_add_rmsnorm(4, 64, A, MIS, A, 1e-6, A, None), ALIGN),
    (lambda: L.medusa_add_rmsnorm(4, 64, A, None, None, 1e-6, A, None), NULL),
    (lambda: L.medusa_rope_qkv(0, 4, 2, 64, 100, A, A, A, 1e4, A, A, A, None), SHAPE),
    (lambda: L.medusa_rope_qkv(1, 4, 2, 63, 100, A, A, A, 1e4, A, A, A, None), SHAPE),
    (lambda: L.medusa_rope_qkv(1, 4, 2, 64, 100, A, A, A, 0.0, A, A, A, None), VALUE),
    (lambda: L.medusa_rope_qkv(1, 4, 2, 64, 100, A, A, None, 1e4, A, A, A, None), NULL),
    (lambda: L.medusa_silu_mul(4, 12, A, A, None), SHAPE),
    (lambda: L.medusa_silu_mul(4, 64, A, None, None), NULL),
])
def test_decoder_piece_validation(call, code):
    assert call() == code
    assert L.medusa_last_error().decode() != ""


def test_packed_heads_validation_and_sizes():
    assert L.medusa_heads_packed_bytes(5, 4096, 32000) == 5 * 2000 * 128 * 1024
    assert L.medusa_heads_packed_bytes(0, 4096, 32000) == 0
    assert L.medusa_heads_packed_bytes(9, 4096, 32000) == 0
    assert L.medusa_heads_pack(1, 0, 64, 100, A, A + 4096, None) == SHAPE
    assert L.medusa_heads_pack(0, 2, 64, 100, A, A + 4096, None) == DTYPE
    assert L.medusa_heads_pack(1, 2, 60, 100, A, A + 4096, None) == SHAPE
    assert L.medusa_heads_pack(1, 2, 64, 100, A, A, None) == ALIAS
    assert L.medusa_heads_pack(1, 2, 64, 100, None, A, None) == NULL
    ws = L.medusa_heads_workspace(1, 8, 4096, 32000, 5, 10)
    call = L.medusa_lm_head_topk_packed
    assert call(0, 8, 4096, 32000, 5, 10, A, A, A, A, None, A, ws, None) == DTYPE
    assert call(1, 17, 4096, 32000, 5, 10, A, A, A, A, None, A, ws, None) == SHAPE
    assert call(1, 8, 4096, 32000, 5, 10, A, None, A, A, None, A, ws, None) == NULL
    assert call(1, 8, 4096, 32000, 5, 10, A, A, A, A, None, A, 16, None) == WS
    hp = L.medusa_heads_packed
    assert hp(0, 8, 4096, 32000, 5, 10, A, A, A, A, A, A, None, None, A, ws, None) == DTYPE
    assert hp(1, 8, 4096, 32000, 5, 10, A, None, A, A, A, A, None, None, A, ws, None) == NULL
    assert hp(1, 8, 4096, 32000, 5, 10, A, A, A, A, A, A, None, None, A, 16, None) == WS
    assert hp(1, 8, 4100, 32000, 5, 10, A, A, A, A, A, A, None, None, A, ws, None) == SHAPE
    # the workspace covers the packed call at batch 1 too
    assert L.medusa_heads_workspace(1, 1, 4096, 32000, 5, 10) >= 256 + 2 * 5 * 250 * 10 * 4 + 5 * 2 * 4096 * 2


def test_tree_candidates_validation():
    tc = L.medusa_tree_candidates
    assert tc(0, 5, 2, 3, A, A, A, A, A, A, A + 4096, None) == SHAPE
    assert tc(1, 257, 2, 3, A, A, A, A, A, A, A + 4096, None) == SHAPE
    assert tc(1, 5, 9, 3, A, A, A, A, A, A, A + 4096, None) == SHAPE
    assert tc(1, 5, 2, 65, A, A, A, A, A, A, A + 4096, None) == SHAPE
    assert tc(1, 5, 2, 3, None, A, A, A, A, A, A + 4096, None) == NULL
    assert tc(1, 5, 2, 3, A, A, A, A, A, A, A, None) == ALIAS


def test_linear_workspace_and_validation():
    # a narrow output splits its reduction: 8 blocks of 128 outputs over
    # eleven 256-element chunks -> 11 slices of [M][V] float32
    assert L.medusa_linear_workspace(1, 2816, 1024) == 11 * 1 * 1024 * 4
    assert L.medusa_linear_workspace(15, 2816, 1024) >= 11 * 15 * 1024 * 4
    assert L.medusa_linear_workspace(1, 4096, 32000) == 256      # 250 blocks: no split
    assert L.medusa_linear_workspace(65, 1024, 1024) == 256      # more than one M tile: no split
    assert L.medusa_linear_workspace(1, 200, 1024) == 256        # one chunk: nothing to split
    assert L.medusa_linear_workspace(0, 1024, 1024) == 0
    assert L.medusa_linear_workspace(1, 1020, 1024) == 0
    need = L.medusa_linear_workspace(1, 2816, 1024)
    assert L.medusa_linear(0, 1, 2816, 1024, A, A, A, A, need, None) == DTYPE
    assert L.medusa_linear(1, 1, 2816, 1024, None, A, A, A, need, None) == NULL
    assert L.medusa_linear(1, 1, 2816, 1024, A, A, A, A, need - 4, None) == WS
    assert L.medusa_linear(1, 0, 2816, 1024, A, A, A, A, need, None) == SHAPE


def test_binding_rejects_cpu_tensors():
    import torch
    with pytest.raises(ValueError):
        md._lib._ptr(torch.zeros(4), "x")


def test_philox_uniforms_validation():
    f = L.medusa_philox_uniforms
    assert f(1, 2, 0, 0, 4, A, None) == SHAPE
    assert f(1, 2, 0, 17, 4, A, None) == SHAPE
    assert f(1, 2, 0, 1, 257, A, None) == SHAPE
    assert f(1, 2, -1, 1, 4, A, None) == VALUE
    assert f(1, 2, 0, 1, 4, None, None) == NULL
    assert f(1, 2, 0, 1, 4, MIS, None) == ALIGN


@pytest.mark.parametrize("kw,code", [
    (dict(B=0), SHAPE), (dict(T=300), SHAPE), (dict(V=0), SHAPE), (dict(D=10), SHAPE), (dict(p_max=0), SHAPE),
    (dict(t=0.0), VALUE), (dict(t=-1.0), VALUE), (dict(eps=0.0), VALUE), (dict(delta=1.0), VALUE),
    (dict(delta=0.0), VALUE), (dict(logits=None), NULL), (dict(nxt=None), NULL), (dict(best=MIS), ALIGN),
])
def test_sample_typical_validation(kw, code):
    a = dict(B=1, T=7, V=100, p_max=4, D=3, logits=A, ret=A, best=A, acc=A, t=0.7, eps=0.09, delta=0.3, nxt=A)
    a.update(kw)
    rc = L.medusa_sample_typical(a["B"], a["T"], a["V"], a["p_max"], a["D"], a["logits"], a["ret"], a["best"],
                                 a["acc"], a["t"], a["eps"], a["delta"], 5, 6, a["nxt"], None)
    assert rc == code
