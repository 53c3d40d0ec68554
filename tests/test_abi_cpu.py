"""C-ABI checks that need no GPU: the library loads, exports every function include/absa.h
declares, and rejects bad arguments with the documented status before any HIP call."""
import ctypes
import os
import re
import subprocess

import pytest

from block_sparse_attention_34_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "absa.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libabsa.so is not built (python -m block_sparse_attention_34_amd.build)")
    return _lib.load()


def header_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:absa_status|int32_t|const char\*)\s+(absa_\w+)\s*\(", text,
                                 flags=re.M)))


def test_header_declares_the_boundary():
    fns = header_functions()
    for name in ("absa_select", "absa_attend", "absa_dense", "absa_num_blocks", "absa_select_workspace",
                 "absa_select_workspace_layout", "absa_status_string", "absa_version"):
        assert name in fns
    assert sorted(_lib.EXPORTED) == fns


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = set(line.split()[-1] for line in out.splitlines() if line.strip())
    for name in header_functions():
        assert name in exported, name
        assert hasattr(lib, name)


def test_struct_layouts_match_header():
    # compile a tiny C program that prints sizeof/offsetof of the header structs
    src = r'''
#include <stdio.h>
#include <stddef.h>
#include "absa.h"
int main(void) {
  printf("%zu %zu %zu %zu %zu %zu %zu %zu %zu %zu %zu\n", sizeof(absa_problem), offsetof(absa_problem, scale),
         offsetof(absa_problem, out_bf16), sizeof(absa_select_params),
         offsetof(absa_select_params, seed), offsetof(absa_select_params, mode), sizeof(absa_blocklist),
         sizeof(absa_fp8_operands), offsetof(absa_fp8_operands, qk_int8), sizeof(absa_cluster_lists),
         offsetof(absa_cluster_lists, clusters));
  return 0;
}
'''
    import tempfile
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "t.c")
        open(c, "w").write(src)
        exe = os.path.join(d, "t")
        subprocess.run(["gcc", "-I" + os.path.dirname(HEADER), c, "-o", exe], check=True)
        vals = [int(x) for x in subprocess.run([exe], capture_output=True, text=True).stdout.split()]
    P, SP, BL = _lib.AbsaProblem, _lib.AbsaSelectParams, _lib.AbsaBlockList
    F8 = _lib.AbsaFp8Operands
    assert vals == [ctypes.sizeof(P), P.scale.offset, P.out_bf16.offset, ctypes.sizeof(SP), SP.seed.offset,
                    SP.mode.offset, ctypes.sizeof(BL), ctypes.sizeof(F8), F8.qk_int8.offset,
                    ctypes.sizeof(_lib.AbsaClusterLists), _lib.AbsaClusterLists.clusters.offset]


def prob(**kw):
    base = dict(B=1, H=2, L=1024, d=64, T=4, Hs=16, Ws=16, q_block=64, kv_block=16, scale=0.0, out_bf16=0)
    base.update(kw)
    return _lib.AbsaProblem(**base)


def params(**kw):
    base = dict(keep=0.25, clusters=4, kmeans_steps=3, select_scale_log2=0.0, seed=0, stream=0, mode=0)
    base.update(kw)
    return _lib.AbsaSelectParams(**base)


def test_version_and_strings(lib):
    assert lib.absa_version() == 10000
    assert lib.absa_status_string(0) == b"ok"
    assert lib.absa_status_string(-4).startswith(b"workspace")
    assert lib.absa_status_string(12345) == b"unknown status"


def test_num_blocks_and_shape_errors(lib):
    nq, nk = ctypes.c_int32(), ctypes.c_int32()
    assert lib.absa_num_blocks(ctypes.byref(prob()), ctypes.byref(nq), ctypes.byref(nk)) == 0
    assert (nq.value, nk.value) == (16, 64)
    p = prob(L=75600, T=21, Hs=45, Ws=80, d=128, q_block=128)
    assert lib.absa_num_blocks(ctypes.byref(p), ctypes.byref(nq), ctypes.byref(nk)) == 0
    assert (nq.value, nk.value) == (591, 4725)
    assert lib.absa_num_blocks(ctypes.byref(prob(T=5)), ctypes.byref(nq), ctypes.byref(nk)) == _lib.ABSA_ERR_SHAPE
    assert lib.absa_num_blocks(ctypes.byref(prob(L=0)), ctypes.byref(nq), ctypes.byref(nk)) == _lib.ABSA_ERR_SHAPE
    assert lib.absa_num_blocks(None, ctypes.byref(nq), ctypes.byref(nk)) == _lib.ABSA_ERR_INVALID_ARG
    assert lib.absa_num_blocks(ctypes.byref(prob()), None, ctypes.byref(nk)) == _lib.ABSA_ERR_INVALID_ARG
    for bad in (dict(d=96), dict(q_block=32), dict(kv_block=8), dict(kv_block=256)):
        assert lib.absa_num_blocks(ctypes.byref(prob(**bad)), ctypes.byref(nq), ctypes.byref(nk)) == \
            _lib.ABSA_ERR_UNSUPPORTED
    assert lib.absa_num_blocks(ctypes.byref(prob(scale=float("nan"))), ctypes.byref(nq), ctypes.byref(nk)) == \
        _lib.ABSA_ERR_INVALID_ARG


def test_workspace_size_and_layout(lib):
    n = ctypes.c_size_t()
    assert lib.absa_select_workspace(ctypes.byref(prob()), ctypes.byref(params()), ctypes.byref(n)) == 0
    offs = (ctypes.c_size_t * 5)()
    assert lib.absa_select_workspace_layout(ctypes.byref(prob()), ctypes.byref(params()), offs) == 0
    # kbar^T [2][64][64] f32, mu [32][4][64] f32, n_j [32][4] i32, s [32][64] f32, each
    # 256-aligned; no logit region (SIZE_MAX): one-list selection keeps the logits on chip
    assert list(offs) == [0, 32768, 32768 + 32768, 65536 + 512, 2 ** 64 - 1]
    # + per-split (max, normaliser) of each centroid: 2 splits of the 64 blocks here,
    # + the block means' bf16 heads and tails [2][2][64][64]
    assert n.value == 65536 + 512 + 8192 + 32 * 4 * 2 * 8 + 2 * 2 * 64 * 64 * 2
    for bad, code in ((dict(keep=0.0), -1), (dict(keep=1.5), -1), (dict(keep=float("nan")), -1),
                      (dict(clusters=3), -3), (dict(clusters=-1), -1), (dict(kmeans_steps=65), -1),
                      (dict(mode=7), -1), (dict(select_scale_log2=float("inf")), -1)):
        assert lib.absa_select_workspace(ctypes.byref(prob()), ctypes.byref(params(**bad)),
                                         ctypes.byref(n)) == code, bad


FAKE = 0x10000  # an aligned address that is never dereferenced: validation fails first


def lists(cap=64, count=FAKE, kv=FAKE, w=FAKE):
    return _lib.AbsaBlockList(count, kv, w, cap)


def test_select_validation(lib):
    n = ctypes.c_size_t()
    lib.absa_select_workspace(ctypes.byref(prob()), ctypes.byref(params()), ctypes.byref(n))
    ws = n.value
    P, S = ctypes.byref(prob()), ctypes.byref(params())
    call = lib.absa_select
    assert call(P, S, None, FAKE, ctypes.byref(lists()), None, FAKE, ws, None) == _lib.ABSA_ERR_INVALID_ARG
    assert call(P, S, FAKE + 8, FAKE, ctypes.byref(lists()), None, FAKE, ws, None) == _lib.ABSA_ERR_ALIGNMENT
    assert call(P, S, FAKE, FAKE, None, None, FAKE, ws, None) == _lib.ABSA_ERR_INVALID_ARG
    assert call(P, S, FAKE, FAKE, ctypes.byref(lists(cap=63)), None, FAKE, ws, None) == _lib.ABSA_ERR_SHAPE
    assert call(P, S, FAKE, FAKE, ctypes.byref(lists(kv=FAKE + 2)), None, FAKE, ws, None) == \
        _lib.ABSA_ERR_ALIGNMENT
    assert call(P, S, FAKE, FAKE, ctypes.byref(lists()), None, FAKE, ws - 1, None) == _lib.ABSA_ERR_WORKSPACE
    assert call(P, S, FAKE, FAKE, ctypes.byref(lists()), None, None, ws, None) == _lib.ABSA_ERR_WORKSPACE
    assert call(P, S, FAKE, FAKE, ctypes.byref(lists()), None, FAKE + 16, ws, None) == _lib.ABSA_ERR_ALIGNMENT
    assert call(P, S, FAKE, FAKE, ctypes.byref(lists()), FAKE + 1, FAKE, ws, None) == _lib.ABSA_ERR_ALIGNMENT
    big = prob(L=200000, T=2, Hs=250, Ws=400, d=128, q_block=128)  # NK = 12500 > 12288
    assert call(ctypes.byref(big), S, FAKE, FAKE, ctypes.byref(lists(cap=1 << 20)), None, FAKE, 1 << 62,
                None) == _lib.ABSA_ERR_UNSUPPORTED


def test_attend_and_dense_validation(lib):
    P = ctypes.byref(prob())
    assert lib.absa_attend(P, FAKE, FAKE, FAKE, ctypes.byref(lists()), None, None) == _lib.ABSA_ERR_INVALID_ARG
    assert lib.absa_attend(P, FAKE, FAKE, FAKE, None, FAKE, None) == _lib.ABSA_ERR_INVALID_ARG
    assert lib.absa_attend(P, FAKE, FAKE, FAKE + 4, ctypes.byref(lists()), FAKE, None) == \
        _lib.ABSA_ERR_ALIGNMENT
    assert lib.absa_attend(P, FAKE, FAKE, FAKE, ctypes.byref(lists(cap=0)), FAKE, None) == _lib.ABSA_ERR_SHAPE
    assert lib.absa_attend(ctypes.byref(prob(Ws=15)), FAKE, FAKE, FAKE, ctypes.byref(lists()), FAKE, None) == \
        _lib.ABSA_ERR_SHAPE
    assert lib.absa_dense(P, FAKE, None, FAKE, FAKE, None) == _lib.ABSA_ERR_INVALID_ARG
    assert lib.absa_dense(ctypes.byref(prob(d=32)), FAKE, FAKE, FAKE, FAKE, None) == _lib.ABSA_ERR_UNSUPPORTED
    assert lib.absa_dense(ctypes.byref(prob(out_bf16=2)), FAKE, FAKE, FAKE, FAKE, None) == \
        _lib.ABSA_ERR_INVALID_ARG


def test_attend_rejects_heads_beyond_32bit_buffer_offsets(lib):
    # the bf16 attention kernels address a head's K and V with 32-bit buffer offsets and use
    # 0x7FFFFFF0 as the base of entries outside a list: L*d*2 + one 64-key tile must stay below it
    big = prob(L=1 << 23, T=128, Hs=256, Ws=256, d=128, q_block=128)   # L*d*2 = 2^31
    assert lib.absa_attend(ctypes.byref(big), FAKE, FAKE, FAKE, ctypes.byref(lists(cap=1 << 19)), FAKE, None) == \
        _lib.ABSA_ERR_UNSUPPORTED
    assert lib.absa_dense(ctypes.byref(big), FAKE, FAKE, FAKE, FAKE, None) == _lib.ABSA_ERR_UNSUPPORTED
    assert lib.absa_attend_clusters(ctypes.byref(big), FAKE, FAKE, FAKE, ctypes.byref(cl_lists(cap=1 << 19)),
                                    FAKE, None) == _lib.ABSA_ERR_UNSUPPORTED
    big64 = prob(L=1 << 24, T=256, Hs=256, Ws=256, d=64, q_block=128)  # L*d*2 = 2^31 at d = 64
    assert lib.absa_dense(ctypes.byref(big64), FAKE, FAKE, FAKE, FAKE, None) == _lib.ABSA_ERR_UNSUPPORTED


def test_attend_pairs_validation(lib):
    n = ctypes.c_size_t()
    # 2 heads x ceil(1024 / 128) pairs: counts, [NK] indices and [NK][2] weights, then the work
    # queues of the persistent grid, 256-byte regions
    assert lib.absa_attend_pairs_workspace(ctypes.byref(prob()), ctypes.byref(n)) == 0
    assert n.value == 256 + 16 * 64 * 4 + 16 * 64 * 8 + 256
    ws = n.value
    assert lib.absa_attend_pairs_workspace(ctypes.byref(prob()), None) == _lib.ABSA_ERR_INVALID_ARG
    assert lib.absa_attend_pairs_workspace(ctypes.byref(prob(q_block=128)), ctypes.byref(n)) == \
        _lib.ABSA_ERR_UNSUPPORTED
    big_nk = prob(L=12289 * 16, T=12289, Hs=16, Ws=1)
    assert lib.absa_attend_pairs_workspace(ctypes.byref(big_nk), ctypes.byref(n)) == _lib.ABSA_ERR_UNSUPPORTED
    a = lib.absa_attend_pairs
    P, L = ctypes.byref(prob()), ctypes.byref(lists())
    assert a(ctypes.byref(prob(q_block=128)), FAKE, FAKE, FAKE, L, FAKE, FAKE, ws, None) == _lib.ABSA_ERR_UNSUPPORTED
    assert a(P, FAKE, FAKE, FAKE, L, None, FAKE, ws, None) == _lib.ABSA_ERR_INVALID_ARG
    assert a(P, FAKE, FAKE, FAKE + 4, L, FAKE, FAKE, ws, None) == _lib.ABSA_ERR_ALIGNMENT
    assert a(P, FAKE, FAKE, FAKE, None, FAKE, FAKE, ws, None) == _lib.ABSA_ERR_INVALID_ARG
    assert a(P, FAKE, FAKE, FAKE, ctypes.byref(lists(cap=0)), FAKE, FAKE, ws, None) == _lib.ABSA_ERR_SHAPE
    assert a(P, FAKE, FAKE, FAKE, L, FAKE, None, ws, None) == _lib.ABSA_ERR_WORKSPACE
    assert a(P, FAKE, FAKE, FAKE, L, FAKE, FAKE, ws - 1, None) == _lib.ABSA_ERR_WORKSPACE
    assert a(P, FAKE, FAKE, FAKE, L, FAKE, FAKE + 16, ws, None) == _lib.ABSA_ERR_ALIGNMENT
    big = prob(L=1 << 23, T=128, Hs=256, Ws=256, d=128)   # L*d*2 = 2^31: beyond 32-bit buffer offsets
    assert a(ctypes.byref(big), FAKE, FAKE, FAKE, L, FAKE, FAKE, ws, None) == _lib.ABSA_ERR_UNSUPPORTED


def test_attend_balanced_validation(lib):
    n = ctypes.c_size_t()
    assert lib.absa_attend_balanced_workspace(ctypes.byref(n)) == 0
    assert n.value == 256
    assert lib.absa_attend_balanced_workspace(None) == _lib.ABSA_ERR_INVALID_ARG
    ws = n.value
    a = lib.absa_attend_balanced
    P, L = ctypes.byref(prob(q_block=128)), ctypes.byref(lists())
    assert a(P, FAKE, FAKE, FAKE, L, FAKE, None, ws, None) == _lib.ABSA_ERR_WORKSPACE
    assert a(P, FAKE, FAKE, FAKE, L, FAKE, FAKE, ws - 1, None) == _lib.ABSA_ERR_WORKSPACE
    assert a(P, FAKE, FAKE, FAKE, L, FAKE, FAKE + 16, ws, None) == _lib.ABSA_ERR_ALIGNMENT
    assert a(P, FAKE, FAKE, FAKE, L, None, FAKE, ws, None) == _lib.ABSA_ERR_INVALID_ARG
    assert a(P, FAKE, FAKE, FAKE + 4, L, FAKE, FAKE, ws, None) == _lib.ABSA_ERR_ALIGNMENT
    assert a(P, FAKE, FAKE, FAKE, None, FAKE, FAKE, ws, None) == _lib.ABSA_ERR_INVALID_ARG
    assert a(P, FAKE, FAKE, FAKE, ctypes.byref(lists(cap=0)), FAKE, FAKE, ws, None) == _lib.ABSA_ERR_SHAPE
    big = prob(L=1 << 23, T=128, Hs=256, Ws=256, d=128, q_block=128)   # beyond 32-bit buffer offsets
    assert a(ctypes.byref(big), FAKE, FAKE, FAKE, L, FAKE, FAKE, ws, None) == _lib.ABSA_ERR_UNSUPPORTED


def test_select_noalloc_validation(lib):
    P, S = ctypes.byref(prob()), ctypes.byref(params())
    call = lib.absa_select_noalloc
    assert lib.absa_status_string(_lib.ABSA_ERR_TOO_LARGE).startswith(b"problem needs more")
    assert call(P, S, None, FAKE, ctypes.byref(lists()), None, None) == _lib.ABSA_ERR_INVALID_ARG
    assert call(P, S, FAKE + 8, FAKE, ctypes.byref(lists()), None, None) == _lib.ABSA_ERR_ALIGNMENT
    assert call(P, S, FAKE, FAKE, ctypes.byref(lists(cap=63)), None, None) == _lib.ABSA_ERR_SHAPE
    assert call(P, S, FAKE, FAKE, ctypes.byref(lists()), FAKE + 1, None) == _lib.ABSA_ERR_ALIGNMENT
    # the workspace of the 720p Wan shape with 5 heads (about 87 MiB) exceeds the fixed 64 MiB buffer
    p2 = prob(H=5, L=75600, T=21, Hs=45, Ws=80, d=128, q_block=128)
    n = ctypes.c_size_t()
    assert lib.absa_select_workspace(ctypes.byref(p2), S, ctypes.byref(n)) == 0 and n.value > 64 << 20
    assert call(ctypes.byref(p2), S, FAKE, FAKE, ctypes.byref(lists(cap=4725)), None, None) == \
        _lib.ABSA_ERR_TOO_LARGE
    import torch
    if not torch.cuda.is_available():   # a valid call reaches its first HIP call, which fails here
        assert call(P, S, FAKE, FAKE, ctypes.byref(lists()), None, None) == _lib.ABSA_ERR_HIP


def test_select_profile_validation(lib):
    n = ctypes.c_size_t()
    lib.absa_select_workspace(ctypes.byref(prob()), ctypes.byref(params()), ctypes.byref(n))
    ws = n.value
    P, S = ctypes.byref(prob()), ctypes.byref(params())
    ms = (ctypes.c_float * 5)()
    call = lib.absa_select_profile
    assert call(P, S, FAKE, FAKE, ctypes.byref(lists()), FAKE, ws, None, None, 5) == _lib.ABSA_ERR_INVALID_ARG
    assert call(P, S, FAKE, FAKE, ctypes.byref(lists()), FAKE, ws, None, ms, -1) == _lib.ABSA_ERR_INVALID_ARG
    assert call(P, S, None, FAKE, ctypes.byref(lists()), FAKE, ws, None, ms, 5) == _lib.ABSA_ERR_INVALID_ARG
    assert call(P, S, FAKE, FAKE, ctypes.byref(lists(cap=63)), FAKE, ws, None, ms, 5) == _lib.ABSA_ERR_SHAPE
    assert call(P, S, FAKE, FAKE, ctypes.byref(lists()), FAKE, ws - 1, None, ms, 5) == _lib.ABSA_ERR_WORKSPACE
    assert call(P, S, FAKE, FAKE, ctypes.byref(lists()), FAKE + 16, ws, None, ms, 5) == _lib.ABSA_ERR_ALIGNMENT


def fp8_ops(**kw):
    base = dict(q8=FAKE, sq=FAKE, k8=FAKE, sk=FAKE, kbar=FAKE, v8t=FAKE, sv=FAKE, mu=FAKE)
    base.update(kw)
    return _lib.AbsaFp8Operands(**base)


def test_fp8_validation(lib):
    P = ctypes.byref(prob(d=128, q_block=128))
    n = ctypes.c_size_t()
    assert lib.absa_fp8_workspace(P, ctypes.byref(n)) == 0 and n.value > 0
    assert lib.absa_fp8_workspace(ctypes.byref(prob(d=64)), ctypes.byref(n)) == _lib.ABSA_ERR_UNSUPPORTED
    assert lib.absa_fp8_workspace(ctypes.byref(prob(d=128, kv_block=32)), ctypes.byref(n)) == \
        _lib.ABSA_ERR_UNSUPPORTED
    assert lib.absa_fp8_workspace(P, None) == _lib.ABSA_ERR_INVALID_ARG
    ws = n.value
    O = ctypes.byref(fp8_ops())
    q = lib.absa_quantize_fp8
    assert q(P, FAKE, FAKE, FAKE, O, FAKE, ws - 1, None) == _lib.ABSA_ERR_WORKSPACE
    assert q(P, FAKE, FAKE, FAKE, O, None, ws, None) == _lib.ABSA_ERR_WORKSPACE
    assert q(P, FAKE, FAKE, FAKE, O, FAKE + 16, ws, None) == _lib.ABSA_ERR_ALIGNMENT
    assert q(P, FAKE, None, FAKE, O, FAKE, ws, None) == _lib.ABSA_ERR_INVALID_ARG
    assert q(P, FAKE, FAKE, FAKE, ctypes.byref(fp8_ops(mu=None)), FAKE, ws, None) == _lib.ABSA_ERR_INVALID_ARG
    assert q(P, FAKE, FAKE, FAKE, ctypes.byref(fp8_ops(sv=FAKE + 4)), FAKE, ws, None) == _lib.ABSA_ERR_ALIGNMENT
    assert q(P, FAKE, FAKE, FAKE, None, FAKE, ws, None) == _lib.ABSA_ERR_INVALID_ARG
    assert q(P, FAKE, FAKE, FAKE, ctypes.byref(fp8_ops(qk_int8=2)), FAKE, ws, None) == _lib.ABSA_ERR_INVALID_ARG
    a = lib.absa_attend_fp8
    assert a(ctypes.byref(prob(d=128, q_block=64)), O, None, FAKE, None) == _lib.ABSA_ERR_UNSUPPORTED
    assert a(P, O, None, None, None) == _lib.ABSA_ERR_INVALID_ARG
    assert a(P, O, None, FAKE + 8, None) == _lib.ABSA_ERR_ALIGNMENT
    assert a(P, O, ctypes.byref(lists(cap=0)), FAKE, None) == _lib.ABSA_ERR_SHAPE
    assert a(P, ctypes.byref(fp8_ops(q8=None)), None, FAKE, None) == _lib.ABSA_ERR_INVALID_ARG


def cl_lists(**kw):
    base = dict(count=FAKE, kv_idx=FAKE, w=FAKE, label=FAKE, cap=64, clusters=4)
    base.update(kw)
    return _lib.AbsaClusterLists(**base)


def test_cluster_validation(lib):
    P = ctypes.byref(prob())
    S = ctypes.byref(params())
    n, n1 = ctypes.c_size_t(), ctypes.c_size_t()
    assert lib.absa_select_clusters_workspace(P, S, ctypes.byref(n)) == 0
    assert lib.absa_select_workspace(P, S, ctypes.byref(n1)) == 0 and n.value > n1.value
    ws = n.value
    sel = lib.absa_select_clusters
    assert sel(P, S, FAKE, FAKE, ctypes.byref(cl_lists()), FAKE, ws - 1, None) == _lib.ABSA_ERR_WORKSPACE
    assert sel(P, S, FAKE, FAKE, ctypes.byref(cl_lists(cap=63)), FAKE, ws, None) == _lib.ABSA_ERR_SHAPE
    assert sel(P, S, FAKE, FAKE, ctypes.byref(cl_lists(clusters=2)), FAKE, ws, None) == _lib.ABSA_ERR_SHAPE
    assert sel(P, S, FAKE, FAKE, ctypes.byref(cl_lists(label=None)), FAKE, ws, None) == _lib.ABSA_ERR_INVALID_ARG
    assert sel(P, S, FAKE, FAKE, ctypes.byref(cl_lists(w=FAKE + 2)), FAKE, ws, None) == _lib.ABSA_ERR_ALIGNMENT
    assert sel(P, S, None, FAKE, ctypes.byref(cl_lists()), FAKE, ws, None) == _lib.ABSA_ERR_INVALID_ARG
    att = lib.absa_attend_clusters
    P128 = ctypes.byref(prob(q_block=128))
    assert att(P, FAKE, FAKE, FAKE, ctypes.byref(cl_lists()), FAKE, None) == _lib.ABSA_ERR_UNSUPPORTED  # Bq 64
    assert att(P128, FAKE, FAKE, FAKE, ctypes.byref(cl_lists(clusters=3)), FAKE, None) == _lib.ABSA_ERR_UNSUPPORTED
    assert att(P128, FAKE, FAKE, FAKE, None, FAKE, None) == _lib.ABSA_ERR_INVALID_ARG
    assert att(P128, FAKE, FAKE, FAKE, ctypes.byref(cl_lists(cap=10)), FAKE, None) == _lib.ABSA_ERR_SHAPE
    assert att(P128, FAKE, FAKE, FAKE, ctypes.byref(cl_lists()), None, None) == _lib.ABSA_ERR_INVALID_ARG


def test_binding_fails_loudly_without_gpu_tensors():
    import torch
    import block_sparse_attention_34_amd as absa
    p = absa.Problem(1, 2, 1024, 64, 4, 16, 16, 64, 16)
    x = torch.zeros((1, 2, 1024, 64), dtype=torch.bfloat16)
    with pytest.raises(TypeError):
        absa.dense(p, x, x, x)
    with pytest.raises(TypeError):
        absa.select(p, x, x, 0.25)


def test_hip_failure_is_reported_without_gpu(lib):
    """With no GPU present, a call that passes validation fails at its first HIP call and returns
    ABSA_ERR_HIP (no crash, no exception across the ABI)."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present: this case is only meaningful without one")
    assert lib.absa_dense(ctypes.byref(prob()), FAKE, FAKE, FAKE, FAKE, None) == _lib.ABSA_ERR_HIP
