"""AB-Attention block-sparse attention on MI355X (gfx950): Python binding.

Argument marshalling only: every step of selection and attention runs in the
HIP kernels of ``libabsa.so`` (C ABI in ``include/absa.h``).  PyTorch supplies
device memory and the current HIP stream.  There is no CPU path: calls fail if
the library is missing or a tensor is not on the GPU.
"""
import ctypes
import math
from dataclasses import dataclass
from typing import NamedTuple, Optional, Tuple

from . import _lib
from ._lib import SEL_ALL, SEL_SIP, SEL_TOPK, AbsaError  # noqa: F401

__all__ = [
    "Problem", "BlockLists", "select", "select_noalloc", "select_profile", "SELECT_KERNELS", "attend",
    "attend_balanced", "attend_balanced_workspace_bytes", "attend_pairs",
    "attend_pairs_workspace_bytes", "dense", "num_blocks", "select_workspace_bytes",
    "workspace_layout", "alloc_lists", "library", "SEL_SIP", "SEL_TOPK", "SEL_ALL", "AbsaError",
    "Fp8Operands", "alloc_fp8", "fp8_workspace_bytes", "quantize_fp8", "attend_fp8",
    "ClusterLists", "alloc_cluster_lists", "select_clusters_workspace_bytes", "select_clusters", "attend_clusters",
]

_MODES = {"sip": SEL_SIP, "topk": SEL_TOPK, "all": SEL_ALL}


def library() -> ctypes.CDLL:
    return _lib.load()


@dataclass(frozen=True)
class Problem:
    B: int
    H: int
    L: int
    d: int
    T: int
    Hs: int
    Ws: int
    q_block: int
    kv_block: int
    scale: float = 0.0
    out_bf16: bool = False

    def c(self) -> _lib.AbsaProblem:
        return _lib.AbsaProblem(self.B, self.H, self.L, self.d, self.T, self.Hs, self.Ws, self.q_block,
                                self.kv_block, float(self.scale), int(bool(self.out_bf16)))

    @property
    def nq(self) -> int:
        return -(-self.L // self.q_block)

    @property
    def nk(self) -> int:
        return -(-self.L // self.kv_block)

    @property
    def rows(self) -> int:
        return self.B * self.H * self.nq

    @property
    def sigma(self) -> float:
        return self.scale if self.scale > 0 else 1.0 / math.sqrt(self.d)


class BlockLists(NamedTuple):
    count: "object"   # torch.int32 [rows]
    kv_idx: "object"  # torch.int32 [rows, cap]
    inv_pi: "object"  # torch.float32 [rows, cap]

    def c(self) -> _lib.AbsaBlockList:
        return _lib.AbsaBlockList(self.count.data_ptr(), self.kv_idx.data_ptr(), self.inv_pi.data_ptr(),
                                  int(self.kv_idx.shape[1]))


def _params(keep, clusters, kmeans_steps, select_scale_log2, seed, stream_id, mode):
    m = _MODES[mode] if isinstance(mode, str) else int(mode)
    return _lib.AbsaSelectParams(float(keep), int(clusters), int(kmeans_steps), float(select_scale_log2),
                                 int(seed) & 0xFFFFFFFFFFFFFFFF, int(stream_id) & 0xFFFFFFFF, m)


def _stream():
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check_qkv(prob: Problem, *ts):
    import torch
    for t in ts:
        if not isinstance(t, torch.Tensor) or t.dtype != torch.bfloat16 or not t.is_cuda:
            raise TypeError("Q, K, V must be bfloat16 tensors on the GPU")
        if not t.is_contiguous() or tuple(t.shape) != (prob.B, prob.H, prob.L, prob.d):
            raise ValueError(f"expected contiguous [B,H,L,d] = {(prob.B, prob.H, prob.L, prob.d)}, "
                             f"got {tuple(t.shape)}")


def _check_out(prob: Problem, out, device):
    """A caller-supplied output: [B,H,L,d], contiguous, on the inputs' GPU, bf16 if out_bf16 else fp32."""
    import torch
    want = torch.bfloat16 if prob.out_bf16 else torch.float32
    if not isinstance(out, torch.Tensor) or not out.is_cuda or out.device != device:
        raise ValueError("out must be a tensor on the same GPU as Q, K, V")
    if out.dtype != want:
        raise ValueError(f"out must be {want} (out_bf16={bool(prob.out_bf16)}), got {out.dtype}")
    if not out.is_contiguous() or tuple(out.shape) != (prob.B, prob.H, prob.L, prob.d):
        raise ValueError(f"out must be contiguous [B,H,L,d] = {(prob.B, prob.H, prob.L, prob.d)}, "
                         f"got {tuple(out.shape)}")


def _check_lists(prob: Problem, lists, device, need_cap_nk: bool):
    """Block lists: int32 count [rows], int32 kv_idx and fp32 inv_pi [rows, cap], contiguous, on the
    inputs' GPU; cap >= 1 (>= NK when the lists are written by a selection)."""
    import torch
    count, kv_idx, inv_pi = lists
    for t, dt, name in ((count, torch.int32, "count"), (kv_idx, torch.int32, "kv_idx"),
                        (inv_pi, torch.float32, "inv_pi")):
        if not isinstance(t, torch.Tensor) or t.dtype != dt or not t.is_cuda or t.device != device:
            raise ValueError(f"lists.{name} must be a {dt} tensor on the same GPU as Q and K")
        if not t.is_contiguous():
            raise ValueError(f"lists.{name} must be contiguous")
    if tuple(count.shape) != (prob.rows,):
        raise ValueError(f"lists.count must have shape [rows] = [{prob.rows}], got {tuple(count.shape)}")
    if kv_idx.dim() != 2 or kv_idx.shape[0] != prob.rows or kv_idx.shape != inv_pi.shape:
        raise ValueError(f"lists.kv_idx and lists.inv_pi must both be [rows, cap] with rows = {prob.rows}")
    cap = kv_idx.shape[1]
    if cap < 1 or (need_cap_nk and cap < prob.nk):
        raise ValueError(f"lists capacity {cap} is too small (needs >= {prob.nk if need_cap_nk else 1})")


def num_blocks(prob: Problem) -> Tuple[int, int]:
    nq, nk = ctypes.c_int32(), ctypes.c_int32()
    p = prob.c()
    _lib.check(library().absa_num_blocks(ctypes.byref(p), ctypes.byref(nq), ctypes.byref(nk)),
               "absa_num_blocks")
    return nq.value, nk.value


def select_workspace_bytes(prob: Problem, keep: float, clusters: int = 0, kmeans_steps: int = 0,
                           select_scale_log2: float = 0.0, seed: int = 0, stream_id: int = 0,
                           mode="sip") -> int:
    n = ctypes.c_size_t()
    p = prob.c()
    sp = _params(keep, clusters, kmeans_steps, select_scale_log2, seed, stream_id, mode)
    _lib.check(library().absa_select_workspace(ctypes.byref(p), ctypes.byref(sp), ctypes.byref(n)),
               "absa_select_workspace")
    return n.value


def workspace_layout(prob: Problem, keep: float, clusters: int = 0, kmeans_steps: int = 0,
                     mode="sip") -> Tuple[int, int, int, int, int]:
    """Offsets of (kbar^T, mu, n_j, s, logits) inside the selection workspace."""
    offs = (ctypes.c_size_t * 5)()
    p = prob.c()
    sp = _params(keep, clusters, kmeans_steps, 0.0, 0, 0, mode)
    _lib.check(library().absa_select_workspace_layout(ctypes.byref(p), ctypes.byref(sp), offs),
               "absa_select_workspace_layout")
    return tuple(int(x) for x in offs)


def alloc_lists(prob: Problem, device="cuda", cap: Optional[int] = None) -> BlockLists:
    import torch
    cap = prob.nk if cap is None else cap
    return BlockLists(torch.zeros(prob.rows, dtype=torch.int32, device=device),
                      torch.zeros((prob.rows, cap), dtype=torch.int32, device=device),
                      torch.zeros((prob.rows, cap), dtype=torch.float32, device=device))


def select(prob: Problem, q, k, keep: float, *, clusters: int = 0, kmeans_steps: int = 0,
           select_scale_log2: float = 0.0, seed: int = 0, stream_id: int = 0, mode="sip",
           lists: Optional[BlockLists] = None, want_pi: bool = False, workspace=None):
    """IBCS + SIP (or TOPK / ALL) block selection.  Returns (lists, pi or None, workspace)."""
    import torch
    _check_qkv(prob, q, k)
    lists = alloc_lists(prob, q.device) if lists is None else lists
    _check_lists(prob, lists, q.device, need_cap_nk=True)
    pi = torch.empty((prob.rows, prob.nk), dtype=torch.float32, device=q.device) if want_pi else None
    nbytes = select_workspace_bytes(prob, keep, clusters, kmeans_steps, select_scale_log2, seed,
                                    stream_id, mode)
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    p = prob.c()
    sp = _params(keep, clusters, kmeans_steps, select_scale_log2, seed, stream_id, mode)
    bl = lists.c()
    st = library().absa_select(ctypes.byref(p), ctypes.byref(sp), q.data_ptr(), k.data_ptr(),
                               ctypes.byref(bl), pi.data_ptr() if pi is not None else None,
                               workspace.data_ptr(), workspace.numel(), _stream())
    _lib.check(st, "absa_select")
    return lists, pi, workspace


def select_noalloc(prob: Problem, q, k, keep: float, lists: BlockLists, *, clusters: int = 0,
                   kmeans_steps: int = 0, select_scale_log2: float = 0.0, seed: int = 0, stream_id: int = 0,
                   mode="sip", pi=None):
    """``select`` into caller-given ``lists`` (and ``pi`` [rows, NK] fp32 if given) through
    absa_select_noalloc: no workspace and no device allocation by this call; the library's fixed
    64 MiB per-device scratch buffer holds the intermediates (calls overlapping on one device race).
    Raises AbsaError(ABSA_ERR_TOO_LARGE) for problems whose workspace exceeds it."""
    import torch
    _check_qkv(prob, q, k)
    _check_lists(prob, lists, q.device, need_cap_nk=True)
    if pi is not None:
        if (not isinstance(pi, torch.Tensor) or pi.dtype != torch.float32 or pi.device != q.device
                or not pi.is_contiguous() or tuple(pi.shape) != (prob.rows, prob.nk)):
            raise ValueError(f"pi must be a contiguous fp32 [rows, NK] = {(prob.rows, prob.nk)} tensor on Q's GPU")
    p = prob.c()
    sp = _params(keep, clusters, kmeans_steps, select_scale_log2, seed, stream_id, mode)
    bl = lists.c()
    st = library().absa_select_noalloc(ctypes.byref(p), ctypes.byref(sp), q.data_ptr(), k.data_ptr(),
                                       ctypes.byref(bl), pi.data_ptr() if pi is not None else None, _stream())
    _lib.check(st, "absa_select_noalloc")
    return lists, pi


SELECT_KERNELS = ("block means", "k-means", "logit normalisers", "scores", "sampling")


def select_profile(prob: Problem, q, k, keep: float, *, clusters: int = 0, kmeans_steps: int = 0,
                   select_scale_log2: float = 0.0, seed: int = 0, stream_id: int = 0, mode="sip",
                   lists: Optional[BlockLists] = None, workspace=None):
    """One ``select`` timed kernel by kernel (HIP events on the current stream; waits for it).
    Returns (lists, {kernel name: ms}) with the names of SELECT_KERNELS."""
    import torch
    _check_qkv(prob, q, k)
    lists = alloc_lists(prob, q.device) if lists is None else lists
    _check_lists(prob, lists, q.device, need_cap_nk=True)
    nbytes = select_workspace_bytes(prob, keep, clusters, kmeans_steps, select_scale_log2, seed, stream_id, mode)
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    p = prob.c()
    sp = _params(keep, clusters, kmeans_steps, select_scale_log2, seed, stream_id, mode)
    bl = lists.c()
    ms = (ctypes.c_float * len(SELECT_KERNELS))()
    st = library().absa_select_profile(ctypes.byref(p), ctypes.byref(sp), q.data_ptr(), k.data_ptr(),
                                       ctypes.byref(bl), workspace.data_ptr(), workspace.numel(), _stream(), ms,
                                       len(SELECT_KERNELS))
    _lib.check(st, "absa_select_profile")
    return lists, dict(zip(SELECT_KERNELS, (float(x) for x in ms)))


def attend(prob: Problem, q, k, v, lists: BlockLists, out=None):
    """Block-sparse attention over ``lists`` with 1/pi weights.  Returns O [B,H,L,d]."""
    import torch
    _check_qkv(prob, q, k, v)
    _check_lists(prob, lists, q.device, need_cap_nk=False)
    odt = torch.bfloat16 if prob.out_bf16 else torch.float32
    if out is None:
        out = torch.zeros((prob.B, prob.H, prob.L, prob.d), dtype=odt, device=q.device)
    else:
        _check_out(prob, out, q.device)
    p = prob.c()
    bl = lists.c()
    st = library().absa_attend(ctypes.byref(p), q.data_ptr(), k.data_ptr(), v.data_ptr(), ctypes.byref(bl),
                               out.data_ptr(), _stream())
    _lib.check(st, "absa_attend")
    return out


def attend_balanced_workspace_bytes() -> int:
    """Bytes of workspace ``attend_balanced`` needs (its work queues)."""
    n = ctypes.c_size_t()
    _lib.check(library().absa_attend_balanced_workspace(ctypes.byref(n)), "absa_attend_balanced_workspace")
    return int(n.value)


def attend_balanced(prob: Problem, q, k, v, lists: BlockLists, out=None, workspace=None):
    """``attend`` through absa_attend_balanced: a persistent grid that takes row pairs from per-XCD work
    queues (the same output as ``attend``).  ``workspace``: a uint8 tensor on Q's GPU of at least
    attend_balanced_workspace_bytes() bytes (allocated when None).  Returns O [B,H,L,d]."""
    import torch
    _check_qkv(prob, q, k, v)
    _check_lists(prob, lists, q.device, need_cap_nk=False)
    odt = torch.bfloat16 if prob.out_bf16 else torch.float32
    if out is None:
        out = torch.zeros((prob.B, prob.H, prob.L, prob.d), dtype=odt, device=q.device)
    else:
        _check_out(prob, out, q.device)
    nbytes = attend_balanced_workspace_bytes()
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    elif (not isinstance(workspace, torch.Tensor) or workspace.dtype != torch.uint8 or workspace.device != q.device
          or workspace.numel() < nbytes):
        raise ValueError(f"workspace must be a uint8 tensor of at least {nbytes} bytes on Q's GPU")
    p = prob.c()
    bl = lists.c()
    st = library().absa_attend_balanced(ctypes.byref(p), q.data_ptr(), k.data_ptr(), v.data_ptr(), ctypes.byref(bl),
                                        out.data_ptr(), workspace.data_ptr(), workspace.numel(), _stream())
    _lib.check(st, "absa_attend_balanced")
    return out


def attend_pairs_workspace_bytes(prob: Problem) -> int:
    """Bytes of workspace ``attend_pairs`` needs (64-query blocks)."""
    n = ctypes.c_size_t()
    p = prob.c()
    _lib.check(library().absa_attend_pairs_workspace(ctypes.byref(p), ctypes.byref(n)), "absa_attend_pairs_workspace")
    return int(n.value)


def attend_pairs(prob: Problem, q, k, v, lists: BlockLists, out=None, workspace=None):
    """``attend`` for 64-query blocks through absa_attend_pairs: adjacent query blocks share one
    128-query row of the two-row kernel over the union of their lists.  Returns O [B,H,L,d]."""
    import torch
    _check_qkv(prob, q, k, v)
    _check_lists(prob, lists, q.device, need_cap_nk=False)
    odt = torch.bfloat16 if prob.out_bf16 else torch.float32
    if out is None:
        out = torch.zeros((prob.B, prob.H, prob.L, prob.d), dtype=odt, device=q.device)
    else:
        _check_out(prob, out, q.device)
    nbytes = attend_pairs_workspace_bytes(prob)
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    p = prob.c()
    bl = lists.c()
    st = library().absa_attend_pairs(ctypes.byref(p), q.data_ptr(), k.data_ptr(), v.data_ptr(), ctypes.byref(bl),
                                     out.data_ptr(), workspace.data_ptr(), workspace.numel(), _stream())
    _lib.check(st, "absa_attend_pairs")
    return out


def dense(prob: Problem, q, k, v, out=None):
    """Dense attention softmax(scale Q K^T) V.  Returns O [B,H,L,d]."""
    import torch
    _check_qkv(prob, q, k, v)
    odt = torch.bfloat16 if prob.out_bf16 else torch.float32
    if out is None:
        out = torch.zeros((prob.B, prob.H, prob.L, prob.d), dtype=odt, device=q.device)
    else:
        _check_out(prob, out, q.device)
    p = prob.c()
    st = library().absa_dense(ctypes.byref(p), q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                              _stream())
    _lib.check(st, "absa_dense")
    return out


# ----------------------------------------------------------------------------- FP8 (E4M3) path

class Fp8Operands(NamedTuple):
    """Quantised operands (absa_fp8_operands): device tensors owned by the caller."""
    q8: "object"    # uint8 [B,H,L,128]
    sq: "object"    # float32 [B,H,L]
    k8: "object"    # uint8 [B,H,L,128]
    sk: "object"    # float32 [B,H,NK]
    kbar: "object"  # float32 [B,H,128]
    v8t: "object"   # uint8 [B,H,NK,128,16]
    sv: "object"    # float32 [B,H,128]
    mu: "object"    # int16 (bf16 bits) [B,H,NK,32,4]
    qk_int8: bool = False  # q8/k8 hold INT8 codes instead of E4M3

    def c(self) -> _lib.AbsaFp8Operands:
        return _lib.AbsaFp8Operands(*(t.data_ptr() for t in self[:8]), int(bool(self.qk_int8)))


def alloc_fp8(prob: Problem, device, qk_int8: bool = False) -> Fp8Operands:
    import torch
    B, H, L, nk = prob.B, prob.H, prob.L, prob.nk
    u8, f32 = torch.uint8, torch.float32
    return Fp8Operands(
        torch.empty((B, H, L, 128), dtype=u8, device=device), torch.empty((B, H, L), dtype=f32, device=device),
        torch.empty((B, H, L, 128), dtype=u8, device=device), torch.empty((B, H, nk), dtype=f32, device=device),
        torch.empty((B, H, 128), dtype=f32, device=device), torch.empty((B, H, nk, 128, 16), dtype=u8, device=device),
        torch.empty((B, H, 128), dtype=f32, device=device), torch.empty((B, H, nk, 32, 4), dtype=torch.int16,
                                                                        device=device), bool(qk_int8))


def fp8_workspace_bytes(prob: Problem) -> int:
    n = ctypes.c_size_t()
    p = prob.c()
    _lib.check(library().absa_fp8_workspace(ctypes.byref(p), ctypes.byref(n)), "absa_fp8_workspace")
    return n.value


def quantize_fp8(prob: Problem, q, k, v, ops: Optional[Fp8Operands] = None, workspace=None,
                 qk_int8: bool = False):
    """E4M3 operands of bf16 Q, K, V (d = 128, Bk = 16); with ``qk_int8`` Q and K get INT8 codes.
    Returns (ops, workspace)."""
    import torch
    _check_qkv(prob, q, k, v)
    ops = alloc_fp8(prob, q.device, qk_int8) if ops is None else ops
    nbytes = fp8_workspace_bytes(prob)
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    p = prob.c()
    o = ops.c()
    st = library().absa_quantize_fp8(ctypes.byref(p), q.data_ptr(), k.data_ptr(), v.data_ptr(), ctypes.byref(o),
                                     workspace.data_ptr(), workspace.numel(), _stream())
    _lib.check(st, "absa_quantize_fp8")
    return ops, workspace


def attend_fp8(prob: Problem, ops: Fp8Operands, lists: Optional[BlockLists], out=None):
    """FP8 block-sparse attention over ``lists`` (None: every key, weight 1).  Returns O."""
    import torch
    odt = torch.bfloat16 if prob.out_bf16 else torch.float32
    if out is None:
        out = torch.zeros((prob.B, prob.H, prob.L, prob.d), dtype=odt, device=ops.q8.device)
    else:
        _check_out(prob, out, ops.q8.device)
    if lists is not None:
        _check_lists(prob, lists, ops.q8.device, need_cap_nk=False)
    p = prob.c()
    o = ops.c()
    bl = lists.c() if lists is not None else None
    st = library().absa_attend_fp8(ctypes.byref(p), ctypes.byref(o), ctypes.byref(bl) if bl is not None else None,
                                   out.data_ptr(), _stream())
    _lib.check(st, "absa_attend_fp8")
    return out


# ----------------------------------------------------------------------------- per-cluster lists

class ClusterLists(NamedTuple):
    """Per-cluster lists (absa_cluster_lists): the union of a row's cluster samples."""
    count: "object"   # torch.int32 [rows]
    kv_idx: "object"  # torch.int32 [rows, cap]
    w: "object"       # torch.float32 [rows, cap, C]
    label: "object"   # torch.uint8 [rows, Bq]

    def c(self) -> _lib.AbsaClusterLists:
        return _lib.AbsaClusterLists(self.count.data_ptr(), self.kv_idx.data_ptr(), self.w.data_ptr(),
                                     self.label.data_ptr(), int(self.kv_idx.shape[1]), int(self.w.shape[2]))


def _check_cluster_lists(prob: Problem, lists, device):
    """Per-cluster lists: int32 count [rows], int32 kv_idx [rows, cap] with cap >= NK, fp32 w
    [rows, cap, C], uint8 label [rows, Bq]; contiguous, on the inputs' GPU."""
    import torch
    count, kv_idx, w, label = lists
    for t, dt, name in ((count, torch.int32, "count"), (kv_idx, torch.int32, "kv_idx"),
                        (w, torch.float32, "w"), (label, torch.uint8, "label")):
        if not isinstance(t, torch.Tensor) or t.dtype != dt or not t.is_cuda or t.device != device:
            raise ValueError(f"lists.{name} must be a {dt} tensor on the same GPU as Q and K")
        if not t.is_contiguous():
            raise ValueError(f"lists.{name} must be contiguous")
    if tuple(count.shape) != (prob.rows,) or kv_idx.dim() != 2 or kv_idx.shape[0] != prob.rows:
        raise ValueError(f"lists.count / kv_idx must be [rows] / [rows, cap] with rows = {prob.rows}")
    if kv_idx.shape[1] < prob.nk:
        raise ValueError(f"lists capacity {kv_idx.shape[1]} is below NK = {prob.nk}")
    if w.dim() != 3 or tuple(w.shape[:2]) != tuple(kv_idx.shape):
        raise ValueError("lists.w must be [rows, cap, C]")
    if tuple(label.shape) != (prob.rows, prob.q_block):
        raise ValueError(f"lists.label must be [rows, Bq] = {(prob.rows, prob.q_block)}")


def alloc_cluster_lists(prob: Problem, clusters: int = 4, device="cuda") -> ClusterLists:
    import torch
    C = clusters or 4
    return ClusterLists(torch.zeros(prob.rows, dtype=torch.int32, device=device),
                        torch.zeros((prob.rows, prob.nk), dtype=torch.int32, device=device),
                        torch.zeros((prob.rows, prob.nk, C), dtype=torch.float32, device=device),
                        torch.zeros((prob.rows, prob.q_block), dtype=torch.uint8, device=device))


def select_clusters_workspace_bytes(prob: Problem, keep: float, clusters: int = 0, kmeans_steps: int = 0,
                                    select_scale_log2: float = 0.0, seed: int = 0, stream_id: int = 0,
                                    mode="sip") -> int:
    n = ctypes.c_size_t()
    p = prob.c()
    sp = _params(keep, clusters, kmeans_steps, select_scale_log2, seed, stream_id, mode)
    _lib.check(library().absa_select_clusters_workspace(ctypes.byref(p), ctypes.byref(sp), ctypes.byref(n)),
               "absa_select_clusters_workspace")
    return n.value


def select_clusters(prob: Problem, q, k, keep: float, *, clusters: int = 0, kmeans_steps: int = 0,
                    select_scale_log2: float = 0.0, seed: int = 0, stream_id: int = 0, mode="sip",
                    lists: Optional[ClusterLists] = None, workspace=None):
    """IBCS + one SIP (or TOPK / ALL) sample per cluster.  Returns (lists, workspace)."""
    import torch
    _check_qkv(prob, q, k)
    lists = alloc_cluster_lists(prob, clusters, q.device) if lists is None else lists
    _check_cluster_lists(prob, lists, q.device)
    nbytes = select_clusters_workspace_bytes(prob, keep, clusters, kmeans_steps, select_scale_log2, seed,
                                             stream_id, mode)
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    p = prob.c()
    sp = _params(keep, clusters, kmeans_steps, select_scale_log2, seed, stream_id, mode)
    cl = lists.c()
    st = library().absa_select_clusters(ctypes.byref(p), ctypes.byref(sp), q.data_ptr(), k.data_ptr(),
                                        ctypes.byref(cl), workspace.data_ptr(), workspace.numel(), _stream())
    _lib.check(st, "absa_select_clusters")
    return lists, workspace


def attend_clusters(prob: Problem, q, k, v, lists: ClusterLists, out=None):
    """Attention over per-cluster lists (each query over its cluster's sample).  Returns O."""
    import torch
    _check_qkv(prob, q, k, v)
    _check_cluster_lists(prob, lists, q.device)
    odt = torch.bfloat16 if prob.out_bf16 else torch.float32
    if out is None:
        out = torch.zeros((prob.B, prob.H, prob.L, prob.d), dtype=odt, device=q.device)
    else:
        _check_out(prob, out, q.device)
    p = prob.c()
    cl = lists.c()
    st = library().absa_attend_clusters(ctypes.byref(p), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                        ctypes.byref(cl), out.data_ptr(), _stream())
    _lib.check(st, "absa_attend_clusters")
    return out
