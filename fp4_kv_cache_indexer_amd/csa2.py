"""Thin ctypes binding of libcsa2.so (include/csa2.h).

Argument marshalling only: every step runs in the HIP library.  Tensors are
torch tensors on the GPU (torch supplies device memory and the current
stream); outputs and workspaces the caller does not pass are allocated with
torch.  Non-zero statuses raise ``Csa2Error`` with the library's message.
The module refuses to work without the built library: there is no fallback.
"""

import ctypes
import os

import torch

# CSA2_LIBRARY may name another build of the same library (e.g. one whose
# host code carries AddressSanitizer)
_LIB_PATH = os.environ.get("CSA2_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libcsa2.so")
_lib = None

LATENT_DIM = 512
IDX_HEADS = 32
IDX_DIM = 128
BLOCK_POS = 8


class Csa2Error(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"csa2 status {status}: {msg}")
        self.status = status


class IndexerArgs(ctypes.Structure):
    _fields_ = [
        ("n_rows", ctypes.c_int32),
        ("n_seq", ctypes.c_int64),
        ("row_seq", ctypes.c_void_p),
        ("n_valid", ctypes.c_void_p),
        ("n_ent", ctypes.c_int64),
        ("top_k", ctypes.c_int32),
        ("q", ctypes.c_void_p),
        ("head_w", ctypes.c_void_p),
        ("keys", ctypes.c_void_p),
        ("block_keys", ctypes.c_void_p),
        ("keep_blocks", ctypes.c_int32),
        ("cand", ctypes.c_void_p),
        ("n_cand", ctypes.c_int32),
        ("out_idx", ctypes.c_void_p),
        ("out_score", ctypes.c_void_p),
        ("out_blocks", ctypes.c_void_p),
        ("cand_blocks", ctypes.c_void_p),
        ("n_cand_blocks", ctypes.c_int32),
        ("key_format", ctypes.c_int32),
        ("key_scales", ctypes.c_void_p),
    ]


class AppendArgs(ctypes.Structure):
    _fields_ = [
        ("n_rows", ctypes.c_int32),
        ("n_seq", ctypes.c_int64),
        ("row_seq", ctypes.c_void_p),
        ("pos", ctypes.c_void_p),
        ("m", ctypes.c_int32),
        ("x_bf16", ctypes.c_void_p),
        ("gate_bf16", ctypes.c_void_p),
        ("pend_x", ctypes.c_void_p),
        ("pend_gate", ctypes.c_void_p),
        ("n_ent", ctypes.c_int64),
        ("codes", ctypes.c_void_p),
        ("scales", ctypes.c_void_p),
        ("key_bf16", ctypes.c_void_p),
        ("key_format", ctypes.c_int32),
        ("keys", ctypes.c_void_p),
        ("key_scales", ctypes.c_void_p),
        ("block_keys", ctypes.c_void_p),
        ("swa", ctypes.c_void_p),
        ("swa_cap", ctypes.c_int32),
    ]


class AttnArgs(ctypes.Structure):
    _fields_ = [
        ("n_rows", ctypes.c_int32),
        ("n_heads", ctypes.c_int32),
        ("n_seq", ctypes.c_int64),
        ("row_seq", ctypes.c_void_p),
        ("q_bf16", ctypes.c_void_p),
        ("codes", ctypes.c_void_p),
        ("scales", ctypes.c_void_p),
        ("n_ent", ctypes.c_int64),
        ("idx", ctypes.c_void_p),
        ("top_k", ctypes.c_int32),
        ("swa", ctypes.c_void_p),
        ("swa_cap", ctypes.c_int32),
        ("swa_start", ctypes.c_void_p),
        ("swa_len", ctypes.c_void_p),
        ("sm_scale", ctypes.c_float),
        ("out", ctypes.c_void_p),
        ("lse", ctypes.c_void_p),
        ("swa_max", ctypes.c_int32),
    ]


EXPORTS = (
    "csa2_abi_version", "csa2_status_string", "csa2_last_error",
    "csa2_kv_compress_quantize", "csa2_index_block_summary",
    "csa2_index_key_quantize", "csa2_index_block_summary_fp4", "csa2_decode_append",
    "csa2_indexer_topk_workspace", "csa2_indexer_topk", "csa2_indexer_topk_static", "csa2_append_indexer_topk",
    "csa2_sparse_attn_workspace", "csa2_sparse_attn_decode", "csa2_attn_plan_override",
    "csa2_kernel_timer_start", "csa2_kernel_timer_stop", "csa2_mfma_dot_probe",
    "csa2_probe_scan_read", "csa2_probe_mfma_valu", "csa2_probe_gather",
)

KEY_E4M3, KEY_FP4 = 0, 1          # index-key formats (CSA2_KEY_*)

SITES = dict(kv_quant=1, block_summary=2, score_flat=3, score_coarse=4, score_pool=5,
             score_cand=6, select=7, attn=8, attn_combine=9, filter=10, append=11)


def lib():
    """Load libcsa2.so (once) and declare the signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is not built (run __graft_entry__.build())")
    L = ctypes.CDLL(_LIB_PATH)
    i32, i64, vp, sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t
    L.csa2_abi_version.restype = i32
    L.csa2_abi_version.argtypes = []
    L.csa2_status_string.restype = ctypes.c_char_p
    L.csa2_status_string.argtypes = [i32]
    L.csa2_last_error.restype = ctypes.c_char_p
    L.csa2_last_error.argtypes = []
    L.csa2_kv_compress_quantize.restype = i32
    L.csa2_kv_compress_quantize.argtypes = [vp, vp, i64, i64, i32, i64, vp, vp, i64, vp]
    L.csa2_index_block_summary.restype = i32
    L.csa2_index_block_summary.argtypes = [vp, i64, i64, i64, i64, vp, vp]
    L.csa2_index_key_quantize.restype = i32
    L.csa2_index_key_quantize.argtypes = [vp, i64, i64, i64, vp, vp, i64, vp]
    L.csa2_index_block_summary_fp4.restype = i32
    L.csa2_index_block_summary_fp4.argtypes = [vp, vp, i64, i64, i64, i64, vp, vp]
    L.csa2_decode_append.restype = i32
    L.csa2_decode_append.argtypes = [ctypes.POINTER(AppendArgs), vp]
    L.csa2_indexer_topk_workspace.restype = sz
    L.csa2_indexer_topk_workspace.argtypes = [ctypes.POINTER(IndexerArgs)]
    L.csa2_indexer_topk.restype = i32
    L.csa2_indexer_topk.argtypes = [ctypes.POINTER(IndexerArgs), vp, sz, vp]
    L.csa2_append_indexer_topk.restype = i32
    L.csa2_append_indexer_topk.argtypes = [ctypes.POINTER(AppendArgs), ctypes.POINTER(IndexerArgs), vp, sz, vp]
    L.csa2_indexer_topk_static.restype = i32
    L.csa2_indexer_topk_static.argtypes = [ctypes.POINTER(IndexerArgs), vp]
    L.csa2_sparse_attn_workspace.restype = sz
    L.csa2_sparse_attn_workspace.argtypes = [ctypes.POINTER(AttnArgs)]
    L.csa2_attn_plan_override.restype = i32
    L.csa2_attn_plan_override.argtypes = [i32, i32]
    L.csa2_mfma_dot_probe.restype = i32
    L.csa2_mfma_dot_probe.argtypes = [vp, vp, i32, i32, vp, vp, vp]
    L.csa2_probe_scan_read.restype = i32
    L.csa2_probe_scan_read.argtypes = [vp, i32, i32, i32, i32, i32, vp, vp]
    L.csa2_probe_mfma_valu.restype = i32
    L.csa2_probe_mfma_valu.argtypes = [i32, i32, i32, i32, vp, vp]
    L.csa2_probe_gather.restype = i32
    L.csa2_probe_gather.argtypes = [vp, vp, i64, vp, i32, i32, i32, vp, vp]
    L.csa2_sparse_attn_decode.restype = i32
    L.csa2_sparse_attn_decode.argtypes = [ctypes.POINTER(AttnArgs), vp, sz, vp]
    L.csa2_kernel_timer_start.restype = i32
    L.csa2_kernel_timer_start.argtypes = [i32, i32]
    L.csa2_kernel_timer_stop.restype = i32
    L.csa2_kernel_timer_stop.argtypes = [ctypes.POINTER(i32), ctypes.POINTER(ctypes.c_float)]
    _lib = L
    return L


def _check(st):
    if st != 0:
        L = lib()
        raise Csa2Error(st, L.csa2_last_error().decode() or L.csa2_status_string(st).decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev(t, name):
    if t is not None and not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t is not None and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def abi_version():
    return lib().csa2_abi_version()


def status_string(st):
    return lib().csa2_status_string(st).decode()


def last_error():
    return lib().csa2_last_error().decode()


def kernel_timer_start(site, max_launches):
    """Time the next launches from one site (a name in SITES) with HIP events."""
    _check(lib().csa2_kernel_timer_start(SITES[site], max_launches))


def kernel_timer_stop():
    """Returns (launches timed, total milliseconds)."""
    n = ctypes.c_int32(0)
    ms = ctypes.c_float(0.0)
    _check(lib().csa2_kernel_timer_stop(ctypes.byref(n), ctypes.byref(ms)))
    return n.value, ms.value


def kv_compress_quantize(x, m, gate=None, codes=None, scales=None, n_tok=None,
                         out_seq_stride=0, stream=None):
    """x, gate: bf16 [S, T, 512].  Returns (codes uint8 [S, T//m, 256],
    scales uint8 [S, T//m, 32]) unless caller-owned outputs (possibly with
    ``out_seq_stride``) are given."""
    _dev(x, "x"), _dev(gate, "gate")
    S, T = x.shape[0], x.shape[1] if n_tok is None else n_tok
    E = T // m
    if codes is None:
        codes = torch.empty((S, E, LATENT_DIM // 2), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((S, E, LATENT_DIM // 16), dtype=torch.uint8, device=x.device)
    _check(lib().csa2_kv_compress_quantize(
        _ptr(x), _ptr(gate), S, T, m, x.shape[1], _ptr(codes), _ptr(scales), out_seq_stride,
        _stream(stream)))
    return codes, scales


def index_block_summary(keys, summ=None, blk_begin=0, blk_end=None, stream=None):
    """keys uint8 [S, N, 128] -> summaries uint8 [S, ceil(N/8), 128]."""
    _dev(keys, "keys")
    S, N = keys.shape[0], keys.shape[1]
    nb = (N + BLOCK_POS - 1) // BLOCK_POS
    if summ is None:
        summ = torch.empty((S, nb, IDX_DIM), dtype=torch.uint8, device=keys.device)
    blk_end = nb if blk_end is None else blk_end
    _check(lib().csa2_index_block_summary(_ptr(keys), S, N, blk_begin, blk_end, _ptr(summ),
                                          _stream(stream)))
    return summ


def index_key_quantize(k, codes=None, scales=None, n_ent=None, out_seq_stride=0, stream=None):
    """bf16 index keys [S, T, 128] -> FP4 codes uint8 [S, N, 64] and scales
    uint8 [S, N, 4] (N = n_ent or T)."""
    _dev(k, "k")
    S, T = k.shape[0], k.shape[1]
    N = T if n_ent is None else n_ent
    if codes is None:
        codes = torch.empty((S, N, 64), dtype=torch.uint8, device=k.device)
    if scales is None:
        scales = torch.empty((S, N, 4), dtype=torch.uint8, device=k.device)
    _check(lib().csa2_index_key_quantize(_ptr(k), S, N, T, _ptr(codes), _ptr(scales), out_seq_stride,
                                         _stream(stream)))
    return codes, scales


def index_block_summary_fp4(codes, scales, summ=None, blk_begin=0, blk_end=None, stream=None):
    """FP4 index keys [S, N, 64] + [S, N, 4] -> E4M3 block keys [S, ceil(N/8), 128]."""
    _dev(codes, "codes")
    _dev(scales, "scales")
    S, N = codes.shape[0], codes.shape[1]
    nb = (N + 7) // 8
    if summ is None:
        summ = torch.empty((S, nb, 128), dtype=torch.uint8, device=codes.device)
    blk_end = nb if blk_end is None else blk_end
    _check(lib().csa2_index_block_summary_fp4(_ptr(codes), _ptr(scales), S, N, blk_begin, blk_end, _ptr(summ),
                                              _stream(stream)))
    return summ


def _append_struct(x, pos, codes, scales, key, keys, m=1, gate=None, pend_x=None, pend_gate=None,
                   key_scales=None, block_keys=None, swa=None, row_seq=None):
    for name, t in (("x", x), ("pos", pos), ("codes", codes), ("scales", scales), ("key", key),
                    ("keys", keys), ("gate", gate), ("pend_x", pend_x), ("pend_gate", pend_gate),
                    ("key_scales", key_scales), ("block_keys", block_keys), ("swa", swa),
                    ("row_seq", row_seq)):
        _dev(t, name)
    a = AppendArgs()
    a.n_rows = x.shape[0]
    a.n_seq = codes.shape[0]
    a.row_seq = _ptr(row_seq)
    a.pos = _ptr(pos)
    a.m = m
    a.x_bf16 = _ptr(x)
    a.gate_bf16 = _ptr(gate)
    a.pend_x = _ptr(pend_x)
    a.pend_gate = _ptr(pend_gate)
    a.n_ent = codes.shape[1]
    a.codes = _ptr(codes)
    a.scales = _ptr(scales)
    a.key_bf16 = _ptr(key)
    a.key_format = KEY_FP4 if key_scales is not None else KEY_E4M3
    a.keys = _ptr(keys)
    a.key_scales = _ptr(key_scales)
    a.block_keys = _ptr(block_keys)
    a.swa = _ptr(swa)
    a.swa_cap = 0 if swa is None else swa.shape[1]
    return a


def decode_append(x, pos, codes, scales, key, keys, m=1, gate=None, pend_x=None, pend_gate=None,
                  key_scales=None, block_keys=None, swa=None, row_seq=None, stream=None):
    """Append one token per row (x: bf16 [R, 512], pos: int64 [R]) to the
    caches of sequences row_seq (identity when None): window ring slot
    pos % swa_cap, the pending group for m > 1, and when a group completes
    entry pos // m (codes/scales), its index key (key: bf16 [R, 128]; E4M3
    keys [S, N, 128] or FP4 keys [S, N, 64] with key_scales [S, N, 4]) and
    the summary of its block (block_keys [S, ceil(N/8), 128])."""
    a = _append_struct(x, pos, codes, scales, key, keys, m, gate, pend_x, pend_gate, key_scales, block_keys,
                       swa, row_seq)
    _check(lib().csa2_decode_append(ctypes.byref(a), _stream(stream)))


def append_indexer_topk(x, pos, codes, scales, key, q, keys, top_k, block_keys, m=1, gate=None, pend_x=None,
                        pend_gate=None, key_scales=None, swa=None, row_seq=None, head_w=None, n_valid=None,
                        keep_blocks=2048, out_idx=None, out_score=None, out_blocks=None, workspace=None,
                        stream=None):
    """decode_append(...) then indexer_topk(q, keys, top_k, block_keys=...)
    over the same rows and caches, as one library call (the append runs
    inside the coarse scan's launch).  Returns out_idx."""
    a = _append_struct(x, pos, codes, scales, key, keys, m, gate, pend_x, pend_gate, key_scales, block_keys,
                       swa, row_seq)
    for t, nm in ((q, "q"), (head_w, "head_w"), (n_valid, "n_valid")):
        _dev(t, nm)
    R = q.shape[0]
    if out_idx is None:
        out_idx = torch.empty((R, top_k), dtype=torch.int32, device=q.device)
    b = _indexer_struct(q, keys, top_k, head_w, row_seq, n_valid, block_keys, keep_blocks, None,
                        out_idx, out_score, out_blocks, None, key_scales)
    L = lib()
    need = L.csa2_indexer_topk_workspace(ctypes.byref(b))
    if workspace is None:
        workspace = torch.zeros(max(need, 256), dtype=torch.uint8, device=q.device)
    _check(L.csa2_append_indexer_topk(ctypes.byref(a), ctypes.byref(b), _ptr(workspace), workspace.numel(),
                                      _stream(stream)))
    return out_idx


def window_append(x, pos, swa, row_seq=None, stream=None):
    """Write one token per row (x: bf16 [R, 512]) into window rings only
    (swa: uint8 [S, cap, 512], slot pos % cap of sequence row_seq[r]), for
    layers without a global cache of their own."""
    for name, t in (("x", x), ("pos", pos), ("swa", swa), ("row_seq", row_seq)):
        _dev(t, name)
    a = AppendArgs()
    a.n_rows = x.shape[0]
    a.n_seq = swa.shape[0]
    a.row_seq = _ptr(row_seq)
    a.pos = _ptr(pos)
    a.m = 1
    a.x_bf16 = _ptr(x)
    a.swa = _ptr(swa)
    a.swa_cap = swa.shape[1]
    _check(lib().csa2_decode_append(ctypes.byref(a), _stream(stream)))


def _indexer_struct(q, keys, top_k, head_w, row_seq, n_valid, block_keys, keep_blocks, cand,
                    out_idx, out_score, out_blocks, cand_blocks=None, key_scales=None):
    a = IndexerArgs()
    a.n_rows = q.shape[0]
    a.n_seq = keys.shape[0]
    a.row_seq = _ptr(row_seq)
    a.n_valid = _ptr(n_valid)
    a.n_ent = keys.shape[1]
    a.top_k = top_k
    a.q = _ptr(q)
    a.head_w = _ptr(head_w)
    a.keys = _ptr(keys)
    a.block_keys = _ptr(block_keys)
    a.keep_blocks = keep_blocks
    a.cand = _ptr(cand)
    a.n_cand = 0 if cand is None else cand.shape[1]
    a.out_idx = _ptr(out_idx)
    a.out_score = _ptr(out_score)
    a.out_blocks = _ptr(out_blocks)
    a.cand_blocks = _ptr(cand_blocks)
    a.n_cand_blocks = 0 if cand_blocks is None else cand_blocks.shape[1]
    a.key_format = KEY_E4M3 if key_scales is None else KEY_FP4
    a.key_scales = _ptr(key_scales)
    return a


def indexer_topk_workspace(q, keys, top_k, block_keys=None, keep_blocks=2048, cand=None, cand_blocks=None,
                           key_scales=None):
    a = _indexer_struct(q, keys, top_k, None, None, None, block_keys, keep_blocks, cand,
                        None, None, None, cand_blocks, key_scales)
    return lib().csa2_indexer_topk_workspace(ctypes.byref(a))


def indexer_topk(q, keys, top_k, head_w=None, row_seq=None, n_valid=None, block_keys=None,
                 keep_blocks=2048, cand=None, out_idx=None, out_score=None, out_blocks=None,
                 workspace=None, stream=None, cand_blocks=None, key_scales=None):
    """q uint8 [R, 32, 128]; keys uint8 [S, N, 128] (E4M3), or FP4 codes
    [S, N, 64] with key_scales uint8 [S, N, 4].  Returns out_idx int32
    [R, top_k] (ascending, -1 padded).  cand_blocks int32 [R, B]: select among
    the positions of these blocks (e.g. a Full layer's out_blocks)."""
    for t, nm in ((q, "q"), (keys, "keys"), (head_w, "head_w"), (row_seq, "row_seq"),
                  (n_valid, "n_valid"), (block_keys, "block_keys"), (cand, "cand"),
                  (cand_blocks, "cand_blocks"), (key_scales, "key_scales")):
        _dev(t, nm)
    R = q.shape[0]
    if out_idx is None:
        out_idx = torch.empty((R, top_k), dtype=torch.int32, device=q.device)
    a = _indexer_struct(q, keys, top_k, head_w, row_seq, n_valid, block_keys, keep_blocks, cand,
                        out_idx, out_score, out_blocks, cand_blocks, key_scales)
    L = lib()
    need = L.csa2_indexer_topk_workspace(ctypes.byref(a))
    if workspace is None:
        # must be zero before first use; the library leaves it zeroed after
        workspace = torch.zeros(max(need, 256), dtype=torch.uint8, device=q.device)
    _check(L.csa2_indexer_topk(ctypes.byref(a), _ptr(workspace), workspace.numel(), _stream(stream)))
    return out_idx


STATIC_SCRATCH_BYTES = 64 << 20   # CSA2_STATIC_SCRATCH_BYTES


def indexer_topk_static(q, keys, top_k, head_w=None, row_seq=None, n_valid=None, block_keys=None,
                        keep_blocks=2048, cand=None, out_idx=None, out_score=None, out_blocks=None,
                        stream=None, cand_blocks=None, key_scales=None):
    """indexer_topk without a workspace: the library's static per-GPU scratch
    (at most STATIC_SCRATCH_BYTES; larger requests raise).  Calls that
    overlap on one GPU race; keep them on one stream."""
    for t, nm in ((q, "q"), (keys, "keys"), (head_w, "head_w"), (row_seq, "row_seq"),
                  (n_valid, "n_valid"), (block_keys, "block_keys"), (cand, "cand"),
                  (cand_blocks, "cand_blocks"), (key_scales, "key_scales")):
        _dev(t, nm)
    R = q.shape[0]
    if out_idx is None:
        out_idx = torch.empty((R, top_k), dtype=torch.int32, device=q.device)
    a = _indexer_struct(q, keys, top_k, head_w, row_seq, n_valid, block_keys, keep_blocks, cand,
                        out_idx, out_score, out_blocks, cand_blocks, key_scales)
    _check(lib().csa2_indexer_topk_static(ctypes.byref(a), _stream(stream)))
    return out_idx


def _attn_struct(q, codes, scales, idx, swa, swa_start, swa_len, row_seq, sm_scale, out, lse,
                 swa_max=0):
    a = AttnArgs()
    a.n_rows = q.shape[0]
    a.n_heads = q.shape[1]
    a.n_seq = q.shape[0] if codes is None else codes.shape[0]
    if swa is not None and codes is not None and swa.shape[0] != codes.shape[0]:
        raise ValueError("swa and codes must hold the same sequences")
    if codes is None and swa is not None:
        a.n_seq = swa.shape[0]
    a.row_seq = _ptr(row_seq)
    a.q_bf16 = _ptr(q)
    a.codes = _ptr(codes)
    a.scales = _ptr(scales)
    a.n_ent = 0 if codes is None else codes.shape[1]
    a.idx = _ptr(idx)
    a.top_k = 0 if idx is None else idx.shape[1]
    a.swa = _ptr(swa)
    a.swa_cap = 0 if swa is None else swa.shape[1]
    a.swa_start = _ptr(swa_start)
    a.swa_len = _ptr(swa_len)
    a.sm_scale = float(sm_scale)
    a.out = _ptr(out)
    a.lse = _ptr(lse)
    a.swa_max = int(swa_max)
    return a


def mfma_dot_probe(q, k, stream=None):
    """q uint8 [n_q, 128], k uint8 [n_k, 128] E4M3 (n_q, n_k multiples of 16):
    the 128-term dot products through the fp16 and the fp8 matrix-core paths,
    as float32 [n_q, n_k] each."""
    _dev(q, "q"), _dev(k, "k")
    nq, nk = q.shape[0], k.shape[0]
    o16 = torch.empty((nq, nk), dtype=torch.float32, device=q.device)
    o8 = torch.empty((nq, nk), dtype=torch.float32, device=q.device)
    _check(lib().csa2_mfma_dot_probe(_ptr(q), _ptr(k), nq, nk, _ptr(o16), _ptr(o8), _stream(stream)))
    return o16, o8


def probe_scan_read(keys, chunk, full_lines, nontemporal, stream=None):
    """Timing probe: read keys uint8 [n_rows, n_keys, 128] in the block-summary
    scan's shape (chunks of `chunk` keys per workgroup); returns the
    per-thread XOR words."""
    _dev(keys, "keys")
    if keys.dim() != 3 or keys.shape[2] != 128 or keys.dtype != torch.uint8:
        raise ValueError("probe_scan_read: keys must be uint8 [n_rows, n_keys, 128]")
    n_rows, n_keys = keys.shape[0], keys.shape[1]
    wgs = n_rows * ((n_keys + chunk - 1) // chunk)
    out = torch.empty(wgs * 256, dtype=torch.int32, device=keys.device)
    _check(lib().csa2_probe_scan_read(_ptr(keys), n_rows, n_keys, int(chunk), int(bool(full_lines)),
                                      int(bool(nontemporal)), _ptr(out), _stream(stream)))
    return out


def probe_mfma_valu(n_valu, threads, iters, n_wg, stream=None):
    """Timing probe: MFMA chains with n_valu independent FMAs per MFMA."""
    out = torch.empty(n_wg * threads, dtype=torch.float32, device="cuda")
    _check(lib().csa2_probe_mfma_valu(int(n_valu), int(threads), int(iters), int(n_wg), _ptr(out), _stream(stream)))
    return out


def probe_gather(codes, scales, ids, n_wg, whole_lines, stream=None):
    """Timing probe: the attention gather's reads of FP4 entries (codes uint8
    [n_ent, 256], scales uint8 [n_ent, 32]) for ids int32 [n_rows, 512]."""
    _dev(codes, "codes"), _dev(scales, "scales"), _dev(ids, "ids")
    if (codes.dim() != 2 or codes.shape[1] != 256 or scales.shape != (codes.shape[0], 32)
            or ids.dim() != 2 or ids.shape[1] != 512 or ids.dtype != torch.int32):
        raise ValueError("probe_gather: codes [n_ent, 256], scales [n_ent, 32], ids int32 [n_rows, 512]")
    out = torch.empty(n_wg * 128, dtype=torch.int32, device=codes.device)
    _check(lib().csa2_probe_gather(_ptr(codes), _ptr(scales), codes.shape[0], _ptr(ids), ids.shape[0], int(n_wg),
                                   int(bool(whole_lines)), _ptr(out), _stream(stream)))
    return out


def attn_plan_override(heads_per_wg=0, n_split=0):
    """Pin the attention geometry (16 or 64 heads per workgroup, key splits per
    row) for later calls; (0, 0) restores the automatic plan."""
    _check(lib().csa2_attn_plan_override(int(heads_per_wg), int(n_split)))


def sparse_attn_workspace(q, idx, swa=None, swa_len=None, codes=None, swa_max=0):
    a = _attn_struct(q, codes, None, idx, swa, None, swa_len, None, 0.0, None, None, swa_max)
    return lib().csa2_sparse_attn_workspace(ctypes.byref(a))


def sparse_attn_decode(q, codes, scales, idx, swa=None, swa_start=None, swa_len=None,
                       row_seq=None, sm_scale=0.0, out=None, lse=None, workspace=None,
                       stream=None, swa_max=0):
    """q bf16 [R, H, 512]; codes/scales [S, N, 256]/[S, N, 32]; idx int32
    [R, k]; swa uint8 [S, cap, 512].  swa_max: bound on every swa_len (0 =
    cap), e.g. 128 for prefill rows over one shared run of window tokens.
    Returns (out float32 [R, H, 512], lse float32 [R, H])."""
    for t, nm in ((q, "q"), (codes, "codes"), (scales, "scales"), (idx, "idx"), (swa, "swa"),
                  (swa_start, "swa_start"), (swa_len, "swa_len"), (row_seq, "row_seq")):
        _dev(t, nm)
    R, H = q.shape[0], q.shape[1]
    if out is None:
        out = torch.empty((R, H, LATENT_DIM), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((R, H), dtype=torch.float32, device=q.device)
    a = _attn_struct(q, codes, scales, idx, swa, swa_start, swa_len, row_seq, sm_scale, out, lse,
                     swa_max)
    L = lib()
    need = L.csa2_sparse_attn_workspace(ctypes.byref(a))
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    _check(L.csa2_sparse_attn_decode(ctypes.byref(a), _ptr(workspace),
                                     0 if workspace is None else workspace.numel(),
                                     _stream(stream)))
    return out, lse
