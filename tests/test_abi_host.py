"""Host-side checks of the C ABI (no GPU needed): the built library loads,
exports every function include/csa2.h declares, and its argument
validation rejects bad requests with the documented status before anything
touches the GPU."""

import ctypes
import os
import re

import pytest

from fp4_kv_cache_indexer_amd import csa2 as C

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "csa2.h")

needs_lib = pytest.mark.skipif(not os.path.exists(C._LIB_PATH), reason="libcsa2.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(csa2_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("csa2_kv_compress_quantize", "csa2_indexer_topk", "csa2_sparse_attn_decode",
                     "csa2_index_block_summary"):
        assert required in names
    assert sorted(C.EXPORTS) == names


@needs_lib
def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(C._LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name


@needs_lib
def test_version_and_status_strings():
    L = C.lib()
    assert C.abi_version() == 2
    assert C.status_string(0) == "ok"
    assert C.status_string(3) == "workspace too small"
    assert L.csa2_last_error() is not None


def _idx_args(**kw):
    a = C.IndexerArgs()
    a.n_rows = 2
    a.n_seq = 2
    a.n_ent = 4096
    a.top_k = 512
    a.q = ctypes.c_void_p(0x1000)
    a.keys = ctypes.c_void_p(0x2000)
    a.out_idx = ctypes.c_void_p(0x3000)
    a.keep_blocks = 2048
    for k, v in kw.items():
        setattr(a, k, v)
    return a


@needs_lib
def test_indexer_validation_without_gpu():
    L = C.lib()
    ws = ctypes.c_void_p(0x10000)
    # (fields, status, whether the size query -- which checks no pointers -- fails too)
    cb = dict(cand_blocks=ctypes.c_void_p(0x6000), n_cand_blocks=4)
    cases = [
        (dict(top_k=0), 2, True), (dict(top_k=4096), 2, True), (dict(q=None), 1, False),
        (dict(keys=ctypes.c_void_p(0x2001)), 1, False),
        (dict(block_keys=ctypes.c_void_p(0x4000), cand=ctypes.c_void_p(0x5000), n_cand=4), 1, True),
        (dict(block_keys=ctypes.c_void_p(0x4000), keep_blocks=0), 2, True),
        (dict(cand=ctypes.c_void_p(0x5000), n_cand=0), 1, True),
        (dict(n_ent=-1), 1, True), (dict(n_seq=-1), 1, True),
        (dict(cb, cand=ctypes.c_void_p(0x5000), n_cand=4), 1, True),
        (dict(cb, block_keys=ctypes.c_void_p(0x4000)), 1, True),
        (dict(cand_blocks=ctypes.c_void_p(0x6000), n_cand_blocks=0), 1, True),
        (dict(cand_blocks=ctypes.c_void_p(0x6002), n_cand_blocks=4), 1, False),
        (dict(key_format=7), 2, True),
        (dict(key_format=1), 1, False),                                  # FP4 without scales
        (dict(key_format=1, key_scales=ctypes.c_void_p(0x7002)), 1, False),
    ]
    for kw, status, ws_fails in cases:
        a = _idx_args(**kw)
        assert L.csa2_indexer_topk(ctypes.byref(a), ws, 1 << 30, None) == status, kw
        assert C.last_error() != ""
        assert (L.csa2_indexer_topk_workspace(ctypes.byref(a)) == 0) == ws_fails, kw
    # the size query needs no data pointers
    a = _idx_args(q=None, keys=None, out_idx=None)
    assert L.csa2_indexer_topk_workspace(ctypes.byref(a)) > 0
    # too small a workspace is refused before any launch
    a = _idx_args()
    need = L.csa2_indexer_topk_workspace(ctypes.byref(a))
    assert need >= 2 * 4096 * 4 + 2 * 4096 * 4
    assert L.csa2_indexer_topk(ctypes.byref(a), ws, need - 1, None) == 3
    # hierarchical workspace grows with the kept pool
    ah = _idx_args(block_keys=ctypes.c_void_p(0x4000))
    assert L.csa2_indexer_topk_workspace(ctypes.byref(ah)) > need
    # block-pool mode sizes its stage by 8 positions per block
    ab = _idx_args(cand_blocks=None, n_cand_blocks=300)
    assert L.csa2_indexer_topk_workspace(ctypes.byref(ab)) == need   # no blocks pointer: flat
    ab.cand_blocks = ctypes.c_void_p(0x6000)
    assert L.csa2_indexer_topk_workspace(ctypes.byref(ab)) > 0


@needs_lib
def test_static_indexer_refuses_oversized_requests_without_gpu():
    """csa2_indexer_topk_static validates like csa2_indexer_topk and refuses a
    request whose scratch exceeds the static array, before touching the GPU."""
    L = C.lib()
    a = _idx_args(q=None)
    assert L.csa2_indexer_topk_static(ctypes.byref(a), None) == 1
    big = _idx_args(n_rows=64, n_seq=64, n_ent=262144)
    assert L.csa2_indexer_topk_workspace(ctypes.byref(big)) > C.STATIC_SCRATCH_BYTES
    assert L.csa2_indexer_topk_static(ctypes.byref(big), None) == 3
    assert "static" in C.last_error()
    zero = _idx_args(n_rows=0)
    assert L.csa2_indexer_topk_static(ctypes.byref(zero), None) == 0


@needs_lib
def test_attn_and_cache_write_validation_without_gpu():
    L = C.lib()
    a = C.AttnArgs()
    a.n_rows, a.n_heads, a.top_k = 1, 48, 512
    assert L.csa2_sparse_attn_decode(ctypes.byref(a), None, 0, None) == 2
    a.n_heads = 64
    a.q_bf16 = ctypes.c_void_p(0x1000)
    a.out = ctypes.c_void_p(0x2000)
    assert L.csa2_sparse_attn_decode(ctypes.byref(a), None, 0, None) == 1   # idx/codes missing
    a.idx, a.codes, a.scales = ctypes.c_void_p(0x3000), ctypes.c_void_p(0x4000), ctypes.c_void_p(0x5000)
    a.swa_len, a.swa_cap = ctypes.c_void_p(0x6000), 0
    assert L.csa2_sparse_attn_decode(ctypes.byref(a), None, 0, None) == 1   # bad swa_cap
    a.swa_cap, a.swa = 128, ctypes.c_void_p(0x7000)
    need = L.csa2_sparse_attn_workspace(ctypes.byref(a))
    assert need > 0                                                         # one row -> key splits
    assert L.csa2_sparse_attn_decode(ctypes.byref(a), None, 0, None) == 3
    # swa_max bounds every window: outside [0, swa_cap] is rejected; with many
    # rows over one long shared window buffer it alone keeps each row in one
    # split (no partials to merge, so no workspace)
    for bad in (-1, 129):
        a.swa_max = bad
        assert L.csa2_sparse_attn_decode(ctypes.byref(a), None, 0, None) == 1
    a.n_rows, a.swa_cap, a.swa_max = 4096, 4223, 0
    assert L.csa2_sparse_attn_workspace(ctypes.byref(a)) > 0
    a.swa_max = 128
    assert L.csa2_sparse_attn_workspace(ctypes.byref(a)) == 0
    p = ctypes.c_void_p(0x1000)
    assert L.csa2_kv_compress_quantize(p, None, 1, 16, 3, 0, p, p, 0, None) == 2
    assert L.csa2_kv_compress_quantize(p, None, 1, 16, 2, 8, p, p, 0, None) == 1
    assert L.csa2_kv_compress_quantize(None, None, 1, 16, 2, 0, p, p, 0, None) == 1
    assert L.csa2_kv_compress_quantize(p, None, 0, 16, 2, 0, p, p, 0, None) == 0   # nothing to do
    assert L.csa2_index_block_summary(p, 1, 17, 0, 4, p, None) == 1               # 3 blocks only
    assert L.csa2_index_block_summary(p, 1, 17, 2, 2, p, None) == 0
    # FP4 index keys: sizes, strides and alignment are checked before any launch
    assert L.csa2_index_key_quantize(p, -1, 8, 0, p, p, 0, None) == 1
    assert L.csa2_index_key_quantize(p, 2, 8, 7, p, p, 0, None) == 1              # stride < n_ent
    assert L.csa2_index_key_quantize(None, 2, 8, 0, p, p, 0, None) == 1
    assert L.csa2_index_key_quantize(ctypes.c_void_p(0x1008), 2, 8, 0, p, p, 0, None) == 1
    assert L.csa2_index_key_quantize(None, 0, 8, 0, None, None, 0, None) == 0      # nothing to do
    assert L.csa2_index_block_summary_fp4(p, p, 1, 17, 0, 4, p, None) == 1         # 3 blocks only
    assert L.csa2_index_block_summary_fp4(None, p, 1, 17, 0, 3, p, None) == 1
    assert L.csa2_index_block_summary_fp4(p, p, 1, 17, 1, 1, p, None) == 0


@needs_lib
def test_decode_append_validation_without_gpu():
    L = C.lib()
    p = ctypes.c_void_p(0x1000)

    def args(**kw):
        a = C.AppendArgs()
        a.n_rows, a.n_seq, a.m, a.n_ent = 2, 2, 1, 64
        a.pos, a.x_bf16, a.codes, a.scales, a.key_bf16, a.keys = p, p, p, p, p, p
        for k, v in kw.items():
            setattr(a, k, v)
        return a

    cases = [
        (dict(m=3), 2), (dict(key_format=5), 2), (dict(n_rows=-1), 1), (dict(pos=None), 1),
        (dict(keys=None), 1), (dict(m=2), 1),                          # m > 1 needs pend_x
        (dict(codes=None), 1),                                          # window-only rows need swa
        (dict(m=2, pend_x=p, gate_bf16=p), 1),                          # a gate needs pend_gate
        (dict(key_format=1), 1),                                        # FP4 keys need key_scales
        (dict(swa=p, swa_cap=0), 1), (dict(x_bf16=ctypes.c_void_p(0x1008)), 1),
        (dict(codes=ctypes.c_void_p(0x1004)), 1),
    ]
    for kw, status in cases:
        a = args(**kw)
        assert L.csa2_decode_append(ctypes.byref(a), None) == status, kw
        assert C.last_error() != ""
    assert L.csa2_decode_append(ctypes.byref(args(n_rows=0, pos=None)), None) == 0   # nothing to do
    w = args(codes=None, swa=ctypes.c_void_p(0x2002), swa_cap=128)
    assert L.csa2_decode_append(ctypes.byref(w), None) == 1                          # swa misaligned


def test_attn_plan_override_without_gpu():
    """The plan override takes 0/16/64 heads per workgroup and 0..64 splits,
    refuses anything else, and changes the workspace the plan asks for."""
    L = C.lib()
    for hpw, ns in ((32, 0), (0, 65), (-16, 1), (16, -1)):
        assert L.csa2_attn_plan_override(hpw, ns) == 1, (hpw, ns)          # CSA2_EINVAL
    a = C.AttnArgs()
    a.n_rows, a.n_heads, a.n_seq, a.top_k, a.n_ent = 4, 64, 4, 512, 8192
    try:
        assert L.csa2_attn_plan_override(64, 1) == 0
        assert L.csa2_sparse_attn_workspace(ctypes.byref(a)) == 0        # one split: no partials
        assert L.csa2_attn_plan_override(64, 4) == 0
        ws4 = L.csa2_sparse_attn_workspace(ctypes.byref(a))
        assert ws4 >= 4 * 4 * 64 * 512 * 4                              # 4 splits of [R][H][512] float32
        assert L.csa2_attn_plan_override(16, 1) == 0                   # raised to the narrow kernel's least
        assert L.csa2_sparse_attn_workspace(ctypes.byref(a)) == 0       # 512 keys: one split still fits
    finally:
        assert L.csa2_attn_plan_override(0, 0) == 0


def test_indexer_workspace_passes_without_gpu():
    """One-stage calls whose score block would pass 512 MiB plan passes of at
    least 256 rows: 4096 rows over 524,288 entries fit in about 0.52 GB; small
    calls keep one pass; the candidate area appears only with the filter."""
    L = C.lib()

    def ws(R, N, **kw):
        a = C.IndexerArgs()
        a.n_rows, a.n_seq, a.n_ent, a.top_k, a.key_format = R, 1, N, 512, 0
        for name, v in kw.items():
            setattr(a, name, v)
        return L.csa2_indexer_topk_workspace(ctypes.byref(a))

    big = ws(4096, 524288)
    assert 256 * 524288 * 4 <= big < 1 << 30, big
    assert ws(4097, 524288) < 1 << 30
    assert ws(300, 6007) >= 300 * 6008 * 4                  # one pass
    few = ws(8, 1 << 20)                                      # filter path: candidate area
    assert few >= 8 * (1 << 20) * (4 + 8), few
    assert ws(256, 1 << 20) < 256 * (1 << 20) * 8            # long-row select: no candidate area


@needs_lib
def test_probe_validation_without_gpu():
    """The timing probes refuse bad sizes and pointers before any launch."""
    L = C.lib()
    p = ctypes.c_void_p(4096)                    # aligned, never dereferenced: validation fails first
    assert L.csa2_probe_scan_read(p, 8, 1024, 8, 1, 1, p, None) == 1          # chunk < 16
    assert L.csa2_probe_scan_read(None, 8, 1024, 256, 1, 1, p, None) == 1     # keys missing
    assert L.csa2_probe_scan_read(ctypes.c_void_p(4097), 8, 1024, 256, 1, 1, p, None) == 1   # misaligned
    assert L.csa2_probe_scan_read(p, 1 << 12, 1 << 24, 16, 1, 1, p, None) == 1   # > 2^20 workgroups
    assert L.csa2_probe_mfma_valu(5, 256, 16, 1, p, None) == 1                 # FMAs per MFMA not offered
    assert L.csa2_probe_mfma_valu(4, 128, 16, 1, p, None) == 1                 # 128 threads
    assert L.csa2_probe_mfma_valu(4, 256, 0, 1, p, None) == 1                  # no iterations
    assert L.csa2_probe_gather(p, p, 0, p, 4, 1, 1, p, None) == 1              # no entries
    assert L.csa2_probe_gather(p, None, 16, p, 4, 1, 1, p, None) == 1          # scales missing
    assert L.csa2_probe_gather(p, p, 16, p, 4, 70000, 1, p, None) == 1         # too many workgroups
    assert b"probe" in L.csa2_last_error()
