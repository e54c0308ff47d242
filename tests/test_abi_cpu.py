"""The C-ABI library loads, exports every function of include/qsa.h, and rejects bad
arguments on the host before launching anything (no GPU needed)."""
import ctypes
import os

import pytest

from block_sparse_attention_06_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        from block_sparse_attention_06_amd import build
        build.build()
    return _lib.load()


def test_every_header_function_is_exported_and_declared(lib):
    names = _lib.header_functions()
    assert len(names) >= 13
    assert sorted(_lib.SIGNATURES) == names
    for n in names:
        assert hasattr(lib, n), n
    assert lib.qsa_abi_version() == 3


def test_probe_library_is_separate():
    # The benchmark's probes live in their own library and header; libqsa.so exports
    # only the QSA calls.
    from block_sparse_attention_06_amd import probe
    if not os.path.exists(probe.PROBE_LIB_PATH):
        from block_sparse_attention_06_amd import build
        build.build()
    assert _lib.header_functions(probe.HEADER_PATH) == sorted(probe.SIGNATURES)
    plib = probe.load()
    qlib = _lib.load()
    for name in ("qsa_probe_gather", "qsa_probe_write"):
        assert hasattr(plib, name)
        assert not hasattr(qlib, name)
    assert plib.qsa_probe_gather(None, 4096, None, 1, 1, None, None) == 1
    assert plib.qsa_probe_write(None, 4096, 0, None) == 1
    # rejected on the host before any launch: a misaligned pointer, a ragged size
    assert plib.qsa_probe_write(8, 4096, 0, None) == 1
    assert plib.qsa_probe_write(16, 4095, 0, None) == 1


P = ctypes.c_void_p
FAKE = P(0x1000)       # 16-byte aligned, never dereferenced: calls fail validation first
MISALIGNED = P(0x1004)


def _err(lib):
    return lib.qsa_last_error().decode()


def test_pool_validation(lib):
    assert lib.qsa_pool_keys(FAKE, 128, 10, 128, 3, FAKE, 128, None) == 2
    assert "r=3" in _err(lib)
    assert lib.qsa_pool_keys(None, 128, 10, 128, 4, FAKE, 128, None) == 1
    assert lib.qsa_pool_keys(MISALIGNED, 128, 10, 128, 4, FAKE, 128, None) == 1
    assert "aligned" in _err(lib)
    assert lib.qsa_pool_keys(FAKE, 64, 10, 128, 4, FAKE, 128, None) == 1  # stride < d
    assert lib.qsa_pool_keys(FAKE, 128, 0, 128, 4, FAKE, 128, None) == 0  # nothing to do


def test_scores_validation(lib):
    args = dict(batch=1, lq=64, h=4, di=128, r=4, q=FAKE, qbs=0, w=FAKE, wbs=0, kp=FAKE, kbs=0,
                nblk=100, pos0=0, sl=None, s=FAKE, ld=100, sbs=0)

    def call(**kw):
        a = {**args, **kw}
        return lib.qsa_index_scores(a["batch"], a["lq"], a["h"], a["di"], a["r"], a["q"],
                                    a["qbs"], a["w"], a["wbs"], a["kp"], a["kbs"], a["nblk"],
                                    a["pos0"], a["sl"], a["s"], a["ld"], a["sbs"], None)

    assert call(h=5) == 2
    assert call(di=96) == 2
    assert call(ld=98) == 1          # ld < nblk
    assert call(ld=102) == 1         # ld % 4 != 0
    assert call(pos0=-1) == 1
    assert call(q=None) == 1
    assert call(s=MISALIGNED) == 1
    assert call(lq=0) == 0


def test_topk_and_attention_validation(lib):
    assert lib.qsa_topk_blocks(1, 10, 4, 2050, FAKE, 100, 0, 100, 0, None, FAKE, None, 0,
                               None) == 1  # budget % r
    assert lib.qsa_topk_blocks(1, 10, 4, 8, FAKE, 100, 0, 100, 0, None, FAKE, None, 0,
                               None) == 2  # 2 blocks < 4
    assert lib.qsa_topk_blocks(1, 10, 4, 8192, FAKE, 100, 0, 100, 0, None, FAKE, None, 0,
                               None) == 2  # 2048 blocks > 1024
    assert lib.qsa_sparse_attn_fwd(10, 100, 24, 5, 256, 4, 512, FAKE, FAKE, FAKE, FAKE, 0,
                                   ctypes.c_float(0.1), FAKE, None, None) == 1  # 24 % 5
    assert lib.qsa_sparse_attn_fwd(10, 100, 34, 2, 256, 4, 512, FAKE, FAKE, FAKE, FAKE, 0,
                                   ctypes.c_float(0.1), FAKE, None, None) == 2  # 17 per group
    assert lib.qsa_sparse_attn_fwd(10, 100, 24, 2, 192, 4, 512, FAKE, FAKE, FAKE, FAKE, 0,
                                   ctypes.c_float(0.1), FAKE, None, None) == 2  # d=192
    assert lib.qsa_sparse_attn_fwd(10, 100, 24, 2, 256, 4, 512, FAKE, FAKE, FAKE, FAKE, 95,
                                   ctypes.c_float(0.1), FAKE, None, None) == 1  # rows past Lk
    assert lib.qsa_sparse_attn_fwd(10, 100, 24, 2, 256, 4, 512, FAKE, FAKE, FAKE, FAKE, 0,
                                   ctypes.c_float(float("nan")), FAKE, None, None) == 1


def test_tiled_attention_validation(lib):
    f = ctypes.c_float(0.1)
    # the shared checks of the per-row entry point
    assert lib.qsa_sparse_attn_fwd_tiled(10, 100, 24, 5, 256, 4, 512, FAKE, FAKE, FAKE, FAKE, 0,
                                         f, 0, FAKE, None, None) == 1  # 24 % 5
    assert lib.qsa_sparse_attn_fwd_tiled(10, 100, 24, 2, 256, 4, 512, FAKE, FAKE, FAKE, FAKE, 95,
                                         f, 0, FAKE, None, None) == 1  # rows past Lk
    # kept lists beyond the tile's LDS (512 blocks), and a bad sharing threshold
    assert lib.qsa_sparse_attn_fwd_tiled(10, 100, 24, 2, 256, 4, 513, FAKE, FAKE, FAKE, FAKE, 0,
                                         f, 0, FAKE, None, None) == 2
    assert lib.qsa_sparse_attn_fwd_tiled(10, 100, 24, 2, 256, 4, 512, FAKE, FAKE, FAKE, FAKE, 0,
                                         f, 66, FAKE, None, None) == 1
    assert lib.qsa_sparse_attn_fwd_tiled(10, 100, 24, 2, 256, 4, 512, FAKE, FAKE, FAKE, FAKE, 0,
                                         f, -1, FAKE, None, None) == 1
    assert lib.qsa_sparse_attn_fwd_tiled(0, 100, 24, 2, 256, 4, 512, None, None, None, None, 0,
                                         f, 65, None, None, None) == 0  # nothing to do


def test_attention_rows_per_launch_query(lib):
    assert lib.qsa_sparse_attn_fwd_rows_per_launch(2, 192) == 0   # d unsupported
    assert lib.qsa_sparse_attn_fwd_rows_per_launch(0, 256) == 0
    n = lib.qsa_sparse_attn_fwd_rows_per_launch(2, 256)
    assert n == -1 or n >= 2                                       # -1: no device to ask


def test_workspace_queries_and_short_workspace(lib):
    # 512 kept blocks = 128 steps of 4: 64 waves of 2 steps, merged 4 per workgroup,
    # so 16 (o[256], m, l) fp32 partials per (sequence, head)
    n = lib.qsa_sparse_attn_decode_workspace_bytes(8, 24, 256, 512)
    assert n >= 8 * 24 * 16 * 258 * 4
    assert lib.qsa_sparse_attn_decode(8, 24, 2, 256, 4, 512, FAKE, FAKE, FAKE, 1 << 29, 1 << 20,
                                      FAKE, FAKE, ctypes.c_float(0.06), FAKE, None, FAKE, n - 1,
                                      None) == 3
    assert "workspace" in _err(lib)
    p = lib.qsa_prefill_workspace_bytes(131072, 131072, 4, 2048, 4096)
    assert p >= 4096 * 32768 * 4
    d = lib.qsa_decode_workspace_bytes(8, 24, 256, 1 << 20, 4, 2048)
    assert d >= 8 * 262144 * 4 + n
    assert lib.qsa_topk_workspace_bytes(1, 10, 10, 2048, 4) == 0
    assert lib.qsa_topk_workspace_bytes(1, 10, 32768, 2048, 4) == 0
    # rows longer than one workgroup's 32768 candidates use a two-level selection:
    # 8 rows x 256 segments x 16 kept (value, id) pairs plus one boundary per segment
    assert lib.qsa_topk_workspace_bytes(8, 1, 262144, 2048, 4) >= 8 * 256 * (16 + 1) * 8


def test_backward_validation_and_workspace(lib):
    f = ctypes.c_float(0.0625)

    def bwd(lq=10, lk=100, hq=24, hkv=2, d=256, r=4, n_sel=512, q=FAKE, k=FAKE, v=FAKE,
            sel=FAKE, pos0=0, scale=f, out=FAKE, lse=FAKE, dout=FAKE, dq=FAKE, dk=FAKE, dv=FAKE,
            ws=FAKE, ws_bytes=1 << 40):
        return lib.qsa_sparse_attn_bwd(lq, lk, hq, hkv, d, r, n_sel, q, k, v, sel, pos0, scale,
                                       out, lse, dout, dq, dk, dv, ws, ws_bytes, None)

    assert bwd(hkv=5) == 1                        # 24 % 5
    assert bwd(d=192) == 2
    assert bwd(r=3) == 2
    assert bwd(n_sel=2048) == 2
    assert bwd(pos0=95) == 1                      # rows past Lk
    assert bwd(scale=ctypes.c_float(float("inf"))) == 1
    assert bwd(lse=None) == 1 and "null" in _err(lib)
    assert bwd(dout=None) == 1
    assert bwd(dk=MISALIGNED) == 1 and "aligned" in _err(lib)
    assert bwd(lq=1 << 22, lk=1 << 23, n_sel=1024) == 1  # lq * n_sel >= 2^31
    n = lib.qsa_sparse_attn_bwd_workspace_bytes(10, 100, 24, 4, 512)
    # D [lq][hq] fp32, four int32 arrays of lq * n_sel (block, row) pairs, 26 block starts
    assert n >= 10 * 24 * 4 + 4 * 10 * 512 * 4 + 26 * 4
    assert bwd(ws_bytes=n - 1) == 3 and "workspace" in _err(lib)
    assert bwd(ws=MISALIGNED) == 3


def test_warmup_validation(lib):
    f = ctypes.c_float(0.0625)
    # target: heads per group, head dim, positions, ld
    assert lib.qsa_indexer_kl_target(10, 100, 24, 5, 256, 4, FAKE, FAKE, 0, f, FAKE, FAKE, 28,
                                     None) == 1
    assert lib.qsa_indexer_kl_target(10, 100, 24, 2, 192, 4, FAKE, FAKE, 0, f, FAKE, FAKE, 28,
                                     None) == 2
    assert lib.qsa_indexer_kl_target(10, 100, 24, 6, 256, 4, FAKE, FAKE, 0, f, FAKE, FAKE, 28,
                                     None) == 2 and "hkv" in _err(lib)  # > 4 KV groups
    assert lib.qsa_indexer_kl_target(10, 100, 24, 2, 256, 4, FAKE, FAKE, 95, f, FAKE, FAKE, 28,
                                     None) == 1
    assert lib.qsa_indexer_kl_target(10, 100, 24, 2, 256, 4, FAKE, FAKE, 0, f, FAKE, FAKE, 24,
                                     None) == 1 and "ld" in _err(lib)  # ld < lk / r
    assert lib.qsa_indexer_kl_target(10, 100, 24, 2, 256, 4, FAKE, FAKE, 0, f, None, FAKE, 28,
                                     None) == 1
    assert lib.qsa_indexer_kl_target(0, 100, 24, 2, 256, 4, None, None, 0, f, None, None, 28,
                                     None) == 0  # nothing to do
    # loss: ld, null pointers
    assert lib.qsa_indexer_kl_loss(10, 25, 4, 0, FAKE, FAKE, 26, FAKE, FAKE, None) == 1
    assert lib.qsa_indexer_kl_loss(10, 25, 4, 0, FAKE, None, 28, FAKE, FAKE, None) == 1
    assert lib.qsa_indexer_kl_loss(10, 25, 3, 0, FAKE, FAKE, 28, FAKE, FAKE, None) == 2
    # indexer backward: heads, dims, alignment
    assert lib.qsa_index_scores_bwd(10, 5, 128, 4, FAKE, FAKE, FAKE, 25, 0, FAKE, 28, FAKE,
                                    FAKE, FAKE, None, 0, None) == 2
    assert lib.qsa_index_scores_bwd(10, 4, 96, 4, FAKE, FAKE, FAKE, 25, 0, FAKE, 28, FAKE,
                                    FAKE, FAKE, None, 0, None) == 2
    assert lib.qsa_index_scores_bwd(10, 4, 128, 4, FAKE, FAKE, FAKE, 25, 0, MISALIGNED, 28,
                                    FAKE, FAKE, FAKE, None, 0, None) == 1
    assert lib.qsa_index_scores_bwd(10, 4, 128, 4, FAKE, FAKE, FAKE, 25, 0, FAKE, 22, FAKE,
                                    FAKE, FAKE, None, 0, None) == 1  # ld < nblk


def test_varlen_validation_and_workspace(lib):
    f = ctypes.c_float(0.0625)

    def sel_call(batch=2, cu_q=FAKE, cu_k=FAKE, max_lq=100, max_lk=200, h=4, di=128, r=4,
                 budget=256, ws_bytes=1 << 40, kp=FAKE):
        return lib.qsa_prefill_varlen_select(batch, cu_q, cu_k, max_lq, max_lk, h, di, r, budget,
                                             FAKE, FAKE, FAKE, kp, FAKE, 64, FAKE, ws_bytes, None,
                                             None)

    assert sel_call(batch=0) == 1
    assert sel_call(cu_q=None) == 1 and "cu_seqlens" in _err(lib)
    assert sel_call(max_lq=300) == 1                   # max_lq > max_lk
    assert sel_call(r=3) == 2
    assert sel_call(h=5) == 2
    assert sel_call(budget=258) == 1
    assert sel_call(kp=MISALIGNED) == 1 and "aligned" in _err(lib)
    assert sel_call(max_lk=1 << 24) == 2               # 2^22 blocks and more
    need = lib.qsa_prefill_varlen_workspace_bytes(2, 100, 200, 4, 256, 64)
    # two sequences x 64 rows of 50 block scores (ld 52), fp32
    assert need >= 2 * 64 * 52 * 4
    assert sel_call(ws_bytes=need - 1) == 3 and "workspace" in _err(lib)

    def attn_call(batch=2, total_q=100, hq=24, hkv=2, d=256, n_sel=64, scale=f, out=FAKE,
                  max_lk=0):
        return lib.qsa_sparse_attn_varlen_fwd(batch, FAKE, FAKE, total_q, max_lk, hq, hkv, d, 4,
                                              n_sel, FAKE, FAKE, FAKE, FAKE, scale, out, None,
                                              None)

    assert attn_call(hkv=5) == 1
    assert attn_call(d=192) == 2
    assert attn_call(n_sel=2048) == 2
    assert attn_call(total_q=-1) == 1
    assert attn_call(scale=ctypes.c_float(float("nan"))) == 1
    assert attn_call(out=MISALIGNED) == 1
    assert attn_call(max_lk=-1) == 1
    assert attn_call(total_q=0) == 0                   # nothing to do


def test_attention_launch_count_query(lib):
    # Unsupported arguments are -1; no rows are no launches. (With no GPU the occupancy
    # is unknown and every row goes in one launch per KV-group pass.)
    assert lib.qsa_sparse_attn_fwd_launches(10, 100, 0, 256) == -1
    assert lib.qsa_sparse_attn_fwd_launches(10, 100, 2, 192) == -1
    assert lib.qsa_sparse_attn_fwd_launches(0, 100, 2, 256) == 0
    assert lib.qsa_sparse_attn_fwd_launches(10, 100, 2, 256) >= 1


def test_pooled_key_encoding_validation(lib):
    from block_sparse_attention_06_amd.ops import _PooledPe

    def pool(rope_dim, theta, d=128, first=0):
        st = _PooledPe(rope_dim, theta)
        return lib.qsa_pool_keys_pe(FAKE, d, 10, d, 4, first, ctypes.byref(st), FAKE, d, None)

    assert pool(24, 1e4) == 2 and "rope_dim" in _err(lib)    # not a multiple of 16
    assert pool(256, 1e4) == 2                                # wider than d_idx
    assert pool(64, 1.0) == 1 and "rope_theta" in _err(lib)
    assert pool(64, float("inf")) == 1
    assert pool(64, 1e4, first=-1) == 1
    assert pool(64, 1e4, d=60) == 2                           # d_idx not a multiple of 8
    st = _PooledPe(64, 1e4)
    assert lib.qsa_pool_keys_pe(FAKE, 128, 0, 128, 4, 0, ctypes.byref(st), FAKE, 128, None) == 0
    # the whole-path drivers check the encoding before launching anything
    bad = _PooledPe(20, 1e4)
    assert lib.qsa_prefill_select(64, 64, 0, 4, 128, 4, 256, FAKE, FAKE, FAKE, 0, None, FAKE,
                                  FAKE, 64, FAKE, 1 << 40, ctypes.byref(bad), None) == 2


def test_decode_noalloc_rejects_sizes_beyond_its_scratch(lib):
    # The allocation-free decode step checks its workspace need against the static
    # scratch on the host and returns QSA_ERR_WORKSPACE (3) before anything else.
    args = (4, 24, 2, 256, 4, 128, 4, 2048, FAKE, FAKE, FAKE, FAKE, 0, FAKE, FAKE, 0)
    tail = (FAKE, ctypes.c_float(0.0625), FAKE, FAKE, None, None)
    big = lib.qsa_decode_forward_noalloc(64, *args[1:], 1 << 20, *tail)
    assert big == 3 and "scratch" in _err(lib)
    assert lib.qsa_decode_workspace_bytes(64, 24, 256, 1 << 20, 4, 2048) > 32 << 20
    # within the limit it gets past the size check (here to argument validation)
    assert lib.qsa_decode_workspace_bytes(8, 24, 256, 1 << 20, 4, 2048) <= 32 << 20
    stride = (1 << 20) * 2 * 256
    assert lib.qsa_decode_forward_noalloc(8, 24, 2, 256, 4, 128, 3, 2048, FAKE, FAKE, FAKE, FAKE,
                                          (1 << 18) * 128, FAKE, FAKE, stride, 1 << 20,
                                          *tail) == 2  # r = 3
    assert "r=3" in _err(lib)



def test_fused_selection_validation(lib):
    from block_sparse_attention_06_amd.ops import _FusedTuning

    def call(lq=64, lk=64, tuning=None, ws_bytes=1 << 40, budget=256):
        tp = None if tuning is None else ctypes.byref(tuning)
        return lib.qsa_prefill_select_fused(lq, lk, 0, 4, 128, 4, budget, FAKE, FAKE, FAKE, 0,
                                            None, FAKE, FAKE, 64, FAKE, ws_bytes, None, tp, None)

    assert call(tuning=_FusedTuning(0, 0, 4096)) == 2 and "cap" in _err(lib)
    assert call(lk=4 << 24) == 2 and "2^24" in _err(lib)
    assert call(budget=258) == 1
    need = lib.qsa_prefill_fused_workspace_bytes(64, 64, 4, 256, 64)
    # one chunk of scores, lists of 2048 entries per row and piece, counts, flags
    assert need >= 64 * 16 * 4 + 64 * 2048 * 8
    assert call(ws_bytes=need - 1) == 3 and "workspace" in _err(lib)
    assert lib.qsa_prefill_fused_workspace_bytes(0, 64, 4, 256, 64) == 0


def test_binding_defaults_for_the_selection():
    # Host logic of the binding: the default selection chunk keeps its fp32 score rows
    # within 8 GiB (65536 rows at 128K, 8192 at 1M, whole short prefills), and the fused
    # selection is the default above 16384 blocks.
    from block_sparse_attention_06_amd import ops
    assert ops.default_row_chunk(131072, 131072) == 65536
    assert ops.default_row_chunk(8192, 1048576) == 8192
    assert ops.default_row_chunk(32768, 32768) == 32768
    assert ops.default_row_chunk(100, 100) == 100
    assert ops.default_row_chunk(1 << 20, 1 << 22) == 4096  # never below 4096 rows
    for lq, lk in ((131072, 131072), (8192, 1048576), (70000, 1 << 22)):
        rc = ops.default_row_chunk(lq, lk)
        assert rc * ops.score_ld(lk // 4) * 4 <= max(ops.SCORE_CHUNK_BYTES, 4096 * ops.score_ld(lk // 4) * 4)
    assert not ops.prefer_fused_select(32768 * 2)    # 16384 blocks: the two-kernel path
    assert ops.prefer_fused_select(131072)           # 32768 blocks: fused
