"""The C ABI library: loads without a GPU, exports every declared symbol, rejects bad arguments
on the host before any launch (these calls never reach a kernel)."""
import ctypes
import os
import re
import subprocess

import pytest

import dsa_lightning_indexer_02_amd as dsa
from dsa_lightning_indexer_02_amd._lib import Dims, PagedCache

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsa.h")

OK, INVALID, UNSUPPORTED, WS_SMALL = 0, 1, 2, 3
FAKE = 0x10000          # aligned, never dereferenced: every call below fails validation first


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(dsa.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return dsa.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dsa_[a-z_0-9]+)\s*\(", text)))


def test_exports_match_header(lib):
    decl = declared_functions()
    assert decl == sorted(dsa.EXPORTS)
    nm = subprocess.run(["nm", "-D", "--defined-only", dsa.LIB_PATH], capture_output=True, text=True,
                        check=True).stdout
    exported = set(re.findall(r" T (dsa_\w+)", nm))
    missing = [f for f in decl if f not in exported]
    assert not missing, missing
    for f in decl:
        assert hasattr(lib, f)


def test_version_and_strings(lib):
    assert lib.dsa_abi_version() == 2
    assert lib.dsa_status_string(3) == b"DSA_ERR_WORKSPACE_TOO_SMALL"


def _err(lib):
    return lib.dsa_last_error().decode()


def test_indexer_argument_errors(lib):
    f = lib.dsa_indexer_logits
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 8, 65, 128, 0, FAKE, 8, None) == UNSUPPORTED
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 8, 64, 100, 0, FAKE, 8, None) == UNSUPPORTED
    assert f(None, FAKE, FAKE, FAKE, FAKE, 4, 8, 64, 128, 0, FAKE, 8, None) == INVALID
    assert "q8" in _err(lib)
    assert f(FAKE + 4, FAKE, FAKE, FAKE, FAKE, 4, 8, 64, 128, 0, FAKE, 8, None) == INVALID
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 8, 64, 128, 0, FAKE, 6, None) == INVALID   # ld < S
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 10, 64, 128, 0, FAKE, 10, None) == INVALID  # ld % 4
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, -1, 8, 64, 128, 0, FAKE, 8, None) == INVALID
    assert f(None, None, None, None, None, 0, 8, 64, 128, 0, None, 8, None) == OK         # T = 0
    # more query rows than one launch's 16-row tiles cover on the grid's second dimension
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 16 * 65536 + 1, 8, 64, 128, 0, FAKE, 8, None) == UNSUPPORTED
    assert "query rows per call" in _err(lib)


def test_topk_argument_errors(lib):
    f = lib.dsa_topk
    assert f(FAKE, 8, 4, 8, 0, 0, FAKE, None, 0, None) == INVALID                     # k = 0
    need = lib.dsa_topk_workspace_size(4, 100000, 2048)
    assert need > 0 and lib.dsa_topk_workspace_size(4, 32768, 2048) == 0
    assert f(FAKE, 100000, 4, 100000, 0, 2048, FAKE, FAKE, need - 1, None) == WS_SMALL
    assert f(FAKE, 100000, 4, 100000, 0, 4096, FAKE, FAKE, 1 << 40, None) == UNSUPPORTED
    assert f(FAKE, 8, 4, 8, 0, 64, None, None, 0, None) == INVALID
    assert f(None, 8, 0, 8, 0, 64, None, None, 0, None) == OK


def test_mla_argument_errors(lib):
    f = lib.dsa_sparse_mla_fwd
    sm = ctypes.c_float(0.1)
    assert f(FAKE, FAKE, FAKE, 4, 8, 128, 512, 512, 64, 0, sm, FAKE, None, None, None, 0, None) == UNSUPPORTED
    assert f(FAKE, FAKE, FAKE, 4, 8, 129, 576, 512, 64, 0, sm, FAKE, None, None, None, 0, None) == UNSUPPORTED
    assert f(FAKE, FAKE, FAKE, 4, 8, 128, 576, 512, 0, 0, sm, FAKE, None, None, None, 0, None) == INVALID
    assert f(FAKE, FAKE, FAKE, 4, 8, 128, 576, 512, 64, 0, ctypes.c_float(0.0), FAKE, None, None, None, 0,
             None) == INVALID
    assert f(FAKE, FAKE, None, 4, 8, 128, 576, 512, 64, 0, sm, FAKE, None, None, None, 0, None) == INVALID
    assert f(FAKE, FAKE, FAKE, 4, 8, 128, 576, 512, 64, 0, sm, FAKE, FAKE + 8, None, None, 0, None) == INVALID
    # fp16 staging: the workspace holds the fp16 copy of the S latent rows (576/512 only)
    ws = lib.dsa_sparse_mla_workspace_size
    assert ws(4, 8, 128, 576, 512, 64) == 8 * 576 * 2
    assert ws(4, 9, 128, 576, 512, 64) == (9 * 576 * 2 + 255) // 256 * 256
    assert ws(4, 8, 128, 80, 64, 64) == 0 and ws(0, 8, 128, 576, 512, 64) == 0
    need = ws(4, 8, 128, 576, 512, 64)
    assert f(FAKE, FAKE, FAKE, 4, 8, 128, 576, 512, 64, 0, sm, FAKE, None, None, FAKE, need - 1, None) == WS_SMALL
    assert f(FAKE, FAKE, FAKE, 4, 8, 128, 576, 512, 64, 0, sm, FAKE, None, None, FAKE + 8, need, None) == INVALID
    assert "aligned" in _err(lib)


def test_fused_argument_errors(lib):
    d = Dims(64, 128, 128, 576, 512, 2048, 0.07)
    c = PagedCache(FAKE, FAKE, FAKE, 100, 64, FAKE, 100, FAKE)
    need = lib.dsa_prefill_workspace_size(ctypes.byref(d), 4096, 4096)
    assert need >= 4096 * 4096 * 4
    f = lib.dsa_prefill_paged
    args = [FAKE, FAKE, FAKE, FAKE, FAKE, None, None, None, FAKE]
    assert f(ctypes.byref(c), 0, ctypes.byref(d), 4096, 0, *args, need - 1, None) == WS_SMALL
    assert f(ctypes.byref(c), 0, ctypes.byref(d), 4096, 0, *args[:-1], FAKE + 16, need, None) == INVALID
    bad_bs = PagedCache(FAKE, FAKE, FAKE, 100, 48, FAKE, 100, FAKE)
    assert f(ctypes.byref(bad_bs), 0, ctypes.byref(d), 4096, 0, *args, need, None) == INVALID
    small_tbl = PagedCache(FAKE, FAKE, FAKE, 100, 64, FAKE, 10, FAKE)
    assert f(ctypes.byref(small_tbl), 0, ctypes.byref(d), 4096, 0, *args, need, None) == INVALID
    d_bad = Dims(64, 128, 128, 576, 512, 4096, 0.07)
    assert f(ctypes.byref(c), 0, ctypes.byref(d_bad), 4096, 0, *args, need, None) == UNSUPPORTED
    assert f(ctypes.byref(c), 0, ctypes.byref(d), 0, 0, *args, 0, None) == OK
    g = lib.dsa_decode_paged
    need_d = lib.dsa_decode_workspace_size(ctypes.byref(d), 64, 131072)
    assert need_d > 64 * 131072 * 4
    no_lens = PagedCache(FAKE, FAKE, FAKE, 100000, 64, FAKE, 2048, None)
    assert g(ctypes.byref(no_lens), 64, 131072, ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, None, None,
             None, FAKE, need_d, None) == INVALID
    c2 = PagedCache(FAKE, FAKE, FAKE, 100000, 64, FAKE, 2048, FAKE)
    assert g(ctypes.byref(c2), 64, 131072, ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, None, None, None,
             FAKE, need_d - 1, None) == WS_SMALL
    assert g(ctypes.byref(c2), 0, 131072, ctypes.byref(d), None, None, None, None, None, None, None, None,
             None, 0, None) == OK
    # the decode batch cap follows the indexer's LDS prefix table (12288 sequences)
    assert g(ctypes.byref(c2), 12289, 131072, ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, None, None, None,
             FAKE, 1 << 40, None) == UNSUPPORTED
    assert "12288" in _err(lib)
    hdr = open(os.path.join(ROOT, "include", "dsa.h")).read()
    assert "B <= 12288" in hdr


def test_quantize_and_append_argument_errors(lib):
    f = lib.dsa_quantize_fp8_rows
    assert f(FAKE, 10, 12, FAKE, FAKE, None) == UNSUPPORTED          # D not a multiple of 8
    assert f(FAKE, 10, 1024, FAKE, FAKE, None) == UNSUPPORTED
    assert f(None, 10, 128, FAKE, FAKE, None) == INVALID
    assert f(FAKE, 10, 128, FAKE + 8, FAKE, None) == INVALID          # misaligned codes
    assert f(None, 0, 128, None, None, None) == OK                    # nothing to do
    g = lib.dsa_append_paged
    c = PagedCache(FAKE, FAKE, FAKE, 100, 64, FAKE, 4, None)
    assert g(ctypes.byref(c), 2, FAKE, FAKE, 5, 100, 576, FAKE, FAKE, None) == UNSUPPORTED   # D_I
    assert g(ctypes.byref(c), 2, FAKE, FAKE, 5, 128, 570, FAKE, FAKE, None) == UNSUPPORTED   # D_qk
    assert g(ctypes.byref(c), 2, None, FAKE, 5, 128, 576, FAKE, FAKE, None) == INVALID
    bad_bs = PagedCache(FAKE, FAKE, FAKE, 100, 48, FAKE, 4, None)
    assert g(ctypes.byref(bad_bs), 2, FAKE, FAKE, 5, 128, 576, FAKE, FAKE, None) == INVALID
    assert g(ctypes.byref(c), 0, FAKE, FAKE, 5, 128, 576, FAKE, FAKE, None) == INVALID       # tokens, no sequences
    assert g(None, 0, None, None, 0, 128, 576, None, None, None) == OK


def test_kl_loss_and_backward_argument_errors(lib):
    f = lib.dsa_indexer_kl_loss
    sm = ctypes.c_float(0.07)
    assert f(FAKE, FAKE, 4, 8, 129, 576, sm, 0, FAKE, 8, FAKE, FAKE, None) == UNSUPPORTED   # H > 128
    assert f(FAKE, FAKE, 4, 8, 128, 580, sm, 0, FAKE, 8, FAKE, FAKE, None) == UNSUPPORTED   # D_qk
    assert f(FAKE, FAKE, 4, 8, 128, 576, sm, 0, FAKE, 6, FAKE, FAKE, None) == INVALID       # ld < S
    assert f(FAKE, FAKE, 4, 0, 128, 576, sm, 0, FAKE, 8, FAKE, FAKE, None) == INVALID       # no keys
    assert f(FAKE, FAKE, 4, 8, 128, 576, ctypes.c_float(0.0), 0, FAKE, 8, FAKE, FAKE, None) == INVALID
    assert f(FAKE, FAKE, 4, 8, 128, 576, sm, 0, FAKE, 8, FAKE, None, None) == INVALID       # loss
    assert "loss" in _err(lib)
    assert f(None, None, 0, 8, 128, 576, sm, 0, None, 8, None, None, None) == OK            # T = 0
    g = lib.dsa_indexer_bwd
    need = lib.dsa_indexer_bwd_workspace_size(64, 64, 128)
    assert need > 0 and lib.dsa_indexer_bwd_workspace_size(0, 64, 128) == 0
    args = [FAKE, FAKE, FAKE, FAKE, FAKE, 64, 64, 64, 128, 0, FAKE, 64, FAKE, FAKE, FAKE, FAKE, need, None]
    bad = list(args)
    bad[8] = 100                                                                            # D_I
    assert g(*bad) == UNSUPPORTED
    bad = list(args)
    bad[16] = need - 1
    assert g(*bad) == WS_SMALL
    bad = list(args)
    bad[14] = None                                                                          # dk
    assert g(*bad) == INVALID
    bad = list(args)
    bad[5] = 0                                                                              # T = 0, S > 0
    assert g(*bad) == INVALID
    bad = list(args)
    bad[11] = 66                                                                            # ld % 4
    assert g(*bad) == INVALID
    assert g(None, None, None, None, None, 0, 0, 64, 128, 0, None, 4, None, None, None, None, 0, None) == OK
    h = lib.dsa_indexer_bwd_listed
    largs = args[:10] + [FAKE, 2048] + args[10:]
    assert len(largs) == 20
    bad = list(largs)
    bad[11] = 0                                                                             # k
    assert h(*bad) == INVALID
    bad = list(largs)
    bad[10] = None                                                                          # indices
    assert h(*bad) == INVALID
    assert "indices" in _err(lib)
    bad = list(largs)
    bad[18] = need - 1
    assert h(*bad) == WS_SMALL
    bad = list(largs)
    bad[8] = 100                                                                            # D_I
    assert h(*bad) == UNSUPPORTED
    assert h(None, None, None, None, None, 0, 0, 64, 128, 0, None, 16, None, 4, None, None, None, None, 0,
             None) == OK


def test_kl_sparse_argument_errors(lib):
    f = lib.dsa_indexer_kl_loss_sparse
    sm = ctypes.c_float(0.07)
    assert f(FAKE, FAKE, FAKE, 4096, FAKE, 4, 8, 128, 576, sm, 0, FAKE, 8, FAKE, FAKE, None) == UNSUPPORTED   # k
    assert f(FAKE, FAKE, FAKE, 64, None, 4, 8, 128, 576, sm, 0, FAKE, 8, FAKE, FAKE, None) == INVALID         # lse
    assert "lse" in _err(lib)
    assert f(FAKE, FAKE, None, 64, FAKE, 4, 8, 128, 576, sm, 0, FAKE, 8, FAKE, FAKE, None) == INVALID         # indices
    assert f(None, None, None, 64, None, 0, 8, 128, 576, sm, 0, None, 8, None, None, None) == OK              # T = 0


def test_profile_events_host_side(lib):
    # no recording active: end reports nothing; begin refuses a NULL array or an empty capacity
    assert lib.dsa_profile_end() == 0
    assert lib.dsa_profile_begin(None, 4) == INVALID
    assert lib.dsa_profile_begin(FAKE, 0) == INVALID
    assert lib.dsa_profile_kernel_name(0) == b"" and lib.dsa_profile_kernel_name(-1) == b""
    # begin / end without a launch in between records nothing (no event is touched)
    assert lib.dsa_profile_begin(FAKE, 4) == OK
    assert lib.dsa_profile_end() == 0


def test_topk_noalloc_rejects_on_the_host(lib):
    # 600 rows of 131072 scores need 600 * 4 chunks * 2048 * 8 bytes of candidates, above the
    # 32 MiB array: refused before any device call (this runs without a GPU)
    assert lib.dsa_topk_noalloc(FAKE, 131072, 600, 131072, 0, 2048, FAKE, None) == UNSUPPORTED
    assert "scratch" in _err(lib)
    assert lib.dsa_topk_noalloc(FAKE, 131072, 4, 131072, 0, 0, FAKE, None) == INVALID     # k
    assert lib.dsa_topk_noalloc(None, 8, 0, 8, 0, 16, None, None) == OK                   # T = 0
    assert dsa.TOPK_NOALLOC_SCRATCH_BYTES == 32 << 20
    assert "DSA_TOPK_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)" in open(HEADER).read()


def test_sparse_mla_bwd_argument_errors(lib):
    f = lib.dsa_sparse_mla_bwd
    sm = ctypes.c_float(0.07)
    need = lib.dsa_sparse_mla_bwd_workspace_size(8, 100, 128, 2048)
    # chunk buffers: fp16 ds / p tiles, fp32 contributions, the key map
    assert need == 8 * 2 * 128 * 2048 * 2 + 8 * 2048 * 576 * 4 + (100 * 8 * 4 + 255) // 256 * 256
    assert lib.dsa_sparse_mla_bwd_workspace_size(0, 100, 128, 2048) == 0
    big = lib.dsa_sparse_mla_bwd_workspace_size(100000, 131072, 64, 2047)   # 512-row chunks, heads to 64
    assert big == 512 * 2 * 64 * 2048 * 2 + 512 * 2048 * 576 * 4 + 131072 * 512 * 4
    args = [FAKE, FAKE, FAKE, FAKE, FAKE, 8, 100, 128, 576, 512, 2048, 0, sm, FAKE, FAKE, FAKE, need, None]
    bad = list(args)
    bad[8] = 80                                                    # D_qk (only 576 / 512 is built)
    assert f(*bad) == UNSUPPORTED
    bad = list(args)
    bad[7] = 129                                                   # H
    assert f(*bad) == UNSUPPORTED
    bad = list(args)
    bad[16] = need - 1
    assert f(*bad) == WS_SMALL
    bad = list(args)
    bad[3] = None                                                  # lse
    assert f(*bad) == INVALID
    assert "lse" in _err(lib)
    bad = list(args)
    bad[12] = ctypes.c_float(0.0)                                  # sm_scale
    assert f(*bad) == INVALID
    bad = list(args)
    bad[10] = 0                                                    # k
    assert f(*bad) == INVALID
    assert f(None, None, None, None, None, 0, 0, 128, 576, 512, 16, 0, sm, None, None, None, 0, None) == OK

