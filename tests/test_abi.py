"""The C-ABI library loads, exports every symbol include/attn.h declares, and rejects bad
arguments on the host before any HIP call (CPU only: no kernel is launched here)."""
import ctypes
import os
import re

import pytest

from attention_forward_03_amd import _lib
import attention_forward_03_amd as attn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "attn.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = _declared_functions()
    assert names == sorted(_lib.EXPORTED)


def test_library_exports_every_declared_symbol():
    L = _lib.lib()
    for name in _declared_functions():
        assert hasattr(L, name), name
    assert L.attn_abi_version() == 100


def test_library_links_no_vendor_kernel_libraries():
    # the hot path is hand-written: no BLAS / CK / MIOpen / Triton dependency
    import subprocess
    out = subprocess.run(["ldd", _lib.LIB_PATH], capture_output=True, text=True).stdout
    for bad in ("rocblas", "hipblaslt", "MIOpen", "composable", "triton", "torch"):
        assert bad.lower() not in out.lower(), bad


def test_status_strings():
    L = _lib.lib()
    assert L.attn_status_string(0) == b"ATTN_SUCCESS"
    assert L.attn_status_string(3) == b"ATTN_ERROR_WORKSPACE_TOO_SMALL"
    assert L.attn_status_string(99) == b"ATTN_STATUS_UNKNOWN"


def _fwd_args(**kw):
    a = _lib.FwdArgs()
    base = dict(batch=2, num_q_heads=4, num_kv_heads=4, seqlen_q=64, seqlen_k=64, head_dim=32,
                dtype=_lib.ATTN_F32, causal=0, window=0, softmax_scale=0.0, softcap=0.0)
    base.update(kw)
    for k, v in base.items():
        setattr(a, k, v)
    for name in ("q_stride", "k_stride", "v_stride", "o_stride"):
        arr = getattr(a, name)
        st = kw.get(name, (4 * 64 * 32, 64 * 32, 32))
        for i in range(3):
            arr[i] = st[i]
    return a


FAKE = 0x10000  # never dereferenced: every case below fails validation first


@pytest.mark.parametrize("kw,status", [
    (dict(batch=0), _lib.ATTN_ERROR_INVALID_VALUE),
    (dict(num_q_heads=6, num_kv_heads=4), _lib.ATTN_ERROR_INVALID_VALUE),
    (dict(head_dim=96), _lib.ATTN_ERROR_NOT_SUPPORTED),           # fp32: 32, 64, 128 only
    (dict(head_dim=96, dtype=_lib.ATTN_BF16, q_stride=(8192, 2048, 96), k_stride=(8192, 2048, 96),
          v_stride=(8192, 2048, 96), o_stride=(8192, 2048, 96), batch=0), _lib.ATTN_ERROR_INVALID_VALUE),
    (dict(head_dim=80, dtype=_lib.ATTN_BF16), _lib.ATTN_ERROR_NOT_SUPPORTED),
    (dict(dtype=_lib.ATTN_FP8_E4M3), _lib.ATTN_ERROR_NOT_SUPPORTED),             # head_dim 32
    (dict(dtype=_lib.ATTN_FP8_E4M3, head_dim=128, q_scale=0.0, k_scale=1.0, v_scale=1.0),
     _lib.ATTN_ERROR_INVALID_VALUE),
    (dict(dtype=_lib.ATTN_FP8_E4M3, head_dim=128, q_scale=1.0, k_scale=float("inf"), v_scale=1.0),
     _lib.ATTN_ERROR_INVALID_VALUE),
    (dict(window=16), _lib.ATTN_ERROR_INVALID_VALUE),
    (dict(causal=2), _lib.ATTN_ERROR_INVALID_VALUE),
    (dict(seqlen_q=-1), _lib.ATTN_ERROR_INVALID_VALUE),
    (dict(softcap=float("nan")), _lib.ATTN_ERROR_INVALID_VALUE),
    (dict(q_stride=(8192, 2048, 30)), _lib.ATTN_ERROR_NOT_SUPPORTED),
    (dict(k_stride=(8192, 2048, 16)), _lib.ATTN_ERROR_INVALID_VALUE),
    (dict(v_stride=(8192, -2048, 32)), _lib.ATTN_ERROR_INVALID_VALUE),
    (dict(sinks=FAKE + 2), _lib.ATTN_ERROR_INVALID_VALUE),
])
def test_fwd_rejects_bad_arguments(kw, status):
    L = _lib.lib()
    a = _fwd_args(**kw)
    st = L.attn_fwd(ctypes.byref(a), FAKE, FAKE, FAKE, FAKE, None, None)
    assert st == status, L.attn_last_error_message()
    assert len(L.attn_last_error_message()) > 0


def test_fwd_rejects_null_and_misaligned_pointers():
    L = _lib.lib()
    a = _fwd_args()
    assert L.attn_fwd(None, FAKE, FAKE, FAKE, FAKE, None, None) == _lib.ATTN_ERROR_INVALID_VALUE
    assert L.attn_fwd(ctypes.byref(a), None, FAKE, FAKE, FAKE, None, None) == _lib.ATTN_ERROR_INVALID_VALUE
    assert L.attn_fwd(ctypes.byref(a), FAKE + 8, FAKE, FAKE, FAKE, None, None) == _lib.ATTN_ERROR_NOT_SUPPORTED
    assert L.attn_fwd(ctypes.byref(a), FAKE, FAKE, FAKE, FAKE, FAKE + 2, None) == _lib.ATTN_ERROR_INVALID_VALUE
    a.cu_seqlens_q = FAKE
    assert L.attn_fwd(ctypes.byref(a), FAKE, FAKE, FAKE, FAKE, None, None) == _lib.ATTN_ERROR_INVALID_VALUE


def test_fwd_empty_query_is_a_no_op():
    L = _lib.lib()
    a = _fwd_args(seqlen_q=0)
    assert L.attn_fwd(ctypes.byref(a), None, None, None, None, None, None) == _lib.ATTN_SUCCESS


def _paged_args(**kw):
    a = _lib.FwdPagedArgs()
    base = dict(num_seqs=4, num_q_heads=8, num_kv_heads=2, head_dim=128, page_size=16, max_pages_per_seq=64,
                num_pages=256, max_seqlen_q=512, dtype=_lib.ATTN_BF16, causal=1, window=0, softmax_scale=0.0,
                softcap=0.0)
    base.update(kw)
    for k, v in base.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("kw,status", [
    (dict(num_seqs=0), _lib.ATTN_ERROR_INVALID_VALUE),
    (dict(num_q_heads=6, num_kv_heads=4), _lib.ATTN_ERROR_INVALID_VALUE),
    (dict(head_dim=80), _lib.ATTN_ERROR_NOT_SUPPORTED),
    (dict(head_dim=512), _lib.ATTN_ERROR_NOT_SUPPORTED),
    (dict(dtype=_lib.ATTN_F32), _lib.ATTN_ERROR_NOT_SUPPORTED),
    (dict(dtype=_lib.ATTN_FP8_E4M3), _lib.ATTN_ERROR_NOT_SUPPORTED),
    (dict(page_size=32), _lib.ATTN_ERROR_NOT_SUPPORTED),
    (dict(max_pages_per_seq=0), _lib.ATTN_ERROR_INVALID_VALUE),
    (dict(num_pages=0), _lib.ATTN_ERROR_INVALID_VALUE),
    (dict(max_seqlen_q=-1), _lib.ATTN_ERROR_INVALID_VALUE),
    (dict(causal=0, window=8), _lib.ATTN_ERROR_INVALID_VALUE),
    (dict(causal=3), _lib.ATTN_ERROR_INVALID_VALUE),
    (dict(softmax_scale=float("inf")), _lib.ATTN_ERROR_INVALID_VALUE),
    (dict(sinks=FAKE + 1), _lib.ATTN_ERROR_INVALID_VALUE),
])
def test_fwd_paged_rejects_bad_arguments(kw, status):
    L = _lib.lib()
    a = _paged_args(**kw)
    st = L.attn_fwd_paged(ctypes.byref(a), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, 0, None)
    assert st == status, L.attn_last_error_message()
    assert len(L.attn_last_error_message()) > 0


def test_fwd_paged_rejects_null_and_misaligned_pointers():
    L = _lib.lib()
    a = _paged_args()
    assert L.attn_fwd_paged(None, *([FAKE] * 7), None, None, 0, None) == _lib.ATTN_ERROR_INVALID_VALUE
    for i in range(7):
        ptrs = [FAKE] * 7
        ptrs[i] = None
        assert L.attn_fwd_paged(ctypes.byref(a), *ptrs, None, None, 0, None) == _lib.ATTN_ERROR_INVALID_VALUE, i
    for i, bad in ((0, FAKE + 8), (1, FAKE + 8), (2, FAKE + 8), (6, FAKE + 8)):
        ptrs = [FAKE] * 7
        ptrs[i] = bad
        assert L.attn_fwd_paged(ctypes.byref(a), *ptrs, None, None, 0, None) == _lib.ATTN_ERROR_NOT_SUPPORTED, i
    for i in (3, 4, 5):
        ptrs = [FAKE] * 7
        ptrs[i] = FAKE + 2
        assert L.attn_fwd_paged(ctypes.byref(a), *ptrs, None, None, 0, None) == _lib.ATTN_ERROR_INVALID_VALUE, i
    assert L.attn_fwd_paged(ctypes.byref(a), *([FAKE] * 7), FAKE + 2, None, 0, None) == _lib.ATTN_ERROR_INVALID_VALUE


def test_fwd_paged_empty_chunks_are_a_no_op():
    L = _lib.lib()
    a = _paged_args(max_seqlen_q=0)
    assert L.attn_fwd_paged(ctypes.byref(a), *([None] * 9), 0, None) == _lib.ATTN_SUCCESS


def test_fwd_paged_workspace():
    L = _lib.lib()
    a = _paged_args()
    need = L.attn_fwd_paged_workspace_size(ctypes.byref(a))
    # K and V of 4 sequences x 64 pages x 16 tokens x 2 heads x 128 x bf16
    assert need == 2 * 4 * 64 * 16 * 2 * 128 * 2
    assert L.attn_fwd_paged_workspace_size(ctypes.byref(_paged_args(head_dim=64))) == 0
    assert L.attn_fwd_paged_workspace_size(ctypes.byref(_paged_args(num_seqs=0))) == 0
    ptrs = [FAKE] * 7
    assert L.attn_fwd_paged(ctypes.byref(a), *ptrs, None, FAKE, need - 1, None) == \
        _lib.ATTN_ERROR_WORKSPACE_TOO_SMALL
    assert L.attn_fwd_paged(ctypes.byref(a), *ptrs, None, FAKE + 16, need, None) == _lib.ATTN_ERROR_INVALID_VALUE


def _dec_kw(**kw):
    base = dict(num_seqs=64, num_q_heads=32, num_kv_heads=8, head_dim=128, max_pages_per_seq=2048,
                max_seq_len=32768, q_dtype=_lib.ATTN_BF16, kv_dtype=_lib.ATTN_BF16)
    base.update(kw)
    return base


def test_decode_plan_is_a_deterministic_integer_function():
    assert attn.decode_plan(**_dec_kw()) == (1024, 32)
    assert attn.decode_plan(**_dec_kw(num_splits=9)) == (3648, 9)
    # a split never exceeds 4096 tokens, whatever is asked for
    assert attn.decode_plan(**_dec_kw(num_splits=7)) == (4096, 8)
    assert attn.decode_plan(**_dec_kw(num_splits=1)) == (4096, 8)
    # a short single sequence still gets 256-token splits
    assert attn.decode_plan(**_dec_kw(num_seqs=1, max_seq_len=1000, max_pages_per_seq=63)) == (256, 4)
    # many query heads per KV head: longer splits keep the partial results small next to
    # the K/V bytes (at least 512 * G / kv_bytes tokens) ...
    assert attn.decode_plan(**_dec_kw(num_kv_heads=1)) == (2048, 16)
    assert attn.decode_plan(**_dec_kw(num_kv_heads=2)) == (4096, 8)
    assert attn.decode_plan(**_dec_kw(kv_dtype=_lib.ATTN_FP8_E4M3, num_kv_heads=1)) == (2048, 16)
    # ... while the grid keeps at least 384 waves (a wave takes two tiles of 16 query heads)
    assert attn.decode_plan(**_dec_kw(num_seqs=1, num_kv_heads=1)) == (256, 128)
    assert attn.decode_plan(**_dec_kw(num_seqs=8, num_kv_heads=1)) == (256, 128)
    assert attn.decode_plan(**_dec_kw(num_seqs=32, num_kv_heads=1)) == (1024, 32)
    # the same choices when the longest sequence falls just short of a power of two (the
    # decode workload's lengths: max 32567)
    assert attn.decode_plan(**_dec_kw(num_kv_heads=1, max_seq_len=32567)) == (2048, 16)
    assert attn.decode_plan(**_dec_kw(num_kv_heads=2, max_seq_len=32567)) == (4096, 8)
    assert attn.decode_plan(**_dec_kw(max_seq_len=32567)) == (1024, 32)
    ln, n = attn.decode_plan(**_dec_kw(num_seqs=1, max_seq_len=2_000_000, max_pages_per_seq=125000,
                                       num_splits=1000))
    assert ln == 2000 and n == 1000
    for forced in (1, 2, 3, 7, 9, 31, 64, 100):
        ln, n = attn.decode_plan(**_dec_kw(num_splits=forced))
        assert ln % 16 == 0 and ln <= 4096 and n == -(-32768 // ln)
        assert (n <= forced and ln == -(-(-(-32768 // forced)) // 16) * 16) or ln == 4096


def test_decode_plan_of_the_cooperative_fp8_kernel():
    """fp8 KV, at most 16 query heads per KV head, even Hkv: one workgroup per (split,
    sequence), two per CU (the LDS of their page stages). The splits are sized so that the
    expected workgroup count, with lengths taken as half the maximum and one partial split
    per sequence, is three quarters of the 2 x 256 workgroups the device holds at once
    (256 compute units without a device); at least 256 tokens, at most 4096, then spread
    evenly over the maximum length."""
    def expect(num_seqs, max_len):
        room = 0.75 * 2 * 256 - 0.5 * num_seqs
        want = num_seqs * 0.5 * max_len / room if room > 0 else 4096
        ln = min(max(256, -(-int(want * 1e6) // 10 ** 6)), 4096)
        n = -(-max_len // ln)
        ln = -(-(-(-max_len // n)) // 16) * 16
        return ln, -(-max_len // ln)
    fp8 = dict(kv_dtype=_lib.ATTN_FP8_E4M3)
    cases = [(64, 32768, (2992, 11)), (64, 8192, (752, 11)), (16, 32768, (704, 47)),
             (128, 16384, (3280, 5)), (1024, 32768, (4096, 8)), (1, 1000, (256, 4))]
    for num_seqs, max_len, want in cases:
        got = attn.decode_plan(**_dec_kw(num_seqs=num_seqs, max_seq_len=max_len,
                                         max_pages_per_seq=-(-max_len // 16), **fp8))
        assert got == want == expect(num_seqs, max_len), (num_seqs, max_len, got)
    # an odd Hkv takes the one-wave kernel and its plan: 896-token splits rounded up to a
    # power of two (1024), then doubled to 512 * G / kv_bytes = 2048 (the grid keeps its
    # 384 waves)
    assert attn.decode_plan(**_dec_kw(num_q_heads=28, num_kv_heads=7, **fp8)) == (2048, 16)


def test_decode_workspace_size():
    ln, n = attn.decode_plan(**_dec_kw())
    assert attn.decode_workspace_size(**_dec_kw()) == 64 * 32 * n * 128 * 4 + 64 * 32 * n * 4
    assert attn.decode_workspace_size(**_dec_kw(head_dim=64)) == 0  # invalid args -> 0


@pytest.mark.parametrize("kw,status", [
    (dict(num_q_heads=30), _lib.ATTN_ERROR_INVALID_VALUE),
    (dict(num_q_heads=65536 * 17, num_kv_heads=65536), _lib.ATTN_ERROR_NOT_SUPPORTED),
    (dict(head_dim=64), _lib.ATTN_ERROR_NOT_SUPPORTED),
    (dict(sinks=FAKE + 2), _lib.ATTN_ERROR_INVALID_VALUE),
    (dict(max_seq_len=40000), _lib.ATTN_ERROR_INVALID_VALUE),
    (dict(q_dtype=_lib.ATTN_F32), _lib.ATTN_ERROR_NOT_SUPPORTED),
    (dict(kv_dtype=_lib.ATTN_F16), _lib.ATTN_ERROR_NOT_SUPPORTED),
    (dict(num_splits=-1), _lib.ATTN_ERROR_INVALID_VALUE),
])
def test_decode_rejects_bad_arguments(kw, status):
    L = _lib.lib()
    a = attn._decode_args(**_dec_kw(**kw))
    st = L.attn_decode_paged(ctypes.byref(a), FAKE, FAKE, FAKE, None, None, FAKE, FAKE, FAKE, None,
                             FAKE, 1 << 30, None)
    assert st == status, L.attn_last_error_message()


def test_decode_checks_scales_and_workspace():
    L = _lib.lib()
    a = attn._decode_args(**_dec_kw(kv_dtype=_lib.ATTN_FP8_E4M3))
    st = L.attn_decode_paged(ctypes.byref(a), FAKE, FAKE, FAKE, None, None, FAKE, FAKE, FAKE, None,
                             FAKE, 1 << 30, None)
    assert st == _lib.ATTN_ERROR_INVALID_VALUE
    a = attn._decode_args(**_dec_kw())
    st = L.attn_decode_paged(ctypes.byref(a), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None,
                             FAKE, 1 << 30, None)
    assert st == _lib.ATTN_ERROR_INVALID_VALUE
    st = L.attn_decode_paged(ctypes.byref(a), FAKE, FAKE, FAKE, None, None, FAKE, FAKE, FAKE, None,
                             FAKE, 1024, None)
    assert st == _lib.ATTN_ERROR_WORKSPACE_TOO_SMALL


def test_decode_noalloc_checks_arguments_and_its_limit():
    """The allocation-free decode rejects bad arguments, and calls whose partial results
    exceed its built-in scratch, on the host before any HIP call."""
    L = _lib.lib()
    a = attn._decode_args(**_dec_kw(num_q_heads=30))
    st = L.attn_decode_paged_noalloc(ctypes.byref(a), FAKE, FAKE, FAKE, None, None, FAKE, FAKE, FAKE, None, None)
    assert st == _lib.ATTN_ERROR_INVALID_VALUE
    a = attn._decode_args(**_dec_kw())
    st = L.attn_decode_paged_noalloc(ctypes.byref(a), FAKE, FAKE, FAKE, None, None, FAKE, None, FAKE, None, None)
    assert st == _lib.ATTN_ERROR_INVALID_VALUE  # no seq_lens
    # 64 sequences of up to 32768 tokens, Hq = 32: 34 MB of partials, within the 64 MiB
    assert attn.decode_workspace_size(**_dec_kw()) <= attn.DECODE_NOALLOC_MAX_WORKSPACE
    big = _dec_kw(num_seqs=512)
    assert attn.decode_workspace_size(**big) > attn.DECODE_NOALLOC_MAX_WORKSPACE
    a = attn._decode_args(**big)
    st = L.attn_decode_paged_noalloc(ctypes.byref(a), FAKE, FAKE, FAKE, None, None, FAKE, FAKE, FAKE, None, None)
    assert st == _lib.ATTN_ERROR_WORKSPACE_TOO_SMALL
    assert b"scratch" in L.attn_last_error_message()


def test_decode_noalloc_limit_matches_the_header():
    text = open(os.path.join(ROOT, "include", "attn.h")).read()
    m = re.search(r"#define ATTN_DECODE_NOALLOC_MAX_WORKSPACE \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == attn.DECODE_NOALLOC_MAX_WORKSPACE


@pytest.mark.parametrize("args", [
    (None, 256, 10, 0, FAKE, FAKE),          # no operands
    (FAKE, 0, 10, 0, FAKE, FAKE),            # no workgroups
    (FAKE, 70000, 10, 0, FAKE, FAKE),        # too many workgroups
    (FAKE, 256, 0, 0, FAKE, FAKE),           # no iterations
    (FAKE, 256, 10, 2, FAKE, FAKE),          # unknown vector mix
    (FAKE, 256, 10, 0, FAKE + 4, FAKE),      # clocks not 8-byte aligned
    (FAKE, 256, 10, 0, None, FAKE),          # no clocks
])
def test_probe_mfma_rejects_bad_arguments(args):
    L = _lib.lib()
    assert L.attn_probe_mfma(*args, None) == _lib.ATTN_ERROR_INVALID_VALUE, L.attn_last_error_message()


@pytest.mark.parametrize("args", [
    (None, 1 << 20, 32, FAKE),               # no buffer
    (FAKE, 0, 32, FAKE),                     # no bytes
    (FAKE, (1 << 20) + 16, 32, FAKE),        # not a multiple of 32768 * workgroups
    (FAKE, 1 << 20, 0, FAKE),                # no workgroups
    (FAKE + 8, 1 << 20, 32, FAKE),           # misaligned buffer
    (FAKE, 1 << 20, 32, None),               # no sink
])
def test_probe_hbm_read_rejects_bad_arguments(args):
    L = _lib.lib()
    assert L.attn_probe_hbm_read(*args, None) == _lib.ATTN_ERROR_INVALID_VALUE, L.attn_last_error_message()


def test_flush_rejects_bad_arguments():
    L = _lib.lib()
    assert L.attn_flush_caches(None, 1 << 20, None) == _lib.ATTN_ERROR_INVALID_VALUE
    assert L.attn_flush_caches(FAKE, 0, None) == _lib.ATTN_ERROR_INVALID_VALUE
    assert L.attn_flush_caches(FAKE, 24, None) == _lib.ATTN_ERROR_INVALID_VALUE
    assert L.attn_flush_caches(FAKE + 8, 1 << 20, None) == _lib.ATTN_ERROR_INVALID_VALUE
