"""C ABI checks that need no GPU: the library loads, exports every function
include/dsa.h declares, sizes workspaces, and rejects bad arguments on the host
before anything is launched (pointers here are never dereferenced)."""
import ctypes
import os
import re
import subprocess

import pytest

import sparse_attention_03_amd as dsa

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "dsa.h")
FAKE = 0x10000  # 64 KiB-aligned, never dereferenced by host validation


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:dsa_status|size_t|const char\*|int32_t)\s+(\w+)\s*\(", text, re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("dsa_indexer_scores", "dsa_topk", "dsa_translate_pages", "sparse_mla_decode",
              "sparse_mla_prefill", "dsa_workspace_size", "dsa_status_str", "dsa_last_error",
              "dsa_abi_version", "dsa_quantize_q", "dsa_cache_insert", "dsa_topk_sharded", "dsa_msa_decode",
              "dsa_indexer_scores_prefix", "sparse_mla_decode_noalloc", "dsa_check_debug_flag"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = dsa.load()
    for n in declared_functions():
        assert hasattr(lib, n), n
    assert set(declared_functions()) == set(dsa.EXPORTS)
    assert lib.dsa_abi_version() == 2
    # the release build compiles the device notes out (no HIP call is made)
    assert lib.dsa_check_debug_flag() == -1


def test_debug_library_exports_every_declared_symbol():
    """libdsa_debug.so (DSA_DEBUG=1) is built beside libdsa.so with the same
    entry points; it is opened here without routing any call through it."""
    assert os.path.exists(dsa.DEBUG_LIB_PATH), "build with python -m sparse_attention_03_amd.build"
    lib = ctypes.CDLL(dsa.DEBUG_LIB_PATH)
    for n in declared_functions():
        assert hasattr(lib, n), n
    lib.dsa_abi_version.restype = ctypes.c_int32
    assert lib.dsa_abi_version() == 2


SANITIZE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "sanitize")
CSRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "sparse_attention_03_amd", "csrc")


def test_host_abi_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    """api.cpp, built for the host alone with ASan + UBSan and linked with
    launch stubs that touch every buffer extent their kernels would (see
    tests/sanitize/launch_stubs.cpp), runs every entry point on decode,
    speculative, prefill, sharded, MSA and shared-prefix shapes with buffers
    of exactly their documented sizes, and the argument errors.  Any
    out-of-bounds access of a host plan, undefined behaviour or unexpected
    status fails the run."""
    clang = "/opt/rocm/llvm/bin/clang++"
    if not os.path.exists(clang):
        pytest.skip("ROCm clang++ is not installed")
    exe = tmp_path / "abi_driver"
    cmd = [clang, "-std=c++17", "-g", "-O1", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-x", "c++",
           os.path.join(CSRC, "api.cpp"), os.path.join(SANITIZE, "launch_stubs.cpp"),
           os.path.join(SANITIZE, "abi_driver.cpp"), "-o", str(exe)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=120)
    assert run.returncode == 0, (run.stdout + run.stderr)[-4000:]
    assert "abi driver ok" in run.stdout


def test_struct_layouts_match_the_c_compiler(tmp_path):
    """ctypes mirrors of the argument structs have the C compiler's layout."""
    structs = {"dsa_cache": dsa.Cache, "dsa_batch": dsa.Batch, "dsa_indexer_args": dsa.IndexerArgs,
               "dsa_topk_args": dsa.TopkArgs, "dsa_mla_args": dsa.MlaArgs, "dsa_quant_q_args": dsa.QuantQArgs,
               "dsa_insert_args": dsa.InsertArgs, "dsa_topk_sharded_args": dsa.TopkShardedArgs,
               "dsa_msa_args": dsa.MsaArgs, "dsa_indexer_prefix_args": dsa.IndexerPrefixArgs}
    lines = ["#include <stdio.h>", "#include <stddef.h>", f'#include "{HEADER}"', "int main(void) {"]
    for cname, py in structs.items():
        lines.append(f'printf("{cname} %zu\\n", sizeof({cname}));')
        for f, _ in py._fields_:
            lines.append(f'printf("{cname}.{f} %zu\\n", offsetof({cname}, {f}));')
    lines.append("return 0; }")
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", str(src), "-o", str(exe)], check=True)
    got = dict(l.split() for l in subprocess.run([str(exe)], capture_output=True, text=True).stdout.splitlines())
    for cname, py in structs.items():
        assert int(got[cname]) == ctypes.sizeof(py), cname
        for f, _ in py._fields_:
            assert int(got[f"{cname}.{f}"]) == getattr(py, f).offset, f"{cname}.{f}"


def _batch(**kw):
    b = dict(num_requests=1, num_rows=1, req_row_start=FAKE, tok_req=FAKE, tok_vis=FAKE, block_table=None,
             bt_stride=0, max_vis=8192, max_rows_per_req=1)
    b.update(kw)
    return dsa.Batch(**b)


def _cache(fmt=dsa.KEY_FP8, plog2=13, page_bytes=132 * 8192, pages=1, base=FAKE):
    return dsa.Cache(base, page_bytes, plog2, pages, fmt)


def _idx_args(**kw):
    a = dict(batch=_batch(), keys=_cache(), q=FAKE, q_fmt=dsa.Q_BF16, q_scale=None, w=FAKE, scores=FAKE, ld=8192)
    a.update(kw)
    return dsa.IndexerArgs(**a)


@pytest.mark.parametrize("mut,status", [
    (dict(q=None), dsa.DSA_ERR_INVALID_ARG),
    (dict(q=FAKE + 8), dsa.DSA_ERR_INVALID_ARG),
    (dict(ld=100), dsa.DSA_ERR_INVALID_ARG),
    (dict(ld=8194), dsa.DSA_ERR_INVALID_ARG),
    (dict(q_fmt=7), dsa.DSA_ERR_UNSUPPORTED),
    (dict(q_fmt=dsa.Q_FP8), dsa.DSA_ERR_INVALID_ARG),            # FP8 q without q_scale
    (dict(q_fmt=dsa.Q_FP8, q_scale=FAKE, keys=_cache(fmt=dsa.KEY_MXFP4, page_bytes=68 * 8192)),
     dsa.DSA_ERR_UNSUPPORTED),                                    # FP8 q runs against FP8 keys only
    (dict(keys=_cache(fmt=dsa.KEY_NVFP4, page_bytes=71 * 8192)), dsa.DSA_ERR_INVALID_ARG),  # NVFP4 page < 72 B/token
    (dict(keys=_cache(fmt=9)), dsa.DSA_ERR_UNSUPPORTED),
    (dict(keys=_cache(plog2=3)), dsa.DSA_ERR_INVALID_ARG),
    (dict(keys=_cache(page_bytes=1000)), dsa.DSA_ERR_INVALID_ARG),
    (dict(keys=_cache(base=None)), dsa.DSA_ERR_INVALID_ARG),
    (dict(batch=_batch(max_vis=9000)), dsa.DSA_ERR_INVALID_ARG),  # non-paged page too small
    (dict(batch=_batch(num_rows=0)), dsa.DSA_ERR_INVALID_ARG),
    (dict(batch=_batch(block_table=FAKE, bt_stride=1, max_vis=8192), keys=_cache(plog2=6, page_bytes=132 * 64)),
     dsa.DSA_ERR_INVALID_ARG),                                    # block-table row too short
])
def test_indexer_rejects_bad_arguments(mut, status):
    lib = dsa.load()
    a = _idx_args(**mut)
    assert lib.dsa_indexer_scores(ctypes.byref(a), None) == status
    assert lib.dsa_last_error().decode() != ""


def _prefix_args(**kw):
    base = _idx_args(batch=_batch(num_requests=4, num_rows=4, block_table=FAKE, bt_stride=128, max_vis=8192),
                     keys=_cache(plog2=6, page_bytes=132 * 64, pages=512))
    a = dict(base=base, num_groups=1, group_row_start=FAKE, group_first_req=FAKE, prefix_len=4096,
             max_rows_per_group=4, workspace=FAKE, workspace_bytes=1 << 40)
    a.update(kw)
    return dsa.IndexerPrefixArgs(**a)


@pytest.mark.parametrize("mut,status", [
    (dict(num_groups=0), dsa.DSA_ERR_INVALID_ARG),
    (dict(num_groups=5), dsa.DSA_ERR_INVALID_ARG),          # more groups than requests
    (dict(group_row_start=None), dsa.DSA_ERR_INVALID_ARG),
    (dict(group_first_req=None), dsa.DSA_ERR_INVALID_ARG),
    (dict(prefix_len=100), dsa.DSA_ERR_INVALID_ARG),        # not a multiple of the page size
    (dict(prefix_len=8256), dsa.DSA_ERR_INVALID_ARG),       # beyond max_vis
    (dict(prefix_len=-64), dsa.DSA_ERR_INVALID_ARG),
    (dict(max_rows_per_group=0), dsa.DSA_ERR_INVALID_ARG),
    (dict(workspace=None), dsa.DSA_ERR_WORKSPACE),
    (dict(workspace_bytes=16), dsa.DSA_ERR_WORKSPACE),
])
def test_indexer_prefix_rejects_bad_arguments(mut, status):
    lib = dsa.load()
    assert lib.dsa_indexer_scores_prefix(ctypes.byref(_prefix_args(**mut)), None) == status
    assert lib.dsa_last_error().decode() != ""


def test_indexer_prefix_rejects_fp8_q_and_missing_table():
    lib = dsa.load()
    a = _prefix_args()
    a.base.q_fmt = dsa.Q_FP8
    a.base.q_scale = FAKE
    assert lib.dsa_indexer_scores_prefix(ctypes.byref(a), None) == dsa.DSA_ERR_UNSUPPORTED
    a = _prefix_args()
    a.base.batch.block_table = None
    a.base.batch.max_vis = 64
    assert lib.dsa_indexer_scores_prefix(ctypes.byref(a), None) == dsa.DSA_ERR_INVALID_ARG


def _topk_args(**kw):
    a = dict(batch=_batch(), scores=FAKE, ld=8192, k=2048, idx=FAKE, rows=None, page_size_log2=0, num_pages=0,
             count=None, workspace=FAKE, workspace_bytes=1 << 40)
    a.update(kw)
    return dsa.TopkArgs(**a)


@pytest.mark.parametrize("mut,status", [
    (dict(k=0), dsa.DSA_ERR_INVALID_ARG),
    (dict(k=2049), dsa.DSA_ERR_INVALID_ARG),
    (dict(idx=None), dsa.DSA_ERR_INVALID_ARG),
    (dict(ld=8191), dsa.DSA_ERR_INVALID_ARG),
    (dict(workspace=None), dsa.DSA_ERR_WORKSPACE),
    (dict(workspace_bytes=100), dsa.DSA_ERR_WORKSPACE),
    (dict(workspace=FAKE + 64), dsa.DSA_ERR_WORKSPACE),
    (dict(rows=FAKE, page_size_log2=2, num_pages=4), dsa.DSA_ERR_INVALID_ARG),
    (dict(rows=FAKE, page_size_log2=13, num_pages=0), dsa.DSA_ERR_INVALID_ARG),           # pool size needed
    (dict(rows=FAKE, page_size_log2=13, num_pages=1 << 18), dsa.DSA_ERR_INVALID_ARG),     # rows past int32
])
def test_topk_rejects_bad_arguments(mut, status):
    assert dsa.load().dsa_topk(ctypes.byref(_topk_args(**mut)), None) == status


def _sharded_args(**kw):
    a = dict(num_rows=4, num_shards=8, scores=FAKE, ld=8192, tok_vis=FAKE, max_vis=65536, k=2048, cand=0,
             idx=FAKE, count=None, resend=None, workspace=FAKE, workspace_bytes=1 << 40)
    a.update(kw)
    return dsa.TopkShardedArgs(**a)


@pytest.mark.parametrize("mut,status", [
    (dict(num_rows=0), dsa.DSA_ERR_INVALID_ARG),
    (dict(num_shards=0), dsa.DSA_ERR_INVALID_ARG),
    (dict(num_shards=17), dsa.DSA_ERR_INVALID_ARG),
    (dict(k=0), dsa.DSA_ERR_INVALID_ARG),
    (dict(k=2049), dsa.DSA_ERR_INVALID_ARG),
    (dict(cand=-1), dsa.DSA_ERR_INVALID_ARG),
    (dict(cand=2049), dsa.DSA_ERR_INVALID_ARG),
    (dict(max_vis=0), dsa.DSA_ERR_INVALID_ARG),
    (dict(ld=8188), dsa.DSA_ERR_INVALID_ARG),          # < ceil(65536 / 8)
    (dict(ld=8194), dsa.DSA_ERR_INVALID_ARG),          # not a multiple of 4
    (dict(scores=FAKE + 4), dsa.DSA_ERR_INVALID_ARG),
    (dict(tok_vis=None), dsa.DSA_ERR_INVALID_ARG),
    (dict(idx=None), dsa.DSA_ERR_INVALID_ARG),
    (dict(workspace=None), dsa.DSA_ERR_WORKSPACE),
    (dict(workspace=FAKE + 64), dsa.DSA_ERR_WORKSPACE),
    (dict(workspace_bytes=100), dsa.DSA_ERR_WORKSPACE),
])
def test_topk_sharded_rejects_bad_arguments(mut, status):
    lib = dsa.load()
    assert lib.dsa_topk_sharded(ctypes.byref(_sharded_args(**mut)), None) == status
    assert lib.dsa_last_error().decode() != ""


def test_topk_sharded_workspace_size():
    a = _sharded_args()
    n = dsa.dsa_workspace_size(dsa.OP_TOPK_SHARDED, a)
    # at least the local top-k positions and the exchange buffer (W*T*k*(4+8) bytes)
    assert n >= 8 * 4 * 2048 * 12
    assert dsa.dsa_workspace_size(dsa.OP_TOPK_SHARDED, _sharded_args(num_shards=17)) == 0
    assert dsa.dsa_workspace_size(dsa.OP_TOPK_SHARDED, _sharded_args(cand=3000)) == 0


def _msa_args(**kw):
    a = dict(batch=_batch(block_table=FAKE, bt_stride=1024, max_vis=131072), index_keys=FAKE, kv=FAKE,
             num_blocks=1024, num_kv_heads=4, num_q_heads=64, top_blocks=16, q_idx=FAKE, q=FAKE, k_scale=1.0,
             v_scale=1.0, sm_scale=0.088, sel_blocks=FAKE, out=FAKE, lse=None, workspace=FAKE,
             workspace_bytes=1 << 40)
    a.update(kw)
    return dsa.MsaArgs(**a)


@pytest.mark.parametrize("mut,status", [
    (dict(num_kv_heads=0), dsa.DSA_ERR_INVALID_ARG),
    (dict(num_kv_heads=9), dsa.DSA_ERR_INVALID_ARG),
    (dict(num_q_heads=66), dsa.DSA_ERR_INVALID_ARG),       # not a multiple of Hkv
    (dict(num_q_heads=68), dsa.DSA_ERR_INVALID_ARG),       # 17 per group
    (dict(top_blocks=0), dsa.DSA_ERR_INVALID_ARG),
    (dict(top_blocks=17), dsa.DSA_ERR_INVALID_ARG),
    (dict(batch=_batch(block_table=None, max_vis=131072)), dsa.DSA_ERR_INVALID_ARG),
    (dict(batch=_batch(block_table=FAKE, bt_stride=1000, max_vis=131072)), dsa.DSA_ERR_INVALID_ARG),
    (dict(index_keys=None), dsa.DSA_ERR_INVALID_ARG),
    (dict(kv=FAKE + 8), dsa.DSA_ERR_INVALID_ARG),
    (dict(q=None), dsa.DSA_ERR_INVALID_ARG),
    (dict(out=None), dsa.DSA_ERR_INVALID_ARG),
    (dict(num_blocks=0), dsa.DSA_ERR_INVALID_ARG),
    (dict(workspace=None), dsa.DSA_ERR_WORKSPACE),
    (dict(workspace_bytes=64), dsa.DSA_ERR_WORKSPACE),
])
def test_msa_rejects_bad_arguments(mut, status):
    lib = dsa.load()
    assert lib.dsa_msa_decode(ctypes.byref(_msa_args(**mut)), None) == status
    assert lib.dsa_last_error().decode() != ""


def test_msa_workspace_size():
    a = _msa_args()
    # block scores (rows x Hkv x blocks fp32) + two partial results of 16 x 128 + 32 fp32 per (row, group)
    assert dsa.dsa_workspace_size(dsa.OP_MSA_DECODE, a) == 1 * 4 * 1024 * 4 + 1 * 4 * 2 * (16 * 128 + 32) * 4


def _mla_args(**kw):
    a = dict(num_rows=4, num_heads=12, q=FAKE, latents=_cache(fmt=dsa.LAT_FP8, plog2=6, page_bytes=640 * 64, pages=10),
             rows=FAKE, k=2048, sm_scale=0.07, num_splits=0, out=FAKE, lse=None, workspace=FAKE,
             workspace_bytes=1 << 40)
    a.update(kw)
    return dsa.MlaArgs(**a)


@pytest.mark.parametrize("mut,status", [
    (dict(num_heads=0), dsa.DSA_ERR_INVALID_ARG),
    (dict(num_heads=129), dsa.DSA_ERR_INVALID_ARG),
    (dict(k=0), dsa.DSA_ERR_INVALID_ARG),
    (dict(sm_scale=float("nan")), dsa.DSA_ERR_INVALID_ARG),
    (dict(sm_scale=-1.0), dsa.DSA_ERR_INVALID_ARG),
    (dict(out=FAKE + 4), dsa.DSA_ERR_INVALID_ARG),
    (dict(latents=_cache(fmt=0)), dsa.DSA_ERR_UNSUPPORTED),
    (dict(latents=_cache(fmt=dsa.LAT_NVFP4, plog2=6, page_bytes=383 * 64)), dsa.DSA_ERR_INVALID_ARG),
    (dict(latents=_cache(fmt=dsa.LAT_FP8, plog2=6, page_bytes=580 * 64)), dsa.DSA_ERR_INVALID_ARG),
    (dict(workspace=None), dsa.DSA_ERR_WORKSPACE),
    (dict(workspace_bytes=10), dsa.DSA_ERR_WORKSPACE),
])
def test_mla_rejects_bad_arguments(mut, status):
    lib = dsa.load()
    a = _mla_args(**mut)
    assert lib.sparse_mla_decode(ctypes.byref(a), None) == status


def test_translate_rejects_bad_arguments():
    lib = dsa.load()
    b = _batch()
    assert lib.dsa_translate_pages(None, 2048, ctypes.byref(b), 6, 10, FAKE, None) == dsa.DSA_ERR_INVALID_ARG
    assert lib.dsa_translate_pages(FAKE, 0, ctypes.byref(b), 6, 10, FAKE, None) == dsa.DSA_ERR_INVALID_ARG
    assert lib.dsa_translate_pages(FAKE, 2048, ctypes.byref(b), 30, 10, FAKE, None) == dsa.DSA_ERR_INVALID_ARG
    assert lib.dsa_translate_pages(FAKE, 2048, ctypes.byref(b), 6, 0, FAKE, None) == dsa.DSA_ERR_INVALID_ARG
    assert lib.dsa_translate_pages(FAKE, 2048, ctypes.byref(b), 6, 1 << 25, FAKE, None) == dsa.DSA_ERR_INVALID_ARG


def test_workspace_sizes():
    t = _topk_args(batch=_batch(num_rows=192, max_vis=65536, num_requests=32))
    n = dsa.dsa_workspace_size(dsa.OP_TOPK, t)
    assert n >= 192 * (16 + 8192 * 8)
    assert n % 256 == 0
    m = _mla_args(num_rows=192, num_heads=12, num_splits=4)
    assert dsa.dsa_workspace_size(dsa.OP_MLA_DECODE, m) >= 192 * 4 * 12 * 512 * 4
    assert dsa.dsa_workspace_size(dsa.OP_MLA_PREFILL, m) == 0      # one split: no partials
    assert dsa.dsa_workspace_size(dsa.OP_MLA_DECODE, _mla_args(num_splits=1)) == 0
    assert dsa.dsa_workspace_size(dsa.OP_TOPK, _topk_args(k=0)) == 0
    assert dsa.dsa_workspace_size(dsa.OP_INDEXER, _idx_args()) == 0


def test_status_strings():
    lib = dsa.load()
    assert lib.dsa_status_str(0) == b"DSA_OK"
    assert lib.dsa_status_str(4) == b"DSA_ERR_HIP"


def _qq_args(**kw):
    a = dict(num_rows=4, q=FAKE, w=FAKE, fmt=dsa.Q_FP8, q_out=FAKE, q_scale=FAKE, w_folded=None)
    a.update(kw)
    return dsa.QuantQArgs(**a)


@pytest.mark.parametrize("mut,status", [
    (dict(num_rows=-1), dsa.DSA_ERR_INVALID_ARG),
    (dict(fmt=dsa.Q_BF16), dsa.DSA_ERR_UNSUPPORTED),
    (dict(q=None), dsa.DSA_ERR_INVALID_ARG),
    (dict(q=FAKE + 2), dsa.DSA_ERR_INVALID_ARG),
    (dict(q_out=FAKE + 8), dsa.DSA_ERR_INVALID_ARG),
    (dict(q_scale=None), dsa.DSA_ERR_INVALID_ARG),
    (dict(w=None, w_folded=FAKE), dsa.DSA_ERR_INVALID_ARG),        # folding needs w
    (dict(fmt=dsa.Q_MXFP4, w_folded=FAKE), dsa.DSA_ERR_INVALID_ARG),  # folding is FP8 only
])
def test_quantize_q_rejects_bad_arguments(mut, status):
    assert dsa.load().dsa_quantize_q(ctypes.byref(_qq_args(**mut)), None) == status


def test_quantize_q_zero_rows_launches_nothing():
    assert dsa.load().dsa_quantize_q(ctypes.byref(_qq_args(num_rows=0, q=None, q_out=None, q_scale=None)), None) == 0


def _ins_args(**kw):
    a = dict(num_tokens=3, num_requests=2, tok_req=FAKE, tok_pos=FAKE, block_table=FAKE, bt_stride=4,
             key_vals=FAKE, keys=_cache(fmt=dsa.KEY_FP8, plog2=6, page_bytes=132 * 64, pages=8),
             lat_vals=FAKE, latents=_cache(fmt=dsa.LAT_FP8, plog2=6, page_bytes=640 * 64, pages=8))
    a.update(kw)
    return dsa.InsertArgs(**a)


@pytest.mark.parametrize("mut,status", [
    (dict(num_tokens=-1), dsa.DSA_ERR_INVALID_ARG),
    (dict(key_vals=None, lat_vals=None), dsa.DSA_ERR_INVALID_ARG),
    (dict(keys=_cache(fmt=7, plog2=6, page_bytes=132 * 64, pages=8)), dsa.DSA_ERR_UNSUPPORTED),
    (dict(keys=_cache(fmt=dsa.KEY_NVFP4, plog2=6, page_bytes=68 * 64, pages=8)), dsa.DSA_ERR_INVALID_ARG),
    (dict(keys=_cache(fmt=dsa.KEY_FP8, plog2=6, page_bytes=131 * 64, pages=8)), dsa.DSA_ERR_INVALID_ARG),
    (dict(latents=_cache(fmt=dsa.LAT_NVFP4, plog2=6, page_bytes=352 * 64, pages=8)), dsa.DSA_ERR_INVALID_ARG),
    (dict(latents=_cache(fmt=dsa.LAT_FP8, plog2=5, page_bytes=640 * 64, pages=8)), dsa.DSA_ERR_INVALID_ARG),
    (dict(key_vals=FAKE + 2), dsa.DSA_ERR_INVALID_ARG),
    (dict(lat_vals=FAKE + 8), dsa.DSA_ERR_INVALID_ARG),
    (dict(tok_pos=None), dsa.DSA_ERR_INVALID_ARG),
    (dict(num_requests=0), dsa.DSA_ERR_INVALID_ARG),
    (dict(bt_stride=0), dsa.DSA_ERR_INVALID_ARG),
])
def test_cache_insert_rejects_bad_arguments(mut, status):
    assert dsa.load().dsa_cache_insert(ctypes.byref(_ins_args(**mut)), None) == status
