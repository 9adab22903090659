"""C ABI checks that need no GPU: the library loads, exports every symbol the
header declares, the ctypes struct matches the C layout, and host-side
validation returns the documented status codes. No compute entry point is
called here."""
import ctypes
import os
import re
import shutil
import subprocess
import sys

import pytest

from block_diffusion_draft_dflash_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dflash.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dflash_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        pytest.fail("libdflash.so is not built (run __graft_entry__.build())")
    return B.load()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert names, "no declarations parsed"
    assert sorted(B.EXPORTED) == names
    for n in names:
        assert hasattr(lib, n), n


def test_abi_version_and_error_string(lib):
    assert lib.dflash_abi_version() == 106
    assert isinstance(lib.dflash_last_error(), bytes)


def test_struct_layout_matches_c(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    src = tmp_path / "layout.c"
    src.write_text(
        '#include <stdio.h>\n#include <stddef.h>\n#include "dflash.h"\n'
        "int main(void){printf(\"%zu\", sizeof(dflash_block_attn_params));"
        + "".join(f'printf(" %zu", offsetof(dflash_block_attn_params, {f}));'
                  for f, _ in B.BlockAttnParams._fields_)
        + "return 0;}\n")
    exe = tmp_path / "layout"
    subprocess.check_call([gcc, "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)])
    vals = [int(x) for x in subprocess.check_output([str(exe)]).split()]
    assert vals[0] == ctypes.sizeof(B.BlockAttnParams)
    for (f, _), off in zip(B.BlockAttnParams._fields_, vals[1:]):
        assert getattr(B.BlockAttnParams, f).offset == off, f


def P(**kw):
    base = dict(num_reqs=8, num_q_heads=32, num_kv_heads=8, head_dim=128, dtype=B.DFLASH_BF16,
                total_ctx=10000, total_blk=128, max_blk_len=16, scale=128 ** -0.5, causal=False,
                window=0, split_keys=0)
    base.update(kw)
    return B.make_block_attn_params(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(), B.DFLASH_OK),
    (dict(dtype=B.DFLASH_F32), B.DFLASH_OK),
    (dict(num_reqs=0), B.DFLASH_ERR_INVALID_ARG),
    (dict(num_q_heads=30), B.DFLASH_ERR_INVALID_ARG),
    (dict(num_kv_heads=0), B.DFLASH_ERR_INVALID_ARG),
    (dict(head_dim=96), B.DFLASH_ERR_UNSUPPORTED),
    (dict(head_dim=63), B.DFLASH_ERR_INVALID_ARG),
    (dict(dtype=7), B.DFLASH_ERR_INVALID_ARG),
    (dict(total_ctx=-1), B.DFLASH_ERR_INVALID_ARG),
    (dict(max_blk_len=200), B.DFLASH_ERR_INVALID_ARG),
    (dict(max_blk_len=0), B.DFLASH_ERR_INVALID_ARG),
    (dict(window=64), B.DFLASH_ERR_INVALID_ARG),          # window without causal
    (dict(window=64, causal=True), B.DFLASH_OK),
    (dict(window=-1, causal=True), B.DFLASH_ERR_INVALID_ARG),
    (dict(split_keys=100), B.DFLASH_ERR_INVALID_ARG),
    (dict(split_keys=128), B.DFLASH_OK),
    (dict(scale=float("nan")), B.DFLASH_ERR_INVALID_ARG),
    (dict(total_ctx=2 ** 30), B.DFLASH_ERR_INVALID_ARG),
    (dict(total_ctx=0), B.DFLASH_OK),
    (dict(total_blk=0, max_blk_len=0), B.DFLASH_OK),
])
def test_block_attention_validation(lib, kw, status):
    p = P(**kw)
    assert B.dflash_block_attention_check(p) == status, B.dflash_last_error()
    if status != B.DFLASH_OK:
        assert B.dflash_last_error()
        assert B.dflash_block_attention_workspace_size(p) == 0


def _host_lens(ctx, blk):
    return dict(host_cu_ctx_lens=[0] + list(__import__("itertools").accumulate(ctx)),
                host_cu_blk_lens=[0] + list(__import__("itertools").accumulate(blk)))


@pytest.mark.parametrize("ctx,blk,over,status", [
    ([1000] * 8 + [0] * 0, [16] * 8, {}, B.DFLASH_OK),
    ([2000] * 5, [16] * 5, dict(num_reqs=4), B.DFLASH_ERR_INVALID_ARG),      # [R] != totals
    ([1250] * 8, [16] * 7 + [17], dict(total_blk=129), B.DFLASH_ERR_INVALID_ARG),  # > max_blk_len
    ([1250] * 8, [16] * 8, dict(total_ctx=10001), B.DFLASH_ERR_INVALID_ARG),  # ctx end mismatch
])
def test_host_lengths_validation(lib, ctx, blk, over, status):
    kw = dict(total_ctx=sum(ctx), total_blk=sum(blk), num_reqs=len(ctx))
    kw.update(over)
    kw.update(_host_lens(ctx, blk))
    p = P(**kw)
    assert B.dflash_block_attention_check(p) == status, B.dflash_last_error()


def test_host_lengths_shape_errors(lib):
    good = _host_lens([1250] * 8, [16] * 8)
    p = P(**good)
    assert B.dflash_block_attention_check(p) == B.DFLASH_OK
    # a decreasing step, a nonzero start, only one of the two arrays
    bad = dict(good, host_cu_ctx_lens=[0, 2000, 1000] + good["host_cu_ctx_lens"][3:])
    assert B.dflash_block_attention_check(P(**bad)) == B.DFLASH_ERR_INVALID_ARG
    bad = dict(good, host_cu_blk_lens=[1] + good["host_cu_blk_lens"][1:])
    assert B.dflash_block_attention_check(P(**bad)) == B.DFLASH_ERR_INVALID_ARG
    with pytest.raises(ValueError):
        P(host_cu_ctx_lens=good["host_cu_ctx_lens"])
    q = P()
    q.host_cu_ctx_lens = ctypes.cast(p._host_lens[0], ctypes.c_void_p)
    assert B.dflash_block_attention_check(q) == B.DFLASH_ERR_INVALID_ARG


def _paged_call(lib, p, pg):
    # validation happens before any pointer is touched; NULL device pointers
    return lib.dflash_block_attention_paged(ctypes.byref(p), ctypes.byref(pg) if pg else None,
                                            None, None, None, None, None, None, None, None, None,
                                            None, 0, None)


def test_paged_validation(lib):
    pg = B.PagedCtx(None, 64, 16, 1000)
    assert _paged_call(lib, P(), None) == B.DFLASH_ERR_INVALID_ARG
    assert _paged_call(lib, P(), B.PagedCtx(None, 64, 8, 1000)) == B.DFLASH_ERR_UNSUPPORTED
    assert _paged_call(lib, P(), B.PagedCtx(None, 64, 16, 0)) == B.DFLASH_ERR_INVALID_ARG
    assert _paged_call(lib, P(), B.PagedCtx(None, 0, 16, 10)) == B.DFLASH_ERR_INVALID_ARG
    assert _paged_call(lib, P(split_keys=32768), pg) == B.DFLASH_ERR_INVALID_ARG
    assert _paged_call(lib, P(), pg) == B.DFLASH_ERR_INVALID_ARG  # block_table NULL
    assert _paged_call(lib, P(total_blk=0, max_blk_len=0), pg) == B.DFLASH_OK  # nothing to do
    # the paged workspace holds at least the packed one; a split past the paged cap has none
    assert B.dflash_block_attention_paged_workspace_size(P()) >= \
        B.dflash_block_attention_workspace_size(P())
    assert B.dflash_block_attention_paged_workspace_size(P(split_keys=32768)) == 0


def test_phase_trace_build(lib):
    # the diagnostic build appends its records to the product workspace layout
    # and is the only library exporting the layout query
    from block_diffusion_draft_dflash_amd.build import TRACE_LIB
    assert not hasattr(lib, "dflash_phase_trace_layout")
    tr = ctypes.CDLL(TRACE_LIB)
    f = tr.dflash_phase_trace_layout
    f.restype = ctypes.c_size_t
    f.argtypes = [ctypes.POINTER(B.BlockAttnParams), ctypes.c_int, ctypes.POINTER(ctypes.c_int64),
                  ctypes.POINTER(ctypes.c_int64)]
    tr.dflash_block_attention_workspace_size.restype = ctypes.c_size_t
    tr.dflash_block_attention_workspace_size.argtypes = [ctypes.POINTER(B.BlockAttnParams)]
    for kw in (dict(), dict(num_reqs=64, total_ctx=64 * 3000, total_blk=64 * 16), dict(split_keys=128)):
        p = P(**kw)
        nm, ng = ctypes.c_int64(), ctypes.c_int64()
        off = f(ctypes.byref(p), 0, ctypes.byref(nm), ctypes.byref(ng))
        assert off == B.dflash_block_attention_workspace_size(p)
        assert nm.value >= 8 and ng.value == p.num_reqs * 8 * 4
        assert tr.dflash_block_attention_workspace_size(ctypes.byref(p)) == off + 64 * (nm.value + ng.value)


def test_kv_scatter_validation(lib):
    f = lib.dflash_kv_scatter
    assert f(7, None, None, None, 4, 8, 128, None, None, 64, None) == B.DFLASH_ERR_INVALID_ARG
    assert f(B.DFLASH_BF16, None, None, None, 4, 1, 2, None, None, 64, None) == B.DFLASH_ERR_UNSUPPORTED
    assert f(B.DFLASH_BF16, None, None, None, 0, 8, 128, None, None, 64, None) == B.DFLASH_OK
    assert f(B.DFLASH_BF16, None, None, None, 4, 8, 128, None, None, 64, None) == B.DFLASH_ERR_INVALID_ARG
    assert f(B.DFLASH_BF16, None, None, None, -1, 8, 128, None, None, 64, None) == B.DFLASH_ERR_INVALID_ARG


def test_block_qkv_validation(lib):
    f = lib.dflash_block_qkv
    fake = 4096  # never dereferenced: every case fails (or returns) before a launch
    args = lambda t=4, h=4096, hq=32, hkv=8, dh=128, eps=1e-6, ptr=fake, ws=fake, wsb=1 << 30: (
        ptr, None, ptr, ptr, t, h, hq, hkv, dh, eps, ptr, ptr, ptr, ws, wsb, None)
    assert f(*args(t=0, ptr=None, ws=None, wsb=0)) == B.DFLASH_OK          # nothing to do
    assert f(*args(dh=96)) == B.DFLASH_ERR_UNSUPPORTED
    assert f(*args(h=100)) == B.DFLASH_ERR_UNSUPPORTED
    assert f(*args(h=16384)) == B.DFLASH_ERR_UNSUPPORTED
    assert f(*args(hq=30)) == B.DFLASH_ERR_INVALID_ARG                       # Hq % Hkv
    assert f(*args(t=-1)) == B.DFLASH_ERR_INVALID_ARG
    assert f(*args(eps=float("nan"))) == B.DFLASH_ERR_INVALID_ARG
    assert f(*args(ptr=None)) == B.DFLASH_ERR_INVALID_ARG
    assert f(*args(ptr=fake + 2)) == B.DFLASH_ERR_INVALID_ARG               # misaligned
    assert f(*args(ws=None)) == B.DFLASH_ERR_WORKSPACE
    assert f(*args(ws=fake + 16)) == B.DFLASH_ERR_WORKSPACE                 # not 256-aligned
    assert f(*args(wsb=16)) == B.DFLASH_ERR_WORKSPACE
    assert "workspace" in lib.dflash_last_error().decode()


def test_o_proj_validation(lib):
    f = lib.dflash_o_proj
    fake = 4096
    assert f(None, None, 0, 4096, 4096, None, None, 0, None) == B.DFLASH_OK
    assert f(fake, fake, 4, 4000, 4096, fake, fake, 1 << 30, None) == B.DFLASH_ERR_UNSUPPORTED
    assert f(fake, fake, 4, 4096, 100, fake, fake, 1 << 30, None) == B.DFLASH_ERR_UNSUPPORTED
    assert f(None, fake, 4, 4096, 4096, fake, fake, 1 << 30, None) == B.DFLASH_ERR_INVALID_ARG
    assert f(fake, fake, 4, 4096, 4096, fake, None, 0, None) == B.DFLASH_ERR_WORKSPACE


def test_layer_workspace_sizes(lib):
    # small T splits H across workgroups (f32 partials); large T needs only the normed rows
    small = B.dflash_block_qkv_workspace_size(128, 4096, 32, 8, 128)
    assert small >= 128 * 4096 * 2 + 2 * 128 * 6144 * 4 and small % 256 == 0
    assert B.dflash_block_qkv_workspace_size(4096, 4096, 32, 8, 128) == 4096 * 4096 * 2
    assert B.dflash_o_proj_workspace_size(4096, 4096, 4096) == 0
    assert B.dflash_o_proj_workspace_size(128, 4096, 4096) >= 2 * 128 * 4096 * 4
    assert B.dflash_block_qkv_workspace_size(-1, 4096, 32, 8, 128) == 0
    # the host plan of the projections at 128 rows: q/k/v (N = 6144, K = 4096) on
    # 48 wide column tiles x 5 uneven K slices; o_proj (8 steps a slice on wide
    # tiles: too short) on 64 narrow tiles x 4 slices; the fc combine (K = 5 x
    # 4096) on 32 wide tiles x 8 slices; one f32 [T, N] partial per slice
    assert small == 128 * 4096 * 2 + 5 * 128 * 6144 * 4
    assert B.dflash_o_proj_workspace_size(128, 4096, 4096) == 4 * 128 * 4096 * 4
    assert B.dflash_fc_combine_workspace_size(128, 4096, 5) == 128 * 20480 * 2 + 8 * 128 * 4096 * 4


def test_workspace_sizes(lib):
    bf = B.dflash_block_attention_workspace_size(P())
    assert bf > 0 and bf % 256 == 0
    # f32 runs unsplit and needs no workspace
    assert B.dflash_block_attention_workspace_size(P(dtype=B.DFLASH_F32)) == 0
    # more context -> at least as much workspace; forced small splits -> more
    assert B.dflash_block_attention_workspace_size(P(total_ctx=100000)) >= bf
    assert B.dflash_block_attention_workspace_size(P(split_keys=64)) > \
        B.dflash_block_attention_workspace_size(P(split_keys=4096))
    # the plan is a pure function of the parameters
    assert B.dflash_block_attention_workspace_size(P()) == bf


def test_context_kv_workspace_size(lib):
    n = B.dflash_context_kv_workspace_size(131072, 4096, 8, 128)
    assert n >= 2 * 1024 * 4096 * 2  # the folded K and V weights (bf16)
    assert B.dflash_context_kv_workspace_size(-1, 4096, 8, 128) == 0


def test_binding_requires_library(tmp_path):
    with pytest.raises(RuntimeError):
        B.load.__wrapped__(str(tmp_path / "missing.so")) if hasattr(B.load, "__wrapped__") else \
            _load_fresh(str(tmp_path / "missing.so"))


def _load_fresh(path):
    saved = B._lib
    B._lib = None
    try:
        return B.load(path)
    finally:
        B._lib = saved


def test_prepare_inputs_validation(lib):
    import ctypes
    good = dict(num_reqs=2, max_num_reqs=3, max_num_tokens=8, num_query_per_req=3,
                num_speculative_steps=2, block_size=16, block_table_stride=4, max_model_len=100,
                mask_token_id=5, sample_from_anchor=0, num_states=2, num_target_tokens=4)
    fake = ctypes.c_void_p(4096)
    pin = B.PrepareIn(*([fake] * len(B.PREP_IN)))
    pout = B.PrepareOut(*([fake] * len(B.PREP_OUT)))
    f = lambda **ch: lib.dflash_prepare_inputs(ctypes.byref(B.PrepareParams(**dict(good, **ch))),
                                               ctypes.byref(pin), ctypes.byref(pout), None)
    assert f(num_reqs=0) == B.DFLASH_ERR_INVALID_ARG
    assert f(max_num_reqs=1) == B.DFLASH_ERR_INVALID_ARG
    assert f(max_num_tokens=5) == B.DFLASH_ERR_INVALID_ARG
    assert f(num_speculative_steps=3) == B.DFLASH_ERR_INVALID_ARG        # must be nqpr - 1 here
    assert f(block_size=0) == B.DFLASH_ERR_INVALID_ARG
    assert f(num_target_tokens=0) == B.DFLASH_ERR_INVALID_ARG
    nul = B.PrepareIn(*([fake] * (len(B.PREP_IN) - 1) + [None]))
    assert lib.dflash_prepare_inputs(ctypes.byref(B.PrepareParams(**good)), ctypes.byref(nul),
                                     ctypes.byref(pout), None) == B.DFLASH_ERR_INVALID_ARG


def test_fc_combine_validation(lib):
    f = lib.dflash_fc_combine
    fake = 4096
    assert f(None, None, 0, 4096, 5, None, None, 0, None) == B.DFLASH_OK
    assert f(fake, fake, 4, 100, 5, fake, fake, 1 << 30, None) == B.DFLASH_ERR_UNSUPPORTED
    assert f(fake, fake, 4, 4096, 0, fake, fake, 1 << 30, None) == B.DFLASH_ERR_INVALID_ARG
    assert f(fake, fake, 4, 4096, 5, fake, None, 0, None) == B.DFLASH_ERR_WORKSPACE
    assert B.dflash_fc_combine_workspace_size(128, 4096, 5) >= 128 * 4096 * 5 * 2


def test_noalloc_rejects_before_touching_the_gpu(lib):
    # host-side checks of the allocation-free entry point return before any
    # HIP call: invalid parameters, a batch whose workspace exceeds the
    # library's per-GPU scratch, and an empty batch (nothing to do)
    f = lambda p: lib.dflash_block_attention_noalloc(ctypes.byref(p), None, None, None, None, None,
                                                     None, None, None, None, None)
    assert f(P(num_reqs=0)) == B.DFLASH_ERR_INVALID_ARG
    big = P(total_ctx=1 << 24, split_keys=64)
    assert B.dflash_block_attention_workspace_size(big) > B.NOALLOC_SCRATCH_BYTES
    assert f(big) == B.DFLASH_ERR_WORKSPACE
    assert "scratch" in lib.dflash_last_error().decode()
    assert f(P(total_blk=0, max_blk_len=0)) == B.DFLASH_OK


def test_noalloc_scratch_size_matches_header():
    text = open(HEADER).read()
    m = re.search(r"#define DFLASH_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == B.NOALLOC_SCRATCH_BYTES


_NO_DEVICE_CHILD = r"""
import ctypes, sys
sys.path.insert(0, sys.argv[1])
from block_diffusion_draft_dflash_amd import binding as B
lib = B.load()
fake = ctypes.c_void_p(1 << 40)  # valid-looking, aligned; never dereferenced on the host
rc = lib.dflash_qk_norm_rope(B.DFLASH_BF16, fake, fake, fake, fake, fake, 16, 32, 8, 128,
                             ctypes.c_float(1e-6), fake, 4096, None)
print(rc, lib.dflash_last_error().decode())
"""


def test_launch_without_a_device_reports_a_hip_error():
    # A call whose arguments pass every host check, made where the HIP runtime
    # has no device: the launch fails and the call says so (DFLASH_ERR_HIP with
    # the runtime's message) instead of crashing or reporting success.
    env = dict(os.environ, HIP_VISIBLE_DEVICES="-1", ROCR_VISIBLE_DEVICES="-1",
               CUDA_VISIBLE_DEVICES="-1", DFLASH_VALIDATE="0")
    res = subprocess.run([sys.executable, "-c", _NO_DEVICE_CHILD, ROOT], env=env,
                         capture_output=True, text=True, timeout=300)
    assert res.returncode == 0, res.stderr[-2000:]
    rc, _, msg = res.stdout.strip().splitlines()[-1].partition(" ")
    assert int(rc) == B.DFLASH_ERR_HIP, res.stdout
    assert "HIP error" in msg, msg


_BIG_GRID_CHILD = r"""
import ctypes, sys
sys.path.insert(0, sys.argv[1])
from block_diffusion_draft_dflash_amd import binding as B
lib = B.load()
fake = ctypes.c_void_p(1 << 40)
# 2^40 rows of 40 heads: more workgroups than one launch addresses
rc = lib.dflash_qk_norm_rope(B.DFLASH_BF16, fake, fake, fake, fake, fake, 1 << 40, 32, 8, 128,
                             ctypes.c_float(1e-6), fake, 4096, None)
print(rc, lib.dflash_last_error().decode())
"""


def test_grid_beyond_one_launch_is_refused():
    # a grid that would not fit 32 bits is refused before any launch (the
    # runtime's "invalid configuration" error), never truncated into a launch
    # that covers part of the rows
    env = dict(os.environ, HIP_VISIBLE_DEVICES="-1", ROCR_VISIBLE_DEVICES="-1",
               CUDA_VISIBLE_DEVICES="-1", DFLASH_VALIDATE="0")
    res = subprocess.run([sys.executable, "-c", _BIG_GRID_CHILD, ROOT], env=env,
                         capture_output=True, text=True, timeout=300)
    assert res.returncode == 0, res.stderr[-2000:]
    rc, _, msg = res.stdout.strip().splitlines()[-1].partition(" ")
    assert int(rc) == B.DFLASH_ERR_HIP, res.stdout
    assert "configuration" in msg, msg


_TRACE_CHILD = r"""
import ctypes, sys
sys.path.insert(0, sys.argv[1])
from block_diffusion_draft_dflash_amd import binding as B
lib = B.load()
fake = ctypes.c_void_p(1 << 40)
ctx, blk = [0, 700, 1900, 2400], [0, 16, 32, 48]
p = B.make_block_attn_params(3, 32, 8, 128, B.DFLASH_BF16, 2400, 48, 16, 128 ** -0.5, False, 0, 0,
                             host_cu_ctx_lens=ctx, host_cu_blk_lens=blk)
ws = lib.dflash_block_attention_workspace_size(ctypes.byref(p))
rc = lib.dflash_block_attention(ctypes.byref(p), None, fake, fake, fake, fake, fake, fake, fake, fake,
                                fake, ws, None)
print(rc, ws)
"""


def test_trace_mode_logs_the_work_split():
    # DFLASH_TRACE prints each attention call's decomposition before the launch
    # (here the launch itself then fails: no device is visible to the child)
    env = dict(os.environ, HIP_VISIBLE_DEVICES="-1", ROCR_VISIBLE_DEVICES="-1",
               CUDA_VISIBLE_DEVICES="-1", DFLASH_VALIDATE="0", DFLASH_TRACE="1")
    res = subprocess.run([sys.executable, "-c", _TRACE_CHILD, ROOT], env=env, capture_output=True,
                         text=True, timeout=300)
    assert res.returncode == 0, res.stderr[-2000:]
    rc, ws = (int(x) for x in res.stdout.split()[-2:])
    assert rc == B.DFLASH_ERR_HIP
    log = res.stderr
    assert "dflash trace: block_attention packed: 3 requests, Hq 32, Hkv 8, Dh 128" in log, log
    assert "plan: host, split" in log and f"workspace {ws} bytes" in log, log
    for r, (c, b) in enumerate([(700, 16), (1200, 16), (500, 16)]):
        assert f"request {r}: {c} context + {b} block rows" in log, log
    env["DFLASH_TRACE"] = "0"
    quiet = subprocess.run([sys.executable, "-c", _TRACE_CHILD, ROOT], env=env, capture_output=True,
                           text=True, timeout=300)
    assert "dflash trace" not in quiet.stderr
