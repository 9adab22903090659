"""Exercise every host-side path of libdflash under AddressSanitizer and
UndefinedBehaviorSanitizer (host code only; run by test_host_sanitizers.py in a
child process with the sanitizer runtime preloaded, on a machine with or
without a GPU).

Device pointers are fake (aligned, never dereferenced on the host): each call
either fails validation before it would touch them, or validates, plans the
work on the host (split sizes, the host schedule with its launch order) and
then reaches the HIP launch, which fails without a GPU (DFLASH_ERR_HIP) or is
not reached here because the argument checks reject the call first. Any
out-of-bounds access or undefined behaviour in the validation and planning code
aborts the process with the sanitizer's report."""
import ctypes
import itertools
import os
import sys

import numpy as np

sys.path.insert(0, sys.argv[2])
import torch  # noqa: E402

# The fake pointers must never reach a real launch: run only where no GPU is
# visible (the parent also hides every device from this process).
if torch.cuda.device_count() > 0:
    print("host sanitizer driver: a GPU is visible; not running", flush=True)
    sys.exit(3)

from block_diffusion_draft_dflash_amd import binding as B  # noqa: E402

lib = B.load(sys.argv[1])
FAKE = ctypes.c_void_p(1 << 40)  # 256-byte aligned, never dereferenced on the host
OK_OR_HIP = (B.DFLASH_OK, B.DFLASH_ERR_HIP)


def P(**kw):
    base = dict(num_reqs=8, num_q_heads=32, num_kv_heads=8, head_dim=128, dtype=B.DFLASH_BF16,
                total_ctx=10000, total_blk=128, max_blk_len=16, scale=128 ** -0.5, causal=False,
                window=0, split_keys=0)
    base.update(kw)
    return B.make_block_attn_params(**base)


def attention(p, paged=False, prologue=None, ws_bytes=1 << 40):
    pro = B.QkPrologue(FAKE, FAKE, FAKE, FAKE, 4096, 1e-6) if prologue else None
    pro_ref = ctypes.byref(pro) if pro is not None else None
    if paged:
        pg = B.PagedCtx(FAKE, 64, 16, 100000)
        return lib.dflash_block_attention_paged(ctypes.byref(p), ctypes.byref(pg), pro_ref, FAKE, FAKE,
                                                FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws_bytes, None)
    return lib.dflash_block_attention(ctypes.byref(p), pro_ref, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                      FAKE, FAKE, FAKE, ws_bytes, None)


def cu(lengths):
    return [0] + list(itertools.accumulate(int(x) for x in lengths))


rng = np.random.default_rng(7)
calls = 0
codes = {}

# validation of odd parameter sets (every status is acceptable; no report may fire)
for kw in [dict(), dict(num_reqs=0), dict(num_q_heads=30), dict(num_kv_heads=0), dict(head_dim=96),
           dict(head_dim=64), dict(dtype=B.DFLASH_F32), dict(dtype=7), dict(total_ctx=-1),
           dict(max_blk_len=200), dict(max_blk_len=0), dict(window=64), dict(window=64, causal=True),
           dict(split_keys=100), dict(split_keys=64), dict(split_keys=1 << 24),
           dict(total_ctx=2 ** 30), dict(total_ctx=2 ** 62, total_blk=2 ** 62), dict(total_ctx=0),
           dict(total_blk=0, max_blk_len=0), dict(num_q_heads=2 ** 31 - 1, num_kv_heads=1),
           dict(num_reqs=70000, total_ctx=70000 * 10, total_blk=70000 * 16),
           dict(num_q_heads=128, num_kv_heads=1, max_blk_len=64, total_blk=512)]:
    p = P(**kw)
    lib.dflash_block_attention_check(ctypes.byref(p))
    lib.dflash_block_attention_workspace_size(ctypes.byref(p))
    lib.dflash_block_attention_paged_workspace_size(ctypes.byref(p))
    for paged, fused in itertools.product((False, True), (False, True)):
        attention(p, paged, fused)
        calls += 1

# host-planned batches: random varlen requests up to the host table's 64, with
# empty contexts and blocks, windows, forced splits and more units than the table
for trial in range(400):
    # every other batch in the DFLASH_VALIDATE mode (its device reads fail here)
    os.environ["DFLASH_VALIDATE"] = "1" if trial % 2 else "0"
    r = int(rng.integers(1, 80))
    ctx = rng.integers(0, 9000, r) * (rng.random(r) > 0.1)
    blk = rng.integers(0, 65, r) * (rng.random(r) > 0.1)
    causal = bool(rng.random() < 0.4)
    window = int(rng.integers(1, 5000)) if causal and rng.random() < 0.5 else 0
    split = int(rng.choice([0, 0, 0, 64, 128, 4096]))
    hkv = int(rng.choice([1, 2, 4, 8]))
    hq = hkv * int(rng.choice([1, 2, 4, 8, 16]))
    dh = int(rng.choice([64, 128]))
    maxb = max(1, int(blk.max())) if blk.sum() else 0
    p = P(num_reqs=r, num_q_heads=hq, num_kv_heads=hkv, head_dim=dh, total_ctx=int(ctx.sum()),
          total_blk=int(blk.sum()), max_blk_len=maxb, causal=causal, window=window, split_keys=split,
          host_cu_ctx_lens=cu(ctx), host_cu_blk_lens=cu(blk))
    st = lib.dflash_block_attention_check(ctypes.byref(p))
    ws = lib.dflash_block_attention_workspace_size(ctypes.byref(p))
    for paged, fused in itertools.product((False, True), (False, True)):
        rc = attention(p, paged, fused and maxb <= 64, ws_bytes=max(ws, 1))
        codes[rc] = codes.get(rc, 0) + 1
        assert st != B.DFLASH_OK or rc in OK_OR_HIP + (B.DFLASH_ERR_UNSUPPORTED, B.DFLASH_ERR_INVALID_ARG), rc
        calls += 1
    lib.dflash_block_attention_noalloc(ctypes.byref(p), None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                       FAKE, None)

os.environ["DFLASH_VALIDATE"] = "0"

# the other entry points' planners and checks (then once more in the DFLASH_VALIDATE mode)
for t, h in itertools.product([0, 1, 5, 128, 255, 256, 1000, 4096], [64, 512, 4096, 8192]):
    lib.dflash_context_kv_workspace_size(t, h, 8, 128)
    lib.dflash_context_kv(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, t, h, 8, 128, ctypes.c_float(1e-6), FAKE,
                          32768, FAKE, FAKE, FAKE, 1 << 40, None)
    lib.dflash_block_qkv_workspace_size(t, h, 32, 8, 128)
    lib.dflash_block_qkv(FAKE, FAKE, FAKE, FAKE, t, h, 32, 8, 128, ctypes.c_float(1e-6), FAKE, FAKE,
                         FAKE, FAKE, 1 << 40, None)
    lib.dflash_o_proj_workspace_size(t, h, 4096)
    lib.dflash_o_proj(FAKE, FAKE, t, h, 4096, FAKE, FAKE, 1 << 40, None)
    for taps in (1, 5):
        lib.dflash_fc_combine_workspace_size(t, h, taps)
        lib.dflash_fc_combine(FAKE, FAKE, t, h, taps, FAKE, FAKE, 1 << 40, None)
    lib.dflash_qk_norm_rope(B.DFLASH_BF16, FAKE, FAKE, FAKE, FAKE, FAKE, t, 32, 8, 128,
                            ctypes.c_float(1e-6), FAKE, 4096, None)
    lib.dflash_kv_scatter(B.DFLASH_BF16, FAKE, FAKE, FAKE, t, 8, 128, FAKE, FAKE, 100000, None)
    calls += 10
# sizes whose products would not fit 32 bits: every query returns 0 and every
# call an error status, with no overflow on the way
big = 1 << 30
for t in (1, 300, 1 << 40):
    assert lib.dflash_context_kv_workspace_size(t, 4096, big, 128) == 0
    assert lib.dflash_context_kv_workspace_size(t, big, 8, 128) == 0
    assert lib.dflash_block_qkv_workspace_size(t, 4096, big, big, 128) == 0
    assert lib.dflash_fc_combine_workspace_size(t, 4096, big) == 0
    for h, hkv in ((4096, big), (4096, 1 << 24), (big, 8)):
        assert lib.dflash_context_kv(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, t, h, hkv, 128, ctypes.c_float(1e-6),
                                     FAKE, 32768, FAKE, FAKE, FAKE, 1 << 40, None) < 0
    assert lib.dflash_block_qkv(FAKE, FAKE, FAKE, FAKE, t, 4096, big, big, 128, ctypes.c_float(1e-6), FAKE,
                                FAKE, FAKE, FAKE, 1 << 40, None) < 0
    assert lib.dflash_fc_combine(FAKE, FAKE, t, 4096, big, FAKE, FAKE, 1 << 40, None) < 0
    calls += 6
assert lib.dflash_o_proj_workspace_size(1 << 40, 4096, 4096) == 0
os.environ["DFLASH_VALIDATE"] = "1"
for t in (1, 300):
    lib.dflash_qk_norm_rope(B.DFLASH_BF16, FAKE, FAKE, FAKE, FAKE, FAKE, t, 32, 8, 128,
                            ctypes.c_float(1e-6), FAKE, 4096, None)
    lib.dflash_kv_scatter(B.DFLASH_BF16, FAKE, FAKE, FAKE, t, 8, 128, FAKE, FAKE, 100000, None)
    lib.dflash_context_kv(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, t, 4096, 8, 128, ctypes.c_float(1e-6), FAKE,
                          32768, FAKE, FAKE, FAKE, 1 << 40, None)
    calls += 3
os.environ["DFLASH_VALIDATE"] = "0"
lib.dflash_rope_table(FAKE, 4096, 128, ctypes.c_double(1e6), None)
# most random batches pass the checks and reach the planners and the launch
assert codes.get(B.DFLASH_ERR_HIP, 0) + codes.get(B.DFLASH_OK, 0) > 800, codes
print(f"host sanitizer driver: {calls} calls (batch status counts {codes}), no report", flush=True)
