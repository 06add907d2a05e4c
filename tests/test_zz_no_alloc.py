"""basp_seq_to_head_unfused_noalloc (the library's own workspace) against
basp_seq_to_head_unfused with a caller-owned workspace, through the C ABI,
bit for bit, and against the oracle (MI355X only).

Two calls in a row, the second with a smaller input, so that the second call
runs on an array that still holds the first call's larger contents; then the
largest plan the array admits, and the first plan above it (rejected before
any device call).
"""
import numpy as np
import pytest
import torch

import oracle
from sequence_re_layout_amd import inputs

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from sequence_re_layout_amd import binding as b
else:  # collected on a machine without a GPU: every test here is skipped
    b = None

MODE = {"basp": 1, "ulysses": 0}


def needs_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def bits(t):
    return inputs.raw_bits(t.cpu())


def noalloc_matches(shape, mode, layout, dtype):
    """One call of each entry point on the same inputs; both outputs must
    be equal bit for bit and equal to the oracle's."""
    N, B, S, Hq, Hkv, d = shape
    code, tdt = (b.BASP_INT32, torch.int32) if dtype == "int32" else (b.BASP_BF16, torch.bfloat16)
    plan = b.basp_plan_create_ex(N, B, S, Hq, Hkv, d, code, MODE[mode], layout)
    i = plan.info
    assert b.basp_unfused_workspace_bytes(plan) <= b.BASP_NOALLOC_SCRATCH_BYTES
    nq, nkv = i["q_elems"], i["kv_elems"]
    if dtype == "int32":
        q, k, v = (inputs.tags_int32(nq, 0), inputs.tags_int32(nkv, nq), inputs.tags_int32(nkv, nq + nkv))
    else:
        q, k, v = (inputs.normal_bf16(nq, inputs.SEED_Q), inputs.normal_bf16(nkv, inputs.SEED_K),
                   inputs.normal_bf16(nkv, inputs.SEED_V))
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    ws = torch.empty(b.basp_unfused_workspace_bytes(plan), dtype=torch.uint8, device="cuda")
    ref = torch.empty(i["qkv_elems"], dtype=tdt, device="cuda")
    b.basp_seq_to_head_unfused(plan, qd, kd, vd, ref, ws)
    out = torch.empty(i["qkv_elems"], dtype=tdt, device="cuda")
    out.view(torch.int16 if out.element_size() == 2 else torch.int32).fill_(-1)
    b.basp_seq_to_head_unfused_noalloc(plan, qd, kd, vd, out)
    torch.cuda.synchronize()
    got = bits(out)
    assert np.array_equal(got, bits(ref)), "differs from the caller-workspace entry point"
    want = oracle.seq_to_head_qkv(inputs.raw_bits(q), inputs.raw_bits(k), inputs.raw_bits(v),
                                  MODE[mode], N, B, S, Hq, Hkv, d, layout)
    assert np.array_equal(got, want), "differs from the oracle"


@pytest.mark.parametrize("mode", ["basp", "ulysses"])
def test_noalloc_two_calls_second_smaller(mode):
    needs_gpu()
    print("noalloc two calls", mode, flush=True)
    noalloc_matches((4, 2, 1024, 8, 8, 64), mode, 0, "bf16")     # 12 MiB of workspace
    noalloc_matches((6, 3, 6 * 37, 12, 6, 40), mode, 1, "int32")  # smaller, ragged, token-major


def test_noalloc_largest_plan_and_the_limit():
    needs_gpu()
    print("noalloc largest plan", flush=True)
    big = (8, 2, 4096, 16, 8, 64)   # workspace exactly the array's size
    plan = b.basp_plan_create(*big, b.BASP_BF16, b.BASP_MODE_BASP)
    assert b.basp_unfused_workspace_bytes(plan) == b.BASP_NOALLOC_SCRATCH_BYTES
    noalloc_matches(big, "basp", 0, "bf16")
    noalloc_matches((4, 2, 64, 8, 4, 16), "ulysses", 0, "bf16")   # then a small one again
    over = b.basp_plan_create(8, 2, 4104, 16, 8, 64, b.BASP_BF16, b.BASP_MODE_BASP)
    i = over.info
    x = torch.empty(i["qkv_elems"], dtype=torch.bfloat16, device="cuda")
    with pytest.raises(b.BaspError) as e:
        b.basp_seq_to_head_unfused_noalloc(over, x[:i["q_elems"]], x[:i["kv_elems"]], x[:i["kv_elems"]],
                                           torch.empty_like(x))
    assert e.value.status == b.BASP_ERR_UNSUPPORTED
    empty = b.basp_plan_create(8, 2, 0, 16, 8, 64, b.BASP_BF16, b.BASP_MODE_BASP)
    z = torch.empty(0, dtype=torch.bfloat16, device="cuda")
    b.basp_seq_to_head_unfused_noalloc(empty, z, z, z, z)
    torch.cuda.synchronize()
