"""pst_decode_attn_noalloc: the entry point that allocates nothing, against
pst_decode_attn (same plan, same kernels: the outputs must be identical),
called twice in a row with the second input smaller, and its size limit."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import workloads  # noqa: E402

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a GPU", allow_module_level=True)

import prefix_shared_tree_amd as pst  # noqa: E402


def _pair(spec, out_dtype="f32", **plan_kw):
    """Outputs of pst_decode_attn and of pst_decode_attn_noalloc on the same plan."""
    q, k, v = workloads.make_tensors(spec, "cuda")
    tree = pst.Tree.from_spec(spec, out_dtype=out_dtype)
    plan = pst.Plan(tree, **plan_kw)
    ref, ref_lse = pst.decode_attn(plan, q, k, v)
    out = torch.full_like(ref, float("nan"))
    lse = torch.full_like(ref_lse, float("nan"))
    pst.decode_attn_noalloc(plan, q, k, v, out=out, lse=lse)
    torch.cuda.synchronize()
    print(f"  {spec.name}: workspace {plan.workspace_bytes} bytes", flush=True)
    return ref, ref_lse, out, lse


def test_noalloc_matches_decode_attn_twice_smaller_second():
    # First the few-shot tree (18 MiB of partials), then the tiny float32
    # tree (20 KiB): the second call reuses the array the first filled.
    for name in ("3", "1"):
        ref, ref_lse, out, lse = _pair(workloads.config(name))
        assert torch.equal(out, ref) and torch.equal(lse, ref_lse), name


def test_noalloc_skewed_mqa_and_flattened():
    # The largest partials of the workloads (5-mqa, 81 MiB) and a flattened plan.
    ref, ref_lse, out, lse = _pair(workloads.config("5-mqa"))
    assert torch.equal(out, ref) and torch.equal(lse, ref_lse)
    ref, ref_lse, out, lse = _pair(workloads.config("3"), flatten=256)
    assert torch.equal(out, ref) and torch.equal(lse, ref_lse)


def test_noalloc_bf16_output():
    # bf16 output: the partials in the array are fp16 with their scales; the
    # document-QA tree, then the smaller few-shot tree.
    for name in ("2", "3"):
        ref, ref_lse, out, lse = _pair(workloads.config(name), out_dtype="bf16")
        assert out.dtype == torch.bfloat16
        assert torch.equal(out, ref) and torch.equal(lse, ref_lse), name


def test_noalloc_refuses_plans_beyond_its_array():
    # One 600,000-token node cut into 64-token pieces: 9,375 partial slots of
    # 32 heads x 129 floats, about 148 MiB, beyond the 128 MiB array.
    n = 600_000
    spec = workloads.TreeSpec("long", np.array([-1]), np.array([n]), np.array([0]), np.array([0]), 32, 1, 128,
                              "bf16", 5)
    tree = pst.Tree.from_spec(spec, out_dtype="f32")
    plan = pst.Plan(tree, fixed_chunk=64)
    assert plan.workspace_bytes > pst.NOALLOC_SCRATCH_BYTES
    q = torch.zeros((1, 32, 128), dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros((1, n, 128), dtype=torch.bfloat16, device="cuda")
    out = torch.zeros((1, 32, 128), dtype=torch.float32, device="cuda")
    with pytest.raises(pst.PstError) as e:
        pst.decode_attn_noalloc(plan, q, kv, kv, out=out)
    assert e.value.code == "PST_E_WORKSPACE" and "bytes" in str(e.value)
    assert torch.count_nonzero(out) == 0  # nothing was launched
