"""The seeded generator: determinism, shapes and the popularity statistics
that "Multi-LoRA serving: S-LoRA, Punica and adapter batching" ("How many
adapters are actually in a batch?") reports for a Zipf batch of 64."""
import numpy as np
import pytest

from workloads import bf16_bits_from_f32, f32_from_bf16_bits, make_workload, zipf_probs


def test_bf16_rne():
    v = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 1.0 + 2 ** -8 + 2 ** -20], np.float32)
    b = bf16_bits_from_f32(v)
    # ties to even: 1 + 2^-8 -> 1.0 (0x3F80); 1 + 3*2^-8 -> 1 + 2^-6 (0x3F82); above the tie rounds up
    assert list(b) == [0x3F80, 0x3F80, 0x3F82, 0xC020, 0x3F81]
    assert np.array_equal(f32_from_bf16_bits(b)[[0, 3]], np.array([1.0, -2.5], np.float32))


def test_deterministic_and_shapes():
    a = make_workload("c1")
    b = make_workload("c1")
    assert np.array_equal(a.x(), b.x()) and np.array_equal(a.w0(), b.w0())
    assert np.array_equal(a.free_order, b.free_order)
    A, B = a.adapter_AB(1)
    assert A.shape == (8, 256) and B.shape == (8, 256) and A.dtype == np.float32
    c = make_workload("c1", seed=1)
    assert not np.array_equal(a.x(), c.x())
    assert sorted(a.free_order) == list(range(64))


def test_c4_segments():
    wl = make_workload("c4")
    lens = [r.n_tokens for r in wl.requests]
    assert len(lens) == 16 and all(64 <= n <= 1024 for n in lens)
    assert sum(1 for r in wl.requests if r.adapter_id < 0) == 2


def test_c3_nulls_and_kv():
    wl = make_workload("c3")
    ra = wl.row_adapter()
    assert ra.shape == (256,) and int((ra < 0).sum()) == 26
    assert sum(1 for op in wl.setup_ops if op[0] == "alloc_kv") == 2000


def expected_distinct(n_adapters, s, batch):
    p = zipf_probs(n_adapters, s)
    return float(np.sum(1.0 - (1.0 - p) ** batch))


def test_zipf_distinct_adapters():
    # closed form E[distinct] = sum_k 1 - (1 - p_k)^64 for Zipf(1.0) over 1000 adapters = 43.9,
    # inside the 33-62 range the page's simulation reports for batches of 64
    e = expected_distinct(1000, 1.0, 64)
    assert 43.5 < e < 44.5 and 33 <= e <= 62
    counts = [len(set(r.adapter_id for r in make_workload("c2", seed=s).requests)) for s in range(40)]
    assert abs(np.mean(counts) - e) < 3.0 * np.std(counts) / np.sqrt(len(counts)) + 0.5
    assert 25 <= min(counts) and max(counts) <= 62


def test_fp8_base_draw():
    """The FP8 base: codes with no NaN, each row's largest |w| at the top code
    (448 after its scale), and scale * value within half an E4M3 step of the
    same fp32 draw the bf16 base rounds (relative 2^-4 for normal values)."""
    import torch
    wl = make_workload("c1")
    codes, scale = wl.w0_fp8()
    assert codes.dtype == np.uint8 and codes.shape == (wl.d_out[0], wl.d_in[0]) and scale.shape == (wl.d_out[0],)
    assert not np.any((codes & 0x7F) == 0x7F)
    vals = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    assert np.all(np.abs(vals).max(axis=1) == 448.0)
    w = wl.w0().astype(np.float64)          # c1 is fp32: the draw itself
    approx = vals * scale.astype(np.float64)[:, None]
    normal = np.abs(vals) >= 2.0 ** -6
    assert np.all(np.abs(approx - w)[normal] <= 2.0 ** -4 * np.abs(w)[normal] * 1.0001)
    assert np.all(np.abs(approx - w)[~normal] <= 2.0 ** -10 * scale[:, None].repeat(w.shape[1], 1)[~normal] * 1.0001)


def test_stack_projection_groups_and_inputs():
    """The stack workload's layer inputs follow the model (q, k, v read the attention
    block's input, o the attention output, gate and up the MLP block's input, down the MLP
    activation), and the projections that share an input form the calls' groups."""
    from workloads.gen import LLAMA7B_XSRC, proj_groups_of
    wl = make_workload("c5", cache=False)
    assert list(wl.proj_names) == ["q", "k", "v", "o", "gate", "up", "down"]
    assert tuple(wl.x_input_of_proj) == LLAMA7B_XSRC
    assert wl.proj_groups() == [[0, 1, 2], [3], [4, 5], [6]]
    for g in wl.proj_groups():
        assert len({wl.d_in[p] for p in g}) == 1, "a group shares x, so its d_in"
        assert len({wl.x_input_of_proj[p] for p in g}) == 1
    # runs only: equal inputs that are not next to each other stay apart
    assert proj_groups_of([0, 0, 1, 0]) == [[0, 1], [2], [3]]
    assert proj_groups_of([]) == []


def test_stack_call_work_accounting():
    """bench.py's per-call work of the stack step: the projections' bytes add up, x is
    counted once per shared shrink launch, and a call makes one shrink and one decode
    expand launch for all its projections but one GEMM per projection."""
    import bench
    wl = make_workload("c5", cache=False)
    singles = [[p] for p in range(wl.n_proj)]
    w1, l1 = bench.stack_call_work(wl, singles)
    wg, lg = bench.stack_call_work(wl, wl.proj_groups())
    for key in ("gemm", "gemm_flops", "bgmv_expand", "sgmv_expand"):
        assert sum(w[key] for w in wg) == sum(w[key] for w in w1), key
    dec = sum(1 for r in wl.decode_requests() if r.adapter_id >= 0)
    pre = sum(r.n_tokens for r in wl.prefill_requests() if r.adapter_id >= 0)
    saved = sum((len(g) - 1) * wl.d_in[g[0]] * wl.elem_bytes for g in wl.proj_groups())
    assert sum(w["bgmv_shrink"] for w in w1) - sum(w["bgmv_shrink"] for w in wg) == dec * saved
    assert sum(w["sgmv_shrink"] for w in w1) - sum(w["sgmv_shrink"] for w in wg) == pre * saved
    for g, launches in zip(wl.proj_groups(), lg):
        assert launches == {"gemm": len(g), "bgmv_expand": 1, "sgmv_expand": len(g), "bgmv_shrink": 1,
                            "sgmv_shrink": 1}
