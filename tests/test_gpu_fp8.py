"""GPU parity of the FP8 base (base_gemm_fp8, lora_linear_fp8) through the C
ABI, against the oracle's FP8-base LoRA-linear.

The base weight is W0[n, k] = scale[n] * e4m3(code[n, k]) ("Multi-LoRA
serving: S-LoRA, Punica and adapter batching", Interaction with how the
adapters were trained: a quantized base with 16-bit adapters); x and the
adapters are bf16.  Bar: max |err| <= 2e-2 x RMS of the oracle's output per
call; rows without an adapter bit for bit equal to base_gemm_fp8; runs
deterministic.
"""
import numpy as np
import pytest

import oracle
from tests.gpu_helpers import bf16_bits, bits, parity, to_np
from workloads import make_workload
from workloads.device import batch_index, build_pool, oracle_adapters

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import heterogeneous_adapter_gemm_amd as hg
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    hg.library()
    yield
    torch.cuda.synchronize()


def say(*a):
    print("[case]", *a, flush=True)


def dev(arr):
    import heterogeneous_adapter_gemm_amd as hg
    if arr.dtype == np.uint8:
        return torch.from_numpy(np.ascontiguousarray(arr)).to("cuda")
    return hg.device_tensor(arr)


def random_fp8(g, n, k):
    """Codes from a normal draw at a per-row scale, as the generator makes them, with every
    finite code value (subnormals, zero, +-448) planted in row 0."""
    w = g.standard_normal((n, k)).astype(np.float32) * 0.05
    amax = np.abs(w).max(axis=1)
    scale = (amax / 448.0).astype(np.float32)
    codes = torch.from_numpy(np.clip(w / scale[:, None], -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    codes[0, :min(k, finite.size)] = finite[:min(k, finite.size)]
    return np.ascontiguousarray(codes), scale


# decode (64-row tiles of 16, 32 and 64 columns: N below 8192, from 8192, from 10240),
# 65-128 and 129-256 rows, more than 256 (two row blocks), ragged rows and columns (N a
# multiple of 4, not of 16, 32 or 64), one K step and several
SHAPES = [(1, 16, 128), (37, 48, 256), (64, 4096, 4096), (48, 8200, 384), (64, 10244, 256), (100, 520, 1152),
          (129, 1004, 640), (256, 1024, 512), (300, 272, 640), (9, 4, 128)]


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_base_gemm_fp8(M, N, K):
    import heterogeneous_adapter_gemm_amd as hg
    say("base_gemm_fp8", M, N, K)
    g = np.random.default_rng(M * 13 + N + K)
    x = bf16_bits(g.standard_normal((M, K)).astype(np.float32))
    codes, scale = random_fp8(g, N, K)
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    hg.base_gemm_fp8(dev(x), dev(codes), dev(scale), y, M, N, K)
    y2 = torch.empty_like(y)
    hg.base_gemm_fp8(dev(x), dev(codes), dev(scale), y2, M, N, K)
    torch.cuda.synchronize()
    assert np.array_equal(bits(y), bits(y2)), "two runs must agree bit for bit"
    parity(to_np(y), oracle.lora_linear_fp8base(x, codes, scale, [-1] * M, {}), what=f"fp8 gemm {M}x{N}x{K}")


def test_base_gemm_fp8_errors():
    import heterogeneous_adapter_gemm_amd as hg
    x = torch.zeros((4, 192), dtype=torch.bfloat16, device="cuda")
    q = torch.zeros((8, 192), dtype=torch.uint8, device="cuda")
    s = torch.ones(8, dtype=torch.float32, device="cuda")
    y = torch.zeros((4, 8), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(hg.LoraError):
        hg.base_gemm_fp8(x, q, s, y, 4, 8, 192)        # K not a multiple of 128
    with pytest.raises(hg.LoraError):
        hg.base_gemm_fp8(x, q, s, y, 4, 6, 128)        # N not a multiple of 4
    hg.base_gemm_fp8(x, q, s, y, 0, 8, 128)            # M = 0: no-op


def _fp8_workload_call(wl, pool, codes, scale, with_rows=None):
    from heterogeneous_adapter_gemm_amd import lora_plan_destroy
    idx = batch_index(wl, pool)
    xd = dev(wl.x())
    y = torch.zeros((wl.T, wl.d_out[0]), dtype=torch.bfloat16, device="cuda")
    plan = pool.plan(idx.get("seg_start"), idx.get("seg_slot"), idx.get("token_slot"))
    pool.linear_fp8(plan, 0, 0, xd, dev(codes), dev(scale), y)
    torch.cuda.synchronize()
    lora_plan_destroy(plan)
    return y


@pytest.mark.parametrize("cfg", ["c2", "c3"])
def test_lora_linear_fp8_decode_configs_all_rows(cfg):
    """The decode workloads (4096 x 4096, 64 rows, rank 16; 4096 -> 11008, 256 rows,
    mixed ranks, 10 % null rows) with their base as E4M3 codes: every row against the
    oracle, null rows bit for bit equal to base_gemm_fp8."""
    import heterogeneous_adapter_gemm_amd as hg
    wl = make_workload(cfg, cache=False)
    say(cfg, "fp8 base: build pool")
    pool, _ = build_pool(wl)
    wl.cache = True
    codes, scale = wl.w0_fp8()
    y = _fp8_workload_call(wl, pool, codes, scale)
    want = oracle.lora_linear_fp8base(wl.x(), codes, scale, wl.row_adapter(), oracle_adapters(wl))
    parity(to_np(y), want, what=f"{cfg} fp8 base, all rows")
    yb = torch.empty_like(y)
    hg.base_gemm_fp8(dev(wl.x()), dev(codes), dev(scale), yb, wl.T, wl.d_out[0], wl.d_in[0])
    torch.cuda.synchronize()
    null = wl.row_adapter() < 0
    if null.any():
        assert np.array_equal(bits(y)[null], bits(yb)[null])


def test_lora_linear_fp8_prefill_and_decode_rows():
    """A plan with prefill segments (with, without and of an adapter, ragged) and decode
    rows over an FP8 base: the segments' expand runs on its own after the base GEMM,
    reading the unrounded base of their rows."""
    from heterogeneous_adapter_gemm_amd import DevicePool, LORA_BF16, lora_plan_destroy
    d_in, d_out, P = 1024, 1040, 512
    ranks, alphas = [16, 64, 8], [32.0, 7.0, 3.0]
    g = np.random.default_rng(33)
    n_pages = 4 * sum(r * (d_in // P + -(-d_out // P)) for r in ranks) + 32
    pool = DevicePool(LORA_BF16, P, n_pages, g.permutation(n_pages), 1, [d_in], [d_out], 8, 64, 512, 8)
    ad = {}
    for i, (r, al) in enumerate(zip(ranks, alphas)):
        A = bf16_bits((g.standard_normal((r, d_in)) * d_in ** -0.5).astype(np.float32))
        B = bf16_bits((g.standard_normal((r, d_out)) * 0.05).astype(np.float32))
        pool.page_in(i, r, al, A.reshape(-1), B.reshape(-1))
        ad[i] = (r, al, A, B)
    lens, sad = [130, 1, 0, 77], [0, -1, 2, 1]
    dec = g.choice([-1, 0, 1, 2], 45).astype(np.int32)
    T = sum(lens) + dec.size
    row_ad = np.concatenate([np.full(n, a, np.int32) for n, a in zip(lens, sad)] + [dec])
    x = bf16_bits(g.standard_normal((T, d_in)).astype(np.float32))
    codes, scale = random_fp8(g, d_out, d_in)
    st = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    say("fp8 base prefill + decode", T, "rows")
    plan = pool.plan(st, [-1 if a < 0 else pool.slot_of(a) for a in sad],
                     [-1 if a < 0 else pool.slot_of(int(a)) for a in dec])
    y = torch.zeros((T, d_out), dtype=torch.bfloat16, device="cuda")
    pool.linear_fp8(plan, 0, 0, dev(x), dev(codes), dev(scale), y)
    torch.cuda.synchronize()
    lora_plan_destroy(plan)
    parity(to_np(y), oracle.lora_linear_fp8base(x, codes, scale, row_ad, ad), what="fp8 base prefill + decode")
