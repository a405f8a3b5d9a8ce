"""The decode entry point that allocates nothing (lora_linear_decode_noalloc),
through the C ABI, against lora_linear_decode on the same pool and inputs:
bit-identical outputs (same kernels, same reduction orders), with the base
and as the delta alone, and the oracle's bar on the full output, on two calls
in a row, the second with fewer rows (so it reads the scratch the first one
left); a call too large for the static scratch is refused before any device
work.  (The delta alone is checked bit for bit against lora_linear_decode,
whose delta-only path the parity tests hold to the oracle: its bf16 outputs,
rounded once, reach the 2e-2 x RMS bar by rounding alone when the largest
delta sits just above a power of two.)"""
import numpy as np
import pytest

import oracle
from tests.gpu_helpers import bf16_bits, bits, parity, to_np

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def say(*a):
    print("[case]", *a, flush=True)


def _pool(d_in, d_out, ranks, seed, max_tokens):
    from heterogeneous_adapter_gemm_amd import LORA_BF16, DevicePool
    g = np.random.default_rng(seed)
    P = 1024
    n_pages = sum(r * (-(-d_in // P) + -(-d_out // P)) for r in ranks) + 64
    pool = DevicePool(LORA_BF16, P, n_pages, g.permutation(n_pages), 1, [d_in], [d_out], len(ranks) + 2, 64,
                      max_tokens, 4)
    ad = {}
    for i, r in enumerate(ranks):
        A = bf16_bits(g.standard_normal((r, d_in)).astype(np.float32) * d_in ** -0.5)
        B = bf16_bits(g.standard_normal((r, d_out)).astype(np.float32) * 0.05)
        alpha = float(2 * r if i % 2 else 3.0 + i)
        pool.page_in(i, r, alpha, A.reshape(-1), B.reshape(-1))
        ad[i] = (r, alpha, A, B)
    torch.cuda.synchronize()
    pool.drop_host_copies()
    return pool, ad, g


def test_noalloc_decode_matches_lora_linear_decode():
    import heterogeneous_adapter_gemm_amd as hg
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    hg.library()
    d_in, d_out = 1024, 11008
    pool, ad, g = _pool(d_in, d_out, [8, 64, 16, 33, 4], seed=91, max_tokens=512)
    # output RMS about 1.3: the bf16 rounding of the largest outputs (up to 2^-8 of
    # |y|) then stays below the 2e-2 x RMS bar (a power of two at about 5 RMS would not)
    w0 = bf16_bits(g.standard_normal((d_out, d_in)).astype(np.float32) * 0.04)
    wd = hg.device_tensor(w0)
    # two calls in a row, the second smaller: 256 rows (separate shrink / GEMM / expand
    # launches), then 40 rows (the GEMM and shrink in one launch)
    for T in (256, 40):
        row_ad = g.choice([-1, 0, 1, 2, 3, 4], T).astype(np.int32)
        ts = [-1 if a < 0 else pool.slot_of(int(a)) for a in row_ad]
        x = bf16_bits(g.standard_normal((T, d_in)).astype(np.float32))
        xd = hg.device_tensor(x)
        say("noalloc decode", T, "rows x", d_in, "->", d_out)
        y_na = torch.zeros((T, d_out), dtype=torch.bfloat16, device="cuda")
        pool.linear_decode_noalloc(0, 0, xd, wd, y_na, ts)
        d_na = torch.zeros_like(y_na)
        pool.linear_decode_noalloc(0, 0, xd, None, d_na, ts)
        torch.cuda.synchronize()
        y_ref = torch.zeros_like(y_na)
        pool.linear_decode(0, 0, xd, wd, y_ref, ts)
        d_ref = torch.zeros_like(y_na)
        pool.linear_decode(0, 0, xd, None, d_ref, ts)
        torch.cuda.synchronize()
        assert np.array_equal(bits(y_na), bits(y_ref)), f"T={T}: outputs differ from lora_linear_decode"
        assert np.array_equal(bits(d_na), bits(d_ref)), f"T={T}: delta differs from lora_linear_decode"
        parity(to_np(y_na), oracle.lora_linear(x, w0, row_ad, ad), what=f"noalloc T={T}")
    # 400 rows x 11008 outputs need more than the 16 MiB scratch: refused, nothing written
    T = 400
    xd = torch.zeros((T, d_in), dtype=torch.bfloat16, device="cuda")
    y = torch.full((T, d_out), 5.0, dtype=torch.bfloat16, device="cuda")
    say("noalloc decode too large for the scratch:", T, "rows")
    with pytest.raises(hg.LoraError) as e:
        pool.linear_decode_noalloc(0, 0, xd, wd, y, [0] * T)
    assert e.value.code == hg.LORA_EINVAL and "scratch" in str(e.value)
    torch.cuda.synchronize()
    assert torch.all(y == 5.0)
