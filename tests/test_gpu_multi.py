"""lora_linear_multi: several projections of one layer that share x, their shrinks
in shared launches, then each projection's base GEMM and expand.  Each
projection's output must equal one lora_linear call's bit for bit (the same
kernels run on the same data in the same order; only the launches that hold
them differ), and the oracle's within the output bar.

Pool: 2 layers x 5 projections, four of them 1024 -> {1536, 1024, 520, 2048}
and one 512 -> 1024 (another d_in, so it cannot join the others), 8 adapters
of ranks 1 .. 64 in 512-element pages.  Batches: prefill segments with
decode rows (more than 64 rows, so the shrinks run in their own launches),
segments alone, decode rows alone, a decode batch of at most 64 rows (its GEMM
and shrink share one launch per projection: the call runs as single calls),
and the delta alone (w0 = NULL into a zeroed y).
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from tests.gpu_helpers import bf16_bits, bits, parity, to_np

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

N_LAYERS, P = 2, 512
D_IN = [1024, 1024, 1024, 1024, 512]
D_OUT = [1536, 1024, 520, 2048, 1024]
RANKS = [8, 16, 32, 64, 1, 33, 16, 8]
ALPHA = [16.0, 3.5, 64.0, 2.0, 1.0, 70.0, 32.0, 5.0]


def say(*a):
    print("[case]", *a, flush=True)


@pytest.fixture(scope="module")
def setup():
    import heterogeneous_adapter_gemm_amd as hg
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    hg.library()
    g = np.random.default_rng(41)
    per_rank = N_LAYERS * sum(-(-i // P) + -(-o // P) for i, o in zip(D_IN, D_OUT))
    n_pages = per_rank * sum(RANKS) + 128
    pool = hg.DevicePool(hg.LORA_BF16, P, n_pages, g.permutation(n_pages), N_LAYERS, D_IN, D_OUT, 10, 64, 512, 16,
                         max_multi=4)
    mats = {}
    for a, r in enumerate(RANKS):
        As, Bs = [], []
        for l in range(N_LAYERS):
            for p in range(len(D_IN)):
                A = bf16_bits((g.standard_normal((r, D_IN[p])) * D_IN[p] ** -0.5).astype(np.float32))
                B = bf16_bits((g.standard_normal((r, D_OUT[p])) * 0.05).astype(np.float32))
                mats[(a, l, p)] = (A, B)
                As.append(A.reshape(-1))
                Bs.append(B.reshape(-1))
        pool.page_in(a, r, ALPHA[a], np.concatenate(As), np.concatenate(Bs))
    torch.cuda.synchronize()
    yield pool, mats, g
    pool.close()


def run_case(setup, layer, seg_lens, seg_ad, dec_ad, projs, with_w0=True, check_oracle=False):
    import heterogeneous_adapter_gemm_amd as hg
    pool, mats, g = setup
    T = sum(seg_lens) + len(dec_ad)
    say(f"layer {layer} segments {seg_lens} decode rows {len(dec_ad)} projections {projs} w0 {with_w0}")
    d_in = D_IN[projs[0]]
    x = bf16_bits(g.standard_normal((T, d_in)).astype(np.float32))
    ws = [bf16_bits((g.standard_normal((D_OUT[p], d_in)) * 0.03).astype(np.float32)) for p in projs]
    # y before the call: random with w0 (overwritten), zero for the delta alone (y += delta)
    y0 = [bf16_bits(g.standard_normal((T, D_OUT[p])).astype(np.float32)) if with_w0 else
          np.zeros((T, D_OUT[p]), np.uint16) for p in projs]
    xd = hg.device_tensor(x)
    wd = [hg.device_tensor(w) if with_w0 else None for w in ws]
    st = np.concatenate([[0], np.cumsum(seg_lens)]).astype(np.int32)
    seg_slots = [-1 if a < 0 else pool.slot_of(a) for a in seg_ad]
    dec_slots = [-1 if a < 0 else pool.slot_of(a) for a in dec_ad]
    plan = pool.plan(st, seg_slots, dec_slots)
    single = [hg.device_tensor(v) for v in y0]
    multi = [hg.device_tensor(v) for v in y0]
    for i, p in enumerate(projs):
        pool.linear(plan, layer, p, xd, wd[i], single[i])
    pool.linear_multi(plan, layer, projs, xd, wd, multi)
    torch.cuda.synchronize()
    hg.lora_plan_destroy(plan)
    for i, p in enumerate(projs):
        assert np.array_equal(bits(single[i]), bits(multi[i])), f"projection {p}: multi call differs from the single call"
    if check_oracle:
        ra = np.concatenate([np.full(n, a, np.int32) for n, a in zip(seg_lens, seg_ad)] + [np.asarray(dec_ad, np.int32)])
        for i, p in enumerate(projs):
            ids = {int(a) for a in ra if a >= 0}
            ads = {a: (RANKS[a], ALPHA[a], *mats[(a, layer, p)]) for a in ids}
            want = oracle.lora_linear(x, ws[i] if with_w0 else None, ra, ads)
            if with_w0:
                parity(to_np(multi[i]), want, what=f"multi layer {layer} projection {p}")
            else:
                parity_delta(to_np(multi[i]), want, what=f"multi layer {layer} projection {p} delta only")


def parity_delta(got, want, what):
    """The delta alone: rows of adapters with scales from 1/32 to 2 put the largest
    output near 15 x the RMS, so storing the exact result as bf16 (unit roundoff
    2^-8) can alone exceed 2e-2 x RMS.  Bar per element: 2e-2 x RMS plus that
    rounding, 2^-8 x |oracle|."""
    rms = float(np.sqrt(np.mean(want ** 2)))
    excess = np.abs(got - want) - 2.0 ** -8 * np.abs(want)
    print(f"[parity] {what} max(|err| - 2^-8 |want|) {excess.max():.4e}  rms {rms:.4e}", flush=True)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    assert excess.max() <= 2e-2 * rms, f"{what}: error beyond bf16 rounding {excess.max():.4e} > 2e-2 x RMS {rms:.4e}"


def test_multi_mixed_batch_equals_single_calls_and_oracle(setup):
    rng = np.random.default_rng(1)
    dec = [int(a) for a in rng.integers(-1, len(RANKS), 90)]
    run_case(setup, 1, [70, 0, 129, 200, 3], [2, 1, -1, 3, 5], dec, [0, 1, 2, 3], check_oracle=True)


def test_multi_prefill_only_and_decode_only(setup):
    run_case(setup, 0, [64, 300, 17], [3, 6, 0], [], [3, 1])
    rng = np.random.default_rng(2)
    run_case(setup, 1, [], [], [int(a) for a in rng.integers(-1, len(RANKS), 130)], [2, 0, 3])


def test_multi_short_decode_runs_as_single_calls(setup):
    rng = np.random.default_rng(3)
    run_case(setup, 0, [], [], [int(a) for a in rng.integers(-1, len(RANKS), 40)], [0, 1, 2, 3], check_oracle=True)


def test_multi_delta_only(setup):
    rng = np.random.default_rng(4)
    dec = [int(a) for a in rng.integers(-1, len(RANKS), 80)]
    run_case(setup, 1, [33, 128], [7, 4], dec, [1, 3, 0], with_w0=False, check_oracle=True)


def test_multi_one_projection_and_errors(setup):
    import heterogeneous_adapter_gemm_amd as hg
    pool, _, _ = setup
    run_case(setup, 0, [65], [5], [0, 1, 2], [2])
    x = torch.zeros((8, 1024), dtype=torch.bfloat16, device="cuda")
    ys = [torch.zeros((8, D_OUT[p]), dtype=torch.bfloat16, device="cuda") for p in range(5)]
    ws = [torch.zeros((D_OUT[p], D_IN[p]), dtype=torch.bfloat16, device="cuda") for p in range(5)]
    plan = pool.plan(None, None, [pool.slot_of(0)] * 8)
    with pytest.raises(hg.LoraError):   # more projections than the pool's max_multi
        pool.linear_multi(plan, 0, [0, 1, 2, 3, 0], x, ws[:4] + ws[:1], ys[:4] + ys[:1])
    with pytest.raises(hg.LoraError):   # projection 4 reads another d_in
        pool.linear_multi(plan, 0, [0, 4], x, [ws[0], ws[4]], [ys[0], ys[4]])
    with pytest.raises(hg.LoraError):   # w0 for some projections only
        pool.linear_multi(plan, 0, [0, 1], x, [ws[0], None], [ys[0], ys[1]])
    torch.cuda.synchronize()
    hg.lora_plan_destroy(plan)
