"""GPU parity: the HIP path (through the C ABI) against the oracle.

Every test prints what it runs before the GPU step.  Floating-point bar:
max |err| <= 2e-2 x RMS(oracle output) per call; integer/byte work (page
contents, tables) bitwise; invariances bitwise, the kernels being
deterministic (fixed reduction orders, no float atomics).
"""
import numpy as np
import pytest

import oracle
from oracle.pool_model import PoolModel
from tests.gpu_helpers import TOL, bf16_bits, bits, parity, to_np
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


def dev(arr):
    from heterogeneous_adapter_gemm_amd import device_tensor
    return device_tensor(arr)


def say(*a):
    print("[case]", *a, flush=True)


# ---------------------------------------------------------------------------
# base GEMM
GEMM_SHAPES = [(1, 16, 64), (37, 48, 136), (64, 4096, 256), (100, 272, 520), (256, 640, 1024),
               (300, 512, 256), (777, 520, 328), (1024, 768, 512)]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("M,N,K", GEMM_SHAPES)
def test_base_gemm(dtype, M, N, K):
    import heterogeneous_adapter_gemm_amd as hg
    say("base_gemm", dtype, M, N, K)
    g = np.random.default_rng(M * 7 + N * 3 + K)
    xf = g.standard_normal((M, K)).astype(np.float32)
    wf = (g.standard_normal((N, K)) * 0.05).astype(np.float32)
    x, w = (bf16_bits(xf), bf16_bits(wf)) if dtype == "bf16" else (xf, wf)
    xd, wd = dev(x), dev(w)
    y = torch.empty((M, N), dtype=xd.dtype, device="cuda")
    hg.base_gemm(hg.LORA_BF16 if dtype == "bf16" else hg.LORA_F32, xd, wd, y, M, N, K)
    torch.cuda.synchronize()
    want = oracle.lora_linear(x, w, [-1] * M, {})
    parity(to_np(y), want, what=f"gemm {dtype} {M}x{N}x{K}")


# long batches (M > 256, K % 128 == 0): tiles of 192 rows (one round; with halves) and of
# 256 rows (one full round; the last round's tiles in 2, 4, 8 and 16 pieces)
LONG_GEMM_SHAPES = [(2961, 4096, 256), (2070, 11008, 128), (4096, 4096, 256), (1811, 11008, 128),
                    (1552, 11008, 128), (2070, 8192, 128), (2961, 11008, 128)]


@pytest.mark.parametrize("M,N,K", LONG_GEMM_SHAPES)
def test_base_gemm_long_tile_heights(M, N, K):
    """Rows from every 64-row block (the 192- and 256-row tiles both cut through them), all
    columns, against the oracle; bit for bit equal to a second run."""
    import heterogeneous_adapter_gemm_amd as hg
    bm, tiles, rem, npc = long_tiles(M, N)
    say("base_gemm long", M, N, K, f"tiles of {bm} rows: {tiles}, {rem} cut in {npc}")
    g = np.random.default_rng(M + N + K)
    x = bf16_bits(g.standard_normal((M, K)).astype(np.float32))
    w = bf16_bits((g.standard_normal((N, K)) * 0.05).astype(np.float32))
    xd, wd = dev(x), dev(w)
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    y2 = torch.empty_like(y)
    hg.base_gemm(hg.LORA_BF16, xd, wd, y, M, N, K)
    hg.base_gemm(hg.LORA_BF16, xd, wd, y2, M, N, K)
    torch.cuda.synchronize()
    assert np.array_equal(bits(y), bits(y2))
    rows = sorted(set(int(r) for t in range(-(-M // 64)) for r in g.integers(64 * t, min(64 * (t + 1), M), 2)))
    parity(to_np(y)[rows], oracle.lora_linear(x, w, [-1] * M, {}, rows=rows), what=f"gemm long {M}x{N}x{K}")


# 65 to 256 rows, K % 64 == 0: the x-through-LDS tiles, one case per tile shape (64 x 64,
# 128 x 64, 128 x 128), with ragged rows and columns and K of one step or not a multiple of
# the pipeline depth
MID_SHAPES = [(77, 1004, 192), (80, 11008, 128), (200, 11008, 64), (256, 4096, 320), (129, 2048, 4096)]


@pytest.mark.parametrize("M,N,K", MID_SHAPES)
def test_base_gemm_mid_batches(M, N, K):
    import heterogeneous_adapter_gemm_amd as hg
    say("base_gemm mid", M, N, K)
    g = np.random.default_rng(M * 5 + N + K * 11)
    x = bf16_bits(g.standard_normal((M, K)).astype(np.float32))
    w = bf16_bits((g.standard_normal((N, K)) * 0.05).astype(np.float32))
    xd, wd = dev(x), dev(w)
    y = torch.empty((M, N), dtype=xd.dtype, device="cuda")
    hg.base_gemm(hg.LORA_BF16, xd, wd, y, M, N, K)
    torch.cuda.synchronize()
    parity(to_np(y), oracle.lora_linear(x, w, [-1] * M, {}), what=f"gemm mid {M}x{N}x{K}")


def test_base_gemm_errors():
    import heterogeneous_adapter_gemm_amd as hg
    x = torch.zeros((4, 12), dtype=torch.bfloat16, device="cuda")
    y = torch.zeros((4, 8), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(hg.LoraError):
        hg.base_gemm(hg.LORA_BF16, x, x, y, 4, 8, 12)          # K not a multiple of 8
    with pytest.raises(hg.LoraError):
        hg.base_gemm(7, x, x, y, 4, 8, 8)
    hg.base_gemm(hg.LORA_BF16, x, x, y, 0, 8, 8)               # M = 0: no-op


# ---------------------------------------------------------------------------
# whole LoRA-linear on the configurations
def run_workload(wl, pool, layer=0, proj=0, with_base=True, x=None, y=None):
    idx = batch_index(wl, pool)
    xd = dev(wl.x(layer, proj)) if x is None else x
    wd = dev(wl.w0(layer, proj)) if with_base else None
    if y is None:
        y = torch.zeros((wl.T, wl.d_out[proj]), dtype=xd.dtype, device="cuda")
    plan = pool.plan(idx.get("seg_start"), idx.get("seg_slot"), idx.get("token_slot"))
    pool.linear(plan, layer, proj, xd, wd, y)
    torch.cuda.synchronize()
    from heterogeneous_adapter_gemm_amd import lora_plan_destroy
    lora_plan_destroy(plan)
    return y


def oracle_rows(wl, rows=None, layer=0, proj=0, with_base=True):
    return oracle.lora_linear(wl.x(layer, proj), wl.w0(layer, proj) if with_base else None, wl.row_adapter(),
                              oracle_adapters(wl, layer, proj), rows=rows)


def test_c1_tiny_fp32_full():
    wl = make_workload("c1")
    say("c1 full", wl.T, "rows")
    pool, _ = build_pool(wl)
    y = run_workload(wl, pool)
    parity(to_np(y), oracle_rows(wl), what="c1")
    # the delta alone, against the oracle's delta (base term zero)
    yd = run_workload(wl, pool, with_base=False)
    parity(to_np(yd), oracle_rows(wl, with_base=False), what="c1 delta only")


def test_c1_merged_weight_identity_on_gpu():
    """Each adapter's rows equal x (W0 + gamma B A)^T computed separately."""
    wl = make_workload("c1")
    say("c1 merged identity")
    pool, _ = build_pool(wl)
    y = to_np(run_workload(wl, pool))
    x = wl.x().astype(np.float64)
    ra = wl.row_adapter()
    for a, spec in wl.adapters.items():
        rows = np.nonzero(ra == a)[0]
        if rows.size == 0:
            continue
        A, B = wl.adapter_AB(a)
        merged = wl.w0().astype(np.float64) + (spec.alpha / spec.rank) * (B.astype(np.float64).T @ A.astype(np.float64))
        parity(y[rows], x[rows] @ merged.T, what=f"c1 merged adapter {a}")


def test_c2_decode_full():
    wl = make_workload("c2")
    say("c2 full", wl.T, "rows")
    pool, _ = build_pool(wl)
    y = run_workload(wl, pool)
    parity(to_np(y), oracle_rows(wl), what="c2")
    yd = run_workload(wl, pool, with_base=False)
    parity(to_np(yd), oracle_rows(wl, with_base=False), what="c2 delta only")


def test_c3_decode_mixed_ranks_all_rows():
    """Every row of the 256-row mixed-rank decode batch, with the base (full
    output) and as the delta alone (w0 = NULL into a zeroed y): the delta-only
    bar, 2e-2 x RMS of the oracle's delta, catches a wrong rank-row or page
    that the base term would hide."""
    wl = make_workload("c3", cache=False)
    say("c3 build pool (2000 adapters)")
    pool, _ = build_pool(wl)
    wl.cache = True
    y = to_np(run_workload(wl, pool))
    say("c3 oracle on all", wl.T, "rows")
    parity(y, oracle_rows(wl), what="c3 all rows")
    yd = to_np(run_workload(wl, pool, with_base=False))
    parity(yd, oracle_rows(wl, with_base=False), what="c3 delta only, all rows")
    ra = wl.row_adapter()
    assert np.all(yd[ra < 0] == 0.0), "rows with no adapter must not be touched"


def test_c4_prefill_all_rows():
    """Every row of the 9,551-row prefill batch (37.3 row tiles of 256: the
    last round of tiles and the ragged last tile included), full output and
    delta alone."""
    wl = make_workload("c4")
    say("c4 build pool, T =", wl.T)
    pool, _ = build_pool(wl)
    y = to_np(run_workload(wl, pool))
    say("c4 oracle on all", wl.T, "rows")
    parity(y, oracle_rows(wl), what="c4 all rows")
    del y
    yd = to_np(run_workload(wl, pool, with_base=False))
    parity(yd, oracle_rows(wl, with_base=False), what="c4 delta only, all rows")
    ra = wl.row_adapter()
    assert np.all(yd[ra < 0] == 0.0), "rows of null segments must not be touched"


# ---------------------------------------------------------------------------
# bitwise properties
@pytest.mark.parametrize("n_tokens", [96, 48])
def test_null_rows_equal_base_gemm_bitwise(n_tokens):
    import heterogeneous_adapter_gemm_amd as hg
    wl = make_workload("c3", n_tokens=n_tokens, cache=False)
    say("null rows vs base_gemm", n_tokens)
    pool, _ = build_pool(wl)
    wl.cache = True
    y = run_workload(wl, pool)
    xd, wd = dev(wl.x()), dev(wl.w0())
    yb = torch.empty_like(y)
    hg.base_gemm(hg.LORA_BF16, xd, wd, yb, wl.T, wl.d_out[0], wl.d_in[0])
    torch.cuda.synchronize()
    null = wl.row_adapter() < 0
    assert null.any()
    assert np.array_equal(bits(y)[null], bits(yb)[null])


def test_row_and_page_permutation_invariance_bitwise():
    wl = make_workload("c2", n_tokens=48)
    say("row / page permutation")
    pool, _ = build_pool(wl)
    y = run_workload(wl, pool)
    y2 = run_workload(wl, pool)
    assert np.array_equal(bits(y), bits(y2)), "two runs must agree bit for bit"
    # rows permuted
    perm = np.random.default_rng(5).permutation(wl.T)
    wlp = make_workload("c2", n_tokens=48)
    wlp.requests = [wl.requests[i] for i in perm]
    wlp._memo[("x", 0, 0)] = wl.x()[perm]
    yp = run_workload(wlp, pool)
    assert np.array_equal(bits(yp), bits(y)[perm])
    # physical pages permuted: a different free order
    fo = np.random.default_rng(99).permutation(wl.num_pages).astype(np.int32)
    pool2, _ = build_pool(wl, free_order=fo)
    y3 = run_workload(wl, pool2)
    assert np.array_equal(bits(y3), bits(y))


def test_page_contents_round_trip():
    for name, check_slots in (("c1", None), ("c3", 25)):
        wl = make_workload(name, cache=False)
        say("page contents", name)
        pool, _ = build_pool(wl)
        torch.cuda.synchronize()
        model = PoolModel(wl.num_pages, wl.page_elems, wl.free_order, wl.n_layers, wl.d_in, wl.d_out, wl.max_slots,
                          wl.max_rank)
        model.replay(wl.setup_ops, {a: s.rank for a, s in wl.adapters.items()},
                     {a: s.alpha for a, s in wl.adapters.items()})
        pages = bits(pool.pages).reshape(wl.num_pages, wl.page_elems)
        ids = sorted(model.adapter_slot)[: check_slots or None]
        for a in ids:
            A, B = wl.adapter_AB(a)
            exp = model.expected_pages(model.slot_of(a), 0, 0, A, B)
            for pg, content in exp.items():
                want = content.view(np.int16) if content.dtype == np.uint16 else content.view(np.int32)
                assert np.array_equal(pages[pg], want), f"{name} adapter {a} page {pg}"


@pytest.mark.parametrize("stage_mb", [0, 24])
def test_batched_page_in_contents_all_layers_and_projections(stage_mb):
    """The Llama-7B stack's cold adapters (2 layers x 7 projections) paged in as
    one batch on a side stream, over PCIe by the gather kernel (0) or through a
    24 MB staging area (a few adapters per copy group): every page of every
    layer and projection holds the rank-row chunk the oracle's pool model
    places there, bit for bit."""
    from workloads.device import replay
    wl = make_workload("c5", n_layers=2, cache=False)
    say("batched page-in contents: c5 with 2 layers,", len(wl.cold_adapters), "cold adapters, staging", stage_mb, "MB")
    pool, _ = build_pool(wl, max_tokens=wl.T, max_segments=16, stage_bytes=stage_mb << 20)
    side = torch.cuda.Stream()
    replay(wl, pool, wl.step_ops, stream=side.cuda_stream, settle=True, batch=True)
    torch.cuda.synchronize()
    model = PoolModel(wl.num_pages, wl.page_elems, wl.free_order, wl.n_layers, wl.d_in, wl.d_out, wl.max_slots,
                      wl.max_rank)
    ranks = {a: s.rank for a, s in wl.adapters.items()}
    alphas = {a: s.alpha for a, s in wl.adapters.items()}
    model.replay(wl.setup_ops + wl.step_ops, ranks, alphas)
    pages = bits(pool.pages).reshape(wl.num_pages, wl.page_elems)
    for a in wl.cold_adapters:
        assert pool.slot_of(a) == model.slot_of(a)
        for l in range(wl.n_layers):
            for p in range(wl.n_proj):
                A, B = wl.adapter_AB(a, l, p)
                exp = model.expected_pages(model.slot_of(a), l, p, A, B)
                for pg, content in exp.items():
                    assert np.array_equal(pages[pg], content.view(np.int16)), f"adapter {a} layer {l} proj {p} page {pg}"


# ---------------------------------------------------------------------------
# paths and edge cases on small random layers
def small_pool(dtype, d_in, d_out, ranks, alphas, seed, page_elems, max_tokens=512, max_segments=16, n_layers=1):
    """A pool holding adapters 0..n-1 with the given ranks; returns (pool, adapters, host arrays)."""
    from heterogeneous_adapter_gemm_amd import DevicePool, LORA_BF16, LORA_F32
    g = np.random.default_rng(seed)

    def arr(*shape, std=1.0):
        v = (g.standard_normal(shape) * std).astype(np.float32)
        return bf16_bits(v) if dtype == "bf16" else v
    n_pages = 4 * sum(r * (-(-d_in // page_elems) + -(-d_out // page_elems)) for r in ranks) * n_layers + 64
    pool = DevicePool(LORA_BF16 if dtype == "bf16" else LORA_F32, page_elems, n_pages,
                      g.permutation(n_pages), n_layers, [d_in], [d_out], len(ranks) + 2, 64, max_tokens,
                      max_segments)
    ad = {}
    for i, (r, al) in enumerate(zip(ranks, alphas)):
        A, B = arr(r * n_layers, d_in, std=d_in ** -0.5), arr(r * n_layers, d_out, std=0.05)
        pool.page_in(i, r, al, A.reshape(-1), B.reshape(-1))
        ad[i] = (r, al, A[:r], B[:r])     # layer 0
    w0 = arr(d_out, d_in, std=0.05)
    return pool, ad, w0, arr


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_decode_and_prefill_paths_random_alpha(dtype):
    """BGMV and SGMV on the same rows, ranks 1..64, gamma != 2 (random alpha)."""
    from heterogeneous_adapter_gemm_amd import lora_plan_destroy
    ranks = [1, 7, 16, 33, 64, 8]
    alphas = [0.5, 3.0, 5.5, 70.0, 1.0, 16.0]
    d_in, d_out = 1024, 520 if dtype == "bf16" else 516
    pool, ad, w0, arr = small_pool(dtype, d_in, d_out, ranks, alphas, seed=21,
                                   page_elems=512 if dtype == "bf16" else 256)
    g = np.random.default_rng(22)
    # prefill: ragged segments incl. empty and null ones
    lens = [70, 0, 1, 129, 64, 200, 3]
    sadp = [2, 1, -1, 4, 0, 3, 5]
    T = sum(lens)
    x = arr(T, d_in)
    st = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    slots = [-1 if a < 0 else pool.slot_of(a) for a in sadp]
    row_ad = np.concatenate([np.full(n, a, np.int32) for n, a in zip(lens, sadp)])
    xd, wd = dev(x), dev(w0)
    say("prefill random", dtype, T)
    y = torch.zeros((T, d_out), dtype=xd.dtype, device="cuda")
    pool.linear_prefill(0, 0, xd, wd, y, st, slots)
    torch.cuda.synchronize()
    want = oracle.lora_linear(x, w0, row_ad, ad)
    parity(to_np(y), want, what=f"sgmv {dtype}")
    # the same rows as decode rows (BGMV)
    say("decode random", dtype, T)
    yb = torch.zeros_like(y)
    pool.linear_decode(0, 0, xd, wd, yb, [-1 if a < 0 else pool.slot_of(a) for a in row_ad])
    torch.cuda.synchronize()
    parity(to_np(yb), want, what=f"bgmv {dtype}")
    # mixed plan: first 3 segments prefill, the rest of the rows decode
    npre = int(st[3])
    plan = pool.plan(st[:4], slots[:3], [-1 if a < 0 else pool.slot_of(a) for a in row_ad[npre:]])
    ym = torch.zeros_like(y)
    pool.linear(plan, 0, 0, xd, wd, ym)
    torch.cuda.synchronize()
    lora_plan_destroy(plan)
    parity(to_np(ym), want, what=f"mixed {dtype}")


def test_edge_cases():
    from heterogeneous_adapter_gemm_amd import lora_plan_destroy
    pool, ad, w0, arr = small_pool("bf16", 512, 512, [4, 64], [8.0, 128.0], seed=31, page_elems=512)
    xd, wd = dev(arr(5, 512)), dev(w0)
    y = torch.full((5, 512), 3.0, dtype=torch.bfloat16, device="cuda")
    say("edge: empty plan")
    plan = pool.plan()
    pool.linear(plan, 0, 0, xd, wd, y)            # T = 0: nothing happens
    lora_plan_destroy(plan)
    torch.cuda.synchronize()
    assert torch.all(y == 3.0)
    say("edge: all-null decode batch, delta only")
    pool.linear_decode(0, 0, xd, None, y, [-1] * 5)
    torch.cuda.synchronize()
    assert torch.all(y == 3.0)
    say("edge: single row, max rank")
    y1 = torch.zeros((1, 512), dtype=torch.bfloat16, device="cuda")
    pool.linear_decode(0, 0, xd[:1], wd, y1, [pool.slot_of(1)])
    torch.cuda.synchronize()
    parity(to_np(y1), oracle.lora_linear(bits_to(xd[:1]), w0, [1], ad), what="single row r=64")


def test_decode_ragged_matches_oracle_and_base_gemm():
    """Decode batch on the LDS decode kernel with ragged edges: 37 rows (a
    partial 64-row tile), d_out = 520 (not a multiple of the 16-column tiles'
    K-stagger period), d_in = 1152 (9 K steps of 128, not a multiple of the 4
    stages).  Against the oracle; rows without an adapter bit for bit equal to
    base_gemm; and deterministic."""
    import heterogeneous_adapter_gemm_amd as hg
    d_in, d_out = 1152, 520
    pool, ad, w0, arr = small_pool("bf16", d_in, d_out, [8, 32, 64], [16.0, 5.0, 128.0], seed=51, page_elems=512)
    g = np.random.default_rng(52)
    row_ad = g.choice([-1, 0, 1, 2], 37).astype(np.int32)
    x = arr(37, d_in)
    xd, wd = dev(x), dev(w0)
    say("decode ragged", 37, d_out, d_in)
    ts = [-1 if a < 0 else pool.slot_of(int(a)) for a in row_ad]
    y = torch.zeros((37, d_out), dtype=torch.bfloat16, device="cuda")
    y2 = torch.zeros_like(y)
    pool.linear_decode(0, 0, xd, wd, y, ts)
    pool.linear_decode(0, 0, xd, wd, y2, ts)
    yb = torch.zeros_like(y)
    hg.base_gemm(hg.LORA_BF16, xd, wd, yb, 37, d_out, d_in)
    torch.cuda.synchronize()
    assert np.array_equal(bits(y), bits(y2)), "two runs must agree bit for bit"
    parity(to_np(y), oracle.lora_linear(x, w0, row_ad, ad), what="decode ragged")
    null = row_ad < 0
    assert null.any() and not null.all()
    assert np.array_equal(bits(y)[null], bits(yb)[null])


def test_back_to_back_plans_on_the_null_stream():
    """Plans created and used back to back on the null stream (handle 0), with
    no host synchronisation between them: a plan takes the ring entry the
    previous one used at once, its upload ordered on the device after that
    plan's kernels.  Batches differ in size and grouping, so a call reading
    another plan's index would give wrong rows."""
    from heterogeneous_adapter_gemm_amd import lora_plan_destroy
    d_in, d_out = 1024, 520
    pool, ad, w0, arr = small_pool("bf16", d_in, d_out, [8, 16, 64, 4], [16.0, 5.0, 128.0, 1.0], seed=61,
                                   page_elems=512, max_tokens=128)
    g = np.random.default_rng(62)
    wd = dev(w0)
    cases = []
    for i in range(12):
        T = int(g.integers(1, 129))
        row_ad = g.choice([-1, 0, 1, 2, 3], T).astype(np.int32)
        x = arr(T, d_in)
        cases.append((row_ad, x, dev(x), torch.zeros((T, d_out), dtype=torch.bfloat16, device="cuda")))
    torch.cuda.synchronize()
    say("12 plans back to back on stream 0")
    for row_ad, _, xd, y in cases:
        plan = pool.plan(token_slot=[-1 if a < 0 else pool.slot_of(int(a)) for a in row_ad], stream=0)
        pool.linear(plan, 0, 0, xd, wd, y, stream=0)
        lora_plan_destroy(plan)
    torch.cuda.synchronize()
    for i, (row_ad, x, _, y) in enumerate(cases):
        parity(to_np(y), oracle.lora_linear(x, w0, row_ad, ad), what=f"plan {i} (T={len(row_ad)})")


def test_batched_page_in_beyond_one_launch_and_cross_stream_plan():
    """A page-in batch of 21 adapters over 3 layers (more than one copy launch
    per layer: 16 + 5) on a side stream; a plan created on one stream and used
    on another, with no host synchronisation; every page bit for bit against
    the oracle's pool model, the outputs against the oracle."""
    from heterogeneous_adapter_gemm_amd import DevicePool, LORA_BF16, lora_plan_destroy
    d_in, d_out, P, L = 1024, 1536, 512, 3
    ranks = [(i % 4 + 1) * 4 for i in range(21)]
    g = np.random.default_rng(71)
    n_pages = 2 * L * sum(r * (d_in // P + d_out // P) for r in ranks) + 64
    fo = g.permutation(n_pages).astype(np.int32)
    pool = DevicePool(LORA_BF16, P, n_pages, fo, L, [d_in], [d_out], 24, 16, 64, 4)
    model = PoolModel(n_pages, P, fo, L, [d_in], [d_out], 24, 16)
    blobs = {}
    for i, r in enumerate(ranks):
        A = bf16_bits((g.standard_normal((L * r, d_in)) * d_in ** -0.5).astype(np.float32))
        B = bf16_bits((g.standard_normal((L * r, d_out)) * 0.05).astype(np.float32))
        blobs[i] = (A, B)
    side = torch.cuda.Stream()
    say("page-in batch of 21 adapters, 3 layers, side stream")
    slots = pool.page_in_batch([(i, r, 2.0 * r, blobs[i][0].reshape(-1), blobs[i][1].reshape(-1))
                                for i, r in enumerate(ranks)], stream=side.cuda_stream)
    assert list(slots) == [model.page_in(i, r, 2.0 * r) for i, r in enumerate(ranks)]
    # a plan made on the side stream, used on the main stream (which waits for the copies)
    T = 48
    row_ad = g.choice(np.arange(-1, 21), T).astype(np.int32)
    x = bf16_bits(g.standard_normal((T, d_in)).astype(np.float32))
    w0 = bf16_bits((g.standard_normal((d_out, d_in)) * 0.02).astype(np.float32))
    xd, wd = dev(x), dev(w0)
    y = torch.zeros((T, d_out), dtype=torch.bfloat16, device="cuda")
    say("plan on the side stream, linear on the main stream, layer 2")
    plan = pool.plan(token_slot=[-1 if a < 0 else int(slots[a]) for a in row_ad], stream=side.cuda_stream)
    pool.linear(plan, 2, 0, xd, wd, y, stream=torch.cuda.current_stream().cuda_stream)
    lora_plan_destroy(plan)
    torch.cuda.synchronize()
    pool.drop_host_copies()
    pages = bits(pool.pages).reshape(n_pages, P)
    for i, r in enumerate(ranks):
        for l in range(L):
            A, B = blobs[i][0][l * r:(l + 1) * r], blobs[i][1][l * r:(l + 1) * r]
            for pg, content in model.expected_pages(model.slot_of(i), l, 0, A, B).items():
                assert np.array_equal(pages[pg], content.view(np.int16)), f"adapter {i} layer {l} page {pg}"
    ad = {i: (r, 2.0 * r, blobs[i][0][2 * r:3 * r], blobs[i][1][2 * r:3 * r]) for i, r in enumerate(ranks)}
    parity(to_np(y), oracle.lora_linear(x, w0, row_ad, ad), what="layer 2 after a batched page-in")


def test_page_in_odd_page_counts_and_zero_tails():
    """A page-in batch whose launches hold an odd number of pages (odd ranks:
    125 pages per layer, so the copy's last two-page pass has one page past the
    end) and whose B rows end in a partial page (d_out = 1280 over 512-element
    pages: the last page of each row is half data, half zero tail); every page
    bit for bit against the oracle's pool model, one decode linear against the
    oracle."""
    from heterogeneous_adapter_gemm_amd import DevicePool, LORA_BF16, lora_plan_destroy
    d_in, d_out, P, L = 1024, 1280, 512, 2
    ranks = [3, 5, 7, 1, 9]
    g = np.random.default_rng(73)
    n_pages = L * sum(r * (d_in // P + -(-d_out // P)) for r in ranks) + 40
    fo = g.permutation(n_pages).astype(np.int32)
    pool = DevicePool(LORA_BF16, P, n_pages, fo, L, [d_in], [d_out], 8, 16, 64, 4)
    model = PoolModel(n_pages, P, fo, L, [d_in], [d_out], 8, 16)
    blobs = {}
    for i, r in enumerate(ranks):
        A = bf16_bits((g.standard_normal((L * r, d_in)) * d_in ** -0.5).astype(np.float32))
        B = bf16_bits((g.standard_normal((L * r, d_out)) * 0.05).astype(np.float32))
        blobs[i] = (A, B)
    say("page-in batch of 5 adapters of odd ranks, 125 pages per layer")
    slots = pool.page_in_batch([(i, r, 2.0 * r, blobs[i][0].reshape(-1), blobs[i][1].reshape(-1))
                                for i, r in enumerate(ranks)])
    assert list(slots) == [model.page_in(i, r, 2.0 * r) for i, r in enumerate(ranks)]
    T = 24
    row_ad = g.choice(np.arange(-1, len(ranks)), T).astype(np.int32)
    x = bf16_bits(g.standard_normal((T, d_in)).astype(np.float32))
    w0 = bf16_bits((g.standard_normal((d_out, d_in)) * 0.02).astype(np.float32))
    y = torch.zeros((T, d_out), dtype=torch.bfloat16, device="cuda")
    plan = pool.plan(token_slot=[-1 if a < 0 else int(slots[a]) for a in row_ad])
    pool.linear(plan, 1, 0, dev(x), dev(w0), y)
    lora_plan_destroy(plan)
    torch.cuda.synchronize()
    pool.drop_host_copies()
    pages = bits(pool.pages).reshape(n_pages, P)
    for i, r in enumerate(ranks):
        for l in range(L):
            A, B = blobs[i][0][l * r:(l + 1) * r], blobs[i][1][l * r:(l + 1) * r]
            for pg, content in model.expected_pages(model.slot_of(i), l, 0, A, B).items():
                assert np.array_equal(pages[pg], content.view(np.int16)), f"adapter {i} layer {l} page {pg}"
    ad = {i: (r, 2.0 * r, blobs[i][0][r:2 * r], blobs[i][1][r:2 * r]) for i, r in enumerate(ranks)}
    parity(to_np(y), oracle.lora_linear(x, w0, row_ad, ad), what="layer 1 after a page-in of odd ranks")


@pytest.mark.parametrize("stage", ["min", "two_layers", "none"])
def test_staged_page_in_chunks_and_groups(stage):
    """Page-in through a device staging area (the copy engine brings up to 4
    layers of a group of adapters into it, then a kernel per layer scatters
    them into the pages): 21 adapters of odd ranks over 6 layers, B rows
    ending in a partial page.  'min' is a staging area of one layer of one
    adapter of max_rank, so each copy is one layer of one or two adapters;
    'two_layers' holds two layers of the whole batch, so the layers go in
    chunks of 4 and 2, each in groups of adapters that fit; 'none' is the PCIe
    gather.  Every page bit for bit against the oracle's pool model, and a
    decode linear on the last layer against the oracle, enqueued right after
    the page-in on another stream."""
    from heterogeneous_adapter_gemm_amd import DevicePool, LORA_BF16, lora_plan_destroy
    d_in, d_out, P, L, R = 1024, 1280, 512, 6, 24
    ranks = [(3 * i) % R + 1 for i in range(21)]
    per_layer_rank = d_in + d_out
    stage_bytes = {"min": R * per_layer_rank * 2, "two_layers": 2 * sum(ranks) * per_layer_rank * 2 + 21 * 256,
                   "none": 0}[stage]
    g = np.random.default_rng(75)
    n_pages = L * sum(r * (d_in // P + -(-d_out // P)) for r in ranks) + 40
    fo = g.permutation(n_pages).astype(np.int32)
    pool = DevicePool(LORA_BF16, P, n_pages, fo, L, [d_in], [d_out], 24, R, 64, 4, stage_bytes=stage_bytes)
    model = PoolModel(n_pages, P, fo, L, [d_in], [d_out], 24, R)
    blobs = {}
    for i, r in enumerate(ranks):
        A = bf16_bits((g.standard_normal((L * r, d_in)) * d_in ** -0.5).astype(np.float32))
        B = bf16_bits((g.standard_normal((L * r, d_out)) * 0.05).astype(np.float32))
        blobs[i] = (A, B)
    side = torch.cuda.Stream()
    say("staged page-in", stage, stage_bytes, "bytes of staging, 21 adapters x 6 layers")
    slots = pool.page_in_batch([(i, r, 2.0 * r, blobs[i][0].reshape(-1), blobs[i][1].reshape(-1))
                                for i, r in enumerate(ranks)], stream=side.cuda_stream)
    assert list(slots) == [model.page_in(i, r, 2.0 * r) for i, r in enumerate(ranks)]
    T = 40
    row_ad = g.choice(np.arange(-1, len(ranks)), T).astype(np.int32)
    x = bf16_bits(g.standard_normal((T, d_in)).astype(np.float32))
    w0 = bf16_bits((g.standard_normal((d_out, d_in)) * 0.04).astype(np.float32))
    y = torch.zeros((T, d_out), dtype=torch.bfloat16, device="cuda")
    plan = pool.plan(token_slot=[-1 if a < 0 else int(slots[a]) for a in row_ad])
    pool.linear(plan, L - 1, 0, dev(x), dev(w0), y)
    lora_plan_destroy(plan)
    torch.cuda.synchronize()
    pool.drop_host_copies()
    pages = bits(pool.pages).reshape(n_pages, P)
    for i, r in enumerate(ranks):
        for l in range(L):
            A, B = blobs[i][0][l * r:(l + 1) * r], blobs[i][1][l * r:(l + 1) * r]
            for pg, content in model.expected_pages(model.slot_of(i), l, 0, A, B).items():
                assert np.array_equal(pages[pg], content.view(np.int16)), f"adapter {i} layer {l} page {pg}"
    ad = {i: (r, 2.0 * r, blobs[i][0][(L - 1) * r:L * r], blobs[i][1][(L - 1) * r:L * r]) for i, r in enumerate(ranks)}
    parity(to_np(y), oracle.lora_linear(x, w0, row_ad, ad), what=f"layer {L - 1} after a staged page-in ({stage})")


@pytest.mark.parametrize("T", [64, 200])
def test_heavy_groups_split_by_rows(T):
    """Decode batches where one adapter holds most rows: its shrink work is
    split into units of a few rows and its expand likewise (ragged last
    units), against the oracle; deterministic."""
    from heterogeneous_adapter_gemm_amd import lora_plan_destroy
    d_in, d_out = 1024, 520
    pool, ad, w0, arr = small_pool("bf16", d_in, d_out, [8, 64, 16], [16.0, 128.0, 4.0], seed=81, page_elems=512,
                                   max_tokens=256)
    g = np.random.default_rng(82)
    row_ad = np.full(T, 1, np.int32)
    row_ad[g.choice(T, T // 6, replace=False)] = 0
    row_ad[g.choice(T, 3, replace=False)] = -1
    row_ad[g.choice(T, 2, replace=False)] = 2
    x = arr(T, d_in)
    xd, wd = dev(x), dev(w0)
    say("heavy groups", T, np.bincount(row_ad + 1).tolist())
    ts = [-1 if a < 0 else pool.slot_of(int(a)) for a in row_ad]
    ys = []
    for _ in range(2):
        y = torch.zeros((T, d_out), dtype=torch.bfloat16, device="cuda")
        plan = pool.plan(token_slot=ts)
        pool.linear(plan, 0, 0, xd, wd, y)
        lora_plan_destroy(plan)
        ys.append(y)
    torch.cuda.synchronize()
    assert np.array_equal(bits(ys[0]), bits(ys[1]))
    parity(to_np(ys[0]), oracle.lora_linear(x, w0, row_ad, ad), what=f"heavy groups T={T}")


def bits_to(t):
    """bf16 device tensor -> uint16 numpy bits."""
    return bits(t).view(np.uint16)


def long_tiles(M, N, cus=256):
    """The long-batch GEMM's choice for M x N (M > 256), as the library makes it: tile height
    256 or 192 by an estimated time, the tiles past the last full round cut into pieces (2,
    4, 8 or 16 per tile for height 256, halves for 192) -> (height, tiles, tiles cut, pieces)."""
    def pieces(rem):
        return 16 if rem * 16 <= cus else 8 if rem * 8 <= cus else 4 if rem * 4 <= cus else 2

    def plan(bm):
        tiles = -(-M // bm) * -(-N // 256)
        rem = tiles % cus if tiles > cus else 0
        f = 1.0 if bm == 256 else 0.85
        if tiles <= cus:
            return f * (1.0 - 0.58 * (1.0 - tiles / cus)), tiles, rem
        tail = 0.0
        if rem:
            p = pieces(rem) if bm == 256 else 2
            tail = (0.5 if bm == 256 else 0.58) * -(-2 * rem // cus) if p == 2 else 1.5 / p
        return f * (tiles // cus + tail), tiles, rem
    a, b = plan(256), plan(192)
    if a[0] <= b[0]:
        return 256, a[1], a[2], pieces(a[2]) if a[2] else 0
    return 192, b[1], b[2], 2 if b[2] else 0


# (segment lengths, d_out, height, pieces): 4352 rows x 4096: 272 tiles of 256 x 256, 16
# of them in 16 pieces; 4100 x 4608: 306 tiles, 50 in quarters; 2070 x 11008: 473 tiles
# of 192 x 256, 217 in halves
LONG_CASES = [([1500, 1300, 1552], 4096, 256, 16), ([1400, 1200, 1500], 4608, 256, 4),
              ([700, 600, 770], 11008, 192, 2)]


@pytest.mark.parametrize("lens,d_out,height,n_pieces", LONG_CASES)
def test_long_batch_tail_split_and_fused_expand(lens, d_out, height, n_pieces):
    """Long batches: the tiles past the last full round of the chip (one workgroup per CU)
    run in a second launch cut into pieces; prefill segments (two with adapters, one
    without) get their expand in the GEMM's epilogue.  Rows sampled from every 64-row block,
    all columns, against the oracle; two runs agree bit for bit."""
    from heterogeneous_adapter_gemm_amd import lora_plan_destroy
    d_in = 256
    T = sum(lens)
    bm, tiles, rem, npc = long_tiles(T, d_out)
    assert (bm, npc) == (height, n_pieces) and rem > 0, (bm, tiles, rem, npc)
    pool, ad, w0, arr = small_pool("bf16", d_in, d_out, [16, 64], [32.0, 7.0], seed=41, page_elems=512,
                                   max_tokens=T, max_segments=4)
    sadp = [0, -1, 1]
    x = arr(T, d_in)
    st = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    row_ad = np.concatenate([np.full(n, a, np.int32) for n, a in zip(lens, sadp)])
    xd, wd = dev(x), dev(w0)
    say("long batch tail split", T, d_out, d_in, f"tiles of {bm} rows: {tiles}, {rem} cut in {npc}")
    y = torch.zeros((T, d_out), dtype=torch.bfloat16, device="cuda")
    plan = pool.plan(st, [-1 if a < 0 else pool.slot_of(a) for a in sadp])
    pool.linear(plan, 0, 0, xd, wd, y)
    y2 = torch.zeros_like(y)
    pool.linear(plan, 0, 0, xd, wd, y2)
    torch.cuda.synchronize()
    lora_plan_destroy(plan)
    assert np.array_equal(bits(y), bits(y2)), "two runs (whole and half tiles) must agree bit for bit"
    g = np.random.default_rng(42)
    rows = sorted(set(int(r) for t in range(-(-T // 64)) for r in g.integers(64 * t, min(64 * (t + 1), T), 4)))
    parity(to_np(y)[rows], oracle.lora_linear(x, w0, row_ad, ad, rows=rows), what="tail split + fused")


def test_measurement_probes_run():
    """The measurement probes launch and finish: the read probe over in-range and
    clamped chunk indices (it writes nothing unless its checksum takes one fixed value,
    which a buffer of ones never gives), the matrix-core probe with its checksum."""
    import heterogeneous_adapter_gemm_amd as hg
    say("probes")
    buf = torch.ones(1 << 20, dtype=torch.uint8, device="cuda")          # 128 chunks of 8 KiB
    chunk = torch.tensor([0, 5, 127, 128, -3, 1 << 40], dtype=torch.int64, device="cuda")   # the last three clamped
    out = torch.full((6,), -1.0, dtype=torch.float32, device="cuda")
    hg.lora_probe_read(buf, buf.numel(), chunk, 6, out)
    torch.cuda.synchronize()
    assert torch.all(out == -1.0), "the read probe writes nothing for a buffer of ones"
    res = torch.empty(4 * 8, dtype=torch.float32, device="cuda")
    for shape in (16, 32):
        flops = hg.lora_probe_mfma(shape, 4, 8, res)
        torch.cuda.synchronize()
        assert flops == 8 * 4 * 4 * 8 * 2.0 * (8192 if shape == 16 else 16384)
        assert torch.isfinite(res).all()
