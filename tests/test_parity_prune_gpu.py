"""GPU parity of chunk pruning (EntroPrefill Sec. 3.1-3.2, 4.1-4.2) through the
C ABI: row-chunk masses and priorities against the oracle's float64 values,
and the removal decisions bit-exact against the oracle's greedy proposer run
on the GPU's own float32 priorities and masses, in float32 (floating point
decides the integer outputs, so both sides decide in the same precision);
and against the oracle's own float64 priorities and masses under a band rule
(the scan order and every decision equal unless within a rounding band)."""
import numpy as np
import pytest
import torch

from _parity import dev_tensor, log
from entropy_guided_sparse_amd import synth
from oracle import egs_oracle as O

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def api():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    from entropy_guided_sparse_amd import api as A
    return A


# Priorities: S = ln l + lambda kappa of float32 chunk sums of the pooled
# measure; measured within 3e-6 of the oracle's float64 values.  5e-5 keeps
# ~15x margin over that and stays below the 1e-4 band in which the scan order
# of two chunks may swap.
PRIO_ATOL = 5e-5
# Scan decisions are compared with the oracle's own float64 values: two chunks
# may be scanned in either order when their priorities lie within ORDER_BAND,
# and a decision may go either way when a row sum lands within MASS_BAND of
# its budget (row masses are float32 sums, measured within 3e-6).
ORDER_BAND = 1e-4
MASS_BAND = 5e-5


def _chunks(rng, T, W, k, lo=64):
    """k disjoint chunks with protected gaps, before the observers."""
    edges = np.sort(rng.choice(np.arange(lo, T - W), 2 * k, replace=False))
    return [(int(edges[2 * i]), int(edges[2 * i + 1])) for i in range(k)]


def _run(api, Hq, Hkv, T, W, chunks, eps_s, lam, eps, m0, target, seed=0, n_sink=4):
    cfg = synth.DecodeConfig("prune", 1, Hq, Hkv, 128, T, W, n_sink, 16, 16)
    inp = synth.make_decode(cfg, seed=seed)
    log(f"[prune] Hq={Hq} Hkv={Hkv} T={T} W={W} chunks={len(chunks)} eps={eps} m0={m0} "
        f"target={target} lam={lam}")
    shape = api.DecodeShape(1, Hq, Hkv, 128, T, W, n_sink, 16, 16)
    q = dev_tensor(inp.q_obs_store[0], "bf16")
    k = dev_tensor(inp.k_store[0], "bf16")
    removed, tokens, prio, mass = api.chunk_prune(shape, q, k, chunks, eps_s, lam, eps, m0,
                                                  target, want_row_mass=True)
    torch.cuda.synchronize()
    g_rem = removed.cpu().numpy().astype(bool)
    g_tok = int(tokens.cpu().item())
    g_S = prio.cpu().numpy()
    g_m = mass.cpu().numpy()                          # [k, R]
    mu, A = O.prune_pooled_measure(inp.q_obs[0], inp.k[0], n_sink)
    r_m = O.prune_row_chunk_mass(A, chunks)           # [R, k]
    r_S = O.prune_priorities(mu, chunks, eps_s, lam)[0]
    dm = float(np.abs(g_m.T - r_m).max())
    dS = float(np.abs(g_S - r_S).max())
    log(f"  row mass max|d|={dm:.3e} priority max|d|={dS:.3e} removed={int(g_rem.sum())} "
        f"tokens={g_tok}")
    assert dm <= 1e-4
    assert dS <= PRIO_ATOL
    n = np.array([e - b for (b, e) in chunks])
    o_rem, o_tok = O.prune_greedy(g_S.astype(np.float64), n, g_m.T, eps, m0, target,
                                  dtype=np.float32)
    np.testing.assert_array_equal(g_rem, o_rem)
    assert g_tok == o_tok
    _oracle_scan_agrees(r_S, n, r_m, eps, m0, target, g_rem, g_S)
    # feasibility of the GPU's set on the oracle's own masses (within rounding)
    assert np.all(r_m[:, g_rem].sum(axis=1) <= eps + 1e-4)
    assert g_rem.sum() <= max(len(chunks) - m0, 0)
    return g_rem, g_tok


def _oracle_scan_agrees(S, n, m, eps, m0, target, g_rem, g_S):
    """Band rule for the greedy scan against the oracle's own float64 values.

    Order: the GPU's scan order (its priorities, ties by larger n, then index)
    may invert two chunks only where the oracle's priorities lie within
    ORDER_BAND.  Decisions: walking that order with the oracle's float64 row
    masses, every decision must equal the oracle's, except where a row sum
    after adding the chunk lies within MASS_BAND of eps; there the walk takes
    the GPU's decision and goes on.  Returns the number of such steps."""
    S = np.asarray(S, dtype=np.float64)
    m = np.asarray(m, dtype=np.float64)
    k = len(S)
    order = sorted(range(k), key=lambda i: (float(g_S[i]), -int(n[i]), i))
    So = S[order]
    # no inversion beyond the band: every later chunk's oracle priority is at
    # least the running maximum so far minus the band
    assert np.all(So >= np.maximum.accumulate(So) - ORDER_BAND), "scan order inverted"
    cur = np.zeros(m.shape[0])
    tokens = count = 0
    near = 0
    for p, i in enumerate(order):
        if tokens >= target or count + 1 > k - m0:
            assert not g_rem[order[p:]].any(), ("removed after the scan stopped", p)
            break
        nxt = cur + m[:, i]
        take = bool(np.all(nxt <= eps))
        if np.any(np.abs(nxt - eps) <= MASS_BAND):
            near += 1
            take = bool(g_rem[i])
        assert g_rem[i] == take, ("scan step", p, "chunk", i)
        if take:
            cur = nxt
            tokens += int(n[i])
            count += 1
    log(f"  oracle float64 scan: all {k} decisions equal ({near} within the mass band)")
    return near


@pytest.mark.parametrize("case", ["basic", "tight_rows", "loose_rows", "count_bound",
                                  "nothing_removable", "zero_target", "w_odd"])
def test_chunk_prune(api, case):
    rng = np.random.default_rng(3)
    T, W = 4096, 64
    chunks = _chunks(rng, T, W, 24)
    kw = dict(Hq=8, Hkv=2, T=T, W=W, chunks=chunks, eps_s=0.1, lam=0.5, eps=0.05, m0=2,
              target=T // 2)
    if case == "tight_rows":
        kw.update(eps=0.005)
    elif case == "loose_rows":
        kw.update(eps=10.0, target=10 ** 6)
    elif case == "count_bound":
        kw.update(eps=10.0, target=10 ** 6, m0=20)
    elif case == "nothing_removable":
        kw.update(eps=0.0)
    elif case == "zero_target":
        kw.update(target=0)
    elif case == "w_odd":
        kw.update(W=40, Hq=6, Hkv=3, lam=1.5, chunks=_chunks(rng, T, 40, 31))
    rem, tok = _run(api, **kw)
    if case == "loose_rows":                  # only the count bound k - m0 binds
        assert rem.sum() == 24 - 2
    if case == "count_bound":
        assert rem.sum() == 24 - 20
    if case in ("nothing_removable", "zero_target"):
        assert not rem.any() and tok == 0


@pytest.mark.parametrize("k,eps", [(300, 0.02), (300, 0.3), (700, 0.05)])
def test_chunk_prune_many_chunks(api, k, eps):
    # 300 chunks: rank order, ten fetched batches of the scan; 700: bitonic sort
    rng = np.random.default_rng(k)
    T, W = 8192, 64
    chunks = _chunks(rng, T, W, k, lo=8)
    _run(api, 8, 2, T, W, chunks, 0.1, 0.5, eps, 5, T // 3, seed=k)


def test_chunk_prune_single_and_unit_chunks(api):
    _run(api, 4, 2, 1024, 32, [(100, 101)], 0.2, 0.3, 1.0, 0, 10)
    _run(api, 4, 2, 1024, 32, [(5, 6), (6, 9), (9, 300), (400, 401), (500, 990)], 0.2, 0.3,
         0.5, 1, 10 ** 6)


def test_chunk_prune_full_context(api):
    """One 128k prompt with 32 query / 8 KV heads, 64 observers and 64 candidate
    documents (the decode workload's shape at batch 1, the launch the bench
    times): priorities against the oracle's pooled measure, the row masses of
    three sampled heads against the oracle's rows, the greedy decisions
    replayed on the GPU's values, and feasibility."""
    cfg = synth.DECODE_CONFIGS["decode-retain-b8-128k"]
    inp = synth.make_decode(cfg, seed=11, batch=1)
    Hq, Hkv, W, T = cfg.n_q_heads, cfg.n_kv_heads, cfg.n_obs, cfg.cache_len
    chunks = synth.prune_chunks(T, W, 64, seed=11)
    eps, m0, target = 0.1, 4, T // 2
    log(f"[prune full] Hq={Hq} Hkv={Hkv} T={T} W={W} chunks=64")
    shape = api.DecodeShape(1, Hq, Hkv, cfg.head_dim, T, W, cfg.n_sink, cfg.n_recent,
                            cfg.n_keep)
    q = dev_tensor(inp.q_obs_store[0], "bf16")
    k = dev_tensor(inp.k_store[0], "bf16")
    removed, tokens, prio, mass = api.chunk_prune(shape, q, k, chunks, 0.1, 0.5, eps, m0,
                                                  target, want_row_mass=True)
    torch.cuda.synchronize()
    g_rem = removed.cpu().numpy().astype(bool)
    g_tok = int(tokens.cpu().item())
    g_S = prio.cpu().numpy()
    g_m = mass.cpu().numpy().T                        # [R, k]
    del q, k
    cl = [tuple(map(int, c)) for c in chunks]
    mu, _ = O.prune_pooled_measure(inp.q_obs[0], inp.k[0], cfg.n_sink, rows=False)
    r_S = O.prune_priorities(mu, cl, 0.1, 0.5)[0]
    dS = float(np.abs(g_S - r_S).max())
    dm = 0.0
    for h in (0, 13, Hq - 1):
        r_m = O.prune_row_chunk_mass(O.prune_head_rows(inp.q_obs[0], inp.k[0], h)[None], cl)
        dm = max(dm, float(np.abs(g_m[h * W:(h + 1) * W] - r_m).max()))
    log(f"  priority max|d|={dS:.3e} sampled row mass max|d|={dm:.3e} "
        f"removed={int(g_rem.sum())} tokens={g_tok}")
    assert dS <= PRIO_ATOL and dm <= 1e-4
    n = chunks[:, 1] - chunks[:, 0]
    o_rem, o_tok = O.prune_greedy(g_S.astype(np.float64), n, g_m, eps, m0, target,
                                  dtype=np.float32)
    np.testing.assert_array_equal(g_rem, o_rem)
    assert g_tok == o_tok == int(n[g_rem].sum())
    # the oracle's own decisions need every row's masses; they are formed here
    # head by head from the oracle's rows (the GPU's masses are not used)
    r_all = np.concatenate([O.prune_row_chunk_mass(O.prune_head_rows(inp.q_obs[0], inp.k[0],
                                                                     h)[None], cl)
                            for h in range(Hq)], axis=0)
    assert float(np.abs(g_m - r_all).max()) <= 1e-4
    _oracle_scan_agrees(r_S, n, r_all, eps, m0, target, g_rem, g_S)
    assert np.all(g_m[:, g_rem].astype(np.float64).sum(axis=1) <= eps + 1e-5)
    # chunks never hold more than a row's whole mass (protected tokens hold the rest)
    assert np.all(g_m.astype(np.float64).sum(axis=1) <= 1.0 + 1e-4)


def test_prune_certificate(api):
    """U(y, t) on the GPU's row masses: float64 on both sides over the same
    float32 inputs (only the order of the sums differs), weak duality against
    the greedy removal, and the trivial and scalar-price cases."""
    cfg = synth.DecodeConfig("cert", 1, 8, 2, 128, 4096, 64, 4, 16, 16)
    inp = synth.make_decode(cfg, seed=2)
    chunks = synth.prune_chunks(4096, 64, 40, seed=2)
    shape = api.DecodeShape(1, 8, 2, 128, 4096, 64, 4, 16, 16)
    q = dev_tensor(inp.q_obs_store[0], "bf16")
    k = dev_tensor(inp.k_store[0], "bf16")
    eps, m0 = 0.05, 3
    removed, tokens, _, mass = api.chunk_prune(shape, q, k, chunks, 0.1, 0.5, eps, m0, 4096,
                                               want_row_mass=True)
    torch.cuda.synchronize()
    g_m = mass.cpu().numpy().T.astype(np.float64)     # [R, k]
    n = chunks[:, 1] - chunks[:, 0]
    got_tokens = int(tokens.cpu().item())
    rng = np.random.default_rng(8)
    R = g_m.shape[0]
    cases = [(np.zeros(R), 0.0), (np.full(R, 40.0), 2.0)] + \
            [(rng.uniform(0, 200, R), float(rng.uniform(0, 50))) for _ in range(4)]
    for y, t in cases:
        yd = torch.from_numpy(y.astype(np.float32)).cuda()
        U = float(api.prune_certificate(chunks, mass, yd, eps, m0, t).cpu().item())
        want = O.prune_certificate(n, g_m, eps, m0, y.astype(np.float32).astype(np.float64), t)
        log(f"[cert] t={t:.2f} U={U:.6f} oracle={want:.6f} greedy tokens={got_tokens}")
        assert abs(U - want) <= 1e-9 * max(1.0, abs(want))
        assert U >= got_tokens - 1e-6
    assert float(api.prune_certificate(chunks, mass, torch.zeros(R, device="cuda"), eps, m0,
                                       0.0).cpu().item()) == float(n.sum())


@pytest.mark.parametrize("bad", [[[10, 100], [90, 200]], [[10, 100], [100, 4040]],
                                 [[50, 50], [60, 70]], [[-5, 10]], [[3000, 2000]]])
def test_chunk_prune_invalid_device_bounds(api, bad):
    """Chunk bounds handed over in device memory are checked on the device:
    overlapping, observer-reaching, empty, negative or reversed chunks remove
    nothing and report removed_tokens = -1 (all accesses stay in bounds)."""
    T, W = 4096, 64
    cfg = synth.DecodeConfig("prune-bad", 1, 8, 2, 128, T, W, 4, 16, 16)
    inp = synth.make_decode(cfg, seed=21)
    shape = api.DecodeShape(1, 8, 2, 128, T, W, 4, 16, 16)
    q = dev_tensor(inp.q_obs_store[0], "bf16")
    k = dev_tensor(inp.k_store[0], "bf16")
    b = torch.tensor(bad, dtype=torch.int32, device="cuda")
    removed, tokens, prio, _ = api.chunk_prune(shape, q, k, b, 0.1, 0.5, 1.0, 0, T)
    torch.cuda.synchronize()
    log(f"[prune bad bounds] {bad} -> tokens {int(tokens.item())}")
    assert int(tokens.item()) == -1
    assert not removed.cpu().numpy().any()
    assert torch.isnan(prio).all()
    # the same call on valid device bounds still works after a failed one
    good = torch.tensor([[10, 100], [100, 200], [300, 4032]], dtype=torch.int32, device="cuda")
    removed, tokens, prio, _ = api.chunk_prune(shape, q, k, good, 0.1, 0.5, 1.0, 0, T)
    torch.cuda.synchronize()
    assert int(tokens.item()) >= 0 and torch.isfinite(prio).all()
