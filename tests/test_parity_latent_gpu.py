"""GPU parity of latent decoding (EntropyInfer Sec. 4.3, App. B) through the C
ABI: a decode loop over a prompt cache with compressions after N_D generated
tokens and every `interval` tokens after that, against the oracle's loop.

At each compression the GPU's keep set must satisfy the band rule on the
oracle's scores (exact outside a 1e-4/L band around the cutoff; sinks and
recent entries kept); the oracle then continues from the GPU's keep set, so
both sides hold the same cache and every step's output is compared."""
import numpy as np
import pytest
import torch

from _parity import ATTN_MAX_ABS, ATTN_REL_L2, attn_errors, dev_tensor, log
from entropy_guided_sparse_amd import synth
from oracle import egs_oracle as O

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def api():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    from entropy_guided_sparse_amd import api as A
    return A


def _bf16(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).bfloat16()


# (B, Hq, Hkv, prompt length, spare capacity, n_keep, N_D, interval, tokens).
# The batch-8 case runs near 4,480 entries in an 8,192-row cache.  The
# attention split the launcher picks is not monotone in the length (a shorter
# list can take a smaller split and so more partials), so the step's workspace
# is sized for every length up to the capacity, not for the capacity alone.
CASES = [(2, 8, 2, 2048, 0, 512, 96, 64, 170),
         (2, 8, 2, 2048, 0, 512, 10, 0, 40),
         (8, 32, 8, 4466, 8192 - 4466 - 24, 4096, 16, 0, 24)]


@pytest.mark.parametrize("B,Hq,Hkv,L0,spare,n_keep,n_delay,interval,T", CASES)
def test_latent_decode_loop(api, B, Hq, Hkv, L0, spare, n_keep, n_delay, interval, T):
    L_ = api.L
    d, W = 128, 64
    n_sink, n_recent = 4, 256
    cfg = synth.DecodeConfig("latent", B, Hq, Hkv, d, L0, W, n_sink, n_recent, n_keep)
    inp = synth.make_decode(cfg, seed=5)
    log(f"[latent] B={B} Hq={Hq} L0={L0} cap={L0 + T + spare} T={T} n_delay={n_delay} "
        f"interval={interval}")
    rng = np.random.default_rng(6)
    # generated tokens: Gaussian, with queries drawn towards random prompt keys
    steps = []
    for _ in range(T):
        q = rng.standard_normal((B, Hq, d))
        for b in range(B):
            for h in range(Hq):
                t = int(rng.integers(L0))
                q[b, h] += 0.5 * inp.k[b, h // (Hq // Hkv), t]
        k = rng.standard_normal((B, Hkv, d))
        v = rng.standard_normal((B, Hkv, d))
        steps.append(tuple(_bf16(x) for x in (q, k, v)))
    C = L0 + T + spare
    shape = api.DecodeShape(B, Hq, Hkv, d, C, W, n_sink, n_recent, n_keep)
    prm = api.RetainParams(entropy_kind=L_.EGS_SHANNON, zeta=0.5, tau=1.0)
    k_cache = torch.zeros((B, Hkv, C, d), dtype=torch.bfloat16, device="cuda")
    v_cache = torch.zeros_like(k_cache)
    k_cache[:, :, :L0] = dev_tensor(inp.k_store, "bf16")
    v_cache[:, :, :L0] = dev_tensor(inp.v_store, "bf16")
    q_win = dev_tensor(inp.q_obs_store, "bf16").clone()
    ntot = min(C, n_sink + n_recent + n_keep)
    keep_buf = torch.empty((B * Hkv * ntot,), dtype=torch.int32, device="cuda")
    out = torch.empty((B, Hq, d), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(L_.LIB.egs_latent_decode_workspace(shape.c()), dtype=torch.uint8,
                     device="cuda")
    st = L_.LatentStateC(length=L0, generated=0, n_delay=n_delay, interval=interval,
                         compressed=0)
    outs, keeps = [], {}
    for s, (q, k, v) in enumerate(steps, 1):
        api.latent_decode_step(shape, prm, st, q.cuda(), k.cuda(), v.cuda(), q_win, k_cache,
                               v_cache, out=out, keep_idx=keep_buf, workspace=ws)
        outs.append(out.float().cpu().numpy())
        if st.compressed:
            n = st.length
            keeps[s] = keep_buf[:B * Hkv * n].view(B, Hkv, n).cpu().numpy()
        torch.cuda.synchronize()
    assert st.generated == T
    assert sorted(keeps) == [s for s in range(1, T + 1) if O.latent_due(s, n_delay, interval)]

    def follow(step, b, g, keep, mu):
        got = keeps[step][b, g]
        L = mu.size
        band = 1e-4 / L
        assert got[:n_sink].tolist() == list(range(n_sink))
        assert got[-n_recent:].tolist() == list(range(L - n_recent, L))
        cand = np.arange(n_sink, L - n_recent)
        sel = np.isin(cand, got)
        sc = mu[cand]
        c = np.sort(sc)[::-1][n_keep - 1]
        assert not np.any((sc > c + band) & ~sel) and not np.any((sc < c - band) & sel)
        return got

    to64 = lambda t: t.float().numpy().astype(np.float64)
    r_outs, events = O.latent_decode(inp.k, inp.v, inp.q_obs,
                                     [(to64(q), to64(k), to64(v)) for (q, k, v) in steps],
                                     n_sink, n_recent, n_keep, n_delay, interval,
                                     keep_fn=follow)
    worst = 0.0
    for s in range(T):
        ma, rel = attn_errors(outs[s], r_outs[s])
        worst = max(worst, ma)
        assert ma <= ATTN_MAX_ABS and rel <= ATTN_REL_L2, (s, ma, rel)
    log(f"  {len(events)} compressions, worst step max|d|={worst:.3e}")
