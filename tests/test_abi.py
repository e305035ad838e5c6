"""Host-side checks of the C ABI (no GPU needed): libegs.so loads, exports every
entry point include/egs.h declares, and rejects invalid arguments on the host
with a status and a message before anything is launched."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "egs.h")


def _declared():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(egs_[a-z0-9_]+)\s*\(", txt)))


@pytest.fixture(scope="module")
def L():
    from entropy_guided_sparse_amd import _lib
    return _lib


def test_header_declares_the_boundary():
    names = _declared()
    for n in ["egs_entropy_score", "egs_allocate_budget", "egs_select_blocks",
              "egs_sparse_prefill_attn", "egs_kv_retain", "egs_sparse_decode_attn"]:
        assert n in names


def test_library_exports_every_declared_symbol(L):
    lib = ctypes.CDLL(L.LIB_PATH)
    missing = [n for n in _declared() if not hasattr(lib, n)]
    assert not missing, missing
    # the binding mirrors the header one to one
    assert sorted(L.SIGNATURES) == _declared()


def test_abi_version_and_status_strings(L):
    assert L.LIB.egs_abi_version() == 7
    for st in range(5):
        assert L.LIB.egs_status_string(st).decode().startswith("EGS_")


def _shape(L, **kw):
    base = dict(n_q_heads=4, n_kv_heads=2, head_dim=64, seq_len=2048, block_size=64,
                segment_size=512, probe_len=64, dtype=L.EGS_BF16, sm_scale=0.0)
    base.update(kw)
    return L.PrefillShapeC(**base)


FAKE = ctypes.c_void_p(1 << 20)   # never dereferenced: every call below fails first


@pytest.fixture(autouse=True)
def _no_device(request):
    # The error-path calls pass placeholder pointers.  They are rejected on the
    # host, but a mistake in a case would launch a kernel on them: never run
    # these where a HIP device is visible.
    if request.node.name.startswith(("test_header", "test_library", "test_abi_version")):
        return
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("host-only error-path checks do not run where a device is visible")


@pytest.mark.parametrize("kw,status", [
    (dict(seq_len=2000), "EINVAL"),          # N % L_S != 0
    (dict(segment_size=500), "EINVAL"),      # L_S % L_B != 0
    (dict(probe_len=0), "EINVAL"),
    (dict(probe_len=1024), "EINVAL"),        # P > L_S
    (dict(n_q_heads=5), "EINVAL"),           # Hq % Hkv != 0
    (dict(dtype=7), "EINVAL"),
    (dict(sm_scale=-1.0), "EINVAL"),
    (dict(head_dim=96), "ENOTSUP"),
    (dict(block_size=40, segment_size=480, seq_len=1920), "ENOTSUP"),
    (dict(block_size=512, segment_size=1024), "ENOTSUP"),
])
def test_prefill_shape_errors(L, kw, status):
    sc = _shape(L, **kw)
    st = L.LIB.egs_entropy_score(ctypes.byref(sc), 0, 0, 2.0, FAKE, FAKE, FAKE, FAKE, FAKE,
                                 1 << 30, None)
    assert st == getattr(L, "EGS_" + status)
    assert L.LIB.egs_last_error().decode()
    assert L.LIB.egs_entropy_score_workspace(ctypes.byref(sc)) == 0


def test_entropy_score_argument_errors(L):
    sc = _shape(L)
    ws = L.LIB.egs_entropy_score_workspace(ctypes.byref(sc))
    assert ws > 0
    call = lambda pool=0, kind=0, alpha=2.0, q=FAKE, wsb=ws: L.LIB.egs_entropy_score(
        ctypes.byref(sc), pool, kind, alpha, q, FAKE, FAKE, FAKE, FAKE, wsb, None)
    # max/min pooling is validated like the mean probe before anything launches
    assert call(pool=1, q=None) == L.EGS_EINVAL
    assert call(pool=1, wsb=ws - 1) == L.EGS_EWORKSPACE
    assert call(pool=9) == L.EGS_EINVAL
    assert call(kind=5) == L.EGS_EINVAL
    assert call(kind=1, alpha=0.0) == L.EGS_EINVAL
    assert call(kind=1, alpha=float("inf")) == L.EGS_EINVAL
    assert call(q=None) == L.EGS_EINVAL
    assert "q is NULL" in L.LIB.egs_last_error().decode()
    assert call(q=ctypes.c_void_p((1 << 20) + 2)) == L.EGS_EINVAL   # misaligned
    assert call(wsb=ws - 1) == L.EGS_EWORKSPACE


def test_budget_and_select_errors(L):
    sc = _shape(L)
    pol = L.BudgetPolicyC(mode=9)
    assert L.LIB.egs_allocate_budget(ctypes.byref(sc), ctypes.byref(pol), FAKE, FAKE, FAKE,
                                     None) == L.EGS_EINVAL
    pol = L.BudgetPolicyC(mode=L.EGS_BUDGET_ALG3, base_tokens=0.0, entropy_threshold=1e-5)
    assert L.LIB.egs_allocate_budget(ctypes.byref(sc), ctypes.byref(pol), FAKE, FAKE, FAKE,
                                     None) == L.EGS_EINVAL
    pol = L.BudgetPolicyC(mode=L.EGS_BUDGET_PROPORTIONAL, frac_min=0.5, frac_max=0.1)
    assert L.LIB.egs_allocate_budget(ctypes.byref(sc), ctypes.byref(pol), FAKE, FAKE, FAKE,
                                     None) == L.EGS_EINVAL
    pol = L.BudgetPolicyC(mode=L.EGS_BUDGET_FIXED, frac=0.25)
    assert L.LIB.egs_allocate_budget(ctypes.byref(sc), None, FAKE, FAKE, FAKE,
                                     None) == L.EGS_EINVAL
    assert L.LIB.egs_allocate_budget(ctypes.byref(sc), ctypes.byref(pol), None, FAKE, FAKE,
                                     None) == L.EGS_EINVAL
    CB = 2048 // 64
    for kmax in (0, CB + 1):
        assert L.LIB.egs_select_blocks(ctypes.byref(sc), FAKE, FAKE, kmax, FAKE, FAKE,
                                       None) == L.EGS_EINVAL
    assert L.LIB.egs_sparse_prefill_attn(ctypes.byref(sc), FAKE, FAKE, FAKE, FAKE, FAKE, 0,
                                         FAKE, None, FAKE, 1 << 30, None) == L.EGS_EINVAL
    # out aliasing q
    assert L.LIB.egs_sparse_prefill_attn(ctypes.byref(sc), FAKE, ctypes.c_void_p(2 << 20),
                                         ctypes.c_void_p(3 << 20), FAKE, FAKE, 4, FAKE, None,
                                         FAKE, 1 << 30, None) == L.EGS_EINVAL
    # the bf16 MFMA path needs the packed-V workspace, Hkv * N * d * 2 bytes,
    # and 8 KB of work-queue counters
    aws = L.LIB.egs_sparse_prefill_attn_workspace(ctypes.byref(sc))
    assert aws == 2 * 2048 * 64 * 2 + 8192
    assert L.LIB.egs_sparse_prefill_attn(ctypes.byref(sc), FAKE, ctypes.c_void_p(2 << 20),
                                         ctypes.c_void_p(3 << 20), FAKE, FAKE, 4,
                                         ctypes.c_void_p(4 << 20), None, FAKE, aws - 1,
                                         None) == L.EGS_EWORKSPACE
    sc32 = _shape(L, dtype=L.EGS_F32)
    assert L.LIB.egs_sparse_prefill_attn_workspace(ctypes.byref(sc32)) == 0


def _dshape(L, **kw):
    base = dict(batch=2, n_q_heads=8, n_kv_heads=2, head_dim=128, cache_len=4096, n_obs=64,
                n_sink=4, n_recent=256, n_keep=512, dtype=L.EGS_BF16, sm_scale=0.0)
    base.update(kw)
    return L.DecodeShapeC(**base)


def test_decode_totals_and_workspace(L):
    sc = _dshape(L)
    assert L.LIB.egs_kv_retain_total(ctypes.byref(sc)) == 4 + 256 + 512
    sc = _dshape(L, n_keep=8000)
    assert L.LIB.egs_kv_retain_total(ctypes.byref(sc)) == 4096   # keep everything
    assert L.LIB.egs_kv_retain_workspace(ctypes.byref(sc)) > 0


@pytest.mark.parametrize("kw,status", [
    (dict(n_q_heads=7), "EINVAL"),
    (dict(n_obs=0), "EINVAL"),
    (dict(n_obs=5000), "EINVAL"),
    (dict(n_sink=-1), "EINVAL"),
    (dict(dtype=1), "ENOTSUP"),          # f32 decode
    (dict(head_dim=96), "ENOTSUP"),
    (dict(n_obs=129), "ENOTSUP"),
    (dict(n_q_heads=68, n_kv_heads=2), "ENOTSUP"),
])
def test_decode_shape_errors(L, kw, status):
    sc = _dshape(L, **kw)
    prm = L.RetainParamsC(0, 2.0, 0.5, 1.0, 0, 1.0)
    st = L.LIB.egs_kv_retain(ctypes.byref(sc), ctypes.byref(prm), FAKE, FAKE, FAKE, None, FAKE,
                             FAKE, FAKE, None, None, FAKE, 1 << 40, None)
    assert st == getattr(L, "EGS_" + status)
    assert L.LIB.egs_kv_retain_total(ctypes.byref(sc)) == -1


def test_retain_param_errors(L):
    sc = _dshape(L)
    ws = L.LIB.egs_kv_retain_workspace(ctypes.byref(sc))

    def call(prm, k_out=FAKE, v_out=FAKE, wsb=ws):
        return L.LIB.egs_kv_retain(ctypes.byref(sc), ctypes.byref(prm), FAKE, FAKE, FAKE, None,
                                   FAKE, k_out, v_out, None, None, FAKE, wsb, None)

    P = lambda **kw: L.RetainParamsC(**{**dict(entropy_kind=0, renyi_alpha=2.0, zeta=0.5,
                                                 tau=1.0, raw_logit_mode=0, info_alpha=1.0),
                                        **kw})
    assert call(P(zeta=0.0)) == L.EGS_EINVAL
    assert call(P(zeta=1.5)) == L.EGS_EINVAL
    assert call(P(tau=0.0)) == L.EGS_EINVAL
    assert call(P(info_alpha=1.5)) == L.EGS_EINVAL
    assert call(P(entropy_kind=1, renyi_alpha=-1.0)) == L.EGS_EINVAL
    assert call(P(raw_logit_mode=2)) == L.EGS_EINVAL
    assert call(P(), v_out=None) == L.EGS_EINVAL
    assert call(P(), wsb=ws - 1) == L.EGS_EWORKSPACE
    # decode attention
    assert L.LIB.egs_sparse_decode_attn(ctypes.byref(sc), FAKE, FAKE, FAKE, 0, FAKE, FAKE,
                                        1 << 30, None) == L.EGS_EINVAL
    assert L.LIB.egs_sparse_decode_attn(ctypes.byref(sc), FAKE, FAKE, FAKE, 5000, FAKE, FAKE,
                                        1 << 30, None) == L.EGS_EINVAL
    aws = L.LIB.egs_sparse_decode_attn_workspace(ctypes.byref(sc), 772)
    if aws > 0:
        assert L.LIB.egs_sparse_decode_attn(ctypes.byref(sc), FAKE, FAKE, FAKE, 772, FAKE, FAKE,
                                            aws - 1, None) == L.EGS_EWORKSPACE


def test_page_retain_capacity_and_errors(L):
    # L = 4096, page 16: 256 pages; sinks 0..3 -> page 0; recent 3840.. -> pages 240..255
    sc = _dshape(L)
    cap = lambda S, K, mode: L.LIB.egs_page_retain_capacity(ctypes.byref(sc), S, K, mode)
    assert cap(16, 32, L.EGS_PAGE_GROUP) == 1 + 16 + 32
    assert cap(16, 32, L.EGS_PAGE_LAYER_UNION) == 1 + 16 + 2 * 32       # 2 KV groups
    assert cap(16, 32, L.EGS_PAGE_HEAD_UNION) == 1 + 16 + 4 * 32        # 4 heads per group
    assert cap(16, 1000, L.EGS_PAGE_HEAD_UNION) == 256                  # every page
    assert cap(1, 0, L.EGS_PAGE_GROUP) == 4 + 256                       # token pages
    assert cap(0, 4, L.EGS_PAGE_GROUP) == -1
    assert cap(16, -1, L.EGS_PAGE_GROUP) == -1
    assert cap(16, 4, 7) == -1
    assert L.LIB.egs_page_retain_workspace(ctypes.byref(sc), 16, 32, L.EGS_PAGE_GROUP) > 0
    ws = L.LIB.egs_page_retain_workspace(ctypes.byref(sc), 16, 32, L.EGS_PAGE_GROUP)
    call = lambda S=16, K=32, mode=0, ts=FAKE, wsb=ws: L.LIB.egs_page_retain(
        ctypes.byref(sc), S, K, mode, ts, FAKE, FAKE, FAKE, wsb, None)
    assert call(S=0) == L.EGS_EINVAL
    assert call(mode=3) == L.EGS_EINVAL
    assert call(ts=None) == L.EGS_EINVAL
    assert call(wsb=ws - 1) == L.EGS_EWORKSPACE
    big = _dshape(L, cache_len=1 << 20, n_obs=64)
    assert L.LIB.egs_page_retain(ctypes.byref(big), 2, 4, 0, FAKE, FAKE, FAKE, FAKE, 1 << 40,
                                 None) == L.EGS_ENOTSUP                 # 2^19 pages


def test_latent_step_errors(L):
    # capacity 300, W = 64: every case below is rejected before any launch
    sc = _dshape(L, cache_len=300, n_sink=4, n_recent=16, n_keep=32)
    prm = L.RetainParamsC(0, 2.0, 0.5, 1.0, 0, 1.0)
    ws = L.LIB.egs_latent_decode_workspace(ctypes.byref(sc))
    assert ws > 0

    def call(wsb=ws, **kw):
        base = dict(length=100, generated=0, n_delay=5, interval=0, compressed=0)
        base.update(kw)
        st = L.LatentStateC(**base)
        return L.LIB.egs_latent_decode_step(ctypes.byref(sc), ctypes.byref(prm), ctypes.byref(st),
                                            FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE,
                                            wsb, None)

    assert call(length=300) == L.EGS_EINVAL          # no room for the new entry
    assert call(length=63) == L.EGS_EINVAL           # fewer entries than observers
    assert call(interval=10) == L.EGS_EINVAL         # re-compression inside one window
    assert call(n_delay=-1) == L.EGS_EINVAL
    assert call(generated=-2) == L.EGS_EINVAL
    assert call(wsb=ws - 1) == L.EGS_EWORKSPACE
    assert L.LIB.egs_latent_decode_step(ctypes.byref(sc), ctypes.byref(prm), None, FAKE, FAKE,
                                        FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, ws,
                                        None) == L.EGS_EINVAL


def test_chunk_prune_errors(L):
    import numpy as np
    sc = _dshape(L, batch=1, cache_len=4096, n_obs=64)
    P = lambda **kw: L.PruneParamsC(**{**dict(eps_s=0.1, lam=0.5, eps=0.05, m0=0, target=100,
                                              zeta=0.5, tau=1.0), **kw})
    ws = L.LIB.egs_chunk_prune_workspace(ctypes.byref(sc), 3)
    assert ws > 0

    def call(bounds=FAKE, nk=3, prm=None, wsb=ws, shape=sc):
        # chunk_bounds is device memory (never read on the host)
        return L.LIB.egs_chunk_prune(ctypes.byref(shape), ctypes.byref(prm or P()), FAKE, FAKE,
                                     bounds, nk, FAKE, FAKE, FAKE, None, FAKE, wsb, None)

    assert call(bounds=None) == L.EGS_EINVAL
    assert call(bounds=ctypes.c_void_p((1 << 20) + 2)) == L.EGS_EINVAL       # misaligned
    assert call(nk=0) == L.EGS_EINVAL
    assert call(prm=P(eps_s=0.0)) == L.EGS_EINVAL
    assert call(prm=P(lam=-1.0)) == L.EGS_EINVAL
    assert call(prm=P(target=-1)) == L.EGS_EINVAL
    assert call(wsb=ws - 1) == L.EGS_EWORKSPACE
    assert call(shape=_dshape(L, batch=2, cache_len=4096, n_obs=64)) == L.EGS_EINVAL
    big = _dshape(L, batch=1, n_q_heads=128, n_kv_heads=8, cache_len=4096, n_obs=128)
    assert call(shape=big) == L.EGS_ENOTSUP                                  # 16384 rows


def test_prune_certificate_errors(L):
    import numpy as np
    ws = L.LIB.egs_prune_certificate_workspace(2)
    assert ws > 0 and L.LIB.egs_prune_certificate_workspace(0) == 0

    def call(bounds=FAKE, nk=2, R=512, eps=0.1, m0=0, t=1.0, wsb=ws, mass=FAKE):
        return L.LIB.egs_prune_certificate(bounds, nk, R, mass, FAKE, eps, m0, t, FAKE, FAKE,
                                           wsb, None)

    assert call(bounds=None) == L.EGS_EINVAL
    assert call(nk=0) == L.EGS_EINVAL
    assert call(R=0) == L.EGS_EINVAL
    assert call(R=8193) == L.EGS_EINVAL
    assert call(eps=-0.5) == L.EGS_EINVAL
    assert call(t=-1.0) == L.EGS_EINVAL
    assert call(t=float("nan")) == L.EGS_EINVAL
    assert call(m0=-1) == L.EGS_EINVAL
    assert call(mass=None) == L.EGS_EINVAL
    assert call(wsb=ws - 1) == L.EGS_EWORKSPACE


@pytest.mark.parametrize("B,Hq,Hkv,cap", [(8, 32, 8, 8192), (1, 4, 1, 131136), (2, 8, 2, 2218)])
def test_latent_workspace_holds_every_length(L, B, Hq, Hkv, cap):
    # A latent step runs decode attention over n = length + 1 <= capacity
    # entries with the split the launcher picks for n, which is not monotone in
    # n.  The step's workspace must hold the partials of every such n on top of
    # the retention scratch and the kept rows (regions are laid out back to back).
    sc = _dshape(L, batch=B, n_q_heads=Hq, n_kv_heads=Hkv, cache_len=cap, n_obs=64, n_sink=4,
                 n_recent=256, n_keep=4096)
    total = L.LIB.egs_latent_decode_workspace(ctypes.byref(sc))
    assert total > 0
    ntot = min(cap, 4 + 256 + 4096)
    rest = (L.LIB.egs_kv_retain_workspace(ctypes.byref(sc))
            + B * Hkv * ntot * (4 + 2 * 2 * sc.head_dim))
    worst = max(L.LIB.egs_sparse_decode_attn_workspace(ctypes.byref(sc), n)
                for n in range(64, cap + 1))
    assert worst + rest <= total


def test_entropy_score_static_rejects_large_shapes(L):
    # the static scratch holds EGS_STATIC_SCRATCH_BYTES; a 262144-token layer
    # with 32 / 8 heads needs more and is refused before any launch
    big = _shape(L, n_q_heads=32, n_kv_heads=8, head_dim=128, seq_len=262144, block_size=128,
                 segment_size=8192)
    assert L.LIB.egs_entropy_score_workspace(ctypes.byref(big)) > L.EGS_STATIC_SCRATCH_BYTES
    assert L.LIB.egs_entropy_score_static(ctypes.byref(big), 0, 0, 2.0, FAKE, FAKE, FAKE, FAKE,
                                          None) == L.EGS_EWORKSPACE
    ok = _shape(L, n_q_heads=32, n_kv_heads=8, head_dim=128, seq_len=131072, block_size=128,
                segment_size=8192)
    assert L.LIB.egs_entropy_score_workspace(ctypes.byref(ok)) <= L.EGS_STATIC_SCRATCH_BYTES
    # the same argument checks as egs_entropy_score
    sc = _shape(L)
    assert L.LIB.egs_entropy_score_static(ctypes.byref(sc), 7, 0, 2.0, FAKE, FAKE, FAKE, FAKE,
                                          None) == L.EGS_EINVAL
    assert L.LIB.egs_entropy_score_static(ctypes.byref(sc), 0, 1, -1.0, FAKE, FAKE, FAKE, FAKE,
                                          None) == L.EGS_EINVAL
    assert L.LIB.egs_entropy_score_static(ctypes.byref(sc), 0, 0, 2.0, None, FAKE, FAKE, FAKE,
                                          None) == L.EGS_EINVAL


def test_score_select_errors(L):
    sc = _shape(L)
    ws = L.LIB.egs_entropy_score_workspace(ctypes.byref(sc))
    good = L.BudgetPolicyC(mode=L.EGS_BUDGET_FIXED, frac=0.25, entropy_threshold=0.5)

    def call(pol=good, k_max=8, wsb=ws, pool=0, kind=0, q=FAKE, rig=FAKE):
        return L.LIB.egs_score_select(ctypes.byref(sc), pool, kind, 2.0,
                                      None if pol is None else ctypes.byref(pol), q, FAKE, k_max,
                                      FAKE, FAKE, rig, FAKE, FAKE, FAKE, FAKE, wsb, None)

    assert call(pol=None) == L.EGS_EINVAL
    assert call(pol=L.BudgetPolicyC(mode=9, entropy_threshold=0.5)) == L.EGS_EINVAL
    assert call(pol=L.BudgetPolicyC(mode=L.EGS_BUDGET_FIXED, frac=-1.0)) == L.EGS_EINVAL
    assert call(k_max=0) == L.EGS_EINVAL
    assert call(k_max=33) == L.EGS_EINVAL            # C_B = 32
    assert call(wsb=ws - 1) == L.EGS_EWORKSPACE
    assert call(pool=5) == L.EGS_EINVAL
    assert call(q=None) == L.EGS_EINVAL
    assert call(rig=None) == L.EGS_EINVAL
    assert "rigid" in L.LIB.egs_last_error().decode()


def test_binding_checks_host_chunk_bounds():
    # host bounds are checked by the Python binding before anything reaches
    # the device (the library itself checks device bounds on the device)
    import numpy as np
    import torch
    from entropy_guided_sparse_amd import api
    from entropy_guided_sparse_amd._lib import EgsError
    dev = torch.device("cpu")   # never reached: every case fails the check
    for bad, limit in (([[10, 100], [90, 200]], 4032), ([[10, 100], [100, 4040]], 4032),
                       ([[50, 50]], 4032), ([[10, 10]], None)):
        with pytest.raises(EgsError):
            api.chunk_bounds_device(np.array(bad), dev, limit=limit)
