"""Step-level parity on the GPU: each kernel of the gen block against the oracle's
definition of that step, on seeded inputs with ragged tails (M, N, L not multiples of
the tile sizes)."""
import numpy as np
import pytest

import oracle as O
import workloads as W
from gpu_helpers import BLOCK_TOL, BLOCK_TOL_F32, bf16_faithful, dev, host, log, rel_max_err

pytestmark = pytest.mark.gpu

RNG_SEED = 7


def rnd(tag, shape, std=1.0, dtype="bf16", mean=0.0):
    return W.maybe_bf16(W.normal(99, RNG_SEED, tag, shape, std, mean), dtype)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("rows,D", [(1, 64), (37, 256), (300, 4096)])
def test_rmsnorm(lib, dtype, rows, D):
    log(f"rmsnorm {dtype} rows={rows} D={D}")
    x = rnd(f"x{rows}{D}", (rows, D), 1.0, dtype)
    g = rnd(f"g{D}", (D,), 0.1, dtype, 1.0)
    y = dev(np.zeros_like(x), dtype)
    lib.op_rmsnorm(dev(x, dtype), dev(g, dtype), y, 1e-6)
    ref = O.rms_norm(x, g, 1e-6)
    err = rel_max_err(host(y), ref)
    log(f"  err={err:.3e}")
    assert err <= (BLOCK_TOL if dtype == "bf16" else BLOCK_TOL_F32)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("M,N,K", [(64, 64, 64), (300, 200, 128), (513, 520, 256), (1024, 768, 1024),
                                   (297, 1536, 512), (297, 704, 512), (297, 512, 704), (297, 512, 1024)])
@pytest.mark.parametrize("epi", [0, 1, 2])
def test_linear(lib, dtype, M, N, K, epi):
    import torch
    log(f"linear {dtype} M={M} N={N} K={K} epi={epi}")
    x = rnd(f"lx{M}{K}", (M, K), 1.0, dtype)
    wn = 2 * N if epi == 2 else N
    w = rnd(f"lw{wn}{K}", (wn, K), 0.05, dtype)
    r = rnd(f"lr{M}{N}", (M, N), 1.0, dtype)
    y = dev(np.zeros((M, N), np.float32), dtype)
    rd = dev(r, dtype)
    lib.op_linear(dev(x, dtype), dev(w, dtype), y, rd if epi == 1 else None, epi)
    torch.cuda.synchronize()
    if epi == 0:
        ref = O.linear(x, w)
    elif epi == 1:
        ref = r + O.linear(x, w)
    else:
        ref = O.swiglu(O.linear(x, w[:N]), O.linear(x, w[N:]))
    if dtype == "bf16":
        # exact fp32 accumulation + one rounding to bf16: within the bf16 rounding bound
        f = bf16_faithful(host(y), ref)
        log(f"  bf16-rounding units={f:.3f}  err/RMS={rel_max_err(host(y), ref):.3e}")
        assert f <= 1.0
    else:
        err = rel_max_err(host(y), ref)
        log(f"  err={err:.3e}")
        assert err <= BLOCK_TOL_F32


@pytest.mark.parametrize("M,N,K", [(2000, 8104, 1024), (2000, 8104, 512), (2000, 9000, 256), (600, 4000, 64)])
def test_linear_swiglu_many_tiles(lib, M, N, K):
    """SwiGLU launches with more 256 x 128 output tiles than the chip has CUs (512, and 568: an
    uneven number per CU), so one workgroup runs several tiles and a tile's outputs are stored
    while the next tile's first k-tiles load; with K = 512 and 256 the k range is too short to
    carry all of them, with K = 64 a single k-tile carries none.  Ragged last rows (2000 = 7 x 256
    + 208) and columns (8104 = 63 x 128 + 40).  Sampled rows, among them every tile's first and
    last, against the oracle at the bf16 rounding bound."""
    import torch
    log(f"linear swiglu M={M} N={N} K={K}")
    x = rnd(f"sx{M}{K}", (M, K), 1.0)
    w = rnd(f"sw{N}{K}", (2 * N, K), 0.05)
    y = dev(np.full((M, N), np.nan, np.float32), "bf16")
    lib.op_linear(dev(x, "bf16"), dev(w, "bf16"), y, None, 2)
    torch.cuda.synchronize()
    got = host(y)
    assert np.isfinite(got).all()                      # every output written
    rows = sorted(set([r for t in range(0, M, 256) for r in (t, min(t + 255, M - 1))] +
                      list(np.random.default_rng(M + N + K).integers(0, M, 24))))
    ref = O.swiglu(O.linear(x[rows], w[:N]), O.linear(x[rows], w[N:]))
    f = bf16_faithful(got[rows], ref)
    log(f"  {len(rows)} rows: bf16-rounding units={f:.3f}")
    assert f <= 1.0


def test_linear_resid_in_place(lib):
    import torch
    M, N, K = 260, 256, 192
    x = rnd("ipx", (M, K))
    w = rnd("ipw", (N, K), 0.05)
    h = rnd("iph", (M, N))
    hd = dev(h, "bf16")
    lib.op_linear(dev(x, "bf16"), dev(w, "bf16"), hd, hd, 1)
    torch.cuda.synchronize()
    assert rel_max_err(host(hd), h + O.linear(x, w)) <= BLOCK_TOL


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d,Hq,Hkv,N,plen", [(128, 8, 2, 50, [7, 400]), (64, 4, 2, 50, [7, 400]),
                                              (128, 8, 2, 99, [0, 45, 130])])
def test_qknorm_rope(lib, dtype, d, Hq, Hkv, N, plen):
    import torch
    B = len(plen)
    log(f"qknorm_rope {dtype} d={d}")
    qkvw = (Hq + 2 * Hkv) * d
    x = rnd(f"qk{d}{N}{B}", (B * N, qkvw), 1.3, dtype)
    gq = rnd(f"gq{d}", (d,), 0.1, dtype, 1.0)
    gk = rnd(f"gk{d}", (d,), 0.1, dtype, 1.0)
    t = dev(x, dtype)
    ws = torch.empty(lib.op_workspace_size(B, N, Hkv, d, max(plen), lib.GEN_BF16 if dtype == "bf16" else lib.GEN_F32),
                     dtype=torch.uint8, device="cuda")
    lib.op_qknorm_rope(t, B, N, Hq, Hkv, d, plen, dev(gq, dtype), dev(gk, dtype), 1e-6, 1e6, ws)
    got = host(t).reshape(B, N, Hq + 2 * Hkv, d)
    xr = x.reshape(B, N, Hq + 2 * Hkv, d)
    for b in range(B):
        c, s = O.rope_cos_sin(plen[b] + np.arange(N), d, 1e6, np.float32)
        q = O.apply_rope(O.rms_norm(xr[b, :, :Hq], gq, 1e-6), c, s)
        k = O.apply_rope(O.rms_norm(xr[b, :, Hq:Hq + Hkv], gk, 1e-6), c, s)
        tol = BLOCK_TOL if dtype == "bf16" else BLOCK_TOL_F32
        assert rel_max_err(got[b, :, :Hq], q) <= tol
        assert rel_max_err(got[b, :, Hq:Hq + Hkv], k) <= tol
        np.testing.assert_array_equal(got[b, :, Hq + Hkv:], xr[b, :, Hq + Hkv:])   # v untouched


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d,Hq,Hkv,N,plen", [(128, 8, 2, 200, [37, 0]), (64, 4, 2, 64, [32, 32]),
                                              (128, 4, 4, 130, [400, 5]), (128, 8, 1, 1, [3, 64]),
                                              (128, 8, 2, 99, [0, 45, 130]), (128, 6, 2, 70, [10, 0]),
                                              (64, 16, 2, 150, [64, 3])])
def test_attention(lib, dtype, d, Hq, Hkv, N, plen):
    import torch
    B = len(plen)
    log(f"attention {dtype} d={d} Hq={Hq} Hkv={Hkv} N={N} plen={plen}")
    qkvw = (Hq + 2 * Hkv) * d
    x = rnd(f"at{d}{N}{Hq}{Hkv}{B}", (B * N, qkvw), 1.0, dtype)
    pk = [rnd(f"apk{b}{d}{plen[b]}", (plen[b], Hkv, d), 1.0, dtype) for b in range(B)]
    pv = [rnd(f"apv{b}{d}{plen[b]}", (plen[b], Hkv, d), 1.0, dtype) for b in range(B)]
    out = torch.zeros(B * N, Hq * d, device="cuda", dtype=torch.bfloat16 if dtype == "bf16" else torch.float32)
    gdt = lib.GEN_BF16 if dtype == "bf16" else lib.GEN_F32
    ws = torch.empty(lib.op_workspace_size(B, N, Hkv, d, max(plen), gdt), dtype=torch.uint8, device="cuda")
    pkd = [dev(p, dtype) if p.size else None for p in pk]
    pvd = [dev(p, dtype) if p.size else None for p in pv]
    lib.op_attention(dev(x, dtype), B, N, Hq, Hkv, d, pkd, pvd, plen, out, ws)
    got = host(out).reshape(B, N, Hq, d)
    xr = x.reshape(B, N, Hq + 2 * Hkv, d)
    for b in range(B):
        K = np.concatenate([pk[b], xr[b, :, Hq:Hq + Hkv]])
        V = np.concatenate([pv[b], xr[b, :, Hq + Hkv:]])
        ref = O.attention(xr[b, :, :Hq], K, V)
        err = rel_max_err(got[b], ref)
        if dtype == "bf16":
            # Rounding P to bf16 ahead of the P.V product perturbs each weight by at most 2^-9 of
            # itself, so an output element moves by at most 2^-9 sum_j a_j |v_j| (the same attention
            # applied to |V|); the output itself is rounded once (2^-8 |ref|).  Slack 1e-3 RMS covers
            # fp32 summation order.
            pv_bound = O.attention(xr[b, :, :Hq], K, np.abs(V))
            bound = (2.0 ** -8 * np.abs(ref) + 2.0 ** -9 * pv_bound
                     + 1e-3 * np.sqrt(np.mean(ref.astype(np.float64) ** 2)))
            worst = float(np.max(np.abs(got[b] - ref) / bound))
            log(f"  b={b} err={err:.3e} worst/bound={worst:.3f}")
            assert worst <= 1.0
        else:
            log(f"  b={b} err={err:.3e}")
            assert err <= BLOCK_TOL_F32


def test_flow_euler_cfg(lib):
    import torch
    n = 3 * 64 * 64 + 3   # ragged tail past the float4 vector width
    x, c, u = (W.normal(98, 0, t, (n,)) for t in ("x", "c", "u"))
    for scale, s, sn in [(4.0, 1.0, 0.75), (1.0, 0.75, 0.0), (2.5, 0.01, 0.0)]:
        xd = torch.from_numpy(x).cuda()
        lib.flow_euler_cfg(xd, torch.from_numpy(c).cuda(), torch.from_numpy(u).cuda(), scale, s, sn, 0.02)
        ref = O.euler_step(x, O.cfg_mix(c, u, scale), s, sn, 0.02)
        np.testing.assert_allclose(host(xd), ref, rtol=1e-5, atol=1e-5)
    xd = torch.from_numpy(x).cuda()
    lib.flow_euler_cfg(xd, torch.from_numpy(c).cuda(), None, 1.0, 0.5, 0.25, 0.02)
    np.testing.assert_allclose(host(xd), O.euler_step(x, c, 0.5, 0.25, 0.02), rtol=1e-5, atol=1e-5)


def test_flow_euler_dual_cfg(lib):
    import torch
    n = 3 * 64 * 64 + 3
    x, c, i, u = (W.normal(98, 1, t, (n,)) for t in ("x", "c", "i", "u"))
    for s_txt, s_img, sg, sn in [(4.0, 2.0, 1.0, 0.75), (4.0, 1.0, 0.5, 0.25), (1.0, 1.0, 0.3, 0.0),
                                 (1.0, 3.0, 0.01, 0.0), (7.5, 1.5, 0.9, 0.8)]:
        xd = torch.from_numpy(x).cuda()
        lib.flow_euler_dual_cfg(xd, torch.from_numpy(c).cuda(), torch.from_numpy(i).cuda(),
                                torch.from_numpy(u).cuda(), s_txt, s_img, sg, sn, 0.02)
        ref = O.euler_step(x, O.dual_cfg_mix(c, i, u, s_txt, s_img), sg, sn, 0.02)
        np.testing.assert_allclose(host(xd), ref, rtol=1e-5, atol=1e-5)
    xd = torch.from_numpy(x).cuda()        # image guidance off: no uncond branch needed
    lib.flow_euler_dual_cfg(xd, torch.from_numpy(c).cuda(), torch.from_numpy(i).cuda(), None, 4.0, 1.0, 0.5, 0.25,
                            0.02)
    np.testing.assert_allclose(host(xd), O.euler_step(x, O.dual_cfg_mix(c, i, None, 4.0, 1.0), 0.5, 0.25, 0.02),
                               rtol=1e-5, atol=1e-5)


# experts up to 32 run one instance of the router, 33-64 another (four 16-expert blocks); D = 64
# gives each of the router's four waves a single 16-column group
@pytest.mark.parametrize("T,D,E,k,dt", [(300, 256, 32, 8, "bf16"), (4096, 2048, 32, 8, "bf16"), (17, 128, 6, 2, "bf16"),
                                        (300, 256, 64, 8, "bf16"), (33, 64, 40, 4, "bf16"),
                                        (300, 512, 48, 6, "f32"), (4096, 2048, 32, 8, "f32")])
def test_moe_route_exact_sets(lib, T, D, E, k, dt):
    import torch
    log(f"route T={T} D={D} E={E} k={k} {dt}")
    u = rnd(f"ru{T}{D}", (T, D), dtype=dt)
    wr = rnd(f"rw{E}{D}", (E, D), 1.0 / np.sqrt(D), dtype=dt)
    idx = torch.empty(T, k, dtype=torch.int32, device="cuda")
    wt = torch.empty(T, k, dtype=torch.float32, device="cuda")
    lib.moe_route(dev(u, dt), dev(wr, dt), k, idx, wt, lib.GEN_BF16 if dt == "bf16" else lib.GEN_F32)
    gi, gw = idx.cpu().numpy(), wt.cpu().numpy()
    ridx, rw, p = O.route_topk(u.astype(np.float64), wr.astype(np.float64), k)
    srt = np.sort(p, axis=1)[:, ::-1]
    gap = srt[:, k - 1] - srt[:, k] if k < E else np.full(T, np.inf)
    near = gap < 1e-6
    same = np.array([set(gi[t]) == set(ridx[t]) for t in range(T)])
    log(f"  mismatched={int((~same).sum())} near-ties={int(near.sum())}")
    assert np.all(same | near)
    np.testing.assert_allclose(gw.sum(1), 1.0, atol=1e-6)
    ok = same & ~near
    np.testing.assert_allclose(np.sort(gw[ok], 1), np.sort(rw[ok], 1), rtol=1e-4, atol=1e-6)
