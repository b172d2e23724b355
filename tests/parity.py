"""GPU-vs-oracle comparison helpers for the parity tests (GPU runs only)."""
from __future__ import annotations

import numpy as np

import oracle
from tests import actpack

TOL_Y = 2e-2          # max |y_gpu - y| <= TOL_Y * RMS(y)  (bf16 activations, fp32 accumulation)
TOL_W = 1e-6          # gate weights
TOL_LOGIT = (1e-7, 2.0 ** -21)   # fp32 logits: 1e-7 + 8 eps32 (|l| + ||x_t|| ||w_e||)


def run_gpu(layer, stream=None) -> dict:
    """Run the C entry points one by one and copy every intermediate to the host."""
    import torch
    layer.steps(bf16=False, stream=stream)
    layer.combine(bf16=True, stream=stream)
    torch.cuda.synchronize()
    T, k = layer.T, layer.k
    r = dict(idx=layer.topk_idx.cpu().numpy(), w=layer.topk_w.cpu().numpy(), logits=layer.logits.cpu().numpy(),
             counts=layer.counts.cpu().numpy(), offsets=layer.offsets.cpu().numpy(),
             perm=layer.perm.cpu().numpy(), inv=layer.inv.cpu().numpy(), tiles=layer.tiles.cpu().numpy(),
             x_packed=layer.x_packed.cpu().numpy(), h_packed=layer.h_packed.cpu().numpy(),
             y_perm=layer.y_perm.cpu().numpy(), y32=layer.y32.cpu().numpy(),
             y16=layer.y16.view(torch.int16).cpu().numpy().view(np.uint16))
    assert r["idx"].shape == (T, k)
    return r


def check_tiles(tiles: np.ndarray, offsets: np.ndarray, perm: np.ndarray, n: int, E: int):
    """The row-tile table (include/moe_mxfp4.h): every expert's grouped rows cut into tiles of
    8 rows (n <= 6E, 48 ints per slot) or 128 rows (132 ints per slot), in expert order; each slot
    holds {expert, first position, rows, tiles in use} and the assignment id of every row; then
    empty slots (expert -1)."""
    bm = 8 if n <= 6 * E else 128
    ints = max(48, 4 + bm)
    slots = -(-n // bm) + min(E, n)
    t = tiles[: slots * ints].reshape(slots, ints)
    s = 0
    for e in range(E):
        for p0 in range(int(offsets[e]), int(offsets[e + 1]), bm):
            rows = min(bm, int(offsets[e + 1]) - p0)
            assert list(t[s, :3]) == [e, p0, rows], (s, t[s, :4], e, p0, rows)
            assert np.array_equal(t[s, 4:4 + rows], perm[p0:p0 + rows])
            s += 1
    assert np.all(t[:, 3] == s), "every slot records the number of tiles in use"
    assert np.all(t[s:, 0] == -1)


def rne_bf16_bits(y32: np.ndarray) -> np.ndarray:
    u = y32.astype(np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def oracle_with_adoption(inp, gpu_idx: np.ndarray, tokens=None, act4: bool = False):
    """Oracle run; for near-tie tokens whose GPU selection differs, adopt the GPU's set when every
    expert it picked scores within 1e-6 of the oracle's k-th largest logit."""
    o = oracle.forward(inp, tokens=tokens, act4=act4, preact=not act4)
    flagged = np.nonzero(o["flagged"])[0]
    adopt = {}
    for t in flagged:
        if not np.array_equal(o["idx"][t], gpu_idx[t]):
            srt = np.sort(o["logits"][t])[::-1]
            kth = srt[inp.k - 1]
            if np.all(o["logits"][t, gpu_idx[t]] >= kth - oracle.NEAR_TIE):
                adopt[int(t)] = gpu_idx[t]
    if adopt:
        o = oracle.forward(inp, tokens=tokens, override_idx=adopt, act4=act4, preact=not act4)
    o["n_flagged"], o["n_adopted"] = int(len(flagged)), len(adopt)
    return o


# ---- derived per-element bars of the intermediates -----------------------------------------
# The packed activations the expert GEMMs read are hi + lo MX6 encodings of bf16 rows; the x and h
# checks bound that encoding's error by 2^-8 of the 32-value block maximum (SPLIT_REL).  The bars
# of h and y_perm charge each GEMM stage for (1) the measured encoding error of the operand it was
# given, propagated through the stage's weights under a random-sign model (Hoeffding: a sum of
# independent terms X_d with |X_d| <= c_d exceeds LAMBDA * sqrt(sum c_d^2) with probability at most
# 2 exp(-LAMBDA^2 / 2) = 4.6e-11), (2) its fp32 accumulation, at most gamma(K) * sum |a_d w_d| with
# gamma(K) = 2^-24 (K/32 + 64) (a rounding per 32-value block step plus 64 inside one instruction),
# and (3) its output rounding: bf16 (one ulp, as the oracle rounds too) and the 2^-8 split for h;
# fp16 (2^-11 relative) for y_perm.  The oracle's values are the expected values throughout.
SPLIT_REL = 2.0 ** -8
LAMBDA = 7.0
SILU_LIP = 1.1          # max |d silu / dg| on [-7, 7] is 1.0998


def gamma_acc(K: int) -> float:
    return 2.0 ** -24 * (K / 32 + 64)


def ulp_bf16(v: np.ndarray) -> np.ndarray:
    """Spacing of bf16 values at |v| (8 significant bits); normal range, 2^-133 below it."""
    a = np.maximum(np.abs(v), 2.0 ** -126)
    return np.ldexp(1.0, np.frexp(a)[1] - 8)


def _block_max(v: np.ndarray) -> np.ndarray:
    """max |v| over each 32-value block of the last axis, repeated over the block."""
    sh = v.shape
    m = np.abs(v).reshape(*sh[:-1], sh[-1] // 32, 32).max(-1)
    return np.repeat(m, 32, axis=-1)


def _silu(v):
    return v / (1.0 + np.exp(-v))


_E2M1_F32 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0, -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0],
                     np.float32)
_BYTE_PAIR = np.stack([_E2M1_F32[np.arange(256) & 15], _E2M1_F32[np.arange(256) >> 4]], axis=-1)   # [256][2]


def weights_f32(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """MXFP4 rows [R][K/2] codes, [R][K/32] scales -> float32 [R][K] (exact for scale bytes 2..251,
    which hold every scale of the workloads), by a byte lookup: a faster stand-in for the oracle's decoder in
    the tolerance arithmetic only (tests/test_parity_cpu.py checks the two agree)."""
    R, half = codes.shape
    v = _BYTE_PAIR[codes].reshape(R, half * 2 // 32, 32)
    return (v * np.ldexp(np.float32(1.0), scales.astype(np.int32) - 127)[..., None]).reshape(R, half * 2)


def h_bar(inp, o, pos, t, dx, xs_rows, w_gu) -> np.ndarray:
    """Per-element bar of the GPU's (decoded) h against the oracle's h at positions pos."""
    I, L = inp.I, inp.swiglu_limit
    w = w_gu.astype(np.float32)
    var = (dx.astype(np.float32) ** 2) @ (w * w).T                   # [n][2I]
    acc = np.abs(xs_rows).astype(np.float32) @ np.abs(w).T
    dlt = LAMBDA * np.sqrt(var.astype(np.float64)) * 1.01 + gamma_acc(inp.D) * acc.astype(np.float64) * 1.01
    dg, du = dlt[:, :I], dlt[:, I:]
    gc = np.clip(np.array([o["g"][p] for p in pos]), -L, L)
    uc = np.clip(np.array([o["u"][p] for p in pos]), -L, L)
    sg = _silu(gc)
    dpre = SILU_LIP * (np.abs(uc) + du) * dg + (np.abs(sg) + SILU_LIP * dg) * du + 2.0 ** -20 * (np.abs(sg * uc) + 2.0 ** -10)
    ho = np.array([o["h"][p] for p in pos])
    rnd = dpre + ulp_bf16(np.abs(ho) + dpre)
    return rnd + SPLIT_REL * (_block_max(ho) + _block_max(rnd))


def y_perm_bar(inp, o, pos, dh, hs_rows, w_dn) -> np.ndarray:
    """Per-element bar of the GPU's y_perm rows (fp16, gate applied) against w * z of the oracle."""
    k = inp.k
    w = w_dn.astype(np.float32)
    var = (dh.astype(np.float32) ** 2) @ (w * w).T                   # [n][D]
    acc = np.abs(hs_rows).astype(np.float32) @ np.abs(w).T
    dz = LAMBDA * np.sqrt(var.astype(np.float64)) * 1.01 + gamma_acc(inp.I) * acc.astype(np.float64) * 1.01
    a = o["perm"][pos]
    wo = o["w"][a // k, a % k][:, None]
    zo = np.array([o["z"][p] for p in pos])
    q = wo * zo
    return q, np.abs(wo) * dz + TOL_W * (np.abs(zo) + dz) + 2.0 ** -11 * (np.abs(q) + np.abs(wo) * dz) + 2.0 ** -25


def compare(inp, g: dict, o: dict, check_h: bool = True) -> dict:
    """Assert parity of every intermediate; returns the measured errors."""
    T, k, D, I = inp.T, inp.k, inp.D, inp.I
    stats = dict(n_flagged=o["n_flagged"], n_adopted=o["n_adopted"])
    # router logits (fp32 debug output)
    # fp32 summation error is a small multiple of eps32 * sum_d |x_d w_d| <= eps32 ||x_t|| ||w_e||
    dl = np.abs(g["logits"].astype(np.float64) - o["logits"])
    xn = np.sqrt((oracle.bf16_to_f64(inp.x_bf16) ** 2).sum(axis=1))
    wn = np.sqrt((inp.w_router.astype(np.float64) ** 2).sum(axis=1))
    tol = TOL_LOGIT[0] + TOL_LOGIT[1] * (np.abs(o["logits"]) + xn[:, None] * wn[None, :])
    stats["max_dlogit"] = float(dl.max())
    stats["max_dlogit_over_tol"] = float((dl / tol).max())
    assert np.all(dl <= tol), (dl / tol).max()
    # selection and permutation: bit-exact
    assert np.array_equal(g["idx"], o["idx"]), np.argwhere(g["idx"] != o["idx"])[:5]
    assert np.array_equal(g["counts"], o["counts"])
    assert np.array_equal(g["offsets"], o["offsets"])
    assert np.array_equal(g["perm"], o["perm"])
    assert np.array_equal(g["inv"], o["inv"])
    check_tiles(g["tiles"], o["offsets"], o["perm"], T * k, inp.E)
    dw = np.abs(g["w"].astype(np.float64) - o["w"]).max()
    stats["max_dw"] = float(dw)
    assert dw <= TOL_W, dw
    assert np.allclose(g["w"].sum(axis=1), 1.0, atol=4 * 2 ** -24 * k)
    tokens = o["tokens"]
    # x split: hi + lo within 2^-8 of the block maximum, on every row the experts read (past
    # 65536 tokens on every 97th row and the evaluated tokens, to bound the host memory)
    rows = np.arange(T) if T <= 65536 else np.unique(np.concatenate([np.arange(0, T, 97), tokens]))
    rbx = actpack.row_bytes(D)
    xrows = np.asarray(g["x_packed"]).reshape(-1)[: T * rbx].reshape(T, rbx)[rows]
    xs = actpack.decode_sum(xrows, D, len(rows))
    x = oracle.bf16_to_f64(inp.x_bf16[rows])
    bmax = _block_max(x)
    assert np.all(np.abs(xs - x) <= bmax * SPLIT_REL)
    stats["x_split_max_rel"] = float((np.abs(xs - x) / np.maximum(bmax, 1e-30)).max())
    row_of = np.full(T, -1, np.int64)
    row_of[rows] = np.arange(len(rows))
    pos = np.array(sorted(o["z"].keys()), dtype=np.int64)
    rms_y = float(np.sqrt(np.mean(o["y"] ** 2)))
    stats["rms_y"] = rms_y
    if pos.size:
        rb = actpack.row_bytes(I)
        hbuf = np.asarray(g["h_packed"]).reshape(-1)[: T * k * rb].reshape(T * k, rb)
        worst_h = worst_yp = 0.0
        h_err_ulp = 0.0
        yp_err = 0.0
        n_h_ulp = 0
        for e in range(inp.E):
            pe = pos[(pos >= o["offsets"][e]) & (pos < o["offsets"][e + 1])]
            if pe.size == 0:
                continue
            t = o["perm"][pe] // k
            xr = row_of[t]
            assert np.all(xr >= 0)
            dx = xs[xr] - x[xr]
            hs = actpack.decode_sum(hbuf[pe], I, len(pe))
            ho = np.array([o["h"][p] for p in pe])
            if check_h:
                w_gu = weights_f32(inp.gu_codes[e], inp.gu_scales[e])
                tol_h = h_bar(inp, o, pe, t, dx, xs[xr], w_gu)
                del w_gu
                dh_abs = np.abs(hs - ho)
                worst_h = max(worst_h, float((dh_abs / tol_h).max()))
                h_err_ulp = max(h_err_ulp, float((dh_abs / ulp_bf16(ho)).max()))
                n_h_ulp += int((dh_abs > ulp_bf16(ho)).sum())
                assert np.all(dh_abs <= tol_h), (e, float((dh_abs / tol_h).max()))
            w_dn = weights_f32(inp.dn_codes[e], inp.dn_scales[e])
            q, tol_yp = y_perm_bar(inp, o, pe, hs - ho, hs, w_dn)
            del w_dn
            dyp = np.abs(g["y_perm"][pe].astype(np.float64) - q)
            worst_yp = max(worst_yp, float((dyp / tol_yp).max()))
            yp_err = max(yp_err, float(dyp.max()))
            assert np.all(dyp <= tol_yp), (e, float((dyp / tol_yp).max()))
        if check_h:
            stats["h_err_over_bar_max"] = worst_h
            stats["h_err_max_in_bf16_ulps"] = h_err_ulp
            stats["h_elements_beyond_1_ulp"] = n_h_ulp
        stats["y_perm_err_over_bar_max"] = worst_yp
        stats["y_perm_err_over_rms_y"] = yp_err / rms_y
    dy = np.abs(g["y32"][tokens].astype(np.float64) - o["y"])
    stats["y_max_err_over_rms"] = float(dy.max() / rms_y)
    stats["y_rms_err_over_rms"] = float(np.sqrt(np.mean(dy ** 2)) / rms_y)
    assert dy.max() <= TOL_Y * rms_y, stats
    assert np.array_equal(g["y16"], rne_bf16_bits(g["y32"]))
    return stats


def record_stats(case: str, stats: dict) -> None:
    """Append a case's error statistics as one JSON line to parity_stats.jsonl in the directory named
    by MOE_PARITY_STATS_DIR (nothing is written when it is unset)."""
    import json
    import os
    d = os.environ.get("MOE_PARITY_STATS_DIR")
    if not d:
        return
    try:
        os.makedirs(d, exist_ok=True)
        with open(os.path.join(d, "parity_stats.jsonl"), "a") as f:
            f.write(json.dumps(dict(case=case, **stats)) + "\n")
    except OSError:
        pass
