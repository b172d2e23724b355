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
    o = oracle.forward(inp, tokens=tokens, act4=act4)
    flagged = np.nonzero(o["flagged"])[0]
    adopt = {}
    for t in flagged:
        if not np.array_equal(o["idx"][t], gpu_idx[t]):
            srt = np.sort(o["logits"][t])[::-1]
            kth = srt[inp.k - 1]
            if np.all(o["logits"][t, gpu_idx[t]] >= kth - oracle.NEAR_TIE):
                adopt[int(t)] = gpu_idx[t]
    if adopt:
        o = oracle.forward(inp, tokens=tokens, override_idx=adopt, act4=act4)
    o["n_flagged"], o["n_adopted"] = int(len(flagged)), len(adopt)
    return o


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
    # x split: hi + lo within 2^-8 of the block maximum (past 65536 tokens on every 97th row and
    # the evaluated tokens, to bound the host memory of the check)
    rows = np.arange(T) if T <= 65536 else np.unique(np.concatenate([np.arange(0, T, 97), o["tokens"]]))
    rbx = actpack.row_bytes(D)
    xrows = np.asarray(g["x_packed"]).reshape(-1)[: T * rbx].reshape(T, rbx)[rows]
    xs = actpack.decode_sum(xrows, D, len(rows))
    x = oracle.bf16_to_f64(inp.x_bf16[rows])
    bmax = np.repeat(np.abs(x).reshape(len(rows), -1, 32).max(-1), 32, axis=1)
    assert np.all(np.abs(xs - x) <= bmax * 2.0 ** -8)
    stats["x_split_max_rel"] = float((np.abs(xs - x) / np.maximum(bmax, 1e-30)).max())
    tokens = o["tokens"]
    pos = sorted(o["z"].keys())
    rms_y = float(np.sqrt(np.mean(o["y"] ** 2)))
    stats["rms_y"] = rms_y
    if check_h and pos:
        rb = actpack.row_bytes(I)
        hrows = np.asarray(g["h_packed"]).reshape(-1)[: T * k * rb].reshape(T * k, rb)[pos]
        hs = actpack.decode_sum(hrows, I, len(pos))
        ho = np.array([o["h"][p] for p in pos])
        dh = np.abs(hs - ho).max() / max(np.abs(ho).max(), 1e-30)
        stats["h_max_err_rel_max"] = float(dh)
        assert dh <= 2e-2, dh
    if pos:
        a = o["perm"][pos]
        q = np.array([o["w"][ai // k, ai % k] * o["z"][p] for p, ai in zip(pos, a)])
        dq = np.abs(g["y_perm"][pos].astype(np.float64) - q).max() / rms_y
        stats["y_perm_err_over_rms"] = float(dq)
        assert dq <= TOL_Y, dq
    dy = np.abs(g["y32"][tokens].astype(np.float64) - o["y"])
    stats["y_max_err_over_rms"] = float(dy.max() / rms_y)
    stats["y_rms_err_over_rms"] = float(np.sqrt(np.mean(dy ** 2)) / rms_y)
    assert dy.max() <= TOL_Y * rms_y, stats
    assert np.array_equal(g["y16"], rne_bf16_bits(g["y32"]))
    return stats
