"""GPU parity on every matrix of the full-size workloads, every element, through the C ABI.

For each matrix of the Qwen3-4B layer set (36 x 7), the Qwen2.5-7B step
(28 x 7 and the 152064 x 3584 lm_head) and the 151936 x 2560 tied embedding:
  * nwc_dequant must return the input bit for bit (every element);
  * nwc_matvec must put every output within |y - y_ref| <= 1e-3 sum_j |w_ij x_j|
    + 1e-6 of the C oracle's float64 row sums (oracle/nwc_oracle.c).
For every layer, q, k, v and gate, up also run as grouped launches
(nwc_matvec_group: outputs bit-equal to the single calls and in tolerance) and
encoded as one concatenated matrix each (q||k||v, gate||up: dequantized bit for
bit, every output in tolerance against the oracle's sums with q's activation).
The matrices are the seeded host draws every consumer uses (synth); host work
(drawing, encoding, the oracle's sums) runs on a background thread a few
matrices ahead of the GPU.
"""
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

import synth as S
from oracle import fast as F
from synth import configs as C

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from decode_matvec_amd import nwc  # noqa: E402

from . import blob_layout as BL  # noqa: E402

DEV = "cuda"
RTOL, ATOL = 1e-3, 1e-6


def _host(m, cols=0, rows=0):
    """Host side of one matrix: draws, blob, activation and the oracle's sums."""
    w = S.blocked_normal_bf16(m["w_seed"], (m["n"], m["k"]), np.float32(m["sigma"]))
    blob = nwc.encode(w, cols_per_lane=cols, rows_per_wave=rows)
    x = S.activation_bf16(m["x_seed"], m["k"])
    y_ref, A = F.matvec_bf16(w, x)
    return m, w, blob, x, y_ref, A


def _prepared(mats, ahead=3, **kw):
    """(m, w, blob, x, y_ref, A) in order, prepared `ahead` matrices in advance."""
    with ThreadPoolExecutor(1) as ex:
        futs = [ex.submit(_host, m, **kw) for m in mats[:ahead]]
        for i in range(len(mats)):
            if i + ahead < len(mats):
                futs.append(ex.submit(_host, mats[i + ahead], **kw))
            yield futs[i].result()
            futs[i] = None


def _check_one(m, w, blob, x, y_ref, A):
    """Dequantize and multiply one matrix; returns (dequant equal, outputs out of
    tolerance, largest err / tolerance, the DeviceMatrix, its activation, its output)."""
    dm = nwc.DeviceMatrix(blob, DEV)
    wd = torch.from_numpy(w.view(np.int16)).to(DEV)
    out = torch.empty_like(wd)
    dm.dequant(out)
    xd = torch.from_numpy(x.view(np.int16)).to(DEV)
    y = torch.full((m["n"],), float("nan"), dtype=torch.float32, device=DEV)
    dm.matvec(xd, y)
    same = bool(torch.equal(out, wd))
    del out, wd
    bad, ratio = _tol(y, y_ref, A)
    return same, bad, ratio, dm, xd, y


def _tol(y, y_ref, A):
    err = np.abs(y.cpu().numpy().astype(np.float64) - y_ref)
    return int((~(err <= RTOL * A + ATOL)).sum()), float(np.max(err / (RTOL * A + ATOL)))


# Projections that read one input in a decoder layer: run as one launch
# (nwc_matvec_group, each matrix with its own activation here) and, as the
# pages' fuse() does, encoded as one concatenated matrix.
FUSED = (("qkv", ("q", "k", "v")), ("gate_up", ("gate", "up")))


def _check_layer(layer):
    """Group launches and fused (concatenated) encodings of one layer, element by element."""
    fails = []
    for fname, parts in FUSED:
        mem = [layer[p] for p in parts]
        ys = [torch.full((e["m"]["n"],), float("nan"), dtype=torch.float32, device=DEV) for e in mem]
        nwc.matvec_group([e["dm"] for e in mem], [e["x"] for e in mem], ys)
        for e, y in zip(mem, ys):
            bad, _ = _tol(y, e["y_ref"], e["A"])
            if bad or not torch.equal(y, e["y"]):
                fails.append((e["m"]["label"], "group", bad))
        w = np.concatenate([e["w"] for e in mem])
        dm = nwc.DeviceMatrix(nwc.encode(w), DEV)
        wd = torch.from_numpy(w.view(np.int16)).to(DEV)
        out = torch.empty_like(wd)
        dm.dequant(out)
        same = bool(torch.equal(out, wd))
        del out, wd
        y = torch.full((w.shape[0],), float("nan"), dtype=torch.float32, device=DEV)
        dm.matvec(mem[0]["x"], y)
        y_ref, A = F.matvec_bf16(w, mem[0]["xh"])
        bad, _ = _tol(y, y_ref, A)
        if bad or not same:
            fails.append((f"{mem[0]['m']['label']}:{fname}", "fused", same, bad))
    return fails


def _run(mats, what, **kw):
    t0 = time.time()
    fails = []
    worst = 0.0
    layer, n_layers = {}, 0
    for i, (m, w, blob, x, y_ref, A) in enumerate(_prepared(mats, **kw)):
        same, bad, ratio, dm, xd, y = _check_one(m, w, blob, x, y_ref, A)
        worst = max(worst, ratio)
        if not same or bad:
            fails.append((m["label"], same, bad))
        if m["name"] in ("q", "k", "v", "gate", "up"):
            layer[m["name"]] = dict(m=m, w=w, dm=dm, x=xd, xh=x, y=y, y_ref=y_ref, A=A)
        if m["name"] == "down":
            fails += _check_layer(layer)
            layer, n_layers = {}, n_layers + 1
        if i % 50 == 49:
            print(f"  {what}: {i + 1}/{len(mats)} matrices checked ({time.time() - t0:.0f}s)", flush=True)
    print(f"{what}: {len(mats)} matrices, every element dequantized bit-exact and every output in tolerance "
          f"(largest err / tolerance {worst:.2e}); {n_layers} layers of grouped q,k,v and gate,up launches and "
          f"fused q||k||v, gate||up encodings likewise; {time.time() - t0:.0f}s", flush=True)
    assert not fails, f"{len(fails)} failures: {fails[:5]}"


@pytest.mark.timeout(900)
def test_qwen3_4b_layer_set_every_matrix():
    mats = list(C.qwen3_matrices())
    assert len(mats) == 252
    _run(mats, "qwen3_4b layer set")


@pytest.mark.timeout(900)
def test_qwen25_7b_step_every_matrix():
    mats = list(C.qwen25_matrices())
    assert len(mats) == 197 and mats[-1]["name"] == "lm_head"
    _run(mats, "qwen25_7b step", ahead=2)


def test_tied_embedding_table_gather_lm_head():
    m = C.embedding_matrix()
    m, w, blob, x, y_ref, A = _host(m)
    same, bad, _, dm, _, _ = _check_one(m, w, blob, x, y_ref, A)
    assert same and bad == 0
    ids = S.token_ids(C.EMBED["ids_seed"], m["n"], C.N_IDS)
    ids[:3] = [0, m["n"] - 1, ids[5]]
    out = torch.full((len(ids), m["k"]), -1, dtype=torch.int16, device=DEV)
    dm.gather(torch.from_numpy(ids).to(DEV), out)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().view(np.uint16), w[ids])


@pytest.mark.timeout(600)
@pytest.mark.parametrize("cols", [48, 64])
def test_layer_shapes_through_the_lds_region_path(cols):
    # Items of 48 or 64 columns per lane take more code rows (5 to 8) than the
    # register window holds (4), so every item of these matrices is staged into
    # the wave's LDS region, with direct HBM->LDS loads for the rows past the
    # prefetch: the full-size shapes of both layer sets on that path, every
    # element of the dequantization and every matvec output.
    mats = [m for m in C.qwen3_matrices(1)] + [m for m in C.qwen25_matrices(1, lm_head=False)]
    fails = []
    for m, w, blob, x, y_ref, A in _prepared(mats, cols=cols):
        h = BL.header(blob)
        rows = np.frombuffer(blob[h["off_items"]:h["off_items"] + 8 * h["n_items"]].tobytes(), "<u4")[1::2]
        assert h["cols_per_lane"] == cols and rows.min() > 4
        same, bad, _, _, _, _ = _check_one(m, w, blob, x, y_ref, A)
        if not same or bad:
            fails.append((m["label"], same, bad))
    assert not fails, fails
