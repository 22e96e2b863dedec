"""GPU parity of each kernel, through the C ABI, against the oracle.

Inputs come from seeded generators (bf16 inputs are rounded to bf16 before
either side sees them); the oracle runs in float64.  Sizes span several
tiles and a ragged tail.
"""
import numpy as np
import pytest

from oracle import model as om
from orca_selective_iteration_amd import lib as L
from orca_selective_iteration_amd import synth
from tests.util import TOL, rel_err

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda"


def tdt(dtype):
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def odt(dtype):
    return L.ORCA_BF16 if dtype == "bf16" else L.ORCA_F32


def draw(rng, shape, scale, dtype, shift=0.0):
    a = (shift + scale * rng.standard_normal(shape)).astype(np.float32)
    return synth.round_to_bf16(a) if dtype == "bf16" else a


def dev(a, dtype):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV, tdt(dtype))


def host(t):
    torch.cuda.synchronize()
    return t.float().cpu().numpy()


# ------------------------------------------------------------------ LayerNorm

@pytest.mark.parametrize("dtype,rows,hidden", [
    ("f32", 7, 64), ("f32", 5, 12288), ("bf16", 37, 1024), ("bf16", 130, 5120),
    ("bf16", 3, 12288), ("bf16", 1, 64),
    # widths at and past the register-array sizes the launcher picks from
    ("bf16", 9, 6144), ("bf16", 17, 6148), ("bf16", 5, 2052), ("f32", 3, 10244),
    ("f32", 11, 4100)])
def test_layernorm(dtype, rows, hidden):
    print(f"case layernorm {dtype} rows={rows} hidden={hidden}", flush=True)
    rng = np.random.default_rng(rows * 7 + hidden)
    x = (0.3 + 2 * rng.standard_normal((rows, hidden))).astype(np.float32)
    g = draw(rng, hidden, 0.02, dtype, 1.0)
    b = draw(rng, hidden, 0.02, dtype)
    out = torch.empty((rows, hidden), dtype=tdt(dtype), device=DEV)
    L.orca_op_layernorm(odt(dtype), torch.from_numpy(x).to(DEV), dev(g, dtype), dev(b, dtype),
                        out, rows, hidden, 1e-5)
    ref = om.layer_norm(x.astype(np.float64), g.astype(np.float64), b.astype(np.float64), 1e-5)
    assert rel_err(host(out), ref) < TOL[dtype]


# ------------------------------------------------------------------ Linear

LINEAR_CASES = [
    ("bf16", 1, 128, 64), ("bf16", 7, 192, 64), ("bf16", 130, 384, 256),
    ("bf16", 300, 1024, 1024), ("bf16", 257, 3072, 1024), ("bf16", 129, 128, 4096),
    ("f32", 7, 192, 64), ("f32", 65, 256, 128), ("f32", 1, 64, 64),
    # few tiles: the split-K path when a workspace is given
    ("bf16", 33, 640, 2048), ("bf16", 64, 1536, 512), ("bf16", 31, 320, 4096),
    ("bf16", 64, 128, 64), ("bf16", 200, 1280, 2048), ("bf16", 1000, 640, 1024),
]
# shapes whose tiles are too few to fill the GPU: split-K must be taken
SPLIT_EXPECTED = {(33, 640, 2048), (64, 1536, 512), (31, 320, 4096), (200, 1280, 2048),
                  (1000, 640, 1024)}


def _linear_case(dtype, m, n, k, epi, workspace):
    rng = np.random.default_rng(m * 1000 + n + k + epi)
    a = draw(rng, (m, k), 1.0, dtype)
    w = draw(rng, (n, k), 0.02 * 32 / np.sqrt(k), dtype)
    b = draw(rng, n, 0.02, dtype)
    ref = om.linear(a.astype(np.float64), w.astype(np.float64), b.astype(np.float64))
    if epi == L.ORCA_EPI_BIAS_RESID:
        init = rng.standard_normal((m, n)).astype(np.float32)
        out = torch.from_numpy(init).to(DEV)
        ref = init.astype(np.float64) + ref
    else:
        out = torch.empty((m, n), dtype=tdt(dtype), device=DEV)
        if epi == L.ORCA_EPI_BIAS_GELU:
            ref = om.gelu_tanh(ref)
    ws, nb = None, 0
    if workspace:
        nb = L.orca_op_linear_workspace_bytes(odt(dtype), m, n, k)
        # poison the partial buffer: every element it holds must be written
        ws = torch.full((max(nb, 4) // 4,), float("nan"), dtype=torch.float32, device=DEV)
    L.orca_op_linear(odt(dtype), epi, dev(a, dtype), dev(w, dtype), dev(b, dtype), out, m, n, k,
                     ws, nb)
    return host(out), ref, nb


@pytest.mark.parametrize("epi", [L.ORCA_EPI_BIAS, L.ORCA_EPI_BIAS_GELU, L.ORCA_EPI_BIAS_RESID])
@pytest.mark.parametrize("dtype,m,n,k", LINEAR_CASES)
@pytest.mark.parametrize("workspace", [False, True])
def test_linear(dtype, m, n, k, epi, workspace):
    print(f"case linear {dtype} m={m} n={n} k={k} epi={epi} ws={workspace}", flush=True)
    got, ref, nb = _linear_case(dtype, m, n, k, epi, workspace)
    if workspace:
        if dtype == "f32":
            assert nb == 0
        elif (m, n, k) in SPLIT_EXPECTED:
            assert nb > 0
    assert np.isfinite(got).all()
    assert rel_err(got, ref) < TOL[dtype]


@pytest.mark.parametrize("variant", ["0", "3", "6", "7", "8", "10", "11", "12", "13", "14",
                                     "15"])
@pytest.mark.parametrize("m,n,k,epi", [
    (300, 1024, 1024, L.ORCA_EPI_BIAS_GELU), (520, 768, 2048, L.ORCA_EPI_BIAS_RESID),
    (64, 1536, 512, L.ORCA_EPI_BIAS), (33, 640, 2048, L.ORCA_EPI_BIAS_GELU)])
def test_linear_every_variant(variant, m, n, k, epi, monkeypatch):
    """Each tile variant (pinned), and the split-K path, against the oracle."""
    print(f"case linear variant {variant} m={m} n={n} k={k} epi={epi}", flush=True)
    monkeypatch.setenv("ORCA_GEMM_VARIANT", variant)
    got, ref, nb = _linear_case("bf16", m, n, k, epi, True)
    if variant == "10":
        assert nb > 0
    assert rel_err(got, ref) < TOL["bf16"]


# edges of the four-wave tiles (variants 12 and 14: 256 x 256, 13 and 15:
# 256 x 192; 14 and 15 load through LDS DMA in 32-wide K steps): the
# shortest K (one 64-wide step: fewer K steps than LDS stages), an odd step
# count (12 and 13 fall back to the eight-wave form), one row, rows and
# columns that end inside a tile
@pytest.mark.parametrize("variant", ["12", "13", "14", "15"])
@pytest.mark.parametrize("m,n,k", [(1, 128, 128), (100, 256, 64), (257, 448, 128),
                                   (300, 640, 192), (513, 1344, 384), (2176, 1024, 640)])
@pytest.mark.parametrize("epi", [L.ORCA_EPI_BIAS, L.ORCA_EPI_BIAS_GELU, L.ORCA_EPI_BIAS_RESID])
def test_four_wave_edges(variant, m, n, k, epi, monkeypatch):
    print(f"case four-wave variant {variant} m={m} n={n} k={k} epi={epi}", flush=True)
    monkeypatch.setenv("ORCA_GEMM_VARIANT", variant)
    got, ref, _ = _linear_case("bf16", m, n, k, epi, False)
    assert np.isfinite(got).all()
    assert rel_err(got, ref) < TOL["bf16"]


@pytest.mark.parametrize("variant", ["12", "13", "14", "15"])
def test_four_wave_is_deterministic(variant, monkeypatch):
    """Two launches on the same inputs give the same bits."""
    monkeypatch.setenv("ORCA_GEMM_VARIANT", variant)
    m, n, k = 700, 1536, 1024
    rng = np.random.default_rng(7)
    a = dev(draw(rng, (m, k), 1.0, "bf16"), "bf16")
    w = dev(draw(rng, (n, k), 0.02, "bf16"), "bf16")
    b = dev(draw(rng, n, 0.02, "bf16"), "bf16")
    outs = []
    for _ in range(2):
        out = torch.empty((m, n), dtype=torch.bfloat16, device=DEV)
        L.orca_op_linear(L.ORCA_BF16, L.ORCA_EPI_BIAS_GELU, a, w, b, out, m, n, k)
        outs.append(out.view(torch.int16).cpu().numpy())
    assert np.array_equal(outs[0], outs[1])


# persistent four-wave launches (more than one round of tiles: one
# workgroup per CU walks its XCD's share of them): the same bits as one
# workgroup per tile (ORCA_GEMM_PERSIST=0; only the tile-to-workgroup
# assignment differs), and sampled rows, the ragged last row tile among
# them, against the oracle.  (1100, 20480, 256) on 256 x 256: 5 x 80 = 400
# tiles, no tail; (1100, 20224, 256): 5 x 79 = 395 tiles, not a multiple of
# the 8 XCDs (three XCDs take one tile more); (1600, 15360, 512) on 256 x
# 192: 7 x 80 = 560 tiles; (2176, 15360, 2048) on 256 x 256: 9 x 60 = 540
# tiles = 512 persistent + a 28-tile split-K tail.
@pytest.mark.parametrize("m,n,k,variant,epi", [
    (1100, 20480, 256, "12", L.ORCA_EPI_BIAS_GELU),
    (1100, 20224, 256, "12", L.ORCA_EPI_BIAS),
    (1600, 15360, 512, "13", L.ORCA_EPI_BIAS),
    (2176, 15360, 2048, "12", L.ORCA_EPI_BIAS_RESID)])
def test_persistent_launch(m, n, k, variant, epi, monkeypatch):
    print(f"case persistent m={m} n={n} k={k} variant={variant} epi={epi}", flush=True)
    monkeypatch.setenv("ORCA_GEMM_VARIANT", variant)
    rng = np.random.default_rng(m + n + k)
    a = draw(rng, (m, k), 1.0, "bf16")
    w = draw(rng, (n, k), 0.02 * 32 / np.sqrt(k), "bf16")
    b = draw(rng, n, 0.02, "bf16")
    init = rng.standard_normal((m, n)).astype(np.float32)
    nb = L.orca_op_linear_workspace_bytes(L.ORCA_BF16, m, n, k)
    ws = torch.empty(max(nb, 4), dtype=torch.uint8, device=DEV)
    da, dw, db = dev(a, "bf16"), dev(w, "bf16"), dev(b, "bf16")
    outs = []
    for persist in ("1", "0"):
        monkeypatch.setenv("ORCA_GEMM_PERSIST", persist)
        if epi == L.ORCA_EPI_BIAS_RESID:
            out = torch.from_numpy(init).to(DEV)
        else:
            out = torch.empty((m, n), dtype=torch.bfloat16, device=DEV)
        L.orca_op_linear(L.ORCA_BF16, epi, da, dw, db, out, m, n, k, ws, nb)
        outs.append(out)
    bits = [o.view(torch.int32 if o.dtype == torch.float32 else torch.int16).cpu().numpy()
            for o in outs]
    assert np.array_equal(bits[0], bits[1])
    rows = np.array(sorted({0, 1, 255, 256, m // 2, m - 2, m - 1}))
    ref = om.linear(a[rows].astype(np.float64), w.astype(np.float64), b.astype(np.float64))
    if epi == L.ORCA_EPI_BIAS_RESID:
        ref = init[rows].astype(np.float64) + ref
    elif epi == L.ORCA_EPI_BIAS_GELU:
        ref = om.gelu_tanh(ref)
    got = host(outs[0])[rows]
    assert np.isfinite(got).all()
    assert rel_err(got, ref) < TOL["bf16"]


def test_linear_empty_batch_is_noop():
    out = torch.full((4, 128), 3.0, device=DEV)
    a = torch.zeros((4, 64), device=DEV, dtype=torch.bfloat16)
    L.orca_op_linear(L.ORCA_BF16, L.ORCA_EPI_BIAS_RESID, a, a, a, out, 0, 128, 64)
    assert bool((host(out) == 3.0).all())


# ------------------------------------------------------------- QKV + append

@pytest.mark.parametrize("dtype,m,hidden,heads,variant", [
    ("bf16", 7, 256, 2, None), ("bf16", 133, 512, 8, None), ("bf16", 64, 1024, 8, None),
    ("f32", 7, 64, 4, None), ("f32", 70, 256, 8, None),
    ("bf16", 300, 512, 4, "6"), ("bf16", 300, 512, 4, "0"), ("bf16", 300, 512, 4, "10"),
    ("bf16", 300, 512, 4, "8"), ("bf16", 300, 512, 4, "11"), ("bf16", 300, 512, 4, "12"),
    ("bf16", 300, 512, 4, "13"), ("bf16", 257, 768, 6, "12"), ("bf16", 70, 1024, 16, "13"),
    ("bf16", 40, 1024, 8, "10"), ("bf16", 300, 512, 4, "14"), ("bf16", 300, 512, 4, "15"),
    ("bf16", 257, 768, 6, "14"), ("bf16", 70, 1024, 16, "15")])
def test_qkv_split_and_append(dtype, m, hidden, heads, variant, monkeypatch):
    if variant is not None:
        monkeypatch.setenv("ORCA_GEMM_VARIANT", variant)
    print(f"case qkv {dtype} m={m} hidden={hidden} heads={heads} variant={variant}", flush=True)
    rng = np.random.default_rng(m + hidden)
    d = hidden // heads
    cap = 3 * m + 5
    a = draw(rng, (m, hidden), 1.0, dtype)
    w = draw(rng, (3 * hidden, hidden), 0.02, dtype)
    b = draw(rng, 3 * hidden, 0.02, dtype)
    dst = rng.permutation(cap)[:m].astype(np.int32)
    # one layer's pool [heads][cap][2][d]: key rows 7, value rows -7
    kvp = torch.empty((heads, cap, 2, d), dtype=tdt(dtype), device=DEV)
    kvp[:, :, 0] = 7.0
    kvp[:, :, 1] = -7.0
    kp, vp = kvp[:, :, 0], kvp[:, :, 1]
    q = torch.empty((m, hidden), dtype=tdt(dtype), device=DEV)
    nb = L.orca_op_linear_workspace_bytes(odt(dtype), m, 3 * hidden, hidden)
    ws = torch.empty(max(nb, 1), dtype=torch.uint8, device=DEV)
    L.orca_op_qkv(odt(dtype), dev(a, dtype), dev(w, dtype), dev(b, dtype), q, kvp,
                  torch.from_numpy(dst).to(DEV), m, hidden, heads, cap, ws, nb)
    ref = om.linear(a.astype(np.float64), w.astype(np.float64), b.astype(np.float64))
    assert rel_err(host(q), ref[:, :hidden]) < TOL[dtype]
    kh, vh = host(kp), host(vp)
    k_rows = kh[:, dst, :].transpose(1, 0, 2).reshape(m, hidden)
    v_rows = vh[:, dst, :].transpose(1, 0, 2).reshape(m, hidden)
    assert rel_err(k_rows, ref[:, hidden:2 * hidden]) < TOL[dtype]
    assert rel_err(v_rows, ref[:, 2 * hidden:]) < TOL[dtype]
    untouched = np.setdiff1d(np.arange(cap), dst)
    assert np.all(kh[:, untouched] == 7.0) and np.all(vh[:, untouched] == -7.0)


# ------------------------------------------------------------------ attention

ATTN_CASES = [
    # dtype, hidden, heads, [(q_len, kv_len) ...]
    ("bf16", 512, 4, [(1, 1), (1, 5), (1, 511), (1, 512), (1, 513), (1, 1100), (1, 2047), (517, 0),
                      (1, 2048), (1, 4200), (1, 0), (2, 0), (63, 0), (64, 0), (65, 0), (200, 0)]),
    ("bf16", 512, 8, [(1, 3), (1, 700), (1, 1500), (37, 0), (129, 0), (1, 0)]),
    ("f32", 64, 4, [(1, 3), (1, 4), (2, 0), (3, 0)]),
    ("f32", 128, 4, [(1, 600), (1, 1), (40, 0), (1, 0)]),
    ("f32", 256, 8, [(1, 1025), (17, 0), (1, 9)]),
    ("f32", 512, 4, [(1, 513), (70, 0), (1, 2)]),
]


@pytest.mark.parametrize("dtype,hidden,heads,shape", ATTN_CASES)
def test_split_attention(dtype, hidden, heads, shape):
    print(f"case attention {dtype} hidden={hidden} heads={heads} n={len(shape)}", flush=True)
    _attention_case(dtype, hidden, heads, shape)


# both prefill forms (64-key steps, two workgroups per CU; 32-key steps,
# three per CU), pinned: whole prompts of 1-517 rows, prompt chunks over a
# cached prefix (initiation rows with kv_len > 0), beside increments; head
# dims 128 and 64
PREFILL_CASES = [
    (512, 4, [(517, 0), (200, 130), (65, 0), (1, 300), (2, 0), (31, 33), (129, 1), (64, 0)]),
    (512, 8, [(300, 0), (97, 200), (1, 40), (33, 0), (128, 128)]),
]


# both forms and both workgroup orders (longest-first; grouped by (request,
# head) per XCD) on whole prompts and chunks: the order only moves where a
# tile runs, so every output row must match the oracle either way
@pytest.mark.parametrize("order", ["0", "1"])
@pytest.mark.parametrize("keys", ["64", "32"])
@pytest.mark.parametrize("hidden,heads,shape", PREFILL_CASES)
def test_prefill_forms(keys, order, hidden, heads, shape, monkeypatch):
    print(f"case prefill keys={keys} order={order} hidden={hidden} heads={heads} "
          f"n={len(shape)}", flush=True)
    monkeypatch.setenv("ORCA_PF_KEYS", keys)
    monkeypatch.setenv("ORCA_PF_ORDER", order)
    _attention_case("bf16", hidden, heads, shape)


def _attention_case(dtype, hidden, heads, shape):
    rng = np.random.default_rng(hidden + heads + len(shape))
    q_len = [s[0] for s in shape]
    kv_len = [s[1] for s in shape]
    work = synth.custom_workload(1, hidden, heads, 128, dtype, q_len, kv_len)
    model = dm_for(work, fill=False)
    try:
        d = hidden // heads
        rows = work.rows
        # synthetic pool: cached entries and this iteration's appended entries
        kp = draw(rng, model.k_pool.shape, 1.0, dtype)
        vp = draw(rng, model.v_pool.shape, 1.0, dtype)
        model.k_pool.copy_(torch.from_numpy(kp))
        model.v_pool.copy_(torch.from_numpy(vp))
        q = draw(rng, (rows, hidden), 1.0, dtype)
        o = torch.full((rows, hidden), 5.0, dtype=tdt(dtype), device=DEV)
        reqs = model.descriptors()
        L.orca_op_attention(model.ctx, 0, reqs, dev(q, dtype), o, model.ws, model.ws_bytes)
        got = host(o)
        ref = np.zeros((rows, hidden))
        for (off, ql, kvl, _, base) in reqs:
            n = kvl + ql
            k_all = kp[0, :, base:base + n, :].transpose(1, 0, 2).reshape(n, hidden)
            v_all = vp[0, :, base:base + n, :].transpose(1, 0, 2).reshape(n, hidden)
            ref[off:off + ql] = om.request_attention(q[off:off + ql].astype(np.float64),
                                                     k_all.astype(np.float64),
                                                     v_all.astype(np.float64), kvl, heads)
        for (off, ql, kvl, _, _) in reqs:
            e = rel_err(got[off:off + ql], ref[off:off + ql])
            assert e < TOL[dtype], (off, ql, kvl, e)
    finally:
        model.close()


def dm_for(work, fill=True, **kw):
    from orca_selective_iteration_amd.runner import DeviceModel
    return DeviceModel(work, device=DEV, fill_caches=fill, **kw)


# hybrid launches of the four-wave tiles: the last, at most half-full round
# of tiles split over K (fp32 partials added by the tail reduce with the
# epilogue).  (1100, 15360, 4096) on 256 x 256 tiles: 5 x 60 = 300 tiles =
# one round + 44 tail tiles in 4 splits; (1100, 14400, 4096) on 256 x 192:
# 5 x 75 = 375 tiles = one round + 119 in 2 splits.  The whole output is
# compared with the same launch without the tail (ORCA_GEMM_TAIL=0: only the
# summation order differs), and sampled rows, among them the ragged last row
# tile, with the oracle.
@pytest.mark.parametrize("variant,n", [("12", 15360), ("13", 14400)])
@pytest.mark.parametrize("epi", [L.ORCA_EPI_BIAS, L.ORCA_EPI_BIAS_GELU, L.ORCA_EPI_BIAS_RESID])
def test_hybrid_split_tail(variant, n, epi, monkeypatch):
    m, k = 1100, 4096
    print(f"case hybrid tail variant {variant} m={m} n={n} k={k} epi={epi}", flush=True)
    monkeypatch.setenv("ORCA_GEMM_VARIANT", variant)
    rng = np.random.default_rng(n + epi)
    a = draw(rng, (m, k), 1.0, "bf16")
    w = draw(rng, (n, k), 0.02 * 32 / np.sqrt(k), "bf16")
    b = draw(rng, n, 0.02, "bf16")
    init = rng.standard_normal((m, n)).astype(np.float32) if epi == L.ORCA_EPI_BIAS_RESID else None
    nb = L.orca_op_linear_workspace_bytes(L.ORCA_BF16, m, n, k)
    assert nb > 0, "expected a split tail"
    ad, wd, bd = dev(a, "bf16"), dev(w, "bf16"), dev(b, "bf16")
    outs = []
    for tail in ("1", "0"):
        monkeypatch.setenv("ORCA_GEMM_TAIL", tail)
        out = (torch.from_numpy(init).to(DEV) if init is not None
               else torch.empty((m, n), dtype=torch.bfloat16, device=DEV))
        ws = torch.full((nb // 4,), float("nan"), dtype=torch.float32, device=DEV)
        L.orca_op_linear(L.ORCA_BF16, epi, ad, wd, bd, out, m, n, k, ws, nb)
        outs.append(host(out))
    assert np.isfinite(outs[0]).all()
    assert rel_err(outs[0], outs[1]) < 1e-2
    rows = np.concatenate([np.arange(0, 8), np.arange(500, 508), np.arange(m - 40, m)])
    ref = om.linear(a[rows].astype(np.float64), w.astype(np.float64), b.astype(np.float64))
    if epi == L.ORCA_EPI_BIAS_GELU:
        ref = om.gelu_tanh(ref)
    if init is not None:
        ref = init[rows].astype(np.float64) + ref
    assert rel_err(outs[0][rows], ref) < TOL["bf16"]


# main-and-helper tails (the last round more than half full;
# ORCA_GEMM_SK_MIN=0 takes them at these small K): (1100, 20480, 2048) on
# 256 x 256: 400 tiles = 256 + 144, 32 K steps a tile, 144 mains taking 24,
# 112 helpers the other 8 of one or two tiles each; (1100, 15168, 2560) on
# 256 x 192: 395 = 256 + 139, 40 steps, mains 28; (1100, 20032, 2048): 395
# tiles, the last column tile 64 wide.  The workspace starts as NaN (a
# partial tile the reduce reads but no workgroup wrote shows), the output is
# compared with the launch without a tail and with the oracle on sampled
# rows, and a second call gives the same bits (the partial tiles are added
# in a fixed order).
@pytest.mark.parametrize("m,n,k,variant", [
    (1100, 20480, 2048, "12"), (1100, 15168, 2560, "13"), (1100, 20032, 2048, "12")])
@pytest.mark.parametrize("epi", [L.ORCA_EPI_BIAS, L.ORCA_EPI_BIAS_GELU, L.ORCA_EPI_BIAS_RESID])
def test_main_helper_tail(m, n, k, variant, epi, monkeypatch):
    print(f"case main-and-helper tail variant {variant} m={m} n={n} k={k} epi={epi}", flush=True)
    monkeypatch.setenv("ORCA_GEMM_VARIANT", variant)
    monkeypatch.setenv("ORCA_GEMM_SK_MIN", "0")
    rng = np.random.default_rng(n + k + epi)
    a = draw(rng, (m, k), 1.0, "bf16")
    w = draw(rng, (n, k), 0.02 * 32 / np.sqrt(k), "bf16")
    b = draw(rng, n, 0.02, "bf16")
    init = rng.standard_normal((m, n)).astype(np.float32) if epi == L.ORCA_EPI_BIAS_RESID else None
    nb = L.orca_op_linear_workspace_bytes(L.ORCA_BF16, m, n, k)
    assert nb > 0, "expected a main-and-helper tail"
    ad, wd, bd = dev(a, "bf16"), dev(w, "bf16"), dev(b, "bf16")
    outs = []
    for tail in ("1", "1", "0"):
        monkeypatch.setenv("ORCA_GEMM_TAIL", tail)
        out = (torch.from_numpy(init).to(DEV) if init is not None
               else torch.empty((m, n), dtype=torch.bfloat16, device=DEV))
        ws = torch.full((nb // 4,), float("nan"), dtype=torch.float32, device=DEV)
        L.orca_op_linear(L.ORCA_BF16, epi, ad, wd, bd, out, m, n, k, ws, nb)
        outs.append(host(out))
    assert np.isfinite(outs[0]).all()
    assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32))
    assert rel_err(outs[0], outs[2]) < 1e-2
    rows = np.concatenate([np.arange(0, 8), np.arange(700, 708), np.arange(m - 40, m)])
    ref = om.linear(a[rows].astype(np.float64), w.astype(np.float64), b.astype(np.float64))
    if epi == L.ORCA_EPI_BIAS_GELU:
        ref = om.gelu_tanh(ref)
    if init is not None:
        ref = init[rows].astype(np.float64) + ref
    assert rel_err(outs[0][rows], ref) < TOL["bf16"]


def test_main_helper_tail_qkv(monkeypatch):
    """The QKV projection with a main-and-helper tail (hidden 7168: 5 x 84 =
    420 tiles = 256 + 164, 112 K steps a tile): the same Q rows and pool
    slots as the launch without a tail, and the oracle's on sampled rows."""
    m, hidden, heads = 1100, 7168, 56
    d, cap = hidden // heads, 1500
    monkeypatch.setenv("ORCA_GEMM_VARIANT", "12")
    monkeypatch.setenv("ORCA_GEMM_SK_MIN", "0")
    nb = L.orca_op_linear_workspace_bytes(L.ORCA_BF16, m, 3 * hidden, hidden)
    assert nb > 0
    rng = np.random.default_rng(7)
    a = draw(rng, (m, hidden), 1.0, "bf16")
    w = draw(rng, (3 * hidden, hidden), 0.02, "bf16")
    b = draw(rng, 3 * hidden, 0.02, "bf16")
    dst = rng.permutation(cap)[:m].astype(np.int32)
    res = []
    for tail in ("1", "0"):
        monkeypatch.setenv("ORCA_GEMM_TAIL", tail)
        kvp = torch.zeros((heads, cap, 2, d), dtype=torch.bfloat16, device=DEV)
        kp, vp = kvp[:, :, 0], kvp[:, :, 1]
        q = torch.empty((m, hidden), dtype=torch.bfloat16, device=DEV)
        ws = torch.full((nb // 4,), float("nan"), dtype=torch.float32, device=DEV)
        L.orca_op_qkv(L.ORCA_BF16, dev(a, "bf16"), dev(w, "bf16"), dev(b, "bf16"), q, kvp,
                      torch.from_numpy(dst).to(DEV), m, hidden, heads, cap, ws, nb)
        res.append((host(q), host(kp), host(vp)))
    for x, y in zip(res[0], res[1]):
        assert np.isfinite(x).all()
        assert rel_err(x, y) < 1e-2
    rows = np.concatenate([np.arange(0, 4), np.arange(m - 20, m)])
    ref = om.linear(a[rows].astype(np.float64), w.astype(np.float64), b.astype(np.float64))
    assert rel_err(res[0][0][rows], ref[:, :hidden]) < TOL["bf16"]
    kref = ref[:, hidden:2 * hidden].reshape(len(rows), heads, d).transpose(1, 0, 2)
    vref = ref[:, 2 * hidden:].reshape(len(rows), heads, d).transpose(1, 0, 2)
    assert rel_err(res[0][1][:, dst[rows]], kref) < TOL["bf16"]
    assert rel_err(res[0][2][:, dst[rows]], vref) < TOL["bf16"]


def test_hybrid_split_tail_qkv(monkeypatch):
    """The QKV projection's split tail: the same Q rows and pool slots as the
    launch without it, and the oracle's on sampled rows."""
    m, hidden, heads = 1100, 5120, 40       # 256 x 256 tiles: 300 = 256 + 44
    d, cap = hidden // heads, 1500
    monkeypatch.setenv("ORCA_GEMM_VARIANT", "12")
    nb = L.orca_op_linear_workspace_bytes(L.ORCA_BF16, m, 3 * hidden, hidden)
    assert nb > 0
    rng = np.random.default_rng(5)
    a = draw(rng, (m, hidden), 1.0, "bf16")
    w = draw(rng, (3 * hidden, hidden), 0.02, "bf16")
    b = draw(rng, 3 * hidden, 0.02, "bf16")
    dst = rng.permutation(cap)[:m].astype(np.int32)
    res = []
    for tail in ("1", "0"):
        monkeypatch.setenv("ORCA_GEMM_TAIL", tail)
        kvp = torch.zeros((heads, cap, 2, d), dtype=torch.bfloat16, device=DEV)
        kp, vp = kvp[:, :, 0], kvp[:, :, 1]
        q = torch.empty((m, hidden), dtype=torch.bfloat16, device=DEV)
        ws = torch.full((nb // 4,), float("nan"), dtype=torch.float32, device=DEV)
        L.orca_op_qkv(L.ORCA_BF16, dev(a, "bf16"), dev(w, "bf16"), dev(b, "bf16"), q, kvp,
                      torch.from_numpy(dst).to(DEV), m, hidden, heads, cap, ws, nb)
        res.append((host(q), host(kp), host(vp)))
    for x, y in zip(res[0], res[1]):
        assert rel_err(x, y) < 1e-2
    rows = np.concatenate([np.arange(0, 4), np.arange(m - 20, m)])
    ref = om.linear(a[rows].astype(np.float64), w.astype(np.float64), b.astype(np.float64))
    assert rel_err(res[0][0][rows], ref[:, :hidden]) < TOL["bf16"]
    kref = ref[:, hidden:2 * hidden].reshape(len(rows), heads, d).transpose(1, 0, 2)
    assert rel_err(res[0][1][:, dst[rows]], kref) < TOL["bf16"]
