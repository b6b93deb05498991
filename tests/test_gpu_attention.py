"""GPU parity of the fused quantized attention against the oracle (R3).

Whole path per workload: calibration (static scales) -> quantization -> attention, with the
FP8 inputs compared bit-exactly and the output within rel-L2 1e-2 and max-abs 5e-2 of the
oracle.  At full size the oracle evaluates sampled query rows (each row is independent).
The error against unquantized float64 attention is printed, not gated.
"""
import math

import numpy as np
import pytest
import torch

import precision_quantized_attention_amd as kq
import workloads as W
from kq_testutil import MAX_ABS_TOL, REL_L2_TOL, max_abs, rel_l2, sample_rows, to_dev
from oracle import attention as A
from oracle import formats as F
from oracle import pipeline as OP
from precision_quantized_attention_amd.pipeline import QuantizedSDPA

pytestmark = pytest.mark.gpu


def _run(bits, mode="fp8", positions=None, stats=False):
    B, H, N, d = bits[0].shape
    x = [to_dev(b) for b in bits]
    m = QuantizedSDPA(B, H, N, d, mode=mode, positions=positions, want_stats=stats)
    m.calibrate(*x)
    o = m.forward(*x)
    torch.cuda.synchronize()
    if m.fuse_q:
        m.quantize(*x)          # forward() formed Q's codes in the kernel: write them for the checks
    return m, o


_QZ = {}


def _oracle_inputs(cfg):
    """The oracle's quantization of a workload, once per process (cfg 5's RoPE and FP4 steps
    take tens of seconds)."""
    if cfg not in _QZ:
        c = W.config(cfg)
        _QZ[cfg] = OP.quantize_inputs(*W.qkv_bits(cfg), mode=c.mode,
                                      positions=W.positions(c) if c.rope else None)
    return _QZ[cfg]


def _check_codes(m, qz):
    c = m.buf
    assert np.array_equal(c.q8.cpu().numpy(), qz.codes["q"])
    assert np.array_equal(c.k8.cpu().numpy(), qz.codes["k"])
    B, H, N, d = qz.codes["v"].shape
    vt = c.v8t.cpu().numpy()[:, :, :N].transpose(0, 2, 1).reshape(B, H, N, d)
    assert np.array_equal(vt, qz.codes["v"])
    assert not np.any(c.v8t.cpu().numpy()[:, :, N:])


def _compare(o_gpu, o_ref, label):
    e, a = rel_l2(o_gpu, o_ref), max_abs(o_gpu, o_ref)
    print(f"{label}: rel_l2 {e:.3e} max_abs {a:.3e} (|O| max {np.abs(o_ref).max():.3g})",
          flush=True)
    assert e <= REL_L2_TOL, (label, e)
    assert a <= MAX_ABS_TOL, (label, a)
    return e, a


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_attention_config(cfg):
    c = W.config(cfg)
    print(f"attention cfg{cfg} {c.name} B={c.B} H={c.H} N={c.N} mode={c.mode} rope={c.rope}",
          flush=True)
    bits = W.qkv_bits(cfg)
    pos = W.positions(c) if c.rope else None
    m, o = _run(bits, mode=c.mode, positions=pos, stats=True)
    qz = _oracle_inputs(cfg)
    for n in "qkv":
        assert m.amax[n] == qz.amax[n] and m.scales[n] == qz.scale[n]
    _check_codes(m, qz)
    if cfg == 1:
        rows, heads = np.arange(c.N), [(b, h) for b in range(c.B) for h in range(c.H)]
    else:
        rows = sample_rows(c.N, 24, seed=cfg)
        heads = [(0, 0), (c.B - 1, c.H - 1), (c.B // 2, 7 % c.H)]
    o_np = o.cpu().numpy()
    stats = m.buf.stats.cpu().numpy()
    sub = {n: np.stack([qz.codes[n][b, h] for b, h in heads])[None] for n in "qkv"}
    O, M, L = A.attention_r3(sub["q"], sub["k"], sub["v"], qz.scale["q"][0], qz.scale["k"][0],
                             qz.scale["v"][0], m.sm_scale, rows=rows)
    got = np.stack([o_np[b, h][rows] for b, h in heads])
    _compare(got, O[0], f"cfg{cfg} vs oracle")
    # row statistics: same offset up to a float32 tie at an integer, same 2^M * l
    st = np.stack([stats[b, h][rows] for b, h in heads])
    assert np.all(np.abs(st[..., 0] - M[0]) <= 1)
    tot_gpu = st[..., 1].astype(np.float64) * np.exp2(st[..., 0])
    tot_ref = L[0].astype(np.float64) * np.exp2(M[0])
    assert np.allclose(tot_gpu, tot_ref, rtol=1e-2)
    # reported, not gated: error of the quantized path against float64 attention
    xs = [W.bits_to_f32(b) for b in bits]
    if c.rope:
        from oracle import rope as R
        tab = R.table(pos)
        xs[0], xs[1] = R.apply(xs[0], tab), R.apply(xs[1], tab)
    sel = [np.stack([x[b, h] for b, h in heads])[None] for x in xs]
    ref64 = A.attention_fp64(sel[0], sel[1], sel[2], 1 / math.sqrt(128), rows=rows)
    print(f"cfg{cfg} vs unquantized fp64: rel_l2 {rel_l2(got, ref64[0]):.3e} "
          f"(oracle itself: {rel_l2(O[0], ref64[0]):.3e})", flush=True)


_E4M3_POS = np.unique(F.e4m3_decode(np.arange(0x7F, dtype=np.uint8)))    # 0 .. 448
_MID = (_E4M3_POS[1:] + _E4M3_POS[:-1]) / 2


def _near_ties(q8, k8, c1, rel=1e-5):
    """Count of scores whose exact 448 p (R3, oracle definition) lies within `rel` of an E4M3
    rounding midpoint: the elements whose code a float32-order difference could flip."""
    raw = F.e4m3_decode(q8) @ F.e4m3_decode(k8).T
    t = F.fl32(raw * float(c1)).astype(np.float64)
    x = F.fl32(np.exp2(t - np.ceil(np.max(t, axis=1, keepdims=True)))).astype(np.float64) * 448.0
    i = np.clip(np.searchsorted(_MID, x), 1, len(_MID) - 1)
    d = np.minimum(np.abs(x - _MID[i]), np.abs(x - _MID[i - 1]))
    return int(np.sum(d <= rel * x)), x.size


@pytest.mark.parametrize("cfg,heads", [(2, None), (3, [(0, 0), (0, 23)]), (5, [(3, 23)])],
                         ids=["cfg2-every-head", "cfg3-heads-0-and-23", "cfg5-b3-h23"])
def test_attention_whole_heads(cfg, heads):
    """Every query row of whole heads against the oracle (cfg 2: the whole tensor; cfg 3: head
    0 and head 23, which runs entirely through the key split of the last round; cfg 5: the
    last head of the last batch), with the gate on every element."""
    c = W.config(cfg)
    print(f"whole heads cfg{cfg} {c.name}", flush=True)
    bits = W.qkv_bits(cfg)
    pos = W.positions(c) if c.rope else None
    m, o = _run(bits, mode=c.mode, positions=pos)
    qz = _oracle_inputs(cfg)
    _check_codes(m, qz)
    heads = heads or [(b, h) for b in range(c.B) for h in range(c.H)]
    o_np = o.cpu().numpy()
    c1, _ = A.constants(qz.scale["q"][0], qz.scale["k"][0], qz.scale["v"][0], m.sm_scale)
    worst, num, den, ties, n_el = 0.0, 0.0, 0.0, 0, 0
    for b, h in heads:
        sl = (slice(b, b + 1), slice(h, h + 1))
        O, _, _ = A.attention_r3(qz.codes["q"][sl], qz.codes["k"][sl], qz.codes["v"][sl],
                                 qz.scale["q"][0], qz.scale["k"][0], qz.scale["v"][0],
                                 m.sm_scale)
        d = o_np[b, h].astype(np.float64) - O[0, 0]
        worst = max(worst, float(np.max(np.abs(d))))
        num += float(np.sum(d ** 2))
        den += float(np.sum(O[0, 0].astype(np.float64) ** 2))
        if len(heads) <= 2 or h % 8 == 0:
            t_, n_ = _near_ties(qz.codes["q"][b, h], qz.codes["k"][b, h], c1)
            ties, n_el = ties + t_, n_el + n_
    e = math.sqrt(num / den)
    print(f"cfg{cfg} {len(heads)} whole heads: rel_l2 {e:.3e} max_abs {worst:.3e}; "
          f"scores within 1e-5 of an E4M3 midpoint: {ties} of {n_el}", flush=True)
    assert e <= REL_L2_TOL and worst <= MAX_ABS_TOL, (e, worst)


@pytest.mark.parametrize("N", [1, 2, 5, 63, 64, 65, 127, 128, 129, 255, 257, 1000])
def test_attention_ragged_lengths(N):
    print(f"ragged N={N}", flush=True)
    bits = [W.random_bits(1, 2, N, 128, seed=500 + 3 * N + t, outliers=(N > 100)) for t in range(3)]
    m, o = _run(bits)
    qz = OP.quantize_inputs(*bits)
    _check_codes(m, qz)
    O, _, _ = OP.attention(qz)
    _compare(o.cpu().numpy(), O, f"N={N}")


def test_attention_batch_heads_and_fp4_small():
    print("B=2 H=3 N=300 fp4+rope", flush=True)
    c = W.config(5)
    pos = W.positions(c)[450:750]
    bits = [W.random_bits(2, 3, 300, 128, seed=800 + t, outliers=True) for t in range(3)]
    m, o = _run(bits, mode="fp4", positions=pos)
    qz = OP.quantize_inputs(*bits, mode="fp4", positions=pos)
    _check_codes(m, qz)
    O, _, _ = OP.attention(qz)
    _compare(o.cpu().numpy(), O, "B2H3 fp4 rope")


@pytest.mark.parametrize("B,H,N", [(1, 2, 256), (1, 1, 4096), (1, 3, 8704), (1, 2, 1000),
                                   (1, 2, 65)])
def test_attention_key_split_matches_single_pass(B, H, N):
    """The workspace path splits the query blocks of a partial last round along the keys and
    merges the parts; it must agree with the single-pass kernel (same codes, float32 order
    only) and with the oracle on sampled rows."""
    print(f"key split B={B} H={H} N={N}", flush=True)
    bits = [W.random_bits(B, H, N, 128, seed=900 + 7 * N + H + t, outliers=True) for t in range(3)]
    m = QuantizedSDPA(B, H, N, 128, want_stats=True)
    x = [to_dev(b) for b in bits]
    m.calibrate(*x)
    m.quantize(*x)
    nbytes = kq.kq_attn_workspace_size(B, H, N)
    print(f"  workspace {nbytes} bytes", flush=True)
    assert nbytes > 0                  # every shape here leaves the last round partly idle
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    b = m.buf
    sc = [m.scales[n][0] for n in "qkv"]
    o1 = torch.empty_like(b.o)
    st1 = torch.empty_like(b.stats)
    kq.kq_attn_quant_fwd(b.q8, b.k8, b.v8t, *sc, m.sm_scale, o1, row_stats=st1)
    o2 = torch.empty_like(b.o)
    st2 = torch.empty_like(b.stats)
    kq.kq_attn_quant_fwd_ws(b.q8, b.k8, b.v8t, *sc, m.sm_scale, o2, ws, row_stats=st2)
    torch.cuda.synchronize()
    a1, a2 = o1.cpu().numpy(), o2.cpu().numpy()
    assert rel_l2(a2, a1) <= 1e-5 and max_abs(a2, a1) <= 1e-4, (rel_l2(a2, a1), max_abs(a2, a1))
    s1, s2 = st1.cpu().numpy(), st2.cpu().numpy()
    assert np.array_equal(s1[..., 0], s2[..., 0])
    assert np.allclose(s1[..., 1], s2[..., 1], rtol=1e-5)
    with pytest.raises(kq.KQError):            # too small a workspace is rejected
        kq.kq_attn_quant_fwd_ws(b.q8, b.k8, b.v8t, *sc, m.sm_scale, o2, ws[: nbytes - 16])
    qz = OP.quantize_inputs(*bits)
    rows = sample_rows(N, 8, seed=N)
    hs = [(0, 0), (B - 1, H - 1)]
    sub = {n: np.stack([qz.codes[n][bb, hh] for bb, hh in hs])[None] for n in "qkv"}
    O, _, _ = A.attention_r3(sub["q"], sub["k"], sub["v"], qz.scale["q"][0], qz.scale["k"][0],
                             qz.scale["v"][0], m.sm_scale, rows=rows)
    _compare(np.stack([a2[bb, hh][rows] for bb, hh in hs]), O[0], f"split B{B} H{H} N{N}")


def test_attention_beyond_2_31_elements():
    """4200 heads of N = 4096: Q, K, V hold 2.2e9 elements each (more than 2^31) and O 8.8 GB
    of float32, so element and byte offsets pass 32 bits in every kernel of the path.  Head h
    is seeded base head h % 8 rolled by h // 8 rows along the tokens (all heads distinct, the
    set of values that of the base), so the oracle rebuilds any head from the base."""
    B, H, N, d, nbase = 1, 4200, 4096, 128, 8
    assert B * H * N * d > 2 ** 31
    print(f"large: B={B} H={H} N={N} ({B * H * N * d} elements per tensor)", flush=True)
    base = [W.random_bits(1, nbase, N, d, seed=1500 + t, outliers=True) for t in range(3)]
    shifts = torch.arange(H // nbase + 1, device="cuda")
    tok = torch.arange(N, device="cuda")
    x = []
    for b in base:
        bd = to_dev(b)[0]
        full = torch.empty((B, H, N, d), dtype=torch.bfloat16, device="cuda")
        for j in range(nbase):
            cnt = len(range(j, H, nbase))
            idx = (tok[None, :] - shifts[:cnt, None]) % N          # np.roll by h // 8 rows
            full[0, j::nbase] = bd[j][idx]
        x.append(full)
        del bd
    m = QuantizedSDPA(B, H, N, d)
    m.calibrate(*x)
    o = m.forward(*x)
    m.quantize(*x)              # Q's codes into buf.q8 for the checks below (o is unchanged)
    torch.cuda.synchronize()
    del x
    qz = OP.quantize_inputs(*base)
    for n in "qkv":
        assert m.amax[n] == qz.amax[n] and m.scales[n] == qz.scale[n], n
    heads = [0, 2099, 4097, H - 1]                     # 4097 * N * d > 2^31
    roll = lambda a, h: np.roll(a[0, h % nbase], h // nbase, axis=0)
    for h in heads:
        assert np.array_equal(m.buf.q8[0, h].cpu().numpy(), roll(qz.codes["q"], h)), h
        assert np.array_equal(m.buf.k8[0, h].cpu().numpy(), roll(qz.codes["k"], h)), h
        assert np.array_equal(m.buf.v8t[h, :, :N].cpu().numpy().T, roll(qz.codes["v"], h)), h
    rows = sample_rows(N, 8, seed=77)
    sub = {n: np.stack([roll(qz.codes[n], h) for h in heads])[None] for n in "qkv"}
    O, _, _ = A.attention_r3(sub["q"], sub["k"], sub["v"], qz.scale["q"][0], qz.scale["k"][0],
                             qz.scale["v"][0], m.sm_scale, rows=rows)
    rows_d = torch.from_numpy(rows).cuda()
    got = np.stack([o[0, h].index_select(0, rows_d).cpu().numpy() for h in heads])
    _compare(got, O[0], f"H={H} N={N}")
    del o, m
    torch.cuda.empty_cache()


@pytest.mark.parametrize("gain", [8.0, 16.0])
def test_attention_large_score_gaps(gain):
    """Rows whose scores jump by ~130 (gain 8) or ~260 (gain 16) in the exp2 domain after the
    first key tiles: the single-pass kernel must move its row reference (the guarded rescale of
    the accumulators by an exact power of two) and, on the rows where the big keys score far
    below, clamp block offsets more than 2^126 below the reference; the key split merges parts
    whose references differ by the same amounts."""
    print(f"score gaps gain={gain}", flush=True)
    H, N = 2, 320
    bits = W.score_gap_bits(H, N, gain, seed=77 + int(gain))
    m = QuantizedSDPA(1, H, N, 128, want_stats=True)
    x = [to_dev(b) for b in bits]
    m.calibrate(*x)
    m.quantize(*x)
    qz = OP.quantize_inputs(*bits)
    _check_codes(m, qz)
    O, M, L = OP.attention(qz)
    assert M[0, :, ::2].min() > 100 and M[0, :, 1::2].max() < 20   # the gaps exist
    b = m.buf
    sc = [m.scales[n][0] for n in "qkv"]
    o1 = torch.empty_like(b.o)
    st1 = torch.empty_like(b.stats)
    kq.kq_attn_quant_fwd(b.q8, b.k8, b.v8t, *sc, m.sm_scale, o1, row_stats=st1)
    nbytes = kq.kq_attn_workspace_size(1, H, N)
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device="cuda")
    o2 = torch.empty_like(b.o)
    kq.kq_attn_quant_fwd_ws(b.q8, b.k8, b.v8t, *sc, m.sm_scale, o2, ws)
    torch.cuda.synchronize()
    _compare(o1.cpu().numpy(), O, f"gap {gain} single pass")
    _compare(o2.cpu().numpy(), O, f"gap {gain} key split")
    st = st1.cpu().numpy()
    assert np.all(np.abs(st[..., 0] - M) <= 1)
    assert np.allclose(st[..., 1].astype(np.float64) * np.exp2(st[..., 0].astype(np.float64) - M),
                       L.astype(np.float64), rtol=1e-4)


def _scaled_bits(qk_scale, v_scale, seed):
    return [W.random_bits(1, 2, 300, 128, seed=seed + t, outliers=True,
                          scale=(v_scale if t == 2 else qk_scale)) for t in range(3)]


@pytest.mark.parametrize("qk,vs,sm", [(1e-3, 1e-3, None), (20.0, 1.0, None), (1.0, 1.0, 1.0),
                                      (1.0, 1.0, 0.02)])
def test_attention_scale_ranges(qk, vs, sm):
    """c1 = s_q s_k sm_scale log2 e away from its usual value: all inputs scaled by 1e-3 (the
    static scales follow the amax), Q and K scaled by 20 (row offsets up to ~11000; the score
    bound c1 448^2 128 is 25 times 2^20, so the host launches the exp2 argument in the
    definition's unfused order), and softmax scales 1 (bound 0.71 times 2^20: the fused argument
    near its limit) and 0.02 (peaked and nearly flat rows)."""
    print(f"scale ranges qk x{qk} v x{vs} sm={sm}", flush=True)
    bits = _scaled_bits(qk, vs, 2100)
    x = [to_dev(b) for b in bits]
    m = QuantizedSDPA(1, 2, 300, 128, sm_scale=sm, want_stats=True)
    m.calibrate(*x)
    o = m.forward(*x)
    m.quantize(*x)
    torch.cuda.synchronize()
    qz = OP.quantize_inputs(*bits)
    _check_codes(m, qz)
    O, M, _ = OP.attention(qz, sm_scale=m.sm_scale)
    print(f"  row offsets M in [{M.min():.0f}, {M.max():.0f}]", flush=True)
    _compare(o.cpu().numpy(), O, f"qk x{qk} v x{vs} sm={m.sm_scale:.4g}")
    b = m.buf                                    # the single pass (no key split) as well
    o1 = torch.empty_like(b.o)
    kq.kq_attn_quant_fwd(b.q8, b.k8, b.v8t, *[m.scales[n][0] for n in "qkv"], m.sm_scale, o1)
    torch.cuda.synchronize()
    _compare(o1.cpu().numpy(), O, f"qk x{qk} v x{vs} sm={m.sm_scale:.4g} single pass")


def test_attention_extreme_score_magnitudes():
    """Q and K scaled by 1000: scores reach ~1e7 in the exp2 domain, where a float32 ulp is ~1,
    so the softmax is ill-conditioned (a float32 BMM1 moves single probabilities by factors
    near 2 against the exact-sum definition) and element-wise parity is not defined there.
    The kernel must stay finite and form convex combinations of V's rows (up to P's
    quantization, within 1/16), and agree with the oracle in rel-L2."""
    print("extreme score magnitudes", flush=True)
    bits = _scaled_bits(1000.0, 1.0, 2200)
    x = [to_dev(b) for b in bits]
    m = QuantizedSDPA(1, 2, 300, 128)
    m.calibrate(*x)
    o = m.forward(*x).cpu().numpy().astype(np.float64)
    qz = OP.quantize_inputs(*bits)
    O, M, _ = OP.attention(qz)
    print(f"  row offsets M up to {M.max():.3g}", flush=True)
    assert np.isfinite(o).all()
    from oracle import formats as F
    vd = F.e4m3_decode(qz.codes["v"]) * float(qz.scale["v"][0])         # [1, 2, N, d]
    lo, hi = vd.min(axis=2, keepdims=True), vd.max(axis=2, keepdims=True)
    slack = (hi - lo) / 16 + 1e-6
    assert np.all(o >= lo - slack) and np.all(o <= hi + slack)
    e = rel_l2(o, O)
    print(f"  rel_l2 vs oracle {e:.3e}, max_abs {max_abs(o, O):.3e} (|O| max {np.abs(O).max():.3g})",
          flush=True)
    assert e <= REL_L2_TOL


def test_attention_deterministic():
    bits = [b[:, :4] for b in W.qkv_bits(2)]
    m, o1 = _run(bits)
    o1 = o1.clone()
    o2 = m.forward(*[to_dev(b) for b in bits])
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


def test_attention_rejects_row_layout_v():
    x = torch.zeros((1, 1, 64, 128), dtype=torch.uint8, device="cuda")
    o = torch.empty((1, 1, 64, 128), dtype=torch.float32, device="cuda")
    with pytest.raises(kq.KQError):
        kq.kq_attn_quant_fwd(x, x, x, 1.0, 1.0, 1.0, 0.1, o, v_layout=kq.KQ_LAYOUT_ROWS)


def test_attention_every_e4m3_code_in_q_and_k():
    """Q and K holding every finite E4M3 code (both signs, subnormals, +-448): the kernel's
    on-chip conversion of the codes for the first product must be exact."""
    import oracle.formats as F
    N, d = 256, 128
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    rng = np.random.default_rng(5)
    q8 = rng.choice(codes, size=(1, 1, N, d)).astype(np.uint8)
    k8 = rng.choice(codes, size=(1, 1, N, d)).astype(np.uint8)
    v8 = rng.choice(codes, size=(1, 1, N, d)).astype(np.uint8)
    s_q = s_k = np.float32(2.0 ** -9)             # keep t = raw * c1 in a moderate range
    s_v = np.float32(1.0 / 64)
    sm = np.float32(1 / math.sqrt(128))
    ld = kq.kq_vt_ld(N)
    vt = np.zeros((1, d, ld), np.uint8)
    vt[0, :, :N] = v8[0, 0].T
    dq, dk, dv = (torch.from_numpy(x).cuda() for x in (q8, k8, vt))
    o = torch.empty((1, 1, N, d), dtype=torch.float32, device="cuda")
    kq.kq_attn_quant_fwd(dq, dk, dv, s_q, s_k, s_v, sm, o)
    torch.cuda.synchronize()
    O, _, _ = A.attention_r3(q8, k8, v8, s_q, s_k, s_v, sm)
    _compare(o.cpu().numpy(), O, "every E4M3 code")
    assert F.e4m3_decode(codes).max() == 448.0


def _fused_vs_unfused(m, x):
    """O and row statistics of forward() (Q quantized in the attention kernel) and of
    quantize() + attention() (Q through the FP8 quantizer), each with the pipeline's workspace,
    and the single pass of both without one."""
    o_f = m.forward(*x).clone()
    st_f = m.buf.stats.clone()
    m.quantize(*x)
    o_u = m.attention().clone()
    st_u = m.buf.stats.clone()
    b = m.buf
    sc = [m.scales[n][0] for n in "qkv"]
    o1_f, o1_u = torch.empty_like(b.o), torch.empty_like(b.o)
    kq.kq_attn_quant_fwd_qbf16(x[0], m.scales["q"][1], b.k8, b.v8t, *sc, m.sm_scale, o1_f, None)
    kq.kq_attn_quant_fwd(b.q8, b.k8, b.v8t, *sc, m.sm_scale, o1_u)
    torch.cuda.synchronize()
    assert torch.equal(o_f, o_u) and torch.equal(st_f, st_u)
    assert torch.equal(o1_f, o1_u)
    return o_f


@pytest.mark.parametrize("case", ["cfg1", "ragged300", "q_past_calibration", "cfg3"])
def test_fused_q_quantization_equals_the_quantizer(case):
    """FP8 mode's forward() quantizes Q inside the attention kernel (kq_attn_quant_fwd_qbf16)
    with the FP8 quantizer's conversion, so O and the row statistics equal, bit for bit, those of
    quantizing Q first: single pass and key split (cfg3's last round), ragged N, and Q scaled
    past its calibrated amax so that both sides clamp codes at +-448."""
    print(f"fused Q quantization: {case}", flush=True)
    bits = (W.qkv_bits(1) if case == "cfg1" else W.qkv_bits(3) if case == "cfg3"
            else _scaled_bits(1.0, 1.0, 2300 if case == "ragged300" else 2400))
    x = [to_dev(b) for b in bits]
    B, H, N, d = x[0].shape
    m = QuantizedSDPA(B, H, N, d, want_stats=True)
    assert m.fuse_q
    m.calibrate(*x)
    if case == "q_past_calibration":
        x[0] = x[0] * 4                          # exact in bf16; |q| * inv reaches 4 * 448
    _fused_vs_unfused(m, x)
    if case == "q_past_calibration":
        q8 = m.buf.q8.cpu().numpy()
        assert np.any((q8 & 0x7F) == 0x7E), "no code clamped at 448"


def test_fused_q_every_bf16_value():
    """Q holding every finite bf16 value (65280 of them, both signs, subnormals, values far past
    the clamp) in a 512 x 128 tile: the in-kernel codes equal the quantizer's, so the fused and
    the unfused attention agree bit for bit."""
    bits = np.arange(65536, dtype=np.uint16)
    bits = bits[(bits & 0x7F80) != 0x7F80]                      # drop Inf and NaN
    rng = np.random.default_rng(11)
    qb = np.concatenate([bits, rng.choice(bits, 512 * 128 - bits.size)])
    rng.shuffle(qb)
    qb = qb.reshape(1, 1, 512, 128)
    kb = W.random_bits(1, 1, 512, 128, seed=2500, outliers=True)
    vb = W.random_bits(1, 1, 512, 128, seed=2501, outliers=True)
    x = [to_dev(b) for b in (qb, kb, vb)]
    m = QuantizedSDPA(1, 1, 512, 128, want_stats=True)
    m.calibrate(x[1], x[1], x[2])                # Q's scale from K's amax: most of Q clamps
    _fused_vs_unfused(m, x)

