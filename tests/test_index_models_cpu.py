"""CPU models of five kernels' index schemes, with bounds asserted (no GPU).

Each model replays one kernel's addressing in Python -- the same tile plan,
the same LDS layout, the same per-lane offsets -- with every LDS and buffer
access checked against its bounds and every read checked to hit a slot that
was written, and the result it assembles compared with the definition (the
oracle, or the column matrix written out).  A wrong offset, a missed halo
column or an out-of-range read fails here before any GPU run.

* `im2col_staged_kernel` (kernels_im2col.hip): the chunk plan of
  `staged_plan` (32 KB of LDS rows, the pitch W + 2*(W/64) + 2 halves,
  element j at j + 2*(j/64)), the rows a chunk of L output pixels needs, and
  the column-matrix pieces it writes (rows k >= K zero), against the column
  matrix from its definition.
* `wgrad_tap_kernel` (kernels_backward.hip): the band plan of
  `tap_plan` (80 KB per block less the 48 KB G ring and the plane skew), the
  KW column-shifted copies of 16 channel planes (plane pitch R*OW + 8 halves),
  cut from the three 16-byte pieces around each copy piece, the per-tap
  offsets and the 32-pixel step walk, against the oracle's weight gradient.

* `dwm_kernel` (kernels_dwmfma.hip): the banded-MFMA depthwise plan, the
  input chunks in the double-buffered LDS planes, the zero-padded Toeplitz
  table and the lane fragments, the MFMA operand layouts, the fp16 stage and
  the 16-byte store pieces, against the oracle.
* `halo32_kernel` in its depth-stepped form (kernels_halo32.hip): the tile
  and box choice, the loader items of one input depth plane, the phase-split
  LDS positions and the per-tap offsets, for first, middle and last tiles
  along every axis, against X itself (zero outside); and its epilogue's
  paired whole-line stores (two pixel tiles exchanged by 8-lane row shifts),
  every output written once with its own value.
* `pw_kernel` over a flat pixel axis (kernels_pointwise.hip, the explicit
  im2col route's GEMM): pixel tiles over all images' padded column rows, the
  producer's per-octet image split and the epilogue's per-group image offset,
  against the column-matrix product.

The constants below are the kernels' own (kTapCT, kTapLds, kTapRingBytes,
kMaxLds, kTrow, kLdc and the 32 KB stage): a change there must change them
here.
"""
import itertools

import numpy as np
import pytest

from oracle import backward as obwd
from oracle import oracle

# ---------------------------------------------------------------- im2col

IM2COL_STAGE_BYTES = 32 * 1024


def _pad3(v, d):
    return [d] * (3 - len(v)) + list(v)


def _im2col_geo(xs, ws, attrs):
    nsp = len(xs) - 2
    st = attrs.get("strides", [1] * nsp)
    dl = attrs.get("dilations", [1] * nsp)
    pads = attrs.get("pads", [0] * (2 * nsp))
    out, pb = oracle.output_dims(list(xs[2:]), list(ws[2:]), st, dl, "NOTSET", pads)
    D, H, W = _pad3(xs[2:], 1)
    OD, OH, OW = _pad3(out, 1)
    KD, KH, KW = _pad3(ws[2:], 1)
    sd, sh, sw = _pad3(st, 1)
    dd, dh, dw = _pad3(dl, 1)
    pd, ph, pw = _pad3(pb, 0)
    G = attrs.get("group", 1)
    return dict(n=xs[0], C=xs[1], G=G, Cg=xs[1] // G, D=D, H=H, W=W, OD=OD, OH=OH, OW=OW,
                KD=KD, KH=KH, KW=KW, sd=sd, sh=sh, sw=sw, dd=dd, dh=dh, dw=dw, pd=pd, ph=ph, pw=pw)


def _staged_plan(cp, Pp):
    pitch = cp["W"] + 2 * (cp["W"] >> 6) + 2
    rows = IM2COL_STAGE_BYTES // (pitch * 2)
    if rows < 2:
        return None
    lmax = (rows - 2) * cp["OW"] + 1
    L = min(lmax // 8 * 8, 4096, Pp)
    if L < 8:
        return None
    rows = min(rows, (L - 1) // cp["OW"] + 2)
    return dict(L=L, nchunk=-(-Pp // L), rows=rows, pitch=pitch)


IM2COL_CASES = [
    ([2, 3, 64, 64], [96, 3, 4, 4], dict(strides=[4, 4])),
    ([1, 3, 224, 224], [64, 3, 16, 16], dict(strides=[16, 16])),
    ([1, 8, 28, 28], [32, 8, 14, 14], dict(strides=[14, 14])),
    ([1, 12, 32, 32], [64, 12, 3, 3], dict(pads=[1, 1, 1, 1])),
    ([2, 3, 20, 20], [16, 3, 3, 3], dict(pads=[1, 1, 1, 1])),
    ([1, 32, 8, 8], [64, 8, 3, 3], dict(group=4, pads=[1, 1, 1, 1])),
    ([1, 8, 8, 16, 16], [32, 8, 2, 4, 4], dict(strides=[2, 4, 4])),
    ([3, 4, 96], [16, 4, 5], dict(strides=[2], pads=[2, 2])),
    ([1, 3, 20, 20], [16, 3, 5, 5], dict(dilations=[2, 2])),
    ([1, 16, 30, 30], [24, 16, 5, 5], dict(strides=[5, 5])),
    ([1, 1, 40, 1100], [8, 1, 3, 3], dict(pads=[1, 1, 1, 1])),      # wide rows: several chunks
    ([1, 1, 9, 5000], [8, 1, 2, 3], dict(strides=[1, 2], pads=[0, 1, 0, 1])),
    ([1, 2, 4, 20, 30], [8, 2, 3, 3, 3], dict(pads=[1, 1, 1, 1, 1, 1], strides=[1, 2, 2])),
]


@pytest.mark.parametrize("ci", range(len(IM2COL_CASES)))
def test_im2col_staged_index_model(ci):
    xs, ws, attrs = IM2COL_CASES[ci]
    cp = _im2col_geo(xs, ws, attrs)
    K = cp["Cg"] * cp["KD"] * cp["KH"] * cp["KW"]
    Kp = max(16, -(-K // 8) * 8)
    P = cp["OD"] * cp["OH"] * cp["OW"]
    Pp = -(-P // 8) * 8
    sg = _staged_plan(cp, Pp)
    assert sg is not None, "every case here takes the staged kernel"
    x = np.random.default_rng([7400, ci]).standard_normal(xs)
    x3 = x.reshape(cp["n"], cp["C"], cp["D"], cp["H"], cp["W"])
    col = np.full((cp["n"] * cp["G"], Kp, Pp), np.nan)
    skew = lambda j: j + 2 * (j >> 6)
    for ng in range(cp["n"] * cp["G"]):
        n, g = divmod(ng, cp["G"])
        for c, kd, kh, chunk in itertools.product(range(cp["Cg"]), range(cp["KD"]), range(cp["KH"]),
                                                  range(sg["nchunk"])):
            P0 = chunk * sg["L"]
            Pend = min(P0 + sg["L"], Pp)
            Pv = min(Pend, P)
            assert P0 < P
            R0 = P0 // cp["OW"]
            nrows = (Pv - 1) // cp["OW"] - R0 + 1
            assert nrows <= sg["rows"], (nrows, sg)
            lds = np.full(sg["rows"] * sg["pitch"], np.nan)
            for r in range(nrows):            # the chunk's input rows, staged
                od, oh = divmod(R0 + r, cp["OH"])
                idd = od * cp["sd"] - cp["pd"] + kd * cp["dd"]
                ih = oh * cp["sh"] - cp["ph"] + kh * cp["dh"]
                ok = 0 <= idd < cp["D"] and 0 <= ih < cp["H"]
                for j in range(cp["W"]):
                    a = r * sg["pitch"] + skew(j)
                    assert skew(j) < sg["pitch"] and a < lds.size
                    lds[a] = x3[n, g * cp["Cg"] + c, idd, ih, j] if ok else 0.0
            kbase = ((c * cp["KD"] + kd) * cp["KH"] + kh) * cp["KW"]
            for kw in range(cp["KW"]):        # one 8-pixel piece per lane
                for o in range((Pend - P0) // 8):
                    p0 = P0 + 8 * o
                    R, ow = divmod(p0, cp["OW"])
                    v = np.zeros(8)
                    for e in range(8):
                        if p0 + e < Pv:
                            iw = ow * cp["sw"] + kw * cp["dw"] - cp["pw"]
                            if 0 <= iw < cp["W"]:
                                a = (R - R0) * sg["pitch"] + skew(iw)
                                assert not np.isnan(lds[a]), "read of an unstaged LDS slot"
                                v[e] = lds[a]
                        ow += 1
                        if ow == cp["OW"]:
                            ow, R = 0, R + 1
                    assert p0 + 8 <= Pp
                    col[ng, kbase + kw, p0:p0 + 8] = v
        for chunk in range(sg["nchunk"]):     # rows K .. Kp-1 written as zeros
            P0 = chunk * sg["L"]
            col[ng, K:Kp, P0:P0 + min(sg["L"], Pp - P0)] = 0
    assert not np.isnan(col).any(), "unwritten column-matrix entries"
    ref = np.zeros_like(col)                  # the column matrix from its definition
    for ng in range(cp["n"] * cp["G"]):
        n, g = divmod(ng, cp["G"])
        for k in range(K):
            c, rem = divmod(k, cp["KD"] * cp["KH"] * cp["KW"])
            kd, rem = divmod(rem, cp["KH"] * cp["KW"])
            kh, kw = divmod(rem, cp["KW"])
            for p in range(P):
                R, ow = divmod(p, cp["OW"])
                od, oh = divmod(R, cp["OH"])
                idd = od * cp["sd"] - cp["pd"] + kd * cp["dd"]
                ih = oh * cp["sh"] - cp["ph"] + kh * cp["dh"]
                iw = ow * cp["sw"] - cp["pw"] + kw * cp["dw"]
                if 0 <= idd < cp["D"] and 0 <= ih < cp["H"] and 0 <= iw < cp["W"]:
                    ref[ng, k, p] = x3[n, g * cp["Cg"] + c, idd, ih, iw]
    assert np.array_equal(col, ref), np.argwhere(col != ref)[:5]


# ------------------------------------------------------------ weight taps

TAP_CT = 16                      # kTapCT: input channels per block
TAP_LDS = 80 * 1024              # kTapLds
TAP_RING = 4 * 3 * 4 * 64 * 16   # kTapRingBytes: 4 waves x 3 steps x 4 tiles x 1 KB

TAP_CASES = [
    ([1, 16, 16, 16], [2, 16, 3, 3], (1, 1, 1, 1), (1, 1), TAP_LDS),
    ([1, 16, 8, 64], [1, 16, 1, 3], (0, 1, 0, 1), (1, 1), TAP_LDS),
    ([1, 16, 16, 16], [1, 16, 3, 3], (2, 2, 2, 2), (2, 2), TAP_LDS),
    ([1, 16, 40, 48], [1, 16, 3, 3], (1, 1, 1, 1), (1, 1), TAP_RING + 16 * 1024),  # one-row bands
    ([1, 16, 18, 16], [1, 16, 3, 3], (0, 1, 0, 1), (1, 1), TAP_LDS),
    ([1, 16, 1, 64], [1, 16, 1, 5], (0, 2, 0, 2), (1, 1), TAP_LDS),
    ([2, 32, 8, 24], [2, 32, 3, 3], (1, 1, 1, 1), (1, 1), TAP_LDS),
]


@pytest.mark.parametrize("ci", range(len(TAP_CASES)))
def test_wgrad_tap_index_model(ci):
    xs, ws, pads, dil, lds_bytes = TAP_CASES[ci]
    n, C, H, W = xs
    M, Cg, KH, KW = ws
    ph, pw, phe, pwe = pads
    dh, dw = dil
    OH = H + ph + phe - (KH - 1) * dh
    OW = W + pw + pwe - (KW - 1) * dw
    assert W % 8 == 0 and OW % 8 == 0 and Cg % TAP_CT == 0 and pw <= 8 and (KW - 1) * dw - pw <= 8
    per_row = TAP_CT * KW * OW * 2
    skew_bytes = TAP_CT * KW * 8 * 2
    span = (KH - 1) * dh
    rmax = (lds_bytes - TAP_RING - skew_bytes) // per_row
    assert rmax >= span + 1
    BR = min(OH, rmax - span)                 # output rows per band
    R = BR + span                             # input rows a band needs
    nband = -(-OH // BR)
    assert R * per_row + skew_bytes + TAP_RING <= lds_bytes
    taps = KH * KW
    rng = np.random.default_rng([7500, ci])
    x = rng.standard_normal(xs)
    g = rng.standard_normal([n, M, OH, OW])
    dwo = np.zeros([M, Cg * taps])
    W8, OW8 = W // 8, OW // 8
    CP = R * OW + 8                           # plane pitch (halves)
    toff = [(t % KW) * TAP_CT * CP + (t // KW) * dh * OW for t in range(taps)]
    for ct in range(Cg // TAP_CT):
        c0 = ct * TAP_CT
        for nn, band in itertools.product(range(n), range(nband)):
            oh0 = band * BR
            cpy = np.full(KW * TAP_CT * CP, np.nan)
            for i in range(TAP_CT * R * OW8):    # one 8-column piece per item
                c, r2 = divmod(i, R * OW8)
                rr, u = divmod(r2, OW8)
                ih = oh0 - ph + rr
                rok = 0 <= ih < H
                pieces = [x[nn, c0 + c, ih, 8 * pu:8 * pu + 8] if (rok and 0 <= pu < W8) else np.zeros(8)
                          for pu in (u - 1, u, u + 1)]
                win = np.concatenate(pieces)
                for kw in range(KW):
                    s = kw * dw - pw
                    assert -8 <= s <= 8
                    dst = c * CP + rr * OW + 8 * u + kw * TAP_CT * CP
                    assert dst + 8 <= cpy.size
                    cpy[dst:dst + 8] = win[8 + s:16 + s]
            bandpix = min(BR, OH - oh0) * OW
            for m in range(M):
                for q in range(4):               # lane group q: pixels 8q.. of each 32-pixel step
                    r, ow = divmod(8 * q, OW)
                    for st in range(-(-bandpix // 32)):
                        p = st * 32 + 8 * q
                        if p < bandpix:
                            a = g[nn, m].ravel()[oh0 * OW + p: oh0 * OW + p + 8]
                            for cc in range(TAP_CT):
                                cb = cc * CP + r * OW + ow
                                for t in range(taps):
                                    o = cb + toff[t]
                                    assert o + 8 <= cpy.size
                                    bv = cpy[o:o + 8]
                                    assert not np.isnan(bv).any(), "read of an unwritten copy slot"
                                    dwo[m, (c0 + cc) * taps + t] += a @ bv
                        ow += 32
                        while ow >= OW:
                            ow -= OW
                            r += 1
    ref = obwd.conv_backward_weight(x, g, ws, pads=[ph, pw, phe, pwe], dilations=list(dil))
    err = np.max(np.abs(dwo.reshape(ref.shape) - ref))
    assert err < 1e-9, err


# --------------------------------------------------- banded-MFMA depthwise

DWM_THREADS = 256            # kThreads
DWM_MAX_CHUNKS = 2           # kMaxChunks
DWM_MAX_LDS = 80 * 1024      # kMaxLds
DWM_RG = 4                   # kRG
DWM_TROW, DWM_TBASE = 64, 24  # kTrow, kTbase

DWM_CASES = [
    # (x, w, attrs): the two depthwise workloads' planes and the GPU test shapes
    ([1, 2, 56, 56], [2, 1, 7, 7], dict(group=2, auto_pad="SAME_UPPER")),
    ([1, 2, 56, 56], [2, 1, 7, 7], dict(group=2, auto_pad="SAME_UPPER", dilations=[2, 2])),
    ([1, 2, 16, 24], [4, 1, 5, 5], dict(group=2, auto_pad="SAME_LOWER")),
    ([1, 1, 31, 40], [1, 1, 3, 3], dict(group=1, dilations=[2, 1], pads=[2, 4, 3, 6])),
    ([1, 1, 13, 64], [1, 1, 7, 3], dict(group=1, dilations=[1, 2], pads=[3, 2, 3, 2])),
    ([1, 1, 20, 32], [1, 1, 3, 17], dict(group=1, auto_pad="SAME_UPPER")),
    ([1, 1, 18, 16], [1, 1, 5, 9], dict(group=1, dilations=[1, 2], auto_pad="SAME_UPPER")),
    ([1, 1, 8, 8], [1, 1, 3, 3], dict(group=1, auto_pad="SAME_LOWER")),
    ([1, 1, 61, 48], [1, 1, 7, 7], dict(group=1, pads=[0, 11, 0, 3])),
    ([1, 1, 8, 16], [1, 1, 3, 3], dict(group=1, pads=[1, 1, 1, 1])),
    ([1, 1, 100, 40], [1, 1, 5, 5], dict(group=1, auto_pad="SAME_UPPER")),   # two row groups
]


def _dwm_plan(cp):
    """dwm_try: the kernel's geometry, or None where it does not fit."""
    S = (8 - cp["pw"] % 8) % 8
    if S + 16 + cp["dw"] * (cp["KW"] - 1) > 32:
        return None
    TW = -(-cp["OW"] // 16)
    TV = -(-cp["OH"] // (16 * DWM_RG))
    pitch = 16 * (TW - 1) + 32 + 8
    if cp["W"] + cp["pw"] + S > pitch - 8:
        return None
    NR = 16 * DWM_RG * TV + cp["dh"] * (cp["KH"] - 1)
    bufh = -(-(NR * pitch + 8 * ((NR + 3) // 4)) // 8) * 8
    sp = 16 * TW + 8
    stgh = 64 * TV * sp + 8 * 16 * TV
    no = cp["OH"] * cp["OW"] // 8
    if no > 2 * DWM_THREADS:
        return None
    lds = (2 * bufh * 2 + 2 * stgh * 2 + -(-(cp["KH"] * cp["KW"] * 2) // 16) * 16
           + 2 * cp["KH"] * DWM_TROW * 2 + 16)
    xch = cp["H"] * cp["W"] // 8
    if lds > DWM_MAX_LDS or xch > DWM_MAX_CHUNKS * DWM_THREADS:
        return None
    return dict(S=S, TW=TW, TV=TV, pitch=pitch, NR=NR, bufh=bufh, sp=sp, stgh=stgh, no=no, xch=xch,
                nitem=TV * TW)


def _dwm_geo(xs, ws, attrs):
    # 2-D geometry with the auto_pad rules resolved by the oracle
    dl = attrs.get("dilations", [1, 1])
    out, pb = oracle.output_dims(list(xs[2:]), list(ws[2:]), [1, 1], dl,
                                 attrs.get("auto_pad", "NOTSET"), attrs.get("pads", [0] * 4))
    return dict(H=xs[2], W=xs[3], OH=out[0], OW=out[1], KH=ws[2], KW=ws[3], dh=dl[0], dw=dl[1],
                ph=pb[0], pw=pb[1])


@pytest.mark.parametrize("ci", range(len(DWM_CASES)))
def test_dwm_depthwise_index_model(ci):
    xs, ws, attrs = DWM_CASES[ci]
    cp = _dwm_geo(xs, ws, attrs)
    assert cp["W"] % 8 == 0 and cp["OW"] % 8 == 0
    f = _dwm_plan(cp)
    assert f is not None, "every case here takes the banded-MFMA kernel"
    pitch, S, bufh, sp = f["pitch"], f["S"], f["bufh"], f["sp"]
    in_row = lambda r, pt=pitch: r * pt + 8 * (r >> 2)
    rng = np.random.default_rng([7420, ci])
    x = rng.standard_normal(xs)
    w = rng.standard_normal(ws)
    bias = rng.standard_normal(ws[0])
    M, Mg = ws[0], ws[0] // xs[1]
    out_sz = cp["OH"] * cp["OW"]
    ref = oracle.fusedconv(x, w, bias, None, **attrs)
    KH, KW, dh, dw = cp["KH"], cp["KW"], cp["dh"], cp["dw"]
    cw8 = cp["W"] // 8
    for n, m in itertools.product(range(xs[0]), range(M)):
        # both LDS buffers zeroed once; this plane goes into buffer b
        b = (n + m) & 1
        lds = np.zeros(2 * bufh)
        plane = x[n, m // Mg].reshape(-1)
        for tid, kk in itertools.product(range(DWM_THREADS), range(DWM_MAX_CHUNKS)):
            c = tid + kk * DWM_THREADS
            cc = min(c, f["xch"] - 1)
            row, col = divmod(cc, cw8)
            dst = in_row(row + cp["ph"]) + col * 8 + cp["pw"] + S
            assert col * 8 + 7 + cp["pw"] + S < pitch and dst + 8 <= bufh
            lds[b * bufh + dst:b * bufh + dst + 8] = plane[cc * 8:cc * 8 + 8]
        # zero-padded kernel rows, two copies one half apart
        wk = w[m, 0]
        trow = np.zeros(2 * KH * DWM_TROW)
        for idx in range(2 * KH * DWM_TROW):
            cpy, r = divmod(idx, KH * DWM_TROW)
            kh, i = divmod(r, DWM_TROW)
            d = i + cpy - DWM_TBASE
            if d >= 0 and d % dw == 0 and d // dw < KW:
                trow[idx] = wk[kh, d // dw]
        # A operand: lane (j, q) holds T_kh[j][8q .. 8q+7]
        A = np.zeros((KH, 16, 32))
        for j, q in itertools.product(range(16), range(4)):
            i0 = DWM_TBASE + 8 * q - j - S
            assert 0 <= i0 and i0 + 8 <= DWM_TROW
            base = (i0 & 1) * KH * DWM_TROW + 2 * (i0 >> 1)
            for kh in range(KH):
                A[kh, j, 8 * q:8 * q + 8] = trow[base + kh * DWM_TROW:base + kh * DWM_TROW + 8]
        stage = np.full(2 * f["stgh"], np.nan)
        sb = ((n + m + 1) & 1) * f["stgh"]
        for wave in range(DWM_THREADS // 64):
          for it in range(wave, f["nitem"], 4):
            v, t = divmod(it, f["TW"])
            # B operand of input fragment s: lane (r, q) reads row 64v + 4r + s,
            # columns 16t + 8q .. +7, inside its own buffer
            frag = []
            for s in range(DWM_RG + dh * (KH - 1)):
                B = np.zeros((32, 16))
                for r, q in itertools.product(range(16), range(4)):
                    a = in_row(64 * v + 4 * r + s) + 16 * t + 8 * q
                    assert 64 * v + 4 * r + s < f["NR"] and 16 * t + 8 * q + 8 <= pitch - 8
                    assert a + 8 <= bufh
                    B[8 * q:8 * q + 8, r] = lds[b * bufh + a:b * bufh + a + 8]
                frag.append(B)
            for p in range(DWM_RG):
                D = np.full((16, 16), bias[m])
                for kh in range(KH):
                    D += A[kh] @ frag[p + dh * kh]
                # lane (r, q): 4 consecutive outputs into the stage, one 8-byte write
                for r, q in itertools.product(range(16), range(4)):
                    row, oc = 64 * v + 4 * r + p, 16 * t + 4 * q
                    a = in_row(row, sp) + oc
                    assert a % 4 == 0 and oc + 4 <= sp - 8 and a + 4 <= f["stgh"]
                    stage[sb + a:sb + a + 4] = D[4 * q:4 * q + 4, r]
        # the stage to Y: piece o (8 outputs), lanes past the last piece dropped
        y = np.full(out_sz, np.nan)
        writes = np.zeros(out_sz, dtype=int)
        ow8 = cp["OW"] // 8
        for tid, kk in itertools.product(range(DWM_THREADS), range(2)):
            o = tid + kk * DWM_THREADS
            oc = min(o, f["no"] - 1)
            row, col = divmod(oc, ow8)
            a = in_row(row, sp) + col * 8
            assert a % 8 == 0 and a + 8 <= f["stgh"]
            piece = stage[sb + a:sb + a + 8]
            assert not np.isnan(piece).any(), "read of an unwritten stage slot"
            if o < f["no"]:
                y[oc * 8:oc * 8 + 8] = piece
                writes[oc * 8:oc * 8 + 8] += 1
        assert (writes == 1).all(), "every output stored exactly once"
        np.testing.assert_allclose(y.reshape(cp["OH"], cp["OW"]), ref[n, m], rtol=1e-12, atol=1e-12)
        # the exact loop for planes with a non-finite input, same buffer
        for oh, ow in itertools.product(range(cp["OH"]), range(cp["OW"])):
            s = bias[m]
            for kh, kw in itertools.product(range(KH), range(KW)):
                a = in_row(oh + dh * kh) + ow + dw * kw + S
                assert a < bufh
                s += lds[b * bufh + a] * wk[kh, kw]
            assert abs(s - ref[n, m, oh, ow]) <= 1e-12 * max(1.0, abs(s))


# ------------------------------------------------- fp32 halo, depth-stepped

H32_LDC, H32_CB, H32_MAX_LDS, H32_MAX_TAPS = 20, 16, 64 * 1024, 64  # kLdc, kCB, kMaxLds, kMaxTaps

H32_DS_CASES = [
    # (x, w, strides, pads, dilations): 3-D convs whose full-depth box does not fit
    ([1, 16, 32, 64, 64], [128, 16, 3, 3, 3], [1, 2, 2], [1] * 6, [1, 1, 1]),  # the 3-D workload's planes
    ([1, 32, 6, 16, 16], [48, 32, 3, 3, 3], [1, 1, 1], [1] * 6, [1, 1, 1]),
    ([2, 20, 5, 24, 40], [24, 20, 3, 3, 3], [2, 2, 2], [1, 0, 1, 2, 1, 0], [1, 1, 1]),
    ([1, 16, 7, 30, 30], [32, 16, 3, 5, 5], [1, 2, 2], [0, 2, 2, 1, 2, 2], [2, 1, 1]),
]


def _h32_choose(cp, wgp, ds):
    """choose32_wgp: tile, box and per-box tap offsets, or None."""
    cd = lambda a, b: -(-a // b)
    bn = 64 * wgp
    order = []
    for w in (16, 32, 64, 128, 256):
        if w > bn:
            break
        th = bn // w
        if th > 1 and cp["OH"] == 1 and cp["OD"] == 1:
            continue
        order.append((cd(cp["OH"], th) * th * cd(cp["OW"], w) * w / (cp["OH"] * cp["OW"]), -w, w))
    for _, _, tw in sorted(order):
        th = bn // tw
        h = dict(TH=th, TW=tw, taps2=cp["KH"] * cp["KW"] if ds else cp["KD"] * cp["KH"] * cp["KW"])
        BD = 1 if ds else (cp["KD"] - 1) * cp["dd"] + 1
        BH = (th - 1) * cp["sh"] + (cp["KH"] - 1) * cp["dh"] + 1
        BW = (tw - 1) * cp["sw"] + (cp["KW"] - 1) * cp["dw"] + 1
        h.update(BH=BH, BW=BW, ND=1 if ds else cd(BD, cp["sd"]), NH=cd(BH, cp["sh"]), NW=cd(BW, cp["sw"]))
        h.update(LH=cp["sh"] * h["NH"], LW=cp["sw"] * h["NW"])
        bpos = (1 if ds else cp["sd"]) * h["ND"] * h["LH"] * h["LW"]
        if (1 if ds else 2) * bpos * H32_LDC * 4 > H32_MAX_LDS:
            continue
        if cd(cp["OH"], th) * th * cd(cp["OW"], tw) * tw > 2.0 * cp["OH"] * cp["OW"]:
            continue
        h["box_pos"] = bpos
        h["tap_off"] = []
        for t in range(h["taps2"]):
            kw, kh, kd = t % cp["KW"], (t // cp["KW"]) % cp["KH"], 0 if ds else t // (cp["KW"] * cp["KH"])
            ad, ah, aw = kd * cp["dd"], kh * cp["dh"], kw * cp["dw"]
            h["tap_off"].append((((ad % cp["sd"]) * h["ND"] + ad // cp["sd"]) * h["LH"] + (ah % cp["sh"]) * h["NH"]
                                 + ah // cp["sh"]) * h["LW"] + (aw % cp["sw"]) * h["NW"] + aw // cp["sw"])
        return h
    return None


@pytest.mark.parametrize("ci", range(len(H32_DS_CASES)))
def test_halo32_depth_stepped_index_model(ci):
    xs, ws, st, pads, dl = H32_DS_CASES[ci]
    C, D, H, W = xs[1:]
    M, Cg, KD, KH, KW = ws
    out, pb = oracle.output_dims([D, H, W], [KD, KH, KW], st, dl, "NOTSET", pads)
    cp = dict(D=D, H=H, W=W, OD=out[0], OH=out[1], OW=out[2], KD=KD, KH=KH, KW=KW, sd=st[0], sh=st[1],
              sw=st[2], dd=dl[0], dh=dl[1], dw=dl[2], pd=pb[0], ph=pb[1], pw=pb[2])
    wgps = [4, 2] if M <= 64 else [2]
    taps = KD * KH * KW
    full = None if taps > H32_MAX_TAPS else next((h for g in wgps if (h := _h32_choose(cp, g, False))), None)
    assert full is None, "every case here needs the depth-stepped form"
    h = next((h for g in wgps if (h := _h32_choose(cp, g, True))), None)
    assert h is not None and h["taps2"] <= H32_MAX_TAPS
    ph = lambda a, s, n: a if s == 1 else (a % s) * n + a // s
    x = np.random.default_rng([7440, ci]).standard_normal((C, D, H, W))
    box = h["box_pos"] * H32_LDC
    tiles_h, tiles_w = -(-cp["OH"] // h["TH"]), -(-cp["OW"] // h["TW"])
    # first, last and a middle tile along each axis
    pick = lambda n: sorted({0, n // 2, n - 1})
    for od0, th_i, tw_i in itertools.product(pick(cp["OD"]), pick(tiles_h), pick(tiles_w)):
        oh0, ow0 = th_i * h["TH"], tw_i * h["TW"]
        bh0, bw0, z0 = oh0 * cp["sh"] - cp["ph"], ow0 * cp["sw"] - cp["pw"], od0 * cp["sd"] - cp["pd"]
        kds = [kd for kd in range(KD) if 0 <= z0 + kd * cp["dd"] < D]   # planes inside the input
        h_lo, h_hi = max(bh0, 0), min(bh0 + h["BH"], H)
        w_lo, w_hi = max(bw0, 0), min(bw0 + h["BW"], W)
        g_lo, g_hi = w_lo >> 2, (w_hi + 3) >> 2
        nh, ngr = max(h_hi - h_lo, 0), max(g_hi - g_lo, 0)
        for cb, kd in itertools.product(range(-(-Cg // H32_CB)), kds):
            idd = z0 + kd * cp["dd"]
            lds = np.zeros(box)
            for i in range(4 * nh * ngr):             # loader items: (channel quad, row, 4 columns)
                cq, r = i & 3, i >> 2
                gi, hh = r % ngr, r // ngr
                ih, iw = h_lo + hh, (g_lo + gi) * 4
                ldst = ph(ih - bh0, cp["sh"], h["NH"]) * h["LW"]
                for e in range(4):
                    if w_lo <= iw + e < w_hi:
                        a = (ldst + ph(iw + e - bw0, cp["sw"], h["NW"])) * H32_LDC + cq * 4
                        assert a + 4 <= box
                        c = cb * H32_CB + cq * 4 + np.arange(4)
                        lds[a:a + 4] = np.where(c < Cg, x[np.minimum(c, Cg - 1), idd, ih, iw + e], 0.0)
            ncb = min(H32_CB, Cg - cb * H32_CB)
            for pu in range(h["TH"] * h["TW"]):       # every pixel, every in-plane tap
                th, tw = divmod(pu, h["TW"])
                oh, ow = oh0 + th, ow0 + tw
                if oh >= cp["OH"] or ow >= cp["OW"]:
                    continue
                for t2 in range(h["taps2"]):
                    kw, kh = t2 % KW, t2 // KW
                    p = th * h["LW"] + tw + h["tap_off"][t2]
                    assert (p + 1) * H32_LDC <= box
                    ih, iw = oh * cp["sh"] - cp["ph"] + kh * cp["dh"], ow * cp["sw"] - cp["pw"] + kw * cp["dw"]
                    got = lds[p * H32_LDC:p * H32_LDC + ncb]
                    if 0 <= ih < H and 0 <= iw < W:
                        want = x[cb * H32_CB:cb * H32_CB + ncb, idd, ih, iw]
                    else:
                        want = np.zeros(ncb)
                    assert np.array_equal(got, want), (od0, th_i, tw_i, cb, kd, pu, t2)


H32_STORE_CASES = [
    # (WGP, TW, TH, OD, OH, OW, Mg, M-block count): output tiles of the fp32 halo kernel
    (4, 256, 1, 1, 1, 4096, 64, 1),    # the 1-D conv's 256-pixel rows (every pair whole)
    (2, 32, 4, 5, 32, 32, 128, 1),     # the 3-D conv's 4 x 32 tiles
    (4, 64, 4, 1, 30, 56, 40, 2),      # last tile column 8 wide (pairs cut), Mg < the tile's rows
    (2, 16, 8, 2, 9, 20, 100, 1),      # TW = 16: tiles 2k, 2k+1 are different rows (no pairing)
    (4, 128, 2, 1, 3, 130, 70, 2),     # OW % 4 != 0: the lane-by-lane path throughout
]


@pytest.mark.parametrize("ci", range(len(H32_STORE_CASES)))
def test_halo32_paired_store_index_model(ci):
    """The fp32 halo kernel's epilogue: lane (r16, q) of wave (wpi, wmi) holds
    pixels 4q .. 4q+3 of pixel tile i for channel m0 + 64*wmi + 16j + r16.
    Where tiles 2k and 2k+1 form 32 whole pixels of one row, the row shifts by
    8 lanes (row_shr / row_shl of a 16-lane DPP row) pair them and store A
    (channels +0 .. 7) and store B (+8 .. 15) each write whole 128-byte lines;
    elsewhere every lane stores its own values.  Every output of the block must
    be written exactly once, with the value computed for that channel and
    pixel, and nothing outside the output."""
    WGP, TW, TH, OD, OH, OW, Mg, nmb = H32_STORE_CASES[ci]
    WGM, BM = 4 // WGP, 64 * (4 // WGP)
    TD = 1
    assert TW * TH == 64 * WGP
    ltw, lth = TW.bit_length() - 1, TH.bit_length() - 1
    out_sz = OD * OH * OW
    vec_y = OW % 4 == 0
    tiles = [(od0, oh0, ow0) for od0 in range(0, OD, TD) for oh0 in range(0, OH, TH) for ow0 in range(0, OW, TW)]
    for mb, (od0, oh0, ow0) in itertools.product(range(nmb), tiles):
        m0 = mb * BM
        written = {}

        def put(m, pix, val, where):
            assert 0 <= m < Mg and 0 <= pix < out_sz, where
            assert (m, pix) not in written, where
            written[(m, pix)] = val

        def pixel_of(pu):
            tw, th, td = pu & (TW - 1), (pu >> ltw) & (TH - 1), pu >> (ltw + lth)
            return od0 + td, oh0 + th, ow0 + tw

        for wave in range(4):
            wpi, wmi = wave % WGP, wave // WGP
            # acc[i][j][lane] -> the (channel, pixel) its 4 values belong to (value e: pixel + e)
            def acc(i, j, r16, q):
                pu = wpi * 64 + i * 16 + q * 4
                d, hh, w = pixel_of(pu)
                return (m0 + wmi * 64 + j * 16 + r16, (d * OH + hh) * OW + w)

            def store_tile(i):
                for r16, q in itertools.product(range(16), range(4)):
                    d, hh, w = pixel_of(wpi * 64 + i * 16 + q * 4)
                    if d >= OD or hh >= OH or w >= OW:
                        continue
                    nv = min(4, OW - w)
                    for j in range(4):
                        m, pix = acc(i, j, r16, q)
                        if m >= Mg:
                            continue
                        for e in range(4 if vec_y and nv == 4 else nv):
                            put(m, pix + e, (m, pix + e), ("tile", wave, i, j, r16, q))

            for ip in (0, 2):
                d, hh, w = pixel_of(wpi * 64 + ip * 16)
                if not (vec_y and TW >= 32 and d < OD and hh < OH and w + 32 <= OW):
                    store_tile(ip)
                    store_tile(ip + 1)
                    continue
                base = (d * OH + hh) * OW + w
                for j in range(4):
                    mrow = m0 + wmi * 64 + j * 16
                    pieces = {"A": [], "B": []}        # 16-byte pieces of each store instruction
                    for q in range(4):                 # one 16-lane DPP row per q
                        v0 = [acc(ip, j, r, q) for r in range(16)]
                        v1 = [acc(ip + 1, j, r, q) for r in range(16)]
                        down = [v1[r - 8] if r >= 8 else None for r in range(16)]   # row_shr:8
                        up = [v0[r + 8] if r < 8 else None for r in range(16)]      # row_shl:8
                        for r16 in range(16):
                            lo = r16 < 8
                            px = 4 * q if lo else 16 + 4 * q
                            for name, ch, val in (("A", mrow + (r16 if lo else r16 - 8), v0[r16] if lo else down[r16]),
                                                  ("B", mrow + (r16 + 8 if lo else r16), up[r16] if lo else v1[r16])):
                                if ch >= Mg:
                                    continue
                                pix = base + px
                                assert val == (ch, pix), (name, wave, ip, j, r16, q)
                                for e in range(4):
                                    put(ch, pix + e, (ch, pix + e), (name, wave, ip, j, r16, q))
                                pieces[name].append(ch * out_sz + pix)
                    # where the pair starts on a 128-byte boundary, each instruction's pieces
                    # make up whole lines: 8 pieces of 4 floats in every line it touches
                    if base % 32 == 0 and out_sz % 32 == 0:
                        for name in ("A", "B"):
                            per_line = {}
                            for a in pieces[name]:
                                per_line.setdefault(a // 32, set()).add(a % 32)
                            assert all(v == set(range(0, 32, 4)) for v in per_line.values()), (name, j)
        # exactly the block's outputs: channels m0 .. m0 + BM (below Mg), pixels of the tile
        want = set()
        for pu in range(64 * WGP):
            d, hh, w = pixel_of(pu)
            if d < OD and hh < OH and w < OW:
                for m in range(m0, min(m0 + BM, Mg)):
                    want.add((m, (d * OH + hh) * OW + w))
        assert set(written) == want
        assert all(v == k for k, v in written.items())


# ------------------------------------------- pointwise GEMM, flat pixel axis

PW_BN, PW_BK = 128, 64       # kBN, kBK

PW_FLAT_CASES = [
    # (n, G, Kp, P, M): column matrices of the explicit im2col route
    (256, 1, 16, 196, 64),     # the SigLIP patch embedding's pixel geometry (256 images of
                               # a 14 x 14 grid; fewer channels, the same tiles and offsets)
    (3, 2, 48, 36, 40),        # groups, P % 8 != 0 (padded rows), M not a multiple of 64
    (5, 1, 112, 1024, 64),     # P a multiple of the tile: tiles end on image boundaries
    (7, 1, 16, 4, 16),         # tiny images: many images per tile
]


@pytest.mark.parametrize("ci", range(len(PW_FLAT_CASES)))
def test_pointwise_flat_axis_index_model(ci):
    n, G, Kp, P, M = PW_FLAT_CASES[ci]
    Mg = M // G
    Pp = -(-P // 8) * 8                       # column row pitch (in_sz of the GEMM view)
    assert P % 4 == 0 and Pp % 8 == 0 and n * M * P * 2 < (1 << 31)
    ntile = -(-(n * Pp) // PW_BN)
    rng = np.random.default_rng([7460, ci])
    col = np.zeros((n, G, Kp, Pp))
    col[..., :P] = rng.standard_normal((n, G, Kp, P))   # padding columns are zeros
    w = rng.standard_normal((G, Mg, Kp))
    flat = col.reshape(-1)
    y = np.full(n * M * P, np.nan)
    writes = np.zeros(n * M * P, dtype=int)
    for g, tile in itertools.product(range(G), range(ntile)):
        p0 = tile * PW_BN
        # producer: 32 pixel octets of the tile, each from one image's column row
        a = np.zeros((Kp, PW_BN))
        for po in range(PW_BN // 8):
            pp = p0 + 8 * po
            nx, pin = divmod(pp, Pp)
            if nx >= n:
                continue                           # pix_ok false: written as zeros
            assert pin + 8 <= Pp                   # an octet never leaves its row
            off = ((nx * G + g) * Kp + np.arange(Kp)) * Pp + pin   # channel rows c
            assert off[-1] + 8 <= flat.size
            a[:, 8 * po:8 * po + 8] = flat[off[:, None] + np.arange(8)]
        acc = w[g] @ a                             # [Mg, 128]
        # epilogue: 4-pixel groups, offsets relative to y + (g*Mg + m)*P
        for q4 in range(PW_BN // 4):
            pg = p0 + 4 * q4
            nq, pin = divmod(pg, Pp)
            if not (nq < n and pin < P):
                continue                           # kOff: dropped
            assert pin + 4 <= P                    # a group is never split
            off = nq * M * P + (g * Mg + np.arange(Mg)) * P + pin      # channels m
            assert off[-1] + 4 <= y.size
            idx = off[:, None] + np.arange(4)
            y[idx] = acc[:, 4 * q4:4 * q4 + 4]
            np.add.at(writes, idx, 1)
    assert (writes == 1).all(), "every output written exactly once"
    ref = np.einsum("gmk,ngkp->ngmp", w, col[..., :P]).reshape(-1)
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)
