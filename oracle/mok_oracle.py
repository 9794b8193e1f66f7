"""CPU oracle for one mixture-of-experts layer in the Mixture-of-Kittens (MoK) style.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module.  The product path (the HIP library and its
Python binding) never calls it, and this module imports nothing from the product.

Everything here is plain NumPy in float64 (the pages fix no precision for the
reference computation), written for a reader to check against the pages by eye:
no blocking, no fusion, no reordering beyond what each definition states.

Sources (three web pages about Cursor's open-sourced Mixture-of-Kittens):
  [L]  Leiphone article "MoK：把 token 调度、跨 GPU 通信和专家计算塞进同一个 GPU 内核",
       sections 01 (MoE 的「通信税」…), 02 (怎么让 token 一边传，一边算),
       03 (一整套高度特化的执行方式)
  [M]  news brief "Cursor开源MoK：GB300 NVL72机架上的确定性MoE训练大内核",
       sections "三个重要的设计决策", "基准测试"
  [S]  setupai.cc page "Cursor 以 MoK 重寫 MoE GPU 執行方式", section "技術深入"
The MX block format follows the OCP Microscaling Formats (MX) v1.0 specification
(e4m3 element encoding, e8m0 shared scale, 32-element blocks).

What each function follows:
  schedule        [L] §01 (count each expert's tokens, choose their positions, keep one
                  expert's rows together for the grouped GEMM); [M] 三个重要的设计决策
                  (one schedule table drives all four transfers)
  dispatch        [L] §02 (the expert owner pulls rows by source position and lays them
                  out itself, already grouped by expert)
  expert_ffn      [L] §02 and [M] 三个重要的设计决策 (SwiGLU expert FFN as grouped GEMM)
  combine         [L] §02 (push each result to its known token) and §03 (the final
                  gate-weighted sum is a step of its own)
  forward         the four steps above, in order
  backward        [L] §02 (reverse-combine then reverse-dispatch) and [M] 三个重要的设计决策
                  (router-weight gradient computed inside the SwiGLU backward); the MXFP8
                  backward: [L] §03 (MXFP8 forward and backward)
  mx_quantize     [L] §02 (MXFP8 activations quantised inside dispatch, grouped GEMM
                  and SwiGLU); scale rule: the ceil reading (see ``mx_scale_exponent``)

Readings taken where the pages are silent:
  * a minibatch is M consecutive routed rows of the expert-sorted order; it may
    straddle experts and the last one may be short;
  * rows of one expert are in ascending (token, slot) order;
  * ids outside [e0, e0+n_local) are not this GPU's rows; -1 is a masked slot;
    ids < -1 or >= E are errors (flagged, skipped);
  * SwiGLU is silu(x W_gate^T) * (x W_up^T), no bias, no clamp;
  * the gate is applied in the combine, summed over slots j in ascending order;
  * tokens with no local slot get Y = 0, dX = 0 and dG = 0;
  * MXFP8 mode quantises X (along D), W_gate/W_up (along D), W_down (along I) and
    H (along I, from its float32 value); all arithmetic between those points is exact
    float64 on the dequantised values;
  * the MXFP8 backward reads a, b as the bfloat16 rows the MXFP8 forward saves, and
    quantises the operands of the two data-gradient GEMMs along their K: dY and W_down
    along D (for u), da, db (from their bfloat16 rows) and W_gate, W_up along I (for dx);
    the weight gradients and dG use unquantised values.
"""
from __future__ import annotations

import concurrent.futures as cf
import os

import numpy as np

E4M3_MAX = 448.0
E4M3_EXP_BIAS = 7
E4M3_MANT_BITS = 3
MX_BLOCK = 32
E8M0_BIAS = 127


# =================================================================================
# Schedule
# =================================================================================
class Schedule:
    """The dispatch table for one GPU's share of the routed pairs.

    counts[e]   rows routed to local expert e
    offsets[e]  first row of expert e (offsets[n_local] = R)
    perm[r]     flat pair index t*k + j held by row r
    pos[t*k+j]  row of pair (t, j), or -1 when the pair is not a local row
    row_expert[r]  local expert of row r
    bad         number of ids that are neither -1 nor in [0, E)
    """

    def __init__(self, counts, offsets, perm, pos, row_expert, bad, M):
        self.counts = counts
        self.offsets = offsets
        self.perm = perm
        self.pos = pos
        self.row_expert = row_expert
        self.bad = bad
        self.M = M

    @property
    def R(self) -> int:
        return int(self.offsets[-1])

    @property
    def n_mb(self) -> int:
        return -(-self.R // self.M) if self.R else 0

    def segments(self) -> list[tuple[int, int, int, int]]:
        """(minibatch, expert, first row, end row) for every non-empty intersection of a
        minibatch window [i*M, min((i+1)*M, R)) with an expert's rows."""
        out = []
        for i in range(self.n_mb):
            lo, hi = i * self.M, min((i + 1) * self.M, self.R)
            for e in range(len(self.counts)):
                a = max(lo, int(self.offsets[e]))
                b = min(hi, int(self.offsets[e + 1]))
                if a < b:
                    out.append((i, e, a, b))
        return out


def schedule(ids: np.ndarray, e0: int, n_local: int, E: int, M: int) -> Schedule:
    """Count each local expert's pairs, turn the counts into offsets and place every
    local pair at its expert's next free row, in ascending (token, slot) order."""
    T, k = ids.shape
    flat = ids.reshape(-1).astype(np.int64)
    bad = int(np.count_nonzero((flat < -1) | (flat >= E)))
    local = (flat >= e0) & (flat < e0 + n_local)
    pair_idx = np.nonzero(local)[0]                # ascending t*k + j
    pair_exp = flat[local] - e0
    counts = np.bincount(pair_exp, minlength=n_local).astype(np.int64)
    offsets = np.zeros(n_local + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    order = np.argsort(pair_exp, kind="stable")    # stable: keeps (token, slot) order
    perm = pair_idx[order]
    pos = np.full(T * k, -1, dtype=np.int64)
    pos[perm] = np.arange(perm.size)
    row_expert = np.repeat(np.arange(n_local), counts)
    return Schedule(counts, offsets, perm, pos, row_expert, bad, M)


# =================================================================================
# Dispatch, expert FFN, combine
# =================================================================================
def dispatch(x: np.ndarray, sch: Schedule, k: int) -> np.ndarray:
    """Row r of the expert-sorted buffer is the pool row of the token that owns pair
    perm[r]."""
    return np.asarray(x, dtype=np.float64)[sch.perm // k]


def silu(a: np.ndarray) -> np.ndarray:
    return a / (1.0 + np.exp(-a))


def sigmoid(a: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-a))


def expert_ffn(xd: np.ndarray, wg: np.ndarray, wu: np.ndarray, wd: np.ndarray):
    """SwiGLU FFN of one expert on its rows.  wg, wu: [I, D]; wd: [D, I].
    Returns (a, b, h, o): gate and up projections, h = silu(a) * b, o = h wd^T."""
    a = xd @ np.asarray(wg, np.float64).T
    b = xd @ np.asarray(wu, np.float64).T
    h = silu(a) * b
    o = h @ np.asarray(wd, np.float64).T
    return a, b, h, o


def combine(o: np.ndarray, gates: np.ndarray, sch: Schedule, T: int, k: int) -> np.ndarray:
    """Y[t] = sum over slots j (ascending) with a local row of gate[t, j] * o[row]."""
    D = o.shape[1] if o.ndim == 2 else 0
    y = np.zeros((T, D), dtype=np.float64)
    g = np.asarray(gates, np.float64)
    for j in range(k):
        rows = sch.pos.reshape(T, k)[:, j]
        has = rows >= 0
        y[has] += g[has, j][:, None] * o[rows[has]]
    return y


# =================================================================================
# MX (OCP MXFP8: e4m3 elements, e8m0 scale per 32-element block)
# =================================================================================
def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """Value of each OCP e4m3 code: sign bit, 4 exponent bits (bias 7), 3 mantissa
    bits; exponent 0 is subnormal (2^-6 * m/8); S.1111.111 is NaN; no infinities."""
    c = np.asarray(codes, dtype=np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    normal = np.ldexp(1.0 + m / 8.0, (e - E4M3_EXP_BIAS).astype(np.int64))
    sub = np.ldexp(m / 8.0, 1 - E4M3_EXP_BIAS)
    v = s * np.where(e == 0, sub, normal)
    return np.where((c & 0x7F) == 0x7F, np.nan, v)


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    """Nearest e4m3 code with ties to an even mantissa; magnitudes above 448
    saturate to 448.  The input is float32 (the precision of the kernels' scaled
    values); every step after the cast is exact in float64."""
    x = np.asarray(v, dtype=np.float32).astype(np.float64)
    sign = np.signbit(x).astype(np.int64) << 7
    a = np.minimum(np.abs(x), E4M3_MAX)
    codes = np.zeros(a.shape, dtype=np.int64)
    min_normal = 2.0 ** (1 - E4M3_EXP_BIAS)                      # 2^-6
    # subnormal range: multiples of 2^-9; rounding may land on 8 * 2^-9 = min normal
    sub = a < min_normal
    q = np.rint(a[sub] / 2.0 ** (1 - E4M3_EXP_BIAS - E4M3_MANT_BITS))   # RNE
    codes[sub] = q.astype(np.int64)            # q == 8 is exactly code 0x08 (min normal)
    nrm = ~sub
    an = a[nrm]
    ex = np.floor(np.log2(an)).astype(np.int64)
    # guard against log2 rounding at exact powers of two
    ex = np.where(np.ldexp(1.0, ex) > an, ex - 1, ex)
    ex = np.where(np.ldexp(1.0, ex + 1) <= an, ex + 1, ex)
    mant = an / np.ldexp(1.0, ex)                               # in [1, 2)
    qm = np.rint((mant - 1.0) * 8.0).astype(np.int64)          # RNE on 3 fraction bits
    carry = qm == 8
    ex = np.where(carry, ex + 1, ex)
    qm = np.where(carry, 0, qm)
    codes[nrm] = ((ex + E4M3_EXP_BIAS) << 3) | qm
    return (codes | sign).astype(np.uint8)


def mx_scale_exponent(amax: np.ndarray) -> np.ndarray:
    """Shared exponent n of a block with largest magnitude amax: the smallest n with
    amax * 2^-n <= 448, i.e. ceil(log2(amax / 448)), clamped to [-127, 127]; n = -127
    for an all-zero block.  Computed exactly: write amax = m * 2^E with m in [1, 2);
    since 448 = 1.75 * 2^8, n = E - 8 when m <= 1.75 and E - 7 otherwise."""
    a = np.asarray(amax, dtype=np.float32).astype(np.float64)
    m, e = np.frexp(a)                 # a = m * 2^e, m in [0.5, 1)
    E = e.astype(np.int64) - 1         # a = (2m) * 2^(e-1)
    mant = 2.0 * m
    n = E - 8 + (mant > 1.75).astype(np.int64)
    n = np.where(a == 0.0, -E8M0_BIAS, n)
    return np.clip(n, -E8M0_BIAS, E8M0_BIAS)


def mx_quantize(v: np.ndarray):
    """Quantise the last axis of v (a multiple of 32) in 32-element blocks.
    Returns (codes uint8, same shape as v; scales uint8, last axis / 32) where the
    scale byte is n + 127 and code = e4m3(v * 2^-n) with v read as float32."""
    x = np.asarray(v, dtype=np.float32)
    K = x.shape[-1]
    assert K % MX_BLOCK == 0, "MX blocks need the quantised axis to be a multiple of 32"
    blk = x.reshape(x.shape[:-1] + (K // MX_BLOCK, MX_BLOCK))
    amax = np.max(np.abs(blk), axis=-1)
    n = mx_scale_exponent(amax)
    scaled = blk.astype(np.float64) * np.ldexp(1.0, -n)[..., None]
    codes = e4m3_encode(scaled.astype(np.float32)).reshape(x.shape)
    return codes, (n + E8M0_BIAS).astype(np.uint8)


def mx_dequantize(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    c = e4m3_decode(codes)
    K = c.shape[-1]
    blk = c.reshape(c.shape[:-1] + (K // MX_BLOCK, MX_BLOCK))
    n = np.asarray(scales, dtype=np.int64) - E8M0_BIAS
    return (blk * np.ldexp(1.0, n)[..., None]).reshape(c.shape)


def mx_roundtrip(v: np.ndarray) -> np.ndarray:
    return mx_dequantize(*mx_quantize(v))


def bf16_round(v: np.ndarray) -> np.ndarray:
    """v rounded to float32 and then to the nearest bfloat16 (ties to even), as float64:
    the top 16 bits of the float32 pattern after adding 0x7FFF plus the lowest kept bit
    (finite values)."""
    u = np.asarray(v, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32).astype(np.float64)


# =================================================================================
# Forward and backward
# =================================================================================
def forward(x, ids, gates, wg, wu, wd, *, e0: int, E: int, M: int, mxfp8: bool = False,
            return_parts: bool = False):
    """The layer on one GPU's share: schedule, dispatch, per-expert SwiGLU FFN, combine.

    x [T, D]; ids, gates [T, k]; wg, wu [n_local, I, D]; wd [n_local, D, I].
    With ``mxfp8`` the FFN runs on MX-dequantised X (blocks along D), weights (blocks
    along each GEMM's K) and H (blocks along I, quantised from float32)."""
    T, k = ids.shape
    n_local = wg.shape[0]
    sch = schedule(ids, e0, n_local, E, M)
    xd = dispatch(x, sch, k)
    D = xd.shape[1] if xd.size else np.asarray(x).shape[1]
    I = wg.shape[1]
    a = np.zeros((sch.R, I))
    b = np.zeros((sch.R, I))
    h = np.zeros((sch.R, I))
    o = np.zeros((sch.R, D))
    for e in range(n_local):
        r0, r1 = int(sch.offsets[e]), int(sch.offsets[e + 1])
        if r0 == r1:
            continue
        xe = xd[r0:r1]
        g_w, u_w, d_w = wg[e], wu[e], wd[e]
        if mxfp8:
            xe = mx_roundtrip(xe)
            g_w, u_w, d_w = mx_roundtrip(g_w), mx_roundtrip(u_w), mx_roundtrip(d_w)
            ae = xe @ np.asarray(g_w, np.float64).T
            be = xe @ np.asarray(u_w, np.float64).T
            he = mx_roundtrip((silu(ae) * be).astype(np.float32))
            oe = he @ np.asarray(d_w, np.float64).T
        else:
            ae, be, he, oe = expert_ffn(xe, g_w, u_w, d_w)
        a[r0:r1], b[r0:r1], h[r0:r1], o[r0:r1] = ae, be, he, oe
    y = combine(o, gates, sch, T, k)
    if return_parts:
        return y, dict(schedule=sch, xd=xd, a=a, b=b, h=h, o=o)
    return y


def backward(dy, x, ids, gates, wg, wu, wd, *, e0: int, E: int, M: int, mxfp8: bool = False):
    """Gradients of the layer output with respect to x, the gates and the three
    weight tensors, for an upstream gradient dy [T, D].

    Per row r of expert e, token t, slot j (g = gates[t, j]):
      u = dy[t] W_down[e]                   (length I)
      dG[t, j] = <u, h>       — equal to <dy[t], o> without forming o
      dh = g u;  da = dh * b * s(a) (1 + a (1 - s(a)));  db = dh * silu(a)
      dW_down[e] += (g dy[t])^T h;  dW_gate[e] += da^T x;  dW_up[e] += db^T x
      dx_row = da W_gate[e] + db W_up[e];   dX[t] = sum over local slots of dx_row
    With ``mxfp8`` (the MXFP8 mode covers the backward, [L] §03): a and b are those of the
    MXFP8 forward, rounded to the bfloat16 rows it saves, and the two GEMMs that produce data gradients read MX round-tripped
    operands, each quantised along that GEMM's K: u from dy rows and W_down quantised
    along D; dx_row from da, db (rounded to bfloat16, the rows the MX quantiser reads)
    and W_gate, W_up quantised along I.  dG and the weight gradients use the
    unquantised u, h, da, db, x and dy.
    Returns dict(dx [T, D], dg [T, k], dwg, dwu [n_local, I, D], dwd [n_local, D, I])."""
    T, k = ids.shape
    n_local, I, D = wg.shape
    sch = schedule(ids, e0, n_local, E, M)
    xd = dispatch(x, sch, k)
    dy64 = np.asarray(dy, np.float64)
    g_all = np.asarray(gates, np.float64).reshape(-1)
    dxr = np.zeros((sch.R, D))
    dg = np.zeros(T * k)
    dwg = np.zeros((n_local, I, D))
    dwu = np.zeros((n_local, I, D))
    dwd = np.zeros((n_local, D, I))
    used = [e for e in range(n_local) if sch.offsets[e + 1] > sch.offsets[e]]
    wq = {}
    if mxfp8:
        # the weights' round trips: W_gate, W_up along D (the forward's a, b); W_down along
        # D (the round trip of its transpose) for u; W_gate, W_up along I for dx.  They are
        # independent, so they run side by side (NumPy releases the interpreter lock)
        mats = [(e, n, m) for e in used for n, m in
                (("g", lambda e: wg[e]), ("u", lambda e: wu[e]), ("dt", lambda e: wd[e].T),
                 ("gt", lambda e: wg[e].T), ("ut", lambda e: wu[e].T))]
        with cf.ThreadPoolExecutor(max_workers=min(16, len(os.sched_getaffinity(0)))) as ex:
            for (e, n, _), v in zip(mats, ex.map(
                    lambda t: mx_roundtrip(np.asarray(t[2](t[0]), np.float64)), mats)):
                wq[e, n] = v
    for e in used:
        r0, r1 = int(sch.offsets[e]), int(sch.offsets[e + 1])
        pairs = sch.perm[r0:r1]
        xe = xd[r0:r1]
        dye = dy64[pairs // k]
        wg_e, wu_e, wd_e = (np.asarray(w[e], np.float64) for w in (wg, wu, wd))
        if mxfp8:
            xq = mx_roundtrip(xe)
            # a and b as the MXFP8 forward saves them for the backward: bfloat16 rows
            a = bf16_round(xq @ wq[e, "g"].T)
            b = bf16_round(xq @ wq[e, "u"].T)
            h = silu(a) * b
            # W_down [D, I] quantised along D: the round trip of its transpose
            u = mx_roundtrip(dye) @ wq[e, "dt"].T
        else:
            a, b, h, _ = expert_ffn(xe, wg_e, wu_e, wd_e)
            u = dye @ wd_e
        g = g_all[pairs][:, None]
        dg[pairs] = np.sum(u * h, axis=1)
        dh = g * u
        s = sigmoid(a)
        da = dh * b * s * (1.0 + a * (1.0 - s))
        db = dh * silu(a)
        dwd[e] = (g * dye).T @ h
        dwg[e] = da.T @ xe
        dwu[e] = db.T @ xe
        if mxfp8:
            # W_gate, W_up [I, D] quantised along I: the round trips of their transposes
            dxr[r0:r1] = (mx_roundtrip(bf16_round(da)) @ wq[e, "gt"].T +
                          mx_roundtrip(bf16_round(db)) @ wq[e, "ut"].T)
        else:
            dxr[r0:r1] = da @ wg_e + db @ wu_e
    dx = np.zeros((T, D))
    pos = sch.pos.reshape(T, k)
    for j in range(k):
        rows = pos[:, j]
        has = rows >= 0
        dx[has] += dxr[rows[has]]
    return dict(dx=dx, dg=dg.reshape(T, k), dwg=dwg, dwu=dwu, dwd=dwd, schedule=sch)


# =================================================================================
# Sampled evaluation (full-size checks of selected outputs)
# =================================================================================
def forward_tokens(tokens, x, ids, gates, wg, wu, wd, *, e0: int, mxfp8: bool = False):
    """Y rows for the listed tokens only (float64), without a schedule: for each local
    expert, the listed tokens routed to it go through its FFN together; then each token's
    gated expert outputs are summed over its slots in ascending j (slots without a local
    expert add nothing).  With ``mxfp8`` the MX round trips sit where ``forward`` puts
    them: X rows and the weights along their K, H along I from float32."""
    tokens = np.asarray(tokens, dtype=np.int64)
    n_local = wg.shape[0]
    k = ids.shape[1]
    D = np.asarray(x).shape[1]
    xs = np.asarray(x, np.float64)[tokens]
    if mxfp8:
        xs = mx_roundtrip(xs)
    sel = np.asarray(ids)[tokens]
    g = np.asarray(gates, np.float64)[tokens]
    used = [e for e in range(n_local) if np.any(sel == e + e0)]
    deq = {}
    if mxfp8:
        # the weight round trips are independent: run them side by side (NumPy's array
        # operations release the interpreter lock)
        mats = [(e, n, w[e]) for e in used for n, w in (("g", wg), ("u", wu), ("d", wd))]
        with cf.ThreadPoolExecutor(max_workers=min(16, len(os.sched_getaffinity(0)))) as ex:
            for (e, n, _), v in zip(mats, ex.map(lambda m: mx_roundtrip(m[2]), mats)):
                deq[e, n] = v
    contrib = np.zeros((len(tokens), k, D))     # gated output of (listed token n, slot j)
    for e in used:
        nn, jj = np.nonzero(sel == e + e0)
        g_w, u_w, d_w = wg[e], wu[e], wd[e]
        if mxfp8:
            g_w, u_w, d_w = deq[e, "g"], deq[e, "u"], deq[e, "d"]
            a = xs[nn] @ np.asarray(g_w, np.float64).T
            b = xs[nn] @ np.asarray(u_w, np.float64).T
            h = mx_roundtrip((silu(a) * b).astype(np.float32))
            o = h @ np.asarray(d_w, np.float64).T
        else:
            _, _, _, o = expert_ffn(xs[nn], g_w, u_w, d_w)
        contrib[nn, jj] = g[nn, jj][:, None] * o
    out = np.zeros((len(tokens), D))
    for j in range(k):
        out += contrib[:, j]
    return out
