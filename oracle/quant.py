"""Oracle: rotate -> clip -> INT2 quantise -> pack (test infrastructure only).

Follows the demotion step of the serving pipeline in [ZAKER]: the oldest
recent token is rotated, clipped, quantised and packed, four 2-bit values per
byte, and moved into INT2 history.  The step order matches [CSDN] 3.1
("multiply by R, clip, INT2-quantise, store").  The rotation and the
per-layer threshold come from [GIST] 2.2A.  The scale/zero-point form is the
one [ZAKER] names for dequantisation.

Readings where the pages leave the step open:

* rotation convention: row vectors, y = x R;
* quantisation group: the d channels of one (token, KV head); the sub-head
  variant splits them into consecutive groups of g channels (g = 64 at
  d = 128), each with its own (scale, zero), which is where the bit-reversal
  permutation of [GIST] 2.2A balances the groups;
* clipping: symmetric clamp to [-tau, tau] before the group min/max;
* quantiser: asymmetric min-max with zero = fp16(min) and
  scale = fp16((max - min) / 3), code = clamp(rint((y - zero) / scale), 0, 3),
  round half to even, dequantised as zero + code * scale;
* degenerate group (scale rounds to 0): all codes 0;
* Lloyd-Max variant (the authors' repository combines the rotation with a
  Lloyd-Max codebook, [GIST] section on code availability; the pages give no
  levels): the 4-level mean-squared-error optimal quantiser of a Gaussian,
  levels +-0.4528 and +-1.5104 standard deviations, taken here in the integer
  ratio 3 : 10, LM_LEVELS = (-10, -3, 3, 10) units.  Per group: mean m and
  population standard deviation s of the clipped values in float64 (two
  passes), zero = fp16(fp32(m)), scale = fp16(fp32(LM_UNIT * s)) with
  LM_UNIT = 0.15104 (so 10 units = 1.5104 s).  With z, u the fp16 values
  widened, the decision thresholds are the midpoints t = fp32(z + u * th),
  th = (-6.5, 0, 6.5), and the code is the number of thresholds the clipped
  value reaches (y >= t).  Dequantised as zero + LM_LEVELS[code] * scale;
* pack order: byte i of a token's row holds channels 4i..4i+3, with channel
  4i+j in bits 2j..2j+1;
* in-page layout (64-token pages, one block per (page, KV head)):
  K codes are 4 planes; plane p holds bytes [p*d/16, (p+1)*d/16) of every
  token's row, token-major.  V codes are byte-column-major: byte i of token o
  sits at i*64 + o.  scale/zero are fp16 pairs (scale, zero) per token; with
  n groups per head they are group-planar: group j of token o at j*64 + o.
"""
from __future__ import annotations

import numpy as np

PAGE = 64
UNIFORM, LLOYD_MAX = "uniform", "lloyd_max"
LM_LEVELS = np.array([-10.0, -3.0, 3.0, 10.0])
LM_THRESHOLDS = np.array([-6.5, 0.0, 6.5])
LM_UNIT = 0.15104


def code_levels(codebook: str) -> np.ndarray:
    """Dequantised level of each code in units of the group scale."""
    if codebook == UNIFORM:
        return np.array([0.0, 1.0, 2.0, 3.0])
    if codebook == LLOYD_MAX:
        return LM_LEVELS.copy()
    raise ValueError("codebook must be 'uniform' or 'lloyd_max'")


def bf16_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns -> float64 (exact)."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def f16_bits_to_f64(bits) -> np.ndarray:
    """IEEE fp16 bit patterns -> float64 (exact)."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def rotate_round_f32(x_bits: np.ndarray, rot: np.ndarray) -> np.ndarray:
    """y = x R for row vectors, accumulated in float64 and rounded once to
    float32.  x_bits: bf16 [..., d]; rot: fp32 [d, d]."""
    return (bf16_to_f64(x_bits) @ np.asarray(rot, dtype=np.float32).astype(np.float64)).astype(np.float32)


def quantize_group_lloyd_max(y: np.ndarray, clip):
    """Clip and quantise the rows of y (float32 [n, d]) to the Lloyd-Max codes
    (one group per row).  Returns the same tuple as :func:`quantize_group`;
    info holds the float32 clipped values and the float64 mean and deviation."""
    y = np.asarray(y, dtype=np.float32)
    tau = np.float32(clip)
    yc = np.minimum(np.maximum(y, -tau), tau)
    y64 = yc.astype(np.float64)
    mean = y64.sum(axis=1) / y64.shape[1]
    dev = np.sqrt(((y64 - mean[:, None]) ** 2).sum(axis=1) / y64.shape[1])
    zero16 = mean.astype(np.float32).astype(np.float16)
    scale16 = (LM_UNIT * dev).astype(np.float32).astype(np.float16)
    z = zero16.astype(np.float64)[:, None]
    u = scale16.astype(np.float64)[:, None]
    codes = np.zeros(yc.shape, np.uint8)
    for th in LM_THRESHOLDS:
        t = (z + u * th).astype(np.float32)       # exact in float64, one rounding to float32
        codes += (yc >= t).astype(np.uint8)
    info = dict(yc=yc, mn=mean, mx=dev, range3=(LM_UNIT * dev).astype(np.float32))
    return codes, scale16.view(np.uint16), zero16.view(np.uint16), info


def quantize_group(y: np.ndarray, clip):
    """Clip and INT2-quantise the rows of y (float32 [n, d]); one group per row.

    Returns (codes uint8 [n, d], scale16 uint16 [n], zero16 uint16 [n], info)
    where info holds the float32 clipped values, group min/max and the fp32
    value (max - min) / 3 before fp16 rounding, for the parity checker."""
    y = np.asarray(y, dtype=np.float32)
    tau = np.float32(clip)
    yc = np.minimum(np.maximum(y, -tau), tau)
    mn = yc.min(axis=1)
    mx = yc.max(axis=1)
    rng3 = (mx - mn) / np.float32(3.0)             # float32 subtract, float32 divide
    zero16 = mn.astype(np.float16)                 # round to nearest even
    scale16 = rng3.astype(np.float16)
    z = zero16.astype(np.float32)[:, None]
    s = scale16.astype(np.float32)[:, None]
    with np.errstate(divide="ignore", invalid="ignore"):
        t = (yc - z) / s                           # float32 subtract, float32 divide
        codes = np.clip(np.rint(t), 0.0, 3.0)
    codes = np.where(s == 0, 0.0, codes).astype(np.uint8)
    info = dict(yc=yc, mn=mn, mx=mx, range3=rng3)
    return codes, scale16.view(np.uint16), zero16.view(np.uint16), info


def pack_codes_row(codes: np.ndarray) -> np.ndarray:
    """[..., d] codes in 0..3 -> [..., d/4] bytes, channel 4i+j in bits 2j."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 0::4] | (c[..., 1::4] << 2) | (c[..., 2::4] << 4) | (c[..., 3::4] << 6)).astype(np.uint8)


def unpack_codes_row(row: np.ndarray) -> np.ndarray:
    """Inverse of :func:`pack_codes_row`."""
    r = np.asarray(row, dtype=np.uint8)
    out = np.stack([(r >> (2 * j)) & 3 for j in range(4)], axis=-1)
    return out.reshape(r.shape[:-1] + (r.shape[-1] * 4,)).astype(np.uint8)


def page_block_bytes(d: int) -> int:
    """Bytes of codes per (page, KV head)."""
    return PAGE * d // 4


def k_byte_offsets(offset, d: int) -> np.ndarray:
    """Positions inside a (page, head) K block of the d/4 row bytes of the
    token at page offset ``offset`` (scalar or array -> [..., d/4])."""
    w = d // 16
    i = np.arange(d // 4)
    o = np.asarray(offset)[..., None]
    return (i // w) * (PAGE * w) + o * w + (i % w)


def v_byte_offsets(offset, d: int) -> np.ndarray:
    """Positions inside a (page, head) V block of the d/4 row bytes of the
    token at page offset ``offset`` (byte-column-major)."""
    i = np.arange(d // 4)
    o = np.asarray(offset)[..., None]
    return i * PAGE + o


def _offsets(kind: str, offset, d: int):
    if kind == "k":
        return k_byte_offsets(offset, d)
    if kind == "v":
        return v_byte_offsets(offset, d)
    raise ValueError("kind must be 'k' or 'v'")


def quantize_rows_grouped(quantize, y: np.ndarray, clip, group: int):
    """Quantise each consecutive block of ``group`` channels of every row of y
    [n, d] as its own group.  Returns codes [n, d] and fp16 bits [n, d/group]
    of scale and zero, and info with the per-group fields reshaped to [n, ng]
    (yc stays [n, d])."""
    n, d = y.shape
    ng = d // group
    codes, s16, z16, info = quantize(np.ascontiguousarray(y).reshape(n * ng, group), clip)
    info = {k: (v.reshape(n, d) if k == "yc" else v.reshape(n, ng)) for k, v in info.items()}
    return codes.reshape(n, d), s16.reshape(n, ng), z16.reshape(n, ng), info


def quantize_pack_ref(kind: str, x_bits: np.ndarray, rot: np.ndarray, clip, dst_slot: np.ndarray,
                      codes_pool: np.ndarray, sz_pool: np.ndarray, src_idx: np.ndarray | None = None,
                      chunk: int = 16384, codebook: str = UNIFORM, group: int | None = None):
    """Demote tokens of one tensor (K or V) of one layer into INT2 pages, in place.

    x_bits   bf16 [n_src][n_kv][d]
    rot      fp32 [n_kv][d][d]   (y = x R per head)
    clip     tau > 0, finite, <= 65504
    dst_slot int32 [n_tok]: physical page * 64 + offset; slots outside
             [0, n_pages*64) are skipped
    src_idx  int32 [n_tok] rows of x, or None for rows 0..n_tok-1; rows
             outside [0, n_src) are skipped
    codes_pool uint8 [n_pages][n_kv][64*d/4]; sz_pool uint16 [n_pages][n_kv][64*d/group][2]
    codebook "uniform" (min-max) or "lloyd_max"
    group    channels per quantisation group (None: the whole head)

    Returns a dict of per-(token, head) diagnostics for the written tokens
    (arrays [n_written][n_kv]...) used by the parity checker."""
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    n_src, n_kv, d = x_bits.shape
    tau = np.float32(clip)
    if not (np.isfinite(tau) and 0 < tau <= 65504):
        raise ValueError("clip must be finite, > 0 and <= 65504")
    if d % 16:
        raise ValueError("head_dim must be a multiple of 16")
    quantize = {UNIFORM: quantize_group, LLOYD_MAX: quantize_group_lloyd_max}[codebook]
    group = d if group is None else int(group)
    if group < 1 or d % group or sz_pool.shape[2] != PAGE * (d // group):
        raise ValueError("group must divide head_dim, and sz_pool hold 64 * head_dim/group pairs per head")
    ng = d // group
    n_pages = codes_pool.shape[0]
    dst = np.asarray(dst_slot, dtype=np.int64).ravel()
    src = np.arange(dst.size) if src_idx is None else np.asarray(src_idx, dtype=np.int64).ravel()
    if src.size != dst.size:
        raise ValueError("src_idx and dst_slot lengths differ")
    keep = (dst >= 0) & (dst < n_pages * PAGE) & (src >= 0) & (src < n_src)
    dst, src = dst[keep], src[keep]
    diag = {k: [] for k in ("slot", "yc", "mn", "mx", "range3", "codes", "scale16", "zero16")}
    for c0 in range(0, dst.size, chunk):
        dd, ss = dst[c0:c0 + chunk], src[c0:c0 + chunk]
        page, off = dd // PAGE, dd % PAGE
        pos = _offsets(kind, off, d)                         # [n, d/4]
        yc_h, mn_h, mx_h, r3_h, cd_h, sc_h, zr_h = ([] for _ in range(7))
        for g in range(n_kv):
            y = rotate_round_f32(x_bits[ss, g, :], rot[g])
            codes, s16, z16, info = quantize_rows_grouped(quantize, y, tau, group)
            codes_pool[page[:, None], g, pos] = pack_codes_row(codes)
            for j in range(ng):
                sz_pool[page, g, j * PAGE + off, 0] = s16[:, j]
                sz_pool[page, g, j * PAGE + off, 1] = z16[:, j]
            if ng == 1:   # one group per head: per-token diagnostics
                s16, z16 = s16[:, 0], z16[:, 0]
                info = {k: (v if k == "yc" else v[:, 0]) for k, v in info.items()}
            yc_h.append(info["yc"]); mn_h.append(info["mn"]); mx_h.append(info["mx"])
            r3_h.append(info["range3"]); cd_h.append(codes); sc_h.append(s16); zr_h.append(z16)
        diag["slot"].append(dd)
        diag["yc"].append(np.stack(yc_h, 1)); diag["mn"].append(np.stack(mn_h, 1))
        diag["mx"].append(np.stack(mx_h, 1)); diag["range3"].append(np.stack(r3_h, 1))
        diag["codes"].append(np.stack(cd_h, 1)); diag["scale16"].append(np.stack(sc_h, 1))
        diag["zero16"].append(np.stack(zr_h, 1))
    return {k: (np.concatenate(v) if v else np.zeros(0)) for k, v in diag.items()}


def read_history_codes(kind: str, codes_pool: np.ndarray, sz_pool: np.ndarray, pages: np.ndarray,
                       offsets: np.ndarray, g: int, d: int):
    """Codes [n][d] and fp16 (scale, zero) bits [n][ng] of the tokens at the
    given (physical page, offset) pairs of KV head g (ng groups per head, from
    the pool's shape; [n] when ng = 1)."""
    pos = _offsets(kind, offsets, d)
    rows = codes_pool[np.asarray(pages)[:, None], g, pos]
    ng = sz_pool.shape[2] // PAGE
    pages, offsets = np.asarray(pages), np.asarray(offsets)
    idx = offsets[:, None] + PAGE * np.arange(ng)[None, :]
    s16, z16 = sz_pool[pages[:, None], g, idx, 0], sz_pool[pages[:, None], g, idx, 1]
    if ng == 1:
        s16, z16 = s16[:, 0], z16[:, 0]
    return unpack_codes_row(rows), s16, z16
