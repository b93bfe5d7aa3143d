"""CPU models of the arithmetic and layouts inside the HIP kernels (no GPU).

These pin the claims the kernels rest on, written out in numpy from the
kernels' own definitions (gdr_device.h, gdr_chunked_sweep.hip):

* the exact three-piece bf16 split of an fp32 value (hi = bf16(x),
  mid = bf16(x - hi), lo = bf16(x - hi - mid), each rounded to nearest even):
  the pieces sum to x exactly; a product with a bf16 value taken as three
  exact piece products and summed in fp32 keeps fp32 accuracy; a product of
  two fp32 values as six piece products loses no more than fp32 rounding;
* the blocked inversion of a unit triangular 64 x 64 matrix (16 x 16 diagonal
  blocks by substitution, then the off-diagonal blocks block row by block
  row) equals numpy's inverse;
* the LDS layouts: the step permutation of the chunked sweeps is a
  permutation, and the swizzled bf16 tiles read by ds_read_b64_tr_b16 put
  the 32 lanes of each half-wave on 64 distinct banks; the step planes of
  the eight-wave chunk kernel (gdr_chunk_bf16.hip) are staged once per
  element and written and read without bank conflicts.
"""
import numpy as np
import pytest

# ------------------------------------------------------------------ split --


def bf16_rne(x):
    """fp32 -> nearest bf16 (ties to even), returned as fp32 (the
    conversion v_cvt_pk_bf16_f32 performs)."""
    a = np.ascontiguousarray(np.asarray(x, np.float32))
    u = a.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000).astype(np.uint32)
    return r.view(np.float32)


def split3(x):
    """The kernels' split: each remainder formed in fp32 (exact: it has at
    most 16 significant bits), each piece its nearest bf16."""
    x = np.asarray(x, np.float32)
    hi = bf16_rne(x)
    r1 = (x - hi).astype(np.float32)
    mid = bf16_rne(r1)
    r2 = (r1 - mid).astype(np.float32)
    lo = bf16_rne(r2)
    return hi, mid, lo


def _wide_fp32(rng, n):
    """Values with random sign, significand and exponent over 2^-100..2^100,
    plus random bit patterns from 2^-100 up to bf16 overflow.  Below about
    2^-110 the lower pieces would fall under the normal range and lose bits:
    the split is exact "away from the bottom of the exponent range", where
    the kernels' operands (states, their gradients, residuals, decay
    products of at most 64 steps that have not underflowed) live."""
    a = rng.uniform(1, 2, n) * np.exp2(rng.integers(-100, 100, n)) * rng.choice([-1, 1], n)
    lo_bits = (127 - 100) << 23
    bits = rng.integers(lo_bits, 0x7F7F0000, n, dtype=np.uint64).astype(np.uint32)
    b = bits.view(np.float32) * rng.choice([-1, 1], n).astype(np.float32)
    return np.concatenate([a.astype(np.float32), b])


def test_split_is_exact():
    x = _wide_fp32(np.random.default_rng(1), 200_000)
    hi, mid, lo = split3(x)
    for p in (hi, mid, lo):  # every piece is a bf16 value
        assert np.array_equal(bf16_rne(p), p)
    s = hi.astype(np.float64) + mid.astype(np.float64) + lo.astype(np.float64)
    assert np.array_equal(s, x.astype(np.float64))
    # the remainders were exact in fp32
    assert np.array_equal((x.astype(np.float64) - hi), (x - hi).astype(np.float64))


def test_split_pieces_shrink():
    """Each piece is at most half a bf16 unit of the one before (8 bits of
    significand per piece), so three of them cover fp32's 24."""
    x = _wide_fp32(np.random.default_rng(2), 100_000)
    hi, mid, lo = split3(x)
    ulp = lambda p: np.exp2(np.floor(np.log2(np.abs(p.astype(np.float64)))) - 7)
    nz = hi != 0
    assert np.all(np.abs(mid[nz]) <= ulp(hi[nz]) / 2 * (1 + 1e-12))
    nz = mid != 0
    assert np.all(np.abs(lo[nz]) <= ulp(mid[nz]) / 2 * (1 + 1e-12))


def _fp32_sum(terms):
    """Left-to-right fp32 accumulation (the MFMA accumulates in fp32)."""
    acc = np.zeros_like(terms[0], dtype=np.float32)
    for t in terms:
        acc = (acc + t.astype(np.float32)).astype(np.float32)
    return acc


def test_three_piece_product_with_bf16_is_fp32_accurate():
    rng = np.random.default_rng(3)
    x = rng.standard_normal(100_000).astype(np.float32)
    b = bf16_rne(rng.standard_normal(100_000))
    hi, mid, lo = split3(x)
    # each piece product is exact in fp32 (8 x 8 significant bits)
    for p in (hi, mid, lo):
        assert np.array_equal((p * b).astype(np.float64), p.astype(np.float64) * b)
    got = _fp32_sum([hi * b, mid * b, lo * b]).astype(np.float64)
    exact = x.astype(np.float64) * b
    rel = np.abs(got - exact) / np.abs(exact)
    assert rel.max() <= 2 * 2.0 ** -24


def test_six_piece_product_is_fp32_accurate():
    """fp32 x fp32 as the six piece products hi.hi, hi.mid, mid.hi, hi.lo,
    lo.hi, mid.mid: the dropped terms are below 2^-24 relative."""
    rng = np.random.default_rng(4)
    x = rng.standard_normal(100_000).astype(np.float32)
    y = rng.standard_normal(100_000).astype(np.float32)
    xh, xm, xl = split3(x)
    yh, ym, yl = split3(y)
    got = _fp32_sum([xh * yh, xh * ym, xm * yh, xh * yl, xl * yh, xm * ym]).astype(np.float64)
    exact = x.astype(np.float64) * y.astype(np.float64)
    rel = np.abs(got - exact) / np.abs(exact)
    # the five fp32 additions and the dropped terms (each below 2^-24): a few
    # units of fp32 rounding, against 2^-24 for the rounded fp32 product
    assert rel.max() <= 8 * 2.0 ** -24


def test_piece_dot_products_match_fp32():
    """A 64-term dot product (one tile of a chunk) from the six piece
    products against a plain fp32 dot product: both at the level of fp32
    rounding of the exact value (the pieces add six times as many terms to
    the fp32 accumulator: within three times the plain error)."""
    rng = np.random.default_rng(5)
    x = rng.standard_normal((2000, 64)).astype(np.float32)
    y = rng.standard_normal((2000, 64)).astype(np.float32)
    exact = (x.astype(np.float64) * y.astype(np.float64)).sum(1)
    xh, xm, xl = split3(x)
    yh, ym, yl = split3(y)
    pieces = [xh * yh, xh * ym, xm * yh, xh * yl, xl * yh, xm * ym]
    acc = np.zeros(2000, np.float32)
    for k in range(64):  # k-outer, pieces inner, like the MFMA k-steps
        for p in pieces:
            acc = (acc + p[:, k]).astype(np.float32)
    plain = np.zeros(2000, np.float32)
    for k in range(64):
        plain = (plain + (x[:, k] * y[:, k]).astype(np.float32)).astype(np.float32)
    scale = np.sqrt(((x.astype(np.float64) * y) ** 2).sum(1))
    e_p = np.abs(acc - exact) / scale
    e_f = np.abs(plain - exact) / scale
    assert np.sqrt(np.mean(e_p ** 2)) <= 3 * np.sqrt(np.mean(e_f ** 2))
    assert e_p.max() <= 64 * 2.0 ** -23
    # three pieces against a bf16 operand (the products with k, q, dy): the
    # piece products are exact, so only the accumulation rounds
    b = bf16_rne(y)
    acc3 = np.zeros(2000, np.float32)
    for kk in range(64):
        for pc in (xh, xm, xl):
            acc3 = (acc3 + pc[:, kk] * b[:, kk]).astype(np.float32)
    exact3 = (x.astype(np.float64) * b.astype(np.float64)).sum(1)
    plain3 = np.zeros(2000, np.float32)
    for kk in range(64):
        plain3 = (plain3 + (x[:, kk] * b[:, kk]).astype(np.float32)).astype(np.float32)
    sc3 = np.sqrt(((x.astype(np.float64) * b) ** 2).sum(1))
    assert (np.sqrt(np.mean(((acc3 - exact3) / sc3) ** 2))
            <= 3 * np.sqrt(np.mean(((plain3 - exact3) / sc3) ** 2)))


# ------------------------------------------------------- blocked inversion --


def blocked_unit_triangular_inverse(A, upper=False, dtype=np.float64):
    """(I + A)^-1 for a strictly lower (upper) triangular 64 x 64 A, in the
    kernel's order: the four 16 x 16 diagonal blocks by substitution, then
    L_ik = -T_ii A_ik for the blocks of the triangle, then block row by block
    row T_ij = sum_k L_ik T_kj over k between j and i (the block-row
    equations of (I + A) T = I)."""
    A = A.astype(dtype)
    T = np.zeros((64, 64), dtype)
    blk = lambda M, i, j: M[16 * i:16 * i + 16, 16 * j:16 * j + 16]
    for i in range(4):  # diagonal blocks, one column c at a time
        Ad = blk(A, i, i)
        X = np.zeros((16, 16), dtype)
        for c in range(16):
            order = range(15, -1, -1) if upper else range(16)
            for t in order:
                acc = dtype(1.0) if t == c else dtype(0.0)
                rs = range(t + 1, 16) if upper else range(t)
                for r in rs:
                    acc -= Ad[t, r] * X[r, c]
                X[t, c] = acc
        blk(T, i, i)[:] = X
    L = {}
    for i in range(4):
        for k in range(4):
            if (k > i) if upper else (k < i):
                L[i, k] = -blk(T, i, i) @ blk(A, i, k)
    rows = range(2, -1, -1) if upper else range(1, 4)
    for i in rows:
        js = range(i + 1, 4) if upper else range(i)
        for j in js:
            ks = range(i + 1, j + 1) if upper else range(j, i)
            blk(T, i, j)[:] = sum(L[i, k] @ blk(T, k, j) for k in ks)
    return T


def _decay_gram(rng, strong, upper):
    """A of the forward (or Bm of the reverse) pass from seeded unit k rows,
    beta and a running product of g, as the prep kernel forms it."""
    k = rng.standard_normal((64, 192))
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    mu = 2.0 if strong else -2.0
    g = np.exp(-np.exp(rng.normal(mu, 0.5, 64)))
    beta = 1 / (1 + np.exp(-rng.standard_normal(64)))
    KK = k @ k.T
    gam = np.zeros((64, 64))  # gam[r][t] = product of g over r+1..t
    for t in range(64):
        p = 1.0
        for r in range(t - 1, -1, -1):
            p *= g[r + 1]
            gam[r, t] = p
    A = np.zeros((64, 64))
    for t in range(64):
        for r in range(t):
            if upper:
                A[r, t] = gam[r, t] * beta[t] * KK[t, r]   # Bm[t'=r][s=t]
            else:
                A[t, r] = gam[r, t] * KK[t, r] * beta[r]
    return A


@pytest.mark.parametrize("upper", [False, True])
@pytest.mark.parametrize("strong", [False, True])
def test_blocked_inverse_equals_numpy(upper, strong):
    rng = np.random.default_rng(7 + 2 * upper + strong)
    A = _decay_gram(rng, strong, upper)
    ref = np.linalg.inv(np.eye(64) + A)
    T = blocked_unit_triangular_inverse(A, upper)
    assert np.abs(T - ref).max() <= 1e-12 * max(1.0, np.abs(ref).max())
    # triangular, unit diagonal
    assert np.array_equal(np.triu(T, 1) if not upper else np.tril(T, -1), np.zeros((64, 64)))
    assert np.allclose(np.diag(T), 1.0)
    # in fp32 arithmetic, at fp32 rounding of the result
    T32 = blocked_unit_triangular_inverse(A.astype(np.float32), upper, np.float32)
    assert np.abs(T32 - ref).max() <= 1e-5 * max(1.0, np.abs(ref).max())


# ------------------------------------------------------------ LDS layouts --


def rstep(ks, lq):
    return 16 * (ks >> 2) + 4 * lq + (ks & 3)


def test_step_permutation():
    """k-step ks of lane quarter lq takes step rstep(ks, lq): every step of
    the 64 exactly once, each k-step's four quarters four distinct steps."""
    steps = sorted(rstep(ks, lq) for ks in range(16) for lq in range(4))
    assert steps == list(range(64))


def test_step_reads_conflict_free():
    """fp32 reads sm[rstep(ks, lq) * 36 + 16 nt + l % 16] of a [64][36]
    stage (E = T U and Y = M E): one wave, 64 lanes of 4 bytes, each on its
    own bank."""
    for ks in range(16):
        for nt in range(2):
            banks = [(rstep(ks, l >> 4) * 36 + 16 * nt + (l & 15)) % 64 for l in range(64)]
            assert len(set(banks)) == 64


def tile_swz(r):
    return (((r >> 1) & 1) << 2) | (((r >> 3) & 1) << 3)


def p_swz(j):
    return (j >> 1) & 6


def kq_row_stride(dkp):
    return dkp + 64 if dkp % 128 == 0 else dkp


def _half_wave_banks(addr_bf16):
    """Banks (4-byte words mod 64) of the 8-byte blocks at these bf16
    element offsets, per half-wave of 32 lanes."""
    out = []
    for h in range(2):
        banks = []
        for a in addr_bf16[32 * h:32 * h + 32]:
            w = (2 * a) // 4
            banks += [w % 64, (w + 1) % 64]
        out.append(banks)
    return out


@pytest.mark.parametrize("dkp", [64, 128, 192, 256])
def test_swizzled_tile_reads_conflict_free(dkp):
    """tile_operand: lane l reads the 8-byte block of row k0 + 8 (l / 16) +
    (l % 16) / 4 (+ 4 for the second read), block (n0 / 4 + l % 4) ^
    tile_swz(row), in a tile of row stride kq_row_stride(dkp) bf16."""
    rs = kq_row_stride(dkp)
    assert (2 * rs) % 256 == 128
    for k0 in range(0, 64, 32):
        for n0 in range(0, dkp, 16):
            for second in (0, 4):
                addr = []
                for l in range(64):
                    lr, lq = l & 15, l >> 4
                    t = k0 + 8 * lq + (lr >> 2) + second
                    cb = (n0 >> 2) + (lr & 3)
                    addr.append(t * rs + 4 * (cb ^ tile_swz(t)))
                for banks in _half_wave_banks(addr):
                    assert len(set(banks)) == 64, (dkp, k0, n0, second)


@pytest.mark.parametrize("dkp", [64, 128, 192, 256])
def test_swizzled_tile_row_writes_conflict_free(dkp):
    """deposit_rows: 16-byte groups (blocks 2c, 2c+1, adjacent under the
    swizzle) of the rows of a chunk; the lanes of a half-wave write
    consecutive groups, i.e. whole rows' worth of blocks."""
    rs = kq_row_stride(dkp)
    ng = dkp // 8  # 8-element groups per row
    for base in range(0, 64 * ng, 32):
        banks = []
        for u in range(base, base + 32):
            t, c = u // ng, u % ng
            a = t * rs + 4 * ((2 * c) ^ tile_swz(t))
            w = (2 * a) // 4
            banks += [w % 64, (w + 1) % 64, (w + 2) % 64, (w + 3) % 64]
        # 32 lanes x 16 bytes = two passes of 64 banks: each bank twice
        counts = np.bincount(banks, minlength=64)
        assert counts.max() == 2, (dkp, base)


def test_state_piece_reads_conflict_free():
    """piece_operand: j-major state pieces [j][32] (rows of 64 bytes), lane l
    reads row k0 + 8 (l / 16) + (l % 16) / 4 (+ 4), block (n0 / 4 + l % 4)
    ^ p_swz(row)."""
    for k0 in range(0, 192, 32):
        for n0 in (0, 16):
            for second in (0, 4):
                addr = []
                for l in range(64):
                    lr, lq = l & 15, l >> 4
                    j = k0 + 8 * lq + (lr >> 2) + second
                    cb = (n0 >> 2) + (lr & 3)
                    addr.append(j * 32 + 4 * (cb ^ p_swz(j)))
                for banks in _half_wave_banks(addr):
                    assert len(set(banks)) == 64, (k0, n0, second)


def step_of(x):
    """Step staged by thread x of the eight-wave chunk kernel
    (gdr_chunk_bf16.hip): half-wave h takes steps c, c + 4, c + 8, c + 12."""
    grp = x >> 5
    return 16 * (grp >> 2) + (grp & 3) + 4 * ((x >> 3) & 3)


def test_step_plane_shares_cover_the_block():
    """The 512 threads stage every (step, 4-row quad) of a 64-step x 32-row
    block exactly once."""
    cells = sorted((step_of(x), x & 7) for x in range(512))
    assert cells == [(t, q) for t in range(64) for q in range(8)]


def test_step_plane_writes_conflict_free():
    """The 8-byte piece writes of the step planes ([64][40] bf16, element
    (t, 4 q)) of each half-wave cover the 64 banks once; four consecutive
    steps (the plain thread order) would not."""
    ys = 40

    def banks(steps_quads):
        b = []
        for t, q in steps_quads:
            w = (2 * (t * ys + 4 * q)) // 4
            b += [w % 64, (w + 1) % 64]
        return b

    for h in range(16):
        xs = range(32 * h, 32 * h + 32)
        assert len(set(banks([(step_of(x), x & 7) for x in xs]))) == 64, h
    plain = banks([(x >> 3, x & 7) for x in range(32)])
    assert len(set(plain)) < 64


def test_step_plane_reads_conflict_free():
    """The 16-byte operand reads of the step planes: lane l reads row
    tw + l % 16, bf16 columns 8 (l / 16) ..; the 16 lanes of each quarter
    (one column block) fall on 64 distinct banks."""
    ys = 40
    for tw in (0, 16, 32, 48):
        for lq in range(4):
            b = []
            for lr in range(16):
                w = (2 * ((tw + lr) * ys + 8 * lq)) // 4
                b += [(w + i) % 64 for i in range(4)]
            assert len(set(b)) == 64, (tw, lq)
