"""CPU tests of the C-ABI boundary: the library loads, exports what include/*.h declares,
rejects every invalid argument with the documented status before any HIP call, and its host
table preparation (thresholds + bucket LUT) reproduces the oracle's nearest code."""
import ctypes
import glob
import os
import re

import numpy as np
import pytest

import dequantization_block_absmax_amd as bq
import oracle
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 1 << 20  # an aligned non-null address; never dereferenced by a rejected call
T16 = synth.table16()
T256 = synth.table256()


def declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        src = open(h).read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        names.update(re.findall(r"\b(bq_\w+)\s*\(", src))
    return sorted(names)


def test_header_declares_the_entry_points():
    names = declared_functions()
    for required in ("bq_quantize_blockwise", "bq_dequantize_blockwise", "bq_quantize_nested",
                     "bq_dequant_q32", "bq_dequantize_nested"):
        assert required in names


@pytest.mark.parametrize("name", declared_functions())
def test_library_exports_declared_symbol(name):
    lib = ctypes.CDLL(bq.LIB_PATH)
    assert hasattr(lib, name)
    assert name in bq.EXPORTS


def test_status_strings():
    for s in range(10):
        assert bq.status_string(s)
    assert bq.status_string(bq.BQ_OK) == "ok"


def q(**kw):
    args = dict(inp=FAKE, dtype=bq.BQ_BF16, n=1000, blocksize=64, table=T16, absmax=FAKE, packed=FAKE,
                stream=0)
    args.update(kw)
    return bq.bq_quantize_blockwise(**args)


def dq(**kw):
    args = dict(out=FAKE, dtype=bq.BQ_BF16, n=1000, blocksize=64, table=T16, absmax=FAKE, packed=FAKE,
                stream=0)
    args.update(kw)
    return bq.bq_dequantize_blockwise(**args)


@pytest.mark.parametrize("fn", [q, dq])
def test_blockwise_validation(fn):
    assert fn(dtype=7) == bq.BQ_ERR_DTYPE
    assert fn(n=-1) == bq.BQ_ERR_SIZE
    for b in (0, 16, 48, 100, 8192, -64):
        assert fn(blocksize=b) == bq.BQ_ERR_BLOCKSIZE
    assert fn(table=None) == bq.BQ_ERR_NULL
    bad_tables = [
        T16[:15],                                    # size
        np.concatenate([T16, [1.0]]),                 # size 17
        T16[::-1],                                    # order
        np.where(np.arange(16) == 3, T16[2], T16),    # duplicate
        np.where(np.arange(16) == 5, np.nan, T16),    # non-finite
        np.where(np.arange(16) == 15, 1.5, T16),      # out of range
        np.where(np.arange(16) == 9, 1e-7, T16),      # tiny nonzero entry
        np.float32(np.linspace(-1, 1, 200)),          # size 200
    ]
    for t in bad_tables:
        assert fn(table=np.float32(t)) == bq.BQ_ERR_TABLE
    assert fn(n=0) == bq.BQ_OK  # nothing enqueued
    assert fn(n=0, inp=None) == bq.BQ_OK if fn is q else fn(n=0, out=None) == bq.BQ_OK
    if fn is q:
        assert fn(inp=None) == bq.BQ_ERR_NULL
        assert fn(inp=FAKE + 8) == bq.BQ_ERR_ALIGNMENT
    else:
        assert fn(out=None) == bq.BQ_ERR_NULL
        assert fn(out=FAKE + 8) == bq.BQ_ERR_ALIGNMENT
    assert fn(absmax=None) == bq.BQ_ERR_NULL
    assert fn(packed=None) == bq.BQ_ERR_NULL
    assert fn(packed=FAKE + 4) == bq.BQ_ERR_ALIGNMENT
    assert fn(absmax=FAKE + 2) == bq.BQ_ERR_ALIGNMENT
    assert fn(n=(2**31) * 32, blocksize=32) == bq.BQ_ERR_SIZE  # more than INT32_MAX blocks


def test_negative_zero_table_entry_is_accepted():
    t = T16.copy()
    t[t == 0] = -0.0
    assert q(n=0, table=t) == bq.BQ_OK


def nstats(**kw):
    args = dict(qabsmax=FAKE, absmax2=FAKE, mean=FAKE, table=T256, blocksize2=256, workspace=FAKE,
                workspace_bytes=bq.bq_nested_workspace_bytes(1000, 64, 256))
    args.update(kw)
    return bq.nested_stats(**args)


def test_nested_validation():
    def call(stats=None, **kw):
        args = dict(inp=FAKE, dtype=bq.BQ_BF16, n=1000, blocksize=64, table=T16,
                    stats=nstats() if stats is None else stats, packed=FAKE, stream=0)
        args.update(kw)
        return bq.bq_quantize_nested(**args)

    assert call(dtype=9) == bq.BQ_ERR_DTYPE
    assert call(blocksize=65) == bq.BQ_ERR_BLOCKSIZE
    assert bq.bq_quantize_nested(FAKE, bq.BQ_BF16, 1000, 64, T16, None, FAKE, 0) == bq.BQ_ERR_NULL
    assert call(stats=nstats(blocksize2=100)) == bq.BQ_ERR_BLOCKSIZE
    assert call(stats=nstats(table=T16)) == bq.BQ_ERR_TABLE  # statistics need 256 entries
    assert call(stats=nstats(table=None)) == bq.BQ_ERR_NULL
    assert call(stats=nstats(qabsmax=None)) == bq.BQ_ERR_NULL
    assert call(stats=nstats(absmax2=None)) == bq.BQ_ERR_NULL
    assert call(stats=nstats(mean=None)) == bq.BQ_ERR_NULL
    assert call(stats=nstats(workspace=None)) == bq.BQ_ERR_WORKSPACE
    assert call(stats=nstats(workspace_bytes=10)) == bq.BQ_ERR_WORKSPACE
    assert call(stats=nstats(workspace=FAKE + 16)) == bq.BQ_ERR_ALIGNMENT
    assert call(stats=nstats(mean=FAKE + 1)) == bq.BQ_ERR_ALIGNMENT
    assert call(stats=nstats(qabsmax=FAKE + 2)) == bq.BQ_ERR_ALIGNMENT
    assert call(stats=nstats(absmax2=FAKE + 2)) == bq.BQ_ERR_ALIGNMENT
    assert call(inp=None) == bq.BQ_ERR_NULL
    assert call(n=0) == bq.BQ_OK
    # the nested dequantize needs no workspace but checks the rest
    st = nstats(workspace=None, workspace_bytes=0)
    assert bq.bq_dequantize_nested(FAKE, bq.BQ_BF16, 0, 64, T16, st, FAKE, 0) == bq.BQ_OK
    assert bq.bq_dequantize_nested(FAKE, bq.BQ_BF16, 1000, 64, T16, nstats(absmax2=None), FAKE, 0) == bq.BQ_ERR_NULL
    assert bq.bq_dequantize_nested(None, bq.BQ_BF16, 1000, 64, T16, st, FAKE, 0) == bq.BQ_ERR_NULL
    assert bq.bq_dequantize_nested(FAKE, bq.BQ_BF16, 1000, 64, T16, nstats(qabsmax=FAKE + 1, workspace=None,
                                                                           workspace_bytes=0), FAKE, 0) \
        == bq.BQ_ERR_ALIGNMENT


def test_noalloc_validation():
    """The allocation-free nested quantize validates like bq_quantize_nested, needs no
    workspace, and refuses inputs whose workspace would exceed its 36 MiB scratch before any
    HIP call."""
    def call(stats=None, **kw):
        args = dict(inp=FAKE, dtype=bq.BQ_BF16, n=1000, blocksize=64, table=T16,
                    stats=nstats(workspace=None, workspace_bytes=0) if stats is None else stats, packed=FAKE,
                    stream=0)
        args.update(kw)
        return bq.bq_quantize_nested_noalloc(**args)

    assert call(n=0) == bq.BQ_OK
    assert call(dtype=9) == bq.BQ_ERR_DTYPE
    assert call(blocksize=65) == bq.BQ_ERR_BLOCKSIZE
    assert call(stats=nstats(table=T16)) == bq.BQ_ERR_TABLE
    assert call(stats=nstats(qabsmax=FAKE + 4)) == bq.BQ_ERR_ALIGNMENT
    assert call(inp=None) == bq.BQ_ERR_NULL
    limit = 36 << 20
    fits = 1 << 29  # 2^29 elements at block size 64: the largest power of two that fits
    assert bq.bq_nested_workspace_bytes(fits, 64) <= limit < bq.bq_nested_workspace_bytes(2 * fits, 64)
    assert call(n=2 * fits) == bq.BQ_ERR_WORKSPACE
    assert call(n=(1 << 33), blocksize=32) == bq.BQ_ERR_WORKSPACE


def test_workspace_bytes():
    assert bq.bq_nested_workspace_bytes(0, 64, 256) == 0
    for n, B in ((2**29, 64), (1000, 32), (8192 * 3 + 1, 4096)):
        nb = -(-n // B)
        need = nb * 4 + (-(-nb // 16384)) * 8  # fp32 block maxima + one fp64 sum per run of 16384 blocks
        ws = bq.bq_nested_workspace_bytes(n, B, 256)
        assert need <= ws < need + 512


def test_q32_validation():
    def call(**kw):
        args = dict(blocks=FAKE, dtype=bq.BQ_BF16, n=4096 * 64, row_len=4096, fmt=bq.BQ_Q32_Q4, out=FAKE,
                    stream=0)
        args.update(kw)
        return bq.bq_dequant_q32(**args)

    assert call(dtype=3) == bq.BQ_ERR_DTYPE
    assert call(fmt=2) == bq.BQ_ERR_FORMAT
    assert call(row_len=48) == bq.BQ_ERR_FORMAT
    assert call(row_len=0) == bq.BQ_ERR_FORMAT
    assert call(n=4096 * 64 + 32) == bq.BQ_ERR_SIZE
    assert call(n=-4096) == bq.BQ_ERR_SIZE
    assert call(n=0) == bq.BQ_OK
    assert call(blocks=None) == bq.BQ_ERR_NULL
    assert call(out=None) == bq.BQ_ERR_NULL
    assert call(blocks=FAKE + 1) == bq.BQ_ERR_ALIGNMENT  # records are 2-byte aligned


def test_iq2xs_validation():
    def enc(**kw):
        args = dict(x=FAKE, dtype=bq.BQ_BF16, n=4096 * 16, row_len=4096, grid=FAKE, scales=FAKE, blocks=FAKE,
                    rejected=FAKE, stream=0)
        args.update(kw)
        return bq.bq_iq2xs_quantize(**args)

    def dec(**kw):
        args = dict(blocks=FAKE, grid=FAKE, n=4096 * 16, row_len=4096, dtype=bq.BQ_BF16, out=FAKE, stream=0)
        args.update(kw)
        return bq.bq_iq2xs_dequantize(**args)

    for call in (enc, dec):
        assert call(dtype=3) == bq.BQ_ERR_DTYPE
        assert call(row_len=128) == bq.BQ_ERR_FORMAT
        assert call(row_len=384) == bq.BQ_ERR_FORMAT  # rows must hold whole superblocks
        assert call(row_len=0) == bq.BQ_ERR_FORMAT
        assert call(n=4096 * 16 + 256) == bq.BQ_ERR_SIZE  # a partial row
        assert call(n=-4096) == bq.BQ_ERR_SIZE
        assert call(n=(1 << 31) * 256, row_len=256) == bq.BQ_ERR_SIZE  # more than INT32_MAX superblocks
        assert call(n=0) == bq.BQ_OK
        assert call(grid=None) == bq.BQ_ERR_NULL
        assert call(blocks=None) == bq.BQ_ERR_NULL
        assert call(blocks=FAKE + 1) == bq.BQ_ERR_ALIGNMENT  # 74-byte records are 2-byte aligned
    for k in ("x", "scales", "rejected"):
        assert enc(**{k: None}) == bq.BQ_ERR_NULL, k
    assert dec(out=None) == bq.BQ_ERR_NULL
    assert enc(x=FAKE + 8) == bq.BQ_ERR_ALIGNMENT
    assert enc(grid=FAKE + 8) == bq.BQ_ERR_ALIGNMENT
    assert enc(scales=FAKE + 1) == bq.BQ_ERR_ALIGNMENT
    assert enc(rejected=FAKE + 2) == bq.BQ_ERR_ALIGNMENT
    assert dec(grid=FAKE + 4) == bq.BQ_ERR_ALIGNMENT
    assert dec(out=FAKE + 8) == bq.BQ_ERR_ALIGNMENT


def test_iq1s_validation():
    def enc(**kw):
        args = dict(x=FAKE, dtype=bq.BQ_BF16, n=4096 * 16, row_len=4096, grid=FAKE, blocks=FAKE, stream=0)
        args.update(kw)
        return bq.bq_iq1s_quantize(**args)

    def dec(**kw):
        args = dict(blocks=FAKE, grid=FAKE, n=4096 * 16, row_len=4096, dtype=bq.BQ_BF16, out=FAKE, stream=0)
        args.update(kw)
        return bq.bq_iq1s_dequantize(**args)

    for call in (enc, dec):
        assert call(dtype=3) == bq.BQ_ERR_DTYPE
        assert call(row_len=384) == bq.BQ_ERR_FORMAT  # rows must hold whole superblocks
        assert call(row_len=0) == bq.BQ_ERR_FORMAT
        assert call(n=4096 * 16 + 256) == bq.BQ_ERR_SIZE
        assert call(n=-4096) == bq.BQ_ERR_SIZE
        assert call(n=(1 << 31) * 256, row_len=256) == bq.BQ_ERR_SIZE
        assert call(n=0) == bq.BQ_OK
        assert call(grid=None) == bq.BQ_ERR_NULL
        assert call(blocks=None) == bq.BQ_ERR_NULL
        assert call(blocks=FAKE + 1) == bq.BQ_ERR_ALIGNMENT  # 50-byte records are 2-byte aligned
    assert enc(x=None) == bq.BQ_ERR_NULL
    assert dec(out=None) == bq.BQ_ERR_NULL
    assert enc(x=FAKE + 8) == bq.BQ_ERR_ALIGNMENT
    assert enc(grid=FAKE + 8) == bq.BQ_ERR_ALIGNMENT
    assert dec(grid=FAKE + 4) == bq.BQ_ERR_ALIGNMENT
    assert dec(out=FAKE + 8) == bq.BQ_ERR_ALIGNMENT


def test_linear_validation():
    def call(**kw):
        args = dict(x=FAKE, dtype=bq.BQ_BF16, M=2, K=4096, N=14336, blocksize=64, table=T16, absmax=FAKE,
                    packed=FAKE, y=FAKE, stream=0)
        args.update(kw)
        return bq.bq_linear_blockwise(**args)

    assert call(dtype=5) == bq.BQ_ERR_DTYPE
    for kw in (dict(M=0), dict(M=5), dict(K=0), dict(K=17), dict(K=-16), dict(N=-1)):
        assert call(**kw) == bq.BQ_ERR_SIZE, kw
    assert call(K=16, N=(2**31) * 32, blocksize=32) == bq.BQ_ERR_SIZE  # more than INT32_MAX blocks
    assert call(K=16, N=67108861, blocksize=4096) == bq.BQ_ERR_SIZE  # more than 2^32 - 1 threads
    assert call(blocksize=48) == bq.BQ_ERR_BLOCKSIZE
    assert call(table=np.float32(T16[::-1])) == bq.BQ_ERR_TABLE
    assert call(table=None) == bq.BQ_ERR_NULL
    assert call(N=0) == bq.BQ_OK  # nothing enqueued
    assert call(N=0, x=None, y=None) == bq.BQ_OK
    for name in ("x", "absmax", "packed", "y"):
        assert call(**{name: None}) == bq.BQ_ERR_NULL, name
    assert call(x=FAKE + 8) == bq.BQ_ERR_ALIGNMENT
    assert call(packed=FAKE + 8) == bq.BQ_ERR_ALIGNMENT
    assert call(absmax=FAKE + 2) == bq.BQ_ERR_ALIGNMENT
    assert call(y=FAKE + 2) == bq.BQ_ERR_ALIGNMENT


def test_gemm_validation():
    def call(**kw):
        args = dict(x=FAKE, dtype=bq.BQ_BF16, M=64, K=4096, N=14336, blocksize=64, table=T16, absmax=FAKE,
                    packed=FAKE, y=FAKE, stream=0)
        args.update(kw)
        return bq.bq_gemm_blockwise(**args)

    assert call(dtype=bq.BQ_F32) == bq.BQ_ERR_DTYPE
    assert call(dtype=5) == bq.BQ_ERR_DTYPE
    for kw in (dict(M=0), dict(M=65535 * 64 + 1), dict(K=0), dict(K=32), dict(K=96), dict(K=-64), dict(N=-1)):
        assert call(**kw) == bq.BQ_ERR_SIZE, kw
    assert call(K=64, N=(2**31) * 32, blocksize=32) == bq.BQ_ERR_SIZE  # more than INT32_MAX blocks
    assert call(K=64, N=536870849, blocksize=4096) == bq.BQ_ERR_SIZE  # more than 2^32 - 1 threads
    assert call(blocksize=48) == bq.BQ_ERR_BLOCKSIZE
    assert call(table=np.float32(T16[::-1])) == bq.BQ_ERR_TABLE
    assert call(table=None) == bq.BQ_ERR_NULL
    assert call(N=0) == bq.BQ_OK  # nothing enqueued
    assert call(N=0, x=None, y=None) == bq.BQ_OK
    for name in ("x", "absmax", "packed", "y"):
        assert call(**{name: None}) == bq.BQ_ERR_NULL, name
    assert call(x=FAKE + 8) == bq.BQ_ERR_ALIGNMENT
    assert call(packed=FAKE + 8) == bq.BQ_ERR_ALIGNMENT
    assert call(absmax=FAKE + 2) == bq.BQ_ERR_ALIGNMENT
    assert call(y=FAKE + 2) == bq.BQ_ERR_ALIGNMENT


# ---- host table preparation vs the oracle ------------------------------------------------

def _search_probes(table, rng):
    """Values next to every midpoint, the entries, random and log-spread values, special
    values, and values around the binary16 subnormal and normal ranges."""
    t = np.asarray(table, np.float64)
    mids = ((t[:-1] + t[1:]) / 2).astype(np.float32)
    near = [mids]
    for k in range(1, 4):
        near.append(np.nextafter(near[-1], np.float32(-2)))
    up = [mids]
    for k in range(1, 4):
        up.append(np.nextafter(up[-1], np.float32(2)))
    entries = np.float32(table)
    rand = rng.uniform(-1, 1, 20000).astype(np.float32)
    logs = (rng.choice([-1, 1], 5000) * 2.0 ** rng.uniform(-30, 0, 5000)).astype(np.float32)
    special = np.float32([0.0, -0.0, 1.0, -1.0, 2.0**-149, -2.0**-149, 2.0**-126, 1 - 2.0**-24,
                          -(1 - 2.0**-24), np.nan, np.inf, -np.inf])
    f16 = np.float32([s * m * 2.0**e for s in (-1, 1) for e in (-26, -25, -24, -20, -15, -14, -13)
                      for m in (1.0, 1.0 + 2.0**-23, 1.5, 2.0 - 2.0**-23)])
    return np.concatenate(near + up + [entries, rand, logs, special, f16])


def _oracle_codes(o, y, table):
    return np.array([o.zero_code(table) if not np.isfinite(v) else o.nearest(v, table) for v in y], np.int32)


TABLES = {
    "table16": T16,
    "table256": T256,
    "hand16": np.float32([-1, -0.875, -0.75, -0.625, -0.5, -0.375, -0.25, -0.125, 0, 0.125, 0.25, 0.375, 0.5,
                          0.625, 0.75, 1]),
    "dyadic256": synth.dyadic_table(256),
    "nf4_like": np.float32(np.sort(np.concatenate([[-1, 0, 1], np.linspace(-0.7, 0.72, 13)]))),
    "tiny_entries": np.float32(np.sort(np.concatenate([[-1, 0, 1, 2.0**-20, -2.0**-20, 2.0**-19],
                                                       np.linspace(0.1, 0.9, 10)]))),
    # symmetric, 16 entries per side spaced 2^-19 apart below 2^-14 (thresholds in the binary16
    # subnormal range), geometric above: binary16 buckets, one compare
    "subnormal16": np.float32(np.sort(np.concatenate([
        s * np.concatenate([np.arange(1, 17) * 2.0**-19, np.geomspace(2.0**-14, 1.0, 112)]) for s in (-1, 1)]))),
    # 200 entries packed into [0.5, 0.5 + 2e-4]: no bucketing keeps <= 3 compares -> search
    "clustered256": np.float32(np.sort(np.concatenate([np.linspace(-1, 0.45, 56),
                                                       0.5 + np.arange(200) * 2.0**-23 * 8]))),
}


@pytest.mark.parametrize("name", sorted(TABLES))
def test_host_search_matches_oracle(name):
    table = TABLES[name]
    assert len(np.unique(table)) == len(table) in (16, 256)
    o = oracle.Oracle()
    y = _search_probes(table, np.random.default_rng(len(name)))
    st, codes, mode, cmp = bq.bq_debug_nearest_codes(table, y)
    assert st == bq.BQ_OK
    expect = _oracle_codes(o, y, table)
    bad = np.nonzero(codes != expect)[0]
    assert bad.size == 0, (name, mode, [(float(y[i]), codes[i], expect[i]) for i in bad[:5]])
    if name == "clustered256":
        assert mode == 2
    if name in ("table16", "hand16"):
        assert mode == 0 and cmp == 1
    if name in ("table256", "subnormal16"):
        assert mode == 3 and cmp == 1


def test_launch_size_limit():
    """A call whose launch would hold more than 2^32 - 1 threads is refused with BQ_ERR_SIZE
    before anything is enqueued (no device is touched: the addresses are never used)."""
    t16, t256 = bq.code_table(T16), bq.code_table(T256)
    assert bq.bq_dequantize_blockwise(FAKE, bq.BQ_BF16, 1 << 36, 4096, t256, FAKE, FAKE, stream=0) == bq.BQ_ERR_SIZE
    assert bq.bq_dequantize_blockwise(FAKE, bq.BQ_BF16, 1 << 37, 4096, t16, FAKE, FAKE, stream=0) == bq.BQ_ERR_SIZE
    assert bq.bq_quantize_blockwise(FAKE, bq.BQ_BF16, 1 << 37, 4096, t16, FAKE, FAKE, stream=0) == bq.BQ_ERR_SIZE
