"""Seeded synthetic inputs for chunked prefill attention over a paged KV cache.

This module only draws and lays out inputs; it holds none of the attention
arithmetic.  The tests, the benchmark and the smoke check feed the same
arrays to the HIP library and to the CPU oracle.

Recipe (one ``numpy.random.default_rng(seed)`` per case, draws in this order):
  1. Q  [R][Hq][d]      float32 N(0, 1) * value_scale
  2. K  [ctx][Hkv][d]   float32 N(0, 1) * value_scale   (logical token order)
  3. V  [ctx][Hkv][d]   float32 N(0, 1) * value_scale
  4. the block table: a permutation of the pool ("permute"), the identity
     ("identity"), or ceil(ctx/ps) pages drawn without replacement from a
     larger pool ("scatter").
Values are rounded to fp16 or bf16 (round to nearest even) and both sides
consume the rounded values.  Pool pages that no logical page uses, and page
slots past ctx, hold 0xFFFF, a NaN in both fp16 and bf16: a kernel that reads
them into its result produces NaN.
"""

from dataclasses import dataclass, field

import numpy as np

POISON = np.uint16(0xFFFF)


def encode_f16(x):
    """float32 -> IEEE binary16 bit patterns, round to nearest even."""
    return np.asarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def encode_bf16(x):
    """float32 -> bfloat16 bit patterns, round to nearest even (finite inputs)."""
    bits = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (bits + np.uint64(0x7FFF) + ((bits >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return rounded.astype(np.uint16)


ENCODERS = {"f16": encode_f16, "bf16": encode_bf16}


@dataclass
class Case:
    """One synthetic workload: raw 16-bit patterns plus its shape."""
    name: str
    history: int
    rows: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    page_size: int
    dtype: str
    q: np.ndarray            # uint16 [R][Hq][d]
    k_pages: np.ndarray      # uint16 [pool][ps][Hkv][d]
    v_pages: np.ndarray      # uint16 [pool][ps][Hkv][d]
    block_table: np.ndarray  # int32 [ceil(ctx/ps)]
    k_contig: np.ndarray     # uint16 [ctx][Hkv][d]
    v_contig: np.ndarray     # uint16 [ctx][Hkv][d]
    piece_rows: int = 0      # 0: the chunk is one call
    extra: dict = field(default_factory=dict)

    @property
    def ctx(self):
        return self.history + self.rows


def make_case(name, history, rows, n_q_heads, n_kv_heads, head_dim, page_size, dtype,
              seed, value_scale=1.0, table="permute", pool_pages=None, piece_rows=0):
    """Draw one case following the module recipe."""
    rng = np.random.default_rng(seed)
    ctx = history + rows
    enc = ENCODERS[dtype]
    q = enc(rng.standard_normal((rows, n_q_heads, head_dim), dtype=np.float32) * np.float32(value_scale))
    k = enc(rng.standard_normal((ctx, n_kv_heads, head_dim), dtype=np.float32) * np.float32(value_scale))
    v = enc(rng.standard_normal((ctx, n_kv_heads, head_dim), dtype=np.float32) * np.float32(value_scale))
    n_pages = -(-ctx // page_size)
    if table == "identity":
        pool = n_pages if pool_pages is None else pool_pages
        bt = np.arange(n_pages, dtype=np.int32)
    elif table == "permute":
        pool = n_pages if pool_pages is None else pool_pages
        bt = rng.permutation(pool)[:n_pages].astype(np.int32)
    elif table == "scatter":
        pool = pool_pages
        bt = rng.choice(pool, size=n_pages, replace=False).astype(np.int32)
    else:
        raise ValueError(table)
    k_pages = lay_out_pages(k, bt, pool, page_size)
    v_pages = lay_out_pages(v, bt, pool, page_size)
    return Case(name, history, rows, n_q_heads, n_kv_heads, head_dim, page_size, dtype,
                q, k_pages, v_pages, bt, k, v, piece_rows)


def lay_out_pages(tokens, block_table, pool_pages, page_size, fill=POISON):
    """Scatter logical tokens [ctx][Hkv][...] into a page pool filled with
    `fill` (for 16-bit data 0xFFFF, a NaN in fp16 and bf16)."""
    ctx = tokens.shape[0]
    pages = np.full((pool_pages, page_size) + tokens.shape[1:], fill, dtype=tokens.dtype)
    n_full = ctx // page_size
    if n_full:
        pages[block_table[:n_full]] = tokens[:n_full * page_size].reshape((n_full, page_size) + tokens.shape[1:])
    tail = ctx - n_full * page_size
    if tail:
        pages[block_table[n_full], :tail] = tokens[n_full * page_size:]
    return pages


# The five workloads: shapes, history lengths and piece sizes of the pages'
# measurements (a 16 Q / 2 KV head, d 256 attention layer; a 2048-row chunk
# at 32K-128K history in production pieces), with random values standing in
# for a real model's activations.
SWEEP_HISTORIES = (1024, 2048, 4096, 8192, 16384, 32768)


def config_case(name):
    if name == "tiny":
        return make_case(name, 512, 64, 4, 1, 64, 16, "f16", seed=0)
    if name == "qwen_like":
        return make_case(name, 8192, 512, 16, 2, 256, 16, "f16", seed=1, value_scale=0.5)
    if name.startswith("sweep_"):
        history = int(name.split("_")[1])
        return make_case(name, history, 2048, 16, 2, 256, 16, "f16", seed=2)
    if name == "piece_64k":
        return make_case(name, 65536, 2048, 32, 4, 128, 16, "bf16", seed=3, piece_rows=256)
    if name == "long_128k":
        return make_case(name, 131072, 2048, 16, 2, 256, 16, "bf16", seed=4,
                         table="scatter", pool_pages=65536, piece_rows=128)
    raise KeyError(name)


CONFIG_NAMES = ("tiny", "qwen_like") + tuple(f"sweep_{h}" for h in SWEEP_HISTORIES) + ("piece_64k", "long_128k")


def exact_flops(history, rows, n_q_heads, head_dim):
    """Attention FLOPs of one chunk call, counting each row's visible keys:
    4 * d * Hq * sum_i (H + i + 1) = 4 d Hq (R H + R (R + 1) / 2)."""
    return 4 * head_dim * n_q_heads * (rows * history + rows * (rows + 1) // 2)


@dataclass
class VarlenCase:
    """A packed batch of sequences over one page pool (see make_varlen_case)."""
    name: str
    seqs: list             # [(history, rows)] per sequence
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    page_size: int
    dtype: str
    q: np.ndarray          # [total_rows][Hq][d] uint16
    k_pages: np.ndarray    # [pool][ps][Hkv][d] uint16
    v_pages: np.ndarray
    block_tables: np.ndarray   # [n][stride] int32
    cu_rows: np.ndarray        # [n + 1] int32
    history_lens: np.ndarray   # [n] int64

    @property
    def max_rows(self):
        return max([r for _, r in self.seqs] + [0])

    @property
    def max_context(self):
        return max([h + r for h, r in self.seqs] + [0])


def make_varlen_case(name, seqs, n_q_heads, n_kv_heads, head_dim, page_size, dtype, seed,
                     value_scale=1.0, shared=(), extra_pool=3):
    """A batch of sequences [(history, rows)]: per sequence, in order, K then
    V [ctx][Hkv][d] N(0, 1) * value_scale; then the pool order (a permutation
    handing each sequence its own pages); then Q [total_rows][Hq][d].
    shared = [(dst, src, n_pages)]: sequence dst's first n_pages logical pages
    are src's (a shared prefix: dst's own tokens there are not stored, so
    its keys there are src's).  Table rows are padded with page 0 (a valid
    page that the kernels never read for that sequence)."""
    rng = np.random.default_rng(seed)
    enc = ENCODERS[dtype]
    ctxs = [h + r for h, r in seqs]
    n_pages = [-(-c // page_size) for c in ctxs]
    pool = sum(n_pages) + extra_pool
    order = rng.permutation(pool)
    stride = max(n_pages + [1])
    tables = np.zeros((len(seqs), stride), dtype=np.int32)
    at = 0
    for s, n in enumerate(n_pages):
        tables[s, :n] = order[at:at + n]
        at += n
    skip = {}
    for dst, src, n in shared:
        tables[dst, :n] = tables[src, :n]
        skip[dst] = n * page_size
    k_pages = np.full((pool, page_size, n_kv_heads, head_dim), POISON, dtype=np.uint16)
    v_pages = np.full((pool, page_size, n_kv_heads, head_dim), POISON, dtype=np.uint16)
    for s, c in enumerate(ctxs):
        k = enc(rng.standard_normal((c, n_kv_heads, head_dim), dtype=np.float32) * np.float32(value_scale))
        v = enc(rng.standard_normal((c, n_kv_heads, head_dim), dtype=np.float32) * np.float32(value_scale))
        j = np.arange(skip.get(s, 0), c)
        k_pages[tables[s, j // page_size], j % page_size] = k[j]
        v_pages[tables[s, j // page_size], j % page_size] = v[j]
    cu = np.concatenate([[0], np.cumsum([r for _, r in seqs])]).astype(np.int32)
    q = enc(rng.standard_normal((int(cu[-1]), n_q_heads, head_dim), dtype=np.float32) * np.float32(value_scale))
    hist = np.array([h for h, _ in seqs], dtype=np.int64)
    return VarlenCase(name, list(seqs), n_q_heads, n_kv_heads, head_dim, page_size, dtype, q, k_pages, v_pages,
                      tables, cu, hist)



@dataclass
class Q8Case:
    """A chunk over 8-bit K/V pages (see make_q8_case)."""
    name: str
    history: int
    rows: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    page_size: int
    dtype: str
    q: np.ndarray          # [R][Hq][d] uint16 (fp16 or bf16 bits)
    k_quant: np.ndarray    # [pool][ps][Hkv][d] int8
    k_scale: np.ndarray    # [pool][ps][Hkv][d/32] uint16 (fp16 bits)
    v_quant: np.ndarray
    v_scale: np.ndarray
    block_table: np.ndarray
    piece_rows: int = 0


def make_q8_case(name, history, rows, n_q_heads, n_kv_heads, head_dim, page_size, dtype, seed,
                 table="permute", pool_pages=None, piece_rows=0):
    """Q as in make_case; then per tensor K, V (logical token order) quants
    uniform in [-127, 127] and fp16 scales 0.002 + 0.01 |N(0, 1)| per block
    of 32 values (values of roughly unit spread); then the block table.  Pool
    slots no token uses hold random quants under 0xFFFF scales (fp16 NaN), so
    reading them poisons the result."""
    rng = np.random.default_rng(seed)
    ctx = history + rows
    q = ENCODERS[dtype](rng.standard_normal((rows, n_q_heads, head_dim), dtype=np.float32))
    nb = head_dim // 32
    tensors = []
    for _ in range(2):
        quant = rng.integers(-127, 128, size=(ctx, n_kv_heads, head_dim), dtype=np.int8)
        scale = (np.float32(0.002) + np.float32(0.01) * np.abs(rng.standard_normal((ctx, n_kv_heads, nb),
                                                                                   dtype=np.float32)))
        tensors.append((quant, scale.astype(np.float16).view(np.uint16)))
    n_pages = -(-ctx // page_size)
    if table == "permute":
        pool = n_pages if pool_pages is None else pool_pages
        bt = rng.permutation(pool)[:n_pages].astype(np.int32)
    elif table == "scatter":
        pool = pool_pages
        bt = rng.choice(pool, size=n_pages, replace=False).astype(np.int32)
    else:
        raise ValueError(table)
    out = []
    for quant, scale in tensors:
        qp = lay_out_pages(quant, bt, pool, page_size, fill=np.int8(0))
        # unused slots: random quants, NaN scales
        used = np.zeros((pool, page_size), dtype=bool)
        j = np.arange(ctx)
        used[bt[j // page_size], j % page_size] = True
        qp[~used] = rng.integers(-127, 128, size=(int((~used).sum()), n_kv_heads, head_dim), dtype=np.int8)
        out += [qp, lay_out_pages(scale, bt, pool, page_size)]
    return Q8Case(name, history, rows, n_q_heads, n_kv_heads, head_dim, page_size, dtype, q, out[0], out[1],
                  out[2], out[3], bt, piece_rows)


@dataclass
class VarlenQ8Case:
    """A batch of sequences over one pool of 8-bit K/V pages (see
    make_varlen_q8_case)."""
    name: str
    seqs: list
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    page_size: int
    dtype: str
    q: np.ndarray          # [total_rows][Hq][d] uint16
    k_quant: np.ndarray    # [pool][ps][Hkv][d] int8
    k_scale: np.ndarray    # [pool][ps][Hkv][d/32] uint16 (fp16 bits)
    v_quant: np.ndarray
    v_scale: np.ndarray
    block_tables: np.ndarray   # [n][stride] int32
    cu_rows: np.ndarray        # [n + 1] int32
    history_lens: np.ndarray   # [n] int64

    @property
    def max_rows(self):
        return max([r for _, r in self.seqs] + [0])

    @property
    def max_context(self):
        return max([h + r for h, r in self.seqs] + [0])


def make_varlen_q8_case(name, seqs, n_q_heads, n_kv_heads, head_dim, page_size, dtype, seed, shared=(),
                        extra_pool=3):
    """make_varlen_case's batch over 8-bit pages: the same table layout
    (shared prefixes included); per sequence, in order, K then V quants
    uniform in [-127, 127] with fp16 scales 0.001 + 0.005 |N(0, 1)| per block
    of 32 values (values mostly below 2, so that a first chunk's rows, whose
    outputs are single V rows, stay below 4: fp16 rounds those by at most
    2^-10); then the pool order; then Q.  Slots no token uses hold random
    quants under 0xFFFF scales (fp16 NaN)."""
    rng = np.random.default_rng(seed)
    ctxs = [h + r for h, r in seqs]
    n_pages = [-(-c // page_size) for c in ctxs]
    pool = sum(n_pages) + extra_pool
    order = rng.permutation(pool)
    stride = max(n_pages + [1])
    tables = np.zeros((len(seqs), stride), dtype=np.int32)
    at = 0
    for s, n in enumerate(n_pages):
        tables[s, :n] = order[at:at + n]
        at += n
    skip = {}
    for dst, src, n in shared:
        tables[dst, :n] = tables[src, :n]
        skip[dst] = n * page_size
    nb = head_dim // 32
    pools = []
    for _ in range(2):
        pools.append([rng.integers(-127, 128, size=(pool, page_size, n_kv_heads, head_dim), dtype=np.int8),
                      np.full((pool, page_size, n_kv_heads, nb), POISON, dtype=np.uint16)])
    for s, c in enumerate(ctxs):
        j = np.arange(skip.get(s, 0), c)
        for quant_pool, scale_pool in pools:
            quant = rng.integers(-127, 128, size=(c, n_kv_heads, head_dim), dtype=np.int8)
            scale = (np.float32(0.001) + np.float32(0.005) * np.abs(rng.standard_normal((c, n_kv_heads, nb),
                                                                                        dtype=np.float32)))
            quant_pool[tables[s, j // page_size], j % page_size] = quant[j]
            scale_pool[tables[s, j // page_size], j % page_size] = scale.astype(np.float16).view(np.uint16)[j]
    cu = np.concatenate([[0], np.cumsum([r for _, r in seqs])]).astype(np.int32)
    q = ENCODERS[dtype](rng.standard_normal((int(cu[-1]), n_q_heads, head_dim), dtype=np.float32))
    hist = np.array([h for h, _ in seqs], dtype=np.int64)
    return VarlenQ8Case(name, list(seqs), n_q_heads, n_kv_heads, head_dim, page_size, dtype, q, pools[0][0],
                        pools[0][1], pools[1][0], pools[1][1], tables, cu, hist)
