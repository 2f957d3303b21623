"""Seeded synthetic workloads for the paged KV-cache hot path.

This module only draws inputs: context lengths, a shuffled free list, query /
key / value values, and the block tables and slot mappings that the block
manager hands out for them.  It computes no attention.  Both the GPU path and
the CPU oracle consume its output.

Recipe (shared by every workload):

* ``numpy.random.default_rng(seed)``; draw order lengths -> pool permutation
  -> Q -> K -> V.
* Values are N(0, 1) fp32, rounded once to the cache dtype with
  round-to-nearest-even (fp16 through numpy, bf16 by the usual bit rounding).
* The pool holds ceil(1.1 x blocks needed) blocks unless a workload fixes its
  size; the free list is a seeded permutation of the pool, so a sequence's
  blocks are scattered.
* Every pool slot starts as a NaN bit pattern: slots the scatter does not
  write must come through bit-identical, and unfilled slots of a last block
  must never reach an output.
* Block-table entries past a sequence's last block point at a pool block no
  sequence holds (still NaN-filled), so a kernel that read past a sequence's
  blocks would produce NaN rather than fault.

The arrays carry raw bits: float32 for fp32, uint16 for fp16/bf16.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

from .block_manager import NULL_BLOCK, BlockManager

F32, F16, BF16, FP8 = 0, 1, 2, 3      # FP8 (E4M3 codes) is a cache storage type only
DTYPE_NAMES = {F32: "f32", F16: "f16", BF16: "bf16", FP8: "fp8_e4m3"}
_NAN_BITS = {F32: np.float32(np.nan), F16: np.uint16(0x7E00), BF16: np.uint16(0x7FC0),
             FP8: np.uint8(0x7F)}


def round_to(x: np.ndarray, dtype: int) -> np.ndarray:
    """fp32 values -> raw bits of the cache dtype (round to nearest even)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == F32:
        return x
    if dtype == F16:
        return x.astype(np.float16).view(np.uint16)
    u = x.view(np.uint32)
    lsb = (u >> 16) & 1
    return ((u + np.uint32(0x7FFF) + lsb) >> 16).astype(np.uint16)


def storage_dtype(dtype: int):
    return {F32: np.float32, F16: np.uint16, BF16: np.uint16, FP8: np.uint8}[dtype]


@dataclass
class Op:
    """One setup or step operation on the cache: a scatter or a block copy."""
    kind: str                     # "scatter" or "copy"
    key: np.ndarray | None = None
    value: np.ndarray | None = None
    slots: np.ndarray | None = None
    pairs: np.ndarray | None = None


@dataclass
class Workload:
    name: str
    mode: str                     # "decode" or "prefill"
    dtype: int
    num_blocks: int
    num_kv_heads: int
    num_q_heads: int
    head_dim: int
    block_size: int
    context_lens: np.ndarray      # int32 [S]
    block_tables: np.ndarray      # int32 [S][max_blocks]
    q: np.ndarray                 # [S][Hq][d] (decode) or [Tq][Hq][d] (prefill)
    scale: float                  # fp32 1/sqrt(d)
    setup: list = field(default_factory=list)   # Ops that fill the history
    step_scatter: Op | None = None              # the step's new-token scatter
    query_start_loc: np.ndarray | None = None   # int32 [S+1] (prefill)
    seq_tokens_key: list = field(default_factory=list)    # per sequence [L][Hkv][d]
    seq_tokens_value: list = field(default_factory=list)
    partition_size: int = 0
    max_context_len: int = 0
    info: dict = field(default_factory=dict)
    window: int = 0               # sliding window in tokens (0: whole context)
    kv_dtype: int = -1            # cache storage dtype (-1: ``dtype``; FP8 for an 8-bit cache)
    k_scale: float = 1.0          # 8-bit cache: stored code = x / scale
    v_scale: float = 1.0

    @property
    def cache_dtype(self) -> int:
        return self.dtype if self.kv_dtype < 0 else self.kv_dtype

    @property
    def S(self) -> int:
        return int(self.context_lens.shape[0])

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    def empty_pools(self):
        nb, H, B, d = self.num_blocks, self.num_kv_heads, self.block_size, self.head_dim
        cd = self.cache_dtype
        st = storage_dtype(cd)
        x = 64 // np.dtype(st).itemsize           # key rows in 64-byte pieces
        k = np.full((nb, H, d // x, B, x), _NAN_BITS[cd], dtype=st)
        v = np.full((nb, H, d, B), _NAN_BITS[cd], dtype=st)
        return k, v

    def kv_bytes(self) -> int:
        """Bytes of live cached K and V that one attention pass reads once per KV head
        (under a sliding window, only the window's tokens)."""
        elt = {F32: 4, F16: 2, BF16: 2, FP8: 1}[self.cache_dtype]
        L = self.context_lens.astype(np.int64)
        if self.window > 0:
            L = np.minimum(L, self.window)
        return int(L.sum()) * 2 * self.num_kv_heads * self.head_dim * elt


def _scale(d: int) -> float:
    return float(np.float32(1.0 / math.sqrt(d)))


def _draw_values(rng, shape, dtype):
    return round_to(rng.standard_normal(shape, dtype=np.float32), dtype)


def _poison_block(bm: BlockManager) -> int:
    held = set()
    for sid in list(bm._seqs):
        held.update(bm.seq(sid).block_table)
    for b in range(bm.num_blocks - 1, -1, -1):
        if b not in held:
            return b
    raise ValueError("pool has no unused block for table padding")


def make_decode(name, seed, context_lens_fn, Hq, Hkv, d, B, dtype, max_context_len,
                num_blocks=None, pool_factor=1.1, partition_size=0, placement="shuffled",
                kv_dtype=-1, k_scale=1.0, v_scale=1.0):
    """Decode workload: every sequence holds ctx[s]-1 history tokens and appends one.

    ``context_lens_fn(rng)`` draws the context lengths (post-append, so they
    include the new token).  The step scatters the S new tokens, then attends.
    ``placement``: "shuffled" hands out physical blocks in a seeded random
    order; "contiguous" in pool order, so each sequence's blocks are
    consecutive and in logical order (an identity-like block table).  The
    values drawn are the same either way.  ``kv_dtype=FP8`` makes the cache
    8-bit (E4M3 codes of x / k_scale, x / v_scale); ``dtype`` stays the type of
    the queries and of the key/value rows written.
    """
    rng = np.random.default_rng(seed)
    ctx = np.asarray(context_lens_fn(rng), dtype=np.int32)
    S = ctx.shape[0]
    if (ctx < 1).any() or (ctx > max_context_len).any():
        raise ValueError("context lengths must lie in [1, max_context_len]")
    need = int(sum(-(-int(L) // B) for L in ctx))
    nb = int(num_blocks) if num_blocks is not None else int(math.ceil(pool_factor * need))
    if nb <= need:
        raise ValueError("pool must hold at least one block more than the workload needs")
    perm = rng.permutation(nb)
    if placement == "contiguous":
        perm = np.arange(nb)
    elif placement != "shuffled":
        raise ValueError(f"unknown placement {placement}")
    bm = BlockManager(nb, B, free_order=perm)
    q = _draw_values(rng, (S, Hq, d), dtype)
    total = int(ctx.astype(np.int64).sum())
    keys = _draw_values(rng, (total, Hkv, d), dtype)
    values = _draw_values(rng, (total, Hkv, d), dtype)
    cu = np.concatenate([[0], np.cumsum(ctx.astype(np.int64))])
    sids, hist_idx, hist_slots, new_slots = [], [], [], []
    for s in range(S):
        sid = bm.new_sequence()
        sids.append(sid)
        slots, copies = bm.append_tokens(sid, int(ctx[s]))
        assert not copies
        hist_idx.append(np.arange(cu[s], cu[s + 1] - 1))
        hist_slots.append(slots[:-1])
        new_slots.append(slots[-1])
    hist_idx = np.concatenate(hist_idx)
    new_idx = cu[1:] - 1
    mbps = -(-max_context_len // B)
    bt = bm.block_table_array(sids, mbps, pad=_poison_block(bm))
    wl = Workload(name=name, mode="decode", dtype=dtype, num_blocks=nb, num_kv_heads=Hkv,
                  num_q_heads=Hq, head_dim=d, block_size=B, context_lens=ctx, block_tables=bt,
                  q=q, scale=_scale(d), partition_size=partition_size,
                  max_context_len=int(max_context_len), kv_dtype=kv_dtype,
                  k_scale=float(np.float32(k_scale)), v_scale=float(np.float32(v_scale)))
    wl.setup.append(Op("scatter", key=np.ascontiguousarray(keys[hist_idx]),
                       value=np.ascontiguousarray(values[hist_idx]),
                       slots=np.concatenate(hist_slots).astype(np.int64)))
    wl.step_scatter = Op("scatter", key=np.ascontiguousarray(keys[new_idx]),
                         value=np.ascontiguousarray(values[new_idx]),
                         slots=np.asarray(new_slots, dtype=np.int64))
    wl.seq_tokens_key = [keys[cu[s]:cu[s + 1]] for s in range(S)]
    wl.seq_tokens_value = [values[cu[s]:cu[s + 1]] for s in range(S)]
    wl.info = {"blocks_needed": need, "tokens": total, "wasted_slots": bm.wasted_slots()}
    return wl


def make_prefill(name, seed, S, chunk, hist_fn, shared_prefix, Hq, Hkv, d, B, dtype,
                 max_context_len, pool_factor=1.1, pair_sharing=True):
    """Chunked-prefill workload over a paged cache with shared prefixes.

    Sequences come in pairs (0,1), (2,3), ...; the first ``shared_prefix``
    tokens of a pair are one draw held in the same physical blocks (reference
    count 2).  Setup writes the shared prefixes, forks the partner, appends the
    partner's own history (copy-on-write if the prefix ends inside a block),
    then the first member's own history.  The step scatters every sequence's
    ``chunk`` new tokens and runs the causal prefill for those rows.
    """
    rng = np.random.default_rng(seed)
    hist = np.asarray(hist_fn(rng), dtype=np.int64)
    assert hist.shape == (S,)
    ctx = (hist + chunk).astype(np.int32)
    if (ctx > max_context_len).any():
        raise ValueError("history + chunk exceeds max_context_len")
    if pair_sharing:
        assert S % 2 == 0 and (hist >= shared_prefix).all()
    # Blocks needed: unique blocks plus copy-on-write copies.
    need = 0
    for s in range(S):
        own = -(-int(ctx[s]) // B)
        if pair_sharing and s % 2 == 1:
            own -= shared_prefix // B          # full shared blocks are not duplicated
        need += own
    nb = int(math.ceil(pool_factor * need)) + 1
    perm = rng.permutation(nb)
    bm = BlockManager(nb, B, free_order=perm)
    Tq = S * chunk
    q = _draw_values(rng, (Tq, Hq, d), dtype)
    # One K/V draw per distinct token: a pair's partner reuses the shared prefix.
    uniq = int(ctx.astype(np.int64).sum()) - (shared_prefix * (S // 2) if pair_sharing else 0)
    kall = _draw_values(rng, (uniq, Hkv, d), dtype)
    vall = _draw_values(rng, (uniq, Hkv, d), dtype)
    seq_k, seq_v, cursor = [], [], 0
    for s in range(S):
        L = int(ctx[s])
        if pair_sharing and s % 2 == 1:
            own = L - shared_prefix
            k = np.concatenate([seq_k[s - 1][:shared_prefix], kall[cursor:cursor + own]])
            v = np.concatenate([seq_v[s - 1][:shared_prefix], vall[cursor:cursor + own]])
            cursor += own
        else:
            k, v = kall[cursor:cursor + L], vall[cursor:cursor + L]
            cursor += L
        seq_k.append(k)
        seq_v.append(v)
    assert cursor == uniq

    sids = [bm.new_sequence() if not (pair_sharing and s % 2 == 1) else None for s in range(S)]
    phase1_k, phase1_v, phase1_s = [], [], []
    phase2_k, phase2_v, phase2_s = [], [], []
    copies_all = []
    hist_done = [0] * S
    for s in range(0, S, 2 if pair_sharing else 1):
        if pair_sharing:
            a = s
            slots, cp = bm.append_tokens(sids[a], shared_prefix)
            assert not cp
            phase1_k.append(seq_k[a][:shared_prefix]); phase1_v.append(seq_v[a][:shared_prefix])
            phase1_s.append(slots)
            sids[a + 1] = bm.fork(sids[a])
            hist_done[a] = hist_done[a + 1] = shared_prefix
            for m in (a + 1, a):            # the partner diverges first
                n = int(hist[m]) - shared_prefix
                slots, cp = bm.append_tokens(sids[m], n)
                copies_all.extend(cp)
                phase2_k.append(seq_k[m][shared_prefix:hist[m]])
                phase2_v.append(seq_v[m][shared_prefix:hist[m]])
                phase2_s.append(slots)
                hist_done[m] = int(hist[m])
        else:
            slots, cp = bm.append_tokens(sids[s], int(hist[s]))
            phase1_k.append(seq_k[s][:hist[s]]); phase1_v.append(seq_v[s][:hist[s]])
            phase1_s.append(slots)
            hist_done[s] = int(hist[s])
    step_k, step_v, step_s = [], [], []
    for s in range(S):
        slots, cp = bm.append_tokens(sids[s], chunk)
        assert not cp, "chunk tokens land in private blocks"
        step_k.append(seq_k[s][hist[s]:]); step_v.append(seq_v[s][hist[s]:])
        step_s.append(slots)

    def cat(xs, shape_tail):
        xs = [x for x in xs if len(x)]
        if not xs:
            return np.zeros((0,) + shape_tail, dtype=storage_dtype(dtype))
        return np.ascontiguousarray(np.concatenate(xs))

    tail = (Hkv, d)
    mbps = -(-max_context_len // B)
    bt = bm.block_table_array(sids, mbps, pad=_poison_block(bm))
    qsl = np.arange(0, Tq + 1, chunk, dtype=np.int32)
    wl = Workload(name=name, mode="prefill", dtype=dtype, num_blocks=nb, num_kv_heads=Hkv,
                  num_q_heads=Hq, head_dim=d, block_size=B, context_lens=ctx, block_tables=bt,
                  q=q, scale=_scale(d), query_start_loc=qsl, max_context_len=int(max_context_len))
    wl.setup.append(Op("scatter", key=cat(phase1_k, tail), value=cat(phase1_v, tail),
                       slots=np.concatenate(phase1_s).astype(np.int64)))
    if copies_all:
        wl.setup.append(Op("copy", pairs=np.asarray(copies_all, dtype=np.int32).reshape(-1, 2)))
    if phase2_s:
        wl.setup.append(Op("scatter", key=cat(phase2_k, tail), value=cat(phase2_v, tail),
                           slots=np.concatenate(phase2_s).astype(np.int64)))
    wl.step_scatter = Op("scatter", key=cat(step_k, tail), value=cat(step_v, tail),
                         slots=np.concatenate(step_s).astype(np.int64))
    wl.seq_tokens_key = seq_k
    wl.seq_tokens_value = seq_v
    wl.info = {"blocks_needed": need, "cow_copies": len(copies_all), "histories": hist.tolist()}
    return wl


def make_sliding_decode(name, seed, context_lens_fn, window, Hq, Hkv, d, B, dtype, max_context_len,
                        partition_size=0, pool_factor=1.1, chunk=None):
    """Decode under a sliding window of ``window`` tokens, with block release.

    Each sequence's history is appended in chunks (default: ``window`` tokens),
    and after every chunk the blocks outside the window of the newest token are
    released (``remove_skipped_blocks``) and return to the free list, where
    later chunks and other sequences take them again; then the new token is
    appended and the release runs once more.  Only the positions still held
    at the end, [first_pos[s], L), carry drawn values: they are scattered by
    the setup (the new token by the step).  Table entries of released blocks
    point at a NaN-filled block no sequence holds, so reading one would show.
    """
    rng = np.random.default_rng(seed)
    ctx = np.asarray(context_lens_fn(rng), dtype=np.int64)
    S = ctx.shape[0]
    if (ctx < 1).any() or (ctx > max_context_len).any() or window < 1:
        raise ValueError("context lengths must lie in [1, max_context_len], window >= 1")
    chunk = int(chunk or window)
    first_blk = np.maximum(0, ctx - window) // B
    held = -(-ctx // B) - first_blk
    need = int(held.sum())
    nb = int(math.ceil(pool_factor * need)) + -(-chunk // B) + 3
    perm = rng.permutation(nb)
    bm = BlockManager(nb, B, free_order=perm)
    q = _draw_values(rng, (S, Hq, d), dtype)
    kept = (ctx - first_blk * B).astype(np.int64)          # positions [first_pos, L)
    total = int(kept.sum())
    keys = _draw_values(rng, (total, Hkv, d), dtype)
    values = _draw_values(rng, (total, Hkv, d), dtype)
    sids, released = [], 0
    for s in range(S):
        sid = bm.new_sequence()
        sids.append(sid)
        pos, L = 0, int(ctx[s])
        while pos < L - 1:
            n = min(chunk, L - 1 - pos)
            bm.append_tokens(sid, n)
            pos += n
            released += bm.remove_skipped_blocks(sid, window)
        bm.append_tokens(sid, 1)                           # the step's token
        released += bm.remove_skipped_blocks(sid, window)
        tbl = bm.seq(sid).block_table
        assert all(b == NULL_BLOCK for b in tbl[:first_blk[s]])
        assert all(b != NULL_BLOCK for b in tbl[first_blk[s]:])
    mbps = -(-max_context_len // B)
    poison = _poison_block(bm)
    bt = bm.block_table_array(sids, mbps, pad=poison)
    bt[bt == NULL_BLOCK] = poison
    cu = np.concatenate([[0], np.cumsum(kept)])
    hist_idx, hist_slots, new_idx, new_slots = [], [], [], []
    for s in range(S):
        p0, L = int(first_blk[s] * B), int(ctx[s])
        pos = np.arange(p0, L)
        slots = bt[s, pos // B].astype(np.int64) * B + pos % B
        hist_idx.append(np.arange(cu[s], cu[s + 1] - 1))
        hist_slots.append(slots[:-1])
        new_idx.append(cu[s + 1] - 1)
        new_slots.append(slots[-1])
    wl = Workload(name=name, mode="decode", dtype=dtype, num_blocks=nb, num_kv_heads=Hkv,
                  num_q_heads=Hq, head_dim=d, block_size=B, context_lens=ctx.astype(np.int32),
                  block_tables=bt, q=q, scale=_scale(d), partition_size=partition_size,
                  max_context_len=int(max_context_len), window=int(window))
    wl.setup.append(Op("scatter", key=np.ascontiguousarray(keys[np.concatenate(hist_idx)]),
                       value=np.ascontiguousarray(values[np.concatenate(hist_idx)]),
                       slots=np.concatenate(hist_slots).astype(np.int64)))
    wl.step_scatter = Op("scatter", key=np.ascontiguousarray(keys[new_idx]),
                         value=np.ascontiguousarray(values[new_idx]),
                         slots=np.asarray(new_slots, dtype=np.int64))
    wl.seq_tokens_key = [keys[cu[s]:cu[s + 1]] for s in range(S)]
    wl.seq_tokens_value = [values[cu[s]:cu[s + 1]] for s in range(S)]
    wl.info = {"blocks_needed": need, "released_blocks": released,
               "first_pos": (first_blk * B).tolist(), "window_tokens": int(np.minimum(ctx, window).sum())}
    return wl


def make_mixed(name, seed, decode_lens_fn, chunk_hist_fn, chunk_lens, Hq, Hkv, d, B, dtype,
               max_context_len, pool_factor=1.1, partition_size=0):
    """One step that batches decode rows with prefill chunks, decode sequences first.

    ``decode_lens_fn(rng)`` draws the decode sequences' context lengths
    (post-append); ``chunk_hist_fn(rng)`` the history of each chunk sequence,
    which then appends ``chunk_lens[i]`` new tokens.  Setup scatters every
    history; the step scatters the decode tokens and the chunk tokens, then
    attends.  query_start_loc is [0, 1, ..., nd, nd + c0, ...]; blocks are
    handed out in a seeded random order.
    """
    rng = np.random.default_rng(seed)
    dctx = np.asarray(decode_lens_fn(rng), dtype=np.int64)
    hist = np.asarray(chunk_hist_fn(rng), dtype=np.int64)
    clen = np.asarray(chunk_lens, dtype=np.int64)
    assert hist.shape == clen.shape
    nd = dctx.shape[0]
    ctx = np.concatenate([dctx, hist + clen]).astype(np.int32)
    qlen = np.concatenate([np.ones(nd, dtype=np.int64), clen])
    if (ctx < 1).any() or (ctx > max_context_len).any() or (clen < 1).any():
        raise ValueError("context lengths must lie in [1, max_context_len], chunks non-empty")
    S = ctx.shape[0]
    need = int(sum(-(-int(L) // B) for L in ctx))
    nb = int(math.ceil(pool_factor * need)) + 1
    perm = rng.permutation(nb)
    bm = BlockManager(nb, B, free_order=perm)
    qsl = np.concatenate([[0], np.cumsum(qlen)]).astype(np.int32)
    q = _draw_values(rng, (int(qsl[-1]), Hq, d), dtype)
    total = int(ctx.astype(np.int64).sum())
    keys = _draw_values(rng, (total, Hkv, d), dtype)
    values = _draw_values(rng, (total, Hkv, d), dtype)
    cu = np.concatenate([[0], np.cumsum(ctx.astype(np.int64))])
    sids, hist_idx, hist_slots, new_idx, new_slots = [], [], [], [], []
    for s in range(S):
        sid = bm.new_sequence()
        sids.append(sid)
        slots, copies = bm.append_tokens(sid, int(ctx[s]))
        assert not copies
        h = int(ctx[s] - qlen[s])
        hist_idx.append(np.arange(cu[s], cu[s] + h))
        hist_slots.append(slots[:h])
        new_idx.append(np.arange(cu[s] + h, cu[s + 1]))
        new_slots.append(slots[h:])
    hist_idx = np.concatenate(hist_idx)
    new_idx = np.concatenate(new_idx)
    mbps = -(-max_context_len // B)
    bt = bm.block_table_array(sids, mbps, pad=_poison_block(bm))
    wl = Workload(name=name, mode="mixed", dtype=dtype, num_blocks=nb, num_kv_heads=Hkv,
                  num_q_heads=Hq, head_dim=d, block_size=B, context_lens=ctx, block_tables=bt,
                  q=q, scale=_scale(d), query_start_loc=qsl, partition_size=partition_size,
                  max_context_len=int(max_context_len))
    wl.setup.append(Op("scatter", key=np.ascontiguousarray(keys[hist_idx]),
                       value=np.ascontiguousarray(values[hist_idx]),
                       slots=np.concatenate(hist_slots).astype(np.int64)))
    wl.step_scatter = Op("scatter", key=np.ascontiguousarray(keys[new_idx]),
                         value=np.ascontiguousarray(values[new_idx]),
                         slots=np.concatenate(new_slots).astype(np.int64))
    wl.seq_tokens_key = [keys[cu[s]:cu[s + 1]] for s in range(S)]
    wl.seq_tokens_value = [values[cu[s]:cu[s + 1]] for s in range(S)]
    wl.info = {"blocks_needed": need, "num_decode_seqs": nd, "chunk_rows": int(clen.sum()),
               "tokens": total}
    return wl


# ---------------------------------------------------------------------------
# The five workloads (sizes as stated for each), plus small variants for tests.
# ---------------------------------------------------------------------------

def tiny_decode_f32():
    """4 sequences, contexts {6,17,33,64}, 8 heads, d 64, B 16, 32-block pool, fp32."""
    return make_decode("tiny_decode_f32", 1, lambda rng: [6, 17, 33, 64], Hq=8, Hkv=8, d=64, B=16,
                       dtype=F32, max_context_len=64, num_blocks=32)


def llama13b_decode_f16(S=64, lo=128, hi=2048, seed=2, partition_size=512, B=16,
                        placement="shuffled"):
    """LLaMA-2-13B-shaped single-layer decode: 40 heads, d 128, B 16, fp16, L ~ U[lo, hi]."""
    return make_decode(f"llama13b_decode_f16_S{S}", seed,
                       lambda rng: rng.integers(lo, hi + 1, size=S), Hq=40, Hkv=40, d=128, B=B,
                       dtype=F16, max_context_len=hi, partition_size=partition_size,
                       placement=placement)


def llama13b_decode_fp8(S=64, lo=128, hi=2048, seed=2, partition_size=512, B=16,
                        k_scale=0.0135, v_scale=0.0135):
    """The LLaMA-2-13B-shaped decode over an 8-bit (E4M3) cache: fp16 queries and inputs,
    per-tensor scales about 6 sigma / 448 of the N(0, 1) values."""
    return make_decode(f"llama13b_decode_fp8_S{S}", seed,
                       lambda rng: rng.integers(lo, hi + 1, size=S), Hq=40, Hkv=40, d=128, B=B,
                       dtype=F16, max_context_len=hi, partition_size=partition_size,
                       kv_dtype=FP8, k_scale=k_scale, v_scale=v_scale)


def long_context_split_f16(S=16, lo=2048, hi=4096, seed=3, partition_size=512):
    """Long-context decode with 512-token split-KV partitions: 40 heads, d 128, B 16, fp16."""
    return make_decode(f"long_split_f16_S{S}", seed, lambda rng: rng.integers(lo, hi + 1, size=S),
                       Hq=40, Hkv=40, d=128, B=16, dtype=F16, max_context_len=4096,
                       partition_size=partition_size)


def lognormal_lengths(S, median=1024, sigma=1.0, lo=16, hi=8192):
    def draw(rng):
        x = rng.lognormal(mean=math.log(median), sigma=sigma, size=S)
        return np.clip(np.rint(x), lo, hi).astype(np.int64)
    return draw


def gqa_decode_bf16(B=16, S=256, seed=4, max_context_len=8192, lengths=None, partition_size=2048):
    """GQA decode: 32 query heads over 8 KV heads, d 128, bf16, lognormal(median 1024) lengths."""
    fn = lengths or lognormal_lengths(S, hi=max_context_len)
    return make_decode(f"gqa_decode_bf16_B{B}_S{S}", seed, fn, Hq=32, Hkv=8, d=128, B=B,
                       dtype=BF16, max_context_len=max_context_len, partition_size=partition_size)


def chunked_prefill_bf16(S=8, chunk=512, hist_lo=1024, hist_hi=3584, shared_prefix=1024, seed=5,
                         Hq=32, Hkv=32, max_context_len=4096, hist_fn=None, pair_sharing=True):
    """Chunked prefill: 512-row chunks over paged histories, pairs sharing their first tokens."""
    fn = hist_fn or (lambda rng: rng.integers(hist_lo, hist_hi + 1, size=S))
    return make_prefill(f"chunked_prefill_bf16_S{S}", seed, S, chunk, fn, shared_prefix, Hq=Hq,
                        Hkv=Hkv, d=128, B=16, dtype=BF16, max_context_len=max_context_len,
                        pair_sharing=pair_sharing)


def mixed_step_f16(nd=64, n_chunks=2, chunk=512, lo=128, hi=2048, hist_lo=1024, hist_hi=1536,
                   seed=6, partition_size=512, Hq=40, Hkv=40, dtype=F16):
    """One LLaMA-2-13B-shaped step: nd decode rows (L ~ U[lo, hi]) batched with n_chunks
    prefill chunks of ``chunk`` rows over histories ~ U[hist_lo, hist_hi]; d 128, B 16."""
    return make_mixed(f"mixed_step_f16_D{nd}_C{n_chunks}x{chunk}", seed,
                      lambda rng: rng.integers(lo, hi + 1, size=nd),
                      lambda rng: rng.integers(hist_lo, hist_hi + 1, size=n_chunks),
                      [chunk] * n_chunks, Hq=Hq, Hkv=Hkv, d=128, B=16, dtype=dtype,
                      max_context_len=max(hi, hist_hi + chunk), partition_size=partition_size)


def sliding_window_gqa_bf16(S=64, lo=1024, hi=16384, window=4096, seed=7, partition_size=-1, B=16):
    """Mistral-7B-shaped sliding-window decode: 32 q / 8 kv heads, d 128, window 4096,
    L ~ U[lo, hi], bf16; blocks before each window released."""
    return make_sliding_decode(f"sliding_window_gqa_bf16_S{S}_W{window}", seed,
                               lambda rng: rng.integers(lo, hi + 1, size=S), window, Hq=32, Hkv=8,
                               d=128, B=B, dtype=BF16, max_context_len=hi,
                               partition_size=partition_size)
