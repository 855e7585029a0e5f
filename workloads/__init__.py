"""Seeded synthetic inputs shaped like the pages' worked examples.

This module is shared by the tests, the benchmark and the smoke check.  It
holds none of the method's arithmetic: it draws random numbers, writes
allocation *scripts* (which sequence grows by how many tokens, which sequence
forks from which) and fills pools with values.  Block tables and slot
mappings come from replaying a script through a block manager -- the C++ one
on the product side, the Python one in the oracle -- so the two can be
compared.  The only thing it knows of the method is the pool layout
[num_blocks, h_kv, block_size, head_dim], which it needs to fill and poison
the pool.

Draw order for a workload with seed S (numpy.random.default_rng(S) for the
script, torch.Generator seeded from S for tensors):
  1. context lengths (when random), 2. block order / growth schedule,
  3. q, 4. pool K, 5. pool V, 6. the new tokens' K and V.
Values are N(0, 1) float32, then rounded to the storage type (torch casts,
round-to-nearest-even).  FP8 pools take one scale per tensor,
amax(|x|) / 448 over that tensor's pool and new-token values, and store
(x / scale) cast to float8_e4m3fn.  Slots not holding a token before the
decode step (unallocated blocks, tail slots, the new token's own slot) are
poisoned with NaN (0x7F for FP8) unless poison=False.

Named workloads (after the pages' examples):
  tiny-f32-4seq          4 sequences, contexts {200, 825, 17, 1}, h_q 8 /
                         h_kv 2, d 64, fp32, 128-block pool, shuffled.
  gqa70b-bf16-47x825     the 12 GiB snapshot: 47 sequences x 825 tokens,
                         h_q 64 / h_kv 8, d 128, bf16, 2,457-block pool
                         (one layer), shuffled free list.
  gqa8b-bf16-256xU4096   256 sequences, contexts uniform in [1, 4096], h_q 32 /
                         h_kv 8, d 128, bf16, growth interleaved across
                         sequences so physical blocks are scattered.
  mha-f16-64x4096        64 sequences x 4096 tokens, h_q = h_kv = 32, d 128,
                         fp16, shuffled 16,384-block pool.
  fp8-prefix-32xU32768   32 sequences, contexts uniform in [8000, 32768],
                         h_q 64 / h_kv 8, d 128, K/V fp8 e4m3 + fp32 scales,
                         bf16 queries; groups of 8 share a 2,048-token
                         (128-block) prefix.
"""

from dataclasses import dataclass, field, replace

import numpy as np
import torch

TORCH_DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16, "fp8": torch.uint8}
ELEMENT_BYTES = {"f32": 4, "f16": 2, "bf16": 2, "fp8": 1}


@dataclass(frozen=True)
class Workload:
    name: str
    num_seqs: int
    h_q: int
    h_kv: int
    head_dim: int
    block_size: int
    q_dtype: str
    kv_dtype: str
    new_dtype: str
    seed: int
    contexts: tuple = ()          # explicit context lengths (after the decode step), or
    context_range: tuple = ()     # (lo, hi) inclusive, drawn uniformly
    layout: str = "chunks"        # "chunks" | "interleaved" | "shared_prefix"
    num_blocks: int = 0           # 0: exactly the blocks the script needs
    extra_blocks: int = 0         # spare blocks on top of what is needed
    shuffle: bool = True          # shuffled free list (else ascending)
    prefix_tokens: int = 0        # shared_prefix: tokens shared by a group
    group_size: int = 1           # shared_prefix: sequences per group
    max_blocks_per_seq: int = 0   # 0: the longest sequence's block count

    @property
    def group(self):
        return self.h_q // self.h_kv


NAMED = {
    "tiny-f32-4seq": Workload("tiny-f32-4seq", 4, 8, 2, 64, 16, "f32", "f32", "f32", 431001,
                              contexts=(200, 825, 17, 1), num_blocks=128),
    "gqa70b-bf16-47x825": Workload("gqa70b-bf16-47x825", 47, 64, 8, 128, 16, "bf16", "bf16", "bf16", 431002,
                                   contexts=(825,) * 47, num_blocks=2457),
    "gqa8b-bf16-256xU4096": Workload("gqa8b-bf16-256xU4096", 256, 32, 8, 128, 16, "bf16", "bf16", "bf16", 431003,
                                     context_range=(1, 4096), layout="interleaved", shuffle=False,
                                     max_blocks_per_seq=256),
    "mha-f16-64x4096": Workload("mha-f16-64x4096", 64, 32, 32, 128, 16, "f16", "f16", "f16", 431004,
                                contexts=(4096,) * 64, num_blocks=16384),
    "fp8-prefix-32xU32768": Workload("fp8-prefix-32xU32768", 32, 64, 8, 128, 16, "bf16", "fp8", "bf16", 431005,
                                     context_range=(8000, 32768), layout="shared_prefix", prefix_tokens=2048,
                                     group_size=8, max_blocks_per_seq=2048),
}


def get(name, **overrides):
    wl = NAMED[name]
    return replace(wl, **overrides) if overrides else wl


@dataclass
class Plan:
    """An allocation script and the sizes it implies."""
    workload: Workload
    context_lens: np.ndarray      # int32 [num_seqs], after the decode step
    num_blocks: int
    max_blocks_per_seq: int
    free_order: np.ndarray        # int32 [num_blocks]
    ops: list = field(default_factory=list)   # ("append", seq, n) / ("fork", parent, child)
    decode_seqs: list = field(default_factory=list)  # one new token each, in this order

    @property
    def max_context_len(self):
        return int(self.context_lens.max()) if len(self.context_lens) else 0


def _ceil_div(a, b):
    return -(-a // b)


def plan(wl: Workload) -> Plan:
    rng = np.random.default_rng(wl.seed)
    if wl.contexts:
        ctx = np.array(wl.contexts, dtype=np.int64)
    else:
        lo, hi = wl.context_range
        ctx = rng.integers(lo, hi, size=wl.num_seqs, endpoint=True)
    bs = wl.block_size
    nb = [_ceil_div(int(c), bs) for c in ctx]
    ops = []
    if wl.layout == "shared_prefix":
        assert wl.prefix_tokens % bs == 0 and all(int(c) > wl.prefix_tokens for c in ctx)
        shared = wl.prefix_tokens // bs
        groups = _ceil_div(wl.num_seqs, wl.group_size)
        needed = groups * shared + sum(n - shared for n in nb)
        for g in range(groups):
            members = list(range(g * wl.group_size, min((g + 1) * wl.group_size, wl.num_seqs)))
            ops.append(("append", members[0], wl.prefix_tokens))
            for child in members[1:]:
                ops.append(("fork", members[0], child))
        for s in range(wl.num_seqs):
            ops.append(("append", s, int(ctx[s]) - 1 - wl.prefix_tokens))
    elif wl.layout == "interleaved":
        needed = sum(nb)
        held = [0] * wl.num_seqs
        target = [int(c) - 1 for c in ctx]
        for s in range(wl.num_seqs):
            ops.append(("append", s, 0))
        open_seqs = [s for s in range(wl.num_seqs) if target[s] > 0]
        while open_seqs:
            k = int(rng.integers(0, len(open_seqs)))
            s = open_seqs[k]
            n = min(bs, target[s] - held[s])       # fills (at most) one more block
            ops.append(("append", s, n))
            held[s] += n
            if held[s] == target[s]:
                open_seqs.pop(k)
    else:
        needed = sum(nb)
        for s in range(wl.num_seqs):
            ops.append(("append", s, max(int(ctx[s]) - 1, 0)))
    num_blocks = wl.num_blocks or (needed + wl.extra_blocks)
    assert num_blocks >= needed, "pool too small for the workload"
    free_order = rng.permutation(num_blocks) if wl.shuffle else np.arange(num_blocks)
    mb = wl.max_blocks_per_seq or max(max(nb), 1)
    # a sequence with an empty context takes no new token this step
    return Plan(wl, ctx.astype(np.int32), int(num_blocks), int(mb), free_order.astype(np.int32), ops,
                [s for s in range(wl.num_seqs) if int(ctx[s]) > 0])


@dataclass
class Replay:
    block_tables: np.ndarray   # int32 [num_seqs, max_blocks_per_seq], -1 past the used blocks
    slot_mapping: np.ndarray   # int64 [num_seqs]: the decode step's slot per sequence (-1: none)
    used_slots: np.ndarray     # int64: every slot holding a token before the decode step


def replay(p: Plan, manager) -> Replay:
    """Run the script through `manager` (append(seq, n) -> (slots, cow), fork,
    block_table(seq) -> (table, n_tokens)) and collect its answers."""
    used = []
    for op, a, b in p.ops:
        if op == "append":
            slots, _ = manager.append(a, b)
            used.extend(slots)
        else:
            manager.fork(a, b)
    new_slots = [-1] * p.workload.num_seqs
    for s in p.decode_seqs:
        slots, _ = manager.append(s, 1)
        new_slots[s] = slots[0]
    bt = np.full((p.workload.num_seqs, p.max_blocks_per_seq), -1, dtype=np.int32)
    for s in range(p.workload.num_seqs):
        table, n = manager.block_table(s)
        assert n == int(p.context_lens[s])
        bt[s, :len(table)] = table
    return Replay(bt, np.array(new_slots, dtype=np.int64), np.unique(np.array(used, dtype=np.int64)))


def _generator(seed, stream, device):
    g = torch.Generator(device=device)
    g.manual_seed(seed * 16 + stream)
    return g


def _randn(shape, gen, device, chunk_rows=512):
    """N(0,1) float32 in row chunks (bounded temporaries for large pools)."""
    out = torch.empty(shape, dtype=torch.float32, device=device)
    for i in range(0, shape[0], chunk_rows):
        rows = min(chunk_rows, shape[0] - i)
        out[i:i + rows] = torch.randn((rows,) + tuple(shape[1:]), generator=gen, device=device)
    return out


def _store(x, dtype):
    return x.to(TORCH_DTYPES[dtype]) if dtype != "fp8" else x


@dataclass
class Tensors:
    q: torch.Tensor
    k_cache: torch.Tensor       # raw storage (uint8 for fp8)
    v_cache: torch.Tensor
    new_k: torch.Tensor         # [num_seqs, h_kv, head_dim] in new_dtype
    new_v: torch.Tensor
    k_scale: float = 1.0
    v_scale: float = 1.0


def make_tensors(p: Plan, rp: Replay, device="cpu", poison=True, pool_seed_offset=0) -> Tensors:
    """Draw q, the pools and the new tokens.  pool_seed_offset selects another
    independent pool (the benchmark's per-layer pools) with the same tables."""
    wl = p.workload
    dev = torch.device(device)
    seed = wl.seed + 1000003 * pool_seed_offset
    shape = (p.num_blocks, wl.h_kv, wl.block_size, wl.head_dim)
    q = _randn((wl.num_seqs, wl.h_q, wl.head_dim), _generator(wl.seed, 3, dev), dev).to(TORCH_DTYPES[wl.q_dtype])
    kf = _randn(shape, _generator(seed, 4, dev), dev)
    vf = _randn(shape, _generator(seed, 5, dev), dev)
    gen_new = _generator(seed, 6, dev)
    nk = _randn((wl.num_seqs, wl.h_kv, wl.head_dim), gen_new, dev).to(TORCH_DTYPES[wl.new_dtype])
    nv = _randn((wl.num_seqs, wl.h_kv, wl.head_dim), gen_new, dev).to(TORCH_DTYPES[wl.new_dtype])
    k_scale = v_scale = 1.0
    if wl.kv_dtype == "fp8":
        k_scale = float(max(kf.abs().max().item(), nk.float().abs().max().item()) / 448.0)
        v_scale = float(max(vf.abs().max().item(), nv.float().abs().max().item()) / 448.0)
        kc = _to_fp8(kf, k_scale)
        vc = _to_fp8(vf, v_scale)
    else:
        kc = kf.to(TORCH_DTYPES[wl.kv_dtype])
        vc = vf.to(TORCH_DTYPES[wl.kv_dtype])
    del kf, vf
    if poison:
        mask = torch.ones(p.num_blocks * wl.block_size, dtype=torch.bool, device=dev)
        mask[torch.from_numpy(rp.used_slots).to(dev)] = False
        mask = mask.view(p.num_blocks, 1, wl.block_size, 1).expand(shape)
        bad = 0x7F if wl.kv_dtype == "fp8" else float("nan")
        kc.masked_fill_(mask, bad)
        vc.masked_fill_(mask, bad)
    return Tensors(q, kc, vc, nk, nv, k_scale, v_scale)


def multi_queries(wl: Workload, new_tokens, device="cpu"):
    """Query rows for several new tokens per sequence: q [sum(new_tokens),
    h_q, head_dim] in q_dtype (seeded N(0,1), its own stream) and the int32
    row offsets query_start [num_seqs + 1]."""
    dev = torch.device(device)
    qs = np.concatenate([[0], np.cumsum(np.asarray(new_tokens, dtype=np.int64))]).astype(np.int32)
    q = _randn((int(qs[-1]), wl.h_q, wl.head_dim), _generator(wl.seed, 7, dev), dev).to(TORCH_DTYPES[wl.q_dtype])
    return q, qs


def _to_fp8(x, scale, chunk_rows=512):
    out = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    s = torch.tensor(scale, dtype=torch.float32, device=x.device)
    for i in range(0, x.shape[0], chunk_rows):
        out[i:i + chunk_rows] = (x[i:i + chunk_rows] / s).to(torch.float8_e4m3fn).view(torch.uint8)
    return out


def kv_bytes(p: Plan, unique=True):
    """Algorithmic K+V bytes one decode call must read: sum over sequences of
    context_len * 2 * h_kv * head_dim * element bytes.  With unique=True,
    prefix blocks shared by several sequences count once."""
    wl = p.workload
    per_token = 2 * wl.h_kv * wl.head_dim * ELEMENT_BYTES[wl.kv_dtype]
    total = int(p.context_lens.astype(np.int64).sum()) * per_token
    if unique and wl.layout == "shared_prefix":
        groups = _ceil_div(wl.num_seqs, wl.group_size)
        dup_seqs = wl.num_seqs - groups
        total -= dup_seqs * wl.prefix_tokens * per_token
    return total
