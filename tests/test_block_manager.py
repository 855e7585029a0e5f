"""The C++ block manager (pkv_bm_*) against the oracle allocator: bit-exact
slots, copy-on-write reports, block tables, free lists and refcounts over
random operation sequences and over the named workloads' allocation scripts.
Host code only; runs without a GPU."""

import numpy as np
import pytest

import paged_kv_cache_431_amd as pkv
import workloads
from oracle import allocator as al


def same_state(cpp, ora, seqs):
    assert cpp.num_free() == ora.num_free()
    assert cpp.free_list() == list(ora.free)
    assert [cpp.refcount(b) for b in range(ora.num_blocks)] == ora.refcount
    for s in seqs:
        assert cpp.block_table(s) == ora.block_table(s)


@pytest.mark.parametrize("seed", range(8))
def test_random_operations_match_oracle(seed):
    rng = np.random.default_rng(100 + seed)
    nb = int(rng.integers(8, 64))
    bs = int(rng.choice([1, 2, 3, 16, 32]))
    order = rng.permutation(nb)
    cpp = pkv.BlockManager(nb, bs, order)
    ora = al.BlockManager(nb, bs, order)
    live, next_id = [], 0
    for _ in range(500):
        op = int(rng.integers(0, 10))
        if op < 6 or not live:
            seq = int(rng.choice(live)) if live and rng.random() < 0.8 else next_id
            n = int(rng.integers(0, 3 * bs + 2))
            try:
                want = ora.append(seq, n)
            except al.OutOfBlocks:
                with pytest.raises(pkv.OutOfBlocks):
                    cpp.append(seq, n)
                same_state(cpp, ora, live)
                continue
            got = cpp.append(seq, n)
            assert got == (want[0], want[1])
            if seq == next_id:
                live.append(seq)
                next_id += 1
        elif op < 8:
            parent = int(rng.choice(live))
            cpp.fork(parent, next_id)
            ora.fork(parent, next_id)
            live.append(next_id)
            next_id += 1
        else:
            seq = int(rng.choice(live))
            cpp.free_seq(seq)
            ora.free_seq(seq)
            live.remove(seq)
        same_state(cpp, ora, live)


def test_invalid_requests_match_oracle():
    cpp = pkv.BlockManager(4, 4)
    for call in (lambda: cpp.append(-1, 1), lambda: cpp.append(0, -2), lambda: cpp.fork(5, 6),
                 lambda: cpp.free_seq(9), lambda: cpp.block_table(3)):
        with pytest.raises(pkv.PkvError) as e:
            call()
        assert e.value.status == pkv.PKV_EINVAL
    cpp.append(0, 1)
    with pytest.raises(pkv.PkvError):
        cpp.fork(0, 0)
    with pytest.raises(pkv.PkvError):
        pkv.BlockManager(4, 4, [0, 1, 1, 2])
    with pytest.raises(pkv.PkvError):
        pkv.BlockManager(0, 16)


def test_47_requests_fit_and_48th_does_not():
    """[OT] 12 GiB budget: 2,457 blocks hold 47 requests of 825 tokens, not 48."""
    cpp = pkv.BlockManager(2457, 16, np.random.default_rng(1).permutation(2457))
    for s in range(47):
        slots, cow = cpp.append(s, 825)
        assert len(cpp.block_table(s)[0]) == 52 and cow == (-1, -1)
    before = cpp.free_list()
    with pytest.raises(pkv.OutOfBlocks):
        cpp.append(47, 825)
    assert cpp.free_list() == before and len(before) == 13


@pytest.mark.parametrize("name", sorted(workloads.NAMED))
def test_workload_scripts_replay_identically(name):
    p = workloads.plan(workloads.get(name))
    cpp = pkv.BlockManager(p.num_blocks, p.workload.block_size, p.free_order)
    ora = al.BlockManager(p.num_blocks, p.workload.block_size, p.free_order)
    a = workloads.replay(p, cpp)
    b = workloads.replay(p, ora)
    assert np.array_equal(a.block_tables, b.block_tables)
    assert np.array_equal(a.slot_mapping, b.slot_mapping)
    assert np.array_equal(a.used_slots, b.used_slots)
    tables, lens = cpp.export(list(range(p.workload.num_seqs)), p.max_blocks_per_seq)
    assert np.array_equal(tables, a.block_tables)
    assert np.array_equal(lens, p.context_lens)
