"""Pins of oracle.attention against things other than itself.

  * a library routine: torch scaled_dot_product_attention in float64 on K/V
    gathered by a different route (flat slot indexing);
  * brute force: pure-Python loops on tiny shapes;
  * closed forms: one cached token -> its V; q = 0 or identical keys -> the
    mean of V; two tokens -> a logistic weight; per-head constant V -> the
    grouped-query head mapping;
  * invariants the pages state: any physical placement of the blocks gives the
    same result, and bytes past the context (tail slots, unused blocks, unused
    block-table entries) are never read.

Each pin is a function returning True/False so that the planted-mistake tests
at the bottom can show that a plausible bug in the oracle fails at least one.
"""

import math

import numpy as np
import pytest
import torch

import oracle.attention as att

# ---------------------------------------------------------------- problem maker


def make_problem(rng, num_seqs, h_q, h_kv, head_dim, block_size, ctxs, extra_blocks=3, poison=True):
    """Random f32 paged problem with a shuffled pool; returns a dict of arrays."""
    nbs = [-(-c // block_size) for c in ctxs]
    num_blocks = sum(nbs) + extra_blocks
    max_blocks = max(max(nbs), 1) + 2
    perm = rng.permutation(num_blocks)
    bt = np.full((num_seqs, max_blocks), -7, dtype=np.int32)  # unused entries are junk
    pos = 0
    for s, nb in enumerate(nbs):
        bt[s, :nb] = perm[pos:pos + nb]
        pos += nb
    kc = rng.standard_normal((num_blocks, h_kv, block_size, head_dim)).astype(np.float32)
    vc = rng.standard_normal((num_blocks, h_kv, block_size, head_dim)).astype(np.float32)
    if poison:
        used = np.zeros((num_blocks, block_size), dtype=bool)
        for s, c in enumerate(ctxs):
            for t in range(c):
                used[bt[s, t // block_size], t % block_size] = True
        kc.transpose(0, 2, 1, 3)[~used] = np.nan   # [blocks, slots, heads, d] view
        vc.transpose(0, 2, 1, 3)[~used] = np.inf
    q = rng.standard_normal((num_seqs, h_q, head_dim)).astype(np.float32)
    return dict(q=q, kc=kc, vc=vc, bt=bt, ctx=np.array(ctxs, dtype=np.int32), bs=block_size)


def run_oracle(p, scale=None, fn=None):
    fn = fn or att.paged_attention_decode
    return fn(p["q"].view(np.uint32), p["kc"].view(np.uint32), p["vc"].view(np.uint32), p["bt"], p["ctx"],
              q_dtype="f32", kv_dtype="f32", block_size=p["bs"], scale=scale)


def gather_flat(cache, bt_row, ctx, bs):
    """[h_kv, ctx, d] via slot = block * bs + offset into a [slots, h_kv, d] view."""
    nb, h_kv, _, d = cache.shape
    flat = np.transpose(cache, (0, 2, 1, 3)).reshape(nb * bs, h_kv, d)
    slots = np.array([bt_row[t // bs] * bs + t % bs for t in range(ctx)], dtype=np.int64)
    return np.transpose(flat[slots], (1, 0, 2)).astype(np.float64)

# ---------------------------------------------------------------- pins


def pin_sdpa(fn, seed=0):
    rng = np.random.default_rng(seed)
    p = make_problem(rng, 4, 8, 2, 16, 4, [9, 1, 13, 20])
    out = run_oracle(p, fn=fn)
    G = 8 // 2
    for s in range(4):
        c = int(p["ctx"][s])
        k = torch.from_numpy(gather_flat(p["kc"], p["bt"][s], c, 4)).repeat_interleave(G, dim=0)
        v = torch.from_numpy(gather_flat(p["vc"], p["bt"][s], c, 4)).repeat_interleave(G, dim=0)
        q = torch.from_numpy(p["q"][s].astype(np.float64))[:, None, :]
        ref = torch.nn.functional.scaled_dot_product_attention(q[None], k[None], v[None])[0, :, 0, :].numpy()
        if not np.allclose(out[s], ref, rtol=1e-12, atol=1e-12):
            return False
    return True


def brute_force(q, kc, vc, bt, ctx, bs, scale):
    S, Hq, D = q.shape
    Hkv = kc.shape[1]
    G = Hq // Hkv
    out = [[[0.0] * D for _ in range(Hq)] for _ in range(S)]
    for s in range(S):
        for g in range(Hq):
            h = g // G
            logits = []
            for t in range(int(ctx[s])):
                b = int(bt[s][t // bs])
                o = t % bs
                logits.append(scale * sum(float(q[s][g][d]) * float(kc[b][h][o][d]) for d in range(D)))
            if not logits:
                continue
            m = max(logits)
            w = [math.exp(z - m) for z in logits]
            tot = sum(w)
            for d in range(D):
                acc = 0.0
                for t in range(int(ctx[s])):
                    b = int(bt[s][t // bs])
                    acc += w[t] * float(vc[b][h][t % bs][d])
                out[s][g][d] = acc / tot
    return np.array(out)


def pin_brute_force(fn, seed=1):
    rng = np.random.default_rng(seed)
    for bs, ctxs, hq, hkv, d in [(1, [3, 1, 5], 2, 1, 4), (2, [7, 2], 4, 2, 3), (16, [40, 17, 1], 6, 3, 8), (3, [0, 10], 2, 2, 5)]:
        p = make_problem(rng, len(ctxs), hq, hkv, d, bs, ctxs)
        out = run_oracle(p, scale=0.37, fn=fn)
        ref = brute_force(p["q"], p["kc"], p["vc"], p["bt"], p["ctx"], bs, 0.37)
        if not np.allclose(out, ref, rtol=1e-12, atol=1e-13):
            return False
    return True


def pin_single_token(fn, seed=2):
    rng = np.random.default_rng(seed)
    p = make_problem(rng, 3, 8, 2, 8, 16, [1, 1, 1])
    out = run_oracle(p, fn=fn)
    for s in range(3):
        b = p["bt"][s, 0]
        for g in range(8):
            if not np.array_equal(out[s, g], p["vc"][b, g // 4, 0].astype(np.float64)):
                return False
    return True


def pin_uniform_weights(fn, seed=3):
    rng = np.random.default_rng(seed)
    p = make_problem(rng, 2, 4, 2, 8, 4, [11, 6])
    p["q"][0] = 0.0                               # q = 0: all logits equal
    for t in range(6):                            # seq 1: identical keys
        p["kc"][p["bt"][1, t // 4], :, t % 4, :] = p["kc"][p["bt"][1, 0], :, 0, :]
    out = run_oracle(p, fn=fn)
    for s in range(2):
        c = int(p["ctx"][s])
        v = gather_flat(p["vc"], p["bt"][s], c, 4)
        for g in range(4):
            if not np.allclose(out[s, g], v[g // 2].mean(axis=0), rtol=1e-13, atol=1e-14):
                return False
    return True


def pin_two_tokens(fn, seed=4):
    rng = np.random.default_rng(seed)
    p = make_problem(rng, 1, 1, 1, 4, 1, [2])
    out = run_oracle(p, scale=0.5, fn=fn)
    k = gather_flat(p["kc"], p["bt"][0], 2, 1)[0]
    v = gather_flat(p["vc"], p["bt"][0], 2, 1)[0]
    qv = p["q"][0, 0].astype(np.float64)
    w1 = 1.0 / (1.0 + math.exp(0.5 * (qv @ k[0] - qv @ k[1])))   # logistic weight of token 1
    return np.allclose(out[0, 0], w1 * v[1] + (1 - w1) * v[0], rtol=1e-12, atol=1e-14)


def pin_gqa_mapping(fn, seed=5):
    rng = np.random.default_rng(seed)
    p = make_problem(rng, 2, 12, 3, 4, 4, [9, 5], poison=False)
    for h in range(3):
        p["vc"][:, h] = float(h + 1)
    out = run_oracle(p, fn=fn)
    for g in range(12):
        if not np.allclose(out[:, g, :], float(g // 4 + 1), rtol=1e-12, atol=0):
            return False
    return True


def pin_placement_invariance(fn, seed=6):
    rng = np.random.default_rng(seed)
    p = make_problem(rng, 3, 4, 1, 8, 4, [13, 4, 9])
    base = run_oracle(p, fn=fn)
    nb = p["kc"].shape[0]
    perm = rng.permutation(nb)              # physical block b moves to perm[b]
    q = dict(p)
    q["kc"] = np.empty_like(p["kc"])
    q["vc"] = np.empty_like(p["vc"])
    q["kc"][perm] = p["kc"]
    q["vc"][perm] = p["vc"]
    bt = p["bt"].copy()
    for s in range(3):
        n = -(-int(p["ctx"][s]) // 4)
        bt[s, :n] = perm[p["bt"][s, :n]]
    q["bt"] = bt
    return np.array_equal(run_oracle(q, fn=fn), base)


def pin_never_reads_past_context(fn, seed=7):
    rng = np.random.default_rng(seed)
    p = make_problem(rng, 3, 4, 2, 8, 4, [10, 3, 0], poison=True)
    out = run_oracle(p, fn=fn)
    if not np.all(np.isfinite(out)):
        return False
    if not np.all(out[2] == 0.0):           # empty context -> 0
        return False
    clean = dict(p)
    clean["kc"] = np.nan_to_num(p["kc"], nan=123.0, posinf=-55.0)
    clean["vc"] = np.nan_to_num(p["vc"], nan=9.0, posinf=77.0)
    return np.array_equal(run_oracle(clean, fn=fn), out)


PINS = [pin_sdpa, pin_brute_force, pin_single_token, pin_uniform_weights, pin_two_tokens,
        pin_gqa_mapping, pin_placement_invariance, pin_never_reads_past_context]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_oracle_passes_pin(pin):
    assert pin(att.paged_attention_decode)


def test_default_scale_is_inverse_sqrt_head_dim():
    rng = np.random.default_rng(8)
    p = make_problem(rng, 2, 4, 2, 16, 4, [7, 12])
    assert np.array_equal(run_oracle(p), run_oracle(p, scale=1.0 / math.sqrt(16)))


def test_kv_scales_fold_linearly():
    rng = np.random.default_rng(9)
    codes_k = rng.integers(0, 0x7E, size=(6, 2, 4, 8), dtype=np.uint8)
    codes_v = rng.integers(0, 0x7E, size=(6, 2, 4, 8), dtype=np.uint8)
    q = rng.standard_normal((2, 4, 8)).astype(np.float32).view(np.uint32)
    bt = np.array([[0, 3, 5], [1, 2, 4]], dtype=np.int32)
    ctx = np.array([11, 9], dtype=np.int32)
    kw = dict(q_dtype="f32", kv_dtype="fp8", block_size=4)
    a = att.paged_attention_decode(q, codes_k, codes_v, bt, ctx, scale=0.25, k_scale=2.0, v_scale=4.0, **kw)
    b = att.paged_attention_decode(q, codes_k, codes_v, bt, ctx, scale=0.5, k_scale=1.0, v_scale=1.0, **kw)
    assert np.allclose(a, 4.0 * b, rtol=1e-12, atol=1e-12)


def test_rejects_bad_inputs():
    rng = np.random.default_rng(10)
    p = make_problem(rng, 1, 3, 2, 4, 4, [5])
    with pytest.raises(ValueError):
        run_oracle(p)                          # h_q not a multiple of h_kv
    p = make_problem(rng, 1, 2, 1, 4, 4, [5])
    p["bt"][0, 1] = 10 ** 6
    with pytest.raises(ValueError):
        run_oracle(p)                          # block id outside the pool

# ---------------------------------------------------------------- planted mistakes


def _mutant(**patches):
    """A copy of the oracle's entry point with some helpers replaced."""
    def fn(*args, **kw):
        saved = {k: getattr(att, k) for k in patches}
        try:
            for k, v in patches.items():
                setattr(att, k, v)
            return att.paged_attention_decode(*args, **kw)
        finally:
            for k, v in saved.items():
                setattr(att, k, v)
    return fn


def _wrong_head_map(q_head, h_q, h_kv):
    return q_head % h_kv                                    # interleaved instead of grouped


def _reads_whole_blocks(cache_bits, block_row, context_len, block_size, dtype, scale=1.0):
    n = -(-context_len // block_size) * block_size          # forgets the tail mask
    full = att.__dict__["_orig_resolve"](cache_bits, block_row, n, block_size, dtype, scale)
    return full


def _no_max_subtraction(q_vec, keys, values, scale):
    if keys.shape[0] == 0:
        return np.zeros(values.shape[1])
    w = np.exp(scale * (keys @ q_vec) * 1.0001)             # a slightly wrong temperature
    return (w @ values) / np.sum(w)


def _off_by_one_position(cache_bits, block_row, context_len, block_size, dtype, scale=1.0):
    if context_len == 0:
        return att.__dict__["_orig_resolve"](cache_bits, block_row, 0, block_size, dtype, scale)
    out = att.__dict__["_orig_resolve"](cache_bits, block_row, context_len + 1, block_size, dtype, scale)
    return out[:, 1:, :]                                   # reads positions 1..ctx instead of 0..ctx-1


att._orig_resolve = att.resolve_sequence

MUTANTS = {
    "wrong_gqa_mapping": _mutant(kv_head_of=_wrong_head_map),
    "reads_tail_slots": _mutant(resolve_sequence=_reads_whole_blocks),
    "wrong_temperature": _mutant(attend=_no_max_subtraction),
    "shifted_positions": _mutant(resolve_sequence=_off_by_one_position),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    fn = MUTANTS[name]
    failures = []
    for pin in PINS:
        try:
            ok = pin(fn)
        except Exception:
            ok = False
        failures.append(not ok)
    assert any(failures), f"no pin catches the planted mistake {name}"
