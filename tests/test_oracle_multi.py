"""Pins of oracle.attention.paged_attention_multi (several new query tokens
per sequence, causal) against things other than itself.

  * a library routine: torch scaled_dot_product_attention with its own
    causal mask (is_causal=True) on a square problem: every cached token of
    the sequence is given a query row, the new tokens' rows are the last m,
    and only those are compared; K/V gathered by flat slot indexing;
  * the decode oracle (pinned on its own in test_oracle_attention.py): new
    token i gives what one decode step gives over the first ctx - m + i + 1
    positions, and m = 1 everywhere is exactly decode;
  * special cases: a token that precedes every cached position (more new
    tokens than cached ones) gets 0; bytes past a context are never read.

Each pin returns True/False so that the planted-mistake tests at the bottom
can show that a plausible bug in the causal bound fails at least one pin.
"""

import numpy as np
import pytest
import torch

import oracle.attention as att
from test_oracle_attention import gather_flat, make_problem


def make_multi(rng, h_q, h_kv, head_dim, block_size, ctxs, ms, poison=True):
    """Paged f32 problem plus q rows for ms[s] new tokens of each sequence."""
    p = make_problem(rng, len(ctxs), h_q, h_kv, head_dim, block_size, ctxs, poison=poison)
    qs = np.concatenate([[0], np.cumsum(ms)]).astype(np.int32)
    p["q"] = rng.standard_normal((int(qs[-1]), h_q, head_dim)).astype(np.float32)
    p["qs"] = qs
    return p


def run_multi(p, fn=None, ctx=None):
    fn = fn or att.paged_attention_multi
    return fn(p["q"].view(np.uint32), p["kc"].view(np.uint32), p["vc"].view(np.uint32), p["bt"],
              p["ctx"] if ctx is None else ctx, p["qs"], q_dtype="f32", kv_dtype="f32", block_size=p["bs"])

# ---------------------------------------------------------------- pins


def pin_sdpa_causal(fn, seed=10):
    """Library causal mask on the whole context, new rows = the last m."""
    rng = np.random.default_rng(seed)
    h_q, h_kv, d, bs = 8, 2, 16, 4
    ctxs, ms = [9, 13, 5, 20], [3, 13, 1, 6]
    p = make_multi(rng, h_q, h_kv, d, bs, ctxs, ms)
    out = fn(p)
    G = h_q // h_kv
    for s, (c, m) in enumerate(zip(ctxs, ms)):
        k = torch.from_numpy(gather_flat(p["kc"], p["bt"][s], c, bs)).repeat_interleave(G, dim=0)
        v = torch.from_numpy(gather_flat(p["vc"], p["bt"][s], c, bs)).repeat_interleave(G, dim=0)
        q_full = torch.from_numpy(rng.standard_normal((h_q, c, d)))       # rows for the older tokens
        q0 = int(p["qs"][s])
        q_full[:, c - m:, :] = torch.from_numpy(p["q"][q0:q0 + m].astype(np.float64)).transpose(0, 1)
        ref = torch.nn.functional.scaled_dot_product_attention(q_full[None], k[None], v[None], is_causal=True)[0]
        ref = ref[:, c - m:, :].transpose(0, 1).numpy()
        if not np.allclose(out[q0:q0 + m], ref, rtol=1e-12, atol=1e-12):
            return False
    return True


def pin_decode_steps(fn, seed=11):
    """Token i of m equals a decode step over the first ctx - m + i + 1 positions."""
    rng = np.random.default_rng(seed)
    ctxs, ms = [17, 4, 33], [5, 4, 2]
    p = make_multi(rng, 4, 4, 8, 8, ctxs, ms)
    out = fn(p)
    for s, (c, m) in enumerate(zip(ctxs, ms)):
        for i in range(m):
            row = int(p["qs"][s]) + i
            lens = np.array(ctxs, dtype=np.int32)
            lens[s] = c - m + i + 1
            ref = att.paged_attention_decode(
                np.repeat(p["q"][row][None], len(ctxs), axis=0).view(np.uint32), p["kc"].view(np.uint32),
                p["vc"].view(np.uint32), p["bt"], lens, q_dtype="f32", kv_dtype="f32", block_size=p["bs"],
                seqs=[s])
            if not np.allclose(out[row], ref[s], rtol=1e-13, atol=1e-13):
                return False
    return True


def pin_one_new_token_is_decode(fn, seed=12):
    rng = np.random.default_rng(seed)
    ctxs = [1, 16, 7, 30]
    p = make_multi(rng, 6, 3, 8, 4, ctxs, [1] * 4)
    out = fn(p)
    ref = att.paged_attention_decode(p["q"].view(np.uint32), p["kc"].view(np.uint32), p["vc"].view(np.uint32),
                                     p["bt"], p["ctx"], q_dtype="f32", kv_dtype="f32", block_size=p["bs"])
    return bool(np.array_equal(out, ref))


def pin_tokens_before_the_cache_get_zero(fn, seed=13):
    """ctx = 3 cached positions, m = 5 new tokens: tokens 0 and 1 see nothing."""
    rng = np.random.default_rng(seed)
    p = make_multi(rng, 2, 1, 8, 4, [3], [5])
    out = fn(p)
    if not (np.all(out[:2] == 0.0) and np.all(np.isfinite(out[2:]))):
        return False
    one = att.paged_attention_decode(p["q"][2:3].view(np.uint32), p["kc"].view(np.uint32), p["vc"].view(np.uint32),
                                     p["bt"], np.array([1], dtype=np.int32), q_dtype="f32", kv_dtype="f32",
                                     block_size=p["bs"])
    return bool(np.allclose(out[2], one[0], rtol=1e-13, atol=1e-13))


def pin_never_reads_past_context(fn, seed=14):
    """Poisoned tail slots (NaN K, inf V) leave every row finite."""
    rng = np.random.default_rng(seed)
    p = make_multi(rng, 4, 2, 8, 8, [5, 19, 8], [5, 3, 8])
    out = fn(p)
    return bool(np.all(np.isfinite(out)))


PINS = [pin_sdpa_causal, pin_decode_steps, pin_one_new_token_is_decode, pin_tokens_before_the_cache_get_zero,
        pin_never_reads_past_context]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_oracle_passes_pin(pin):
    assert pin(run_multi)


def test_rejects_bad_query_rows():
    rng = np.random.default_rng(15)
    p = make_multi(rng, 2, 1, 8, 4, [6, 6], [2, 2])
    p["qs"] = np.array([0, 3, 2], dtype=np.int32)        # decreasing
    with pytest.raises(ValueError):
        run_multi(p)
    p["qs"] = np.array([0, 2, 9], dtype=np.int32)        # past the last row
    with pytest.raises(ValueError):
        run_multi(p)

# ---------------------------------------------------------------- planted mistakes


def _mutant(visible):
    def fn(p):
        saved = att.causal_visible
        att.causal_visible = visible
        try:
            return run_multi(p)
        finally:
            att.causal_visible = saved
    return fn


MUTANTS = {
    "excludes_own_position": _mutant(lambda ctx, m, i: max(0, ctx - m + i)),
    "sees_one_future_token": _mutant(lambda ctx, m, i: min(ctx, max(0, ctx - m + i + 2))),
    "mask_aligned_to_first_position": _mutant(lambda ctx, m, i: min(ctx, i + 1)),
    "no_causal_mask": _mutant(lambda ctx, m, i: ctx),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    fn = MUTANTS[name]
    caught = []
    for pin in PINS:
        try:
            ok = pin(fn)
        except Exception:
            ok = False
        caught.append(not ok)
    assert any(caught), f"no pin catches the planted mistake {name}"
