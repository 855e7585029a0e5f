"""Helpers for the GPU parity tests: one decode step of a workload, run through
the HIP path and through the oracle on the same seeded inputs.

Inputs come only from `workloads` (seeded) and the block managers; expected
values come only from `oracle`.  Nothing the HIP path produces is fed to the
oracle."""

import math

import numpy as np
import torch

import oracle.allocator
import oracle.attention
import oracle.scatter
import paged_kv_cache_431_amd as pkv
import workloads

TOL = {  # max |err| and rel-L2 against the float64 oracle
    "fp8": (6e-2, 1e-3),
    "bf16": (2e-2, 1e-3),
    "f16": (2e-2, 1e-3),
    "f32": (2e-2, 1e-3),
}

# expected decode rows of a workload (oracle output), computed once per session
_ORACLE_DECODE = {}

_BITS = {torch.float32: (torch.int32, np.uint32), torch.float16: (torch.int16, np.uint16),
         torch.bfloat16: (torch.int16, np.uint16), torch.uint8: (torch.uint8, np.uint8)}


def to_bits(t):
    """Raw element bits of a tensor as a NumPy array (on the host)."""
    tdt, ndt = _BITS[t.dtype]
    return t.detach().view(tdt).cpu().numpy().view(ndt)


class Case:
    def __init__(self, wl, poison=True, device="cuda"):
        self.wl = wl
        self.plan = workloads.plan(wl)
        p = self.plan
        bm = pkv.BlockManager(p.num_blocks, wl.block_size, p.free_order)
        self.rp = workloads.replay(p, bm)
        ora = oracle.allocator.BlockManager(p.num_blocks, wl.block_size, p.free_order)
        rp_o = workloads.replay(p, ora)
        assert np.array_equal(self.rp.block_tables, rp_o.block_tables)
        assert np.array_equal(self.rp.slot_mapping, rp_o.slot_mapping)
        self.t = workloads.make_tensors(p, self.rp, device=device, poison=poison)
        self.device = device
        self.block_tables = torch.from_numpy(self.rp.block_tables).to(device)
        self.context_lens = torch.from_numpy(p.context_lens).to(device)
        self.slots = torch.from_numpy(self.rp.slot_mapping).to(device)
        self._oracle_pool = None

    # ---------------------------------------------------------------- HIP path
    def scatter(self, k_cache=None, v_cache=None):
        kc = self.t.k_cache if k_cache is None else k_cache
        vc = self.t.v_cache if v_cache is None else v_cache
        pkv.pkv_reshape_and_cache(self.t.new_k, self.t.new_v, kc, vc, self.slots,
                                  k_scale=self.t.k_scale, v_scale=self.t.v_scale)
        return kc, vc

    def decode(self, out_dtype=torch.float32, num_splits=0, block_tables=None, k_cache=None, v_cache=None,
               workspace=None):
        wl = self.wl
        out = torch.empty((wl.num_seqs, wl.h_q, wl.head_dim), dtype=out_dtype, device=self.device)
        pkv.pkv_paged_attention_decode(
            out, self.t.q, self.t.k_cache if k_cache is None else k_cache,
            self.t.v_cache if v_cache is None else v_cache,
            self.block_tables if block_tables is None else block_tables, self.context_lens,
            max_context_len=self.plan.max_context_len, k_scale=self.t.k_scale, v_scale=self.t.v_scale,
            num_splits=num_splits, workspace=workspace)
        return out

    def multi(self, q, query_start, max_query_len, out_dtype=torch.float32, num_splits=0, out=None, workspace=None):
        """Several new query tokens per sequence (q [T, Hq, D]) over the pools."""
        wl = self.wl
        if out is None:
            out = torch.empty((q.shape[0], wl.h_q, wl.head_dim), dtype=out_dtype, device=self.device)
        qs = torch.from_numpy(np.asarray(query_start, dtype=np.int32)).to(self.device)
        pkv.pkv_paged_attention_multi(
            out, q, self.t.k_cache, self.t.v_cache, self.block_tables, self.context_lens, qs,
            max_query_len=max_query_len, max_context_len=self.plan.max_context_len, k_scale=self.t.k_scale,
            v_scale=self.t.v_scale, num_splits=num_splits, workspace=workspace)
        return out

    # ---------------------------------------------------------------- oracle
    def oracle_pools(self):
        """Pools after the oracle's scatter of the new tokens (host arrays)."""
        if self._oracle_pool is None:
            wl = self.wl
            self._oracle_pool = oracle.scatter.reshape_and_cache(
                to_bits(self.t.new_k), to_bits(self.t.new_v), to_bits(self.t.k_cache), to_bits(self.t.v_cache),
                self.rp.slot_mapping, in_dtype=wl.new_dtype, kv_dtype=wl.kv_dtype, block_size=wl.block_size,
                k_scale=self.t.k_scale, v_scale=self.t.v_scale)
        return self._oracle_pool

    def oracle_decode(self, seqs=None):
        wl = self.wl
        kc, vc = self.oracle_pools()
        return oracle.attention.paged_attention_decode(
            to_bits(self.t.q), kc, vc, self.rp.block_tables, self.plan.context_lens, q_dtype=wl.q_dtype,
            kv_dtype=wl.kv_dtype, block_size=wl.block_size, scale=1.0 / math.sqrt(wl.head_dim),
            k_scale=self.t.k_scale, v_scale=self.t.v_scale, seqs=seqs)

    def oracle_decode_all(self):
        """The oracle's output for every row of the decode step, kept per
        workload for the session: a Case is a pure function of its seeded
        workload, so every Case of one workload has the same expected rows."""
        key = self.wl
        if key not in _ORACLE_DECODE:
            _ORACLE_DECODE[key] = self.oracle_decode()
        return _ORACLE_DECODE[key]

    def oracle_multi(self, q, query_start, seqs=None):
        wl = self.wl
        kc, vc = self.oracle_pools()
        return oracle.attention.paged_attention_multi(
            to_bits(q), kc, vc, self.rp.block_tables, self.plan.context_lens, np.asarray(query_start),
            q_dtype=wl.q_dtype, kv_dtype=wl.kv_dtype, block_size=wl.block_size,
            scale=1.0 / math.sqrt(wl.head_dim), k_scale=self.t.k_scale, v_scale=self.t.v_scale, seqs=seqs)


def errors(got, ref, seqs=None):
    """(max abs error, rel-L2 error) of got vs ref over the rows of `seqs`."""
    g = got.detach().float().cpu().numpy().astype(np.float64)
    if seqs is not None:
        g, ref = g[seqs], ref[seqs]
    diff = g - ref
    max_abs = float(np.max(np.abs(diff))) if diff.size else 0.0
    denom = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(diff)) / denom if denom > 0 else float(np.linalg.norm(diff))
    return max_abs, rel


def assert_close(got, ref, kv_dtype, seqs=None, label=""):
    max_abs, rel = errors(got, ref, seqs)
    tol_abs, tol_rel = TOL[kv_dtype]
    print(f"[parity] {label} max_abs={max_abs:.3e} rel_l2={rel:.3e}", flush=True)
    assert np.all(np.isfinite(got.detach().float().cpu().numpy()[seqs] if seqs is not None else
                              got.detach().float().cpu().numpy())), f"{label}: non-finite output"
    assert max_abs <= tol_abs, f"{label}: max abs error {max_abs} > {tol_abs}"
    assert rel <= tol_rel, f"{label}: rel-L2 error {rel} > {tol_rel}"
    return max_abs, rel
