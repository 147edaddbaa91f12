"""Helpers shared by the GPU tests: build a workload's cache on the device
with the library, and compute the oracle's answer for chosen parts of it.

The oracle only ever sees the seeded inputs (never bytes produced on the
GPU): expected cache bytes and expected outputs are re-derived on the CPU.
"""
from __future__ import annotations

import numpy as np
import torch

import decode_attention_bit_amd as uq
from decode_attention_bit_amd import inputs
from oracle import uq_oracle as O

MAX_ABS = 1e-2        # attention output tolerance: max |gpu - oracle|
REL_L2 = 5e-3         # and ||gpu - oracle||_2 / ||oracle||_2


class Instance:
    """One workload realised on the GPU: cache stored by uq_store."""

    def __init__(self, w: inputs.Workload, dev="cuda", seq_lens=None):
        self.w = w
        self.dev = torch.device(dev)
        self.layout = inputs.make_layout(w, seq_lens=seq_lens)
        self.query = inputs.make_query(w)
        lay = self.layout
        self.cache = torch.zeros((lay.num_blocks, w.block_size, w.Hk, self.w.slot_bytes),
                                 dtype=torch.uint8, device=self.dev)
        self.block_table = torch.from_numpy(lay.block_table).to(self.dev)
        self.seq_lens = torch.from_numpy(lay.seq_lens).to(self.dev)
        self.q_dev = self.query.to(self.dev)
        last = []
        for b in range(w.B):
            L = int(lay.seq_lens[b])
            if b % 8 == 0:
                print(f"  storing {w.name} sequence {b}/{w.B}", flush=True)
            k, v = inputs.make_kv(w, lay, b)
            n_pre = L - 1 if w.name == "mixed" else L   # mixed: last token stored in the step
            if n_pre > 0:
                slots = inputs.slots_for(lay, b, 0, n_pre)
                uq.store(k[:n_pre].to(self.dev), v[:n_pre].to(self.dev), self.cache,
                         torch.from_numpy(slots).to(self.dev))
            if w.name == "mixed":
                last.append((k[L - 1:L], v[L - 1:L], inputs.slots_for(lay, b, L - 1, L)))
        if last:
            self.step_k = torch.cat([x[0] for x in last]).to(self.dev)
            self.step_v = torch.cat([x[1] for x in last]).to(self.dev)
            self.step_slots = torch.from_numpy(np.concatenate([x[2] for x in last])).to(self.dev)
        torch.cuda.synchronize()

    def store_step(self):
        uq.store(self.step_k, self.step_v, self.cache, self.step_slots)

    def decode(self, splits=None, **kw):
        return uq.decode(self.q_dev, self.cache, self.block_table, self.seq_lens, self.w.scale,
                         splits or self.w.num_kv_splits, **kw)

    # ----------------------------------------------------------- oracle side
    def oracle_pairs(self, pairs_by_seq: dict, chunk: int = 2048) -> dict:
        """Oracle output rows {(b, h): (QG, D)} for the given {b: [KV heads]},
        every sequence encoded by the oracle itself. The (sequence, chunk)
        encodes run on a thread pool (numpy releases the GIL in them)."""
        import os
        from concurrent.futures import ThreadPoolExecutor
        w = self.w
        seqs = {}
        for b, heads in pairs_by_seq.items():
            k, v = inputs.make_kv(w, self.layout, b)
            seqs[b] = (inputs.bf16_bits(k)[:, heads], inputs.bf16_bits(v)[:, heads])
        jobs = [(b, i) for b in seqs for i in range(0, int(self.layout.seq_lens[b]), chunk)]

        def enc(job):
            b, i = job
            kb, vb = seqs[b]
            return O.decode_slots(O.encode_slots(kb[i:i + chunk], vb[i:i + chunk]))

        with ThreadPoolExecutor(max(1, min(16, len(os.sched_getaffinity(0))))) as ex:
            done = dict(zip(jobs, ex.map(enc, jobs)))
        qg = w.QG
        qb = inputs.bf16_bits(self.query)
        out = {}
        for b, heads in pairs_by_seq.items():
            parts = [done[(b2, i)] for (b2, i) in jobs if b2 == b]
            K = np.concatenate([p[0] for p in parts])
            V = np.concatenate([p[1] for p in parts])
            for j, h in enumerate(heads):
                q8 = O.query_haircut(qb[b, h * qg:(h + 1) * qg])
                out[(b, h)] = O.attention(q8, K[:, j], V[:, j], w.scale)
        return out

    def gpu_cache_digest(self) -> str:
        """SHA-256 of the whole device cache (copied to the host in pieces)."""
        import hashlib
        h = hashlib.sha256()
        flat = self.cache.view(-1)
        step = 256 << 20
        for i in range(0, flat.numel(), step):
            h.update(flat[i:i + step].cpu().numpy().tobytes())
        return h.hexdigest()


def bf16_half_ulp(x: np.ndarray) -> np.ndarray:
    """Half a bf16 unit in the last place at |x|: the rounding error any bf16
    output of the exact value may carry."""
    a = np.maximum(np.abs(x), 2.0 ** -126)
    return np.ldexp(1.0, np.floor(np.log2(a)).astype(int) - 8)


def check_close(got: np.ndarray, ref: np.ndarray, what: str, allow_output_rounding=False):
    """max-abs <= 1e-2 and rel-L2 <= 5e-3 against the float64 oracle.

    allow_output_rounding adds half a bf16 ulp of the reference to the
    max-abs bound only where |ref| >= 4: there half a bf16 ulp is 2**-6 or
    more, so rounding the exact answer to bf16 alone can exceed 1e-2. Below 4
    the bound is 1e-2 as stated."""
    got = np.asarray(got, dtype=np.float64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    diff = np.abs(got - ref)
    bound = MAX_ABS
    if allow_output_rounding:
        bound = MAX_ABS + np.where(np.abs(ref) >= 4.0, bf16_half_ulp(ref), 0.0)
    err = float(diff.max()) if diff.size else 0.0
    rel = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))
    worst = float(np.abs(ref).flat[int(np.argmax(diff))]) if diff.size else 0.0
    excess = diff - bound
    over = ""
    if diff.size and excess.max() > 0:
        i = int(np.argmax(excess))
        over = f"; over the bound by {excess.flat[i]:.3e} at |ref| = {np.abs(ref).flat[i]:.3f} " \
               f"(error {diff.flat[i]:.3e}), {int((excess > 0).sum())} elements over"
    assert np.all(diff <= bound) and rel <= REL_L2, \
        f"{what}: max-abs {err:.3e} (at |ref| = {worst:.3f}) rel-L2 {rel:.3e}{over}"
    return err, rel


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)
