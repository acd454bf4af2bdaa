"""The five synthetic workloads and one pass of the hot path over each.

A workload owns a predictor (P from its seed, A_g filled through the library's
own project_kv_block from seeded keys) and the per-step inputs and outputs.
``step(l0)`` is one pass of the whole hot path on the current stream:

  project_kv_block  the step's new blocks (decode: the last block of every
                    scored sequence and layer; prefill: the 128 new blocks)
  project_q         every scored layer, sequence and query row
  score_blocks      every scored layer and sequence
  rank_victims      one ranking per (layer, sequence) score row

The new blocks carry the same keys as at set-up, so a step rewrites identical
low-rank keys and every step's outputs are the same: the outputs after a timed
run can be checked against the oracle.

Shapes are those of the decode, batched-decode, prefill and long-context cases
the predictor serves (Llama-3-8B-like and 70B-like head counts and dims); all
data is seeded and synthetic, with no model weights.
"""

import hashlib
from dataclasses import dataclass

import torch

from . import (PRED_FLAG_ZERO_AG, dims, pred_create, pred_destroy, pred_project_kv_block,  # noqa: F401
               pred_project_q, pred_project_step, pred_rank_victims, pred_rank_workspace_bytes,
               pred_score_blocks, pred_score_rows, pred_select_keep)
from . import synth


@dataclass(frozen=True)
class Config:
    name: str
    index: int          # 1..5; seeds are 1000 + index (P) and 2000 + index (data)
    L: int
    Hq: int
    Hk: int
    D: int
    R: int
    B: int
    N: int              # max_blocks (A_g slots per layer)
    n: int              # blocks per sequence that are scored
    S: int              # sequences
    M: int              # query rows per sequence
    step_layers: int    # layers scored per step (the rest rotate in)
    keys: str           # "normal" | "student_t3"
    table: str          # "identity" | "permutation" | "slices"
    planted: int        # planted blocks per layer (keys = 4 x a query)
    new_blocks: int     # blocks re-projected per sequence and layer each step
    description: str

    @property
    def g(self):
        return self.Hq // self.Hk

    @property
    def seed_p(self):
        return 1000 + self.index

    @property
    def seed_data(self):
        return 2000 + self.index

    @property
    def slot_bytes(self):
        return self.Hk * self.B * self.R * 2

    @property
    def blocks_per_step(self):
        return self.step_layers * self.S * self.n

    @property
    def first_pos(self):
        """Position of the first query row: the rows are the context's last M tokens."""
        return self.n * self.B - self.M

    def complete_blocks(self, row):
        """Blocks every token of which is at or before query row ``row``'s position."""
        return min(self.n, (self.first_pos + row + 1) // self.B)


CONFIGS = {
    "tiny": Config("tiny", 1, L=1, Hq=4, Hk=1, D=64, R=16, B=16, N=64, n=64, S=1, M=1, step_layers=1,
                   keys="normal", table="identity", planted=0, new_blocks=1,
                   description="1 layer, nq=4, nkv=1, head_dim=64, r=16, block_size=16, 64 blocks, 1 row"),
    "llama3_8b_decode": Config("llama3_8b_decode", 2, L=32, Hq=32, Hk=8, D=128, R=32, B=16, N=8192, n=8192, S=1,
                               M=1, step_layers=32, keys="normal", table="permutation", planted=82, new_blocks=1,
                               description="32 layers, nq=32, nkv=8, head_dim=128, r=32, block_size=16, 8192 "
                                           "blocks (131k tokens), 1 row, 1% planted blocks, permuted table"),
    "batched_decode": Config("batched_decode", 3, L=1, Hq=32, Hk=8, D=128, R=32, B=16, N=131072, n=2048, S=64, M=1,
                             step_layers=1, keys="normal", table="slices", planted=0, new_blocks=1,
                             description="64 sequences x 2048 blocks (32k tokens) from a 131072-block pool, nq=32, "
                                         "nkv=8, head_dim=128, r=32, block_size=16"),
    "prefill_chunk": Config("prefill_chunk", 4, L=1, Hq=32, Hk=8, D=128, R=64, B=16, N=2048, n=2048, S=1, M=2048,
                            step_layers=1, keys="normal", table="identity", planted=0, new_blocks=128,
                            description="2048 new tokens (128 blocks) on a 30k-token context, nq=32, nkv=8, "
                                        "head_dim=128, r=64, block_size=16, 2048 query rows"),
    "long_context_70b": Config("long_context_70b", 5, L=64, Hq=64, Hk=8, D=128, R=64, B=32, N=32768, n=32768, S=1,
                               M=1, step_layers=1, keys="student_t3", table="identity", planted=0, new_blocks=1,
                               description="64 layers (one scored per step, rotating), nq=64, nkv=8, head_dim=128, "
                                           "r=64, block_size=32, 32768 blocks (1M tokens), Student-t keys"),
}


def _seed(*parts):
    return int(hashlib.sha256(repr(parts).encode()).hexdigest()[:15], 16)


class Workload:
    """Set up a config on the GPU.  ``keep`` = set of (layer, seq, logical block) whose keys
    are copied to the host for oracle checks; ``layers`` limits which layers are filled."""

    def __init__(self, cfg, device="cuda", keep=(), layers=None, chunk_blocks=2048):
        self.cfg = c = cfg
        self.device = device
        self.d = dims(c.L, c.Hq, c.Hk, c.D, c.R, c.B, c.N)
        self.h = pred_create(self.d, c.seed_p, 0)
        self.layers = list(range(c.L)) if layers is None else list(layers)
        keep = set(keep)

        # block tables, logical -> physical, shared by all layers
        if c.table == "identity":
            phys = torch.arange(c.n, dtype=torch.int32).view(1, c.n)
            self.tables = None
        elif c.table == "permutation":
            phys = synth.permutation(c.N, _seed(c.seed_data, "table"))[: c.n].view(1, c.n)
            self.tables = phys.to(device)
        elif c.table == "slices":
            perm = synth.permutation(c.N, _seed(c.seed_data, "table"))
            phys = perm[: c.S * c.n].view(c.S, c.n).contiguous()
            self.tables = phys.to(device)
        else:
            raise ValueError(c.table)
        self.phys = phys if phys.shape[0] == c.S else phys.expand(c.S, c.n)

        # queries for every layer (the step scores step_layers of them)
        self.q = synth.normal_bf16((c.L, c.S, c.M, c.Hq, c.D), _seed(c.seed_data, "q"), device)
        self.planted = (synth.sample_sorted(c.n, c.planted, _seed(c.seed_data, "planted")).tolist()
                        if c.planted else [])
        planted_set = set(self.planted)

        # fill A_g through project_kv_block, keeping the step's re-projected blocks
        nb = c.new_blocks
        self.new_logical = list(range(c.n - nb, c.n))
        self.k_new = torch.empty((c.L, c.S * nb, c.B, c.Hk, c.D), dtype=torch.bfloat16, device=device)
        self.kept = {}
        for l in self.layers:
            for s in range(c.S):
                for c0 in range(0, c.n, chunk_blocks):
                    c1 = min(c.n, c0 + chunk_blocks)
                    shape = (c1 - c0, c.B, c.Hk, c.D)
                    sd = _seed(c.seed_data, "k", l, s, c0)
                    k = (synth.student_t3_bf16(shape, sd, device) if c.keys == "student_t3"
                         else synth.normal_bf16(shape, sd, device))
                    for b in (pb for pb in self.planted if c0 <= pb < c1):
                        for kv in range(c.Hk):
                            k[b - c0, :, kv, :] = self.q[l, s, 0, kv * c.g, :] * 4
                    table = self.phys[s, c0:c1].contiguous().view(1, -1).to(device)
                    pred_project_kv_block(self.h, l, k.view(1, *shape), table)
                    for b in range(max(c0, c.n - nb), c1):
                        self.k_new[l, s * nb + (b - (c.n - nb))] = k[b - c0]
                    for (kl, ks, kb) in keep:
                        if kl == l and ks == s and c0 <= kb < c1:
                            self.kept[(kl, ks, kb)] = k[kb - c0].cpu()
                    del k
        del planted_set
        self.table_new = torch.stack(
            [self.phys[:, c.n - nb:].reshape(-1) for _ in range(c.L)]).contiguous().to(device)

        # step outputs
        nl = c.step_layers
        self.q_proj = torch.empty((nl, c.S, c.M, c.Hq, c.R), dtype=torch.bfloat16, device=device)
        self.scores = torch.empty((nl, c.S, c.n), dtype=torch.float32, device=device)
        self.victims = torch.empty((nl * c.S, c.n), dtype=torch.int32, device=device)
        ws = pred_rank_workspace_bytes(c.n, nl * c.S)
        self.workspace = torch.empty((max(ws, 8) // 8,), dtype=torch.int64, device=device) if ws else None
        torch.cuda.synchronize()

    def keep_setup(self, topk=64):
        """Buffers for the per-row keep sets of the first scored layer and sequence."""
        c = self.cfg
        self.topk = min(topk, c.n)
        self.row_scores = torch.empty((c.M, c.n), dtype=torch.float32, device=self.device)
        self.keep = torch.empty((c.M, self.topk), dtype=torch.int32, device=self.device)
        ws = pred_rank_workspace_bytes(c.n, c.M)
        self.keep_ws = torch.empty((max(ws, 8) // 8,), dtype=torch.int64, device=self.device) if ws else None

    def keep_step(self, l0=0, stream=None):
        """Per-row causal scores of the step's first layer and sequence 0 (from q_proj of the
        last step) and each row's keep set of topk blocks."""
        c = self.cfg
        tab = None if self.tables is None else self.tables[0]
        pred_score_rows(self.h, l0, self.q_proj[0, 0], c.first_pos, tab, c.n, self.row_scores, stream=stream)
        pred_select_keep(self.h, self.row_scores, c.first_pos, c.B, self.topk, self.keep, self.keep_ws,
                         stream=stream)

    def layer0_for_step(self, i):
        c = self.cfg
        return (i * c.step_layers) % c.L

    def step(self, l0=0, stream=None):
        c = self.cfg
        nl = c.step_layers
        pred_project_step(self.h, l0, self.k_new[l0:l0 + nl], self.table_new[l0:l0 + nl], self.q[l0:l0 + nl],
                          self.q_proj, stream=stream)
        pred_score_blocks(self.h, l0, self.q_proj, self.tables, self.scores, stream=stream)
        pred_rank_victims(self.h, self.scores.view(nl * c.S, c.n), self.victims, self.workspace, stream=stream)

    def close(self):
        if self.h is not None:
            torch.cuda.synchronize()
            pred_destroy(self.h)
            self.h = None
