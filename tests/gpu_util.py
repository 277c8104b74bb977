"""Helpers for the GPU tests: device upload/download of bf16 bit arrays and the comparison metrics."""
from __future__ import annotations

import sys

import numpy as np
import torch

DEV = "cuda:0"


def say(msg: str) -> None:
    """Name the case before each GPU step, flushed, so a failing run shows where it was."""
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def up(bits: np.ndarray) -> torch.Tensor:
    """uint16 bf16 bit array -> contiguous int16 device tensor with the same bits."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV)


def down(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().numpy().view(np.uint16)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def pcc(a: np.ndarray, b: np.ndarray) -> float:
    a = a.ravel() - a.mean()
    b = b.ravel() - b.mean()
    return float(a @ b / np.sqrt((a @ a) * (b @ b)))


def metrics(got: np.ndarray, ref: np.ndarray) -> dict:
    err = got - ref
    return {"max_abs": float(np.max(np.abs(err))), "pcc": pcc(got, ref),
            "rel_l2": float(np.linalg.norm(err) / np.linalg.norm(ref))}


class Layer:
    """Device buffers of one layer's inputs (from synth.layer_inputs) plus the output and workspace."""

    def __init__(self, inp: dict, ax):
        self.inp = inp
        self.S, self.Smax = inp["S"], inp["Smax"]
        self.q, self.k, self.v = up(inp["q"]), up(inp["k"]), up(inp["v"])
        self.gq, self.gk = up(inp["gq"]), up(inp["gk"])
        self.Kc, self.Vc = up(inp["Kc"]), up(inp["Vc"])
        cos, sin = ax.rope_tables(self.S + inp["rope_delta"])
        self.cos = torch.from_numpy(cos).to(DEV)
        self.sin = torch.from_numpy(sin).to(DEV)
        self.out = torch.zeros((16, 64, 128), dtype=torch.int16, device=DEV)
        nbytes = ax.expert_attn_workspace_bytes(self.S, self.Smax)
        assert nbytes > 0
        self.ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
        assert self.ws.data_ptr() % 256 == 0
        # shapes the kernels assume
        assert self.Kc.shape == (8, self.Smax, 128) and self.Vc.shape == (8, self.Smax, 128)
        assert self.q.shape == (16, 64, 128) and self.k.shape == (8, 64, 128) and self.v.shape == (8, 64, 128)
        assert self.cos.shape == (64, 64) and self.gq.shape == (128,)

    def run(self, ax, eps: float = 1e-6):
        ax.expert_layer_attn(self.q, self.k, self.v, self.gq, self.gk, self.cos, self.sin, eps, self.Kc, self.Vc,
                             self.S, self.Smax, self.out, self.ws)
        torch.cuda.synchronize()
        return down(self.out)
