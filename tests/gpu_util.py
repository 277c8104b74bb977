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


GUARD_BYTES = 4096   # keeps 256-byte alignment of what lies between the guards
GUARD_BYTE = 0xA5


class Guarded:
    """A device buffer of nbytes between two GUARD_BYTES bands of a fixed byte: every write of a
    kernel must land inside (check() asserts both bands unchanged)."""

    def __init__(self, nbytes: int, fill: int = 0):
        self.nbytes = nbytes
        self.buf = torch.full((nbytes + 2 * GUARD_BYTES,), GUARD_BYTE, dtype=torch.uint8, device=DEV)
        self.t = self.buf[GUARD_BYTES:GUARD_BYTES + nbytes]
        self.t.fill_(fill)
        assert self.t.data_ptr() % 256 == 0

    def check(self, what: str = "buffer") -> None:
        torch.cuda.synchronize()
        head = self.buf[:GUARD_BYTES]
        tail = self.buf[GUARD_BYTES + self.nbytes:]
        assert bool((head == GUARD_BYTE).all()), f"{what}: bytes before the buffer were written"
        assert bool((tail == GUARD_BYTE).all()), f"{what}: bytes after the buffer were written"


def assert_status_clear(ax, ws) -> None:
    """The workspace status word: no bounded wait of any launch on ws gave up."""
    st = ax.workspace_status(ws)
    assert st == 0, f"workspace status word {st:#x} (AX_STATUS_WAIT_EXPIRED = 1)"


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
        # the output and the workspace sit between guard bands; the workspace starts zeroed (its
        # status word is then read back after every call)
        self.out_g = Guarded(16 * 64 * 128 * 2)
        self.out = self.out_g.t.view(torch.int16).view(16, 64, 128)
        nbytes = ax.expert_attn_workspace_bytes(self.S, self.Smax)
        assert nbytes > 0
        self.ws_g = Guarded(nbytes)
        self.ws = self.ws_g.t
        # shapes the kernels assume
        assert self.Kc.shape == (8, self.Smax, 128) and self.Vc.shape == (8, self.Smax, 128)
        assert self.q.shape == (16, 64, 128) and self.k.shape == (8, 64, 128) and self.v.shape == (8, 64, 128)
        assert self.cos.shape == (64, 64) and self.gq.shape == (128,)

    def run(self, ax, eps: float = 1e-6):
        ax.expert_layer_attn(self.q, self.k, self.v, self.gq, self.gk, self.cos, self.sin, eps, self.Kc, self.Vc,
                             self.S, self.Smax, self.out, self.ws)
        torch.cuda.synchronize()
        self.out_g.check("out")
        self.ws_g.check("workspace")
        if self.ws is self.ws_g.t:
            assert_status_clear(ax, self.ws)
        return down(self.out)
