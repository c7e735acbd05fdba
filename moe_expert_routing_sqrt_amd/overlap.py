"""Exposed versus hidden communication of a wave-pipelined MoE layer.

The model of mastering-deepseek-v4 "MoE + Expert-Parallel Overlap (Exp08)"
(Implemented: the overlap simulator; Measured: the speedup saturates at 2x as
the bandwidth crosses the crossover and the exposed communication grows
linearly below it), with the volumes per token-expert pair it takes from the
paper: V_comp = 6*d*d_ff FLOPs (three d x d_ff expert matrices) and
V_comm = 3*d bytes (a row dispatched in one byte per element and returned in
two).  deepmox ch.5 ("The network becomes part of the forward pass") puts the
described training run at about one-to-one cross-node computation to
communication -- the point where overlap pays most.

For compute throughput C (FLOP/s) and bandwidth B (bytes/s) per GPU:
    t_comp = V_comp / C,   t_comm = V_comm / B
    serial     = t_comp + t_comm
    overlapped = max(t_comp, t_comm)              (steady-state wave pipeline)
    exposed    = max(0, t_comm - t_comp),  hidden = min(t_comm, t_comp)
    utilization = t_comp / overlapped,  speedup = serial / overlapped  (<= 2)
    crossover:  B* = C * V_comm / V_comp, i.e. C / B* = V_comp / V_comm = 2 * d_ff

Like the page's simulator it is steady state only: no per-wave variance, no
contention between the transfer and the compute for memory.

Expert-parallel bandwidth on an MI355X node: every GPU has a dedicated xGMI
link to each of its peers, so an even all-to-all over n GPUs moves 1/n of a
GPU's rows to each peer at once; the per-GPU rate for the whole exchange is
n * link bandwidth (the 1/n that stays local costs nothing).
"""
from __future__ import annotations

from typing import Dict, Iterable, List

XGMI_LINK_GBS = 153.0   # per direction, per link
XGMI_LINKS = 7          # links per MI355X (full mesh of 8)


def pair_volumes(d: int, d_ff: int, comm_bytes_per_elem: float = 3.0):
    """(V_comp FLOPs, V_comm bytes) of one token-expert pair."""
    return 6.0 * d * d_ff, comm_bytes_per_elem * d


def crossover_intensity(d: int, d_ff: int, comm_bytes_per_elem: float = 3.0) -> float:
    """FLOPs per byte at which communication exactly hides under compute."""
    vc, vm = pair_volumes(d, d_ff, comm_bytes_per_elem)
    return vc / vm


def crossover_bandwidth(C: float, d: int, d_ff: int, comm_bytes_per_elem: float = 3.0) -> float:
    """Bandwidth (bytes/s) at which t_comm = t_comp for compute throughput C."""
    return C / crossover_intensity(d, d_ff, comm_bytes_per_elem)


def model(C: float, B: float, d: int, d_ff: int, pairs: float = 1.0,
          comm_bytes_per_elem: float = 3.0) -> Dict[str, float]:
    """Times (s) for `pairs` token-expert pairs on one GPU."""
    if C <= 0 or B <= 0:
        raise ValueError("throughput and bandwidth must be positive")
    vc, vm = pair_volumes(d, d_ff, comm_bytes_per_elem)
    t_comp = pairs * vc / C
    t_comm = pairs * vm / B
    serial = t_comp + t_comm
    overlapped = max(t_comp, t_comm)
    return {"t_comp": t_comp, "t_comm": t_comm, "serial": serial, "overlapped": overlapped,
            "exposed": max(0.0, t_comm - t_comp), "hidden": min(t_comm, t_comp),
            "utilization": t_comp / overlapped, "speedup": serial / overlapped,
            "comm_to_comp": t_comm / t_comp}


def ep_bandwidth(n_gpus: int, link_gbs: float = XGMI_LINK_GBS) -> float:
    """Per-GPU all-to-all rate (bytes/s) of an even exchange over n GPUs of a
    full xGMI mesh (one dedicated link per peer)."""
    if not 1 <= n_gpus <= XGMI_LINKS + 1:
        raise ValueError("a full mesh holds at most 8 MI355X")
    if n_gpus == 1:
        return float("inf")
    return n_gpus * link_gbs * 1e9


def sweep(C: float, d: int, d_ff: int, bandwidths: Iterable[float], pairs: float = 1.0,
          comm_bytes_per_elem: float = 3.0) -> List[Dict[str, float]]:
    out = []
    for B in bandwidths:
        r = model(C, B, d, d_ff, pairs, comm_bytes_per_elem)
        r["B"] = B
        out.append(r)
    return out
