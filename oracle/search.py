"""Predictive search for the wave-group partition (oracle).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Method: deep-dive 四、实时调优 › 在线阶段: 预测搜索算法 and its Algorithm 1
(Grouping Tuning Algorithm).  For a candidate partition G = (G_1 .. G_P) of
the T waves, each group's computation takes the GEMM's duration / T per wave;
its communication takes a latency read off a sampled latency-versus-size
curve.  Walking the groups in order, the communication of group i-1 starts
when both the computation of groups up to i-1 and the previous
communication are done; the prediction is the time the last group's
communication ends.  The search evaluates every candidate and keeps the
smallest prediction.

Readings:
* the first group has nothing to communicate before it (the pages evaluate
  the previous group's size inside the loop, which has no predecessor at the
  first group): its communication term is zero;
* the last group's communication also waits for the end of the computation
  and of the previous communication (the max stated for every other group;
  the final line of the printed listing omits it);
* the curve is a list of samples (bytes_k, seconds_k), bytes strictly
  increasing: latency is interpolated linearly in bytes between samples,
  equals the first sample's latency below it (a fixed per-call cost) and
  grows at the last sample's bandwidth (seconds per byte) beyond the last;
  a group of zero bytes costs nothing;
* a group's data size is its contiguous span in bytes (the sum of its
  tiles' elements times the element size);
* candidates are walked in the order of ``enumerate_compositions`` (cut
  masks 0 .. 2^(T-1)-1); among equal predictions the first one wins.
"""

from __future__ import annotations

from typing import List, Sequence, Tuple

from .tiles import enumerate_compositions


def interp_latency(curve_bytes: Sequence[float], curve_seconds: Sequence[float], size: float) -> float:
    """Latency of one collective call on ``size`` bytes, from the sampled curve."""
    if len(curve_bytes) != len(curve_seconds) or len(curve_bytes) == 0:
        raise ValueError("curve needs matching, non-empty samples")
    for a, b in zip(curve_bytes, curve_bytes[1:]):
        if not b > a:
            raise ValueError("curve sizes must increase strictly")
    if size <= 0:
        return 0.0
    if size <= curve_bytes[0]:
        return float(curve_seconds[0])
    n = len(curve_bytes)
    if size >= curve_bytes[-1]:
        return float(curve_seconds[-1]) * (size / float(curve_bytes[-1]))
    for k in range(n - 1):
        x0, x1 = float(curve_bytes[k]), float(curve_bytes[k + 1])
        if x0 <= size <= x1:
            y0, y1 = float(curve_seconds[k]), float(curve_seconds[k + 1])
            return y0 + (y1 - y0) * (size - x0) / (x1 - x0)
    raise AssertionError("unreachable")


def group_bytes(composition: Sequence[int], wave_bytes: Sequence[float]) -> List[float]:
    """Bytes of each group's span: the sum over the waves it holds."""
    if sum(composition) != len(wave_bytes):
        raise ValueError("the composition must cover every wave")
    out, w = [], 0
    for c in composition:
        out.append(float(sum(wave_bytes[w:w + c])))
        w += c
    return out


def predict(composition: Sequence[int], wave_bytes: Sequence[float], duration: float,
            curve_bytes: Sequence[float], curve_seconds: Sequence[float]) -> float:
    """Predicted end of the last group's communication for one candidate."""
    T = len(wave_bytes)
    sizes = group_bytes(composition, wave_bytes)
    t_acc_p = 0.0     # computation finished so far
    t_acc_m = 0.0     # communication finished so far
    for i, c in enumerate(composition):
        t_m = interp_latency(curve_bytes, curve_seconds, sizes[i - 1]) if i > 0 else 0.0
        t_p = duration / T * c
        t_acc_m = max(t_acc_p, t_acc_m) + t_m
        t_acc_p = t_acc_p + t_p
    t_acc_m = max(t_acc_p, t_acc_m) + interp_latency(curve_bytes, curve_seconds, sizes[-1])
    return t_acc_m


def search(wave_bytes: Sequence[float], duration: float, curve_bytes: Sequence[float],
           curve_seconds: Sequence[float]) -> Tuple[tuple, float, List[float]]:
    """Best composition, its prediction, and every candidate's prediction in mask order."""
    T = len(wave_bytes)
    best, best_t, all_t = None, None, []
    for comp in enumerate_compositions(T):
        t = predict(comp, wave_bytes, duration, curve_bytes, curve_seconds)
        all_t.append(t)
        if best_t is None or t < best_t:
            best, best_t = comp, t
    return best, best_t, all_t


def wave_bytes_of(plan, elem_bytes: int = 2) -> List[float]:
    """Bytes of output each wave produces: its tiles' rows x cols x the element size."""
    out = [0.0] * plan.T
    for b, t in enumerate(plan.tile_of_b):
        out[b // plan.W] += plan.tile_rows[t] * plan.tile_cols[t] * elem_bytes
    return out
