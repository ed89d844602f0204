"""Predictive search for the wave-group partition (oracle).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Method: deep-dive 四、实时调优 › 在线阶段: 预测搜索算法 and its Algorithm 1
(Grouping Tuning Algorithm).  For a candidate partition G = (G_1 .. G_P) of
the T waves, each group's computation takes the GEMM's duration / T per wave;
its communication takes a latency read off a sampled latency-versus-size
curve.  A group's communication starts when both its own computation and
the previous group's communication are done; the prediction is the time the
last group's communication ends.  The search evaluates every candidate and
keeps the smallest prediction.  (The page's listing evaluates group i-1's
communication inside the step for group i and adds the last group's after
the loop; the recurrence below is that computation written per group.)

Readings:
* nothing is communicated before the first group's computation ends (the
  listing reads the previous group's size in the step of the first group,
  which has no predecessor);
* the last group's communication also waits for the end of the computation
  and of the previous communication (the max the page states for every
  group; the listing's closing step leaves it out);
* the curve is a list of samples (bytes_k, seconds_k), bytes strictly
  increasing: latency is interpolated linearly in bytes between samples,
  equals the first sample's latency below it (a fixed per-call cost) and
  grows at the last sample's bandwidth (seconds per byte) beyond the last;
  a group of zero bytes costs nothing;
* a group's data size is its contiguous span in bytes (the sum of its
  tiles' elements times the element size);
* candidates are walked in the order of ``enumerate_compositions`` (cut
  masks 0 .. 2^(T-1)-1); among equal predictions the one with more groups
  wins (the page's listing keeps a strict minimum over a candidate order it
  leaves open; more groups start communicating sooner and spread it over
  more of the computation, which the model does not price), and among
  those the first one.
"""

from __future__ import annotations

from typing import List, Sequence, Tuple

from .tiles import enumerate_compositions


def curve_latency(curve_bytes: Sequence[float], curve_seconds: Sequence[float], size: float) -> float:
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
    """Predicted end of the last group's communication for one candidate.

    Group i's computation is done once the waves of groups 0..i are, at
    ``compute_end = duration * (waves so far) / T``.  Its communication starts
    when both that and the previous group's communication are done, and
    lasts the latency of its span:

        comm_end(i) = max(compute_end(i), comm_end(i - 1)) + latency(bytes of group i)

    with comm_end(-1) = 0; the prediction is comm_end of the last group.
    """
    sizes = group_bytes(composition, wave_bytes)
    per_wave = duration / len(wave_bytes)
    waves_done, comm_end = 0, 0.0
    for waves, size in zip(composition, sizes):
        waves_done += waves
        compute_end = per_wave * waves_done
        comm_end = max(compute_end, comm_end) + curve_latency(curve_bytes, curve_seconds, size)
    return comm_end


def search(wave_bytes: Sequence[float], duration: float, curve_bytes: Sequence[float],
           curve_seconds: Sequence[float]) -> Tuple[tuple, float, List[float]]:
    """Best composition, its prediction, and every candidate's prediction in mask order."""
    T = len(wave_bytes)
    best, best_t, all_t = None, None, []
    for comp in enumerate_compositions(T):
        t = predict(comp, wave_bytes, duration, curve_bytes, curve_seconds)
        all_t.append(t)
        if best_t is None or t < best_t or (t == best_t and len(comp) > len(best)):
            best, best_t = comp, t
    return best, best_t, all_t


def wave_bytes_of(plan, elem_bytes: int = 2) -> List[float]:
    """Bytes of output each wave produces: its tiles' rows x cols x the element size."""
    out = [0.0] * plan.T
    for b, t in enumerate(plan.tile_of_b):
        out[b // plan.W] += plan.tile_rows[t] * plan.tile_cols[t] * elem_bytes
    return out
