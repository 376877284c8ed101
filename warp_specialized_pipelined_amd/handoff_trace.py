"""The hand-off ring's debug trace (plans with MIGEMM_F_HANDOFF_DEBUG).

Every wave writes one record per tile of its workgroup into the workspace:
the device's real-time clock (100 MHz) at each step of the acquire / commit /
wait / release protocol and of the consumer's copy, the ring's occupancy right
after its commit, and the tile id (include/migemm.h, migemm_debug_info, gives
the layout).  This module turns a workspace into per-record arrays and a
summary of what the protocol did: where the consumer's work on tile n ran
relative to tile n+1's K loop, how many committed tiles the ring held, how
long the waits took.
"""
from __future__ import annotations

import numpy as np

EVENTS = ("loop_begin", "loop_end", "acquired", "committed", "wait_done", "copy_first",
          "copy_last", "released")
OCCUPANCY = 8
TILE_ID = 9
TICKS_PER_US = 100.0


def records(workspace, info) -> np.ndarray:
    """The trace as uint64 [grid, waves, trace_tiles, trace_words] from a
    workspace (a torch tensor on any device, or a numpy byte array)."""
    raw = workspace.detach().cpu().numpy() if hasattr(workspace, "detach") else workspace
    raw = np.ascontiguousarray(raw).view(np.uint8).reshape(-1)
    n = info.grid * info.waves * info.trace_tiles * info.trace_words
    words = raw[info.trace_offset: info.trace_offset + 8 * n].view(np.uint64)
    return words.reshape(info.grid, info.waves, info.trace_tiles, info.trace_words)


def summarize(rec: np.ndarray, schedule: str) -> dict:
    """Protocol statistics over every wave and every pair of consecutive
    tiles (n, n+1) of a workgroup.  schedule: "overlapped" or "staged"."""
    ev = {e: rec[..., i].astype(np.int64) for i, e in enumerate(EVENTS)}
    present = ev["loop_begin"] != 0
    tiles = present.sum(axis=2)                          # per workgroup and wave
    pair = present[..., :-1] & present[..., 1:]          # (n, n+1) both present
    nxt = {e: v[..., 1:] for e, v in ev.items()}
    cur = {e: v[..., :-1] for e, v in ev.items()}
    us = lambda t: t / TICKS_PER_US

    def frac(mask):
        return float(mask[pair].mean()) if pair.any() else float("nan")

    inside_next_loop = (cur["copy_first"] >= nxt["loop_begin"]) & (cur["copy_last"] <= nxt["loop_end"])
    before_next_loop = (cur["copy_first"] >= cur["committed"]) & (cur["copy_last"] <= nxt["loop_begin"])
    release_after_next_commit = cur["released"] >= nxt["committed"]
    loop_us = us(ev["loop_end"] - ev["loop_begin"])[present]
    copy_us = us(cur["copy_last"] - cur["copy_first"])[pair]
    copy_start_in_loop = us(cur["copy_first"] - nxt["loop_begin"])[pair]
    copy_end_in_loop = us(nxt["loop_end"] - cur["copy_last"])[pair]
    acquire_us = us(ev["acquired"] - ev["loop_end"])[present]
    commit_to_wait = us(ev["wait_done"] - ev["committed"])[present]
    occ = rec[..., OCCUPANCY][present].astype(np.int64)
    q = lambda a: {"median": round(float(np.median(a)), 3), "max": round(float(np.max(a)), 3)} \
        if len(a) else None
    return {
        "schedule": schedule,
        "workgroups": int(rec.shape[0]), "waves": int(rec.shape[1]),
        "tiles_per_workgroup_max": int(tiles.max()) if tiles.size else 0,
        "tile_pairs": int(pair.sum()),
        "copy_of_tile_n_inside_k_loop_of_tile_n_plus_1": frac(inside_next_loop),
        "copy_of_tile_n_before_k_loop_of_tile_n_plus_1": frac(before_next_loop),
        "release_of_tile_n_after_commit_of_tile_n_plus_1": frac(release_after_next_commit),
        "max_committed_unreleased_tiles": int(occ.max()) if occ.size else 0,
        "k_loop_us": q(loop_us),
        "copy_window_us": q(copy_us),
        "copy_first_after_next_loop_begin_us": q(copy_start_in_loop),
        "copy_last_before_next_loop_end_us": q(copy_end_in_loop),
        "acquire_wait_us": q(acquire_us),
        "commit_to_consumer_wait_done_us": q(commit_to_wait),
    }
