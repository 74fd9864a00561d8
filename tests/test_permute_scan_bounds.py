"""Host replay of the three-launch permute's scan loads (k_scan in
csrc/permute.hip): every table entry that any of the 1024 scan threads
loads must lie inside the workspace that nvfp4moe_permute_workspace_size
reports. The index formulas below restate the kernel's: per expert
`parts = 1024 // n_local` threads, `per = ceil(n_chunks / parts)` chunks
each, a thread with an empty range starting at its expert's first entry,
and kScanRegs = 32 entries loaded per batch unconditionally."""

import pytest

K_CHUNK = 256          # flat pairs per histogram workgroup
SCAN_REGS = 32         # entries one scan thread loads per batch
SMALL_MAX = 16384      # largest T*k taking the one-launch form


def workspace_entries(n, n_local):
    n_chunks = (n + K_CHUNK - 1) // K_CHUNK
    return (max(n_chunks, 1) * n_local * 4 + 256) // 4


def max_loaded_entry(n, n_local):
    n_chunks = (n + K_CHUNK - 1) // K_CHUNK
    parts = 1024 // n_local
    per = (n_chunks + parts - 1) // parts
    hi = -1
    for tid in range(1024):
        e, part = tid // parts, tid % parts
        if e >= n_local:
            c0 = c1 = 0
            base = 0
        else:
            c0 = part * per
            c1 = min(c0 + per, n_chunks)
            cnt = max(c1 - c0, 0)
            base = e * n_chunks + (c0 if cnt > 0 else 0)
        cnt = max(c1 - c0, 0)
        # first batch (always), then batches b = 32, 64, ... while b < cnt
        last = SCAN_REGS - 1
        b = SCAN_REGS
        while b < cnt:
            last = b + SCAN_REGS - 1
            b += SCAN_REGS
        hi = max(hi, base + last)
    return hi


@pytest.mark.parametrize("n_local", [1, 2, 3, 4, 7, 8, 16, 48, 100, 384, 1000, 1024])
@pytest.mark.parametrize("n", [SMALL_MAX + 1, SMALL_MAX + 256, 16640, 40000, 262144, 1 << 20])
def test_scan_loads_stay_in_workspace(n, n_local):
    assert max_loaded_entry(n, n_local) < workspace_entries(n, n_local)


def test_replay_catches_the_unclamped_form():
    """The replay is sharp: the earlier form, which formed an empty range's
    address from its start c0, reads past the workspace for one local
    expert and 16385 pairs."""
    n, n_local = SMALL_MAX + 1, 1
    n_chunks = (n + K_CHUNK - 1) // K_CHUNK
    parts = 1024 // n_local
    per = (n_chunks + parts - 1) // parts
    worst = max(part * per for part in range(parts)) + SCAN_REGS - 1
    assert worst >= workspace_entries(n, n_local)
