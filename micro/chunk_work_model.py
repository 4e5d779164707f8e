"""Host model of the octet kernel's per-chunk matrix-core work on the 16x8
frame-structured mask (no GPU): how much of the headline's time padding and
the per-chunk barrier can account for, and what carrying leftover octets
across chunks would recover.

A work-group is 16 waves, one 16-row query tile each, wave w on SIMD w % 4.
Per chunk a wave runs ceil(k/4) passes for its k kept octets (a pass with at
most two real octets skips its second score block: cost 0.75).  The chunk's
time is the busiest SIMD's pass count (the barrier); with a window of c
chunks, the busiest SIMD's count over the window.  With carrying, a wave
runs floor((carry + k) / 4) passes and carries the rest.  Everything is
relative to the kept octets / 4 spread evenly over the SIMDs.

    python micro/chunk_work_model.py
"""
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import workloads as W  # noqa: E402


def model(keep, octets_per_chunk):
    T_k = keep.shape[1]
    nch = -(-T_k // octets_per_chunk)
    pad = np.zeros((16, nch * octets_per_chunk), bool)
    pad[:, :T_k] = keep
    k = pad.reshape(16, nch, octets_per_chunk).sum(2)
    useful = (k / 4).sum() / 4
    S = np.zeros((4, nch))
    Sc = np.zeros((4, nch))
    for wv in range(16):
        S[wv % 4] += np.ceil(k[wv] / 4) - 0.25 * ((k[wv] % 4 != 0) & (k[wv] % 4 <= 2))
        carry = 0
        for c in range(nch):
            t = carry + k[wv, c]
            Sc[wv % 4, c] += t // 4
            carry = t % 4
    win = {c: sum(S[:, i:i + c].sum(1).max() for i in range(0, nch, c)) / useful for c in (1, 2, 4)}
    return S.mean(0).sum() / useful, win, Sc.max(0).sum() / useful


def main():
    w = W.get("wan480_fine")
    rng = np.random.default_rng(0)
    groups = [(h, int(qb)) for h in (0, 7, 21, 33) for qb in rng.choice(w.T_q // 16, 10, replace=False)]
    for opc in (8, 12, 16, 24):
        acc = np.zeros(5)
        for h, qb in groups:
            keep = W.mask_rows_bool(w, [(0, h, qb * 16 + i) for i in range(16)])
            bal, win, carry = model(keep, opc)
            acc += [bal, win[1], win[2], win[4], carry]
        acc /= len(groups)
        print(f"{8 * opc:3d}-key chunks: padded, balanced {acc[0]:.3f} | barrier per chunk {acc[1]:.3f} | "
              f"per 2 chunks {acc[2]:.3f} | per 4 chunks {acc[3]:.3f} | carried, barrier per chunk {acc[4]:.3f}")


if __name__ == "__main__":
    main()
