"""Write the tile-census fixtures in this folder from the CPU oracle only.

Each fixture is the brute-force census of ``oracle.live_tiles`` (every
(query, key) pair checked against original positions) for one workload
shape, layout and tile size, plus the live pair counts of
``oracle.live_pairs``. The quantity is the per-round, per-device live work
whose spread across devices is the load imbalance the pages describe
(Striped Attention summary page, "Key points: Imbalance"; notes page at
phantomic12.github.io ¶1), and whose striped version is about half of each
block in every round ("Summary" ¶2).

Usage: python tests/golden/make_golden.py
"""

import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402

CASES = [
    # (name, seq, n_dev, tile_q, tile_k)
    ("tiny_q64_k16", 256, 4, 64, 16),
    ("tiny_q16_k16", 256, 4, 16, 16),
    ("short_q128_k64", 8192, 8, 128, 64),
    ("short_q128_k128", 8192, 8, 128, 128),
    ("ragged_q128_k64", 8 * 200, 8, 128, 64),
]


def main():
    for name, seq, n_dev, tq, tk in CASES:
        rec = {"seq": seq, "n_dev": n_dev, "tile_q": tq, "tile_k": tk,
               "index": "[round][device]", "source": "oracle.live_tiles / oracle.live_pairs (brute force)"}
        for layout, lname in ((oracle.CONTIGUOUS, "contiguous"), (oracle.STRIPED, "striped")):
            live, full, part = oracle.live_tiles(seq, n_dev, layout, tq, tk)
            rec[lname] = {"live": live.tolist(), "full": full.tolist(), "partial": part.tolist(),
                          "pairs": oracle.live_pairs(seq, n_dev, layout).tolist()}
        path = os.path.join(HERE, f"census_{name}.json")
        with open(path, "w") as f:
            json.dump(rec, f, indent=None, separators=(",", ":"))
            f.write("\n")
        print(path)


if __name__ == "__main__":
    main()
