"""python -m oracle.run_length_study: the exact (ideal) CR of K and V for
packing runs of 16, 32 and 64 slots, on seeded synthetic streams, for the
three token orders.  Oracle code only; the format itself keeps R = 32.
"""

import kvsynth

from .cr import run_length_study


def main():
    print("| data | b | B | order | R = 16 K / V | R = 32 K / V | R = 64 K / V |")
    print("|---|---|---|---|---|---|---|")
    cases = [("clustered, groups of 32", "struct", 32, ((4, 64), (2, 64), (4, 128))),
             ("clustered, groups of 16", "struct", 16, ((4, 128),)),
             ("clustered, groups of 64", "struct", 64, ((4, 128),)),
             ("gaussian", "gauss", 0, ((4, 64), (2, 64), (4, 128)))]
    for name, law, group, shapes in cases:
        for bits, block in shapes:
            streams = []
            for s in range(2):
                if law == "struct":
                    streams.append(kvsynth.structured_kv(1024, 128, block, group, seed=100 + s))
                else:
                    w = kvsynth.Workload("study", 1, 2, 1, 1024, 128, bits, block, "gauss")
                    streams.append(kvsynth.stream_kv(w, s, seed=7, tokens=1024))
            for permute, oname in ((0, "identity"), (1, "greedy"), (2, "sort key")):
                res = run_length_study(streams, bits, block, permute)
                cells = " | ".join(f"{res[r][0]:.2f} / {res[r][1]:.2f}" for r in (16, 32, 64))
                print(f"| {name} | {bits} | {block} | {oname} | {cells} |", flush=True)


if __name__ == "__main__":
    main()
