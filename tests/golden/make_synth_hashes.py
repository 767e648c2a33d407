"""Write synth_sha256.txt: SHA-256 of every array the tiny and decode workloads
generate, so a change to the generators (draw order, dtype, shapes) is caught."""
import hashlib
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))
import synth  # noqa: E402


def digests(i):
    w = synth.workload(i)
    L = w.layers[0]
    arrays = {"x": w.x, "w_router": L.w_router}
    for n in ("gate", "up", "down"):
        arrays[f"{n}.codes"] = getattr(L, n).codes
        arrays[f"{n}.scales"] = getattr(L, n).scales
    arrays.update(b_gate=L.b_gate, b_up=L.b_up, b_down=L.b_down)
    if L.b_router is not None:
        arrays["b_router"] = L.b_router
    return {k: hashlib.sha256(v.tobytes()).hexdigest() for k, v in arrays.items()}


if __name__ == "__main__":
    with open(os.path.join(HERE, "synth_sha256.txt"), "w") as f:
        f.write("# SHA-256 of generated arrays; written by make_synth_hashes.py\n")
        for i in (0, 1):
            for k, v in digests(i).items():
                f.write(f"{i} {k} {v}\n")
