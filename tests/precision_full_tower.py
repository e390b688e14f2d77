"""The bf16 rounding model (precision_model.py) against the fp32 oracle through the whole
2048^2 CFG tower step: 36 layers, 2 x 4096 tokens, prefix 400, cfg 4, step 0 of 50.  Prints each
branch's x0 cosine, the guided x0's and the Euler update's, i.e. what a correct bf16
implementation of the step reaches, next to which the GPU's figures are read.  A script, not a
test (about 40 minutes on 8 cores, 10 GB of memory):

    python tests/precision_full_tower.py [n_layers] [--exact u2,z]

--exact leaves the listed rounding points of precision_model.POINTS in fp32.
"""
import os
import sys
import time

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
import oracle as O            # noqa: E402
import workloads as W         # noqa: E402
from precision_model import gen_block_bf16   # noqa: E402


def cos(a, b):
    a, b = np.asarray(a, np.float64).ravel(), np.asarray(b, np.float64).ravel()
    return float(a @ b / np.linalg.norm(a) / np.linalg.norm(b))


def main():
    args = [a for a in sys.argv[1:] if not a.startswith("--")]
    exact = ()
    if "--exact" in sys.argv:
        exact = tuple(sys.argv[sys.argv.index("--exact") + 1].split(","))
    w = W.CONFIGS[2]
    L = int(args[0]) if args else w.n_layers
    sched = O.sigma_schedule(w.n_steps, w.shift)
    glob = W.tower_globals(w, 0, "bf16")
    x = W.noise_image(w)
    tok = O.patchify(x)
    h0 = O.linear(tok[0], glob["w_in"]) + O.timestep_embed(sched[0], glob["temb_w1"], glob["temb_w2"])
    hr = np.stack([h0, h0])
    hm = hr.copy()
    t0 = time.time()
    for l in range(L):
        wts = W.layer_weights(w, l, 0, "bf16")
        pk = [W.prefix_kv(w, l, s, 0, "bf16")[0] for s in range(2)]
        pv = [W.prefix_kv(w, l, s, 0, "bf16")[1] for s in range(2)]
        hr = O.gen_block(hr, wts, w.dims, pk, pv)
        hm = gen_block_bf16(hm, wts, w.dims, pk, pv, exact=exact)
        print(f"layer {l} {time.time() - t0:.0f} s", flush=True)

    def head(h):
        return O.linear(O.rms_norm(h, glob["g_final"], w.dims.rms_eps), glob["w_out"])
    yr, ym = head(hr), head(hm)
    gr, gm = O.cfg_mix(yr[0], yr[1], w.cfg_scale), O.cfg_mix(ym[0], ym[1], w.cfg_scale)
    xt = tok[0]
    dr = O.euler_step(xt, gr, sched[0], sched[1], w.t_eps) - xt
    dm = O.euler_step(xt, gm, sched[0], sched[1], w.t_eps) - xt
    print(f"|x0_c - x0_u| / |x0_c| = {np.linalg.norm(yr[0] - yr[1]) / np.linalg.norm(yr[0]):.4f}")
    print(f"rounding model (exact: {exact or 'none'}): branch cos {cos(ym[0], yr[0]):.6f} {cos(ym[1], yr[1]):.6f}, "
          f"guided cos {cos(gm, gr):.6f}, dx cos {cos(dm, dr):.6f}")


if __name__ == "__main__":
    main()
