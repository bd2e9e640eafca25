"""Prefill-kernel parity cases run against the debug build (libpkv_debug.so: every
LDS tile buffer NaN-filled before each item), in a process of their own (the
library is chosen when the binding loads). A tile read before its load has landed
would put NaN into the output. Run by tests/test_gpu_lds_poison.py."""

import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(HERE))
sys.path.insert(0, HERE)


def main():
    assert os.environ.get("PKV_LIBRARY") == "libpkv_debug.so"
    import numpy as np
    import torch

    import oracle
    from paged_kv_cache_173_amd import pkv
    from paged_kv_cache_173_amd import workloads as wl
    from gpu_common import Uploaded, compare, dev, dev_i32, run_gpu, run_oracle, say

    assert pkv.LIB_PATH.endswith("libpkv_debug.so")
    ws = pkv.Workspace()
    n = 0
    for P in (1, 5, 16, 64):
        for heads in ((32, 8), (8, 8), (64, 1)):
            for causal in (True, False):
                for sched in (None, (64, 1, 16)):
                    w = wl.batch_prefill(seed=500 + P + heads[0], qo_lens=[1, 7, 64, 130, 300],
                                         prefix_lens=[0, 5, 61, 200, 33], num_qo_heads=heads[0],
                                         num_kv_heads=heads[1], page_size=P, dtype="bf16",
                                         causal=causal, canary=True)
                    label = f"poisoned LDS: prefill P={P} heads={heads} causal={causal} sched={sched}"
                    say(f"[case] {label}")
                    o, lse = run_gpu(pkv, Uploaded(w), ws, sched=sched)
                    O, LSE = run_oracle(w)
                    compare(w, o, lse, O, LSE, label=label)
                    n += 1
    for pre, P, sfx in ((2000, 16, [5, 0, 900]), (333, 8, [17, 1, 64, 0])):
        w = wl.cascade(seed=510 + pre, batch=len(sfx), prefix_len=pre, suffix_lens=sfx,
                       page_size=P, canary=True)
        say(f"[case] poisoned LDS: cascade prefix={pre} P={P}")
        o, lse = run_gpu(pkv, Uploaded(w), ws, sched=(256, 16, 16))
        O, LSE = run_oracle(w)
        compare(w, o, lse, O, LSE, label=f"poisoned LDS: cascade prefix={pre}")
        n += 1
    for R, C in ((64, 64), (7, 13), (128, 128)):
        w = wl.block_sparse(seed=520 + R, num_qo_tokens=333, num_kv_tokens=517, row_block=R,
                            col_block=C, density=0.35, num_qo_heads=8, num_kv_heads=2,
                            dtype="bf16", empty_rows=(1,))
        say(f"[case] poisoned LDS: block-sparse R={R} C={C}")
        plan = pkv.pkv_block_sparse_plan(w.bsr_indptr, w.bsr_indices, w.q.shape[0], w.k.shape[0],
                                         R, C, 8, 2, 128, torch.bfloat16, ws)
        o, lse = pkv.pkv_block_sparse_run(plan, dev(w.q, "bf16"), dev(w.k, "bf16"),
                                          dev(w.v, "bf16"), dev_i32(w.bsr_indptr),
                                          dev_i32(w.bsr_indices), w.sm_scale)
        torch.cuda.synchronize()
        O, LSE = oracle.block_sparse_attention(w.q, w.k, w.v, w.dtype, w.bsr_indptr,
                                               w.bsr_indices, R, C, w.sm_scale)
        compare(w, o.float().cpu().numpy().astype(np.float64),
                lse.cpu().numpy().astype(np.float64), O, LSE, label=f"block-sparse R={R}")
        n += 1
    w = wl.pod(seed=530, qo_lens=[40, 300], prefix_lens=[0, 90], d_lens=[1, 700, 1500],
               canary=True)
    wp, wd = w.prefill, w.decode
    say("[case] poisoned LDS: mixed batch")
    plan = pkv.pkv_pod_plan(wp.qo_indptr, wp.kv.kv_indptr, wp.kv.last_page_len, True,
                            wd.kv.kv_indptr, wd.kv.last_page_len, 32, 8, 128, 16, torch.bfloat16,
                            ws, sched=(64, 1, 16))
    k, v = dev(wp.kv.k_cache, "bf16"), dev(wp.kv.v_cache, "bf16")
    o_p, l_p, o_d, l_d = pkv.pkv_pod_run(plan, k, v, dev(wp.q, "bf16"), dev_i32(wp.qo_indptr),
                                         dev_i32(wp.kv.kv_indptr), dev_i32(wp.kv.kv_indices),
                                         dev(wd.q, "bf16"), dev_i32(wd.kv.kv_indptr),
                                         dev_i32(wd.kv.kv_indices), wp.sm_scale)
    torch.cuda.synchronize()
    for part, o, lse in ((wp, o_p, l_p), (wd, o_d, l_d)):
        O, LSE = run_oracle(part)
        compare(part, o.float().cpu().numpy().astype(np.float64),
                lse.cpu().numpy().astype(np.float64), O, LSE, label=f"mixed batch {part.kind}")
    n += 1
    say(f"lds poison: {n} cases ok")


if __name__ == "__main__":
    main()
