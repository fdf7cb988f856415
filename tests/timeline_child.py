"""Child process of tests/test_timeline_gpu.py: runs two workloads on
libpva_timeline.so (the library with the per-workgroup timeline compiled in)
and saves each output and its timeline records to OUT_DIR/<name>.npz.

Usage: python tests/timeline_child.py OUT_DIR"""
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(HERE))
sys.path.insert(0, HERE)

import numpy as np  # noqa: E402
import torch  # noqa: E402

import packed_varlen_masked_attn_amd as pva  # noqa: E402
from gpu_util import run_bf16, run_fp8, say  # noqa: E402
from timeline_cases import CASES  # noqa: E402


def main(out_dir):
    pva.use_timeline_build()
    for name, (w, kernel) in CASES.items():
        say(f"[timeline child] {name}")
        pva.timeline_clear(kernel)
        out, *_, desc = run_bf16(w) if kernel == "bf16" else run_fp8(w)
        recs = pva.timeline_read(kernel, len(desc.work_items))
        np.savez(os.path.join(out_dir, name + ".npz"), out=out.view(torch.int16).cpu().numpy(), records=recs,
                 items=np.asarray(desc.work_items), version=pva.version())


if __name__ == "__main__":
    main(sys.argv[1])
