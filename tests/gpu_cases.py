"""Helpers shared by the GPU parity tests: run a synth.Case through the HIP
library (via the C-ABI binding) and through the fp64 oracle."""
from __future__ import annotations

import numpy as np
import torch

import decode_attention_slidingdecodegqa_amd as gqa
import oracle
import synth

TOL = {"f32": 1e-4, "bf16": 2e-2}  # max-abs error bars for unit-RMS values
# the planner's mode for units split across slices: wave slices (stream) on the
# sliding geometry, work-group slices (group) on the global one
SPLIT_MODE = {"sliding": "stream", "global": "group"}


def hip_run(case: synth.Case, workspace=None, stream=None, o=None, window=None) -> torch.Tensor:
    if window is not None:
        if case.block_table is None:
            return gqa.gqa_decode_sliding_window(case.q, case.k, case.v, case.seq_lens, window,
                                                 o=o, workspace=workspace, stream=stream)
        return gqa.gqa_decode_sliding_window_paged(case.q, case.k, case.v, case.block_table,
                                                   case.seq_lens, window, o=o,
                                                   workspace=workspace, stream=stream)
    if case.variant == "sliding":
        fn_c, fn_p = gqa.gqa_decode_sliding, gqa.gqa_decode_sliding_paged
    else:
        fn_c, fn_p = gqa.gqa_decode_global, gqa.gqa_decode_global_paged
    if case.block_table is None:
        return fn_c(case.q, case.k, case.v, case.seq_lens, o=o, workspace=workspace,
                    stream=stream)
    return fn_p(case.q, case.k, case.v, case.block_table, case.seq_lens, o=o,
                workspace=workspace, stream=stream)


def oracle_run(case: synth.Case, rows=None, window=None, nthreads=16) -> np.ndarray:
    bt = None if case.block_table is None else synth.to_numpy(case.block_table)
    return oracle.gqa_decode((case.KV, case.D, case.window if window is None else window),
                             synth.to_numpy(case.q), synth.to_numpy(case.k),
                             synth.to_numpy(case.v), synth.to_numpy(case.seq_lens),
                             block_table=bt, rows=rows, nthreads=nthreads)


def to_f64(o: torch.Tensor) -> np.ndarray:
    return o.detach().to(torch.float64).cpu().numpy()


def max_err(a: np.ndarray, b: np.ndarray) -> float:
    if a.size == 0:
        return 0.0
    d = np.abs(a - b)
    if not np.isfinite(d).all():
        return float("inf")
    return float(d.max())


def to_gpu(case: synth.Case) -> synth.Case:
    dev = "cuda"
    return synth.Case(case.variant, case.dtype, case.q.to(dev), case.k.to(dev), case.v.to(dev),
                      case.seq_lens.to(dev),
                      None if case.block_table is None else case.block_table.to(dev),
                      case.cap, case.window, None if case.w_k is None else case.w_k.to(dev))


def to_cpu(case: synth.Case) -> synth.Case:
    return synth.Case(case.variant, case.dtype, case.q.cpu(), case.k.cpu(), case.v.cpu(),
                      case.seq_lens.cpu(),
                      None if case.block_table is None else case.block_table.cpu(),
                      case.cap, case.window, None if case.w_k is None else case.w_k.cpu())


def hip_run_k_eq_v(case: synth.Case, workspace=None, stream=None, o=None) -> torch.Tensor:
    """The values-only global call on the case's v and w_k (its k is not read)."""
    if case.block_table is None:
        return gqa.gqa_decode_global_k_eq_v(case.q, case.v, case.w_k, case.seq_lens, o=o,
                                            workspace=workspace, stream=stream)
    return gqa.gqa_decode_global_k_eq_v_paged(case.q, case.v, case.w_k, case.block_table,
                                              case.seq_lens, o=o, workspace=workspace,
                                              stream=stream)


def oracle_run_k_eq_v(case: synth.Case, rows=None, nthreads=16) -> np.ndarray:
    bt = None if case.block_table is None else synth.to_numpy(case.block_table)
    return oracle.gqa_decode_k_from_v(synth.to_numpy(case.q), synth.to_numpy(case.v),
                                      synth.to_numpy(case.w_k), synth.to_numpy(case.seq_lens),
                                      block_table=bt, rows=rows, nthreads=nthreads)
