"""Why the parity bound is taken on o emitted in fp32.

For bf16 inputs the bound is 2e-2 in max |gpu - oracle| / rms(oracle).  Rounding
the oracle's own o to bf16 (round to nearest even) already exceeds it on the
batched-prefill workload (B2 H4 T2048, dk = dv = 128): the heavy tail of o
makes half a bf16 ulp at the largest outputs worth more than 2e-2 of the RMS.
No implementation can meet the bound with a bf16 o, so parity is measured on
the fp32 o and the bf16 o is checked to be its exact rounding.
"""
import numpy as np
import torch

import workloads
from oracle import kda_oracle


def test_bf16_rounding_of_exact_output_exceeds_bound():
    inp = workloads.config_inputs(workloads.BATCHED_PREFILL)
    o, _ = kda_oracle.forward(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"],
                              heads=(0, 2))
    ob = torch.from_numpy(o).to(torch.bfloat16).double().numpy()
    err = np.max(np.abs(ob - o)) / np.sqrt(np.mean(o ** 2))
    assert err > 2e-2, err
