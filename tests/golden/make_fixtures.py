"""Write the stored oracle fixtures under tests/golden/.

Calls only the fp64 oracle (oracle/) on seeded inputs (ddts_inputs/).  The
pages print no worked numeric example for the DDTS recurrence, so these
files are regression locks on the oracle, not values from the pages.

    python tests/golden/make_fixtures.py
"""
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import ddts_inputs as D  # noqa: E402
import oracle  # noqa: E402


def main():
    x = D.make("tiny")
    o, _ = oracle.fwd(x.q, x.k, x.v, x.g, x.tau, x.beta_hat, None)
    np.savetxt(os.path.join(HERE, "tiny_oracle_out.txt"), o.reshape(-1), fmt="%.17e",
               header="oracle output, tiny workload (B1 T64 H2 dk16 dv16, fp32 inputs, "
                      "seeded), flattened [B,T,H,dv]; written by make_fixtures.py")


if __name__ == "__main__":
    main()
