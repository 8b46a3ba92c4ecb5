"""The pages' byte and operation accounting of one decode step, per head.

TEST INFRASTRUCTURE ONLY.

"Mamba-3: Improved Sequence Modeling using State Space Principles"
(intuitivepapers.ai), sections "Why a recurrent model's decode step is
memory-bound" and "MIMO: a rank-4 state update for the same state size":

* The step reads the N x P state, B and C (N numbers each per rank), the
  P channels of x per rank, and one scalar, at two bytes per number; the
  paper's count is 17,026 bytes for SISO at N=128, P=64 and 18,946 at R=4.
* The paper's operation counts are 5NP - P (SISO) and 4NPR + NP - PR (rank R).
* The page notes that neither count writes the state back; counting the full
  round trip (state read and written, one more P-sized tensor per rank) the
  intensity drops to about 1.2 (SISO) and 3.9 (R=4).
"""


def decode_tensors_read(P, N, R):
    """The tensors a decode step reads, by the page's list: (name, numbers)."""
    return [("state", N * P), ("B", N * R), ("C", N * R), ("x", P * R), ("scalar", 1)]


def decode_bytes_paper(P, N, R, nbytes=2):
    return nbytes * sum(n for _, n in decode_tensors_read(P, N, R))


def decode_bytes_round_trip(P, N, R, nbytes=2):
    """State read and written back, plus B, C, x, one output per rank, a scalar."""
    tensors = [("state read", N * P), ("state write", N * P), ("B", N * R), ("C", N * R),
               ("x", P * R), ("y", P * R), ("scalar", 1)]
    return nbytes * sum(n for _, n in tensors)


def decode_ops_paper(P, N, R):
    """Table-2 style closed form, as printed on the page."""
    if R == 1:
        return 5 * N * P - P
    return 4 * N * P * R + N * P - P * R


def intensity(ops, nbytes):
    return ops / nbytes
