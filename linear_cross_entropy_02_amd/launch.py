"""Launch settings chosen by shape: tokens per chunk C, chunks per dW GEMM G
and whether the dX contraction reads a transposed copy of W.

The settings are the fastest measured (MI355X, one box, alternating runs)
for the head shapes the library is tuned on; between them the rule below
interpolates by hidden size.  They trade workspace for speed: the
exponentials of G chunks are kept so that the fp32 dW tiles are read and
written once per G chunks, and the W^T copy makes the dX contraction read
16-byte fragments.
  * H >= 2048: C = 2048, G = 4 up to H = 4096, G = 2 above (8192 x 8192 x
    128256: 39.4 ms; G = 1: 42.2), with W read as stored wherever the
    library takes it (bf16, V H 2 < 2^31 bytes): at 16384 x 4096 x 128256
    that costs 1-2 % of a step (41.0 against 40.6 ms on one box, 39.5
    against 38.8 on another) and takes the workspace from 0.79 to 0.56 of a
    bf16 T x V buffer (G = 2 with the copy: +4 % at 0.53; C = 4096, G = 1:
    +3.6 % at 0.52).
  * H < 2048: for batches of 32768 tokens or more, G = 1 and the largest
    C of 8192, 16384 and 32768 that is at most half the batch, so that the
    exponentials stay within half of a T x V buffer (65536 x 512 x 16000:
    C = 32768 4.00 ms at 0.55 of the buffer, 16384 4.14 ms, 8192 4.43 ms);
    smaller batches C = 2048, G = 1 reading W as stored (4096 x 512 x 16000:
    0.37 ms; C = 1024, G = 2: 0.43 ms).
  * fp32: one chunk of up to 4096 tokens, G = 1.
C never exceeds the batch (rounded up to 256) and G the number of chunks.
"""
from __future__ import annotations


def suggest_launch(T: int, H: int, V: int, dtype: str = "bf16"):
    """(chunk_tokens, dw_chunks, weight_copy) for a batch of T tokens."""
    if dtype == "f32":
        C, G, wcopy = 4096, 1, True
    elif H >= 2048:
        C = 2048
        G = 4 if H <= 4096 else 2
        wcopy = V * H * 2 >= 2 ** 31
    elif T >= 32768:
        C = max(c for c in (8192, 16384, 32768) if 2 * c <= T)
        G, wcopy = 1, True
    else:
        C, G, wcopy = 2048, 1, False
    tpad = max(256, -(-max(T, 1) // 256) * 256)
    C = min(C, tpad)
    G = max(1, min(G, -(-max(T, 1) // C)))
    return C, G, wcopy
