"""Hand-built int4 expert whose output exposes the int8 codes of its activations.

Int4 group-128 weights with int8 per-row activations (the int4 workload's W4A8
definition): x and the SwiGLU intermediate h are each quantised per row with
s = max|row| / 127 and q = rint(v / s) (ties to even), then multiplied by the
exactly dequantised int4 weights. The expert below makes every step exact, so
its output can be written down by hand:

  token row 0: x = [127, 64, 2.5, 3.5, -2.5, 1.5, 0, ...]  -> s_x = 1,
               codes [127, 64, 2, 4, -2, 2, 0, ...] (half steps round to even)
  token row 1: twice row 0 -> s_x = 2, the same codes
  gate row n:  code 1 at input 1, scale 1            -> g = 64 (row 0), 128 (row 1);
               SiLU(g) = g exactly at these sizes (e^-64 vanishes next to 1)
  up row n:    n < 10: code d_n at input 1, scale s_n -> h[n] = 4096 d_n s_n
               n = 10..13: code 1 at input 2..5, scale 2^-6 -> h[n] = x_hat[2..5]
  h row 0:     127, 2.5, 3.5, -2.5, 126.5, 0.5, 1.5, -1.5, -8, 1.75, 2, 4, -2, 2, 0, ...
               -> s_h = 1, codes 127, 2, 4, -2, 126, 0, 2, -2, -8, 2, 2, 4, -2, 2, 0, ...
  h row 1:     4 h_row0 -> s_h = 4, the same codes
  down row i:  code 1 at input i (i < F), scale 1     -> y[i] = h_hat[i], 0 for i >= F
"""
import numpy as np
import torch

UP_ROWS = [(1, 127 * 2.0 ** -12), (5, 2.0 ** -13), (7, 2.0 ** -13), (-5, 2.0 ** -13),
           (1, 253 * 2.0 ** -13), (1, 2.0 ** -13), (3, 2.0 ** -13), (-3, 2.0 ** -13),
           (-8, 2.0 ** -12), (7, 2.0 ** -14)]
X_ROW0 = [127.0, 64.0, 2.5, 3.5, -2.5, 1.5]
X_CODES = [127, 64, 2, 4, -2, 2]
H_CODES = [127, 2, 4, -2, 126, 0, 2, -2, -8, 2, 2, 4, -2, 2]


def nibbles(codes) -> np.ndarray:
    """Signed codes [rows, K] -> packed bytes [rows, K/2], even K in the low nibble."""
    c = np.asarray(codes, dtype=np.int64) & 0xF
    return (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)


def w4a8_expert(H: int, F: int) -> dict:
    """Weights of the expert above (nn.Linear orientation, packed codes, bf16 scales)."""
    assert H % 128 == 0 and F % 128 == 0 and H >= F >= 16
    gate = np.zeros((F, H), np.int64)
    gate[:, 1] = 1
    up = np.zeros((F, H), np.int64)
    su = np.ones((F, H // 128))
    for n, (d, sn) in enumerate(UP_ROWS):
        up[n, 1], su[n, 0] = d, sn
    for n, c in zip(range(10, 14), range(2, 6)):
        up[n, c], su[n, 0] = 1, 2.0 ** -6
    down = np.zeros((H, F), np.int64)
    down[np.arange(F), np.arange(F)] = 1
    bf = lambda a: torch.tensor(a, dtype=torch.bfloat16)  # noqa: E731
    w = {"gate_q": torch.from_numpy(nibbles(gate)), "gate_s": bf(np.ones((F, H // 128))),
         "up_q": torch.from_numpy(nibbles(up)), "up_s": bf(su),
         "down_q": torch.from_numpy(nibbles(down)), "down_s": bf(np.ones((H, F // 128)))}
    assert w["up_s"].double().numpy().tolist() == su.tolist()  # every scale is a bf16 value
    return w


def tokens(T: int, H: int) -> np.ndarray:
    """T token rows alternating between row 0 and row 1 (twice row 0), float32."""
    x = np.zeros((T, H), np.float32)
    x[:, :6] = X_ROW0
    x[1::2] *= 2
    return x


def expected_y(T: int, H: int, F: int) -> np.ndarray:
    y = np.zeros((T, H))
    y[:, :len(H_CODES)] = H_CODES
    y[1::2] *= 4
    return y


def expected_codes(T: int, H: int, F: int):
    """(x codes [T, H], x scales [T], h codes [T, F], h scales [T]) of the expert above."""
    xq = np.zeros((T, H), np.int8)
    xq[:, :6] = X_CODES
    hq = np.zeros((T, F), np.int8)
    hq[:, :len(H_CODES)] = H_CODES
    xs = np.where(np.arange(T) % 2 == 0, 1.0, 2.0).astype(np.float32)
    hs = np.where(np.arange(T) % 2 == 0, 1.0, 4.0).astype(np.float32)
    return xq, xs, hq, hs
