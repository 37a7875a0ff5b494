"""Alternative token orders for the block partition, int64 index tables.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources:
  * tile-major order -- TRA page ("Resumen Tecnico: Atencion de Radio de Tokens para la Generacion
    Eficiente de Video", gist.science/es/paper/2608.02504), section
    "El Pipeline de TRA", item 3 "Ejecucion Eficiente", bullet "Disposicion
    Tile-Major": video tokens are laid out so that spatial neighbours inside a
    tile are contiguous in the sequence;
  * 3D Hilbert order -- DFSAttn page ("DFSAttn: Dynamic Fine-grained Sparse Attention for Efficient
    Video Generation", gist.science/es/paper/2605.23445),
    section 1, the "Curva de Hilbert" shuffle: tokens are ordered along a 3D
    Hilbert curve so that neighbours in the sequence are neighbours in space and
    time, and every block holds a coherent region.

Readings (also listed with the design notes):
  O1  tile-major: the grid is cut into tiles of tt x P x P tokens
      (tt = N / P^2 frames), tiles ordered (t, y, x) row-major, tokens inside a
      tile row-major in (t, y, x).  With tt = 1 this is the NABLA fractal order,
      so the two agree exactly when N = P^2.
  O2  Hilbert: the 3D Hilbert curve of the smallest cube of side 2^b that holds
      the grid, coordinates (t, y, x) as axes 0, 1, 2, in the transpose form of
      J. Skilling ("Programming the Hilbert curve", AIP Conf. Proc. 707, 2004);
      the tokens of a T x H x W grid are taken in increasing curve index (the
      curve restricted to the grid).  Blocks are N consecutive tokens of that
      order; they are not tiles, so the sliding-tile window does not apply.

Every function returns src with src[f] = original (t, h, w) row-major index of
the token placed at position f.
"""
import numpy as np


def tile_major_positions(T: int, H: int, W: int, P: int, N: int) -> np.ndarray:
    """Reading O1.  Needs N % (P*P) == 0 and T % (N / P^2) == 0, H % P == 0, W % P == 0."""
    if N % (P * P):
        raise ValueError("N must be a multiple of P*P")
    tt = N // (P * P)
    if T % tt or H % P or W % P:
        raise ValueError("T, H, W must be multiples of the tile (N/P^2, P, P)")
    ct, cy, cx, a, y, x = np.meshgrid(np.arange(T // tt), np.arange(H // P), np.arange(W // P),
                                      np.arange(tt), np.arange(P), np.arange(P), indexing="ij")
    src = ((ct * tt + a) * H + cy * P + y) * W + (cx * P + x)
    return src.reshape(-1).astype(np.int64)


def hilbert_index_3d(t: np.ndarray, y: np.ndarray, x: np.ndarray, bits: int) -> np.ndarray:
    """Index along the 3D Hilbert curve of side 2^bits of points (t, y, x), by
    Skilling's method: undo the curve's rotations/reflections level by level
    (top bit first) to get the "transposed" index, Gray-encode it, then read its
    bits interleaved, axis 0 first, most significant level first."""
    X = [np.asarray(t, np.int64).copy(), np.asarray(y, np.int64).copy(), np.asarray(x, np.int64).copy()]
    n = 3
    M = 1 << (bits - 1)
    Q = M
    while Q > 1:
        P = Q - 1
        for i in range(n):
            hit = (X[i] & Q) != 0
            # axis i has the level bit set: reflect the low bits of axis 0
            X[0] = np.where(hit, X[0] ^ P, X[0])
            # otherwise swap the low bits of axes 0 and i
            sw = (X[0] ^ X[i]) & P
            X[0] = np.where(hit, X[0], X[0] ^ sw)
            X[i] = np.where(hit, X[i], X[i] ^ sw)
        Q >>= 1
    for i in range(1, n):
        X[i] = X[i] ^ X[i - 1]
    t_acc = np.zeros_like(X[0])
    Q = M
    while Q > 1:
        t_acc = np.where((X[n - 1] & Q) != 0, t_acc ^ (Q - 1), t_acc)
        Q >>= 1
    for i in range(n):
        X[i] = X[i] ^ t_acc
    h = np.zeros_like(X[0])
    for b in range(bits - 1, -1, -1):
        for i in range(n):
            h = (h << 1) | ((X[i] >> b) & 1)
    return h


def hilbert_positions(T: int, H: int, W: int) -> np.ndarray:
    """Reading O2: tokens of the T x H x W grid in increasing 3D Hilbert index."""
    bits = max(1, int(np.ceil(np.log2(max(T, H, W)))))
    t, y, x = np.meshgrid(np.arange(T), np.arange(H), np.arange(W), indexing="ij")
    h = hilbert_index_3d(t.reshape(-1), y.reshape(-1), x.reshape(-1), bits)
    return np.argsort(h, kind="stable").astype(np.int64)


def block_spread(src: np.ndarray, T: int, H: int, W: int, N: int) -> float:
    """Locality metric: mean over blocks of the mean Euclidean distance of a
    block's tokens to the block's centroid, in token units of (t, y, x)."""
    t, rem = np.divmod(src, H * W)
    y, x = np.divmod(rem, W)
    pts = np.stack([t, y, x], axis=-1).astype(np.float64).reshape(-1, N, 3)
    cen = pts.mean(axis=1, keepdims=True)
    return float(np.linalg.norm(pts - cen, axis=-1).mean())
