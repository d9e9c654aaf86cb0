"""Independent references used by the oracle pins (numpy / torch library routines).

Nothing here calls the oracle or the GPU library.  Pools are built from dense
per-sequence K/V by numpy reshapes and block placement, not by the oracle's
own slot arithmetic; attention is dense softmax attention in float64.
"""
import numpy as np
import torch

BS = 16


def chunk_elems(dtype) -> int:
    """Elements of one 16-byte K chunk for a numpy element type."""
    return 16 // np.dtype(dtype).itemsize


def empty_pools(num_blocks, hkv, d, fill, dtype):
    """K pool [NB, H, D/X, 16, X] and V pool [NB, H, D, 16] filled with `fill`."""
    x = chunk_elems(dtype)
    kp = np.full((num_blocks, hkv, d // x, BS, x), fill, dtype=dtype)
    vp = np.full((num_blocks, hkv, d, BS), fill, dtype=dtype)
    return kp, vp


def k_rows(kp, block, offs):
    """K rows [H, n, D] of physical block `block` at offsets `offs`, by reshaping the chunked tile."""
    tile = kp[block]                      # [H, D/X, 16, X]
    h, nc, _, x = tile.shape
    return np.transpose(tile[:, :, offs, :], (0, 2, 1, 3)).reshape(h, -1, nc * x)


def v_rows(vp, block, offs):
    """V rows [H, n, D] of physical block `block` at offsets `offs` (the tile is dimension-major)."""
    return np.transpose(vp[block][:, :, offs], (0, 2, 1))


def place_dense(dense_k, dense_v, lens, perm_blocks, num_blocks, hkv, d, fill=np.nan, dtype=np.float64):
    """Build pools and a block table from dense per-sequence [L, H, D] arrays.

    Logical block j of sequence s goes to physical block perm_blocks[s][j]; the
    block's 16 rows are the dense rows 16j..16j+15 (padding past L keeps
    `fill`).  The K tile [H, 16, D] is cut into 16-byte chunks of X
    consecutive dimensions and stored chunk-major, [H, D/X, 16, X]; the V tile
    is stored dimension-major, [H, D, 16] -- both by numpy reshapes and
    transposes.
    """
    kp, vp = empty_pools(num_blocks, hkv, d, fill, dtype)
    x = chunk_elems(dtype)
    mb = max([len(p) for p in perm_blocks] + [1])
    bt = np.full((len(lens), mb), -1, dtype=np.int32)
    for s, L in enumerate(lens):
        nb = len(perm_blocks[s])
        bt[s, :nb] = perm_blocks[s]
        for j in range(nb):
            rows = slice(j * BS, min(L, (j + 1) * BS))
            n = rows.stop - rows.start
            k = np.transpose(dense_k[s][rows], (1, 0, 2))           # [H, n, D]
            kp[perm_blocks[s][j], :, :, :n, :] = np.transpose(k.reshape(hkv, n, d // x, x), (0, 2, 1, 3))
            vp[perm_blocks[s][j], :, :, :n] = np.transpose(dense_v[s][rows], (1, 2, 0))  # [H, D, n]
    return kp, vp, bt


def dense_attention_numpy(q, dense_k, dense_v, scale, group):
    """q [B, Hq, D]; dense_k/v: list of [L, Hkv, D]; float64 softmax(q K^T scale) V."""
    B, Hq, D = q.shape
    out = np.zeros((B, Hq, D))
    for s in range(B):
        K, V = dense_k[s], dense_v[s]
        if K.shape[0] == 0:
            continue
        for h in range(Hq):
            g = h // group
            sc = (K[:, g, :] @ q[s, h]) * scale
            w = np.exp(sc - sc.max())
            out[s, h] = (w / w.sum()) @ V[:, g, :]
    return out


def dense_attention_torch(q, dense_k, dense_v, scale, group):
    """Same via torch.nn.functional.scaled_dot_product_attention in float64 on the CPU."""
    B, Hq, D = q.shape
    out = np.zeros((B, Hq, D))
    for s in range(B):
        K, V = dense_k[s], dense_v[s]
        if K.shape[0] == 0:
            continue
        Kt = torch.from_numpy(np.ascontiguousarray(np.repeat(K, group, axis=1).transpose(1, 0, 2)))
        Vt = torch.from_numpy(np.ascontiguousarray(np.repeat(V, group, axis=1).transpose(1, 0, 2)))
        qt = torch.from_numpy(np.ascontiguousarray(q[s][:, None, :]))
        o = torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt, scale=scale)
        out[s] = o[:, 0, :].numpy()
    return out
