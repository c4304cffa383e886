"""Cache layout marshalling (plain data movement, no arithmetic).

bf16 caches are stored in 16-row tiles in the order the matrix-core attention
reads its operands:
  K: [nkv, rows/16, hd/8, 16, 8]  (each tile: 8-dim groups of its 16 rows)
  V: [nkv, rows/16, hd, 16]       (each tile transposed: its 16 rows contiguous)
f32 caches are row-major, [nkv, rows, hd].  These helpers convert between the
row-major view and the tiled ones, for numpy arrays and torch tensors alike.
"""
T = 16   # rows per tile
G8 = 8   # dims per K group


def _perm(t, axes):
    return t.permute(*axes) if hasattr(t, "permute") else t.transpose(axes)


def _copy(t):
    return t.contiguous() if hasattr(t, "contiguous") else t.copy()


def k_to_tiles(k):
    """[nkv, rows, hd] (rows % 16 == 0, hd % 8 == 0) -> [nkv, rows/16, hd/8, 16, 8]."""
    nkv, rows, hd = k.shape
    assert rows % T == 0 and hd % G8 == 0, (rows, hd)
    return _copy(_perm(k.reshape(nkv, rows // T, T, hd // G8, G8), (0, 1, 3, 2, 4)))


def k_from_tiles(t):
    nkv, nt, ng, tr, g8 = t.shape
    assert tr == T and g8 == G8, t.shape
    return _copy(_perm(t, (0, 1, 3, 2, 4))).reshape(nkv, nt * T, ng * G8)


def v_to_tiles(v):
    """[nkv, rows, hd] (rows % 16 == 0) -> [nkv, rows/16, hd, 16]."""
    nkv, rows, hd = v.shape
    assert rows % T == 0, rows
    return _copy(_perm(v.reshape(nkv, rows // T, T, hd), (0, 1, 3, 2)))


def v_from_tiles(t):
    nkv, nt, hd, tr = t.shape
    assert tr == T, t.shape
    return _copy(_perm(t, (0, 1, 3, 2))).reshape(nkv, nt * T, hd)
