"""CPU tests of the offline cache of encoded weights (usw.save / usw.load):
every host encoding kind round-trips byte for byte, the archive holds no
pickled object, and damaged or foreign archives are rejected before any of
their buffers reaches a kernel.  No kernel is launched."""
import numpy as np
import pytest

import unstructured_sparse_weight_amd as usw
import workloads as wl


def case(M, K, keep, seed):
    rng = np.random.default_rng(seed)
    W = wl.weight_normal(M, K, rng)
    return W, wl.mask_bernoulli(M, K, keep, rng)


def same(a, b):
    for name in a.__dataclass_fields__:
        x, y = getattr(a, name), getattr(b, name)
        if isinstance(x, np.ndarray) or isinstance(y, np.ndarray):
            assert x is not None and y is not None and x.dtype == y.dtype and np.array_equal(x, y), name
        else:
            assert x == y, name


def encodings():
    W, mask = case(128, 256, 0.5, 3)
    perms = np.array([np.random.default_rng(t).permutation(16) for t in range(8 * 4)], dtype=np.int32)
    yield "tca_f16", usw.encode_host(W, mask, (64, 64), "f16")
    yield "tca_i4", usw.encode_host(W, mask, (32, 16), "i4")
    yield "union_i4", usw.union_encode_host(W, mask, (64, 64), (2, 2), "i4")
    yield "union_i2_reordered", usw.union_encode_host(W, mask, (16, 64), (4, 1), "i2", perm=perms)
    Wc, maskc = case(256, 64, 0.3, 4)
    yield "cbc", usw.cbc_encode_host(Wc, maskc)


@pytest.mark.parametrize("name,enc", list(encodings()), ids=[n for n, _ in encodings()])
def test_round_trip(tmp_path, name, enc):
    p = tmp_path / f"{name}.npz"
    usw.save(p, enc)
    back = usw.load(p)
    assert type(back) is type(enc)
    same(enc, back)
    with np.load(p, allow_pickle=False) as z:          # plain arrays only
        assert all(z[k].dtype != object for k in z.files)


def test_rejects_damaged_archives(tmp_path):
    W, mask = case(128, 256, 0.5, 5)
    enc = usw.encode_host(W, mask, (64, 64), "f16")
    good = tmp_path / "good.npz"
    usw.save(good, enc)
    with np.load(good) as z:
        fields = {k: z[k] for k in z.files}

    def write(name, **over):
        d = dict(fields)
        for k, v in over.items():
            if v is None:
                d.pop(k)
            else:
                d[k] = v
        p = tmp_path / name
        np.savez(p, **d)
        return p

    bad_off = fields["offsets"].copy()
    bad_off[3] += 1                                     # an offset that disagrees with the bitmaps
    with pytest.raises(usw.UswError):
        usw.load(write("offsets.npz", offsets=bad_off))
    with pytest.raises(ValueError):
        usw.load(write("short.npz", bitmaps=fields["bitmaps"][:-1]))
    with pytest.raises(ValueError):
        usw.load(write("dtype.npz", offsets=fields["offsets"].astype(np.int64)))
    with pytest.raises(ValueError):
        usw.load(write("nokind.npz", kind=None))
    with pytest.raises(ValueError):
        usw.load(write("kind.npz", kind=np.array("dense")))
    with pytest.raises(ValueError):
        usw.load(write("noM.npz", M=None))
    with pytest.raises(ValueError):
        usw.load(write("shape.npz", gt_m=np.array(48, dtype=np.int64)))
    obj = tmp_path / "obj.npz"
    np.savez(obj, kind=np.array([{"x": 1}], dtype=object))
    with pytest.raises(ValueError):                     # pickled content is refused, not run
        usw.load(obj)


def test_rejects_damaged_union_rowmap(tmp_path):
    W, mask = case(64, 128, 0.5, 6)
    perms = np.array([np.random.default_rng(t).permutation(16) for t in range(4 * 2)], dtype=np.int32)
    enc = usw.union_encode_host(W, mask, (16, 64), (2, 2), "i4", perm=perms)
    enc.rowmap = enc.rowmap.copy()
    enc.rowmap[1] = enc.rowmap[0]                       # not a permutation
    p = tmp_path / "rm.npz"
    usw.save(p, enc)
    with pytest.raises(usw.UswError):
        usw.load(p)


def test_save_takes_host_encodings_only(tmp_path):
    with pytest.raises(TypeError):
        usw.save(tmp_path / "x.npz", {"bitmaps": np.zeros(1)})
