"""Device calibration probes (include/ckks_probe.h) through the C interface:
every named probe returns a positive rate, the copy probe's size rule is
enforced on the host, and an unknown name is rejected."""
import pytest

from gpu_util import announce, torch_cuda

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    torch_cuda()
    import private_rns_ckks_amd as L

    return L


def test_probe_rates(lib):
    names = lib.ckks_probe_list()
    assert "copy" in names and "butterfly_ct" in names
    for name in names:
        announce("probe %s" % name)
        rate, ms = lib.ckks_probe_rate(name, copy_bytes=1 << 24)
        assert rate > 0 and ms > 0, name
    # 16 MiB read and written in the measured time
    rate, ms = lib.ckks_probe_rate("copy", copy_bytes=1 << 24)
    assert rate == pytest.approx(2 * (1 << 24) / (ms * 1e-3), rel=1e-6)


@pytest.mark.parametrize("size", [0, 2048, 4096 + 16, (1 << 20) + 2048])
def test_copy_probe_rejects_sizes(lib, size):
    announce("copy probe size %d" % size)
    with pytest.raises(lib.CKKSError) as e:
        lib.ckks_probe_rate("copy", copy_bytes=size)
    assert e.value.code == lib.CKKS_EINVAL


def test_unknown_probe(lib):
    with pytest.raises(lib.CKKSError) as e:
        lib.ckks_probe_rate("no_such_probe")
    assert e.value.code == lib.CKKS_EINVAL
