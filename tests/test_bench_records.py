"""Host checks of bench.py's bookkeeping (no GPU): the HBM-traffic figures it
reports beside the dominant kernels must belong to the kernel sources as they
stand, so a kernel change that is not re-measured shows up here instead of
as a silent null in the bench line."""

import bench


def test_traffic_figures_match_the_current_kernel_sources():
    for (kernel, workload), (nbytes, digest) in bench.MEASURED_TRAFFIC.items():
        assert bench._sources_sha1(kernel) == digest, (kernel, workload)
        assert bench.measured_traffic(kernel, workload) == nbytes


def test_headline_kernels_have_traffic_figures():
    # the dominant kernel of the long-cartridge step and of the decode step
    assert bench.measured_traffic("attn_bwd", "long-cartridge-28l") is not None
    assert bench.measured_traffic("decode", "serving-decode") is not None
