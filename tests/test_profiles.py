"""The committed rocprofv3 summaries under profiles/ describe the committed
kernels: each records the sha256 prefix of the kernel sources it was taken
on (bench.py's kernel_source_hash()), and bench.py's roofline fields use a
summary only when that prefix matches. A kernel change without new
profiles fails here."""
import os
import re

import bench

PROFILES = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "profiles")


def test_every_profile_names_the_current_kernel_sources():
    want = bench.kernel_source_hash()
    names = sorted(os.listdir(PROFILES))
    assert names
    stale = []
    for n in names:
        text = open(os.path.join(PROFILES, n)).read()
        found = re.findall(r"(?:Kernel sources sha256\[:16\]: |kernel_source_sha256_16: )(\w+)",
                           text)
        assert found, f"{n}: no kernel source hash recorded"
        if any(h != want for h in found):
            stale.append(n)
    assert not stale, f"profiles taken on other kernel sources than {want}: {stale}"


def test_headline_counters_and_stats_are_found_by_the_benchmark():
    wl = "ep8_t4096_h7168_bf16_k8"
    assert bench.read_traffic(wl, "ep_copy_kernel") is not None
    assert bench.read_traffic(wl, "ep_combine_kernel") is not None
    got = bench.rocprof_frac(wl, bench.COUNTER_KERNELS["ep_copy_kernel"], 2975055424)
    assert got is not None and got["average_us"] > 0
