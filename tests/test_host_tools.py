"""Host-side helpers of the measurement path (no GPU): kernel-name parsing of
rocprofv3 output and the source hash that ties stored HBM counters to the
kernel code they were taken on."""
from quantized_kv_cache_amd import profiling as P


def test_short_name_strips_namespaces_templates_and_parameters():
    name = ("void qkv::(anonymous namespace)::attn_decode_narrow<0, 4, 64, 128, false, 4>"
            "(qkv::AttnLaunch)")
    assert P.short_name(name) == "attn_decode_narrow"
    assert P.short_name("__amd_rocclr_copyBuffer") == "__amd_rocclr_copyBuffer"
    assert P.short_name("void qkv::(anonymous namespace)::merge_splits_small<1, 256>"
                        "(qkv::AttnLaunch)") == "merge_splits_small"


def test_code_only_ignores_comments_and_blank_lines():
    a = "int x = 1;  // one\n\n// a comment line\nint y = 2;\n"
    b = "int x = 1;\nint y = 2;   \n"
    c = "int x = 1;\nint y = 3;\n"
    assert P._code_only(a) == P._code_only(b)
    assert P._code_only(a) != P._code_only(c)


def test_every_profiled_kernel_has_sources_and_a_stable_hash():
    for k in P.KERNEL_SOURCES:
        h = P.kernel_hash(k)
        assert len(h) == 16 and h == P.kernel_hash(k)


def test_stale_counters_are_never_reported():
    """An HBM-counter summary in profiles/ counts as the kernel's traffic
    only while the kernel's sources hash as they did when it was taken; the
    benchmark reports null otherwise."""
    import glob
    import os
    import re
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    sys.path.insert(0, root)
    import bench
    files = sorted(glob.glob(os.path.join(root, "profiles", "*.counters.txt")))
    assert files
    for f in files:
        txt = open(f).read()
        kernel = re.search(r"^kernel = (\w+)$", txt, flags=re.M).group(1)
        workload = re.search(r"^workload = (\w+)$", txt, flags=re.M).group(1)
        stored = re.search(r"^kernel_source_hash = (\w+)$", txt, flags=re.M).group(1)
        t = bench.stored_traffic(kernel, workload)
        if stored == P.kernel_hash(kernel):
            assert t is not None and t > 0, os.path.basename(f)
        else:
            assert t is None, os.path.basename(f)
