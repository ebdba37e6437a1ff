"""The C ABI from C: a plain C99 program compiled against include/zsmr.h and
linked to libzsmr.so computes, through the host-only entry points, the pages'
tiny example (Psi = 8 parameters on N = 4 ranks: 128, 56, 44 and 32 bytes
per rank under data parallelism and ZeRO-1/2/3, "One Poem Suffices: ZeRO"
section 4.1; 12 and 18 elements of traffic), the owner-broadcast model's
32 bytes and 18 elements (whole units of 2 owned one per rank) with a
caller's owner map set and read back, and refuses an indivisible count and
a short owner map.  No GPU call is made."""
import os
import shutil
import subprocess

import pytest

import zero_sharded_mixed_reduce_amd as z

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")

PROGRAM = r"""
#include <stdio.h>
#include "zsmr.h"
int main(void) {
    const int64_t resident[4] = {128, 56, 44, 32};
    const int64_t traffic[4] = {12, 12, 12, 18};
    for (int32_t stage = 0; stage < 4; ++stage) {
        zsmr_ctx* c = NULL;
        zsmr_bytes b;
        if (zero_init_shards(&c, 8, 4, stage, ZSMR_FP16, ZSMR_FP16, 0, NULL, 0) != ZSMR_OK) return 2;
        if (zero_bytes_per_rank(c, 0, 0, &b) != ZSMR_OK) return 3;
        printf("stage %d resident %lld traffic %lld\n", stage, (long long)b.resident,
               (long long)b.traffic_elems);
        if (b.resident != resident[stage] || b.traffic_elems != traffic[stage]) return 4;
        zero_destroy(c);
    }
    zsmr_ctx* bad = NULL;
    if (zero_init_shards(&bad, 10, 4, 1, ZSMR_BF16, ZSMR_BF16, 0, NULL, 0) != ZSMR_ERR_INDIVISIBLE)
        return 5;
    if (bad != NULL) return 6;
    printf("%s\n", zsmr_strerror(ZSMR_ERR_INDIVISIBLE));
    /* owner broadcast: four units of two, one per rank; then the caller's map */
    const int64_t units[4] = {2, 2, 2, 2};
    zsmr_ctx* o = NULL;
    zsmr_bytes ob;
    if (zero_init_shards(&o, 8, 4, ZSMR_ZERO3_OWNER, ZSMR_BF16, ZSMR_BF16, 0, units, 4) != ZSMR_OK)
        return 7;
    if (zero_bytes_of_rank(o, 1, 0, 0, &ob) != ZSMR_OK) return 8;
    printf("owner resident %lld traffic %lld\n", (long long)ob.resident, (long long)ob.traffic_elems);
    if (ob.resident != 32 || ob.traffic_elems != 18) return 9;
    const int32_t map[4] = {3, 2, 1, 0}, short_map[3] = {0, 1, 2};
    if (zero_set_unit_owners(o, short_map, 3) != ZSMR_ERR_ARG) return 10;
    if (zero_set_unit_owners(o, map, 4) != ZSMR_OK) return 11;
    for (int32_t u = 0; u < 4; ++u) {
        int32_t who = -1;
        if (zero_unit_owner(o, u, &who) != ZSMR_OK || who != map[u]) return 12;
    }
    zero_destroy(o);
    return 0;
}
"""


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs a C compiler")
def test_a_c_program_uses_the_library(tmp_path):
    src = tmp_path / "zsmr_from_c.c"
    src.write_text(PROGRAM)
    exe = tmp_path / "zsmr_from_c"
    pkg = os.path.dirname(z.LIB_PATH)
    cmd = ["gcc", "-std=c99", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"), str(src),
           "-L", pkg, "-lzsmr", f"-Wl,-rpath,{pkg}", f"-Wl,-rpath-link,{os.path.join(ROCM, 'lib')}",
           "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "stage 3 resident 32 traffic 18" in r.stdout
    assert "owner resident 32 traffic 18" in r.stdout
