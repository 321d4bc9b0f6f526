"""The boundary from C: a plain C program, built with gcc against
include/qgemv.h and linked to libqgemv.so (no Python, no torch), calls the
host entry points -- size queries, the reference quantizer, the tern3 and
bin8 packers, validation errors -- and its outputs must equal the Python
binding's byte for byte.  CPU only (no device call)."""
import os
import shutil
import subprocess

import numpy as np
import pytest

import block_quantized_decode_qgemv_amd as qg
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

C_SOURCE = r"""
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
#include "qgemv.h"

static int dump(const char* path, const void* p, size_t n) {
    FILE* f = fopen(path, "wb");
    if (!f) return 1;
    size_t w = fwrite(p, 1, n, f);
    fclose(f);
    return w != n;
}

static void* slurp(const char* path, size_t n) {
    FILE* f = fopen(path, "rb");
    if (!f) return NULL;
    void* p = malloc(n);
    if (p && fread(p, 1, n, f) != n) { free(p); p = NULL; }
    fclose(f);
    return p;
}

int main(int argc, char** argv) {
    if (argc != 2) return 2;
    const char* dir = argv[1];
    char path[4096];
    const int64_t N = 37, K = 1024;
    /* sizes */
    printf("size q4_k %zu\n", qg_packed_size(QG_Q4_K, N, K));
    printf("size tern3 %zu\n", qg_packed_size(QG_TERN3, N, K));
    printf("codes bin8 %zu\n", qg_codes_plane_size(QG_BIN8, N, K));
    printf("block tern3 %d\n", qg_block_size(QG_TERN3));
    /* the reference quantizer on the weights the test wrote */
    snprintf(path, sizeof path, "%s/w.f32", dir);
    float* w = (float*)slurp(path, (size_t)(N * K * 4));
    if (!w) return 3;
    size_t qs = qg_packed_size(QG_Q4_K, N, K);
    void* q = malloc(qs);
    if (qquant(QG_Q4_K, w, N, K, q, 2) != QG_OK) return 4;
    snprintf(path, sizeof path, "%s/q4k.bin", dir);
    if (dump(path, q, qs)) return 5;
    /* tern3 and bin8 packers */
    snprintf(path, sizeof path, "%s/t.i8", dir);
    int8_t* t = (int8_t*)slurp(path, (size_t)(N * K));
    snprintf(path, sizeof path, "%s/s64.u16", dir);
    uint16_t* s64 = (uint16_t*)slurp(path, (size_t)(N * (K / 64) * 2));
    snprintf(path, sizeof path, "%s/b.u8", dir);
    uint8_t* b = (uint8_t*)slurp(path, (size_t)(N * K));
    snprintf(path, sizeof path, "%s/s128.u16", dir);
    uint16_t* s128 = (uint16_t*)slurp(path, (size_t)(N * (K / 128) * 2));
    if (!t || !s64 || !b || !s128) return 6;
    size_t ts = qg_packed_size(QG_TERN3, N, K), bs = qg_packed_size(QG_BIN8, N, K);
    void* tp = malloc(ts);
    void* bp = malloc(bs);
    if (qpack_tern3(t, s64, N, K, tp) != QG_OK) return 7;
    if (qpack_bin8(b, s128, N, K, bp) != QG_OK) return 8;
    snprintf(path, sizeof path, "%s/tern3.bin", dir);
    if (dump(path, tp, ts)) return 9;
    snprintf(path, sizeof path, "%s/bin8.bin", dir);
    if (dump(path, bp, bs)) return 10;
    /* errors come back as codes with a message, and nothing is written: a bad
       code in the last row leaves every byte of the output as it was */
    t[N * K - 1] = 2;
    memset(tp, 0xAB, ts);
    int rc = qpack_tern3(t, s64, N, K, tp);
    int untouched = 1;
    for (size_t i = 0; i < ts; ++i) untouched &= ((unsigned char*)tp)[i] == 0xAB;
    printf("bad code rc %d msg %s untouched %d\n", rc, qg_last_error(), untouched);
    printf("bad shape rc %d\n", qquant(QG_Q4_K, w, N, 100, q, 1));
    printf("strerror %s\n", qg_strerror(QG_ESHAPE));
    free(w); free(q); free(t); free(s64); free(b); free(s128); free(tp); free(bp);
    return 0;
}
"""


@pytest.fixture(scope="module")
def client(tmp_path_factory):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no C compiler")
    lib = qg.lib_path()
    if not os.path.exists(lib):
        pytest.skip("library not built")
    d = tmp_path_factory.mktemp("cabi")
    src = d / "client.c"
    src.write_text(C_SOURCE)
    exe = d / "client"
    subprocess.run([gcc, "-std=c99", "-Wall", "-Werror", "-O1", "-I", os.path.join(ROOT, "include"), str(src),
                    "-o", str(exe), lib, f"-Wl,-rpath,{os.path.dirname(lib)}"], check=True, capture_output=True)
    return d, exe


def test_c_client_matches_binding(client):
    d, exe = client
    n, k = 37, 1024
    w = workloads.student_t_weights(n, k, seed=61)
    t = workloads.ternary_codes(n, k, seed=62)
    s64 = workloads.scale_bits_f16((n, k // 64), seed=63)
    b = workloads.binary_codes(n, k, seed=64)
    s128 = workloads.scale_bits_f16((n, k // 128), seed=65)
    w.tofile(d / "w.f32")
    t.astype(np.int8).tofile(d / "t.i8")
    s64.tofile(d / "s64.u16")
    b.astype(np.uint8).tofile(d / "b.u8")
    s128.tofile(d / "s128.u16")
    out = subprocess.run([str(exe), str(d)], check=True, capture_output=True, text=True, timeout=120).stdout
    assert f"q4_k {qg.qg_packed_size('q4_k', n, k)}" in out
    assert f"tern3 {qg.qg_packed_size('tern3', n, k)}" in out
    assert f"codes bin8 {qg.qg_codes_plane_size('bin8', n, k)}" in out
    assert f"block tern3 {qg.qg_block_size('tern3')}" in out
    np.testing.assert_array_equal(np.fromfile(d / "q4k.bin", np.uint8), qg.qquant("q4_k", w, n_threads=2))
    np.testing.assert_array_equal(np.fromfile(d / "tern3.bin", np.uint8), qg.qpack_tern3(t, s64))
    np.testing.assert_array_equal(np.fromfile(d / "bin8.bin", np.uint8), qg.qpack_bin8(b, s128))
    assert "bad code rc -1" in out and "untouched 1" in out and f"({n - 1}, {k - 1})" in out
    assert "bad shape rc -2" in out
    assert "strerror invalid shape" in out
