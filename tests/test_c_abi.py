"""The C headers from C: a C99 program that includes include/kda.h and
include/kda_prefix_cache.h compiles with warnings as errors, links against
libkda.so and runs calls that need no GPU (checkpoint counting, workspace
sizing, host validation and its error messages, B == 0 no-ops, and the host
prefix cache)."""
import os
import shutil
import subprocess

import pytest

import linear_attention_recurrence_decode_amd as kda

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.skipif(not os.path.exists(kda.LIB_PATH) or shutil.which("gcc") is None,
                                reason="libkda.so not built or no gcc")

PROGRAM = r"""
#include <stdio.h>
#include <string.h>
#include "kda.h"
#include "kda_prefix_cache.h"

#define CHECK(c) do { if (!(c)) { printf("FAILED %s (line %d): %s\n", #c, __LINE__, kda_last_error()); return 1; } } while (0)

int main(void) {
    kda_config cfg;
    int32_t tokens[300];
    int32_t slot = -1, got[2];
    int i;
    kda_pcache* c;

    memset(&cfg, 0, sizeof cfg);
    cfg.num_heads = 4; cfg.head_k = 128; cfg.head_v = 128; cfg.conv_width = 4;
    cfg.act_dtype = KDA_BF16; cfg.l2_eps = 1e-6f; cfg.rms_eps = 1e-6f; cfg.state_dtype = KDA_F32;

    /* checkpoint positions: every multiple of 64 strictly inside (0, 300) and the end */
    CHECK(kda_num_checkpoints(0, 300, 64) == 5);
    CHECK(kda_num_checkpoints(7, 64, 64) == 2);
    CHECK(kda_prefill_workspace_bytes(&cfg, 3, 1000, 0, 0) > 0);

    /* validation on the host: nothing is launched */
    CHECK(kda_decode_step(&cfg, 0, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 1, NULL, NULL, NULL) == KDA_OK);
    CHECK(kda_decode_step(NULL, 1, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 1, NULL, NULL, NULL) == KDA_ERR_INVALID_ARG);
    CHECK(strlen(kda_last_error()) > 0);
    cfg.head_k = 96; cfg.head_v = 96;
    CHECK(kda_decode_step(&cfg, 1, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 1, NULL, NULL, NULL) == KDA_ERR_UNSUPPORTED);
    cfg.head_k = 128; cfg.head_v = 128;
    CHECK(kda_project_output(&cfg, 0, 7168, NULL, NULL, NULL, NULL) == KDA_OK);
    CHECK(kda_project_inputs(&cfg, 4, 100, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL) == KDA_ERR_INVALID_ARG);

    /* the static-workspace prefill refuses, before any device call, a call its
       buffer cannot hold (a paired ring for 256 chains) and invalid arguments */
    CHECK(kda_prefill_varlen_static(&cfg, 512, 100000, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL,
                                    NULL, NULL, 8, NULL, NULL, 0, NULL, NULL, 0, NULL, KDA_PREFILL_PAIRED, NULL,
                                    NULL) == KDA_ERR_WORKSPACE);
    CHECK(strstr(kda_last_error(), "static workspace") != NULL);
    CHECK(kda_prefill_workspace_bytes(&cfg, 512, 100000, 0, KDA_PREFILL_PAIRED) > (size_t)KDA_STATIC_WORKSPACE_BYTES);
    CHECK(kda_prefill_varlen_static(&cfg, -1, 100, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL,
                                    NULL, NULL, 8, NULL, NULL, 0, NULL, NULL, 0, NULL, 0, NULL, NULL)
          == KDA_ERR_INVALID_ARG);

    /* the host prefix cache */
    for (i = 0; i < 300; i++) tokens[i] = (i * 7919) % 1000;
    c = kda_pcache_create(4, 64, KDA_PCACHE_KEEP_ALL, 0);
    CHECK(c != NULL);
    CHECK(kda_pcache_reserve(c, 2, got) == 2);
    CHECK(kda_pcache_insert(c, tokens, 128, got[0], 0) == 1);
    CHECK(kda_pcache_insert(c, tokens, 256, got[1], 0) == 1);
    CHECK(kda_pcache_lookup(c, tokens, 300, &slot) == 0);       /* not visible before its step commits */
    kda_pcache_commit(c, 0);
    CHECK(kda_pcache_lookup(c, tokens, 300, &slot) == 256 && slot == got[1]);
    CHECK(kda_pcache_release(c, slot) == 0);
    CHECK(kda_pcache_lookup(c, tokens, 255, &slot) == 128 && slot == got[0]);
    CHECK(kda_pcache_release(c, slot) == 0);
    CHECK(kda_pcache_release(c, slot) == -1 && strlen(kda_pcache_last_error()) > 0);
    kda_pcache_destroy(c);
    printf("ok\n");
    return 0;
}
"""


def test_headers_compile_as_c99_and_link(tmp_path):
    src = tmp_path / "abi.c"
    src.write_text(PROGRAM)
    exe = tmp_path / "abi"
    libdir = os.path.dirname(kda.LIB_PATH)
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", os.path.join(ROOT, "include"),
           str(src), "-o", str(exe), "-L", libdir, "-l:" + os.path.basename(kda.LIB_PATH), "-Wl,-rpath," + libdir]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr
