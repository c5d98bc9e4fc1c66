"""The C ABI's host-side code under AddressSanitizer (CPU only).

The library is rebuilt with AddressSanitizer on its host code (device code
is unchanged and never runs here), and a small C++ driver linked against it
calls every entry point with arguments the host checks must reject, the
pure host helpers with edge values, and the workspace-size functions; every
error message is read back.  A heap or stack overflow, a use after free or
an uninitialised read in that code makes the driver fail.  No call reaches
the device (there is none here).
"""

import concurrent.futures as cf
import os
import shutil
import subprocess
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "deepseek_v3_context_amd", "csrc")
SOURCES = ["api.hip", "split_rerange.hip", "indexer.hip", "topk.hip", "sparse_mla.hip",
           "gemm.hip"]

DRIVER = textwrap.dedent(r"""
    #include <cstdio>
    #include <cstdint>
    #include <cstring>
    #include "ds32cp.h"

    static int fails = 0;
    #define EXPECT(call, want)                                                     \
      do {                                                                         \
        const int got_ = static_cast<int>(call);                                   \
        const size_t len_ = std::strlen(ds_last_error());                          \
        if (got_ != (want)) {                                                      \
          std::printf("line %d: %s -> %d, want %d (%zu)\n", __LINE__, #call, got_, \
                      (want), len_);                                               \
          ++fails;                                                                 \
        }                                                                          \
      } while (0)

    int main() {
      void* p = reinterpret_cast<void*>(4096);   // never dereferenced: rejected first
      int32_t* ip = static_cast<int32_t*>(p);
      float* fp = static_cast<float*>(p);
      EXPECT(ds_abi_version(), 3);
      EXPECT(ds_cp_local_count(8000, 8, 3), 1000);
      EXPECT(ds_cp_local_count(5, 8, 7), 0);
      EXPECT(ds_cp_local_count(10, 0, 0), -1);
      EXPECT(ds_cp_local_count(-1, 4, 0), -1);
      EXPECT(ds_cp_local_count(int64_t(1) << 40, 2, 0), -1);
      const int32_t cu[] = {0, 8000, 8800, 8805};
      EXPECT(ds_cp_in_seq_local_count(cu, 3, 8, 0), 1101);
      EXPECT(ds_cp_in_seq_local_count(cu, 3, 8, 7), 1100);
      const int32_t bad_cu[] = {0, 5, 3};
      EXPECT(ds_cp_in_seq_local_count(bad_cu, 2, 2, 0), -1);
      EXPECT(ds_cp_in_seq_local_count(nullptr, 2, 2, 0), -1);
      EXPECT(ds_cp_in_seq_local_count(cu, 3, 8, 8), -1);
      // split, rerange, metadata
      EXPECT(cp_split_metadata(nullptr, 1, 8, 4, 0, ip, ip, ip, ip, ip, nullptr, nullptr, 0, nullptr), 1);
      EXPECT(cp_split_metadata(ip, 1, 8, 4, 4, ip, ip, ip, ip, ip, nullptr, nullptr, 0, nullptr), 1);
      EXPECT(cp_split_metadata(ip, 1, 8, 4, 0, ip, ip, ip, ip, ip, p, nullptr, 4, nullptr), 1);
      EXPECT(cp_split_metadata_in_seq(ip, 1, 8, 4, 0, 2, nullptr, ip, ip, ip, ip, nullptr, nullptr, 0, nullptr), 1);
      EXPECT(cp_split_metadata_in_seq(ip, 0, 8, 4, 0, 2, ip, ip, ip, ip, ip, nullptr, nullptr, 0, nullptr), 1);
      EXPECT(cp_split_metadata_in_seq(ip, 1, 8, 4, 0, 2, ip, ip, nullptr, ip, ip, p, p, 4, nullptr), 1);
      EXPECT(kv_rerange(nullptr, 2, 8, 4, 16, nullptr, nullptr), 1);
      EXPECT(kv_rerange(p, 1, 8, 4, 16, reinterpret_cast<void*>(1 << 20), nullptr), 1);
      EXPECT(kv_rerange(p, 2, 8, 4, 16, reinterpret_cast<char*>(p) + 32, nullptr), 1);
      EXPECT(decode_metadata(nullptr, 3, ip, ip, ip, nullptr), 1);
      EXPECT(decode_metadata(nullptr, 0, nullptr, nullptr, nullptr, nullptr), 0);
      // own-KV retention
      EXPECT(kv_cache_write(p, -1, 16, ip, ip, 1, ip, 2, 4, p, 8, nullptr), 1);
      EXPECT(kv_cache_write(p, 4, 16, ip, ip, 1, ip, 2, 0, p, 8, nullptr), 1);
      EXPECT(kv_cache_write(nullptr, 4, 16, ip, ip, 1, ip, 2, 4, p, 8, nullptr), 1);
      EXPECT(kv_cache_write(p, 4, 16, ip, ip, 1, ip, 2, 4, reinterpret_cast<char*>(p) + 16, 8, nullptr), 1);
      EXPECT(kv_cache_write_fp8(p, DS_F32, 4, 576, ip, ip, 1, ip, 2, 64, static_cast<uint8_t*>(p), fp, 8, nullptr), 2);
      EXPECT(kv_cache_write_fp8(p, DS_BF16, 4, 578, ip, ip, 1, ip, 2, 64, static_cast<uint8_t*>(p), fp, 8, nullptr), 2);
      EXPECT(kv_cache_write_fp8(p, DS_BF16, 4, 576, ip, ip, 1, ip, 2, 64, nullptr, fp, 8, nullptr), 1);
      EXPECT(kv_cache_write_fp8(reinterpret_cast<char*>(p) + 2, DS_BF16, 4, 576, ip, ip, 1, ip, 2, 64,
                                static_cast<uint8_t*>(p), fp, 8, nullptr), 1);
      // indexer and top-k
      const size_t ws = indexer_topk_workspace_size(4, 100);
      if (ws < 4 * 100 * sizeof(float)) { std::printf("indexer workspace too small\n"); ++fails; }
      (void)indexer_topk_workspace_size(256, 65536);
      (void)indexer_topk_workspace_size(0, 0);
      EXPECT(indexer_topk(p, DS_BF16, fp, p, DS_BF16, nullptr, 100, ip, ip, nullptr, nullptr, 0, 0, 0,
                          4, 32, 128, 100, 16, ip, nullptr, p, ws, nullptr), 2);
      EXPECT(indexer_topk(p, DS_BF16, fp, p, DS_FP8_E4M3FN, nullptr, 100, ip, ip, nullptr, nullptr, 0, 0, 0,
                          4, 64, 128, 100, 16, ip, nullptr, p, ws, nullptr), 1);
      EXPECT(indexer_topk(p, DS_BF16, fp, p, DS_FP8_E4M3FN_ROWSCALE, fp, 100, ip, ip, nullptr, nullptr, 0, 0, 0,
                          4, 64, 128, 100, 16, ip, nullptr, p, ws, nullptr), 2);
      EXPECT(indexer_topk(p, DS_BF16, fp, p, DS_BF16, nullptr, 100, ip, ip, nullptr, nullptr, 0, 0, 0,
                          4, 64, 128, 100, 4096, ip, nullptr, p, ws, nullptr), 1);
      EXPECT(indexer_topk(p, DS_BF16, fp, p, DS_BF16, nullptr, 100, ip, ip, nullptr, nullptr, 0, 0, 0,
                          4, 64, 128, 100, 16, ip, nullptr, p, ws - 1, nullptr), 3);
      EXPECT(indexer_scores(p, DS_BF16, fp, p, DS_BF16, nullptr, 100, ip, ip, nullptr, nullptr, 0, 0, 0,
                            4, 64, 128, 100, fp, 50, nullptr), 1);
      EXPECT(topk_select(fp, 50, ip, ip, nullptr, nullptr, 0, 0, 0, 100, 4, 100, 16, ip, nullptr, nullptr), 1);
      EXPECT(topk_select(fp, 100, ip, ip, ip, ip, 0, 0, 0, 100, 4, 100, 16, ip, nullptr, nullptr), 1);
      // sparse MLA
      EXPECT(sparse_mla_prefill(p, DS_BF16, p, DS_BF16, nullptr, 100, ip, 4, 96, 512, 64, 64, 0.1f, p,
                                DS_BF16, nullptr, nullptr, 0, nullptr), 2);
      EXPECT(sparse_mla_prefill(p, DS_BF16, p, DS_BF16, nullptr, 100, ip, 4, 128, 512, 64, 64, -1.f, p,
                                DS_BF16, nullptr, nullptr, 0, nullptr), 1);
      const size_t wneed = sparse_mla_prefill_workspace_size(100, DS_FP8_E4M3FN_ROWSCALE);
      if (wneed != 100 * 1152) { std::printf("fp8 prefill workspace %zu\n", wneed); ++fails; }
      EXPECT(sparse_mla_prefill(p, DS_BF16, p, DS_FP8_E4M3FN, fp, 100, ip, 4, 128, 512, 64, 64, 0.1f, p,
                                DS_BF16, nullptr, p, wneed - 1, nullptr), 3);
      const size_t dneed = sparse_mla_workspace_size(32, 128, 512, 2048);
      EXPECT(sparse_mla_decode(p, DS_BF16, p, DS_BF16, nullptr, 100, ip, 32, 128, 512, 64, 2048, 0.1f, p,
                               DS_BF16, nullptr, p, dneed - 1, nullptr), 3);
      EXPECT(sparse_mla_decode_noalloc(p, DS_BF16, p, DS_BF16, nullptr, 100, ip, 4, 96, 512, 64, 64, 0.1f,
                                       p, DS_BF16, nullptr, nullptr), 2);
      if (sparse_mla_decode_noalloc_scratch_bytes() != (size_t(32) << 20)) { std::printf("scratch\n"); ++fails; }
      // projections
      EXPECT(gemm_bf16_nt(p, 64, 0, p, 64, 0, p, DS_BF16, 128, 0, 10, 128, 60, 1, nullptr, 0, nullptr), 2);
      EXPECT(gemm_bf16_nt(p, 64, 0, p, 64, 0, p, DS_BF16, 100, 0, 10, 100, 64, 1, nullptr, 0, nullptr), 2);
      EXPECT(gemm_bf16_nt(p, 32, 0, p, 64, 0, p, DS_BF16, 128, 0, 10, 128, 64, 1, nullptr, 0, nullptr), 1);
      EXPECT(gemm_bf16_nt(nullptr, 64, 0, p, 64, 0, p, DS_BF16, 128, 0, 10, 128, 64, 1, nullptr, 0, nullptr), 1);
      EXPECT(gemm_bf16_nt(reinterpret_cast<char*>(p) + 2, 64, 0, p, 64, 0, p, DS_BF16, 128, 0, 10, 128, 64,
                          1, nullptr, 0, nullptr), 1);
      const size_t gneed = gemm_bf16_nt_workspace_size(64, 128, 7168, 1);
      if (gneed > 0)
        EXPECT(gemm_bf16_nt(p, 7168, 0, p, 7168, 0, p, DS_BF16, 128, 0, 64, 128, 7168, 1, nullptr, 0,
                            nullptr), 3);
      EXPECT(gemm_bf16_nt(p, 64, 0, p, 64, 0, p, DS_BF16, 128, 0, 0, 128, 64, 1, nullptr, 0, nullptr), 0);
      std::printf(fails ? "FAILED %d\n" : "ALL OK\n", fails);
      return fails ? 1 : 0;
    }
""")


def _tool(path, name):
    exe = path if os.path.exists(path) else shutil.which(name)
    if not exe:
        pytest.skip(f"{name} not available")
    return exe


def test_c_abi_host_code_under_address_sanitizer(tmp_path):
    hipcc = _tool("/opt/rocm/bin/hipcc", "hipcc")
    clangxx = _tool("/opt/rocm/llvm/bin/clang++", "clang++")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]
    flags = ["-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-Xclang",
             "-target-feature", "-Xclang", "-packed-fp32-ops", f"-I{ROOT}/include", f"-I{CSRC}"]

    def compile_one(src):
        obj = str(tmp_path / (src + ".o"))
        r = subprocess.run([hipcc, *flags, *san, "-c", os.path.join(CSRC, src), "-o", obj],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        return obj

    with cf.ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    lib = str(tmp_path / "libds32cp_asan.so")
    r = subprocess.run([hipcc, "--offload-arch=gfx950", "-shared", *san[:2], "-o", lib, *objs],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    drv_src = tmp_path / "driver.cpp"
    drv_src.write_text(DRIVER)
    drv = str(tmp_path / "driver")
    r = subprocess.run([clangxx, "-fsanitize=address", "-g", "-std=c++17", "-D__HIP_PLATFORM_AMD__",
                        f"-I{ROOT}/include", "-I/opt/rocm/include", str(drv_src), lib,
                        f"-Wl,-rpath,{tmp_path}", "-o", drv], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", HIP_VISIBLE_DEVICES="")
    r = subprocess.run([drv], capture_output=True, text=True, env=env, timeout=120)
    assert "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
    assert r.returncode == 0 and "ALL OK" in r.stdout, (r.stdout[-2000:], r.stderr[-2000:])
