"""Host test of the attention backward's key-major work order (csrc/attention_order.hpp):
compiled with the host C++ compiler and checked against brute force -- every (key block,
query chunk, query head) item exactly once, lengths non-increasing in launch order, and the
launcher's item count equal to the decoded one."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "tensor_transformer_linear_tp_amd", "csrc")

PROGRAM = r'''
#include <algorithm>
#include <cstdio>
#include <set>
#include <tuple>
#include "attention_order.hpp"
int main() {
  using namespace tps::attn_order;
  int bad = 0, cases = 0;
  for (int causal = 0; causal < 2; ++causal)
    for (long S : {1L, 2L, 31L, 32L, 33L, 127L, 128L, 129L, 500L, 1000L, 2047L, 2048L, 2049L, 4096L, 5000L,
                   8191L, 8192L, 8193L, 12345L, 16384L})
      for (int nq : {1, 2, 4, 8})
        for (int ct : {4, 16, 32, 64, 96, 128, 160, 192, 256}) {
          ++cases;
          const long nkb = (S + kKeyBlock - 1) / kKeyBlock;
          std::set<std::tuple<long, int, int>> want, got;
          for (long k = 0; k < nkb; ++k) {
            const long T = tiles_of_block(S, causal, k);
            for (int c = 0; c < (T + ct - 1) / ct; ++c)
              for (int h = 0; h < nq; ++h) want.insert(std::make_tuple(k, c, h));
          }
          long id = 0, last = 1L << 40;
          KvItem it;
          while (kv_item(S, causal, nq, ct, id, it)) {
            const long T = tiles_of_block(S, causal, it.kbk);
            const long len = std::min(T, (long)(it.chunk + 1) * ct) - (long)it.chunk * ct;
            if (len <= 0 || len > last || !got.insert(std::make_tuple(it.kbk, it.chunk, it.h)).second) {
              ++bad;
              std::printf("S=%ld causal=%d nq=%d ct=%d: item %ld (block %ld chunk %d head %d, %ld tiles)\n",
                          S, causal, nq, ct, id, it.kbk, it.chunk, it.h, len);
              break;
            }
            last = len;
            ++id;
          }
          if (got != want || id != kv_items(S, causal, nq, ct)) {
            ++bad;
            std::printf("S=%ld causal=%d nq=%d ct=%d: %zu items decoded, %zu expected, %ld counted\n", S, causal,
                        nq, ct, got.size(), want.size(), (long)kv_items(S, causal, nq, ct));
          }
        }
  std::printf("cases %d bad %d\n", cases, bad);
  return bad != 0;
}
'''


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs a host C++ compiler")
def test_kv_item_order_against_brute_force(tmp_path):
    src = tmp_path / "order.cpp"
    src.write_text(PROGRAM)
    exe = tmp_path / "order"
    subprocess.run(["g++", "-O1", "-std=c++17", f"-I{CSRC}", str(src), "-o", str(exe)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout[-2000:]
    assert "bad 0" in r.stdout
