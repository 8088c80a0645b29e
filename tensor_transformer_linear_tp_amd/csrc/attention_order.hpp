// Launch order of the attention backward's key-major (dK/dV) work items.
// Plain C++ (host and device): the kernel decodes its item from the
// workgroup index, the launcher counts the items, and a host test checks the
// order against brute force.
#pragma once
#include <stdint.h>

#if defined(__HIPCC__)
#define TPS_HD __host__ __device__
#else
#define TPS_HD
#endif

namespace tps {
namespace attn_order {

constexpr int kQT = 32;          // queries per tile
constexpr int kKeyBlock = 128;   // keys per work item

struct KvItem {
  int64_t kbk;   // key block
  int chunk;     // query chunk of the block (ct tiles each, the last one shorter)
  int h;         // query head
};

// Query tiles of key block k: causal, ceil((S - 128 k) / 32) = T0 - 4 k with
// T0 = ceil(S / 32) (queries before the block see none of its keys); else T0.
TPS_HD inline int64_t tiles_of_block(int64_t S, bool causal, int64_t k) {
  const int64_t T0 = (S + kQT - 1) / kQT;
  return causal ? T0 - 4 * k : T0;
}

// Item `id` in launch order, longest first (the hardware hands workgroups out
// in index order, so the short items fill in at the end): the whole chunks of
// ct tiles, chunk-major (chunk c holds the key blocks with T(k) >= (c + 1) ct,
// a prefix of them since T(k) falls with k), then each block's last, shorter
// chunk by decreasing length v = T(k) mod ct -- when causal the blocks with a
// given v are k = (T0 - v) / 4 mod ct / 4 (every ct / 4-th block), and only
// v = T0 (mod 4) occur.  The query head varies fastest.  ct must be a multiple
// of 4.  Returns false past the last item.
TPS_HD inline bool kv_item(int64_t S, bool causal, int n_q, int ct, int64_t id, KvItem& it) {
  const int64_t T0 = (S + kQT - 1) / kQT, nkb = (S + kKeyBlock - 1) / kKeyBlock;
  for (int c = 0;; ++c) {   // whole chunks
    const int64_t need = (int64_t)(c + 1) * ct;
    const int64_t cnt = T0 < need ? 0 : causal && (T0 - need) / 4 + 1 < nkb ? (T0 - need) / 4 + 1 : nkb;
    if (cnt == 0) break;
    if (id < cnt * n_q) {
      it.kbk = id / n_q;
      it.chunk = c;
      it.h = (int)(id % n_q);
      return true;
    }
    id -= cnt * n_q;
  }
  const int per = ct / 4;   // causal: key blocks per period of T(k) mod ct
  for (int v = causal ? ct - 4 + (int)(T0 % 4) : (int)(T0 % ct); v > 0; v -= causal ? 4 : ct) {
    if (v >= ct || v > T0) continue;
    const int64_t k0 = causal ? ((T0 - v) / 4) % per : 0;
    const int64_t step = causal ? per : 1;
    const int64_t cnt = k0 < nkb ? (nkb - 1 - k0) / step + 1 : 0;
    if (id < cnt * n_q) {
      it.kbk = k0 + step * (id / n_q);
      it.chunk = (int)(tiles_of_block(S, causal, it.kbk) / ct);
      it.h = (int)(id % n_q);
      return true;
    }
    id -= cnt * n_q;
  }
  return false;
}

// Number of items of one sequence (all query heads).
inline int64_t kv_items(int64_t S, bool causal, int n_q, int ct) {
  const int64_t nkb = (S + kKeyBlock - 1) / kKeyBlock;
  int64_t n = 0;
  for (int64_t k = 0; k < nkb; ++k) n += (tiles_of_block(S, causal, k) + ct - 1) / ct;
  return n * n_q;
}

}  // namespace attn_order
}  // namespace tps
