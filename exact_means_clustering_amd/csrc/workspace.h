// Workspace carve-up and the per-thread error text shared by the ABI entry
// points (internal).
#pragma once

#include <stdarg.h>
#include <stdio.h>

#include "kernels.h"

namespace fkm {

inline char* err_buf() {
  static thread_local char buf[512] = "";
  return buf;
}

inline int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(err_buf(), 512, fmt, ap);
  va_end(ap);
  return code;
}

inline size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

// Byte offsets of the scratch regions inside one workspace, 256-byte aligned.
struct Layout {
  size_t chat, hb, wpad, part, cnt, kv0, kv1, hist, dtot, off, frag, gfrag, total;
};

inline Layout make_layout(int64_t N, int D, int K, int B, int dt) {
  Layout L{};
  const int64_t n = N * B;
  const int64_t nseg = (int64_t)B * K;
  size_t o = 0;
  L.chat = o;  o = al256(o + (size_t)nseg * D * dtype_size(dt));
  L.hb = o;    o = al256(o + (size_t)B * kpad(K) * 4);
  L.wpad = o;  o = al256(o + (size_t)B * kpad(K) * 4);
  L.part = o;  o = al256(o + (size_t)B * assign_max_parts(N) * 8);
  L.cnt = o;   o = al256(o + (size_t)nseg * 4);
  L.kv0 = o;   o = al256(o + (size_t)n * 8);
  L.kv1 = o;   o = al256(o + (size_t)n * 8);
  L.hist = o;  o = al256(o + (size_t)sort_hist_words(N, B, K) * 4);
  L.dtot = o;  o = al256(o + ((size_t)1 << kSortWideBits) * 4);
  L.off = o;   o = al256(o + (size_t)(nseg + 1) * 4);
  L.frag = o;  o = al256(o + (size_t)seg_chunks(n) * 2 * D * 4);
  L.gfrag = o; o = al256(o + (size_t)seg_groups(n) * 2 * D * 8);
  L.total = o;
  return L;
}

struct Work {
  void* chat;
  float* hb;
  float* wpad;
  double* part;
  int32_t* cnt;
  SortBuffers sort;
  int32_t* off;
  SegBuffers seg;
};

inline Work carve(void* ws, const Layout& L) {
  auto at = [ws](size_t off) { return static_cast<char*>(ws) + off; };
  Work w;
  w.chat = at(L.chat);
  w.hb = reinterpret_cast<float*>(at(L.hb));
  w.wpad = reinterpret_cast<float*>(at(L.wpad));
  w.part = reinterpret_cast<double*>(at(L.part));
  w.cnt = reinterpret_cast<int32_t*>(at(L.cnt));
  w.sort.kv[0] = reinterpret_cast<uint2*>(at(L.kv0));
  w.sort.kv[1] = reinterpret_cast<uint2*>(at(L.kv1));
  w.sort.hist = reinterpret_cast<uint32_t*>(at(L.hist));
  w.sort.hist_words = (int64_t)((L.dtot - L.hist) / 4);
  w.sort.dtot = reinterpret_cast<uint32_t*>(at(L.dtot));
  w.off = reinterpret_cast<int32_t*>(at(L.off));
  w.seg.frag = reinterpret_cast<float*>(at(L.frag));
  w.seg.gfrag = reinterpret_cast<double*>(at(L.gfrag));
  return w;
}

}  // namespace fkm
