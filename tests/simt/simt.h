// CPU emulation of a HIP workgroup: one std::thread per work-item, barriers for
// __syncthreads and for wave-level exchanges (shuffles, ballots). For integer kernels only.
#pragma once
#include <algorithm>
#include <atomic>
#include <barrier>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <functional>
#include <memory>
#include <thread>
#include <vector>

struct int4 { int x, y, z, w; };
inline int4 make_int4(int x, int y, int z, int w) { return int4{x, y, z, w}; }
struct Dim3 { unsigned x = 0, y = 0, z = 0; };

struct Wave {
  std::barrier<> bar{64};
  uint64_t buf[64];
};
struct Block {
  explicit Block(int nt) : bar(nt), waves(nt / 64) {}
  std::barrier<> bar;
  std::vector<Wave> waves;
  void* lds = nullptr;
};
inline thread_local Dim3 threadIdx, blockIdx;
inline Dim3 blockDim, gridDim;
inline thread_local Block* g_block = nullptr;
inline thread_local int g_lane = 0;

inline Wave& cur_wave() { return g_block->waves[threadIdx.x / 64]; }
inline void __syncthreads() { g_block->bar.arrive_and_wait(); }
inline int __lane_id() { return g_lane; }
template <class T> inline uint64_t to_u64(T v) { uint64_t u = 0; std::memcpy(&u, &v, sizeof(T)); return u; }
template <class T> inline T from_u64(uint64_t u) { T v; std::memcpy(&v, &u, sizeof(T)); return v; }
template <class T> inline T wave_get(T v, int src) {
  Wave& W = cur_wave();
  W.buf[g_lane] = to_u64(v);
  W.bar.arrive_and_wait();
  const T r = (src >= 0 && src < 64) ? from_u64<T>(W.buf[src]) : v;
  W.bar.arrive_and_wait();
  return r;
}
template <class T> inline T __shfl_up(T v, unsigned off, int = 64) {
  const int src = g_lane - (int)off;
  const T r = wave_get(v, src < 0 ? g_lane : src);
  return r;
}
template <class T> inline T __shfl(T v, int src, int = 64) { return wave_get(v, src & 63); }
template <class T> inline T __shfl_xor(T v, int m, int = 64) { return wave_get(v, (g_lane ^ m) & 63); }
inline uint64_t __ballot(int p) {
  Wave& W = cur_wave();
  W.buf[g_lane] = p ? 1 : 0;
  W.bar.arrive_and_wait();
  uint64_t m = 0;
  for (int l = 0; l < 64; ++l) m |= (W.buf[l] ? 1ull : 0ull) << l;
  W.bar.arrive_and_wait();
  return m;
}
inline int __ffsll(unsigned long long v) { return __builtin_ffsll((long long)v); }
inline int __popcll(unsigned long long v) { return __builtin_popcountll(v); }
inline int __builtin_amdgcn_readfirstlane(int v) { return wave_get(v, 0); }
template <class T> inline T atomicAdd(T* p, T v) { return std::atomic_ref<T>(*p).fetch_add(v); }
template <class T> inline T atomicMin(T* p, T v) {
  std::atomic_ref<T> a(*p);
  T cur = a.load();
  while (v < cur && !a.compare_exchange_weak(cur, v)) {}
  return cur;
}
inline int min(int a, int b) { return a < b ? a : b; }
inline int max(int a, int b) { return a > b ? a : b; }
inline int64_t min(int64_t a, int64_t b) { return a < b ? a : b; }
inline int64_t max(int64_t a, int64_t b) { return a > b ? a : b; }

// Runs fn() as a grid of `grid` workgroups of `nt` work-items, one workgroup at a time, each
// with `lds_bytes` of (heap) LDS.
inline void launch(unsigned grid, int nt, size_t lds_bytes, const std::function<void()>& fn) {
  gridDim.x = grid;
  blockDim.x = nt;
  for (unsigned b = 0; b < grid; ++b) {
    auto blk = std::make_unique<Block>(nt);
    std::vector<unsigned char> lds_mem(lds_bytes ? lds_bytes : 1, 0xA5);
    blk->lds = lds_bytes ? lds_mem.data() : nullptr;
    std::vector<std::thread> th;
    th.reserve(nt);
    for (int t = 0; t < nt; ++t)
      th.emplace_back([&, t, b] {
        threadIdx.x = t;
        blockIdx.x = b;
        g_block = blk.get();
        g_lane = t & 63;
        fn();
      });
    for (auto& x : th) x.join();
  }
}
