// CPU stand-in for the HIP device environment (tests only): one wave = 64 std::threads.
#pragma once
#include <cmath>
#include <cstdint>
#include <cstring>
#include <cstdio>
#include <cstdlib>
#include <algorithm>
#include <mutex>
#include <condition_variable>
#include <chrono>
#define __global__
#define __device__
#define __host__
#define __forceinline__ inline
#define __launch_bounds__(x)
typedef int hipError_t;
typedef void *hipStream_t;
#define hipSuccess 0
#define hipErrorInvalidValue 1
struct dim3 { unsigned x, y, z; dim3(unsigned a = 1, unsigned b = 1, unsigned c = 1) : x(a), y(b), z(c) {} };
extern thread_local dim3 threadIdx, blockIdx;
#define hipLaunchKernelGGL(...) (void)0
inline hipError_t hipGetLastError() { return 0; }
inline hipError_t hipOccupancyMaxActiveBlocksPerMultiprocessor(int *b, const void *, int, int) { *b = 2; return 0; }
using std::min; using std::max;
inline float __uint_as_float(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
inline uint32_t __float_as_uint(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

// ---- wave context -----------------------------------------------------------
#include <atomic>
#include <thread>
struct SimWave {
  std::atomic<int> arrived{0}; std::atomic<unsigned> gen{0}; uint64_t buf[64];
  void sync() {
    unsigned g = gen.load(std::memory_order_acquire);
    if (arrived.fetch_add(1, std::memory_order_acq_rel) == 63) {
      arrived.store(0, std::memory_order_relaxed); gen.fetch_add(1, std::memory_order_acq_rel); return;
    }
    auto t0 = std::chrono::steady_clock::now(); int spins = 0;
    while (gen.load(std::memory_order_acquire) == g) {
      if (++spins > 64) { std::this_thread::yield(); spins = 0;
        if (std::chrono::steady_clock::now() - t0 > std::chrono::seconds(10)) {
          fprintf(stderr, "DEADLOCK: cross-lane op reached by only some lanes (block %u lane %u)\n", blockIdx.x, threadIdx.x);
          abort(); } }
    }
  }
};
extern thread_local SimWave *g_wave;
inline int sim_lane() { return threadIdx.x & 63; }
template <class T> inline T sim_exchange(T v, int src) {
  uint64_t u = 0; memcpy(&u, &v, sizeof(T));
  g_wave->buf[sim_lane()] = u; g_wave->sync();
  uint64_t r = g_wave->buf[src & 63]; g_wave->sync();
  T out; memcpy(&out, &r, sizeof(T)); return out;
}
template <class T> inline T __shfl_xor(T v, int mask, int w = 64) { return sim_exchange(v, sim_lane() ^ mask); }
template <class T> inline T __shfl_up(T v, unsigned d, int w = 64) { int s = sim_lane() - (int)d; return sim_exchange(v, s < 0 ? sim_lane() : s); }
template <class T> inline T __shfl_down(T v, unsigned d, int w = 64) { int s = sim_lane() + (int)d; return sim_exchange(v, s > 63 ? sim_lane() : s); }
inline unsigned long long __ballot(int p) {
  g_wave->buf[sim_lane()] = p ? 1 : 0; g_wave->sync();
  unsigned long long r = 0; for (int i = 0; i < 64; ++i) if (g_wave->buf[i]) r |= 1ull << i;
  g_wave->sync(); return r;
}
inline int __any(int p) { return __ballot(p) != 0; }
inline int __ffsll(unsigned long long x) { return x ? __builtin_ctzll(x) + 1 : 0; }
inline int __builtin_amdgcn_readfirstlane(int v) { return sim_exchange(v, 0); }
inline int __builtin_amdgcn_readlane(int v, int l) {
  if (l < 0 || l > 63) { fprintf(stderr, "readlane index %d out of range\n", l); abort(); }
  return sim_exchange(v, l);
}
inline float __builtin_amdgcn_exp2f(float x) { return exp2f(x); }
#define __builtin_amdgcn_fence(a, b) (void)0
// a wave's lanes run in lockstep on the GPU: here they meet at a barrier, so
// LDS written by some lanes is read by the others only after every write
#define __builtin_amdgcn_wave_barrier() g_wave->sync()
// math ops whose values do not steer control flow: stubbed
#define __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, x, y, z) (c)
#define __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, x, y, z) (c)
#define __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, x, y, z) (c)
#define __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, x, y, z) (c)
#define __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, s, h) (bf16x2{(__bf16)0.f, (__bf16)0.f})
#define __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, s, h) (f16x2{(_Float16)0.f, (_Float16)0.f})
#define __builtin_amdgcn_cvt_pk_f32_fp8(w, h) (f32x2{0.f, 0.f})

// ---- shims added for the current kernels ------------------------------------
#define __builtin_amdgcn_s_waitcnt(x) (void)0
#define __builtin_amdgcn_sched_barrier(x) (void)0
struct SimPair { uint32_t v[2]; uint32_t operator[](int i) const { return v[i]; } };
inline SimPair __builtin_amdgcn_permlane16_swap(uint32_t a, uint32_t, bool, bool) {
  uint32_t o = sim_exchange(a, sim_lane() ^ 16); return SimPair{{a, o}};
}
inline SimPair __builtin_amdgcn_permlane32_swap(uint32_t a, uint32_t, bool, bool) {
  uint32_t o = sim_exchange(a, sim_lane() ^ 32); return SimPair{{a, o}};
}
// DPP moves used by the wave scan: row_shr:k (0x110 + k, k < 16) reads lane
// - k of the same 16-lane row; row_bcast:15 (0x142) and row_bcast:31 (0x143)
// read lane 15 of the previous row and lane 31.  Rows outside row_mask, and
// lanes whose source is outside the row, return `old`.
inline int __builtin_amdgcn_update_dpp(int old, int src, int ctrl, int row_mask, int, bool) {
  const int l = sim_lane(), row = l / 16;
  int from = -1;
  if (ctrl > 0x110 && ctrl < 0x120) { const int k = ctrl - 0x110; if (l % 16 >= k) from = l - k; }
  else if (ctrl == 0x142) from = row > 0 ? row * 16 - 1 : -1;
  else if (ctrl == 0x143) from = 31;
  else { fprintf(stderr, "update_dpp: control %#x not simulated\n", ctrl); abort(); }
  const int v = sim_exchange(src, from < 0 ? l : from);
  return ((row_mask >> row) & 1) && from >= 0 ? v : old;
}
// Global-to-LDS load: lane l's `size` bytes land at lds + size * l.
inline void __builtin_amdgcn_global_load_lds(const void *src, void *lds, unsigned size, int, int) {
  memcpy(static_cast<char *>(lds) + size * sim_lane(), src, size);
}
enum { hipDeviceAttributeMaxSharedMemoryPerMultiprocessor = 1, hipDeviceAttributeMaxSharedMemoryPerBlock = 2,
       hipDeviceAttributeMultiprocessorCount = 3 };
inline hipError_t hipGetDevice(int *d) { *d = 0; return 0; }
inline hipError_t hipDeviceGetAttribute(int *v, int a, int) { *v = a == 3 ? 256 : 163840; return 0; }

// E4M3 conversion (v_cvt_pk_fp8_f32: nearest even, no saturation) and the
// clamp used before it, in software
inline float __builtin_amdgcn_fmed3f(float a, float b, float c) {
  return std::max(std::min(a, std::max(b, c)), std::min(b, c));
}
inline uint32_t sim_e4m3(float x) {
  uint32_t u; memcpy(&u, &x, 4);
  const uint32_t sign = (u >> 24) & 0x80u, a = u & 0x7FFFFFFFu;
  if (a > 0x7F800000u || a >= 0x43F00000u) return sign | 0x7Fu;  // NaN, or past 480
  if (a < 0x3C800000u) { float m; memcpy(&m, &a, 4); return sign | (uint32_t)std::nearbyint(m * 512.0f); }
  uint32_t r = a >> 20; const uint32_t rest = a & 0xFFFFFu;
  if (rest > 0x80000u || (rest == 0x80000u && (r & 1u))) ++r;
  r -= (127u - 7u) << 3;
  return sign | (r > 0x7Eu ? 0x7Fu : r);
}
inline int __builtin_amdgcn_cvt_pk_fp8_f32(float a, float b, int old, bool hi) {
  const uint32_t pair = sim_e4m3(a) | (sim_e4m3(b) << 8);
  return hi ? (int)(((uint32_t)old & 0xFFFFu) | (pair << 16)) : (int)(((uint32_t)old & 0xFFFF0000u) | pair);
}

// ---- workgroup shims: one block at a time, all its waves as threads ----------
#define __shared__ static
#define __align__(n) __attribute__((aligned(n)))
struct SimBlock {
  std::mutex mu; std::condition_variable cv; int arrived = 0, total = 0; unsigned gen = 0;
  void sync() {
    std::unique_lock<std::mutex> lk(mu); unsigned g = gen;
    if (++arrived == total) { arrived = 0; ++gen; cv.notify_all(); return; }
    if (!cv.wait_for(lk, std::chrono::seconds(10), [&] { return gen != g; })) {
      fprintf(stderr, "DEADLOCK: __syncthreads reached by %d of %d threads\n", arrived, total); abort(); }
  }
};
extern SimBlock *g_block;
inline void __syncthreads() { g_block->sync(); }
