// ceiling.hip -- memory-system ceilings for the decode's access pattern, as
// measurement references next to the decode kernel (libpkvd_ceiling.so; the
// benchmark's --op stream_read / paged_gather modes load it).  Nothing here
// computes attention: the kernels only read bytes, fold them into a checksum
// (so the loads cannot be dropped) and write one word per lane.
//
//  * stream_read: NW waves each read one contiguous share of a buffer with
//    16-byte non-temporal loads, PF 1 KB wave-loads in flight.
//  * paged_gather: the decode's 16-key blocks.  A block is 16 consecutive key
//    rows of one (page, kv head) tile of K and the same rows of V (16 * D *
//    elt bytes each); the host lists every block a decode call streams (its
//    K and V byte offsets).  NW waves take equal shares of the list, PF
//    blocks in flight, each block read with 16-byte non-temporal loads into
//    registers (as the decode does), or, with LDS staging, copied into a
//    per-wave LDS ring by global_load_lds_dwordx4 and read back from LDS.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kMaxWaves = 8;   // waves per workgroup: one or two per SIMD

__device__ __forceinline__ u32x4 ld_nt(const char* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ uint32_t fold(u32x4 x) { return x.x ^ x.y ^ x.z ^ x.w; }
// acc' = rotl(acc, 1) ^ x: an order-dependent chain, so that the compiler
// consumes the loads in the order they were issued (an XOR of all loads
// could be reassociated into "issue all, wait for all")
__device__ __forceinline__ uint32_t mix(uint32_t acc, uint32_t x) {
  return ((acc << 1) | (acc >> 31)) ^ x;
}

__device__ __forceinline__ int64_t uniform64(int64_t x) {
  const uint64_t u = (uint64_t)x;
  return (int64_t)(((uint64_t)__builtin_amdgcn_readfirstlane((int)(u >> 32)) << 32) |
                   (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)u));
}

// Wave w of NW: [n * w / NW, n * (w + 1) / NW).
__device__ __forceinline__ int64_t share(int64_t n, int w, int nw) { return n * w / nw; }

template <int PF>
__global__ __launch_bounds__(64 * kMaxWaves) void stream_read(const char* src, int64_t chunks,
                                                              int nw, uint32_t* sink) {
  const int lane = threadIdx.x & 63;
  const int gw = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (gw >= nw) return;
  const int64_t c0 = share(chunks, gw, nw), c1 = share(chunks, gw + 1, nw);
  uint32_t acc = 0;
  u32x4 buf[PF];
  // chunk c is the 1 KB at src + c * 1024; chunks past c1 are clamped (re-read)
  auto at = [&](int64_t c) { return src + (c < c1 ? c : c1 - 1) * 1024 + lane * 16; };
  if (c0 < c1) {
#pragma unroll
    for (int s = 0; s < PF; ++s) buf[s] = ld_nt(at(c0 + s));
    for (int64_t c = c0; c < c1; c += PF) {
#pragma unroll
      for (int s = 0; s < PF; ++s) {
        acc = mix(acc, fold(buf[s]));
        buf[s] = ld_nt(at(c + PF + s));
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  sink[(int64_t)gw * 64 + lane] = acc;
}

// Register ring: PF blocks in flight, NL 1 KB wave-loads per block per tensor,
// in PF + 1 buffers: the loads of block i + PF go out before block i is
// consumed (the decode's ring).  As in the decode, the loads have no branch
// around them: past the wave's share they re-read its last block (which the
// caches serve), so the loop runs whole rounds of PF + 1 blocks.
template <int PF, int NL>
__global__ __launch_bounds__(64 * kMaxWaves) void gather_regs(const char* kb, const char* vb,
                                                              const int64_t* __restrict__ koff,
                                                              const int64_t* __restrict__ voff,
                                                              int64_t nblk, int nw,
                                                              uint32_t* sink) {
  constexpr int NB = PF + 1;
  const int lane = threadIdx.x & 63;
  const int gw = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (gw >= nw) return;
  const int64_t b0 = share(nblk, gw, nw), b1 = share(nblk, gw + 1, nw);
  uint32_t acc = 0;
  u32x4 bk[NB][NL], bv[NB][NL];
  auto load = [&](int s, int64_t b) {
    const int64_t bb = uniform64(b < b1 ? b : b1 - 1);   // offsets come from scalar loads
    const char* pk = kb + koff[bb] + lane * 16;
    const char* pv = vb + voff[bb] + lane * 16;
#pragma unroll
    for (int u = 0; u < NL; ++u) {
      bk[s][u] = ld_nt(pk + u * 1024);
      bv[s][u] = ld_nt(pv + u * 1024);
    }
  };
  if (b0 < b1) {
#pragma unroll
    for (int s = 0; s < PF; ++s) load(s, b0 + s);
    for (int64_t b = b0; b < b1; b += NB) {
#pragma unroll
      for (int s = 0; s < NB; ++s) {
        load((s + PF) % NB, b + s + PF);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < NL; ++u) acc = mix(mix(acc, fold(bk[s][u])), fold(bv[s][u]));
      }
    }
  }
  sink[(int64_t)gw * 64 + lane] = acc;
}

// vmcnt(n) with the other counters left alone (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vm() {
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// LDS staging: the same blocks copied into a per-wave LDS ring of PF + 1
// slots by global_load_lds_dwordx4 (each lane's 16 bytes land at the slot
// base + lane * 16), then read back with ds_read_b128.
template <int PF, int NL>
__global__ __launch_bounds__(64 * kMaxWaves) void gather_lds(const char* kb, const char* vb,
                                                          const int64_t* __restrict__ koff,
                                                          const int64_t* __restrict__ voff,
                                                          int64_t nblk,
                                                          int nw, uint32_t* sink) {
  constexpr int kSlot = 2 * NL * 1024;   // bytes of one block (K and V)
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int gw = blockIdx.x * (blockDim.x >> 6) + wv;
  if (gw >= nw) return;
  char* ring = lds + wv * (PF + 1) * kSlot;
  const int64_t b0 = share(nblk, gw, nw), b1 = share(nblk, gw + 1, nw);
  uint32_t acc = 0;
  auto issue = [&](int slot, int64_t b) {
    const int64_t bb = uniform64(b < b1 ? b : b1 - 1);   // offsets come from scalar loads
    const char* pk = kb + koff[bb] + lane * 16;
    const char* pv = vb + voff[bb] + lane * 16;
    char* dst = ring + slot * kSlot;
#pragma unroll
    for (int u = 0; u < NL; ++u) {
      __builtin_amdgcn_global_load_lds(pk + u * 1024,
                                       (__attribute__((address_space(3))) void*)(dst + u * 1024),
                                       16, 0, 0);
      __builtin_amdgcn_global_load_lds(pv + u * 1024,
                                       (__attribute__((address_space(3))) void*)(dst + (NL + u) * 1024),
                                       16, 0, 0);
    }
  };
  if (b0 < b1) {
#pragma unroll
    for (int s = 0; s < PF; ++s) issue(s, b0 + s);
    int slot = 0;
    for (int64_t b = b0; b < b1; ++b) {
      issue((slot + PF) % (PF + 1), b + PF);
      wait_vm<2 * NL * PF>();   // block b's copies have landed
      const char* src = ring + slot * kSlot + lane * 16;
#pragma unroll
      for (int u = 0; u < 2 * NL; ++u) acc = mix(acc, fold(*reinterpret_cast<const u32x4*>(src + u * 1024)));
      slot = slot == PF ? 0 : slot + 1;
    }
    wait_vm<0>();
  }
  sink[(int64_t)gw * 64 + lane] = acc;
}

using GatherFn = void (*)(const char*, const char*, const int64_t*, const int64_t*, int64_t, int,
                         uint32_t*);

template <int NL>
GatherFn gather_fn(int pf, bool lds) {
  switch (pf) {
    case 2: return lds ? &gather_lds<2, NL> : &gather_regs<2, NL>;
    case 3: return lds ? &gather_lds<3, NL> : &gather_regs<3, NL>;
    case 4: return lds ? &gather_lds<4, NL> : &gather_regs<4, NL>;
    case 6: return lds ? nullptr : &gather_regs<6, NL>;
    case 8: return lds || NL == 4 ? nullptr : &gather_regs<8, NL>;   // (8, 4) would spill
    default: return nullptr;
  }
}

}  // namespace

extern "C" {

// Version of this file's argument lists (checked by the caller before any
// launch, so that a stale build is never called with other arguments).
int pkvd_ceiling_abi(void) { return 2; }

// Reads `bytes` (a multiple of 1024) from src with nw waves, wpg waves per
// workgroup (4 or 8); sink holds nw * 64 words.  Returns a hipError_t.
int pkvd_ceiling_stream_read(const void* src, int64_t bytes, int nw, int wpg, uint32_t* sink,
                             void* stream) {
  if (bytes <= 0 || bytes % 1024 || nw < 1 || (wpg != 4 && wpg != 8)) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(stream_read<8>, dim3((nw + wpg - 1) / wpg), dim3(64 * wpg), 0,
                     static_cast<hipStream_t>(stream), static_cast<const char*>(src),
                     bytes / 1024, nw, sink);
  return (int)hipGetLastError();
}

// Reads nblk blocks of block_bytes (2048 or 4096) of K at k + koff[i] and of V
// at v + voff[i] (byte offsets, 16-byte aligned) with nw waves, wpg waves per
// workgroup (4 or 8) and pf blocks in flight per wave (2, 3, 4, 6, or 8 for
// 2 KB blocks; 2-4 with LDS staging); sink holds nw * 64 words.  lds = 1 stages the blocks
// through LDS.  Returns a hipError_t.
int pkvd_ceiling_paged_gather(const void* k, const void* v, const int64_t* koff,
                              const int64_t* voff, int64_t nblk, int block_bytes, int nw, int wpg,
                              int pf, int lds, uint32_t* sink, void* stream) {
  if (nblk <= 0 || nw < 1 || (block_bytes != 2048 && block_bytes != 4096) ||
      (wpg != 4 && wpg != 8))
    return (int)hipErrorInvalidValue;
  const int nl = block_bytes / 1024;
  GatherFn f = nl == 4 ? gather_fn<4>(pf, lds) : gather_fn<2>(pf, lds);
  if (!f) return (int)hipErrorInvalidValue;
  // LDS: a ring of pf + 1 blocks (K and V) per wave
  const size_t lds_bytes = lds ? (size_t)wpg * (pf + 1) * 2 * block_bytes : 0;
  if (lds_bytes > 160 * 1024) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(f, dim3((nw + wpg - 1) / wpg), dim3(64 * wpg), lds_bytes,
                     static_cast<hipStream_t>(stream), static_cast<const char*>(k),
                     static_cast<const char*>(v), koff, voff, nblk, nw, sink);
  return (int)hipGetLastError();
}

}  // extern "C"
