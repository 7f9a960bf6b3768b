// Block-wide radix selection over keys that each thread enumerates (shared by
// the short-row top-k and the sharded top-k merge).
//
// Every thread of an NT-thread workgroup enumerates its keys through
// each(f), which calls f(key) for each of them (0 = empty slot).
// radix_kth finds the digit prefix of the rho-th largest nonzero key: digits
// of 8 bits, starting right below the bits that every nonzero key shares
// (their maximum and minimum agree there), and stopping early once the bin
// that holds the rho-th key is taken whole.  On return, with h = hi:
//   key > threshold  iff  (key >> h) >  (prefix >> h)
//   key ~ threshold  iff  (key >> h) == (prefix >> h)
// and the rho largest keys are every key above the threshold plus rho_eq of
// the keys at it (all of them when the loop stopped early; otherwise they are
// equal keys and the caller picks which, e.g. the lower indices).
//
// The histogram is split into eight copies (lane & 7 picks one, copies 257
// words apart so that equal digits of one instruction land in different LDS
// banks): keys that share leading digits -- scores of one binade -- would
// otherwise serialise up to 64 atomic adds on one address.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

constexpr int kHistCopies = 8;
constexpr int kHistStride = 257;

template <typename KeyT, int NT>
struct RadixLds {
  uint32_t hist[kHistCopies * kHistStride];
  uint32_t wsum[NT / 64];
  KeyT wmax[NT / 64];
  KeyT wmin[NT / 64];
  KeyT prefix;
  int rho;
  int done;
};

template <typename KeyT>
__device__ __forceinline__ KeyT shr_sat(KeyT v, int s) {
  return s >= (int)(8 * sizeof(KeyT)) ? (KeyT)0 : (KeyT)(v >> s);
}


// Inclusive wave prefix sum on DPP lane moves: shifts by 1, 2, 4, 8 within
// 16-lane rows, then lane 15 of each row into the next rows (row_bcast:15 for
// rows 1 and 3, row_bcast:31 for rows 2 and 3).
__device__ __forceinline__ uint32_t wave_incl_scan32(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, false);  // row_shr:8
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false);  // row_bcast:15
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return v;
}

// The value of lane (lane ^ m), m in {1, 2, 4, 8, 16, 32}, by DPP moves and
// lane swaps (no LDS permute): quad permutations for 1 and 2; a quad reversal
// (xor 3) then a half-row mirror (xor 7) for 4; a row rotation by 8 for 8;
// row / half swaps for 16 and 32.
__device__ __forceinline__ uint32_t lane_xor(uint32_t v, int m) {
  switch (m) {
    case 1: return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xf, 0xf, false);  // quad_perm 1,0,3,2
    case 2: return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xf, 0xf, false);  // quad_perm 2,3,0,1
    case 4: {
      const int x3 = __builtin_amdgcn_mov_dpp((int)v, 0x1B, 0xf, 0xf, false);          // quad_perm 3,2,1,0
      return (uint32_t)__builtin_amdgcn_mov_dpp(x3, 0x141, 0xf, 0xf, false);             // row_half_mirror
    }
    case 8: return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x128, 0xf, 0xf, false);  // row_ror:8
    case 16: {
      const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
      return ((threadIdx.x >> 4) & 1) ? r[0] : r[1];
    }
    default: {
      const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
      return ((threadIdx.x >> 5) & 1) ? r[0] : r[1];
    }
  }
}

template <typename KeyT>
__device__ __forceinline__ KeyT lane_xor_key(KeyT v, int m) {
  if constexpr (sizeof(KeyT) == 8) {
    const uint32_t lo = lane_xor((uint32_t)v, m), hi = lane_xor((uint32_t)(v >> 32), m);
    return ((KeyT)hi << 32) | lo;
  } else {
    return lane_xor(v, m);
  }
}

template <typename KeyT>
__device__ __forceinline__ KeyT wave_max_key(KeyT v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const KeyT o = lane_xor_key<KeyT>(v, m);
    v = o > v ? o : v;
  }
  return v;
}

template <typename KeyT, int NT, class Each>
__device__ void radix_kth(Each each, int rho, RadixLds<KeyT, NT>& L, KeyT& prefix_out, int& hi_out, int& rho_out) {
  constexpr int kBits = 8 * sizeof(KeyT);
  constexpr int kWaves = NT / 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // the bits every nonzero key shares
  KeyT mx = 0, mn = (KeyT)~(KeyT)0;
  each([&](KeyT k) {
    if (k != 0) {
      mx = k > mx ? k : mx;
      mn = k < mn ? k : mn;
    }
  });
  mx = wave_max_key<KeyT>(mx);
  mn = (KeyT)~wave_max_key<KeyT>((KeyT)~mn);
  // the histogram starts cleared; each pass's bin owners clear it again
  for (int b = tid; b < kHistCopies * kHistStride; b += NT) L.hist[b] = 0;
  if (lane == 0) {
    L.wmax[wave] = mx;
    L.wmin[wave] = mn;
  }
  __syncthreads();
  mx = L.wmax[0];
  mn = L.wmin[0];
  for (int w = 1; w < kWaves; ++w) {
    mx = L.wmax[w] > mx ? L.wmax[w] : mx;
    mn = L.wmin[w] < mn ? L.wmin[w] : mn;
  }
  const KeyT dif = mx ^ mn;
  int hi = 0;
  if (dif) hi = kBits - (sizeof(KeyT) == 8 ? __clzll((long long)dif) : __clz((int)dif));
  KeyT prefix = hi >= kBits ? (KeyT)0 : (KeyT)(shr_sat<KeyT>(mx, hi) << hi);
  for (;;) {
    const int lo = hi > 8 ? hi - 8 : 0;
    const uint32_t dmask = (1u << (hi - lo)) - 1u;
    uint32_t* mine = L.hist + (lane & (kHistCopies - 1)) * kHistStride;
    const KeyT top = shr_sat<KeyT>(prefix, hi);
    each([&](KeyT k) {
      if (k != 0 && shr_sat<KeyT>(k, hi) == top) atomicAdd(&mine[(uint32_t)(k >> lo) & dmask], 1u);
    });
    __syncthreads();
    // bins in descending order: thread j < 256 owns bin 255 - j
    uint32_t h = 0;
    if (tid < 256) {
#pragma unroll
      for (int c = 0; c < kHistCopies; ++c) {
        h += L.hist[c * kHistStride + 255 - tid];
        L.hist[c * kHistStride + 255 - tid] = 0;  // ready for the next pass
      }
    }
    uint32_t incl = wave_incl_scan32(h);
    if (lane == 63) L.wsum[wave] = incl;
    __syncthreads();
    if (tid < 256) {
      for (int w = 0; w < wave; ++w) incl += L.wsum[w];
      const uint32_t above = incl - h;
      if (above < (uint32_t)rho && incl >= (uint32_t)rho) {
        const int r2 = rho - (int)above;
        L.prefix = prefix | (KeyT)((KeyT)(255 - tid) << lo);
        L.rho = r2;
        L.done = (int)h == r2;
      }
    }
    __syncthreads();
    prefix = L.prefix;
    rho = L.rho;
    hi = lo;
    if (L.done || lo == 0) break;
  }
  prefix_out = prefix;
  hi_out = hi;
  rho_out = rho;
}

}  // namespace dsa
