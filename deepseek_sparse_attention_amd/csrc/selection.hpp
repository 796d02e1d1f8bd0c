// Device helpers shared by the top-k selection kernels: the order-preserving key of a
// score and the histogram search that radix selection is built on.
#pragma once

#include "common.hpp"

namespace dsa {

constexpr int kSelBins = 2048;   // histogram bins per radix pass
constexpr int kSelBinBits = 11;

// Order-preserving uint32 key of a finite score: larger scores get larger keys, and adding
// +0 first turns -0 into +0, so the two tie.  Every finite score maps to a key >= 1.
__device__ __forceinline__ uint32_t sel_key(float f) {
  const uint32_t u = __float_as_uint(f + 0.0f);
  return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}

// Top-down search of hist[0..kSelBins) by one wave: the bin holding the `need`-th largest
// count, and the count strictly above it (both wave-uniform).
__device__ __forceinline__ void wave_find_bin_from_top(const uint32_t* hist, uint32_t need, uint32_t& bin,
                                                       uint32_t& above) {
  const int lane = threadIdx.x & 63;
  constexpr int PER = kSelBins / 64;  // 32 bins per lane, lane 0 holds the top ones
  uint32_t sum = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) sum += hist[kSelBins - 1 - (lane * PER + i)];
  uint32_t total;
  const uint32_t incl = wave_incl_scan_u32(sum, &total);
  // the lane whose 32 bins hold the need-th count (exactly one: counts are cumulative)
  const uint64_t hit = __ballot(incl - sum < need && need <= incl);
  const int L = __builtin_amdgcn_readfirstlane(hit ? (int)__builtin_ctzll(hit) : 0);
  const uint32_t preL = (uint32_t)__builtin_amdgcn_readlane((int)(incl - sum), L);
  // spread that lane's bins over lanes 0..31 and scan them
  const uint32_t c = lane < PER ? hist[kSelBins - 1 - (L * PER + lane)] : 0u;
  uint32_t t2;
  const uint32_t incl2 = preL + wave_incl_scan_u32(c, &t2);
  const uint64_t hit2 = __ballot(lane < PER && incl2 - c < need && need <= incl2);
  const int i2 = hit2 ? (int)__builtin_ctzll(hit2) : 0;
  uint32_t my_bin = 0xFFFFFFFFu, my_above = 0;
  if (lane == i2) {
    my_bin = kSelBins - 1 - (L * PER + i2);
    my_above = incl2 - c;
  }
  bin = wave_min_u32(my_bin);  // exactly one lane found it
  above = wave_min_u32(my_bin == bin ? my_above : 0xFFFFFFFFu);
}

// The same search over a padded histogram: bin b at hist[sel_pad(b)] (one pad word per 32
// bins), so the 32 bins a lane sums lie in distinct LDS banks from the other lanes' (the
// unpadded layout puts every lane's i-th bin in one bank).  kSelPadBins words.
constexpr int kSelPadBins = kSelBins + kSelBins / 32;
__device__ __forceinline__ uint32_t sel_pad(uint32_t b) { return b + (b >> 5); }

// `total`, if given, receives the histogram's total count.
__device__ __forceinline__ void wave_find_bin_padded(const uint32_t* hist, uint32_t need, uint32_t& bin,
                                                     uint32_t& above, uint32_t* total_out = nullptr) {
  const int lane = threadIdx.x & 63;
  constexpr int PER = kSelBins / 64;
  uint32_t sum = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) sum += hist[sel_pad(kSelBins - 1 - (lane * PER + i))];
  uint32_t total;
  const uint32_t incl = wave_incl_scan_u32(sum, &total);
  if (total_out) *total_out = total;
  const uint64_t hit = __ballot(incl - sum < need && need <= incl);
  const int L = __builtin_amdgcn_readfirstlane(hit ? (int)__builtin_ctzll(hit) : 0);
  const uint32_t preL = (uint32_t)__builtin_amdgcn_readlane((int)(incl - sum), L);
  const uint32_t c = lane < PER ? hist[sel_pad(kSelBins - 1 - (L * PER + lane))] : 0u;
  uint32_t t2;
  const uint32_t incl2 = preL + wave_incl_scan_u32(c, &t2);
  const uint64_t hit2 = __ballot(lane < PER && incl2 - c < need && need <= incl2);
  const int i2 = hit2 ? (int)__builtin_ctzll(hit2) : 0;
  uint32_t my_bin = 0xFFFFFFFFu, my_above = 0;
  if (lane == i2) {
    my_bin = kSelBins - 1 - (L * PER + i2);
    my_above = incl2 - c;
  }
  bin = wave_min_u32(my_bin);
  above = wave_min_u32(my_bin == bin ? my_above : 0xFFFFFFFFu);
}

// Bin shift that spreads keys lo..hi over kSelBins bins.
__device__ __forceinline__ int sel_shift(uint32_t lo, uint32_t hi) {
  return hi == lo ? 0 : max(0, 32 - __clz(hi - lo) - kSelBinBits);
}

}  // namespace dsa
