// Device-side helpers shared by the gfx950 kernels of the DSA library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// Position of a query row: sequence b holds L keys (kv_len clamped to [0, Tk]); row i of
// the Tq rows sits at L - Tq + i.
__device__ __forceinline__ int64_t seq_len(const int32_t* kv_len, int b, int Tk) {
  if (!kv_len) return Tk;
  int L = kv_len[b];
  return L < 0 ? 0 : (L > Tk ? Tk : L);
}

// Index of the calling wave in its workgroup, as a wave-uniform (scalar) value.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)); }

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t h) {
  return __uint_as_float(((uint32_t)h) << 16);
}

// fp32 -> bf16 bits, round to nearest even (inputs here are finite).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16_bits(lo) | ((uint32_t)f32_to_bf16_bits(hi) << 16);
}

// Raw buffer resource over [base, base + bytes): loads at offsets past `bytes` return 0
// instead of touching memory (hardware range check), so edge tiles need no clamping.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
// voff: per-lane byte offset (one VGPR); soff: wave-uniform byte offset (SGPR).
__device__ __forceinline__ float buf_load_f32(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, (int)soff, 0));
}

__device__ __forceinline__ u32x4 buf_load_16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0));
}

__device__ __forceinline__ void buf_store_f32(float v, __amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, (int)voff, (int)soff, 0);
}
// A byte offset no buffer range reaches (ranges here stay below 2 GiB): the store is dropped.
constexpr uint32_t kOffNone = 0x80000000u;

// The same buffer resource as its four descriptor words (base address, stride 0, range,
// the flags make_rsrc passes), for stores written as single instructions below.
__device__ __forceinline__ u32x4 rsrc_words(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return u32x4{(uint32_t)a, (uint32_t)(a >> 32) & 0xFFFFu, bytes, 0x00020000u};
}
// Exactly one vector-memory store instruction each: written in assembly, so the compiler
// can neither merge nor drop them.  Loops whose explicit `s_waitcnt vmcnt` waits count the
// stores issued between loads use these (a store outside the range is dropped by the
// hardware, like the buffer stores above).
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void buf_store1_b32(uint32_t v, u32x4 rs, uint32_t voff) {
  asm volatile("buffer_store_dword %0, %1, %2, 0 offen" ::"v"(v), "v"(voff), "s"(rs) : "memory");
}
__device__ __forceinline__ void buf_store1_b64(u32x2 v, u32x4 rs, uint32_t voff) {
  asm volatile("buffer_store_dwordx2 %0, %1, %2, 0 offen" ::"v"(v), "v"(voff), "s"(rs) : "memory");
}
__device__ __forceinline__ void buf_store1_b128(u32x4 v, u32x4 rs, uint32_t voff) {
  asm volatile("buffer_store_dwordx4 %0, %1, %2, 0 offen" ::"v"(v), "v"(voff), "s"(rs) : "memory");
}

// 16-byte global load / store helpers.
__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// MFMA wrappers (gfx950).  Operand layouts (verified on the device):
//  16x16x32: A lane l = row l%16, k = (l/16)*8 + e; B lane l = col l%16, same k;
//            D lane l = col l%16, rows 4*(l/16) + i.
//  32x32x16: A lane l = row l%32, k = (l/32)*8 + e; B lane l = col l%32, same k;
//            D lane l = col l%32, rows 8*(i/4) + 4*(l/32) + i%4.
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// LDS transposed read of 16-bit elements: within each group of 16 lanes, lane i receives
// element j = R[4j + i/4][i%4], where R[r] are the four 16-bit values at lane r's address.
__device__ __forceinline__ i16x4 lds_read_tr16(const void* lds_ptr) {
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(lds_ptr));
}

// ---- DPP (data-parallel primitives) on GFX9: lane permutations inside 16-lane rows,
// executed by the VALU without an LDS round trip.
constexpr int kDppQuadXor1 = 0xB1;  // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;  // quad_perm [2,3,0,1]
constexpr int kDppRowShr1 = 0x111, kDppRowShr2 = 0x112, kDppRowShr4 = 0x114, kDppRowShr8 = 0x118;
constexpr int kDppRowRor4 = 0x124, kDppRowRor8 = 0x128;

template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {  // lanes without a source read 0
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}

// Wave-wide min / max / sum of a uint32, returned as a wave-uniform value.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp<kDppQuadXor1>(v));
  v = max(v, dpp<kDppQuadXor2>(v));
  v = max(v, dpp<kDppRowRor4>(v));
  v = max(v, dpp<kDppRowRor8>(v));
  return max(max((uint32_t)__builtin_amdgcn_readlane((int)v, 0), (uint32_t)__builtin_amdgcn_readlane((int)v, 16)),
             max((uint32_t)__builtin_amdgcn_readlane((int)v, 32), (uint32_t)__builtin_amdgcn_readlane((int)v, 48)));
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) { return ~wave_max_u32(~v); }
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
  v += dpp<kDppQuadXor1>(v);
  v += dpp<kDppQuadXor2>(v);
  v += dpp<kDppRowRor4>(v);
  v += dpp<kDppRowRor8>(v);
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 0) + (uint32_t)__builtin_amdgcn_readlane((int)v, 16) +
         (uint32_t)__builtin_amdgcn_readlane((int)v, 32) + (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
}
// Inclusive prefix sum over the 64 lanes (lane order); *total gets the wave's sum.
__device__ __forceinline__ uint32_t wave_incl_scan_u32(uint32_t v, uint32_t* total) {
  const int lane = threadIdx.x & 63;
  v += dpp<kDppRowShr1>(v);
  v += dpp<kDppRowShr2>(v);
  v += dpp<kDppRowShr4>(v);
  v += dpp<kDppRowShr8>(v);  // inclusive scan inside each 16-lane row
  const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)v, 15);
  const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)v, 31);
  const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)v, 47);
  const uint32_t r3 = (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
  v += (lane >= 16 ? r0 : 0u) + (lane >= 32 ? r1 : 0u) + (lane >= 48 ? r2 : 0u);
  *total = r0 + r1 + r2 + r3;
  return v;
}

// Reductions across the four 16-lane rows of a wave for lanes with the same lane % 16,
// with the gfx950 lane-swap instructions (VALU, no LDS round trip):
// permlane16_swap(x, x) yields rows {r0,r0,r2,r2} and {r1,r1,r3,r3};
// permlane32_swap(x, x) yields halves {lo,lo} and {hi,hi}.
__device__ __forceinline__ float rows_max(float v) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(c[0]), __uint_as_float(c[1]));
}
__device__ __forceinline__ float rows_sum(float v) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);  // (row 2i) + (row 2i+1), same order in both
  auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(c[0]) + __uint_as_float(c[1]);
}

// fp32 -> bf16 pair with the hardware conversion (round to nearest even).
__device__ __forceinline__ uint32_t cvt_bf16x2(float lo, float hi) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));  // one packed convert
}

// Order LDS accesses of one wave: its own earlier LDS writes are visible to its later
// LDS reads from any lane (LDS instructions of a wave complete in order).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Wave-wide reductions over the 16 lanes of a row group (lanes with equal l/16).
__device__ __forceinline__ float group16_max(float v) {
#pragma unroll
  for (int o = 8; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 16));
  return v;
}
__device__ __forceinline__ float group16_sum(float v) {
#pragma unroll
  for (int o = 8; o >= 1; o >>= 1) v += __shfl_xor(v, o, 16);
  return v;
}

// max(x, 0) as one integer max on the bit pattern: negative floats (sign bit set) are
// negative int32 and become +0.0, non-negative floats stay.  A float max would first
// canonicalize x, an extra instruction per element.  Inputs here are finite.
__device__ __forceinline__ float relu(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace dsa
