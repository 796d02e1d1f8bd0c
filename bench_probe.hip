// Measurement kernels for bench.py (not part of the DSA path): the ceilings the hot-path
// kernels are held against on this machine.
//   probe_read:   a streaming read of n16 16-byte words, a contiguous range per workgroup
//                 (the HBM read ceiling);
//   probe_gather: the gather of the sparse attention without its arithmetic: for each of
//                 `rows` index rows of k entries, the row_bytes-wide table rows the entries
//                 name (entries outside [0, table_rows) skipped), read the way the
//                 attention reads them (workgroups per index row or part of it, 32 entries
//                 per step, eight lanes per table row, four steps in flight) and folded
//                 into a checksum.  Its rate on the attention's own index rows is the ceiling of
//                 that access pattern through the caches.
// Plain C ABI; both return a hipError_t value (0 on success).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Workgroup b reads its own contiguous range of the buffer, 1 KB per wave and load, four
// loads in flight per lane, non-temporal: measured on MI355X at 6.9-7.1 TB/s for 0.5-1 GiB
// (a grid-stride pass over the whole buffer, every workgroup one 4 KB block in turn, reached
// 5.3-6.2 TB/s).
__global__ __launch_bounds__(256) void read_kernel(const u32x4* __restrict__ p, size_t n16, size_t chunk16,
                                                   uint32_t* __restrict__ out) {
  uint32_t acc = 0;
  const size_t b0 = (size_t)blockIdx.x * chunk16, b1 = b0 + chunk16 < n16 ? b0 + chunk16 : n16;
  size_t i = b0 + threadIdx.x;
  for (; i + 3 * 256 < b1; i += 4 * 256) {
    const u32x4 a = __builtin_nontemporal_load(p + i), b = __builtin_nontemporal_load(p + i + 256);
    const u32x4 c = __builtin_nontemporal_load(p + i + 512), d = __builtin_nontemporal_load(p + i + 768);
    acc ^= a[0] ^ a[1] ^ a[2] ^ a[3] ^ b[0] ^ b[1] ^ b[2] ^ b[3] ^ c[0] ^ c[1] ^ c[2] ^ c[3] ^ d[0] ^ d[1] ^ d[2] ^ d[3];
  }
  for (; i < b1; i += 256) {
    const u32x4 a = p[i];
    acc ^= a[0] ^ a[1] ^ a[2] ^ a[3];
  }
  out[(size_t)blockIdx.x * 256 + threadIdx.x] = acc;
}

template <int PARTS>  // 16-byte parts per lane (row_bytes / 128, rounded up)
__global__ __launch_bounds__(256) void gather_kernel(const uint8_t* __restrict__ table, int row_bytes,
                                                     int64_t table_rows, const int32_t* __restrict__ idx, int k,
                                                     int per, uint32_t* __restrict__ out) {
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x;
  const int key = tid >> 3, part = tid & 7;  // entry of the step, first 16-byte part
  const int32_t* ix = idx + row * k;
  const int j0 = blockIdx.y * per, j1 = min(k, j0 + per);
  uint32_t acc = 0;
  auto load = [&](int j, u32x4 (&r)[PARTS]) {
    const int s = j < j1 ? ix[j] : -1;
    const bool ok = s >= 0 && s < table_rows;
    const uint8_t* base = table + (ok ? (int64_t)s * row_bytes : 0);
#pragma unroll
    for (int c = 0; c < PARTS; ++c) {
      const int off = (part + 8 * c) * 16;
      r[c] = (ok && off < row_bytes) ? *reinterpret_cast<const u32x4*>(base + off) : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto fold = [&](const u32x4 (&r)[PARTS]) {
#pragma unroll
    for (int c = 0; c < PARTS; ++c) acc ^= r[c][0] ^ r[c][1] ^ r[c][2] ^ r[c][3];
  };
  // four steps of 32 entries in flight
  u32x4 r0[PARTS], r1[PARTS], r2[PARTS], r3[PARTS];
  load(j0 + key, r0);
  load(j0 + 32 + key, r1);
  load(j0 + 64 + key, r2);
  load(j0 + 96 + key, r3);
  for (int j = j0; j < j1; j += 128) {
    fold(r0);
    load(j + 128 + key, r0);
    fold(r1);
    load(j + 160 + key, r1);
    fold(r2);
    load(j + 192 + key, r2);
    fold(r3);
    load(j + 224 + key, r3);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) acc ^= __shfl_xor(acc, o, 64);
  if ((tid & 63) == 0) out[(row * gridDim.y + blockIdx.y) * 4 + (tid >> 6)] = acc;
}

}  // namespace

// out: uint32 [grid * 256]
extern "C" int probe_read(const void* p, size_t n16, uint32_t* out, int grid, void* stream) {
  if (grid < 1) return (int)hipErrorInvalidValue;
  const size_t chunk16 = (n16 + grid - 1) / grid;
  hipLaunchKernelGGL(read_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream, (const u32x4*)p, n16, chunk16, out);
  return (int)hipGetLastError();
}

// splits: workgroups per index row (each takes k / splits entries, rounded up to 128);
// out: uint32 [rows * splits * 4]
extern "C" int probe_gather(const void* table, int row_bytes, int64_t table_rows, const int32_t* idx, int64_t rows,
                            int k, int splits, uint32_t* out, void* stream) {
  if (rows <= 0 || k <= 0) return 0;
  if (splits < 1) return (int)hipErrorInvalidValue;
  const int per = ((k + splits - 1) / splits + 127) / 128 * 128;
  const int ns = (k + per - 1) / per;
  const int parts = (row_bytes + 127) / 128;
  hipStream_t st = (hipStream_t)stream;
  const dim3 grid((unsigned)rows, (unsigned)ns);
  if (parts <= 5)
    hipLaunchKernelGGL(gather_kernel<5>, grid, dim3(256), 0, st, (const uint8_t*)table, row_bytes, table_rows, idx, k,
                       per, out);
  else if (parts <= 9)
    hipLaunchKernelGGL(gather_kernel<9>, grid, dim3(256), 0, st, (const uint8_t*)table, row_bytes, table_rows, idx, k,
                       per, out);
  else
    return (int)hipErrorInvalidValue;
  return (int)hipGetLastError();
}
