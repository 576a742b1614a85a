// Per-tensor amax and scale = amax / 448 over fp16 calibration tensors.
//
// The maximum is taken over the fp16 bit patterns: for a finite fp16 value the
// magnitude bits (bits & 0x7FFF) order exactly like |x|, so an unsigned integer
// maximum is exact and independent of reduction order. Inf (0x7C00) and every
// NaN (above 0x7C00) order above every finite magnitude (at most 0x7BFF), so
// the maximum of the magnitude bits is non-finite exactly when an element is.
#include "kvfp8_internal.h"

namespace kvfp8 {
namespace {

typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));

__global__ void calib_clear(uint32_t* acc, int64_t n) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) acc[i] = 0u;
}

__device__ __forceinline__ u16x2 mag_max(u16x2 m, uint32_t w) {
  return __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, w & 0x7FFF7FFFu));
}

// grid (chunks, n_tensors), 256 threads; each block scans a contiguous chunk
// [lo, hi) of its tensor. The 16-byte aligned middle of the chunk goes through
// the vector loop, which keeps eight 16-byte loads in flight per thread and
// takes the maximum of two magnitudes per packed 16-bit instruction; the at
// most 7 elements before and after it (rows whose length is not a multiple of
// 8 start at any even address) are read one per thread. read_first: see the end.
__global__ __launch_bounds__(256) void calib_amax(const uint16_t* __restrict__ x, int64_t n_elems,
                                                  int64_t chunk, int read_first, uint32_t* acc) {
  constexpr int kUnroll = 8;
  const int64_t t = blockIdx.y;
  const uint16_t* row = x + t * n_elems;
  const int64_t lo = (int64_t)blockIdx.x * chunk;
  const int64_t hi = lo + chunk < n_elems ? lo + chunk : n_elems;
  // elements up to the first 16-byte boundary at or after row + lo
  int64_t head = (int64_t)((16u - ((unsigned)reinterpret_cast<uintptr_t>(row + lo) & 15u)) & 15u) / 2;
  head = head < hi - lo ? head : hi - lo;
  const int64_t vlo = lo + head;
  const int64_t nvec = (hi - vlo) / 8;
  const int64_t vhi = vlo + 8 * nvec;
  uint32_t m = 0u;
  if (threadIdx.x < head) m = row[lo + threadIdx.x] & 0x7FFFu;
  if (threadIdx.x < hi - vhi) m = max(m, (uint32_t)(row[vhi + threadIdx.x] & 0x7FFFu));
  const u32x4* rv = reinterpret_cast<const u32x4*>(row + vlo);
  int64_t i = threadIdx.x;
  u16x2 m2 = {0, 0};
  for (; i + (kUnroll - 1) * 256 < nvec; i += kUnroll * 256) {
    u32x4 w[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) w[u] = __builtin_nontemporal_load(rv + i + u * 256);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
#pragma unroll
      for (int j = 0; j < 4; ++j) m2 = mag_max(m2, w[u][j]);
  }
  for (; i < nvec; i += 256) {
    const u32x4 w = __builtin_nontemporal_load(rv + i);
#pragma unroll
    for (int j = 0; j < 4; ++j) m2 = mag_max(m2, w[j]);
  }
  m = max(m, max((uint32_t)m2[0], (uint32_t)m2[1]));
  // wave reduction, then the block's four wavefronts meet in LDS and one
  // atomic per block folds the result in. The atomics of one tensor all go to
  // one address and are served one after another; with many blocks per tensor
  // (read_first) a block first reads the value folded in so far and skips its
  // atomic when it has nothing larger. Any value it reads was held by acc
  // during this launch (the clear kernel's zero or a later maximum), and acc
  // only grows, so a skip never loses the maximum; an old value costs at most
  // an unneeded atomic. With few blocks per tensor the read's round trip at
  // the end of every block costs more than the atomics it saves.
  __shared__ uint32_t wmax[4];
  for (int off = 32; off > 0; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off));
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t b = max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3]));
    if (read_first ? b > __hip_atomic_load(acc + t, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) : b != 0u)
      atomicMax(acc + t, b);
  }
}

// acc aliases amax_out: read the folded maximum, write amax and scale.
__global__ void calib_finalize(float* amax_out, float* scale_out, int64_t n) {
  int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= n) return;
  uint32_t a = reinterpret_cast<uint32_t*>(amax_out)[t];
  float amax, scale;
  if (a >= 0x7C00u) {
    amax = __uint_as_float(0x7FC00000u);
    scale = amax;
  } else {
    amax = (float)__builtin_bit_cast(_Float16, (uint16_t)a);
    scale = amax / 448.0f;  // IEEE division, correctly rounded
  }
  amax_out[t] = amax;
  scale_out[t] = scale;
}

}  // namespace

hipError_t launch_calibrate(const uint16_t* x, int64_t n_tensors, int64_t n_elems, float* amax,
                            float* scale, hipStream_t stream) {
  uint32_t* acc = reinterpret_cast<uint32_t*>(amax);
  int64_t nb = (n_tensors + 255) / 256;
  calib_clear<<<dim3((unsigned)nb), dim3(256), 0, stream>>>(acc, n_tensors);
  // Aim for about three blocks per CU over the whole input, each scanning
  // 32 to 256 KiB (smaller blocks spend their time starting up and in their
  // atomic; measured on the 48 x 2M-element set: 98 us at 64 KiB, 42 us at
  // 256 KiB), and at most 1024 blocks per tensor.
  const int64_t total = n_tensors * n_elems;
  int64_t chunk = (total + 767) / 768;
  chunk = (chunk + 2047) / 2048 * 2048;
  chunk = chunk < 16384 ? 16384 : (chunk > 131072 ? 131072 : chunk);
  int64_t chunks = (n_elems + chunk - 1) / chunk;
  if (chunks > 1024) {
    chunks = 1024;
    chunk = ((n_elems + chunks - 1) / chunks + 7) / 8 * 8;
    chunks = (n_elems + chunk - 1) / chunk;
  }
  if (chunks < 1) chunks = 1;
  // Read before the atomic from 64 blocks per tensor up (134 MB in two tensors,
  // 382 blocks each: 27.9 -> 23.7 us; 4 GiB: 672 -> 636 us; the same bytes in
  // 48 tensors of 16 blocks: 24.4 us without the read, 31.0 with it).
  const int read_first = chunks >= 64;
  for (int64_t t0 = 0; t0 < n_tensors; t0 += 65535) {
    int64_t nt = n_tensors - t0 < 65535 ? n_tensors - t0 : 65535;
    calib_amax<<<dim3((unsigned)chunks, (unsigned)nt), dim3(256), 0, stream>>>(
        x + t0 * n_elems, n_elems, chunk, read_first, acc + t0);
  }
  calib_finalize<<<dim3((unsigned)nb), dim3(256), 0, stream>>>(amax, scale, n_tensors);
  return hipGetLastError();
}

}  // namespace kvfp8
