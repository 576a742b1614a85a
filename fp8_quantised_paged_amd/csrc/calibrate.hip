// Per-tensor amax and scale = amax / 448 over fp16 calibration tensors.
//
// The maximum is taken over the fp16 bit patterns: for a finite fp16 value the
// magnitude bits (bits & 0x7FFF) order exactly like |x|, so an unsigned integer
// maximum is exact and independent of reduction order. A non-finite element
// (exponent bits all ones) raises the accumulator above every finite magnitude.
#include "kvfp8_internal.h"

namespace kvfp8 {
namespace {

constexpr uint32_t kNonFinite = 0x10000u;

__device__ __forceinline__ uint32_t fold_half(uint32_t h) {
  uint32_t mag = h & 0x7FFFu;
  return (mag >= 0x7C00u) ? kNonFinite : mag;
}

__global__ void calib_clear(uint32_t* acc, int64_t n) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) acc[i] = 0u;
}

// grid (chunks, n_tensors), 256 threads; each block scans a contiguous chunk
// of its tensor. vec8: rows are 16-byte aligned (n_elems % 8 == 0).
__global__ __launch_bounds__(256) void calib_amax(const uint16_t* __restrict__ x, int64_t n_elems,
                                                  int64_t chunk, int vec8, uint32_t* acc) {
  const int64_t t = blockIdx.y;
  const uint16_t* row = x + t * n_elems;
  int64_t lo = (int64_t)blockIdx.x * chunk;
  int64_t hi = lo + chunk < n_elems ? lo + chunk : n_elems;
  uint32_t m = 0u;
  if (vec8) {
    const u32x4* rv = reinterpret_cast<const u32x4*>(row);
    for (int64_t i = lo / 8 + threadIdx.x; i < hi / 8; i += blockDim.x) {
      u32x4 w = __builtin_nontemporal_load(rv + i);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        m = max(m, fold_half(w[j] & 0xFFFFu));
        m = max(m, fold_half(w[j] >> 16));
      }
    }
  } else {
    for (int64_t i = lo + threadIdx.x; i < hi; i += blockDim.x) m = max(m, fold_half(row[i]));
  }
  // wave reduction, then one atomic per wave
  for (int off = 32; off > 0; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off));
  if ((threadIdx.x & 63) == 0 && m != 0u) atomicMax(acc + t, m);
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
  // about 64 KiB of input per block, at most 1024 blocks per tensor
  int64_t chunk = 32768;
  int64_t chunks = (n_elems + chunk - 1) / chunk;
  if (chunks > 1024) {
    chunks = 1024;
    chunk = ((n_elems + chunks - 1) / chunks + 7) / 8 * 8;
    chunks = (n_elems + chunk - 1) / chunk;
  }
  if (chunks < 1) chunks = 1;
  int vec8 = ((n_elems % 8) == 0) && ((reinterpret_cast<uintptr_t>(x) & 15) == 0);
  for (int64_t t0 = 0; t0 < n_tensors; t0 += 65535) {
    int64_t nt = n_tensors - t0 < 65535 ? n_tensors - t0 : 65535;
    calib_amax<<<dim3((unsigned)chunks, (unsigned)nt), dim3(256), 0, stream>>>(
        x + t0 * n_elems, n_elems, chunk, vec8, acc + t0);
  }
  calib_finalize<<<dim3((unsigned)nb), dim3(256), 0, stream>>>(amax, scale, n_tensors);
  return hipGetLastError();
}

}  // namespace kvfp8
