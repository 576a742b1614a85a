// Reduction of FP32 split partials (o, m, l) into the fp16 output and the
// log-sum-exp. One wavefront per (row, head); the split weights go through LDS.
#include "kvfp8_internal.h"

namespace kvfp8 {
namespace {

constexpr int kMaxSplits = 256;
constexpr int kWavesPerBlock = 4;

template <int D>
__global__ __launch_bounds__(64 * kWavesPerBlock) void split_reduce_kernel(
    const float* __restrict__ ws_o, const float* __restrict__ ws_m, const float* __restrict__ ws_l,
    int64_t n_units, int num_splits, uint16_t* __restrict__ out, float* __restrict__ lse) {
  __shared__ float wsh[kWavesPerBlock][kMaxSplits];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t unit = (int64_t)blockIdx.x * kWavesPerBlock + wave;  // (row, head)
  if (unit >= n_units) return;  // whole wave exits together; no block barrier below
  const float* m = ws_m + unit * num_splits;
  const float* l = ws_l + unit * num_splits;

  float mx = -INFINITY;
  for (int s = lane; s < num_splits; s += 64) mx = fmaxf(mx, m[s]);
  for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  const float ref = (mx == -INFINITY) ? 0.0f : mx;

  float den = 0.0f;
  for (int s = lane; s < num_splits; s += 64) {
    float ms = m[s];
    float w = (ms == -INFINITY) ? 0.0f : __expf(ms - ref);
    wsh[wave][s] = w;
    den += w * l[s];
  }
  for (int off = 32; off > 0; off >>= 1) den += __shfl_xor(den, off);
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");

  constexpr int PER = D / 64;  // dims per lane
  float acc[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) acc[j] = 0.0f;
  const float* o = ws_o + unit * (int64_t)num_splits * D + lane * PER;
  for (int s = 0; s < num_splits; ++s) {
    float w = wsh[wave][s];
    if (w != 0.0f) {
      if constexpr (PER == 2) {
        f32x2 v = *reinterpret_cast<const f32x2*>(o + (int64_t)s * D);
        acc[0] += w * v[0];
        acc[1] += w * v[1];
      } else {
        acc[0] += w * o[(int64_t)s * D];
      }
    }
  }
  const float inv = den > 0.0f ? 1.0f / den : 0.0f;
  uint16_t* dst = out + unit * D + lane * PER;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    _Float16 h = (_Float16)(den > 0.0f ? acc[j] * inv : 0.0f);
    dst[j] = __builtin_bit_cast(uint16_t, h);
  }
  if (lse != nullptr && lane == 0) lse[unit] = den > 0.0f ? ref + __logf(den) : -INFINITY;
}

}  // namespace

hipError_t launch_split_reduce(const float* ws_o, const float* ws_m, const float* ws_l,
                               int32_t n_rows, int32_t n_q_heads, int32_t head_dim,
                               int32_t num_splits, uint16_t* out, float* lse,
                               hipStream_t stream) {
  int64_t units = (int64_t)n_rows * n_q_heads;
  if (units == 0) return hipSuccess;
  dim3 grid((unsigned)((units + kWavesPerBlock - 1) / kWavesPerBlock));
  dim3 block(64 * kWavesPerBlock);
  if (head_dim == 128)
    split_reduce_kernel<128><<<grid, block, 0, stream>>>(ws_o, ws_m, ws_l, units, num_splits, out, lse);
  else
    split_reduce_kernel<64><<<grid, block, 0, stream>>>(ws_o, ws_m, ws_l, units, num_splits, out, lse);
  return hipGetLastError();
}

}  // namespace kvfp8
