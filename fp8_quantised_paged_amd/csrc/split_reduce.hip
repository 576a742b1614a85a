// Reduction of FP32 split partials (o, m, l) into the fp16 output and the
// log-sum-exp. One workgroup of four wavefronts per (row, head): every
// wavefront forms the split weights, takes a quarter of the splits for the
// weighted sum of o with its loads batched ahead of use, and the four partial
// sums meet in LDS.
#include "kvfp8_internal.h"

namespace kvfp8 {
namespace {

constexpr int kMaxSplits = 256;
constexpr int kWaves = 4;
constexpr int kBatch = 4;  // splits whose o loads are in flight together per wavefront

template <int D>
__global__ __launch_bounds__(64 * kWaves) void split_reduce_kernel(
    const float* __restrict__ ws_o, const float* __restrict__ ws_m, const float* __restrict__ ws_l,
    int64_t n_units, int num_splits, uint16_t* __restrict__ out, float* __restrict__ lse) {
  constexpr int PER = D / 64;             // dims per lane
  constexpr int SPL = kMaxSplits / 64;    // splits per lane for m and l
  __shared__ float wsh[kMaxSplits];
  __shared__ float part[kWaves][D];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t unit = blockIdx.x;  // (row, head)
  const float* m = ws_m + unit * num_splits;
  const float* l = ws_l + unit * num_splits;
  const float* o = ws_o + unit * (int64_t)num_splits * D + lane * PER;

  // Every load that does not depend on the weights is issued first: this
  // wavefront's first batch of o, and m and l of every split, so the kernel
  // waits for memory once rather than once per step.
  float v[kBatch][PER];
  int s0 = wave * kBatch;
#pragma unroll
  for (int u = 0; u < kBatch; ++u) {
    const int s = min(s0 + u, num_splits - 1);
#pragma unroll
    for (int j = 0; j < PER; ++j) v[u][j] = o[(int64_t)s * D + j];
  }
  float ms[SPL], ls[SPL];
#pragma unroll
  for (int k = 0; k < SPL; ++k) {
    const int s = lane + 64 * k;
    ms[k] = s < num_splits ? m[s] : -INFINITY;
    ls[k] = s < num_splits ? l[s] : 0.0f;
  }

  // global max and weighted normaliser over the splits (every wavefront
  // computes them; wavefront 0 publishes the weights)
  float mx = -INFINITY;
#pragma unroll
  for (int k = 0; k < SPL; ++k) mx = fmaxf(mx, ms[k]);
  for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  const float ref = (mx == -INFINITY) ? 0.0f : mx;
  float den = 0.0f;
#pragma unroll
  for (int k = 0; k < SPL; ++k) {
    const float w = (ms[k] == -INFINITY) ? 0.0f : __expf(ms[k] - ref);
    const int s = lane + 64 * k;
    if (wave == 0 && s < num_splits) wsh[s] = w;
    den += w * ls[k];
  }
  for (int off = 32; off > 0; off >>= 1) den += __shfl_xor(den, off);
  // splits past the last one with a finite m have weight zero: their o is
  // neither loaded nor used (their slots need not have been written)
  int n_live = 0;
#pragma unroll
  for (int k = 0; k < SPL; ++k)
    if (ms[k] != -INFINITY) n_live = lane + 64 * k + 1;
  for (int off = 32; off > 0; off >>= 1) n_live = max(n_live, __shfl_xor(n_live, off));
  __syncthreads();

  float acc[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) acc[j] = 0.0f;
  while (s0 < n_live) {
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const float w = (s0 + u < n_live) ? wsh[s0 + u] : 0.0f;
#pragma unroll
      for (int j = 0; j < PER; ++j) acc[j] += (w != 0.0f) ? w * v[u][j] : 0.0f;
    }
    s0 += kWaves * kBatch;
    if (s0 >= n_live) break;
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int s = min(s0 + u, num_splits - 1);
#pragma unroll
      for (int j = 0; j < PER; ++j) v[u][j] = o[(int64_t)s * D + j];
    }
  }
#pragma unroll
  for (int j = 0; j < PER; ++j) part[wave][lane * PER + j] = acc[j];
  __syncthreads();
  if (wave == 0) {
    const float inv = den > 0.0f ? 1.0f / den : 0.0f;
    uint16_t* dst = out + unit * D + lane * PER;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      float t = 0.0f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) t += part[w][lane * PER + j];
      const _Float16 h = (_Float16)(den > 0.0f ? t * inv : 0.0f);
      dst[j] = __builtin_bit_cast(uint16_t, h);
    }
    if (lse != nullptr && lane == 0) lse[unit] = den > 0.0f ? ref + __logf(den) : -INFINITY;
  }
}

// Few splits (the decode case): one wavefront per (row, head), four per
// workgroup, and every load of the unit -- m, l and this lane's dims of o for
// each split -- issued together, so the kernel waits for memory once. The
// weights and sums are those of split_reduce_kernel; splits with m = -inf get
// weight zero without their o being multiplied.
constexpr int kSmallSplits = 8;
constexpr int kUnitsPerBlock = 4;

template <int D>
__global__ __launch_bounds__(64 * kUnitsPerBlock) void split_reduce_small_kernel(
    const float* __restrict__ ws_o, const float* __restrict__ ws_m, const float* __restrict__ ws_l,
    int64_t n_units, int num_splits, uint16_t* __restrict__ out, float* __restrict__ lse) {
  constexpr int PER = D / 64;  // dims per lane
  const int lane = threadIdx.x & 63;
  const int64_t unit = (int64_t)blockIdx.x * kUnitsPerBlock + (threadIdx.x >> 6);
  if (unit >= n_units) return;  // uniform over the wavefront
  const float* m = ws_m + unit * num_splits;
  const float* l = ws_l + unit * num_splits;
  const float* o = ws_o + unit * (int64_t)num_splits * D + lane * PER;
  float ms[kSmallSplits], ls[kSmallSplits], v[kSmallSplits][PER];
#pragma unroll
  for (int s = 0; s < kSmallSplits; ++s) {
    const int sc = min(s, num_splits - 1);  // loads stay inside the unit; extra splits get weight zero
    ms[s] = s < num_splits ? m[sc] : -INFINITY;
    ls[s] = l[sc];
#pragma unroll
    for (int j = 0; j < PER; ++j) v[s][j] = o[(int64_t)sc * D + j];
  }
  float mx = -INFINITY;
#pragma unroll
  for (int s = 0; s < kSmallSplits; ++s) mx = fmaxf(mx, ms[s]);
  const float ref = (mx == -INFINITY) ? 0.0f : mx;
  float den = 0.0f;
  float acc[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) acc[j] = 0.0f;
#pragma unroll
  for (int s = 0; s < kSmallSplits; ++s) {
    const float w = (ms[s] == -INFINITY) ? 0.0f : __expf(ms[s] - ref);
    den += (w != 0.0f) ? w * ls[s] : 0.0f;
#pragma unroll
    for (int j = 0; j < PER; ++j) acc[j] += (w != 0.0f) ? w * v[s][j] : 0.0f;
  }
  const float inv = den > 0.0f ? 1.0f / den : 0.0f;
  uint16_t* dst = out + unit * D + lane * PER;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const _Float16 h = (_Float16)(den > 0.0f ? acc[j] * inv : 0.0f);
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
  if (num_splits <= kSmallSplits) {
    dim3 grid((unsigned)((units + kUnitsPerBlock - 1) / kUnitsPerBlock));
    dim3 block(64 * kUnitsPerBlock);
    if (head_dim == 128)
      split_reduce_small_kernel<128><<<grid, block, 0, stream>>>(ws_o, ws_m, ws_l, units, num_splits, out, lse);
    else
      split_reduce_small_kernel<64><<<grid, block, 0, stream>>>(ws_o, ws_m, ws_l, units, num_splits, out, lse);
    return hipGetLastError();
  }
  dim3 grid((unsigned)units);
  dim3 block(64 * kWaves);
  if (head_dim == 128)
    split_reduce_kernel<128><<<grid, block, 0, stream>>>(ws_o, ws_m, ws_l, units, num_splits, out, lse);
  else
    split_reduce_kernel<64><<<grid, block, 0, stream>>>(ws_o, ws_m, ws_l, units, num_splits, out, lse);
  return hipGetLastError();
}

}  // namespace kvfp8
