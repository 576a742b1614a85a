// The split-context work plan shared by the split-context attention kernels
// (E4M3 and FP16 caches): every wavefront of every workgroup derives it from
// the context lengths alone, so the kernels need no planning pass.
#pragma once

#include "kvfp8_internal.h"

namespace kvfp8 {

constexpr int kSplitGranule = 64;  // split boundaries fall on multiples of 64 keys

// One (sequence, kv-head, split) work item.
struct SplitItem {
  int b, kvh, s;
  int L;       // the sequence's context length
  int n_used;  // splits the sequence uses (the rest of its S slots are empty)
  int chunk;   // keys per split
  bool valid;
};

// The work plan, computed identically by every wavefront of every workgroup
// from the context lengths alone. All sequences share one split size, set by
// the longest context: C = ceil(L_max / (64 S)) * 64 keys, so the longest
// sequence uses all S splits and a shorter one only ceil(L / C) of them (at
// least one). The non-empty items are numbered in order of sequence, kv-head
// and split, and workgroup `item` takes the item of that number; numbers past
// the last item get none. So the workgroups that have work come first in
// dispatch order and spread evenly over the compute units, and when every
// sequence has the same length the plan is the plain (split, kv-head,
// sequence) grid.
// Wave-wide integer max and inclusive prefix sum with DPP row shifts and the
// gfx9 row broadcasts (lane 15 into rows 1 and 3, lane 31 into rows 2 and 3).
__device__ __forceinline__ int wave_max_i32(int x) {
  x = max(x, __builtin_amdgcn_update_dpp(x, x, 0x111, 0xf, 0xf, false));  // row_shr:1
  x = max(x, __builtin_amdgcn_update_dpp(x, x, 0x112, 0xf, 0xf, false));  // row_shr:2
  x = max(x, __builtin_amdgcn_update_dpp(x, x, 0x114, 0xf, 0xf, false));  // row_shr:4
  x = max(x, __builtin_amdgcn_update_dpp(x, x, 0x118, 0xf, 0xf, false));  // row_shr:8
  x = max(x, __builtin_amdgcn_update_dpp(x, x, 0x142, 0xa, 0xf, false));  // row_bcast:15
  x = max(x, __builtin_amdgcn_update_dpp(x, x, 0x143, 0xc, 0xf, false));  // row_bcast:31
  return __builtin_amdgcn_readlane(x, 63);
}

__device__ __forceinline__ int wave_incl_sum_i32(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);
  return x;
}

__device__ __forceinline__ SplitItem plan_item(const int32_t* __restrict__ seq_lens, int batch, int n_kv_heads,
                                               int S, int item, int lane) {
  const int L0 = lane < batch ? seq_lens[lane] : 0;
  int lmax = L0;
  for (int i = lane + 64; i < batch; i += 64) lmax = max(lmax, seq_lens[i]);
  lmax = wave_max_i32(lmax);
  SplitItem it;
  it.chunk = max(kSplitGranule, ((lmax + kSplitGranule * S - 1) / (kSplitGranule * S)) * kSplitGranule);
  it.valid = false;
  it.b = it.kvh = it.s = it.L = it.n_used = 0;
  int base = 0;  // items of the sequences before b0
  for (int b0 = 0; b0 < batch; b0 += 64) {
    const int bb = b0 + lane;
    const int Lb = b0 == 0 ? L0 : (bb < batch ? seq_lens[bb] : 0);
    const int used = bb < batch ? max(1, (Lb + it.chunk - 1) / it.chunk) : 0;
    const int c = used * n_kv_heads;
    const int incl = wave_incl_sum_i32(c);  // items of sequences b0 .. bb
    const int total = __builtin_amdgcn_readlane(incl, 63);
    if (item < base + total) {
      const uint64_t hit = __ballot(base + incl > item);
      const int src = __builtin_amdgcn_readfirstlane(__ffsll((unsigned long long)hit) - 1);
      const int r = item - base - __builtin_amdgcn_readlane(incl - c, src);
      it.n_used = __builtin_amdgcn_readlane(used, src);
      it.L = __builtin_amdgcn_readlane(Lb, src);
      it.b = b0 + src;
      it.kvh = r / it.n_used;
      it.s = r % it.n_used;
      it.valid = true;
      break;
    }
    base += total;
  }
  return it;
}

}  // namespace kvfp8
