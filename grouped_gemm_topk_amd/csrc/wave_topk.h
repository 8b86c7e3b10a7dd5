// Wave-level top-k selection shared by the gating kernels (prefill gating,
// the fused router launch, the decode routing prologue).
//
// Experts are ranked by logit, larger first, ties to the lower expert index:
// the order of a 64-bit key whose high word is an order-preserving image of
// the float and whose low word is the inverted expert index.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// LDS writes of this wave visible to its other lanes
__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// -0 is folded into +0, so the two compare equal as floats do; 0 is below the
// key of every expert (the "not selectable" key)
__device__ __forceinline__ uint64_t order_key(float f, int e) {
  unsigned u = __float_as_uint(f + 0.0f);
  u ^= (unsigned)((int)u >> 31) | 0x80000000u;
  return ((uint64_t)u << 32) | (uint64_t)(0xffffffffu - (unsigned)e);
}

// Top-k of one token's keys by the calling wave (NV keys per lane, lane l
// holding experts l, l + 64, ...; key 0 = not selectable).  The k largest
// keys lie in the lanes whose own largest key is among the k largest lane
// maxima, so the lane maxima are ranked first (64 compares per lane), those k
// lanes write their NV keys as NV * k candidates, and each candidate is ranked
// among the candidates alone: every key above a top-k key is a top-k key too,
// so for rank < k this is the rank among all keys.  `wk` is per-wave LDS of at
// least 64 + NV * k keys.  Calls sel(i, rank) for each own key i of rank < k.
template <int NV, typename Sel>
__device__ __forceinline__ void wave_topk(uint64_t* wk, const uint64_t* kown, int lane, int k,
                                          Sel sel) {
  uint64_t lm = kown[0];
#pragma unroll
  for (int i = 1; i < NV; ++i) lm = kown[i] > lm ? kown[i] : lm;
  wk[lane] = lm;
  wave_sync_lds();
  int lr = 0;
#pragma unroll
  for (int c = 0; c < 64; c += 2) {
    const ulonglong2 two = *(const ulonglong2*)(wk + c);
    lr += (two.x > lm ? 1 : 0) + (two.y > lm ? 1 : 0);
  }
  uint64_t* cand = wk + 64;
  if (lr < k)
#pragma unroll
    for (int i = 0; i < NV; ++i) cand[lr * NV + i] = kown[i];
  wave_sync_lds();
  if (lr < k) {
    int r[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) r[i] = 0;
    for (int c = 0; c < NV * k; ++c) {
      const uint64_t o = cand[c];
#pragma unroll
      for (int i = 0; i < NV; ++i) r[i] += o > kown[i] ? 1 : 0;
    }
#pragma unroll
    for (int i = 0; i < NV; ++i)
      if (kown[i] != 0ull && r[i] < k) sel(i, r[i]);
  }
}

// the same for nv = ceil(E / 64) keys per lane (1 to 4)
template <typename Sel>
__device__ __forceinline__ void wave_topk_n(int nv, uint64_t* wk, const uint64_t* kown, int lane,
                                            int k, Sel sel) {
  if (nv == 1)
    wave_topk<1>(wk, kown, lane, k, sel);
  else if (nv == 2)
    wave_topk<2>(wk, kown, lane, k, sel);
  else if (nv == 3)
    wave_topk<3>(wk, kown, lane, k, sel);
  else
    wave_topk<4>(wk, kown, lane, k, sel);
}

}  // namespace moe
