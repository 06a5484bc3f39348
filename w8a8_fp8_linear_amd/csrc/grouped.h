// Device helpers shared by the grouped (routed-expert) kernels of both
// expert formats: the tile lookup over the device-side group offsets and the
// ordered per-token sum of the float32 slot rows.
#pragma once

#include "device.h"

namespace w8a8 {

// Which expert and which rows the m-tile `mt` covers, from the device-side
// offsets (each wave computes it; the answer is uniform). The rows are
// clamped to [0, cap), the capacity of the sorted arrays, so inconsistent
// offsets can never address outside them.
__device__ inline bool find_tile(const int32_t* __restrict__ offsets, int E, int BM, int mt, int cap, int& e_out,
                                 int& row0, int& rows) {
  const int lane = threadIdx.x & 63;
  int acc = 0;
  for (int e0 = 0; e0 < E; e0 += 64) {
    const int e = e0 + lane;
    int cnt = 0, start = 0;
    if (e < E) {
      start = offsets[e];
      cnt = offsets[e + 1] - start;
    }
    const int tiles = (cnt + BM - 1) / BM;
    int incl = tiles;
    for (int d = 1; d < 64; d <<= 1) {
      const int v = __shfl_up(incl, d, 64);
      if (lane >= d) incl += v;
    }
    const int excl = incl - tiles;
    const bool hit = e < E && mt >= acc + excl && mt < acc + incl;
    const uint64_t b = __ballot(hit);
    if (b) {
      const int src = __ffsll((unsigned long long)b) - 1;
      const int ex = __shfl(excl, src, 64), st = __shfl(start, src, 64), ct = __shfl(cnt, src, 64);
      const int local = mt - acc - ex;
      e_out = __builtin_amdgcn_readfirstlane(e0 + src);
      row0 = __builtin_amdgcn_readfirstlane(st + local * BM);
      rows = __builtin_amdgcn_readfirstlane(min(BM, ct - local * BM));
      if (row0 < 0 || row0 >= cap) return false;
      rows = min(rows, cap - row0);
      return rows > 0;
    }
    acc += __shfl(incl, 63, 64);
  }
  return false;
}

// Sum of a token's valid float32 slot rows at columns c0 .. c0 + 7, in the
// order j = 0, 1, ... in float32 (deterministic). Slot t * topk + j's row of
// y is the slot itself, or slot_row[slot] when slot_row is given (the down
// projection then wrote its rows in sorted order). The rows are loaded
// (non-temporal: each byte is read once) before any is added; a dropped
// slot's row is not used.
__device__ inline void sum_slots8(const float* __restrict__ y, const int32_t* __restrict__ ids,
                                  const int32_t* __restrict__ slot_row, int64_t t, int topk, int Eids, int H, int c0,
                                  float4& a, float4& b) {
  a = make_float4(0.f, 0.f, 0.f, 0.f);
  b = a;
  constexpr int kBatch = 8;
  for (int j0 = 0; j0 < topk; j0 += kBatch) {
    v4f u[kBatch], v[kBatch];
    bool ok[kBatch];
#pragma unroll
    for (int jj = 0; jj < kBatch; ++jj) {
      const int j = j0 + jj;
      const int64_t slot = t * topk + (j < topk ? j : 0);
      const int id = ids[slot];
      ok[jj] = j < topk && id >= 0 && id < Eids;
      const int64_t row = !ok[jj] ? 0 : slot_row ? (int64_t)slot_row[slot] : slot;
      const v4f* src = reinterpret_cast<const v4f*>(y + row * H + c0);
      u[jj] = __builtin_nontemporal_load(src);
      v[jj] = __builtin_nontemporal_load(src + 1);
    }
#pragma unroll
    for (int jj = 0; jj < kBatch; ++jj) {
      if (!ok[jj]) continue;
      a.x += u[jj][0]; a.y += u[jj][1]; a.z += u[jj][2]; a.w += u[jj][3];
      b.x += v[jj][0]; b.y += v[jj][1]; b.z += v[jj][2]; b.w += v[jj][3];
    }
  }
}

// Columns of thread r (0 <= r < H / 8) of a row: two runs of 4, ca .. ca + 3
// and cb .. cb + 3. The 64 threads of a 512-column block take the block's
// first half as 4-column runs in lane order and the second half likewise, so
// each of a wave's 16-byte load instructions reads 1 KB contiguous. A last,
// shorter block of W columns is split at W / 2 (H is a multiple of 8).
__device__ inline void split_cols8(int r, int H, int& ca, int& cb) {
  const int base = (r >> 6) << 9, l = r & 63;
  const int w = min(512, H - base);
  ca = base + 4 * l;
  cb = base + (w >> 1) + 4 * l;
}

// sum_slots8 over the columns ca .. ca + 3 (a) and cb .. cb + 3 (b).
__device__ inline void sum_slots_split(const float* __restrict__ y, const int32_t* __restrict__ ids,
                                       const int32_t* __restrict__ slot_row, int64_t t, int topk, int Eids, int H,
                                       int ca, int cb, float4& a, float4& b) {
  a = make_float4(0.f, 0.f, 0.f, 0.f);
  b = a;
  constexpr int kBatch = 8;
  for (int j0 = 0; j0 < topk; j0 += kBatch) {
    v4f u[kBatch], v[kBatch];
    bool ok[kBatch];
#pragma unroll
    for (int jj = 0; jj < kBatch; ++jj) {
      const int j = j0 + jj;
      const int64_t slot = t * topk + (j < topk ? j : 0);
      const int id = ids[slot];
      ok[jj] = j < topk && id >= 0 && id < Eids;
      const int64_t row = !ok[jj] ? 0 : slot_row ? (int64_t)slot_row[slot] : slot;
      const float* src = y + row * H;
      u[jj] = __builtin_nontemporal_load(reinterpret_cast<const v4f*>(src + ca));
      v[jj] = __builtin_nontemporal_load(reinterpret_cast<const v4f*>(src + cb));
    }
#pragma unroll
    for (int jj = 0; jj < kBatch; ++jj) {
      if (!ok[jj]) continue;
      a.x += u[jj][0]; a.y += u[jj][1]; a.z += u[jj][2]; a.w += u[jj][3];
      b.x += v[jj][0]; b.y += v[jj][1]; b.z += v[jj][2]; b.w += v[jj][3];
    }
  }
}

__device__ inline uint4 to_bf16x8(float4 a, float4 b) {
  return make_uint4(bf16x2_rne(a.x, a.y), bf16x2_rne(a.z, a.w), bf16x2_rne(b.x, b.y), bf16x2_rne(b.z, b.w));
}

}  // namespace w8a8
