// Split-KV partial states for single-row slices (decode: one new token per
// query head, no grouped heads to pack), on the vector units.
//
// With one query row the matrix unit has nothing to amortise: the streaming
// kernel stages every 64-key tile in LDS for a 32-row MFMA of which one row
// is real, and the chunk streams only as fast as those staged tiles allow.
// Here the workgroup's four waves each take a quarter of the chunk's keys
// and read K and V straight from memory into registers. Within a wave, D/8
// lanes hold one key's D values (8 each, one 16-byte load), so 64 / (D/8)
// keys are scored per step; a lane group keeps an online (max, sum,
// numerator) state of its own over the keys it scores, eight steps of keys
// in flight at a time, and the states are merged at the end, across the
// lane groups and then across the waves. Each K/V byte is read once, so the
// loads are marked nontemporal (measured: 6.97 vs 6.19 TB/s without the
// hint, on 16x32x131072x128 bf16). The merged state is the chunk's
// partial state, in the streaming kernel's split-mode convention (max in
// natural-log units of the scaled score, unnormalised sum and numerator).
// ("Intermediate and advanced extension", workshop table, split-softmax
// row: partial statistics per chunk; "Attention algorithms and data
// movement", lesson 01: partial states merged by rescaled denominators.)
#pragma once

#include "fwd_kernel.hpp"

namespace sattn {

template <class E, int D, bool CAUSAL>
__global__ __launch_bounds__(256) void split_row_kernel(const FwdParams p) {
  constexpr int LPK = D / 8;        // lanes per key
  constexpr int KPS = 64 / LPK;     // keys per wave per step
  constexpr int UNROLL = 8;         // steps in flight
  __shared__ float wm[4], wl[4];
  __shared__ __attribute__((aligned(16))) float wacc[4][D];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kg = lane / LPK;          // this lane's key within a step
  const int dl = (lane % LPK) * 8;    // its first d value
  // block -> (row, chunk), chunk fastest; a row is one (batch, query head)
  const int c = blockIdx.x % p.nchunks;
  const int row = blockIdx.x / p.nchunks;
  const int grp = p.hq / p.hkv;
  const int kvs = (row / p.hq) * p.hkv + (row % p.hq) / grp;
  const uint16_t* kb = p.k + (int64_t)kvs * p.nk * D;
  const uint16_t* vb = p.v + (int64_t)kvs * p.nk * D;
  const int k_begin = c * p.chunk;
  int k_end = min(p.nk, k_begin + p.chunk);
  if (CAUSAL) k_end = max(k_begin, min(k_end, p.off + 1));   // the row sits at position off

  float qv[8];
  {
    const u32x4 w4 = *(const u32x4*)(p.q + (int64_t)row * D + dl);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      qv[2 * j] = E::lo(w4[j]);
      qv[2 * j + 1] = E::hi(w4[j]);
    }
  }
  const float cs = p.c;

  // this wave's keys: a quarter of the chunk, in whole steps
  const int per_wave = ((k_end - k_begin + 4 * KPS - 1) / (4 * KPS)) * KPS;
  const int wk0 = k_begin + wave * per_wave;
  const int wk1 = min(k_end, wk0 + per_wave);
  float m = -INFINITY, l = 0.f, acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  for (int k = wk0; k < wk1; k += KPS * UNROLL) {
    u32x4 kr[UNROLL], vr[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int key = k + u * KPS + kg;
      const bool ok = key < wk1;
      kr[u] = ok ? __builtin_nontemporal_load((const u32x4*)(kb + (int64_t)key * D + dl)) : u32x4{0, 0, 0, 0};
      vr[u] = ok ? __builtin_nontemporal_load((const u32x4*)(vb + (int64_t)key * D + dl)) : u32x4{0, 0, 0, 0};
    }
    float s[UNROLL];
    float mb = -INFINITY;
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      float d = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        d = fmaf(qv[2 * j], E::lo(kr[u][j]), d);
        d = fmaf(qv[2 * j + 1], E::hi(kr[u][j]), d);
      }
#pragma unroll
      for (int o = LPK / 2; o > 0; o >>= 1) d += __shfl_xor(d, o);   // the key's dot product, in all its lanes
      s[u] = (k + u * KPS + kg < wk1) ? d * cs : -INFINITY;
      mb = fmaxf(mb, s[u]);
    }
    // exact update of this lane group's state (all its lanes agree): the
    // exported maximum is the chunk's own, as in the streaming kernel's
    // split mode
    if (mb > m) {
      const float alpha = fast_exp2(m - mb);   // 0 while the state is empty
      l *= alpha;
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] *= alpha;
      m = mb;
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const float pu = (s[u] == -INFINITY) ? 0.f : fast_exp2(s[u] - m);   // keys past the range add nothing
      l += pu;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[2 * j] = fmaf(pu, E::lo(vr[u][j]), acc[2 * j]);
        acc[2 * j + 1] = fmaf(pu, E::hi(vr[u][j]), acc[2 * j + 1]);
      }
    }
  }

  // merge the wave's lane groups (lanes that differ in the key bits hold the
  // same d values), then the four waves
  float mw = m;
#pragma unroll
  for (int o = LPK; o < 64; o <<= 1) mw = fmaxf(mw, __shfl_xor(mw, o));
  const float wgt = (m == -INFINITY) ? 0.f : fast_exp2(m - mw);
  float lw = l * wgt;
  float aw[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) aw[i] = acc[i] * wgt;
#pragma unroll
  for (int o = LPK; o < 64; o <<= 1) {
    lw += __shfl_xor(lw, o);
#pragma unroll
    for (int i = 0; i < 8; ++i) aw[i] += __shfl_xor(aw[i], o);
  }
  if (lane < LPK) {
#pragma unroll
    for (int i = 0; i < 8; ++i) wacc[wave][dl + i] = aw[i];
    if (lane == 0) {
      wm[wave] = mw;
      wl[wave] = lw;
    }
  }
  __syncthreads();
  if (wave != 0) return;
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < 4; ++w) M = fmaxf(M, wm[w]);
  const int64_t prow = (int64_t)row * p.nchunks + c;
  float lt = 0.f;
  for (int e = lane; e < D; e += 64) {
    float a = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) a += (wm[w] == -INFINITY) ? 0.f : wacc[w][e] * fast_exp2(wm[w] - M);
    p.part_acc[prow * D + e] = a;
  }
#pragma unroll
  for (int w = 0; w < 4; ++w) lt += (wm[w] == -INFINITY) ? 0.f : wl[w] * fast_exp2(wm[w] - M);
  if (lane == 0) {
    p.part_m[prow] = M * kLn2;   // natural-log units of the scaled score; -inf for an empty chunk
    p.part_l[prow] = lt;
  }
}

}  // namespace sattn
