// Latency kernel for small batched problems (D = 32 or 64).
//
// When the whole problem is a few dozen query tiles, the streaming kernel's
// serial walk over key tiles (one tile of load latency after another) sets
// the runtime. Here a workgroup of NWAVE (4 or 8) waves owns 32 query rows of
// one head and splits that head's eligible keys between its waves: wave w takes
// key tiles w, w+NWAVE, ... Each wave loads its tile into its own LDS region, runs the
// same MFMA/online-softmax step as the streaming kernel, and keeps a partial
// state (m, l, acc) for its keys. The partial states are then merged
// through LDS with the split-KV rule: M = max m_w, L = sum exp(m_w - M) l_w,
// O = sum exp(m_w - M) acc_w / L ("Attention algorithms and data movement",
// lesson 01; a split with no eligible key is the empty state and weighs 0).
#pragma once

#include "fwd_kernel.hpp"

namespace sattn {

template <class E, int D, int NWAVE, bool CAUSAL>
__global__ __launch_bounds__(NWAVE * 64) void fwd_small_kernel(const FwdParams p) {
  constexpr int BN = 64;
  constexpr int PPR = D / 8;
  constexpr int NI = BN * D * 2 / 1024;   // 1 KiB loads per tile and tensor (one wave)
  constexpr int KK = D / 16;
  constexpr int KB = BN / 32;
  constexpr int DB = D / 32;
  constexpr int TILE = BN * D;            // elements of one K or V tile
  static_assert(D == 32 || D == 64, "small-problem kernel is for D = 32 or 64");
  // Per wave: K and V tile; reused for the partial states after the loop.
  __shared__ __attribute__((aligned(1024))) uint16_t sm[NWAVE][2 * TILE];
  __shared__ float s_m[NWAVE][32];
  __shared__ float s_l[NWAVE][32];

  const int head = blockIdx.x / p.nqt;
  const int qt = blockIdx.x % p.nqt;
  const int q_pos0 = qt * 32;
  const int nq = min(32, p.n - q_pos0);
  const int64_t base = (int64_t)head * p.n * D;
  const int k_end = CAUSAL ? min(p.n, q_pos0 + 32) : p.n;
  const int ntiles = (k_end + BN - 1) / BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hf = lane >> 5;
  const bool row_ok = l32 < nq;
  const int my_pos = q_pos0 + l32;

  u32x4 qreg[KK];
  {
    const uint16_t* qp = p.q + base + (int64_t)(q_pos0 + l32) * D + hf * 8;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      qreg[kk] = row_ok ? *(const u32x4*)(qp + kk * 16) : u32x4{0, 0, 0, 0};
  }
  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;
  float m = -INFINITY;
  float l = 0.f;
  const float c = p.c;

  const uint32_t row_bytes = (uint32_t)D * 2u;
  const __amdgpu_buffer_rsrc_t rk =
      __builtin_amdgcn_make_buffer_rsrc((void*)(p.k + base), (short)0, (int)(k_end * row_bytes), 0x00020000);
  const __amdgpu_buffer_rsrc_t rv =
      __builtin_amdgcn_make_buffer_rsrc((void*)(p.v + base), (short)0, (int)(k_end * row_bytes), 0x00020000);
  uint16_t* sK = sm[wave];
  uint16_t* sV = sm[wave] + TILE;

  int kofs[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) kofs[kk] = l32 * D + (((kk * 2 + hf) ^ swz<D>(l32)) * 8);
  const int g16 = lane >> 4;
  const int tr_key = 4 * (g16 >> 1) + ((lane & 15) >> 2);
  int vofs[2][DB];
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int d0 = db * 32 + 16 * (g16 & 1) + 4 * (lane & 3);
      const int key = tr_key + 8 * x;
      vofs[x][db] = key * D + (((d0 >> 3) ^ swz<D>(key)) * 8) + (d0 & 7);
    }

  for (int t = wave; t < ntiles; t += NWAVE) {
    const int kt0 = t * BN;
    const uint32_t soff = __builtin_amdgcn_readfirstlane((uint32_t)kt0 * row_bytes);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int slot = i * 64 + lane;
      const int key = slot / PPR;
      const uint32_t voff = (uint32_t)key * row_bytes + (uint32_t)(((slot % PPR) ^ swz<D>(key)) * 16);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (__attribute__((address_space(3))) void*)(sK + i * 512), 16, voff,
                                               soff, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (__attribute__((address_space(3))) void*)(sV + i * 512), 16, voff,
                                               soff, 0, 0);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's own tile (wave-private LDS)

    f32x16 s[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
        s[kb] = E::mfma32(*(const u32x4*)(sK + kofs[kk] + kb * 32 * D), qreg[kk], s[kb]);
    }
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kt0 + kb * 32 + 8 * (r >> 2) + 4 * hf + (r & 3);
        if ((key >= k_end) || (CAUSAL && key > my_pos)) s[kb][r] = -INFINITY;
      }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = max_halves(mx);
    // Exact running max (a split may see only masked keys first: keep -inf
    // until a real key arrives, and never form exp2(-inf - -inf)).
    const float m_new = fmaxf(m, mx * c);
    const float alpha = (m_new == -INFINITY) ? 1.0f : fast_exp2(m - m_new);
    m = m_new;
    const float msub = (m == -INFINITY) ? 0.0f : m;
    l *= alpha;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;
    float rs = 0.f;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pv = fast_exp2(fmaf(s[kb][r], c, -msub));
        s[kb][r] = pv;
        rs += pv;
      }
    l += rs;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int o8 = half * 8;
        const u32x4 pb = {E::pack2(s[kb][o8 + 0], s[kb][o8 + 1]), E::pack2(s[kb][o8 + 2], s[kb][o8 + 3]),
                          E::pack2(s[kb][o8 + 4], s[kb][o8 + 5]), E::pack2(s[kb][o8 + 6], s[kb][o8 + 7])};
        const int krow = (kb * 32 + half * 16) * D;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const u32x2 a0 = lds_read_tr16(sV + vofs[0][db] + krow);
          const u32x2 a1 = lds_read_tr16(sV + vofs[1][db] + krow);
          acc[db] = E::mfma32(u32x4{a0[0], a0[1], a1[0], a1[1]}, pb, acc[db]);
        }
      }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // done reading before the next tile's loads
  }

  // ---- partial states to LDS: each wave stores its accumulator in its own
  // lane layout (group g = db*4 + g4 of four floats, then lane), so that the
  // merge below reads the same 16 bytes per lane from every wave.
  constexpr int NG = DB * 4;                          // float4 groups per lane
  const float lt = sum_halves(l);
  f32x4* pacc = reinterpret_cast<f32x4*>(sm[wave]);   // NG x 64 lanes x 16 B fit in one wave's region
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4)
      pacc[(db * 4 + g4) * 64 + lane] =
          f32x4{acc[db][g4 * 4 + 0], acc[db][g4 * 4 + 1], acc[db][g4 * 4 + 2], acc[db][g4 * 4 + 3]};
  if (hf == 0) {
    s_m[wave][l32] = m;
    s_l[wave][l32] = lt;
  }
  __syncthreads();

  // ---- merge: wave w combines groups g = w, w + NWAVE, ... of every row.
  float wgt[NWAVE];
  float big_m = -INFINITY;
#pragma unroll
  for (int wv = 0; wv < NWAVE; ++wv) big_m = fmaxf(big_m, s_m[wv][l32]);
  float big_l = 0.f;
#pragma unroll
  for (int wv = 0; wv < NWAVE; ++wv) {
    const float mw = s_m[wv][l32];
    wgt[wv] = (mw == -INFINITY) ? 0.f : fast_exp2(mw - big_m);
    big_l += wgt[wv] * s_l[wv][l32];
  }
  const float inv = 1.f / big_l;
  for (int g = wave; g < NG; g += NWAVE) {
    f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int wv = 0; wv < NWAVE; ++wv) {
      const f32x4 x = reinterpret_cast<const f32x4*>(sm[wv])[g * 64 + lane];
      o += wgt[wv] * x;
    }
    if (row_ok) {
      const int d = (g >> 2) * 32 + 8 * (g & 3) + 4 * hf;
      *(u32x2*)(p.o + base + (int64_t)(q_pos0 + l32) * D + d) =
          u32x2{E::pack2(o[0] * inv, o[1] * inv), E::pack2(o[2] * inv, o[3] * inv)};
    }
  }
  if (wave == 0 && hf == 0 && row_ok) p.lse[(int64_t)head * p.n + q_pos0 + l32] = (big_m + fast_log2(big_l)) * kLn2;
}

}  // namespace sattn
