// Backward pass of exact softmax attention on gfx950 (dQ, dK, dV).
//
// For the loss sum(dO * O) with O = softmax(S) V, S = scale * Q K^T:
//   P = exp(S - lse)            (recomputed from the saved per-row lse)
//   dV = P^T dO,  dP = dO V^T,  dS = P (dP - Delta),  Delta_i = dO_i . O_i
//   dQ = scale * dS K,  dK = scale * dS^T Q
// ("Attention algorithms and data movement", lesson 03: differentiate the
// normalized row, probabilities recomputed from the saved normalization
// state; lesson 05: grouped KV heads sum their query heads' gradients.)
//
// Two kernels, no atomics, every sum in a fixed order:
//   bwd_dq_kernel   -- a wave owns 32 queries and walks 64-key K/V tiles
//                      (the forward's walk); it also forms Delta and stores it.
//   bwd_dkdv_roles_kernel (D = 128; causal D = 64) -- two waves of one SIMD own 32 keys
//                      and walk 64-query Q/dO tiles of every query head of
//                      their KV head, one forming P and dV, the other dP, dS
//                      and dK; it runs after the dQ kernel on the same stream
//                      and reads Delta.
//   bwd_dkdv_kernel (D = 32; non-causal D = 64) -- the same walk, one wave per 32 keys
//                      forming both.
// MFMA operand layouts follow the forward: a lane owns one row of the 32x32
// accumulator's columns; operands of the transposed products come from
// ds_read_b64_tr_b16 on the natural [row][d] LDS layout, in the row order
// that the packed probabilities imply.
#pragma once

#include "fwd_kernel.hpp"

namespace sattn {

struct BwdParams {
  const uint16_t* q;    // [B, Hq, N, D]
  const uint16_t* k;    // [B, Hkv, N, D]
  const uint16_t* v;
  const uint16_t* o;    // [B, Hq, N, D]
  const uint16_t* dout; // [B, Hq, N, D]
  const float* lse;     // [B, Hq, N]
  float* delta;         // [B, Hq, N] workspace: written by the dQ kernel
  uint16_t* dq;         // [B, Hq, N, D]
  uint16_t* dk;         // [B, Hkv, N, D]
  uint16_t* dv;
  int hq, hkv, n;
  int nk, off;          // dense layout: keys per slice and the position of query 0
                        // (Nk - Nq: queries are the last Nq tokens; 0 for equal lengths)
  int nqt;              // dQ kernel: query tiles per head (varlen: per longest sequence)
  int pair;             // dQ kernel, batched causal: workgroup j takes query tiles nqt-1-j and j
  int pair_kv;          // dK/dV in two roles, batched causal: workgroup j takes key tiles j and nkt-1-j
  int nkt;              // dK/dV kernel: 128-key tiles per KV head (varlen: per longest sequence)
  // varlen: q, o, dout, dq are [T, Hq, D] and k, v, dk, dv [T, Hkv, D]
  // packed tokens, lse and Delta [Hq, T]; sequence s owns tokens
  // [cu_seqlens[s], cu_seqlens[s+1]) and positions count from its start
  const int32_t* cu_seqlens;
  int nseq, total;
  // sparse (dense layout, Nq = Nk): key j is eligible for query i iff
  // (i - win_left <= j <= i + win_right, a negative bound unlimited) or
  // j < n_global or i < n_global, and block (i / bm_q, j / bm_k) of query
  // head h is active in bmask (if given; h reads bmask + h * bm_hstride,
  // bm_nkb blocks per row), and j <= i when causal
  int win_left, win_right, n_global;
  const uint8_t* bmask;
  int bm_q, bm_k, bm_nkb;
  int64_t bm_hstride;
  float c;              // scale * log2(e)
  float scale;
};

// Row layouts of the backward kernels: [B, H, N, D] slices, packed
// variable-length [T, H, D] sequences, and [B, H, N, D] slices under the
// sparse operator's eligibility.
enum { BWD_DENSE = 0, BWD_VARLEN = 1, BWD_SPARSE = 2 };

// The sparse rule on a block of rows [i0, i1] and keys [j0, j1] (window and
// global tokens only; causality and the block mask are checked apart):
// some pair eligible, every pair eligible, and one pair.
__device__ __forceinline__ bool sparse_any(const BwdParams& p, int i0, int i1, int j0, int j1) {
  const bool win = (p.win_left < 0 || j1 >= i0 - p.win_left) && (p.win_right < 0 || j0 <= i1 + p.win_right);
  return win || j0 < p.n_global || i0 < p.n_global;
}
__device__ __forceinline__ bool sparse_all(const BwdParams& p, int i0, int i1, int j0, int j1) {
  const bool win = (p.win_left < 0 || j0 >= i1 - p.win_left) && (p.win_right < 0 || j1 <= i0 + p.win_right);
  return win || j1 < p.n_global || i1 < p.n_global;
}
__device__ __forceinline__ bool sparse_pair(const BwdParams& p, int i, int j) {
  const bool win = (p.win_left < 0 || j >= i - p.win_left) && (p.win_right < 0 || j <= i + p.win_right);
  return win || j < p.n_global || i < p.n_global;
}
// Block-mask bit of query i and key j for query head h (true without a mask).
__device__ __forceinline__ bool sparse_bit(const BwdParams& p, int h, int i, int j) {
  return !p.bmask || p.bmask[(int64_t)h * p.bm_hstride + (int64_t)(i / p.bm_q) * p.bm_nkb + j / p.bm_k] != 0;
}

// One 64-row tile of a [row][D] tensor into LDS (swizzled like the forward's
// K/V tiles): each wave moves its NI 1 KiB pieces.
template <int D, int NW>
struct TileLoader {
  static constexpr int PPR = D / 8;
  static constexpr int NI = 64 * D * 2 / 1024 / NW;
  static_assert(NI >= 1 && (64 * D * 2) % (1024 * NW) == 0, "tile must split into 1 KiB wave loads");
  uint32_t voff[NI];
  __device__ __forceinline__ void init(int wave, int lane, uint32_t row_bytes) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int slot = (wave * NI + i) * 64 + lane;
      const int key = slot / PPR;
      voff[i] = (uint32_t)key * row_bytes + (uint32_t)(((slot % PPR) ^ swz<D>(key)) * 16);
    }
  }
  __device__ __forceinline__ void issue(__amdgpu_buffer_rsrc_t r, uint32_t soff, uint16_t* dst, int wave_u) const {
#pragma unroll
    for (int i = 0; i < NI; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)(dst + (wave_u * NI + i) * 512),
                                               16, voff[i], soff, 0, 0);
  }
};

// ---------------------------------------------------------------- dQ
// NW waves, 32 queries each: 4, or 8 for the non-causal batched layout at
// D = 128, where each staged K/V tile then serves twice the queries.
template <class E, int D, bool CAUSAL, int LAYOUT, int NW>
__global__ __launch_bounds__(NW * 64, 2) void bwd_dq_kernel(const BwdParams p) {
  constexpr int BM = 32 * NW, BN = 64;
  constexpr int KK = D / 16, KB = BN / 32, DB = D / 32;
  constexpr int TILE = BN * D;  // elements of one K or V tile
  __shared__ __attribute__((aligned(1024))) uint16_t sbuf0[2 * TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t sbuf1[2 * TILE];

  // One query tile of a workgroup (two for batched causal pairs).
  auto run_item = [&](int item) {
    // block -> (query head, query tile); heaviest (causal: longest) query
    // tiles first. Dense: heads contiguous per XCD. Varlen: KV head, then
    // sequence, then query tile, then the query heads of the group, as in the
    // varlen forward. Offsets in elements: qbase is row q_pos0 of q/o/dout/dq,
    // kvbase key 0 of k/v, lbase row q_pos0 of lse/Delta.
    // len: queries of the slice; klen: its keys; off: position of query 0
    int len, klen, off = 0, q_pos0, qh;
    int64_t qbase, kvbase, lbase, q_rs, kv_rs;
    if constexpr (LAYOUT == BWD_VARLEN) {
      const int grp = p.hq / p.hkv;
      const int lin = xcd_linear(blockIdx.x);
      const int per_g = p.nseq * p.nqt * grp;
      const int g = lin / per_g;
      const int r1 = lin % per_g;
      const int sq = r1 / (p.nqt * grp);
      const int r2 = r1 % (p.nqt * grp);
      const int qt = p.nqt - 1 - r2 / grp;
      const int h = g * grp + r2 % grp;
      qh = h;
      // clamp the table so that a malformed one cannot address outside [0, T)
      int a = p.cu_seqlens[sq], e = p.cu_seqlens[sq + 1];
      a = min(max(a, 0), p.total);
      e = min(max(e, a), p.total);
      len = e - a;
      klen = len;
      q_pos0 = qt * BM;
      if (q_pos0 >= len) return;  // uniform over the workgroup
      q_rs = (int64_t)p.hq * D;
      kv_rs = (int64_t)p.hkv * D;
      qbase = (int64_t)(a + q_pos0) * q_rs + (int64_t)h * D;
      kvbase = (int64_t)a * kv_rs + (int64_t)g * D;
      lbase = (int64_t)h * p.total + a + q_pos0;
    } else {
      // batched causal pairs: item 0 the longer tile nqt-1-j, item 1 tile j
      const int lin = xcd_linear(blockIdx.x);
      int slice, qt;
      if (CAUSAL && p.pair) {
        const int npairs = (p.nqt + 1) / 2;
        slice = lin / npairs;
        const int j = lin % npairs;
        qt = item == 0 ? p.nqt - 1 - j : j;
        if (item == 1 && qt == p.nqt - 1 - j) return;   // odd count: the middle tile once
      } else {
        if (item > 0) return;
        slice = lin / p.nqt;   // b * Hq + h
        qt = p.nqt - 1 - lin % p.nqt;
      }
      const int b = slice / p.hq, h = slice % p.hq;
      const int kvs = b * p.hkv + h / (p.hq / p.hkv);
      qh = h;
      len = p.n;
      klen = p.nk;
      off = p.off;
      q_pos0 = qt * BM;
      q_rs = D;
      kv_rs = D;
      qbase = ((int64_t)slice * p.n + q_pos0) * D;
      kvbase = (int64_t)kvs * p.nk * D;
      lbase = (int64_t)slice * p.n + q_pos0;
    }
    const int nq = min(BM, len - q_pos0);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    const int l32 = lane & 31, hf = lane >> 5;
    const int qrow = wave * 32 + l32;
    const bool row_ok = qrow < nq;
    const int my_pos = q_pos0 + off + qrow;
    const bool wave_active = wave * 32 < nq;
    const int wave_last_pos = q_pos0 + off + wave * 32 + 31;

    // this lane's query row: Q and dO as MFMA B operands; Delta = dO . O
    u32x4 qreg[KK], dreg[KK];
    float delta = 0.f;
    {
      const int64_t off = qbase + (int64_t)qrow * q_rs + hf * 8;
  #pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        qreg[kk] = row_ok ? *(const u32x4*)(p.q + off + kk * 16) : u32x4{0, 0, 0, 0};
        dreg[kk] = row_ok ? *(const u32x4*)(p.dout + off + kk * 16) : u32x4{0, 0, 0, 0};
        const u32x4 ov = row_ok ? *(const u32x4*)(p.o + off + kk * 16) : u32x4{0, 0, 0, 0};
  #pragma unroll
        for (int j = 0; j < 4; ++j)
          delta += E::lo(dreg[kk][j]) * E::lo(ov[j]) + E::hi(dreg[kk][j]) * E::hi(ov[j]);
      }
    }
    delta = sum_halves(delta);
    // A row with no eligible key (lse = -inf) has every key masked to -inf
    // below; a reference of +inf keeps its P at exp2(-inf) = 0, not NaN.
    float lse2 = row_ok ? p.lse[lbase + qrow] * kLog2e : 0.f;
    if (lse2 == -INFINITY) lse2 = INFINITY;
    if (row_ok && hf == 0) p.delta[lbase + qrow] = delta;

    f32x16 acc[DB];
  #pragma unroll
    for (int db = 0; db < DB; ++db)
  #pragma unroll
      for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;

    const int k_end = CAUSAL ? min(klen, max(0, q_pos0 + off + BM)) : klen;
    const int ntiles = (k_end + BN - 1) / BN;
    const uint32_t row_bytes = (uint32_t)kv_rs * 2u;
    const __amdgpu_buffer_rsrc_t rk =
        __builtin_amdgcn_make_buffer_rsrc((void*)(p.k + kvbase), (short)0, (int)(k_end * row_bytes), 0x00020000);
    const __amdgpu_buffer_rsrc_t rv =
        __builtin_amdgcn_make_buffer_rsrc((void*)(p.v + kvbase), (short)0, (int)(k_end * row_bytes), 0x00020000);
    TileLoader<D, NW> ld;
    ld.init(wave, lane, row_bytes);
    auto issue_tile = [&](int t, uint16_t* sb) {
      const uint32_t soff = __builtin_amdgcn_readfirstlane((uint32_t)(t * BN) * row_bytes);
      ld.issue(rk, soff, sb, wave_u);
      ld.issue(rv, soff, sb + TILE, wave_u);
    };

    int kofs[KK];
  #pragma unroll
    for (int kk = 0; kk < KK; ++kk) kofs[kk] = l32 * D + (((kk * 2 + hf) ^ swz<D>(l32)) * 8);
    const int g16 = lane >> 4;
    const int tr_key = 4 * (g16 >> 1) + ((lane & 15) >> 2);
    int tofs[2][DB];
  #pragma unroll
    for (int x = 0; x < 2; ++x)
  #pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int d0 = db * 32 + 16 * (g16 & 1) + 4 * (lane & 3);
        const int key = tr_key + 8 * x;
        tofs[x][db] = key * D + (((d0 >> 3) ^ swz<D>(key)) * 8) + (d0 & 7);
      }

    // Key tiles walked: [0, ntiles), or under the sparse operator (no global
    // query among the rows) the global-key prefix [0, npre) and then the
    // window band [band0, band0 + nsteps - npre).
    int npre = 0, band0 = 0, nsteps = ntiles;
    if constexpr (LAYOUT == BWD_SPARSE) {
      if (q_pos0 >= p.n_global) {
        npre = min(ntiles, (p.n_global + BN - 1) / BN);
        const int lo = p.win_left < 0 ? 0 : max(0, q_pos0 - p.win_left) / BN;
        const int hi = p.win_right < 0 ? ntiles : min(ntiles, (q_pos0 + BM - 1 + p.win_right) / BN + 1);
        band0 = max(npre, lo);
        nsteps = npre + max(0, hi - band0);
      }
    }
    auto tile_of = [&](int idx) { return idx < npre ? idx : band0 + (idx - npre); };

    auto step = [&](int idx, const uint16_t* cur, uint16_t* nxt) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      if (idx + 1 < nsteps) issue_tile(tile_of(idx + 1), nxt);
      const int kt0 = tile_of(idx) * BN;
      if (!wave_active || (CAUSAL && kt0 > wave_last_pos)) return;
      bool edge = kt0 + BN > klen || (CAUSAL && kt0 + BN - 1 > q_pos0 + off + wave_u * 32);
      if constexpr (LAYOUT == BWD_SPARSE) {
        // the wave's 32 rows lie in one mask row block and the tile's keys in
        // one key block (block_q % 32 == 0, block_k % 64 == 0)
        const int i0 = q_pos0 + wave_u * 32, i1 = min(i0 + 31, len - 1);
        const int j1 = min(kt0 + BN, klen) - 1;
        if (!sparse_bit(p, qh, i0, kt0) || !sparse_any(p, i0, i1, kt0, j1)) return;
        edge = edge || !sparse_all(p, i0, i1, kt0, j1);
      }
      const uint16_t* sK = cur;
      const uint16_t* sV = cur + TILE;
      // S^T = K Q^T and dP^T = V dO^T (keys x queries, one query per lane)
      f32x16 s[KB], dp[KB];
  #pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
  #pragma unroll
        for (int r = 0; r < 16; ++r) {
          s[kb][r] = 0.f;
          dp[kb][r] = 0.f;
        }
  #pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          s[kb] = E::mfma32(*(const u32x4*)(sK + kofs[kk] + kb * 32 * D), qreg[kk], s[kb]);
          dp[kb] = E::mfma32(*(const u32x4*)(sV + kofs[kk] + kb * 32 * D), dreg[kk], dp[kb]);
        }
      }
      // Ineligible keys: S = -inf, so that P = exp2(-inf) = 0 below. Only
      // tiles that straddle the diagonal, the key tail or a sparse block edge
      // take this pass (a select on every element of every tile nearly
      // doubled the tile's VALU work); the scale is > 0, so -inf stays -inf.
      if (edge) {
        if constexpr (LAYOUT == BWD_SPARSE) {
          // the eligibility rule of sparse_pair, as straight-line selects
          const int wlo = p.win_left < 0 ? INT_MIN : my_pos - p.win_left;
          const int whi = p.win_right < 0 ? INT_MAX : my_pos + p.win_right;
          const int hi = CAUSAL ? min(klen - 1, my_pos) : klen - 1;
          const bool grow = my_pos < p.n_global;
  #pragma unroll
          for (int kb = 0; kb < KB; ++kb)
  #pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = kt0 + kb * 32 + 8 * (r >> 2) + 4 * hf + (r & 3);
              const bool ok = (key <= hi) & (((key >= wlo) & (key <= whi)) | (key < p.n_global) | grow);
              s[kb][r] = ok ? s[kb][r] : -INFINITY;
            }
        } else {
          // the last eligible key, as an offset from this lane's first key of the tile
          const int lim = (CAUSAL ? min(klen - 1, my_pos) : klen - 1) - (kt0 + 4 * hf);
  #pragma unroll
          for (int kb = 0; kb < KB; ++kb)
  #pragma unroll
            for (int r = 0; r < 16; ++r)
              if (kb * 32 + 8 * (r >> 2) + (r & 3) > lim) s[kb][r] = -INFINITY;
        }
      }
      // P = exp2(S c - lse log2 e); dS = P (dP - Delta)
  #pragma unroll
      for (int kb = 0; kb < KB; ++kb)
  #pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float pr = fast_exp2(fmaf(s[kb][r], p.c, -lse2));
          s[kb][r] = pr * (dp[kb][r] - delta);
        }
      // dQ^T += K^T dS^T (16 keys per MFMA; K^T by transposing reads)
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
            const u32x2 a0 = lds_read_tr16(sK + tofs[0][db] + krow);
            const u32x2 a1 = lds_read_tr16(sK + tofs[1][db] + krow);
            acc[db] = E::mfma32(u32x4{a0[0], a0[1], a1[0], a1[1]}, pb, acc[db]);
          }
        }
    };
    if (nsteps > 0) {
      issue_tile(tile_of(0), sbuf0);
      int t = 0;
      for (; t + 1 < nsteps; t += 2) {
        step(t, sbuf0, sbuf1);
        step(t + 1, sbuf1, sbuf0);
      }
      if (t < nsteps) step(t, sbuf0, sbuf1);
    }
    // dQ leaves through the idle tile buffers as whole rows (waves 0-3 in
    // sbuf0, 4-7 in sbuf1), once every wave is done with them
    __syncthreads();
    store_tile_rows<E, D>(acc, p.scale, (wave_u < 4 ? sbuf0 : sbuf1) + (wave_u & 3) * 32 * D,
                          p.dq + qbase + (int64_t)wave_u * 32 * q_rs, q_rs, nq - wave_u * 32);
  };
  constexpr int NITEMS = (LAYOUT == BWD_DENSE && CAUSAL) ? 2 : 1;
#pragma unroll 1
  for (int item = 0; item < NITEMS; ++item) {
    if (item > 0) __syncthreads();   // every wave is done with the previous tile's buffers
    run_item(item);
  }
}

// Work of one dK/dV workgroup: up to 128 keys of one KV head, and the walk
// over the 64-query tiles of every query head of the group that see them.
// Workgroup -> (KV head, key tile): KV heads contiguous per XCD (varlen: KV
// head, then sequence), the keys that see the most queries (causal: the
// earliest) first.
template <int D, bool CAUSAL, int LAYOUT>
struct KvWalk {
  static constexpr bool VARLEN = LAYOUT == BWD_VARLEN;
  static constexpr bool SPARSE = LAYOUT == BWD_SPARSE;
  static constexpr int BNK = 128, BMQ = 64;
  static constexpr int TILE = BMQ * D;   // elements of one Q or dO tile
  int grp;
  int len, qlen, off, k0, g;   // keys and queries of the slice, position of query 0, first key, KV head
  int tok0, bq;                // varlen: first token of the sequence; batched: batch index
  int64_t kvbase, q_rs, kv_rs; // key k0 of k/v/dk/dv in elements; row strides
  int nkeys;                   // keys of this workgroup
  int t_begin, per_head, npre, band0, nsteps;

  // false if the workgroup has no keys for this item (uniform over the
  // workgroup); item 1 exists only for paired batched causal grids
  __device__ __forceinline__ bool init(const BwdParams& p, int item = 0) {
    grp = p.hq / p.hkv;
    off = 0;
    tok0 = 0;
    bq = 0;
    const int lin = xcd_linear(blockIdx.x);
    if constexpr (VARLEN) {
      if (item > 0) return false;
      const int per_g = p.nseq * p.nkt;
      g = lin / per_g;
      const int sq = (lin % per_g) / p.nkt;
      const int kt = lin % p.nkt;
      int a = p.cu_seqlens[sq], e = p.cu_seqlens[sq + 1];
      a = min(max(a, 0), p.total);
      e = min(max(e, a), p.total);
      len = e - a;
      qlen = len;
      tok0 = a;
      k0 = kt * BNK;
      if (k0 >= len) return false;
      q_rs = (int64_t)p.hq * D;
      kv_rs = (int64_t)p.hkv * D;
      kvbase = (int64_t)(a + k0) * kv_rs + (int64_t)g * D;
    } else {
      int kvs, kt;   // kvs = b * Hkv + g
      if (CAUSAL && p.pair_kv) {
        // the longer key tile j (its keys see the most queries), then nkt-1-j
        const int npairs = (p.nkt + 1) / 2;
        kvs = lin / npairs;
        const int j = lin % npairs;
        kt = item == 0 ? j : p.nkt - 1 - j;
        if (item == 1 && kt == j) return false;   // odd count: the middle tile once
      } else {
        if (item > 0) return false;
        kvs = lin / p.nkt;
        kt = lin % p.nkt;
      }
      bq = kvs / p.hkv;
      g = kvs % p.hkv;
      len = p.nk;
      qlen = p.n;
      off = p.off;
      k0 = kt * BNK;
      q_rs = D;
      kv_rs = D;
      kvbase = ((int64_t)kvs * p.nk + k0) * D;
    }
    nkeys = min(BNK, len - k0);
    // query tiles: every query head of the group, causal from the tile
    // holding k0; under the sparse operator (no global key among the keys)
    // only the tiles of global queries [t_begin, t_begin + npre) and then the
    // window band from band0
    t_begin = CAUSAL ? max(0, k0 - off) / BMQ : 0;
    const int nqt = (qlen + BMQ - 1) / BMQ;
    per_head = nqt - t_begin;
    npre = 0;
    band0 = t_begin;
    if constexpr (SPARSE) {
      if (k0 >= p.n_global) {
        const int pre_hi = max(t_begin, min(nqt, (p.n_global + BMQ - 1) / BMQ));
        npre = pre_hi - t_begin;
        const int lo = p.win_right < 0 ? 0 : max(0, k0 - p.win_right) / BMQ;
        const int hi = p.win_left < 0 ? nqt : min(nqt, (k0 + BNK - 1 + p.win_left) / BMQ + 1);
        band0 = max(pre_hi, lo);
        per_head = npre + max(0, hi - band0);
      }
    }
    nsteps = per_head * grp;
    return true;
  }
  // the query tiles of query head hh start at qhead(hh) in q/dout and at
  // lhead(hh) in lse/Delta
  __device__ __forceinline__ int64_t qhead(const BwdParams& p, int hh) const {
    return VARLEN ? (int64_t)tok0 * q_rs + (int64_t)hh * D : ((int64_t)bq * p.hq + hh) * p.n * D;
  }
  __device__ __forceinline__ int64_t lhead(const BwdParams& p, int hh) const {
    return VARLEN ? (int64_t)hh * p.total + tok0 : ((int64_t)bq * p.hq + hh) * p.n;
  }
  // step it: its query head, and its first query
  __device__ __forceinline__ int head(int it) const { return g * grp + it / per_head; }
  __device__ __forceinline__ int q0(int it) const {
    const int i = it % per_head;
    return (i < npre ? t_begin + i : band0 + (i - npre)) * BMQ;
  }
  __device__ __forceinline__ uint32_t row_bytes() const { return (uint32_t)q_rs * 2u; }
  // loads of step it's Q and dO tiles, lse and Delta (wave 0) into sb
  template <int NW>
  __device__ __forceinline__ void issue(const BwdParams& p, const TileLoader<D, NW>& ld, int it, uint16_t* sb,
                                        int wave_u, int lane) const {
    const int hh = head(it);
    const int q0_ = q0(it);
    const int rows = min(BMQ, qlen - q0_);
    const uint32_t rb = row_bytes();
    const int64_t qoff = qhead(p, hh) + (int64_t)q0_ * q_rs;
    const int64_t loff = lhead(p, hh) + q0_;
    const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(p.q + qoff), (short)0, (int)(rows * rb), 0x00020000);
    const __amdgpu_buffer_rsrc_t rd = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(p.dout + qoff), (short)0, (int)(rows * rb), 0x00020000);
#pragma unroll
    for (int r = 0; r < BMQ / 64; ++r) {
      ld.issue(rq, (uint32_t)(r * 64) * rb, sb + r * 64 * D, wave_u);
      ld.issue(rd, (uint32_t)(r * 64) * rb, sb + TILE + r * 64 * D, wave_u);
    }
    if (wave_u == 0) {   // lse and Delta of the tile's rows, 4 bytes per lane
      const __amdgpu_buffer_rsrc_t rl = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(p.lse + loff), (short)0, rows * 4, 0x00020000);
      const __amdgpu_buffer_rsrc_t re = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(p.delta + loff), (short)0, rows * 4, 0x00020000);
#pragma unroll
      for (int r = 0; r < BMQ / 64; ++r) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rl, (__attribute__((address_space(3))) void*)(sb + 2 * TILE + r * 128),
                                                 4, (uint32_t)lane * 4u, (uint32_t)r * 256u, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            re, (__attribute__((address_space(3))) void*)(sb + 2 * TILE + 2 * BMQ + r * 128), 4, (uint32_t)lane * 4u,
            (uint32_t)r * 256u, 0, 0);
      }
    }
  }
};

// ---------------------------------------------------------------- dK, dV
template <class E, int D, bool CAUSAL, int LAYOUT>
__global__ __launch_bounds__(256, 1) void bwd_dkdv_kernel(const BwdParams p) {
  constexpr bool SPARSE = LAYOUT == BWD_SPARSE;
  // queries per step, in 64-row sub-tiles (128 measured no faster); 128 keys per workgroup (KvWalk)
  constexpr int NW = 4, BMQ = 64;
  constexpr int KK = D / 16, DB = D / 32;
  constexpr int TILE = BMQ * D;                 // elements of one Q or dO tile
  constexpr int BUF = 2 * TILE + 2 * BMQ * 2;   // Q, dO, then lse and Delta (fp32)
  __shared__ __attribute__((aligned(1024))) uint16_t sbuf0[BUF];
  __shared__ __attribute__((aligned(1024))) uint16_t sbuf1[BUF];

  KvWalk<D, CAUSAL, LAYOUT> wk;
  if (!wk.init(p)) return;   // uniform over the workgroup
  const int len = wk.len, qlen = wk.qlen, off = wk.off, k0 = wk.k0;
  const int64_t kvbase = wk.kvbase, kv_rs = wk.kv_rs;
  const int nkeys = wk.nkeys;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int l32 = lane & 31, hf = lane >> 5;
  const int krow = wave * 32 + l32;
  const bool key_ok = krow < nkeys;
  const int my_key = k0 + krow;
  const bool wave_active = wave * 32 < nkeys;
  const int wave_first_key = k0 + wave * 32;

  // this lane's key: K and V as MFMA B operands (S = Q K^T, dP = dO V^T)
  u32x4 kreg[KK], vreg[KK];
  {
    const int64_t off = kvbase + (int64_t)krow * kv_rs + hf * 8;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      kreg[kk] = key_ok ? *(const u32x4*)(p.k + off + kk * 16) : u32x4{0, 0, 0, 0};
      vreg[kk] = key_ok ? *(const u32x4*)(p.v + off + kk * 16) : u32x4{0, 0, 0, 0};
    }
  }
  f32x16 adk[DB], adv[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      adk[db][r] = 0.f;
      adv[db][r] = 0.f;
    }

  const int nsteps = wk.nsteps;
  TileLoader<D, NW> ld;
  ld.init(wave, lane, wk.row_bytes());
  auto issue_step = [&](int it, uint16_t* sb) { wk.issue(p, ld, it, sb, wave_u, lane); };

  int aofs[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) aofs[kk] = l32 * D + (((kk * 2 + hf) ^ swz<D>(l32)) * 8);
  const int g16 = lane >> 4;
  const int tr_row = 4 * (g16 >> 1) + ((lane & 15) >> 2);
  int tofs[2][DB];
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int d0 = db * 32 + 16 * (g16 & 1) + 4 * (lane & 3);
      const int row = tr_row + 8 * x;
      tofs[x][db] = row * D + (((d0 >> 3) ^ swz<D>(row)) * 8) + (d0 & 7);
    }

  // Pieces of one 32-query block: S = Q K^T and dP = dO V^T, then
  // P = exp2(S c - lse log2 e) and dS = P (dP - Delta) packed as MFMA B
  // operands, then dV^T += dO^T P and dK^T += Q^T dS.
  auto sd_mfma = [&](const uint16_t* sQ, const uint16_t* sD, int qb, f32x16& s, f32x16& dp) {
    u32x4 qa[KK], da[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      qa[kk] = *(const u32x4*)(sQ + aofs[kk] + qb * 32 * D);
      da[kk] = *(const u32x4*)(sD + aofs[kk] + qb * 32 * D);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s[r] = 0.f;
      dp[r] = 0.f;
    }
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      s = E::mfma32(qa[kk], kreg[kk], s);
      dp = E::mfma32(da[kk], vreg[kk], dp);
    }
  };
  // register r of the 32x32 accumulator holds query row qb*32 + 8*(r/4) +
  // 4*hf + r%4; `edge` masks queries past N and, causal, before the key
  auto probs = [&](const float* sL, const float* sE, int qb, const f32x16& s, const f32x16& dp, u32x4 (&pb)[2],
                   u32x4 (&sb)[2], bool edge, int qb0) {
    f32x4 lse4[4], del4[4];
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      lse4[g4] = *(const f32x4*)(sL + qb * 32 + 8 * g4 + 4 * hf);
      del4[g4] = *(const f32x4*)(sE + qb * 32 + 8 * g4 + 4 * hf);
    }
    f32x16 pr, ds;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float x = fast_exp2(fmaf(s[r], p.c, -lse4[r >> 2][r & 3] * kLog2e));
      if (edge) {
        const int qi = qb0 + 8 * (r >> 2) + 4 * hf + (r & 3);
        if (qi >= qlen || (CAUSAL && my_key > qi + off) || (SPARSE && !sparse_pair(p, qi, my_key))) x = 0.f;
      }
      pr[r] = x;
      ds[r] = x * (dp[r] - del4[r >> 2][r & 3]);
    }
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int o8 = half * 8;
      pb[half] = u32x4{E::pack2(pr[o8 + 0], pr[o8 + 1]), E::pack2(pr[o8 + 2], pr[o8 + 3]),
                       E::pack2(pr[o8 + 4], pr[o8 + 5]), E::pack2(pr[o8 + 6], pr[o8 + 7])};
      sb[half] = u32x4{E::pack2(ds[o8 + 0], ds[o8 + 1]), E::pack2(ds[o8 + 2], ds[o8 + 3]),
                       E::pack2(ds[o8 + 4], ds[o8 + 5]), E::pack2(ds[o8 + 6], ds[o8 + 7])};
    }
  };
  auto dvdk_mfma = [&](const uint16_t* sQ, const uint16_t* sD, int qb, const u32x4 (&pb)[2], const u32x4 (&sb)[2]) {
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int qrow = (qb * 32 + half * 16) * D;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const u32x2 a0 = lds_read_tr16(sD + tofs[0][db] + qrow);
        const u32x2 a1 = lds_read_tr16(sD + tofs[1][db] + qrow);
        adv[db] = E::mfma32(u32x4{a0[0], a0[1], a1[0], a1[1]}, pb[half], adv[db]);
        const u32x2 c0 = lds_read_tr16(sQ + tofs[0][db] + qrow);
        const u32x2 c1 = lds_read_tr16(sQ + tofs[1][db] + qrow);
        adk[db] = E::mfma32(u32x4{c0[0], c0[1], c1[0], c1[1]}, sb[half], adk[db]);
      }
    }
  };

  auto step = [&](int it, const uint16_t* cur, uint16_t* nxt) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (it + 1 < nsteps) issue_step(it + 1, nxt);
    const int q0 = wk.q0(it);
    const int hh = wk.head(it);
    if (!wave_active) return;
    // sparse: need / no mask needed for 32-query block qb0 against the wave's
    // keys (one mask row block, one key block)
    const int wkey1 = min(wave_first_key + 31, len - 1);
    auto blk_need = [&](int qb0) {
      return qb0 < qlen && sparse_bit(p, hh, qb0, wave_first_key) &&
             sparse_any(p, qb0, min(qb0 + 31, qlen - 1), wave_first_key, wkey1);
    };
    auto blk_full = [&](int qb0) {
      return blk_need(qb0) && sparse_all(p, qb0, min(qb0 + 31, qlen - 1), wave_first_key, wkey1);
    };
    const uint16_t* sQ = cur;
    const uint16_t* sD = cur + TILE;
    const float* sL = reinterpret_cast<const float*>(cur + 2 * TILE);
    const float* sE = sL + BMQ;
    // Steps whose queries all exist and all come at or after every key of
    // the wave need no mask: one branch-free body in which the second
    // block's S/dP products overlap the first block's exps, and the first
    // block's dV/dK products the second block's.
    if (q0 + BMQ <= qlen && (!CAUSAL || q0 + off >= wave_first_key + 31) &&
        (!SPARSE || (blk_full(q0) && blk_full(q0 + 32)))) {
      static_assert(BMQ == 64, "the unmasked body takes two 32-query blocks");
      f32x16 s0, dp0, s1, dp1;
      u32x4 pb0[2], sb0[2], pb1[2], sb1[2];
      sd_mfma(sQ, sD, 0, s0, dp0);
      __builtin_amdgcn_sched_barrier(0);
      // The wave issues in order and an MFMA occupies the matrix unit for
      // several cycles, so VALU work placed between MFMAs runs beside them.
      sd_mfma(sQ, sD, 1, s1, dp1);
      probs(sL, sE, 0, s0, dp0, pb0, sb0, false, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 24, 0);   // operand and lse/Delta reads
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);  // then VALU
      }
      __builtin_amdgcn_sched_barrier(0);
      dvdk_mfma(sQ, sD, 0, pb0, sb0);
      probs(sL, sE, 1, s1, dp1, pb1, sb1, false, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 16, 0);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
      dvdk_mfma(sQ, sD, 1, pb1, sb1);
      return;
    }
    // Other steps, block by block: blocks wholly before the wave's keys are
    // skipped; blocks that straddle them or the query tail are masked.
#pragma unroll
    for (int qb = 0; qb < BMQ / 32; ++qb) {
      const int qb0 = q0 + qb * 32;
      if (CAUSAL && qb0 + off + 31 < wave_first_key) continue;   // every query of the block precedes the wave's keys
      if (SPARSE && !blk_need(qb0)) continue;
      f32x16 s, dp;
      u32x4 pb[2], sb[2];
      sd_mfma(sQ, sD, qb, s, dp);
      probs(sL, sE, qb, s, dp, pb, sb,
            qb0 + 32 > qlen || (CAUSAL && qb0 + off < wave_first_key + 31) || (SPARSE && !blk_full(qb0)), qb0);
      dvdk_mfma(sQ, sD, qb, pb, sb);
    }
  };
  if (nsteps > 0) {
    issue_step(0, sbuf0);
    int it = 0;
    for (; it + 1 < nsteps; it += 2) {
      step(it, sbuf0, sbuf1);
      step(it + 1, sbuf1, sbuf0);
    }
    if (it < nsteps) step(it, sbuf0, sbuf1);
  }
  // dK and dV leave through the idle buffers as whole rows (dK in sbuf0,
  // dV in sbuf1, a 32-row slice per wave), once every wave is done with them
  __syncthreads();
  store_tile_rows<E, D>(adk, p.scale, sbuf0 + wave_u * 32 * D, p.dk + kvbase + (int64_t)wave_u * 32 * kv_rs, kv_rs,
                        nkeys - wave_u * 32);
  store_tile_rows<E, D>(adv, 1.0f, sbuf1 + wave_u * 32 * D, p.dv + kvbase + (int64_t)wave_u * 32 * kv_rs, kv_rs,
                        nkeys - wave_u * 32);
}


// ---------------------------------------------------------------- dK, dV in two roles (D = 128)
// 8 waves and 128 keys per workgroup; waves w and w + 4, the two waves of one
// SIMD, own the same 32 keys. Wave w (the P role) forms S = Q K^T, the
// probabilities P and dV^T += dO^T P; wave w + 4 (the dS role) forms
// dP = dO V^T, dS = P (dP - Delta) with P taken from its partner through
// LDS, and dK^T += Q^T dS. A 64-query step has two phases split by a
// barrier: S and P beside dP, then dV beside dS and dK, so each wave of a
// SIMD issues 16 MFMAs per 32-query block in each phase and one wave's
// exponentials and dS arithmetic run beside the other's MFMAs. P goes through
// LDS in fp32, so every value and every accumulation order is the one-wave
// kernel's (bwd_dkdv_kernel), bit for bit.
template <class E, int D, bool CAUSAL, int LAYOUT>
__global__ __launch_bounds__(512, 1) void bwd_dkdv_roles_kernel(const BwdParams p) {
  constexpr bool SPARSE = LAYOUT == BWD_SPARSE;
  constexpr int NW = 8, BMQ = 64;   // 128 keys per workgroup (KvWalk)
  constexpr int KK = D / 16, DB = D / 32;
  constexpr int TILE = BMQ * D;                 // elements of one Q or dO tile
  constexpr int BUF = 2 * TILE + 2 * BMQ * 2;   // Q, dO, then lse and Delta (fp32)
  static_assert(D == 64 || D == 128, "two-role layout: 8 waves of 32 keys, D = 64 or 128");
  __shared__ __attribute__((aligned(1024))) uint16_t sbuf0[BUF];
  __shared__ __attribute__((aligned(1024))) uint16_t sbuf1[BUF];
  // P of the current step: [key block][32-query block][register group][lane]
  __shared__ __attribute__((aligned(16))) f32x4 pex[4][2][4][64];

  // Batched causal grids at D = 128 pair key tiles (j, nkt-1-j), so that
  // every workgroup walks about the same number of query steps.
  constexpr int NITEMS = (LAYOUT == BWD_DENSE && CAUSAL && D == 128) ? 2 : 1;
#pragma unroll 1
  for (int item = 0; item < NITEMS; ++item) {
    if (item > 0) __syncthreads();   // the previous item's stores have left the tile buffers
    KvWalk<D, CAUSAL, LAYOUT> wk;
    if (!wk.init(p, item)) continue;   // uniform over the workgroup
    const int len = wk.len, qlen = wk.qlen, off = wk.off, k0 = wk.k0;
    const int64_t kvbase = wk.kvbase, kv_rs = wk.kv_rs;
    const int nkeys = wk.nkeys;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    const int l32 = lane & 31, hf = lane >> 5;
    const bool role_p = wave_u < 4;
    const int kw = wave_u & 3;                    // the pair's 32-key block
    const int krow = kw * 32 + l32;
    const bool key_ok = krow < nkeys;
    const int my_key = k0 + krow;
    const bool wave_active = kw * 32 < nkeys;
    const int wave_first_key = k0 + kw * 32;

    const int nsteps = wk.nsteps;
    TileLoader<D, NW> ld;
    ld.init(wave, lane, wk.row_bytes());
    auto issue_step = [&](int it, uint16_t* sb) { wk.issue(p, ld, it, sb, wave_u, lane); };

    int aofs[KK];
  #pragma unroll
    for (int kk = 0; kk < KK; ++kk) aofs[kk] = l32 * D + (((kk * 2 + hf) ^ swz<D>(l32)) * 8);
    const int g16 = lane >> 4;
    const int tr_row = 4 * (g16 >> 1) + ((lane & 15) >> 2);
    int tofs[2][DB];
  #pragma unroll
    for (int x = 0; x < 2; ++x)
  #pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int d0 = db * 32 + 16 * (g16 & 1) + 4 * (lane & 3);
        const int row = tr_row + 8 * x;
        tofs[x][db] = row * D + (((d0 >> 3) ^ swz<D>(row)) * 8) + (d0 & 7);
      }


    // Which 32-query blocks of a step a pair computes, and which need the
    // element mask (queries past the end; causal: a query before a key of the
    // pair; sparse: a pair the rule drops). Both roles take the same decisions.
    const int wkey1 = min(wave_first_key + 31, len - 1);
    auto blk_need = [&](int hh, int qb0) {
      if (CAUSAL && qb0 + off + 31 < wave_first_key) return false;   // every query precedes the keys
      if constexpr (SPARSE)
        return qb0 < qlen && sparse_bit(p, hh, qb0, wave_first_key) &&
               sparse_any(p, qb0, min(qb0 + 31, qlen - 1), wave_first_key, wkey1);
      return true;
    };
    auto blk_edge = [&](int qb0) {
      return qb0 + 32 > qlen || (CAUSAL && qb0 + off < wave_first_key + 31) ||
             (SPARSE && !sparse_all(p, qb0, min(qb0 + 31, qlen - 1), wave_first_key, wkey1));
    };
    // A operand of S = Q K^T / dP = dO V^T: 32 rows of the tile, k-steps of 16 d
    auto rows_mfma = [&](const uint16_t* sT, int qb, const u32x4 (&breg)[KK], f32x16& acc) {
      u32x4 a[KK];
  #pragma unroll
      for (int kk = 0; kk < KK; ++kk) a[kk] = *(const u32x4*)(sT + aofs[kk] + qb * 32 * D);
  #pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] = 0.f;
  #pragma unroll
      for (int kk = 0; kk < KK; ++kk) acc = E::mfma32(a[kk], breg[kk], acc);
    };
    // acc^T += T^T X for one 32-query block: T^T from transposing reads of the
    // tile, X the packed block (16 queries per MFMA)
    auto tr_mfma = [&](const uint16_t* sT, int qb, const u32x4 (&x)[2], f32x16 (&acc)[DB]) {
  #pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int qrow = (qb * 32 + half * 16) * D;
  #pragma unroll
        for (int db = 0; db < DB; ++db) {
          const u32x2 a0 = lds_read_tr16(sT + tofs[0][db] + qrow);
          const u32x2 a1 = lds_read_tr16(sT + tofs[1][db] + qrow);
          acc[db] = E::mfma32(u32x4{a0[0], a0[1], a1[0], a1[1]}, x[half], acc[db]);
        }
      }
    };
    auto pack16 = [&](const f32x16& v, u32x4 (&x)[2]) {
  #pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int o8 = half * 8;
        x[half] = u32x4{E::pack2(v[o8 + 0], v[o8 + 1]), E::pack2(v[o8 + 2], v[o8 + 3]),
                        E::pack2(v[o8 + 4], v[o8 + 5]), E::pack2(v[o8 + 6], v[o8 + 7])};
      }
    };

    f32x16 acc[DB];   // dV (P role) or dK (dS role), transposed: [d][key]
  #pragma unroll
    for (int db = 0; db < DB; ++db)
  #pragma unroll
      for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;
    if (nsteps > 0) issue_step(0, sbuf0);

    if (role_p) {
      // ---- P role: K as the B operand of S = Q K^T
      u32x4 kreg[KK];
      {
        const int64_t o_ = kvbase + (int64_t)krow * kv_rs + hf * 8;
  #pragma unroll
        for (int kk = 0; kk < KK; ++kk) kreg[kk] = key_ok ? *(const u32x4*)(p.k + o_ + kk * 16) : u32x4{0, 0, 0, 0};
      }
      auto step = [&](int it, const uint16_t* cur, uint16_t* nxt) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();   // tile it visible; every wave is done with tile it-1 and the previous P
        if (it + 1 < nsteps) issue_step(it + 1, nxt);
        const int q0 = wk.q0(it);
        const int hh = wk.head(it);
        const uint16_t* sQ = cur;
        const uint16_t* sD = cur + TILE;
        const float* sL = reinterpret_cast<const float*>(cur + 2 * TILE);
        u32x4 pb[2][2];
        // P = exp2(S c - lse log2 e) of block qb in place, masked on edge
        // blocks, and to LDS for the partner
        auto probs = [&](int qb, int qb0, f32x16& s, auto edge_tag) {
          constexpr bool EDGE = decltype(edge_tag)::value;
  #pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const f32x4 l4 = *(const f32x4*)(sL + qb * 32 + 8 * g4 + 4 * hf);
  #pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int r = g4 * 4 + i;
              float x = fast_exp2(fmaf(s[r], p.c, -l4[i] * kLog2e));
              if constexpr (EDGE) {
                const int qi = qb0 + 8 * g4 + 4 * hf + i;
                if (qi >= qlen || (CAUSAL && my_key > qi + off) || (SPARSE && !sparse_pair(p, qi, my_key))) x = 0.f;
              }
              s[r] = x;
            }
            pex[kw][qb][g4][lane] = f32x4{s[g4 * 4 + 0], s[g4 * 4 + 1], s[g4 * 4 + 2], s[g4 * 4 + 3]};
          }
        };
        if (wave_active) {
  #pragma unroll
          for (int qb = 0; qb < 2; ++qb) {
            const int qb0 = q0 + qb * 32;
            if (!blk_need(hh, qb0)) continue;
            f32x16 s;
            rows_mfma(sQ, qb, kreg, s);
            if (blk_edge(qb0)) probs(qb, qb0, s, std::true_type{});
            else probs(qb, qb0, s, std::false_type{});
            pack16(s, pb[qb]);
          }
        }
        __syncthreads();   // P of both blocks in LDS
        if (wave_active) {
  #pragma unroll
          for (int qb = 0; qb < 2; ++qb)
            if (blk_need(hh, q0 + qb * 32)) tr_mfma(sD, qb, pb[qb], acc);   // dV^T += dO^T P
        }
      };
      int it = 0;
      for (; it + 1 < nsteps; it += 2) {
        step(it, sbuf0, sbuf1);
        step(it + 1, sbuf1, sbuf0);
      }
      if (it < nsteps) step(it, sbuf0, sbuf1);
      __syncthreads();   // every wave is done with the tile buffers, which stage the stores
      store_tile_rows<E, D>(acc, 1.0f, sbuf0 + kw * 32 * D, p.dv + kvbase + (int64_t)kw * 32 * kv_rs, kv_rs,
                            nkeys - kw * 32);
    } else {
      // ---- dS role: V as the B operand of dP = dO V^T
      u32x4 vreg[KK];
      {
        const int64_t o_ = kvbase + (int64_t)krow * kv_rs + hf * 8;
  #pragma unroll
        for (int kk = 0; kk < KK; ++kk) vreg[kk] = key_ok ? *(const u32x4*)(p.v + o_ + kk * 16) : u32x4{0, 0, 0, 0};
      }
      auto step = [&](int it, const uint16_t* cur, uint16_t* nxt) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (it + 1 < nsteps) issue_step(it + 1, nxt);
        const int q0 = wk.q0(it);
        const int hh = wk.head(it);
        const uint16_t* sQ = cur;
        const uint16_t* sD = cur + TILE;
        const float* sE = reinterpret_cast<const float*>(cur + 2 * TILE) + BMQ;
        f32x16 dp[2];
        if (wave_active) {
  #pragma unroll
          for (int qb = 0; qb < 2; ++qb)
            if (blk_need(hh, q0 + qb * 32)) rows_mfma(sD, qb, vreg, dp[qb]);
        }
        __syncthreads();   // the partner's P of both blocks in LDS
        // dS = P (dP - Delta) of block qb, packed
        auto dscores = [&](int qb, u32x4 (&sb)[2]) {
          f32x16 ds;
  #pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const f32x4 pr = pex[kw][qb][g4][lane];
            const f32x4 d4 = *(const f32x4*)(sE + qb * 32 + 8 * g4 + 4 * hf);
  #pragma unroll
            for (int i = 0; i < 4; ++i) ds[g4 * 4 + i] = pr[i] * (dp[qb][g4 * 4 + i] - d4[i]);
          }
          pack16(ds, sb);
        };
        if (wave_active) {
  #pragma unroll
          for (int qb = 0; qb < 2; ++qb) {
            if (!blk_need(hh, q0 + qb * 32)) continue;
            u32x4 sb[2];
            dscores(qb, sb);
            tr_mfma(sQ, qb, sb, acc);   // dK^T += Q^T dS
          }
        }
      };
      int it = 0;
      for (; it + 1 < nsteps; it += 2) {
        step(it, sbuf0, sbuf1);
        step(it + 1, sbuf1, sbuf0);
      }
      if (it < nsteps) step(it, sbuf0, sbuf1);
      __syncthreads();
      store_tile_rows<E, D>(acc, p.scale, sbuf1 + kw * 32 * D, p.dk + kvbase + (int64_t)kw * 32 * kv_rs, kv_rs,
                            nkeys - kw * 32);
    }
  }
}

}  // namespace sattn
