// Streaming attention forward kernel for gfx950 (CDNA4).
//
// One workgroup owns BM = 32 * NW query rows of one (batch, head) slice and
// walks the K/V keys of that slice in tiles of BN keys, keeping the mergeable
// softmax state (running max m, rescaled exp-sum l, rescaled numerator acc)
// in registers, so the score matrix is never stored ("Intermediate and
// advanced extension", workshop table, streaming-attention row; "Logic review
// before implementation": numerator and denominator are both rescaled).
//
// Layout of the work inside a wave (64 lanes, MFMA 32x32x16, fp32 accumulate):
//   * Scores are formed transposed, S^T = K Q^T: the K tile (A operand) comes
//     from LDS, Q^T (B operand) stays in VGPRs for the whole kernel. In the
//     32x32 accumulator a lane holds 16 keys of ONE query (query = lane % 32),
//     so the row max and row sum are in-register reductions plus one exchange
//     with lane ^ 32.
//   * The output is formed transposed too, O^T = V^T P^T: P^T is the B
//     operand and is taken straight from the score registers (no shuffles);
//     V^T (A operand) is read from an LDS tile that is stored transposed
//     ([d][key]). The output accumulator again gives each lane one query, so
//     the rescale factor of a query never leaves its lane.
//   * K/V tiles are fetched from HBM with 16-byte loads into registers one
//     tile ahead (software prefetch) and written to LDS between barriers.
//   * Causal: key tiles that start after a wave's last query are skipped, not
//     masked; the mask (key > query, diagonal kept) runs only on tiles that
//     straddle the diagonal or the key tail.
#pragma once

#include "common.hpp"

namespace sattn {

enum { MODE_DENSE = 0, MODE_VARLEN = 1, MODE_SPLIT = 2 };

struct FwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  float* part_m;
  float* part_l;
  float* part_acc;
  const int32_t* cu_seqlens;
  int heads;       // dense: B*H; split: B*Hq
  int hq, hkv;     // query heads, KV heads (varlen, split)
  int n;           // dense: N; split: Nq
  int nk;          // split: Nk
  int chunk;       // split: keys per chunk
  int nchunks;     // split: C
  int nqt;         // query tiles per slice (dense/split) or per longest sequence (varlen)
  int nseq;        // varlen: S
  int total;       // varlen: T
  float c;         // scale * log2(e)
};

// Where one workgroup's rows and keys live.
struct Work {
  const uint16_t* q;   // row 0 of this query tile
  const uint16_t* k;   // key 0 of the slice
  const uint16_t* v;
  uint16_t* o;         // row 0 of this query tile
  float* lse;          // lse of row 0 of this query tile (stride 1 per row)
  int64_t q_rs;        // row strides in elements
  int64_t kv_rs;
  int q_pos0;          // logical position of row 0
  int nq;              // valid rows in this tile
  int k_begin, k_end;  // keys [k_begin, k_end) of the slice
  int64_t part_row0;   // split: index (slice_row * C + c) of row 0
};

template <int D, int BM, bool CAUSAL, int MODE>
__device__ __forceinline__ bool decode_work(const FwdParams& p, Work& w) {
  const int bid = blockIdx.x;
  if constexpr (MODE == MODE_DENSE) {
    // Heaviest query tiles first (they have the most key tiles when causal);
    // consecutive block ids are different heads of the same query tile.
    const int qt = p.nqt - 1 - bid / p.heads;
    const int head = bid % p.heads;
    const int64_t base = (int64_t)head * p.n * D;
    w.q_pos0 = qt * BM;
    w.nq = min(BM, p.n - w.q_pos0);
    w.q = p.q + base + (int64_t)w.q_pos0 * D;
    w.o = p.o + base + (int64_t)w.q_pos0 * D;
    w.k = p.k + base;
    w.v = p.v + base;
    w.q_rs = D;
    w.kv_rs = D;
    w.lse = p.lse + (int64_t)head * p.n + w.q_pos0;
    w.k_begin = 0;
    w.k_end = CAUSAL ? min(p.n, w.q_pos0 + BM) : p.n;
    return w.nq > 0;
  } else if constexpr (MODE == MODE_VARLEN) {
    const int per_tile = p.nseq * p.hq;
    const int qt = p.nqt - 1 - bid / per_tile;
    const int rem = bid % per_tile;
    const int s = rem / p.hq;
    const int h = rem % p.hq;
    // Clamp the table so that a malformed one cannot address outside [0, T).
    int a = p.cu_seqlens[s];
    int b = p.cu_seqlens[s + 1];
    a = min(max(a, 0), p.total);
    b = min(max(b, a), p.total);
    const int len = b - a;
    w.q_pos0 = qt * BM;
    if (w.q_pos0 >= len) return false;
    w.nq = min(BM, len - w.q_pos0);
    const int g = h / (p.hq / p.hkv);
    w.q_rs = (int64_t)p.hq * D;
    w.kv_rs = (int64_t)p.hkv * D;
    w.q = p.q + (int64_t)(a + w.q_pos0) * w.q_rs + (int64_t)h * D;
    w.o = p.o + (int64_t)(a + w.q_pos0) * w.q_rs + (int64_t)h * D;
    w.k = p.k + (int64_t)a * w.kv_rs + (int64_t)g * D;
    w.v = p.v + (int64_t)a * w.kv_rs + (int64_t)g * D;
    w.lse = p.lse + (int64_t)h * p.total + a + w.q_pos0;
    w.k_begin = 0;
    w.k_end = CAUSAL ? min(len, w.q_pos0 + BM) : len;
    return true;
  } else {
    // Split-KV: block id -> (slice, query tile, chunk), chunk fastest.
    const int c = bid % p.nchunks;
    const int rest = bid / p.nchunks;
    const int qt = rest % p.nqt;
    const int slice = rest / p.nqt;          // b * Hq + h
    const int b = slice / p.hq;
    const int h = slice % p.hq;
    const int g = h / (p.hq / p.hkv);
    w.q_pos0 = qt * BM;
    w.nq = min(BM, p.n - w.q_pos0);
    w.q = p.q + ((int64_t)slice * p.n + w.q_pos0) * D;
    w.o = nullptr;
    w.lse = nullptr;
    const int64_t kvbase = ((int64_t)b * p.hkv + g) * p.nk * D;
    w.k = p.k + kvbase;
    w.v = p.v + kvbase;
    w.q_rs = D;
    w.kv_rs = D;
    w.k_begin = c * p.chunk;
    w.k_end = min(p.nk, w.k_begin + p.chunk);
    w.part_row0 = ((int64_t)slice * p.n + w.q_pos0) * p.nchunks + c;
    return w.nq > 0 && w.k_begin < w.k_end;
  }
}

template <class E, int D, int BN, int NW, bool CAUSAL, int MODE>
__global__ __launch_bounds__(NW * 64) void fwd_kernel(const FwdParams p) {
  constexpr int NT = NW * 64;
  constexpr int BM = NW * 32;
  constexpr int KP = D + 8;      // K tile row pitch (elements): spreads rows over banks
  constexpr int VP = BN + 8;     // V^T tile row pitch (elements)
  constexpr int KK = D / 16;     // MFMA k-steps of Q K^T
  constexpr int KB = BN / 32;    // 32-key blocks per tile
  constexpr int DB = D / 32;     // 32-wide d blocks of the output
  constexpr int TPR = D / 8;     // 16-byte pieces per row
  constexpr int KU = BN * TPR;   // K tile load units (one 16-byte piece each)
  constexpr int VU = (BN / 4) * TPR;  // V tile load units (4 keys x 16 bytes each)
  constexpr int KLOADS = (KU + NT - 1) / NT;
  constexpr int VLOADS = (VU + NT - 1) / NT;
  static_assert(D % 32 == 0 && BN % 32 == 0, "tile shape");

  __shared__ __attribute__((aligned(16))) uint16_t sK[BN * KP];
  __shared__ __attribute__((aligned(16))) uint16_t sV[D * VP];

  Work w;
  if (!decode_work<D, BM, CAUSAL, MODE>(p, w)) return;  // uniform over the workgroup

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hf = lane >> 5;

  // Q^T operand: this lane's query row, 8 consecutive d per k-step.
  const int qrow = wave * 32 + l32;
  const bool row_ok = qrow < w.nq;
  u32x4 qreg[KK];
  {
    const uint16_t* qp = w.q + (int64_t)qrow * w.q_rs + hf * 8;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      qreg[kk] = row_ok ? *(const u32x4*)(qp + kk * 16) : u32x4{0, 0, 0, 0};
  }

  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;
  float m = -INFINITY;  // running max, log2 units (score * scale * log2 e)
  float l = 0.f;        // this lane's part of the rescaled exp-sum

  const int my_pos = w.q_pos0 + qrow;
  const int wave_first_pos = w.q_pos0 + wave * 32;
  const int wave_last_pos = wave_first_pos + 31;
  const bool wave_active = wave * 32 < w.nq;
  const float c = p.c;

  const int ntiles = (w.k_end - w.k_begin + BN - 1) / BN;

  u32x4 kst[KLOADS];
  u32x4 vst[VLOADS][4];

  auto gload = [&](int t) {
    const int kbase = w.k_begin + t * BN;
#pragma unroll
    for (int i = 0; i < KLOADS; ++i) {
      const int u = tid + i * NT;
      const int key = u / TPR, piece = u % TPR;
      const int j = kbase + key;
      kst[i] = (u < KU && j < w.k_end) ? *(const u32x4*)(w.k + (int64_t)j * w.kv_rs + piece * 8)
                                       : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < VLOADS; ++i) {
      const int u = tid + i * NT;
      const int grp = u / TPR, piece = u % TPR;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = kbase + grp * 4 + r;
        vst[i][r] = (u < VU && j < w.k_end)
                        ? *(const u32x4*)(w.v + (int64_t)j * w.kv_rs + piece * 8)
                        : u32x4{0, 0, 0, 0};
      }
    }
  };

  auto sstore = [&]() {
#pragma unroll
    for (int i = 0; i < KLOADS; ++i) {
      const int u = tid + i * NT;
      if (u < KU) {
        const int key = u / TPR, piece = u % TPR;
        *(u32x4*)(sK + key * KP + piece * 8) = kst[i];
      }
    }
#pragma unroll
    for (int i = 0; i < VLOADS; ++i) {
      const int u = tid + i * NT;
      if (u < VU) {
        const int grp = u / TPR, piece = u % TPR;
        // 4 keys x 8 d -> 8 rows of V^T, 4 consecutive keys each.
#pragma unroll
        for (int wd = 0; wd < 4; ++wd) {
          const int d = piece * 8 + wd * 2;
          u32x2 even = {pack_lo16(vst[i][0][wd], vst[i][1][wd]), pack_lo16(vst[i][2][wd], vst[i][3][wd])};
          u32x2 odd = {pack_hi16(vst[i][0][wd], vst[i][1][wd]), pack_hi16(vst[i][2][wd], vst[i][3][wd])};
          *(u32x2*)(sV + d * VP + grp * 4) = even;
          *(u32x2*)(sV + (d + 1) * VP + grp * 4) = odd;
        }
      }
    }
  };

  if (ntiles > 0) gload(0);
  for (int t = 0; t < ntiles; ++t) {
    __syncthreads();  // every wave is done reading the previous tile
    sstore();
    __syncthreads();
    if (t + 1 < ntiles) gload(t + 1);  // next tile's HBM reads overlap this tile's math

    const int kt0 = w.k_begin + t * BN;
    const bool skip = !wave_active || (CAUSAL && kt0 > wave_last_pos);
    if (skip) continue;

    // ---- S^T = K Q^T for BN keys x 32 queries
    f32x16 s[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const u32x4 a = *(const u32x4*)(sK + (kb * 32 + l32) * KP + kk * 16 + hf * 8);
        s[kb] = E::mfma32(a, qreg[kk], s[kb]);
      }
    }

    // ---- mask: key tail, and keys after the query (diagonal kept)
    const bool tail = kt0 + BN > w.k_end;
    const bool diag = CAUSAL && (kt0 + BN - 1 > wave_first_pos);
    if (tail || diag) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kt0 + kb * 32 + 8 * (r >> 2) + 4 * hf + (r & 3);
          const bool bad = (key >= w.k_end) || (CAUSAL && key > my_pos);
          if (bad) s[kb][r] = -INFINITY;
        }
    }

    // ---- online softmax update (fp32)
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = fmaxf(mx, xor32(mx));
    const float m_new = fmaxf(m, mx * c);
    const float alpha = fast_exp2(m - m_new);
    m = m_new;
    float rs = 0.f;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pv = fast_exp2(fmaf(s[kb][r], c, -m_new));
        s[kb][r] = pv;
        rs += pv;
      }
    l = l * alpha + rs;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;

    // ---- O^T += V^T P^T, 16 keys per MFMA
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int o8 = half * 8;
        const u32x4 pb = {E::pack2(s[kb][o8 + 0], s[kb][o8 + 1]), E::pack2(s[kb][o8 + 2], s[kb][o8 + 3]),
                          E::pack2(s[kb][o8 + 4], s[kb][o8 + 5]), E::pack2(s[kb][o8 + 6], s[kb][o8 + 7])};
        const int key0 = kb * 32 + half * 16 + 4 * hf;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const uint16_t* vrow = sV + (db * 32 + l32) * VP + key0;
          const u32x2 a0 = *(const u32x2*)(vrow);
          const u32x2 a1 = *(const u32x2*)(vrow + 8);
          acc[db] = E::mfma32(u32x4{a0[0], a0[1], a1[0], a1[1]}, pb, acc[db]);
        }
      }
  }

  if (!wave_active) return;
  const float lt = l + xor32(l);  // both halves of the wave hold partial sums of one query

  if constexpr (MODE != MODE_SPLIT) {
    if (!row_ok) return;
    const float inv = 1.f / lt;
    uint16_t* op = w.o + (int64_t)qrow * w.q_rs;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = db * 32 + 8 * g4 + 4 * hf;
        const u32x2 outv = {E::pack2(acc[db][g4 * 4 + 0] * inv, acc[db][g4 * 4 + 1] * inv),
                            E::pack2(acc[db][g4 * 4 + 2] * inv, acc[db][g4 * 4 + 3] * inv)};
        *(u32x2*)(op + d) = outv;
      }
    if (hf == 0) w.lse[qrow] = (m + fast_log2(lt)) * kLn2;
  } else {
    if (!row_ok) return;
    const int64_t prow = w.part_row0 + (int64_t)qrow * p.nchunks;
    float* pa = p.part_acc + prow * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = db * 32 + 8 * g4 + 4 * hf;
        *(f32x4*)(pa + d) = f32x4{acc[db][g4 * 4 + 0], acc[db][g4 * 4 + 1], acc[db][g4 * 4 + 2],
                                  acc[db][g4 * 4 + 3]};
      }
    if (hf == 0) {
      p.part_m[prow] = m * kLn2;  // natural-log units of the scaled score
      p.part_l[prow] = lt;
    }
  }
}

// Merge of split-KV partial states: one wave per row, partials summed in
// ascending chunk order ("Attention algorithms and data movement", lesson 01).
template <class E, int D>
__global__ __launch_bounds__(256) void merge_kernel(const float* __restrict__ pm, const float* __restrict__ pl,
                                                    const float* __restrict__ pacc, int64_t rows, int nchunks,
                                                    uint16_t* __restrict__ o, float* __restrict__ lse) {
  constexpr int PER = D >= 64 ? D / 64 : 1;  // d values per lane
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const bool lane_ok = lane * PER < D;
  const float* rm = pm + row * nchunks;
  const float* rl = pl + row * nchunks;
  float big_m = -INFINITY;
  for (int ch = 0; ch < nchunks; ++ch) big_m = fmaxf(big_m, rm[ch]);
  uint16_t* orow = o + row * D;
  if (big_m == -INFINITY) {  // every partial empty: O = 0, lse = -inf
    if (lane_ok)
      for (int e = 0; e < PER; ++e) orow[lane * PER + e] = 0;
    if (lane == 0) lse[row] = -INFINITY;
    return;
  }
  float big_l = 0.f;
  float a[PER];
  for (int e = 0; e < PER; ++e) a[e] = 0.f;
  for (int ch = 0; ch < nchunks; ++ch) {
    const float mc = rm[ch];
    const float wgt = (mc == -INFINITY) ? 0.f : expf(mc - big_m);
    big_l += wgt * rl[ch];
    if (lane_ok) {
      const float* src = pacc + (row * nchunks + ch) * D + lane * PER;
      for (int e = 0; e < PER; ++e) a[e] += wgt * src[e];
    }
  }
  const float inv = 1.f / big_l;
  if (lane_ok) {
    if constexpr (PER == 2) {
      *(uint32_t*)(orow + lane * 2) = E::pack2(a[0] * inv, a[1] * inv);
    } else {
      for (int e = 0; e < PER; ++e) orow[lane * PER + e] = (uint16_t)(E::pack2(a[e] * inv, 0.f) & 0xffffu);
    }
  }
  if (lane == 0) lse[row] = big_m + logf(big_l);
}

}  // namespace sattn
