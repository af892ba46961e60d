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
//     operand and is packed straight from the score registers (no shuffles);
//     V^T (A operand) is read from the row-major [key][d] V tile in LDS with
//     transposing 8-byte reads (ds_read_b64_tr_b16). The output accumulator
//     again gives each lane one query, so the rescale factor of a query never
//     leaves its lane.
//   * K/V tiles go from HBM straight into LDS (buffer loads with the LDS
//     destination, no register staging), two tile buffers deep: one barrier
//     per tile makes tile t visible and frees tile t-1's buffer, into which
//     tile t+1 is then loaded while tile t is computed. Rows are permuted in
//     16-byte pieces (swz below) so both operand reads are conflict free.
//   * Causal: key tiles that start after a wave's last query are skipped, not
//     masked; the mask (key > query, diagonal kept) runs only on tiles that
//     straddle the diagonal or the key tail.
//   * Dense D = 128 runs 8 waves (256 queries) per workgroup, two per SIMD,
//     so each staged K/V tile serves 256 queries.
#pragma once

#include "common.hpp"

namespace sattn {

// DENSE: [B, H, N, D] self-attention, equal query/key lengths.
// VARLEN: packed sequences, grouped KV heads.
// SPLIT: per-chunk partial states over a key range (optionally causal).
// CACHE: [B, Hq, Nq, D] queries against a [B, Hkv, Nk, D] key/value cache;
//        query i sits at logical position i + (Nk - Nq).
// SPARSE: CACHE restricted to a sliding window, global tokens and a
//        block mask; only the key tiles some row needs are visited.
enum { MODE_DENSE = 0, MODE_VARLEN = 1, MODE_SPLIT = 2, MODE_CACHE = 3, MODE_SPARSE = 4 };

// Key tiles a sparse workgroup may list (Nk <= 64 * kSparseMaxTiles).
constexpr int kSparseMaxTiles = 1024;

// Build-time knobs of the design-variant builds (the library sets none):
// one K/V tile buffer, loaded after every wave is done with the previous
// tile, instead of two; causal key tiles after a row's position visited and
// masked instead of skipped.
#ifdef SATTN_SINGLE_BUFFER
constexpr bool kSingleBuffer = true;
#else
constexpr bool kSingleBuffer = false;
#endif
#ifdef SATTN_NO_CAUSAL_SKIP
constexpr bool kCausalSkip = false;
#else
constexpr bool kCausalSkip = true;
#endif

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
  int heads;       // dense: B*H; split, cache: B*Hq
  int hq, hkv;     // query heads, KV heads (varlen, split, cache)
  int n;           // dense: N; split, cache: Nq
  int nk;          // split, cache: Nk
  int off;         // split, cache: Nk - Nq, the logical position of query 0
  int pack;        // split: 1 = a slice is (batch, KV head) holding the Hq/Hkv query heads' rows
  // cache: element strides of the batch, head and row dims of q and of k/v
  // (k and v share them; the head dim d has stride 1). o and lse are dense.
  int64_t qs_b, qs_h, qs_n;
  int64_t ks_b, ks_h, ks_n;
  // sparse: key j is eligible for the query at position p iff
  // (p - win_left <= j <= p + win_right, a negative bound unlimited) or
  // j < n_global or p < n_global, and block (i / bm_q, j / bm_k) of the
  // query index i is active in bmask (if given; head h reads the
  // nqb x nkb bytes at bmask + h * bm_hstride), and j <= p when causal.
  int win_left, win_right, n_global;
  const uint8_t* bmask;
  int bm_q, bm_k, bm_nkb;
  int64_t bm_hstride;
  int chunk;       // split: keys per chunk
  int nchunks;     // split: C
  int nqt;         // query tiles per slice (dense/split) or per longest sequence (varlen)
  int nseq;        // varlen: S
  int total;       // varlen: T
  int pair;        // dense causal: 1 = each workgroup takes query tiles (nqt-1-j, j)
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
  int64_t o_rs;
  int64_t kv_rs;
  int q_pos0;          // logical position of row 0 (pos_mod > 0: of every row with (row0 + r) % pos_mod == 0)
  int pos_mod;         // 0: row r sits at q_pos0 + r; else at q_pos0 + (row0 + r) % pos_mod
  int row0;            // first row of this tile within its slice (used when pos_mod > 0)
  int nq;              // valid rows in this tile
  int k_begin, k_end;  // keys [k_begin, k_end) of the slice
  int64_t part_row0;   // split: index (slice_row * C + c) of row 0
  const uint8_t* bmask;  // sparse: this head's block mask (or null)
};

// Spread of workgroups over the 8 XCDs: blocks are handed out round-robin by
// block id, so remap the id to give XCD x one contiguous range of the
// logical order (and with it whole heads, whose K/V then share one L2).
__device__ __forceinline__ int xcd_linear(int bid) {
  const int per = (int)(gridDim.x / 8);
  return (bid < per * 8) ? (bid % 8) * per + bid / 8 : bid;
}

// Query tiles per workgroup: with enough workgroups to fill the chip, causal
// dense workgroups take the pair (nqt-1-j, j), so every workgroup has the same
// number of key tiles; small grids keep one tile each (shorter serial chain).
template <bool CAUSAL, int MODE>
constexpr int items_per_block() { return (MODE == MODE_DENSE && CAUSAL) ? 2 : 1; }

template <int D, int BM, bool CAUSAL, int MODE>
__device__ __forceinline__ bool decode_work(const FwdParams& p, int item, Work& w) {
  const int bid = blockIdx.x;
  if constexpr (MODE == MODE_DENSE) {
    const int lin = xcd_linear(bid);
    int head, qt;
    if (CAUSAL && p.pair) {
      const int npairs = (p.nqt + 1) / 2;
      head = lin / npairs;
      const int j = lin % npairs;
      qt = (item == 0) ? p.nqt - 1 - j : j;
      if (item == 1 && qt == p.nqt - 1 - j) return false;  // odd count: middle tile once
    } else {
      if (item > 0) return false;
      head = lin / p.nqt;
      qt = p.nqt - 1 - lin % p.nqt;
    }
    const int64_t base = (int64_t)head * p.n * D;
    w.q_pos0 = qt * BM;
    w.nq = min(BM, p.n - w.q_pos0);
    w.q = p.q + base + (int64_t)w.q_pos0 * D;
    w.o = p.o + base + (int64_t)w.q_pos0 * D;
    w.k = p.k + base;
    w.v = p.v + base;
    w.q_rs = D;
    w.o_rs = D;
    w.kv_rs = D;
    w.lse = p.lse + (int64_t)head * p.n + w.q_pos0;
    w.k_begin = 0;
    w.k_end = (CAUSAL && kCausalSkip) ? min(p.n, w.q_pos0 + BM) : p.n;
    w.pos_mod = 0;
    return w.nq > 0;
  } else if constexpr (MODE == MODE_VARLEN) {
    // Logical order: KV head, then sequence, then query tile (heaviest
    // first), then the query heads sharing that KV head; each XCD receives a
    // contiguous range of it, so the workgroups reading one sequence's K/V of
    // one KV head run together on one L2.
    const int grp = p.hq / p.hkv;
    const int lin = xcd_linear(bid);
    const int per_g = p.nseq * p.nqt * grp;
    const int g_kv = lin / per_g;
    const int r1 = lin % per_g;
    const int s = r1 / (p.nqt * grp);
    const int r2 = r1 % (p.nqt * grp);
    const int qt = p.nqt - 1 - r2 / grp;
    const int h = g_kv * grp + r2 % grp;
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
    w.o_rs = w.q_rs;
    w.kv_rs = (int64_t)p.hkv * D;
    w.q = p.q + (int64_t)(a + w.q_pos0) * w.q_rs + (int64_t)h * D;
    w.o = p.o + (int64_t)(a + w.q_pos0) * w.q_rs + (int64_t)h * D;
    w.k = p.k + (int64_t)a * w.kv_rs + (int64_t)g * D;
    w.v = p.v + (int64_t)a * w.kv_rs + (int64_t)g * D;
    w.lse = p.lse + (int64_t)h * p.total + a + w.q_pos0;
    w.k_begin = 0;
    w.k_end = CAUSAL ? min(len, w.q_pos0 + BM) : len;
    w.pos_mod = 0;
    return true;
  } else if constexpr (MODE == MODE_CACHE || MODE == MODE_SPARSE) {
    // Logical order: (batch, KV head), then query tile (heaviest first), then
    // the query heads sharing that KV head, so that the workgroups reading
    // one cache slice run together on one XCD and its L2.
    if (item > 0) return false;
    const int grp = p.hq / p.hkv;
    const int lin = xcd_linear(bid);
    const int per_kv = p.nqt * grp;
    const int kvs = lin / per_kv;                 // b * Hkv + g
    const int r = lin % per_kv;
    const int qt = p.nqt - 1 - r / grp;
    const int h = (kvs % p.hkv) * grp + r % grp;
    const int b = kvs / p.hkv;
    const int row0 = qt * BM;
    const int64_t qslice = ((int64_t)b * p.hq + h) * p.n;
    w.nq = min(BM, p.n - row0);
    w.q_pos0 = row0 + p.off;
    w.q = p.q + b * p.qs_b + h * p.qs_h + row0 * p.qs_n;
    w.o = p.o + (qslice + row0) * D;
    w.lse = p.lse + qslice + row0;
    const int64_t kvbase = b * p.ks_b + (int64_t)(kvs % p.hkv) * p.ks_h;
    w.k = p.k + kvbase;
    w.v = p.v + kvbase;
    w.q_rs = p.qs_n;
    w.o_rs = D;
    w.kv_rs = p.ks_n;
    w.k_begin = 0;
    // causal: keys after the tile's last query are never eligible; a tile
    // whose queries all precede the cache has no key at all
    w.k_end = CAUSAL ? min(p.nk, max(0, w.q_pos0 + BM)) : p.nk;
    w.pos_mod = 0;
    if constexpr (MODE == MODE_SPARSE) {
      w.row0 = row0;
      w.bmask = p.bmask ? p.bmask + h * p.bm_hstride : nullptr;
      if (p.win_right >= 0 && w.q_pos0 >= p.n_global)   // no global query: no row sees past p + win_right
        w.k_end = min(w.k_end, max(0, w.q_pos0 + BM + p.win_right));
    }
    return w.nq > 0;
  } else {
    // Split-KV: block id -> (slice, query tile, chunk), chunk fastest. A
    // slice is one (batch, query head); packed, it is one (batch, KV head)
    // whose rows are the Nq queries of each of its Hq/Hkv query heads in
    // turn (contiguous in [B, Hq, Nq] order), so each K/V chunk is read once
    // for the whole group ("Attention algorithms and data movement", lesson
    // 05: the cache payload is shared by the group's query heads).
    const int c = bid % p.nchunks;
    const int rest = bid / p.nchunks;
    const int qt = rest % p.nqt;
    const int slice = rest / p.nqt;
    const int grp = p.hq / p.hkv;
    int64_t first_row;                       // row of [B*Hq*Nq] where the slice starts
    int nrows, kvs;
    if (p.pack) {                            // slice = b * Hkv + g
      first_row = ((int64_t)(slice / p.hkv) * p.hq + (int64_t)(slice % p.hkv) * grp) * p.n;
      nrows = grp * p.n;
      kvs = slice;
    } else {                                 // slice = b * Hq + h
      first_row = (int64_t)slice * p.n;
      nrows = p.n;
      kvs = (slice / p.hq) * p.hkv + (slice % p.hq) / grp;
    }
    const int row0 = qt * BM;
    w.nq = min(BM, nrows - row0);
    w.row0 = row0;
    w.pos_mod = p.pack ? p.n : 0;
    w.q_pos0 = p.pack ? p.off : row0 + p.off;
    w.q = p.q + (first_row + row0) * D;
    w.o = nullptr;
    w.lse = nullptr;
    const int64_t kvbase = (int64_t)kvs * p.nk * D;
    w.k = p.k + kvbase;
    w.v = p.v + kvbase;
    w.q_rs = D;
    w.o_rs = D;
    w.kv_rs = D;
    w.k_begin = c * p.chunk;
    w.k_end = min(p.nk, w.k_begin + p.chunk);
    // causal: keys after the tile's last position are never eligible; a
    // chunk with none left still writes its rows' empty states
    if (CAUSAL) w.k_end = max(w.k_begin, min(w.k_end, p.pack ? p.off + p.n : w.q_pos0 + BM));
    w.part_row0 = (first_row + row0) * p.nchunks + c;
    return w.nq > 0;
  }
}

// 16-byte piece swizzle of a K/V tile row in LDS. A row of D bf16/fp16
// values is PPR = D/8 pieces; piece p of tile row `key` is stored at position
// p ^ swz(key). LDS serves 256 bytes (64 banks x 4 bytes) per clock: 16 lanes
// of a 16-byte read, 32 lanes of an 8-byte read. swz makes both operand reads
// conflict-free:
//   * K (A of S^T = K Q^T): 16 lanes read one piece of 16 consecutive rows;
//     their positions must be distinct within the 256-byte bank window.
//   * V (transposing 8-byte reads): 32 lanes read 4 pieces of 4 consecutive
//     rows; the four rows' piece groups must land on different banks.
// Direct HBM->LDS loads write 1 KiB contiguous per wave instruction, so rows
// cannot be padded; the permutation does the spreading instead. swz(key)
// depends only on key mod 16, and on nothing that changes between 32-row
// blocks, so per-lane operand offsets are tile independent.
template <int D>
__device__ __forceinline__ int swz(int key) {
  if constexpr (D == 128) return ((key & 3) << 2) | ((key >> 2) & 3);   // 16 pieces: swap 2-bit halves
  else if constexpr (D == 64) return ((key >> 1) & 1) << 2 | ((key >> 2) & 3);  // 8 pieces
  else return (key >> 2) & 3;                                          // 4 pieces
}

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// Transposing LDS read (gfx950 ds_read_b64_tr_b16). Within each group of 16
// lanes, lane j receives element (j % 4) of the 8-byte rows addressed by
// lanes 4e + j/4, e = 0..3, as its element e.
__device__ __forceinline__ u32x2 lds_read_tr16(const uint16_t* lds_byte_ptr) {
  i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(lds_byte_ptr));
  return __builtin_bit_cast(u32x2, r);
}

// Row max / sum across the two half-waves (lanes l and l ^ 32 hold the same
// query in the 32x32 accumulator layout).
__device__ __forceinline__ float max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x),
                                                  __builtin_bit_cast(uint32_t, x), false, false);
  return fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x),
                                                  __builtin_bit_cast(uint32_t, x), false, false);
  return __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
}

// One query tile of BM = 32*NW rows against the keys [k_begin, k_end) of its
// slice. LAZY: keep a stale running max until some row's max has grown by
// more than 2^8 (in exp2 units), so acc/l are rescaled only then. O and lse
// are unchanged mathematically (exp(S - m) with any fixed m >= the values
// seen so far minus 8 stays in [0, 256]). The split path keeps the exact
// chunk max because it is part of the partial-state output.
template <class E, int D, int BN, int NW, bool CAUSAL, int MODE>
__device__ __forceinline__ void attn_rows(const FwdParams& p, const Work& w, uint16_t* sbuf0, uint16_t* sbuf1,
                                          int* tlist, int* tcount) {
  constexpr int PPR = D / 8;               // 16-byte pieces per row
  constexpr int TILE_BYTES = BN * D * 2;   // one K or V tile
  constexpr int NI = TILE_BYTES / 1024 / NW;  // 1 KiB direct loads per wave per tile
  constexpr int KK = D / 16;               // MFMA k-steps of Q K^T
  constexpr int KB = BN / 32;              // 32-key blocks per tile
  constexpr int DB = D / 32;               // 32-wide d blocks of the output
  constexpr bool LAZY = (MODE != MODE_SPLIT);
  // Rows that can have no eligible key in the keys walked here: queries
  // before the cache or an empty cache, or a causal chunk after a query. Their max stays -inf,
  // and exps are then taken against 0 so that masked scores give 0, not NaN.
  constexpr bool EMPTY_ROWS = MODE == MODE_CACHE || MODE == MODE_SPARSE || (CAUSAL && MODE == MODE_SPLIT);
  constexpr bool SPARSE = MODE == MODE_SPARSE;
  constexpr float LAZY_TH = 8.0f;
  static_assert(NI >= 1 && TILE_BYTES % (1024 * NW) == 0, "tile must split into 1 KiB wave loads");
  static_assert(D % 32 == 0 && BN % 32 == 0, "tile shape");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
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
  float m = -INFINITY;  // running (possibly stale) max, log2 units
  float l = 0.f;        // this lane's part of the exp-sum

  // Logical position of this lane's row, and the last position of the wave's
  // rows (packed split rows repeat the Nq positions once per query head).
  const int my_pos = w.pos_mod ? w.q_pos0 + (w.row0 + qrow) % w.pos_mod : w.q_pos0 + qrow;
  const int wave_last_pos = w.pos_mod ? w.q_pos0 + w.pos_mod - 1 : w.q_pos0 + wave * 32 + 31;
  const int wave_first_pos = w.pos_mod ? w.q_pos0 : w.q_pos0 + wave_u * 32;  // wave-uniform lower bound
  const bool wave_active = wave * 32 < w.nq;
  const float c = p.c;
  const int ntiles = (w.k_end - w.k_begin + BN - 1) / BN;

  // Tile loads: buffer loads straight into LDS. The descriptors cover keys
  // [0, k_end) of the slice, so reads past the last key return zeros. Slot
  // s of a tile (16 bytes) holds piece (s % PPR) ^ swz(key) of tile row
  // key = s / PPR; the per-lane byte offsets do not depend on the tile.
  const uint32_t row_bytes = (uint32_t)w.kv_rs * 2u;
  const uint32_t span = (uint32_t)w.k_end * row_bytes;
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc((void*)w.k, (short)0, (int)span, 0x00020000);
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc((void*)w.v, (short)0, (int)span, 0x00020000);
  uint32_t voff[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int slot = (wave * NI + i) * 64 + lane;
    const int key = slot / PPR;
    voff[i] = (uint32_t)key * row_bytes + (uint32_t)(((slot % PPR) ^ swz<D>(key)) * 16);
  }
  // Split mode reads each K/V byte once (a chunk belongs to one workgroup):
  // its tile loads are marked nontemporal (the cache-policy NT bit), which
  // took the causal GQA decode from 5.9 to 6.55 TB/s. The other modes
  // re-read a head's K/V tiles from L2 across its query tiles.
  constexpr int kTileLoadPolicy = MODE == MODE_SPLIT ? 2 : 0;
  auto issue_tile = [&](int t, uint16_t* sb) {
    const uint32_t soff = (uint32_t)(w.k_begin + t * BN) * row_bytes;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      uint16_t* dst = sb + (wave_u * NI + i) * 512;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (__attribute__((address_space(3))) void*)(dst), 16, voff[i],
                                               soff, 0, kTileLoadPolicy);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (__attribute__((address_space(3))) void*)(dst + BN * D), 16,
                                               voff[i], soff, 0, kTileLoadPolicy);
    }
  };

  // Per-lane LDS element offsets of the MFMA A operands (tile independent).
  // K: tile row kb*32 + l32, piece 2*kk + hf (swizzle depends on l32 only).
  int kofs[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) kofs[kk] = l32 * D + (((kk * 2 + hf) ^ swz<D>(l32)) * 8);
  // V via transposing reads: 16-lane group G covers d = db*32 + 16*(G&1) +
  // 0..15 and keys base + 4*(G>>1) + 0..3; lane supplies the 8-byte row
  // piece of key (lane&15)>>2 at d offset 4*(lane&3).
  // The two reads of one operand cover rows tr_key and tr_key + 8 of a
  // 16-row group; their swizzles differ, so each has its own offsets.
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

  // Two ways to keep the softmax state of a row across tiles:
  //  * exact online update: running max, acc/l rescaled when the max grows
  //    (lazily, by more than 2^8 in exp2 units outside the split path);
  //  * fixed reference (FAST): the row's max over the first tile is kept as m
  //    for later tiles, which then need no max and no rescale:
  //    p = exp2(S*c - m). O and lse do not depend on which m is used as long
  //    as nothing overflows; with every tile sum <= 2^64, l <= 2^94 and
  //    acc <= 2^110 for any N < 2^30 and |v| < 2^16.
  //    bf16: a tile sum past 2^64 (scores grown by 2^64 over the first
  //    tile's max) raises `overflow`, and the workgroup recomputes its rows
  //    with the exact update after the walk, as does a workgroup whose acc is
  //    not finite (huge values).
  //    fp16: the limit is 2^15, since each p is rounded to fp16 for the PV
  //    product, whose largest finite value is 65504 (a sum <= 2^15 bounds
  //    every p in it); large logits reach it often, so a 32-key block past it
  //    is redone at once for its rows with the exact update (see the tile
  //    body), which moves their reference up to the running maximum.
  bool overflow = false;
  constexpr float FAST_LIMIT = E::kFastLimit;

  // One tile: wait for its loads, start the next tile's loads into the other
  // buffer, then compute on this one.
  // Sparse mode walks a list of the key tiles some wave needs (built below):
  // entry = tile | (waves that need it) << 16 | (element mask needed) << 24.
  int nact = 0;
  auto body = [&](int /* list index */, int t, int e, const uint16_t* cur, auto mask_tag, auto fast_tag) {
    constexpr bool MASKED = decltype(mask_tag)::value;
    constexpr bool FAST = decltype(fast_tag)::value;
    const int kt0 = w.k_begin + t * BN;
    if (!wave_active || (CAUSAL && kCausalSkip && kt0 > wave_last_pos)) return;
    if (SPARSE && !((e >> (16 + wave_u)) & 1)) return;   // this wave's query block or window skips the tile
    const uint16_t* sK = cur;
    const uint16_t* sV = cur + BN * D;

    // ---- S^T = K Q^T for one 32-key block x 32 queries, then its masks:
    // key tail, and keys after the query (diagonal kept); in sparse mode
    // also the window / global-token rule, only on listed tiles that some
    // row does not wholly see
    auto score_block = [&](f32x16& sb, int kb) {
      u32x4 ka[KK];
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) ka[kk] = *(const u32x4*)(sK + kofs[kk] + kb * 32 * D);
#pragma unroll
      for (int r = 0; r < 16; ++r) sb[r] = 0.f;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) sb = E::mfma32(ka[kk], qreg[kk], sb);
      if constexpr (MASKED && !SPARSE) {
        // only where this wave's rows see a key past the tail or after them
        if (kt0 + BN > w.k_end || (CAUSAL && kt0 + BN - 1 > wave_first_pos))
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kt0 + kb * 32 + 8 * (r >> 2) + 4 * hf + (r & 3);
            if ((key >= w.k_end) || (CAUSAL && key > my_pos)) sb[r] = -INFINITY;
          }
      }
      if constexpr (SPARSE) {
        if ((e >> 24) & 1) {
          const bool row_global = my_pos < p.n_global;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kt0 + kb * 32 + 8 * (r >> 2) + 4 * hf + (r & 3);
            const bool in_win = (p.win_left < 0 || key >= my_pos - p.win_left) &&
                                (p.win_right < 0 || key <= my_pos + p.win_right);
            const bool ok = key < w.k_end && (!CAUSAL || key <= my_pos) && (in_win || key < p.n_global || row_global);
            if (!ok) sb[r] = -INFINITY;
          }
        }
      }
    };
    // p = exp2(S*c - reference) in place; returns the lane's sum
    auto exps = [&](f32x16& sb) {
      const float mref = (EMPTY_ROWS && m == -INFINITY) ? 0.f : m;
      float rs = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pv = fast_exp2(fmaf(sb[r], c, -mref));
        sb[r] = pv;
        rs += pv;
      }
      return rs;
    };
    // ---- O^T += V^T P^T for one 32-key block, 16 keys per MFMA
    auto pv_block = [&](const f32x16& sb, int kb) {
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int o8 = half * 8;
        const u32x4 pb = {E::pack2(sb[o8 + 0], sb[o8 + 1]), E::pack2(sb[o8 + 2], sb[o8 + 3]),
                          E::pack2(sb[o8 + 4], sb[o8 + 5]), E::pack2(sb[o8 + 6], sb[o8 + 7])};
        const int krow = (kb * 32 + half * 16) * D;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const u32x2 a0 = lds_read_tr16(sV + vofs[0][db] + krow);
          const u32x2 a1 = lds_read_tr16(sV + vofs[1][db] + krow);
          acc[db] = E::mfma32(u32x4{a0[0], a0[1], a1[0], a1[1]}, pb, acc[db]);
        }
      }
    };

    f32x16 s[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) score_block(s[kb], kb);

    if constexpr (FAST) {
      // ---- fixed-reference update: exps against the row's reference
      if constexpr (SPARSE) {
        // A row whose first kept key comes after the first tile takes its
        // reference from the first tile that has one (its acc and l are
        // still zero, so nothing needs rescaling).
        if (__builtin_amdgcn_ballot_w64(m == -INFINITY) != 0) {
          float mx = -INFINITY;
#pragma unroll
          for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
          mx = max_halves(mx);
          if (m == -INFINITY) m = mx * c;
        }
      }
      if constexpr (E::kRedoBlocks) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          float rs = exps(s[kb]);
          if constexpr (!MASKED && !SPARSE && KB == 2 && KK == 8) {
            if (kb == 0) {
              // Keep the overlap of a branch-free tile inside the first of the
              // blocks the check below creates: block 0's eight K reads, its
              // MFMAs each with one of block 1's K reads, then block 1's MFMAs
              // each with six VALU of block 0's exps.
              __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);   // DS read
              for (int i = 0; i < 8; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0); // MFMA
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
              }
              for (int i = 0; i < 8; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x402, 6, 0); // VALU incl. transcendental
              }
            }
          }
          // A lane's block sum past the limit (or not finite): some row's
          // scores grew too far above its reference. The wave redoes this
          // block (its K is still in LDS) with the exact update for those
          // rows only: the row's reference moves up to its running maximum,
          // acc and l are rescaled to it, and the exps are taken again. Other
          // rows recompute the same scores and exps bit for bit, so a row's
          // result never depends on the data of other rows.
          if (__builtin_amdgcn_ballot_w64(!(rs <= FAST_LIMIT)) != 0) {
            const bool bad = max_halves(!(rs <= FAST_LIMIT) ? 1.f : 0.f) > 0.f;   // either half of the row
            // read K again rather than keep the first reads' registers alive
            asm volatile("" ::: "memory");
            score_block(s[kb], kb);
            float mx = -INFINITY;
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
            const float m_cand = fmaxf(m, max_halves(mx) * c);
            const bool need = bad && m_cand > m;
            const float alpha = need ? fast_exp2(m - m_cand) : 1.0f;
            m = need ? m_cand : m;
            l *= alpha;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
              for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;
            rs = exps(s[kb]);
          }
          l += rs;
          pv_block(s[kb], kb);
        }
      } else {
        // No branch inside the tile: a sum past the limit only raises the
        // workgroup's flag, and the walk is recomputed with the exact update
        // at the end (a scores growth of 2^64 after the first tile).
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          const float rs = exps(s[kb]);
          l += rs;
          overflow = overflow || !(rs <= FAST_LIMIT);
          pv_block(s[kb], kb);
        }
        if constexpr (!MASKED && !SPARSE && KB == 2 && KK == 8 && DB == 4) {
          // Order of the unmasked tile (one scheduling region), so that each
          // LDS operand read is issued before the MFMA ahead of its own:
          // block 0's eight K reads; block 0's S MFMAs, each with one of
          // block 1's K reads; block 1's S MFMAs, each with six VALU of
          // block 0's exps; the V reads of the first PV MFMA and block 0's P
          // packing; block 0's PV MFMAs, each with the next MFMA's two V
          // reads and six VALU of block 1's exps; block 1's P packing and PV
          // MFMAs, V reads one MFMA ahead. Same arithmetic, same bits.
          __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);    // DS read
          for (int i = 0; i < 8; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          }
          for (int i = 0; i < 8; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x402, 6, 0);  // VALU, transcendental included
          }
          __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
          __builtin_amdgcn_sched_group_barrier(0x402, 8, 0);
          for (int i = 0; i < 8; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x402, 6, 0);
          }
          __builtin_amdgcn_sched_group_barrier(0x402, 8, 0);
          for (int i = 0; i < 8; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
          }
        }
      }
    } else {
      // ---- exact online update (fp32)
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
      mx = max_halves(mx);
      const float m_cand = fmaxf(m, mx * c);
      const bool need = LAZY ? (m_cand > m + LAZY_TH) : (m_cand > m);
      // The branch is taken when any row of the wave needs a rescale, but
      // each row applies only its own decision (alpha = 1 otherwise), so a
      // row's bits never depend on other rows' data.
      if (__builtin_amdgcn_ballot_w64(need) != 0) {
        const float alpha = need ? fast_exp2(m - m_cand) : 1.0f;
        m = need ? m_cand : m;
        l *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;
      }
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) l += exps(s[kb]);
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) pv_block(s[kb], kb);
    }
  };

  auto step = [&](int idx, const uint16_t* cur, uint16_t* nxt, auto mask_tag, auto fast_tag) {
    const int e = SPARSE ? tlist[idx] : idx;
    const int t = SPARSE ? (e & 0xffff) : idx;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();  // tile t visible to all waves; every wave is done with the previous tile
    if constexpr (kSingleBuffer) {  // every tile lives in sbuf0
      body(idx, t, e, sbuf0, mask_tag, fast_tag);
      __syncthreads();  // every wave is done with the one buffer
      if (t + 1 < ntiles) issue_tile(t + 1, sbuf0);
      return;
    }
    if (SPARSE) {
      if (idx + 1 < nact) issue_tile(tlist[idx + 1] & 0xffff, nxt);
    } else if (t + 1 < ntiles) {
      issue_tile(t + 1, nxt);
    }
    body(idx, t, e, cur, mask_tag, fast_tag);
  };

  // Tiles [0, n_full) need no mask for any row of the workgroup (they end
  // before its first query and before the key tail); the rest take the masked
  // body. Tile 0 always takes the exact update: it sets each row's max.
  int n_full = (w.k_end - w.k_begin) / BN;
  if (CAUSAL) n_full = min(n_full, max(0, (w.q_pos0 - w.k_begin + 1) / BN));
  const std::integral_constant<bool, false> no{};
  const std::integral_constant<bool, true> yes{};
  if constexpr (SPARSE) {
    // Wave 0 lists the key tiles in order, 64 candidates per pass: a tile is
    // kept if some wave needs it (its rows' window / global tokens reach the
    // tile, the tile is not after their positions, and their query block's
    // mask bit for the tile's key block is set), and flagged for element
    // masks unless every row of every such wave sees all of its keys.
    if (wave_u == 0) {
      int count = 0;
      for (int base = 0; base < ntiles; base += 64) {
        const int t = base + lane;
        int bits = 0;
        bool full_all = true;
        if (t < ntiles) {
          const int k0 = w.k_begin + t * BN;
          const int k1 = min(k0 + BN, w.k_end) - 1;
          for (int wv = 0; wv < NW; ++wv) {
            const int r0 = wv * 32;
            if (r0 >= w.nq) break;
            const int p0 = w.q_pos0 + r0;
            const int p1 = w.q_pos0 + min(r0 + 32, w.nq) - 1;
            const bool glob = k0 < p.n_global || p0 < p.n_global;
            const bool win = (p.win_left < 0 || k1 >= p0 - p.win_left) && (p.win_right < 0 || k0 <= p1 + p.win_right);
            bool need = (!CAUSAL || k0 <= p1) && (win || glob);
            if (need && w.bmask)
              need = w.bmask[(int64_t)((w.row0 + r0) / p.bm_q) * p.bm_nkb + k0 / p.bm_k] != 0;
            if (!need) continue;
            bits |= 1 << wv;
            const bool win_full = (p.win_left < 0 || k0 >= p1 - p.win_left) && (p.win_right < 0 || k1 <= p0 + p.win_right);
            const bool glob_full = k1 < p.n_global || p1 < p.n_global;
            const bool full = (k0 + BN <= w.k_end) && (!CAUSAL || k1 <= p0) && (win_full || glob_full);
            full_all = full_all && full;
          }
        }
        const uint64_t act = __builtin_amdgcn_ballot_w64(bits != 0);
        const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(act >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)act, 0));
        if (bits != 0) tlist[count + below] = t | (bits << 16) | ((full_all ? 0 : 1) << 24);
        count += __builtin_popcountll(act);
      }
      if (lane == 0) *tcount = count;
    }
    __syncthreads();
    nact = *tcount;
  }
  auto run = [&](auto fast_tag) {
    if constexpr (SPARSE) {
      if (nact == 0) return;
      issue_tile(tlist[0] & 0xffff, sbuf0);
      int n = 0;
      for (; n + 1 < nact; n += 2) {
        step(n, sbuf0, sbuf1, std::true_type{}, fast_tag);
        step(n + 1, sbuf1, sbuf0, std::true_type{}, fast_tag);
      }
      if (n < nact) step(n, sbuf0, sbuf1, std::true_type{}, fast_tag);
      return;
    }
    if (ntiles == 0) return;
    issue_tile(0, sbuf0);
    if (n_full >= 1) step(0, sbuf0, sbuf1, no, no);
    else step(0, sbuf0, sbuf1, yes, no);
    int t = 1;
    for (; t + 1 < n_full; t += 2) {
      step(t, sbuf1, sbuf0, no, fast_tag);
      step(t + 1, sbuf0, sbuf1, no, fast_tag);
    }
    for (; t < ntiles; ++t) {
      if (t & 1) step(t, sbuf1, sbuf0, yes, fast_tag);
      else step(t, sbuf0, sbuf1, yes, fast_tag);
    }
  };
  if constexpr (MODE == MODE_SPLIT) {
    run(no);  // the partial state exports the exact chunk max
  } else {
    run(yes);
    // The tile-sum limit bounds acc only for |v| < 2^16; a numerator that
    // overflowed fp32 (huge values under a large score growth) also takes
    // the exact update.
    // (a sum of magnitudes is inf or NaN iff some element is, or the sum
    // itself overflows, which also means huge values)
    float asum[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) asum[r & 3] += fabsf(acc[db][r]);
    const bool acc_bad = !((asum[0] + asum[1]) + (asum[2] + asum[3]) <= 3.402823466e38f);
    if (__syncthreads_or((overflow || acc_bad) ? 1 : 0)) {  // rare: redo with the exact update
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;
      m = -INFINITY;
      l = 0.f;
      run(no);
      __syncthreads();  // every wave is done with the tile buffers, which the epilogue reuses
    }
  }

  if (!wave_active) return;
  const float lt = sum_halves(l);

  if constexpr (MODE != MODE_SPLIT) {
    // an empty row (no eligible key) gives O = 0 and lse = -inf
    const float inv = (EMPTY_ROWS && lt == 0.f) ? 0.f : 1.f / lt;
    // O leaves through LDS (the idle tile buffers), as whole rows: waves 0-3
    // use slices of sbuf0, waves 4-7 of sbuf1
    store_tile_rows<E, D>(acc, inv, (wave_u < 4 ? sbuf0 : sbuf1) + (wave_u & 3) * 32 * D,
                          w.o + (int64_t)wave_u * 32 * w.o_rs, w.o_rs, w.nq - wave_u * 32);
    if (row_ok && hf == 0) w.lse[qrow] = (m + fast_log2(lt)) * kLn2;
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

template <class E, int D, int BN, int NW, bool CAUSAL, int MODE>
__global__ __launch_bounds__(NW * 64, 2) void fwd_kernel(const FwdParams p) {
  constexpr int BM = NW * 32;
  // Double-buffered K and V tiles, as two distinct arrays so the compiler can
  // tell that reads of one buffer never alias the prefetch into the other
  // (otherwise it makes every LDS read wait for the in-flight prefetch).
  // Each buffer also stages the output rows of up to 4 waves in the
  // epilogue (32 rows of D each), which 64-key tiles fill exactly.
  constexpr int SBUF = (2 * BN * D > 128 * D) ? 2 * BN * D : 128 * D;
  __shared__ __attribute__((aligned(1024))) uint16_t sbuf0[SBUF];
  __shared__ __attribute__((aligned(1024))) uint16_t sbuf1[SBUF];
  __shared__ int tlist[MODE == MODE_SPARSE ? kSparseMaxTiles : 1];
  __shared__ int tcount;
  constexpr int NITEMS = items_per_block<CAUSAL, MODE>();
#pragma unroll 1
  for (int item = 0; item < NITEMS; ++item) {
    if (item > 0) __syncthreads();  // the previous tile's LDS reads are done
    Work w;
    if (!decode_work<D, BM, CAUSAL, MODE>(p, item, w)) continue;  // uniform over the workgroup
    attn_rows<E, D, BN, NW, CAUSAL, MODE>(p, w, sbuf0, sbuf1, tlist, &tcount);
  }
}

// Merge of split-KV partial states, one row per single-wave workgroup (a
// few hundred rows then still spread over every CU); the partials are summed
// in ascending chunk order ("Attention algorithms and data movement", lesson
// 01). The row max and the chunk weights exp(m_c - M) are taken for 64
// chunks at a time, one chunk per lane; the ordered sums then read the
// weights back lane by lane while the accumulator rows of 16 chunks are
// loaded together.
template <class E, int D>
__global__ __launch_bounds__(64) void merge_kernel(const float* __restrict__ pm, const float* __restrict__ pl,
                                                   const float* __restrict__ pacc, int64_t rows, int nchunks,
                                                   uint16_t* __restrict__ o, float* __restrict__ lse) {
  constexpr int PER = D >= 64 ? D / 64 : 1;  // d values per lane
  constexpr int BATCH = 16;                  // chunks whose accumulator rows are in flight together
  const int lane = threadIdx.x;
  const int64_t row = blockIdx.x;
  if (row >= rows) return;
  const bool lane_ok = lane * PER < D;
  const float* rm = pm + row * nchunks;
  const float* rl = pl + row * nchunks;
  float big_m = -INFINITY;
  for (int ch = lane; ch < nchunks; ch += 64) big_m = fmaxf(big_m, rm[ch]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) big_m = fmaxf(big_m, __shfl_xor(big_m, off));
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
  const float* src = pacc + row * nchunks * D + (lane_ok ? lane * PER : 0);
  for (int c0 = 0; c0 < nchunks; c0 += 64) {
    const int n = min(64, nchunks - c0);
    float wgt = 0.f, lc = 0.f;   // this lane's chunk c0 + lane: weight and partial sum
    if (lane < n) {
      const float mc = rm[c0 + lane];
      wgt = (mc == -INFINITY) ? 0.f : expf(mc - big_m);
      lc = rl[c0 + lane];
    }
    for (int j0 = 0; j0 < n; j0 += BATCH) {
      float v[BATCH][PER];
#pragma unroll
      for (int j = 0; j < BATCH; ++j)
#pragma unroll
        for (int e = 0; e < PER; ++e) v[j][e] = (lane_ok && j0 + j < n) ? src[(int64_t)(c0 + j0 + j) * D + e] : 0.f;
#pragma unroll
      for (int j = 0; j < BATCH; ++j) {
        if (j0 + j >= n) break;
        const float wj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wgt), j0 + j));
        big_l = fmaf(wj, __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lc), j0 + j)), big_l);
#pragma unroll
        for (int e = 0; e < PER; ++e) a[e] = fmaf(wj, v[j][e], a[e]);
      }
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
