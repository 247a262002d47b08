// index_score.hip -- lightning-indexer scores over MXFP4 keys with gfx950 scaled MFMA.
//
// Source: "DeepSeek-V4.1-Flash, expliqué pas à pas", CSA2 section (the indexer scores
// each cache entry from the query's indexer query and the entry's indexer key) and
// FP4 KV cache section (indexer queries and keys are OCP MXFP4).
//
// score[q][j] = fma-chain over h = 0..Hi-1 of w[q][h] * max(d_h, 0), starting at +0,
// d_h = exact dot(qhat_h, khat_j) rounded once to fp32.
//
// Layout of the work.  A wavefront takes one page (64 consecutive entries) at a time.
// With Hi a multiple of 32 it issues, per 32-head tile and 32-entry tile, two chained
//   V_MFMA_SCALE_F32_32X32X64_F8F6F4 (A = 32 query heads, B = 32 keys, K = 64 each)
// (score_page32 below); otherwise Hi/16 x 4 MFMAs
//   V_MFMA_SCALE_F32_16X16X128_F8F6F4 (A = 16 query heads, B = 16 keys, K = 128)
// with E8M0 block scales, so one instruction produces 16x16 complete dot products.
// Operand lane l holds row l%16 and the 32-channel block l/16: that is exactly one
// 16-byte slice of a packed key row plus its E8M0 byte, so each key row is fetched
// with four coalesced 16-byte loads per lane group.
// Exactness.  A block of 32 products contributes S_b * 2^E_b with S_b an integer,
// |S_b| <= 32 * 12 * 12 = 4608 (products of twice-E2M1 values), and E_b the block's
// exponent sum u_q + u_k - 256.  When the four E_b span at most s, one block sits at
// the lowest exponent E and every partial sum of the dot is an integer multiple of
// 2^E below 4608 * (1 + 3 * 2^s) * 2^E in magnitude, which is under 2^24 * 2^E for
// s <= 10: every partial sum is then exactly representable in fp32, so the matrix
// unit's result is the exact dot whatever order or width it accumulates in (also
// for the two chained K = 64 instructions of the 32x32x64 form), and the one
// rounding of the definition is the identity.  Entries outside that window (or
// near the fp32 subnormal or overflow range) take an exact integer/fp64 path, so
// results are always bit-identical to the definition.
// The query heads are permuted across MFMA rows so that lane group g ends up holding
// a contiguous run of Hi/4 heads; a 4x4 transpose across lane groups with
// v_permlane32_swap / v_permlane16_swap then leaves every lane with one entry and
// all Hi heads in ascending order, and the fma chain runs with all 64 lanes busy.
#include "common.hpp"
#include "host_common.hpp"
#include "topk_internal.hpp"

#include <algorithm>
#include <mutex>

namespace csa2 {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kMaxSpread = 10;   // exponent-sum span accepted on the MFMA path (every partial sum exact)
constexpr int kMinExpSum = 130;  // keeps every nonzero dot >= 2^-126 (fp32 normal)
constexpr int kMaxExpSum = 360;  // keeps every dot far below fp32 overflow
// (query, entry) scores recomputed on the exact path since the last reset, on this
// device (a diagnostic: the exact path is rare, so the atomics cost nothing measurable)
__device__ unsigned long long g_exact_path_count = 0ull;
CSA2_DEV void count_exact_path() { atomicAdd(&g_exact_path_count, 1ull); }

constexpr int kMaxPagesPerWave = 4;  // pages (of 64 entries) one wavefront scans, all prefetched
constexpr int kWaves = 8;             // wavefronts per workgroup (they share one query staging)
constexpr int kThreads = 64 * kWaves;

// per-query staging record in LDS, for Hi = 16*MT heads
template <int MT>
struct QStage {
  uint4 codes[MT][64];            // A operand of M-tile mt for lane l
  uint32_t scale[(MT + 3) / 4][64];  // byte (mt%4) of word mt/4: E8M0 of lane l in tile mt
  // the same blocks as A operands of the 32x32x64 form (Hi a multiple of 32): 32-head
  // tile m, K-step s, lane l = head row (l%32) and block 2s + l/32; E8M0 in byte
  // (2m+s)%4 of word (2m+s)/4
  uint4 codes32[(MT + 1) / 2][2][64];
  uint32_t scale32[(MT + 3) / 4][64];
  uint8_t u[16 * MT][4];          // E8M0 of head h, block b (plain order, exact path)
  uint32_t stat[MT];  // heads of M-tile mt: largest block-exponent span | min u << 8 | max u << 16
  int row;
  int nvis;
};

// Head held by row rho of M-tile mt: lane group rho/4 owns heads [(rho/4)*4MT, +4MT).
template <int MT>
CSA2_DEV int head_of(int mt, int rho) { return (rho >> 2) * 4 * MT + 4 * mt + (rho & 3); }

// MX32 quantisation of one 32-channel block held by one thread -> 16 packed bytes.
// For a normal power-of-two scale X the hardware V_CVT_SCALEF32_PK_FP4_F32 computes
// round-to-nearest-even(x / X) with saturation and a copied sign bit, which is the
// element rule exactly (checked on gfx950 against every bf16 value); blocks whose
// shared exponent is near the ends of the range take the compare-based rule.
struct QRaw {
  uint4 v[4];  // 32 bf16 values of one block
};
CSA2_DEV void mx32_load(const uint16_t* __restrict__ src, QRaw& r) {
#pragma unroll
  for (int i = 0; i < 4; ++i) r.v[i] = reinterpret_cast<const uint4*>(src)[i];
}
CSA2_DEV void mx32_block(const QRaw& r, uint4& out, uint32_t& u_out) {
  uint32_t raw[16];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    raw[4 * i] = r.v[i].x;
    raw[4 * i + 1] = r.v[i].y;
    raw[4 * i + 2] = r.v[i].z;
    raw[4 * i + 3] = r.v[i].w;
  }
  uint32_t amax_bits = 0;  // |x| as bf16 bits orders like the value
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    amax_bits = max(amax_bits, raw[i] & 0x7FFFu);
    amax_bits = max(amax_bits, (raw[i] >> 16) & 0x7FFFu);
  }
  const uint32_t u = mx_exponent(bf16_to_f32(amax_bits));
  const float X = ldexpf(1.0f, (int)u - 127);
  uint32_t word[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < 16; ++i) {  // element pair (2i, 2i+1) -> byte i
    const uint32_t c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, bf16_to_f32(raw[i] & 0xFFFFu),
                                                                 __uint_as_float(raw[i] & 0xFFFF0000u), X, 0);
    word[i >> 2] |= (c & 0xFFu) << (8 * (i & 3));
  }
  const bool edge = u < 4u || u > 250u;
  // a real (wave-uniform) branch: the compare-based rule only runs when some lane
  // of the wavefront has a block exponent near the ends of the range
  if (__builtin_amdgcn_ballot_w64(edge) != 0ull) {
    if (edge) {
#pragma unroll
      for (int k = 0; k < 4; ++k) word[k] = 0u;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        uint32_t c = e2m1_code(bf16_to_f32(raw[i] & 0xFFFFu), X) | (e2m1_code(bf16_to_f32(raw[i] >> 16), X) << 4);
        word[i >> 2] |= c << (8 * (i & 3));
      }
    }
  }
  out = make_uint4(word[0], word[1], word[2], word[3]);
  u_out = u;
}

// max(d, 0) on the bit pattern: non-negative floats order like signed integers and
// every negative float (including -0) is a negative integer, so this is one integer
// max with no canonicalisation (d is never NaN for visible entries).
CSA2_DEV float relu(float d) { return __int_as_float(max(__float_as_int(d), 0)); }

// Exact d_h for one (query head, entry): integer block sums, fp64 combination in
// block order, one rounding to fp32 (the definition itself).
template <int MT>
CSA2_DEV float exact_dot(const QStage<MT>& st, int h, const uint8_t* __restrict__ krow, uint32_t kscales) {
  const int mt = (h % (4 * MT)) >> 2;
  const int rho = (h / (4 * MT)) * 4 + (h & 3);
  double D = 0.0;
  for (int b = 0; b < 4; ++b) {
    const uint4 qc = st.codes[mt][16 * b + rho];
    const uint32_t qw[4] = {qc.x, qc.y, qc.z, qc.w};
    int S = 0;
    for (int i = 0; i < 32; ++i) {
      uint32_t qn = (qw[i >> 3] >> (4 * (i & 7))) & 15u;
      uint32_t kn = (krow[16 * b + (i >> 1)] >> (4 * (i & 1))) & 15u;
      S += e2m1_twice(qn) * e2m1_twice(kn);
    }
    D += ldexp((double)S, (int)st.u[h][b] + (int)((kscales >> (8 * b)) & 0xFFu) - 256);
  }
  return (float)D;
}

CSA2_DEV float f_of(uint32_t x) { return __uint_as_float(x); }
CSA2_DEV uint32_t u_of(float x) { return __float_as_uint(x); }

// 4x4 transpose of (register index nt) x (lane group g) for four registers.
CSA2_DEV void transpose4(float& r0, float& r1, float& r2, float& r3) {
  auto a = __builtin_amdgcn_permlane32_swap(u_of(r0), u_of(r2), false, false);
  auto b = __builtin_amdgcn_permlane32_swap(u_of(r1), u_of(r3), false, false);
  auto c = __builtin_amdgcn_permlane16_swap(a[0], b[0], false, false);
  auto d = __builtin_amdgcn_permlane16_swap(a[1], b[1], false, false);
  r0 = f_of(c[0]);
  r1 = f_of(c[1]);
  r2 = f_of(d[0]);
  r3 = f_of(d[1]);
}

struct KeyTile {
  uint4 codes[4];   // N-tile nt: 16 bytes of key (16nt + lane%16), block lane/16
                    // (32x32x64 form: [2n + s] = key (32n + lane%32), block 2s + lane/32)
  uint32_t sc[4];   // its E8M0 byte
  uint32_t own;     // the 4 E8M0 bytes of entry `lane` of the page
};

typedef float v16f __attribute__((ext_vector_type(16)));
template <int OA>
CSA2_DEV v16f mfma32_fp4(const uint4& a, const uint4& b, const v16f& c, int asc, int bsc) {
  const v8i av = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
  const v8i bv = {(int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, c, 4, 4, OA, asc, 0, bsc);
}

// One page of keys as B operands of the 32x32x64 form.
CSA2_DEV void load_keys32(KeyTile& t, const uint8_t* __restrict__ idx_codes, const uint8_t* __restrict__ idx_scales,
                          int page, int lane) {
  const int64_t slot0 = (int64_t)__builtin_amdgcn_readfirstlane(page) * kPage;  // uniform
  const uint32_t hf = (uint32_t)lane >> 5, n = (uint32_t)lane & 31u;
  const uint8_t* __restrict__ cb = idx_codes + slot0 * kIdxRowBytes;
  const uint8_t* __restrict__ sb = idx_scales + slot0 * kIdxScaleBytes;
#pragma unroll
  for (uint32_t i = 0; i < 4; ++i) {
    const uint32_t e = 32u * (i >> 1) + n, blk = 2u * (i & 1u) + hf;
    t.codes[i] = *reinterpret_cast<const uint4*>(cb + (e * (uint32_t)kIdxRowBytes + 16u * blk));
    t.sc[i] = sb[e * (uint32_t)kIdxScaleBytes + blk];
  }
  t.own = *reinterpret_cast<const uint32_t*>(sb + (uint32_t)lane * kIdxScaleBytes);
  __builtin_amdgcn_sched_barrier(0);
}

// One page of keys: a wavefront-uniform page base plus fixed 32-bit lane offsets,
// so every load takes the scalar-base + vector-offset form.
CSA2_DEV void load_keys(KeyTile& t, const uint8_t* __restrict__ idx_codes, const uint8_t* __restrict__ idx_scales,
                        int page, int lane) {
  const int64_t slot0 = (int64_t)__builtin_amdgcn_readfirstlane(page) * kPage;  // uniform
  const uint32_t g = (uint32_t)lane >> 4, n = (uint32_t)lane & 15u;
  const uint8_t* __restrict__ cb = idx_codes + slot0 * kIdxRowBytes;
  const uint8_t* __restrict__ sb = idx_scales + slot0 * kIdxScaleBytes;
#pragma unroll
  for (uint32_t nt = 0; nt < 4; ++nt) {
    const uint32_t e = 16u * nt + n;
    t.codes[nt] = *reinterpret_cast<const uint4*>(cb + (e * (uint32_t)kIdxRowBytes + 16u * g));
    t.sc[nt] = sb[e * (uint32_t)kIdxScaleBytes + g];
  }
  t.own = *reinterpret_cast<const uint32_t*>(sb + (uint32_t)lane * kIdxScaleBytes);
  // issue order = use order: the tile is waited for as a unit, oldest first
  __builtin_amdgcn_sched_barrier(0);
}

// Candidate pools: virtual page G holds pool positions 64G .. 64G+63, the members of
// pool blocks 8G .. 8G+7 (blocks of 8 consecutive entries; a block never crosses a
// 64-entry page).  Slot of position e of virtual page G; past the pool's end, or at a
// -1 block, it is a valid stand-in slot whose score is never written.
constexpr int kPoolBlock = 8;
CSA2_DEV int64_t pool_slot(const int32_t* __restrict__ pool_row, int npool, const int32_t* __restrict__ bt_seq,
                           int G, int e) {
  const int r = min(8 * G + (e >> 3), npool - 1);
  const int blk = max(pool_row[r], 0);
  const int64_t j = (int64_t)blk * kPoolBlock + (e & 7);
  return (int64_t)bt_seq[j >> 6] * kPage + (j & 63);
}

// One virtual page of a pool: the same operand layout as load_keys, gathered per lane.
CSA2_DEV void load_keys_pool(KeyTile& t, const uint8_t* __restrict__ idx_codes,
                             const uint8_t* __restrict__ idx_scales, const int32_t* __restrict__ pool_row,
                             int npool, const int32_t* __restrict__ bt_seq, int G, int lane) {
  const uint32_t g = (uint32_t)lane >> 4, n = (uint32_t)lane & 15u;
  int64_t sl[4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) sl[nt] = pool_slot(pool_row, npool, bt_seq, G, 16 * nt + (int)n);
  const int64_t so = pool_slot(pool_row, npool, bt_seq, G, lane);
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    t.codes[nt] = *reinterpret_cast<const uint4*>(idx_codes + sl[nt] * kIdxRowBytes + 16u * g);
    t.sc[nt] = idx_scales[sl[nt] * kIdxScaleBytes + g];
  }
  t.own = *reinterpret_cast<const uint32_t*>(idx_scales + so * kIdxScaleBytes);
  __builtin_amdgcn_sched_barrier(0);
}

// The same as B operands of the 32x32x64 form.
CSA2_DEV void load_keys_pool32(KeyTile& t, const uint8_t* __restrict__ idx_codes,
                               const uint8_t* __restrict__ idx_scales, const int32_t* __restrict__ pool_row,
                               int npool, const int32_t* __restrict__ bt_seq, int G, int lane) {
  const uint32_t hf = (uint32_t)lane >> 5, n = (uint32_t)lane & 31u;
  int64_t sl[2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) sl[nt] = pool_slot(pool_row, npool, bt_seq, G, 32 * nt + (int)n);
  const int64_t so = pool_slot(pool_row, npool, bt_seq, G, lane);
#pragma unroll
  for (uint32_t i = 0; i < 4; ++i) {
    const uint32_t blk = 2u * (i & 1u) + hf;
    t.codes[i] = *reinterpret_cast<const uint4*>(idx_codes + sl[i >> 1] * kIdxRowBytes + 16u * blk);
    t.sc[i] = idx_scales[sl[i >> 1] * kIdxScaleBytes + blk];
  }
  t.own = *reinterpret_cast<const uint32_t*>(idx_scales + so * kIdxScaleBytes);
  __builtin_amdgcn_sched_barrier(0);
}

// Pool positions that hold a visible entry: a prefix of the row (its blocks are in
// ascending order, so only the last valid one can be the sequence's partial block).
CSA2_DEV int pool_visible(const int32_t* __restrict__ pool_row, int npool, int n_visible) {
  const int nb = (n_visible + kPoolBlock - 1) / kPoolBlock;
  const int nvalid = min(npool, nb);
  if (nvalid == 0) return 0;
  const int tail = n_visible % kPoolBlock;
  return (pool_row[nvalid - 1] == nb - 1 && tail != 0) ? kPoolBlock * (nvalid - 1) + tail : kPoolBlock * nvalid;
}

// Scores of one page for one query of the tile: 64 entries starting at logical entry
// G * 64 of the query's sequence, whose keys are in `cur` (physical first slot slot0).
// Returns whether this lane's entry lies outside the window where the MFMA result is
// exact; the caller then recomputes it with exact_entry() after the page loop.
// With lh (uniform), every score written (except those left to the exact path) is
// also counted in the workgroup's digit-1 histogram lh of the selection that follows.
template <int MT>
__device__ __attribute__((always_inline)) inline bool score_page(const QStage<MT>& s, const KeyTile& cur, int G,
                                                                 const float* __restrict__ wq,
                                                                 float* __restrict__ srow, int lane, uint32_t* lh,
                                                                 float& score_out) {
  const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
  int q_span = 0, q_umin = 255, q_umax = 0;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const uint32_t sv = s.stat[mt];
    q_span = max(q_span, (int)(sv & 0xFFu));
    q_umin = min(q_umin, (int)((sv >> 8) & 0xFFu));
    q_umax = max(q_umax, (int)((sv >> 16) & 0xFFu));
  }
  // 16x16 complete dots per MFMA: d[mt][nt][r] = d(head(mt, 4*(lane/16)+r), entry 16nt + lane%16)
  float d[MT][4][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const uint4 qa = s.codes[mt][lane];
    const v8i a = {(int)qa.x, (int)qa.y, (int)qa.z, (int)qa.w, 0, 0, 0, 0};
    const int asc = (int)s.scale[mt >> 2][lane];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const v8i b = {(int)cur.codes[nt].x, (int)cur.codes[nt].y, (int)cur.codes[nt].z, (int)cur.codes[nt].w,
                     0, 0, 0, 0};
      v4f acc;
      switch (mt & 3) {
        case 0: acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, zero, 4, 4, 0, asc, 0, (int)cur.sc[nt]); break;
        case 1: acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, zero, 4, 4, 1, asc, 0, (int)cur.sc[nt]); break;
        case 2: acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, zero, 4, 4, 2, asc, 0, (int)cur.sc[nt]); break;
        default: acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, zero, 4, 4, 3, asc, 0, (int)cur.sc[nt]); break;
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) d[mt][nt][r] = acc[r];
    }
  }
  // lane L <- entry L of the page, register (b, mt, r) <- head b*4MT + 4mt + r
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) transpose4(d[mt][0][r], d[mt][1][r], d[mt][2][r], d[mt][3][r]);

  const int j = G * kPage + lane;
  const uint32_t own = cur.own;
  int kmin = 255, kmax = 0;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int u = (int)((own >> (8 * b)) & 0xFFu);
    kmin = u < kmin ? u : kmin;
    kmax = u > kmax ? u : kmax;
  }
  const bool visible = j < s.nvis;
  const bool exact_needed = visible & (((kmax - kmin) + q_span > kMaxSpread) | (q_umin + kmin < kMinExpSum) |
                                       (q_umax + kmax > kMaxExpSum));
  float acc = 0.0f;
#pragma unroll
  for (int b = 0; b < 4; ++b)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc = fmaf(wq[b * 4 * MT + 4 * mt + r], relu(d[mt][b][r]), acc);
  if (visible) srow[j] = acc;
  if (lh != nullptr && visible && !exact_needed) atomicAdd(&lh[score_key(acc) >> kTopkBinShift], 1u);
  score_out = acc;
  return exact_needed;
}

// score_page with the 32x32x64 form, for Hi a multiple of 32: per 32-head tile m and
// 32-entry tile n, two chained MFMAs (K = 64 each) give D[head row][entry], lane l
// holding entry l%32 and rows 8q + 4(l/32) + i (register 4q + i).  One
// v_permlane32_swap per register pair of the two entry tiles then leaves lane l with
// entry l of the page: rows 8q + i in the first register of the pair and 8q + 4 + i in
// the second, so the fma chain reads every head in ascending order.  The exactness
// window is the one of score_page: inside it both K halves and their sum are exact.
template <int MT>
__device__ __attribute__((always_inline)) inline bool score_page32(const QStage<MT>& s, const KeyTile& cur, int G,
                                                                   const float* __restrict__ wq,
                                                                   float* __restrict__ srow, int lane, uint32_t* lh,
                                                                   float& score_out) {
  static_assert(MT % 2 == 0, "the 32x32x64 form needs Hi a multiple of 32");
  constexpr int M32 = MT / 2;
  int q_span = 0, q_umin = 255, q_umax = 0;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const uint32_t sv = s.stat[mt];
    q_span = max(q_span, (int)(sv & 0xFFu));
    q_umin = min(q_umin, (int)((sv >> 8) & 0xFFu));
    q_umax = max(q_umax, (int)((sv >> 16) & 0xFFu));
  }
  const int j = G * kPage + lane;
  const uint32_t own = cur.own;
  int kmin = 255, kmax = 0;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int u = (int)((own >> (8 * b)) & 0xFFu);
    kmin = u < kmin ? u : kmin;
    kmax = u > kmax ? u : kmax;
  }
  const bool visible = j < s.nvis;
  const bool exact_needed = visible & (((kmax - kmin) + q_span > kMaxSpread) | (q_umin + kmin < kMinExpSum) |
                                       (q_umax + kmax > kMaxExpSum));
  // one 32-head tile at a time (its 32 dots per lane, then its part of the chain):
  // fewer live registers than holding every tile's dots
  const v16f zero = {};
  float acc = 0.0f;
#pragma unroll
  for (int m = 0; m < M32; ++m) {
    float d[2][16];
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      v16f t = zero;
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int p = 2 * m + k;
        const uint4 a = s.codes32[m][k][lane];
        const int asc = (int)s.scale32[p >> 2][lane];
        const int bsc = (int)cur.sc[2 * n + k];
        switch (p & 3) {
          case 0: t = mfma32_fp4<0>(a, cur.codes[2 * n + k], t, asc, bsc); break;
          case 1: t = mfma32_fp4<1>(a, cur.codes[2 * n + k], t, asc, bsc); break;
          case 2: t = mfma32_fp4<2>(a, cur.codes[2 * n + k], t, asc, bsc); break;
          default: t = mfma32_fp4<3>(a, cur.codes[2 * n + k], t, asc, bsc); break;
        }
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) d[n][r] = t[r];
    }
    // lane l <- entry l: rows 8q + i in d[0][4q + i], rows 8q + 4 + i in d[1][4q + i]
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const auto v = __builtin_amdgcn_permlane32_swap(u_of(d[0][r]), u_of(d[1][r]), false, false);
      d[0][r] = f_of(v[0]);
      d[1][r] = f_of(v[1]);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
#pragma unroll
      for (int i = 0; i < 4; ++i) acc = fmaf(wq[32 * m + 8 * q + i], relu(d[0][4 * q + i]), acc);
#pragma unroll
      for (int i = 0; i < 4; ++i) acc = fmaf(wq[32 * m + 8 * q + 4 + i], relu(d[1][4 * q + i]), acc);
    }
  }
  if (visible) srow[j] = acc;
  if (lh != nullptr && visible && !exact_needed) atomicAdd(&lh[score_key(acc) >> kTopkBinShift], 1u);
  score_out = acc;
  return exact_needed;
}

// Page loads and scores in the form the head count takes: 32x32x64 when Hi is a
// multiple of 32, 16x16x128 otherwise.
template <int MT>
CSA2_DEV void load_page(KeyTile& t, const uint8_t* __restrict__ idx_codes, const uint8_t* __restrict__ idx_scales,
                        int page, int lane) {
  if constexpr (MT % 2 == 0) load_keys32(t, idx_codes, idx_scales, page, lane);
  else load_keys(t, idx_codes, idx_scales, page, lane);
}
template <int MT>
CSA2_DEV void load_page_pool(KeyTile& t, const uint8_t* __restrict__ idx_codes, const uint8_t* __restrict__ idx_scales,
                             const int32_t* __restrict__ pool_row, int npool, const int32_t* __restrict__ bt_seq,
                             int G, int lane) {
  if constexpr (MT % 2 == 0) load_keys_pool32(t, idx_codes, idx_scales, pool_row, npool, bt_seq, G, lane);
  else load_keys_pool(t, idx_codes, idx_scales, pool_row, npool, bt_seq, G, lane);
}
template <int MT>
__device__ __attribute__((always_inline)) inline bool score_any(const QStage<MT>& s, const KeyTile& cur, int G,
                                                                const float* __restrict__ wq,
                                                                float* __restrict__ srow, int lane, uint32_t* lh,
                                                                float& score_out) {
  if constexpr (MT % 2 == 0) return score_page32<MT>(s, cur, G, wq, srow, lane, lh, score_out);
  else return score_page<MT>(s, cur, G, wq, srow, lane, lh, score_out);
}

// The definition itself for one entry (integer block sums, one rounding per head,
// the fma chain), for the rare entries flagged by score_page.
template <int MT>
CSA2_DEV float exact_entry(const QStage<MT>& s, const uint8_t* __restrict__ idx_codes,
                           const uint8_t* __restrict__ idx_scales, int64_t slot, const float* __restrict__ wq,
                           float* __restrict__ dst) {
  constexpr int HI = 16 * MT;
  const uint8_t* krow = idx_codes + slot * kIdxRowBytes;
  const uint32_t own = *reinterpret_cast<const uint32_t*>(idx_scales + slot * kIdxScaleBytes);
  float acc = 0.0f;
  for (int h = 0; h < HI; ++h) acc = fmaf(wq[h], relu(exact_dot<MT>(s, h, krow, own)), acc);
  *dst = acc;
  return acc;
}

// HIST (one query per workgroup only): also fill the query's digit-1 histogram
// (copy blockIdx.x % ncopies of hist[q]) of the selection that follows, when
// n_visible[q] > k.
// PB (with HIST, one query per workgroup): also the block maxima of the candidate
// pool that index_pool_build derives from these scores: for each block of 8
// consecutive entries with a visible member, bmax[q][block] = the largest score of its
// visible members (the eight lanes of a page that hold the block, combined with
// DPP), its digit-1 bin counted in copy blockIdx.x % bcopies of bhist[q] when the row
// has more blocks than npool, and nblocks[q] = ceil(n_visible[q] / 8).
// POOL: the row of each query is its candidate pool (pool [nq][npool] blocks of 8
// entries, ld = 8 npool); position p scores member p % 8 of block pool[q][p / 8], and
// workgroup 0 of each query writes the count of visible positions to pool_nvis[q].
template <int MT, int QT, bool HIST, bool POOL = false, bool PB = false>
__global__ __launch_bounds__(kThreads) void index_score_kernel(const uint8_t* __restrict__ idx_codes,
                                                          const uint8_t* __restrict__ idx_scales,
                                                          const uint16_t* __restrict__ q_idx,
                                                          const float* __restrict__ w,
                                                          const int32_t* __restrict__ seq_of_query,
                                                          const int32_t* __restrict__ n_visible,
                                                          const int32_t* __restrict__ block_table, int max_pages,
                                                          int nq, float* __restrict__ scores, int64_t ld,
                                                          int groups_per_wave, int total_groups,
                                                          uint32_t* __restrict__ hist, int k, int ncopies,
                                                          const int32_t* __restrict__ pool, int npool,
                                                          int32_t* __restrict__ pool_nvis, float* __restrict__ bmax,
                                                          int64_t ldb, uint32_t* __restrict__ bhist, int bcopies,
                                                          int32_t* __restrict__ nblocks) {
  static_assert(!HIST || QT == 1, "the fused histogram serves one query per workgroup");
  static_assert(!PB || (HIST && !POOL), "block maxima come from the fused scan of a whole row");
  static_assert(!POOL || QT == 1, "candidate pools are scanned one query per workgroup");
  constexpr int qt = QT;  // queries per workgroup
  constexpr int HI = 16 * MT;
  extern __shared__ __align__(16) unsigned char smem[];
  QStage<MT>* st = reinterpret_cast<QStage<MT>*>(smem);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform across the wavefront
  const int q0 = blockIdx.y * qt;
  const int gfirst = (blockIdx.x * kWaves + wid) * groups_per_wave;
  const int gend = min(gfirst + groups_per_wave, total_groups);
  const int first_row = (q0 < nq) ? (seq_of_query ? seq_of_query[q0] : q0) : 0;

  // ---- physical pages of this wavefront (uniform table reads), the raw query
  // blocks this thread stages, then the first two pages of keys: all in flight
  // together before any of them is used
  const int items = qt * MT * 64;
  // the staging item of this thread, (query, M-tile, lane) -> source block
  auto item_src = [&](int item, const uint16_t*& src) {
    const int qi = item / (MT * 64), rem = item % (MT * 64), mt = rem >> 6, l = rem & 63;
    const int q = q0 + qi;
    src = q_idx + ((int64_t)q * HI + head_of<MT>(mt, l & 15)) * kIndexDim + 32 * (l >> 4);
    return item < items && q < nq;
  };
  // per-query row and visible count (threads tid < qt)
  int my_row = 0, my_nvis = 0;
  if (tid < qt && q0 + tid < nq) {
    my_row = seq_of_query ? seq_of_query[q0 + tid] : q0 + tid;
    my_nvis = n_visible[q0 + tid];
    if (POOL) {
      my_nvis = pool_visible(pool + (int64_t)(q0 + tid) * npool, npool, my_nvis);
      if (blockIdx.x == 0) pool_nvis[q0 + tid] = my_nvis;
    }
  }
  QRaw qraw;  // the first round of staging loads goes out before the key loads
  {
    const uint16_t* src;
    const bool ok = item_src(tid, src);
    mx32_load(ok ? src : q_idx, qraw);  // unconditional (a spare thread reads block 0)
  }
  __builtin_amdgcn_sched_barrier(0);  // keep these loads ahead of the key loads
  // physical page of the wavefront's k-th page (a uniform scalar read each time:
  // an indexed register array would make every later wait conservative)
  const int32_t* __restrict__ bt_row = block_table + (int64_t)first_row * max_pages + gfirst;
  const int npg_all = max(min(gend - gfirst, kMaxPagesPerWave), 1);
  auto page_of = [&](int k) { return gfirst < gend ? bt_row[min(k, npg_all - 1)] : 0; };

  // the wavefront's pages, unconditionally (past its last page -- or with no page at
  // all -- it re-reads a valid page and ignores the data), two in flight at a time:
  // pages 0 and 1 now, page 2 into t0 once page 0 is scored, page 3 into t1 once
  // page 1 is.  Two pages per wavefront keep about 17 MB in flight over the chip at
  // batch 1, enough for the HBM rate, while the query blocks that every workgroup
  // stages first do not queue behind the whole scan's bytes.
  KeyTile t0, t1;
  // the four page numbers are read now.  Every wavefront requests its first pages
  // after the staging: key loads issued earlier queue ahead of the staging's query
  // loads in the compute unit's memory pipeline and delay the first page more than
  // they save (measured at 1M entries, one query: 0.5 us per index_topk call).
  const int pg0 = POOL ? 0 : page_of(0), pg1 = POOL ? 0 : page_of(1), pg2 = POOL ? 0 : page_of(2),
            pg3 = POOL ? 0 : page_of(3);
  const int32_t* __restrict__ pool_row = POOL ? pool + (int64_t)q0 * npool : nullptr;
  const int32_t* __restrict__ bt_seq = block_table + (int64_t)first_row * max_pages;
  auto vpage = [&](int k) { return gfirst + min(k, npg_all - 1); };  // pools: virtual page of the k-th
  // page k of the wavefront into t (k = 0 .. 3)
  auto request_page = [&](KeyTile& t, int k, int pg) __attribute__((always_inline)) {
    if (POOL) load_page_pool<MT>(t, idx_codes, idx_scales, pool_row, npool, bt_seq, vpage(k), lane);
    else load_page<MT>(t, idx_codes, idx_scales, pg, lane);
  };
  auto request_pages = [&]() __attribute__((always_inline)) {
    request_page(t0, 0, pg0);
    request_page(t1, 1, pg1);
  };

  // ---- stage the tile's queries: MXFP4 operands and scales.  Item = (query,
  // M-tile, lane); the 64 items of one (query, M-tile) are one wavefront, whose lanes
  // l, l^16, l^32, l^48 hold the four blocks of one head.
  for (int item0 = 0; item0 < items; item0 += kThreads) {
    const int item = item0 + tid;
    const int qi = item / (MT * 64), rem = item % (MT * 64), mt = rem >> 6, l = rem & 63;
    const int g = l >> 4, rho = l & 15, h = head_of<MT>(mt, rho);
    uint4 codes = make_uint4(0, 0, 0, 0);
    uint32_t u = 127;
    const uint16_t* src;
    if (item_src(item, src)) {
      if (item0 > 0) mx32_load(src, qraw);
      mx32_block(qraw, codes, u);
    }
    int lo = (int)u, hi = (int)u;  // over the head's four blocks
    lo = min(lo, __shfl_xor(lo, 16));
    hi = max(hi, __shfl_xor(hi, 16));
    lo = min(lo, __shfl_xor(lo, 32));
    hi = max(hi, __shfl_xor(hi, 32));
    int span = hi - lo;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {  // over the wavefront's 16 heads
      span = max(span, __shfl_xor(span, o));
      lo = min(lo, __shfl_xor(lo, o));
      hi = max(hi, __shfl_xor(hi, o));
    }
    if (item < items) {
      st[qi].codes[mt][l] = codes;
      st[qi].u[h][g] = (uint8_t)u;
      reinterpret_cast<uint8_t*>(&st[qi].scale[mt >> 2][l])[mt & 3] = (uint8_t)u;
      if (MT % 2 == 0) {  // head h, block g -> tile h/32, step g/2, lane h%32 + 32 (g%2)
        const int l32 = (h & 31) + 32 * (g & 1), p32 = 2 * (h >> 5) + (g >> 1);
        st[qi].codes32[h >> 5][g >> 1][l32] = codes;
        reinterpret_cast<uint8_t*>(&st[qi].scale32[p32 >> 2][l32])[p32 & 3] = (uint8_t)u;
      }
      if (l == 0) st[qi].stat[mt] = (uint32_t)span | ((uint32_t)lo << 8) | ((uint32_t)hi << 16);
    }
  }
  if (tid < qt) {
    st[tid].row = my_row;
    st[tid].nvis = my_nvis;
  }
  uint32_t* lh = reinterpret_cast<uint32_t*>(smem + sizeof(QStage<MT>) * qt);  // HIST only
  uint32_t* lhb = lh + kTopkBins;                                                 // PB only: block maxima
  if (HIST)
#pragma unroll
    for (int i = 0; i < kTopkBins / kThreads; ++i) lh[tid + i * kThreads] = 0u;
  if (PB)
#pragma unroll
    for (int i = 0; i < kTopkBins / kThreads; ++i) lhb[tid + i * kThreads] = 0u;
  request_pages();
  lds_barrier();
  const bool hist_on = HIST && q0 < nq && st[0].nvis > k;  // uniform (rows with n <= k need none)
  // block maxima: a row with at most npool blocks keeps them all and needs no counts
  const bool pb_on = PB && q0 < nq && (st[0].nvis + kPoolBlock - 1) / kPoolBlock > npool;
  if (PB && tid == 0 && blockIdx.x == 0 && q0 < nq) nblocks[q0] = (st[0].nvis + kPoolBlock - 1) / kPoolBlock;
  float ks0 = 0.0f, ks1 = 0.0f, ks2 = 0.0f, ks3 = 0.0f;  // this lane's score on each page (PB)
  if (gfirst < gend) {
  const int npg = gend - gfirst;
  bool same_row = true;  // every query of the tile reads the first query's sequence
  for (int qi = 1; qi < qt; ++qi) same_row &= (q0 + qi >= nq) || (st[qi].row == first_row);

  // entries needing the exact path: bit (i * qt + qi) for page i, query qi
  unsigned long long exact_bits = 0ull;
  // all queries of the tile on one page whose keys are in t
  auto page_all = [&](const KeyTile& t, int i, float& ks) __attribute__((always_inline)) {
    const int G = gfirst + i;
#pragma unroll 1
    for (int qi = 0; qi < qt; ++qi) {
      const QStage<MT>& sq = st[qi];
      if (G * kPage >= sq.nvis) continue;  // uniform
      const bool ex = score_any<MT>(sq, t, G, w + (int64_t)(q0 + qi) * HI, scores + (int64_t)(q0 + qi) * ld,
                                     lane, hist_on ? lh : nullptr, ks);
      exact_bits |= (unsigned long long)ex << (i * qt + qi);
    }
  };

  if (same_row) {
    // the wavefront's (at most four) pages, all requested in the prologue, in
    // straight-line code: the wait for page k leaves pages k+1.. in flight (a loop
    // here would make the compiler wait for every outstanding load at its head)
    page_all(t0, 0, ks0);
    request_page(t0, 2, pg2);
    if (npg > 1) page_all(t1, 1, ks1);
    request_page(t1, 3, pg3);
    if (npg > 2) page_all(t0, 2, ks2);
    if (npg > 3) page_all(t1, 3, ks3);
    // rare: entries whose blocks fall outside the exact window of the MFMA
    while (exact_bits != 0ull) {
      const int b = __builtin_ctzll(exact_bits);
      exact_bits &= exact_bits - 1;
      const int i = b / qt, qi = b % qt;
      const int64_t slot = POOL ? pool_slot(pool_row, npool, bt_seq, gfirst + i, lane)
                                : (int64_t)page_of(i) * kPage + lane;
      const float e = exact_entry<MT>(st[qi], idx_codes, idx_scales, slot, w + (int64_t)(q0 + qi) * HI,
                                      scores + (int64_t)(q0 + qi) * ld + (int64_t)(gfirst + i) * kPage + lane);
      count_exact_path();
      if (HIST && hist_on) atomicAdd(&lh[score_key(e) >> kTopkBinShift], 1u);
      if (PB) {
        if (i == 0) ks0 = e;
        else if (i == 1) ks1 = e;
        else if (i == 2) ks2 = e;
        else ks3 = e;
      }
    }
    if (PB && q0 < nq) {
      // block maxima of this wavefront's pages: lanes 8b' .. 8b'+7 hold block b' of a
      // page; quad swaps and the half-row mirror give each lane its block's maximum
      const float ksv[kMaxPagesPerWave] = {ks0, ks1, ks2, ks3};
      const int nvis = st[0].nvis;
#pragma unroll
      for (int i = 0; i < kMaxPagesPerWave; ++i) {
        if (i < npg) {  // uniform
          const int64_t j = (int64_t)(gfirst + i) * kPage + lane;
          float v = j < nvis ? ksv[i] : -INFINITY;
          v = fmaxf(v, dpp_f<0xB1>(v));
          v = fmaxf(v, dpp_f<0x4E>(v));
          v = fmaxf(v, dpp_f<0x141>(v));
          if ((lane & 7) == 0 && j < nvis) {
            bmax[(int64_t)q0 * ldb + (j >> 3)] = v;
            if (pb_on) atomicAdd(&lhb[score_key(v) >> kTopkBinShift], 1u);
          }
        }
      }
    }
  } else {
    // queries of several sequences share the tile: each query reads its own pages
    for (int i = 0; i < npg; ++i) {
      const int G = gfirst + i;
      for (int qi = 0; qi < qt; ++qi) {
        const QStage<MT>& sq = st[qi];
        if (G * kPage >= sq.nvis) continue;  // uniform
        const int page = block_table[(int64_t)sq.row * max_pages + G];
        const int64_t slot0 = (int64_t)page * kPage;
        KeyTile t;
        load_page<MT>(t, idx_codes, idx_scales, page, lane);
        float unused;
        if (score_any<MT>(sq, t, G, w + (int64_t)(q0 + qi) * HI, scores + (int64_t)(q0 + qi) * ld, lane,
                           nullptr, unused)) {
          exact_entry<MT>(sq, idx_codes, idx_scales, slot0 + lane, w + (int64_t)(q0 + qi) * HI,
                          scores + (int64_t)(q0 + qi) * ld + (int64_t)G * kPage + lane);
          count_exact_path();
        }
      }
    }
  }
  }  // gfirst < gend
  if (HIST && hist_on) {  // every wavefront is done: add the workgroup's counts
    __syncthreads();
    uint32_t* gh = hist + ((size_t)q0 * kTopkHistCopies + blockIdx.x % ncopies) * kTopkBins;
#pragma unroll
    for (int i = 0; i < kTopkBins / kThreads; ++i) {
      const uint32_t c = lh[tid + i * kThreads];
      if (c) atomicAdd(&gh[tid + i * kThreads], c);
    }
  }
  if (PB && pb_on) {  // the block maxima's counts, into the pool selection's histogram
    __syncthreads();
    uint32_t* gb = bhist + ((size_t)q0 * kTopkHistCopies + blockIdx.x % bcopies) * kTopkBins;
#pragma unroll
    for (int i = 0; i < kTopkBins / kThreads; ++i) {
      const uint32_t c = lhb[tid + i * kThreads];
      if (c) atomicAdd(&gb[tid + i * kThreads], c);
    }
  }
}

// ---- scan for queries that share a sequence: two queries per wavefront ----------
// The 32 rows of an M-tile of the 32x32x64 MFMA are (query, head) pairs: two queries
// of 16 heads.  Its output leaves lane l the 16 dots of query l/32 with entry l%32
// for heads 16mt .. 16mt+15, so over the Hi/16 M-tiles a lane holds every head of its
// (query, entry) pair in head order and the weighted ReLU sum needs no lane exchange.
// (On gfx950 the FP4 form of this shape runs at about twice the rate of the
// 16x16x128 one.)  The eight wavefronts of a workgroup (16 queries) share each page
// of keys, staged once in LDS and read as the B operand; each wavefront's queries
// stay in registers as MXFP4 A operands for the whole page range.
constexpr int kQ4Queries = 2 * kWaves;  // queries per workgroup
constexpr int kQ4MinPages = 8;          // fewest pages per workgroup (amortises the query staging)

constexpr int kQ4Group = 4;  // pages staged per workgroup barrier

struct Q4Page {
  uint4 codes[kPage * 4];  // 16-byte chunk c of entry e at 4e + (c ^ ((e >> 2) & 3)): conflict-free reads
  uint32_t sc[kPage];      // entry e: its four E8M0 block exponents (byte b = block b)
  uint32_t estat[kPage];   // entry e: smallest | largest << 8 of its four block exponents
  uint32_t pstat;          // over the page: largest entry span | smallest << 8 | largest << 16
  uint32_t pad[3];
};
struct Q4Smem {
  Q4Page slot[2][kQ4Group];
  int row[kQ4Queries];
  int nvis[kQ4Queries];
};

// A staging step's share of thread tid (pages G .. G + kQ4Group - 1 of the row):
// code chunk tid%256 of pages wid/4 and 2 + wid/4 and the block exponents of entries
// 4(lane%16) .. +3 of page lane/16 (stored by wavefront 0).  Pages at or past Gend
// re-read page Gend - 1; their slots are never read.
typedef uint32_t v4u __attribute__((ext_vector_type(4)));
struct Q4Regs {
  v4u c0, c1;  // pages wid/4 and 2 + wid/4
  v4u s;
};
static_assert(kQ4Group == 4 && kThreads == 512, "staging shares: two code chunks per thread, one scale row per page");

CSA2_DEV void q4_load(Q4Regs& r, const uint8_t* __restrict__ idx_codes, const uint8_t* __restrict__ idx_scales,
                      const int32_t* __restrict__ bt, int G, int Gend, int wid, int lane) {
  const int last = Gend - 1;  // page numbers: uniform scalar reads
  const int pg0 = bt[min(G, last)], pg1 = bt[min(G + 1, last)], pg2 = bt[min(G + 2, last)],
            pg3 = bt[min(G + 3, last)];
  // every wavefront reads the exponent rows (the same 1 KB, served by its L1) though
  // only wavefront 0 stores them: with no load under a condition, each wait below
  // counts exactly the loads issued after the one it waits for
  {
    const int q = lane >> 4;
    const int pg = q == 0 ? pg0 : (q == 1 ? pg1 : (q == 2 ? pg2 : pg3));
    r.s = *reinterpret_cast<const v4u*>(idx_scales + (int64_t)pg * kPage * kIdxScaleBytes +
                                        (uint32_t)(lane & 15) * 16u);
  }
  const uint32_t off = (uint32_t)(((wid & 3) << 6) | lane) * 16u;
  const int pa = (wid >> 2) ? pg1 : pg0, pb = (wid >> 2) ? pg3 : pg2;
  r.c0 = *reinterpret_cast<const v4u*>(idx_codes + (int64_t)pa * kPage * kIdxRowBytes + off);
  r.c1 = *reinterpret_cast<const v4u*>(idx_codes + (int64_t)pb * kPage * kIdxRowBytes + off);
}

template <int C>
CSA2_DEV int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, C, 0xF, 0xF, true);
}

CSA2_DEV void q4_store(Q4Page (&slot)[kQ4Group], const Q4Regs& r, int wid, int lane) {
  {
    const int p = wid >> 2, t = ((wid & 3) << 6) | lane, e = t >> 2, c = t & 3;
    const int at = 4 * e + (c ^ ((e >> 2) & 3));
    *reinterpret_cast<v4u*>(&slot[p].codes[at]) = r.c0;
    *reinterpret_cast<v4u*>(&slot[p + 2].codes[at]) = r.c1;
  }
  if (wid == 0) {  // 16-lane row p holds page p
    const int p = lane >> 4, i = lane & 15;
    const uint32_t wd[4] = {r.s[0], r.s[1], r.s[2], r.s[3]};
    uint32_t es[4];
    int span = 0, lo_all = 255, hi_all = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int lo = 255, hi = 0;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int u = (int)((wd[j] >> (8 * b)) & 0xFFu);
        lo = min(lo, u);
        hi = max(hi, u);
      }
      es[j] = (uint32_t)lo | ((uint32_t)hi << 8);
      span = max(span, hi - lo);
      lo_all = min(lo_all, lo);
      hi_all = max(hi_all, hi);
    }
    *reinterpret_cast<v4u*>(&slot[p].sc[4 * i]) = r.s;
    const v4u esv = {es[0], es[1], es[2], es[3]};
    *reinterpret_cast<v4u*>(&slot[p].estat[4 * i]) = esv;
    // over the row's 16 lanes: quad swaps, then half-row and row mirrors
    span = max(span, dpp_i<0xB1>(span));
    lo_all = min(lo_all, dpp_i<0xB1>(lo_all));
    hi_all = max(hi_all, dpp_i<0xB1>(hi_all));
    span = max(span, dpp_i<0x4E>(span));
    lo_all = min(lo_all, dpp_i<0x4E>(lo_all));
    hi_all = max(hi_all, dpp_i<0x4E>(hi_all));
    span = max(span, dpp_i<0x141>(span));
    lo_all = min(lo_all, dpp_i<0x141>(lo_all));
    hi_all = max(hi_all, dpp_i<0x141>(hi_all));
    span = max(span, dpp_i<0x140>(span));
    lo_all = min(lo_all, dpp_i<0x140>(lo_all));
    hi_all = max(hi_all, dpp_i<0x140>(hi_all));
    if (i == 0) slot[p].pstat = (uint32_t)span | ((uint32_t)lo_all << 8) | ((uint32_t)hi_all << 16);
  }
}

// Whether the MFMA dot of a query (largest head span qs, exponents in [qlo, qhi]) with
// keys of span ks and exponents in [klo, khi] may be inexact.
CSA2_DEV bool q4_inexact(int qs, int qlo, int qhi, int ks, int klo, int khi) {
  return (ks + qs > kMaxSpread) | (qlo + klo < kMinExpSum) | (qhi + khi > kMaxExpSum);
}

// The definition itself for one (query, entry) pair: each query block is quantised
// again from its bf16 values by the element rule (the codes and exponent of the MFMA
// operand), integer block sums, fp64 combination in block order, one rounding per
// head, the fma chain in head order.
CSA2_DEV float q4_exact(const uint16_t* __restrict__ qrow, const float* __restrict__ wq, int hi_count,
                        const uint8_t* __restrict__ krow, uint32_t kscales) {
  float acc = 0.0f;
  for (int h = 0; h < hi_count; ++h) {
    double D = 0.0;
    for (int b = 0; b < 4; ++b) {
      const uint16_t* src = qrow + h * kIndexDim + 32 * b;
      uint32_t amax = 0;
      for (int i = 0; i < 32; ++i) amax = max(amax, (uint32_t)src[i] & 0x7FFFu);
      const uint32_t u = mx_exponent(bf16_to_f32(amax));
      const float X = ldexpf(1.0f, (int)u - 127);
      int S = 0;
      for (int i = 0; i < 32; ++i) {
        const uint32_t qn = e2m1_code(bf16_to_f32(src[i]), X);
        const uint32_t kn = (krow[16 * b + (i >> 1)] >> (4 * (i & 1))) & 15u;
        S += e2m1_twice(qn) * e2m1_twice(kn);
      }
      D += ldexp((double)S, (int)u + (int)((kscales >> (8 * b)) & 0xFFu) - 256);
    }
    acc = fmaf(wq[h], relu((float)D), acc);
  }
  return acc;
}



// NM = Hi / 16 M-tiles; Hi <= 64 keeps a wavefront's operands and weights in registers.
template <int NM>
__global__ __launch_bounds__(kThreads) void index_score_q2_kernel(
    const uint8_t* __restrict__ idx_codes, const uint8_t* __restrict__ idx_scales, const uint16_t* __restrict__ q_idx,
    const float* __restrict__ w, const int32_t* __restrict__ seq_of_query, const int32_t* __restrict__ n_visible,
    const int32_t* __restrict__ block_table, int max_pages, int nq, float* __restrict__ scores, int64_t ld,
    int pages_per_wg) {
  constexpr int HI = 16 * NM;
  constexpr int NSC = (2 * NM + 3) / 4;
  constexpr int S = 2 * NM;  // (N-tile, M-tile) steps of a page
  __shared__ Q4Smem sm;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5, col = lane & 31;
  const int q0 = blockIdx.y * kQ4Queries;
  const int G0 = blockIdx.x * pages_per_wg;
  if (tid < kQ4Queries) {
    const int q = q0 + tid;
    sm.row[tid] = q < nq ? seq_of_query[q] : -1;
    sm.nvis[tid] = q < nq ? (int)min((int64_t)n_visible[q], ld) : 0;
  }

  // A operands: lane l holds row l%32 = (query 2 wid + (l%32)/4 % 2, head 16 mt +
  // 4 ((l%32)/8) + l%4) and, for K-half kh of the MFMA, block 2 kh + l/32
  const int qa_raw = q0 + 2 * wid + ((col >> 2) & 1);
  const bool qa_ok = qa_raw < nq;
  const int qa = qa_ok ? qa_raw : nq - 1;  // a spare row quantises a valid query and is zeroed
  const int head_in_tile = 4 * (col >> 3) + (col & 3);
  uint4 A[NM][2];
  uint32_t asc[NSC];
#pragma unroll
  for (int i = 0; i < NSC; ++i) asc[i] = 0u;
  int span = 0, lo_all = 255, hi_all = 0;
#pragma clang loop unroll(full)
  for (int mt = 0; mt < NM; ++mt) {
    QRaw raw[2];
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
      mx32_load(q_idx + ((int64_t)qa * HI + 16 * mt + head_in_tile) * kIndexDim + 32 * (2 * kh + half), raw[kh]);
    int lo = 255, hi = 0;
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      uint4 c;
      uint32_t u;
      mx32_block(raw[kh], c, u);
      if (!qa_ok) {
        c = make_uint4(0u, 0u, 0u, 0u);
        u = 127u;
      }
      A[mt][kh] = c;
      const int sl = 2 * mt + kh;
      asc[sl >> 2] |= u << (8 * (sl & 3));
      lo = min(lo, (int)u);
      hi = max(hi, (int)u);
    }
    lo = min(lo, __shfl_xor(lo, 32));  // the head's other two blocks
    hi = max(hi, __shfl_xor(hi, 32));
    span = max(span, hi - lo);
    lo_all = min(lo_all, lo);
    hi_all = max(hi_all, hi);
  }
#pragma unroll
  for (int o = 1; o < 32; o <<= 1) {  // over the query's heads (lane bits 0, 1, 3, 4)
    if (o == 4) continue;
    span = max(span, __shfl_xor(span, o));
    lo_all = min(lo_all, __shfl_xor(lo_all, o));
    hi_all = max(hi_all, __shfl_xor(hi_all, o));
  }
  // output side: lane l serves query 2 wid + l/32, whose statistics lane 4(l/32) holds
  const int q_span = __shfl(span, 4 * half), q_lo = __shfl(lo_all, 4 * half), q_hi = __shfl(hi_all, 4 * half);
  const int qo = q0 + 2 * wid + half;
  float wr[HI];
  {
    const float4* wsrc = reinterpret_cast<const float4*>(w + (int64_t)(qo < nq ? qo : nq - 1) * HI);
#pragma unroll
    for (int i = 0; i < HI / 4; ++i) {
      const float4 v = wsrc[i];
      wr[4 * i] = v.x;
      wr[4 * i + 1] = v.y;
      wr[4 * i + 2] = v.z;
      wr[4 * i + 3] = v.w;
    }
  }
  float* __restrict__ srow = scores + (int64_t)qo * ld;
  // score stores go through a buffer resource over the wavefront's two rows: a lane
  // with nothing to write gets an offset past the end, which the hardware drops.  With
  // no branch around them the stores are counted by every later wait, so a wait for
  // staged keys never has to wait for the stores too.
  const __amdgpu_buffer_rsrc_t srsrc = __builtin_amdgcn_make_buffer_rsrc(
      scores + (int64_t)(q0 + 2 * wid) * ld, (short)0, (int)(2 * ld * (int64_t)sizeof(float)), 0x00020000);
  const uint32_t srow_off = (uint32_t)half * (uint32_t)ld * 4u;
  lds_barrier();
  // operands and weights are in registers before the page loop, whose waits then only
  // cover the keys staged ahead
#pragma unroll
  for (int h = 0; h < HI; ++h) asm volatile("" : "+v"(wr[h]));

  // one row of the block table at a time: the first pending query's row, with every
  // pending query of the workgroup that reads it
  uint32_t pending = (nq - q0 >= kQ4Queries) ? (1u << kQ4Queries) - 1u : ((1u << (nq - q0)) - 1u);
  while (pending != 0u) {
    const int row = __builtin_amdgcn_readfirstlane(sm.row[__builtin_ctz(pending)]);
    uint32_t cur = 0u;
    int vmax = 0;
    for (int i = 0; i < kQ4Queries; ++i) {
      const int ri = __builtin_amdgcn_readfirstlane(sm.row[i]);
      const int vi = __builtin_amdgcn_readfirstlane(sm.nvis[i]);
      if (((pending >> i) & 1u) && ri == row) {
        cur |= 1u << i;
        vmax = max(vmax, vi);
      }
    }
    pending &= ~cur;
    const int Gend = min(G0 + pages_per_wg, (vmax + kPage - 1) / kPage);
    if (G0 >= Gend) continue;  // uniform
    const bool active = (cur >> (2 * wid + half)) & 1u;
    const int my_nvis = active ? sm.nvis[2 * wid + half] : 0;
    const int32_t* __restrict__ bt = block_table + (int64_t)row * max_pages;
    const uint16_t* __restrict__ qrow = q_idx + (int64_t)qo * HI * kIndexDim;

    // scores of one page from the slot holding it
    // (pages at or past Gend are computed on whatever the slot holds and write nothing;
    // pairs that need the exact path are left out of the stores and flagged in bits
    // 2p + nt of xbits)
    auto page = [&](const Q4Page& s, int G, int p, uint32_t& xbits) __attribute__((always_inline)) {
      uint4 b[2][2];  // N-tile nt, K-half kh: 16 bytes of entry 32nt + l%32, block 2kh + l/32
      int bsc[2][2];
      const uint8_t* sb = reinterpret_cast<const uint8_t*>(s.sc);
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
          const int e = 32 * nt + col, c = 2 * kh + half;
          b[nt][kh] = s.codes[4 * e + (c ^ ((e >> 2) & 3))];
          bsc[nt][kh] = (int)sb[4 * e + c];
        }
      float acc[2] = {0.0f, 0.0f};
      // step t = (N-tile t % 2, M-tile t / 2), taken in pairs (both N-tiles of one
      // M-tile); a pair's two MFMAs per K-half go out around the VALU work of the pair
      // before it, whose two fma chains (one per N-tile, each in head order) are
      // interleaved so that neither waits on its own previous fma
      auto mf = [&](int t, int kh, const v16f& c) __attribute__((always_inline)) -> v16f {
        const int nt = t & 1, mt = t >> 1, sl = 2 * mt + kh;
        switch (sl & 3) {
          case 0: return mfma32_fp4<0>(A[mt][kh], b[nt][kh], c, (int)asc[sl >> 2], bsc[nt][kh]);
          case 1: return mfma32_fp4<1>(A[mt][kh], b[nt][kh], c, (int)asc[sl >> 2], bsc[nt][kh]);
          case 2: return mfma32_fp4<2>(A[mt][kh], b[nt][kh], c, (int)asc[sl >> 2], bsc[nt][kh]);
          default: return mfma32_fp4<3>(A[mt][kh], b[nt][kh], c, (int)asc[sl >> 2], bsc[nt][kh]);
        }
      };
      const v16f zero = {};
      v16f D0, D1;
#pragma unroll
      for (int p = 0; p <= NM; ++p) {
        v16f T0, T1;
        if (p < NM) {
          T0 = mf(2 * p, 0, zero);
          T1 = mf(2 * p + 1, 0, zero);
        }
        __builtin_amdgcn_sched_barrier(0);
        if (p >= 1) {
          const int mt = p - 1;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            D0[r] = relu(D0[r]);
            D1[r] = relu(D1[r]);
          }
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            acc[0] = fmaf(wr[16 * mt + r], D0[r], acc[0]);
            acc[1] = fmaf(wr[16 * mt + r], D1[r], acc[1]);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
        if (p < NM) {
          D0 = mf(2 * p, 1, T0);
          D1 = mf(2 * p + 1, 1, T1);
        }
      }
      // the sums are complete here for every lane: the MFMAs (which read every lane's
      // operands) must not move into the masked stores below
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) asm volatile("" : "+v"(acc[nt]));
      // rare: pairs outside the window where the MFMA dot is exact
      const int vis = G < Gend ? my_nvis : 0;  // entries of this page the lane may write
      bool need[2] = {false, false};
      const uint32_t ps = s.pstat;
      const bool maybe = (G * kPage < vis) &&
                         q4_inexact(q_span, q_lo, q_hi, (int)(ps & 0xFFu), (int)((ps >> 8) & 0xFFu), (int)(ps >> 16));
      if (__builtin_amdgcn_ballot_w64(maybe) != 0ull) {
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          const int e = 32 * nt + col;
          const uint32_t es = s.estat[e];
          const int klo = (int)(es & 0xFFu), khi = (int)(es >> 8);
          need[nt] = G * kPage + e < vis && q4_inexact(q_span, q_lo, q_hi, khi - klo, klo, khi);
        }
      }
      const int j0 = G * kPage + col;
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const int j = j0 + 32 * nt;
        const uint32_t off = (j < vis && !need[nt]) ? srow_off + (uint32_t)j * 4u : 0xFFFFFFF0u;
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[nt]), srsrc, off, 0, 0);
        xbits |= (uint32_t)need[nt] << (2 * p + nt);
      }
    };

    // steps of kQ4Group pages: two steps staged ahead in registers, two LDS slots
    const int nst = (Gend - G0 + kQ4Group - 1) / kQ4Group;
    // one step: its pages in straight-line code, so every score store is counted by the
    // waits that follow; then the flagged pairs by the definition itself
    auto run = [&](const Q4Page(&sl)[kQ4Group], int G) __attribute__((always_inline)) {
      uint32_t xbits = 0u;
#pragma unroll
      for (int p = 0; p < kQ4Group; ++p) page(sl[p], G + p, p, xbits);
      if (__builtin_amdgcn_ballot_w64(xbits != 0u) != 0ull) {
        while (xbits != 0u) {
          const int bit = __builtin_ctz(xbits);
          xbits &= xbits - 1u;
          const int Gp = G + (bit >> 1), e = 32 * (bit & 1) + col;
          const int64_t slot = (int64_t)bt[Gp] * kPage + e;
          srow[Gp * kPage + e] = q4_exact(qrow, w + (int64_t)qo * HI, HI, idx_codes + slot * kIdxRowBytes,
                                          *reinterpret_cast<const uint32_t*>(idx_scales + slot * kIdxScaleBytes));
          count_exact_path();
        }
        // nothing of this rare branch stays in flight, so the waits after it count only
        // the staging loads and score stores of the common path
        __builtin_amdgcn_s_waitcnt(0);
      }
    };
    // every step's loads are issued, past the last step re-reading the last page, so
    // the wait for one register set never has to assume the other's loads are absent
    Q4Regs r1, r2;
    q4_load(r1, idx_codes, idx_scales, bt, G0, Gend, wid, lane);
    q4_load(r2, idx_codes, idx_scales, bt, G0 + kQ4Group, Gend, wid, lane);
    q4_store(sm.slot[0], r1, wid, lane);
    q4_load(r1, idx_codes, idx_scales, bt, G0 + 2 * kQ4Group, Gend, wid, lane);
    lds_barrier();
    for (int i = 0; i < nst; i += 2) {
      // slot 0: step i; r2: step i+1; r1: step i+2 (each register set keeps its role,
      // so no staged value is ever copied while its load is in flight)
      run(sm.slot[0], G0 + i * kQ4Group);
      if (i + 1 < nst) q4_store(sm.slot[1], r2, wid, lane);
      q4_load(r2, idx_codes, idx_scales, bt, G0 + (i + 3) * kQ4Group, Gend, wid, lane);
      lds_barrier();
      if (i + 1 >= nst) break;
      run(sm.slot[1], G0 + (i + 1) * kQ4Group);
      if (i + 2 < nst) q4_store(sm.slot[0], r1, wid, lane);
      q4_load(r1, idx_codes, idx_scales, bt, G0 + (i + 4) * kQ4Group, Gend, wid, lane);
      lds_barrier();
    }
  }
}

// Queries per workgroup of the scan (1 when every query reads its own sequence, or
// when four staged queries would not fit in 64 KB of LDS).
static int query_tile(const int32_t* soq, int32_t nq, size_t stage_bytes) {
  if (soq == nullptr || nq < 64) return 1;
  if (stage_bytes * 8 <= 64 * 1024) return 8;
  return stage_bytes * 4 <= 64 * 1024 ? 4 : 1;
}

// Pool scans (pool != nullptr) take one query per workgroup over virtual pages of
// the pool (ld = 8 npool).
struct PoolArgs {
  const int32_t* pool = nullptr;
  int npool = 0;
  int32_t* nvis = nullptr;  // [nq] out: visible pool positions
};

// Block maxima of the candidate pool built from the scores (index_topk_pool_build).
struct PoolBuildArgs {
  float* bmax = nullptr;  // [nq][ldb]
  int64_t ldb = 0;
  uint32_t* bhist = nullptr;  // the pool selection's digit-1 histograms
  int32_t* nblocks = nullptr;
  int npool = 0;
};

template <int MT>
static int launch_mt(const csa2_fp4_cache* c, const uint16_t* q_idx, const float* w, const int32_t* soq,
                     const int32_t* nvis, const int32_t* bt, int32_t max_pages, int32_t nq, float* scores, int64_t ld,
                     uint32_t* hist, int k, int* copies, const PoolArgs& pa, hipStream_t stream,
                     const PoolBuildArgs* pb = nullptr, int force_copies = 0) {
  const int total_groups = (int)ceil_div(ld, kPage);
  if (total_groups == 0 || nq == 0) return CSA2_OK;
  // queries per workgroup: several queries of one sequence share each loaded page
  // (queries without a sequence map each read their own pages); the staged queries
  // stay within 64 KB of LDS
  const int qt = pa.pool ? 1 : query_tile(soq, nq, sizeof(QStage<MT>));
  // pages per wavefront: enough wavefronts to cover the chip about twice
  const long long qtiles = ceil_div(nq, qt);
  const long long want_waves = qtiles >= 512 ? 4 * qtiles : 2048;
  int gpw = (int)ceil_div(total_groups * qtiles, want_waves);
  if (gpw < 1) gpw = 1;
  if (gpw > kMaxPagesPerWave) gpw = kMaxPagesPerWave;
  const unsigned gx = ceil_div(total_groups, (long long)kWaves * gpw);
  const dim3 grid(gx, (unsigned)qtiles), block(kThreads);
  const size_t lds = sizeof(QStage<MT>) * qt;
  const int ncopies = force_copies > 0 ? force_copies : topk_hist_copies(gx);
  if (copies != nullptr) *copies = ncopies;
  if (pb != nullptr) {  // one query per workgroup, with its digit-1 counts (the caller checked)
    hipLaunchKernelGGL((index_score_kernel<MT, 1, true, false, true>), grid, block,
                       lds + 2 * kTopkBins * sizeof(uint32_t), stream, c->idx_codes, c->idx_scales, q_idx, w, soq,
                       nvis, bt, max_pages, nq, scores, ld, gpw, total_groups, hist, k, ncopies, nullptr, pb->npool,
                       nullptr, pb->bmax, pb->ldb, pb->bhist, ncopies, pb->nblocks);
  } else if (pa.pool != nullptr) {
    if (hist != nullptr)
      hipLaunchKernelGGL((index_score_kernel<MT, 1, true, true>), grid, block, lds + kTopkBins * sizeof(uint32_t),
                         stream, c->idx_codes, c->idx_scales, q_idx, w, soq, nvis, bt, max_pages, nq, scores, ld, gpw,
                         total_groups, hist, k, ncopies, pa.pool, pa.npool, pa.nvis, nullptr, 0, nullptr, 0, nullptr);
    else
      hipLaunchKernelGGL((index_score_kernel<MT, 1, false, true>), grid, block, lds, stream, c->idx_codes,
                         c->idx_scales, q_idx, w, soq, nvis, bt, max_pages, nq, scores, ld, gpw, total_groups, hist,
                         k, ncopies, pa.pool, pa.npool, pa.nvis, nullptr, 0, nullptr, 0, nullptr);
  } else if (hist != nullptr) {  // one query per workgroup (the caller checked)
    hipLaunchKernelGGL((index_score_kernel<MT, 1, true>), grid, block, lds + kTopkBins * sizeof(uint32_t), stream,
                       c->idx_codes, c->idx_scales, q_idx, w, soq, nvis, bt, max_pages, nq, scores, ld, gpw,
                       total_groups, hist, k, ncopies, nullptr, 0, nullptr, nullptr, 0, nullptr, 0, nullptr);
  } else if (qt == 8) {
    hipLaunchKernelGGL((index_score_kernel<MT, 8, false>), grid, block, lds, stream, c->idx_codes, c->idx_scales,
                       q_idx, w, soq, nvis, bt, max_pages, nq, scores, ld, gpw, total_groups, hist, k, ncopies,
                       nullptr, 0, nullptr, nullptr, 0, nullptr, 0, nullptr);
  } else if (qt == 4) {
    hipLaunchKernelGGL((index_score_kernel<MT, 4, false>), grid, block, lds, stream, c->idx_codes, c->idx_scales,
                       q_idx, w, soq, nvis, bt, max_pages, nq, scores, ld, gpw, total_groups, hist, k, ncopies,
                       nullptr, 0, nullptr, nullptr, 0, nullptr, 0, nullptr);
  } else {
    // one query per workgroup: the kernel index_topk runs, with its counts switched off
    // (no histogram, k past every row).  Its register allocation leaves room for two
    // workgroups per CU where a variant without the counting code does not (batch 8:
    // 63.7 against 73.2 us); with one workgroup per CU (batch 1) that variant was 0.4 us
    // faster, but one kernel for both calls makes the standalone scan time the scan the
    // indexer stage runs.
    hipLaunchKernelGGL((index_score_kernel<MT, 1, true>), grid, block, lds + kTopkBins * sizeof(uint32_t), stream,
                       c->idx_codes, c->idx_scales, q_idx, w, soq, nvis, bt, max_pages, nq, scores, ld, gpw,
                       total_groups, nullptr, INT32_MAX, 1, nullptr, 0, nullptr, nullptr, 0, nullptr, 0, nullptr);
  }
  return launch_status();
}

template <int NM>
static int launch_q2(const csa2_fp4_cache* c, const uint16_t* q_idx, const float* w, const int32_t* soq,
                     const int32_t* nvis, const int32_t* bt, int32_t max_pages, int32_t nq, float* scores, int64_t ld,
                     hipStream_t stream) {
  const long long total_groups = ceil_div(ld, kPage);
  const long long qtiles = ceil_div(nq, kQ4Queries);
  // page chunks: about 2048 workgroups in all, each over at least kQ4MinPages pages.
  // Workgroup (x, y) runs on XCD (y * gx + x) % 8, so with gx a multiple of 8 each
  // XCD's L2 sees one eighth of the pages.
  const long long chunks = std::max(1LL, (2048 + qtiles - 1) / qtiles);
  const int ppw = (int)std::max<long long>(kQ4MinPages, (total_groups + chunks - 1) / chunks);
  const unsigned gx = ceil_div(total_groups, ppw);
  hipLaunchKernelGGL((index_score_q2_kernel<NM>), dim3(gx, (unsigned)qtiles), dim3(kThreads), 0, stream,
                     c->idx_codes, c->idx_scales, q_idx, w, soq, nvis, bt, max_pages, nq, scores, ld, ppw);
  return launch_status();
}

static int launch_hi(const csa2_fp4_cache* cache, const uint16_t* q_idx, const float* w, int32_t Hi,
                     const int32_t* seq_of_query, const int32_t* n_visible, const int32_t* block_table,
                     int32_t max_pages, int32_t nq, float* scores, int64_t ld, uint32_t* hist, int k,
                     int* copies, hipStream_t stream, const PoolArgs& pa = PoolArgs(),
                     const PoolBuildArgs* pb = nullptr, int force_copies = 0) {
  // queries that share sequences, at most 64 heads: two queries per wavefront (two
  // score rows within one buffer resource's 2^31-byte range)
  if (pa.pool == nullptr && hist == nullptr && query_tile(seq_of_query, nq, 0) > 1 && Hi <= 64 &&
      ld < ((int64_t)1 << 28)) {
    if (copies != nullptr) *copies = 1;
    switch (Hi / 16) {
      case 1: return launch_q2<1>(cache, q_idx, w, seq_of_query, n_visible, block_table, max_pages, nq, scores, ld, stream);
      case 2: return launch_q2<2>(cache, q_idx, w, seq_of_query, n_visible, block_table, max_pages, nq, scores, ld, stream);
      case 3: return launch_q2<3>(cache, q_idx, w, seq_of_query, n_visible, block_table, max_pages, nq, scores, ld, stream);
      default: return launch_q2<4>(cache, q_idx, w, seq_of_query, n_visible, block_table, max_pages, nq, scores, ld, stream);
    }
  }
  switch (Hi / 16) {
#define CSA2_MT(m) \
  case m:          \
    return launch_mt<m>(cache, q_idx, w, seq_of_query, n_visible, block_table, max_pages, nq, scores, ld, hist, k, \
                        copies, pa, stream, pb, force_copies);
    CSA2_MT(1)
    CSA2_MT(2)
    CSA2_MT(3)
    CSA2_MT(4)
    CSA2_MT(5)
    CSA2_MT(6)
    CSA2_MT(7)
    default: return launch_mt<8>(cache, q_idx, w, seq_of_query, n_visible, block_table, max_pages, nq, scores, ld,
                                 hist, k, copies, pa, stream, pb, force_copies);
#undef CSA2_MT
  }
}

static int check_args(const csa2_fp4_cache* cache, const uint16_t* q_idx, const float* w, int32_t Hi,
                      const int32_t* n_visible, const int32_t* block_table, int32_t max_pages, int32_t nq,
                      float* scores, int64_t ld) {
  if (!cache_ok(cache)) return CSA2_ERR_NULL;
  if (!cache_shape_ok(cache) || nq < 0 || ld < 0 || max_pages < 0) return CSA2_ERR_SHAPE;
  if (Hi < 16 || Hi > 128 || Hi % 16 != 0) return CSA2_ERR_SHAPE;
  if (nq == 0 || ld == 0) return CSA2_OK;
  if (!q_idx || !w || !n_visible || !block_table || !scores) return CSA2_ERR_NULL;
  if (max_pages < (ld + CSA2_PAGE_SIZE - 1) / CSA2_PAGE_SIZE) return CSA2_ERR_SHAPE;
  if (ld > (int64_t)1 << 30) return CSA2_ERR_SHAPE;
  return CSA2_OK;
}

}  // namespace csa2

using namespace csa2;

extern "C" int csa2_exact_path_count(unsigned long long* count) {
  if (count == nullptr) return CSA2_ERR_NULL;
  return hipMemcpyFromSymbol(count, HIP_SYMBOL(g_exact_path_count), sizeof(*count), 0, hipMemcpyDeviceToHost) ==
                 hipSuccess
             ? CSA2_OK
             : CSA2_ERR_LAUNCH;
}

extern "C" int csa2_exact_path_reset(void) {
  const unsigned long long zero = 0ull;
  return hipMemcpyToSymbol(HIP_SYMBOL(g_exact_path_count), &zero, sizeof(zero), 0, hipMemcpyHostToDevice) ==
                 hipSuccess
             ? CSA2_OK
             : CSA2_ERR_LAUNCH;
}

extern "C" int index_score(const csa2_fp4_cache* cache, const uint16_t* q_idx, const float* w, int32_t Hi,
                           const int32_t* seq_of_query, const int32_t* n_visible, const int32_t* block_table,
                           int32_t max_pages, int32_t nq, float* scores, int64_t ld, hipStream_t stream) {
  const int st = check_args(cache, q_idx, w, Hi, n_visible, block_table, max_pages, nq, scores, ld);
  if (st != CSA2_OK || nq == 0 || ld == 0) return st;
  return launch_hi(cache, q_idx, w, Hi, seq_of_query, n_visible, block_table, max_pages, nq, scores, ld, nullptr, 0,
                   nullptr, stream);
}

extern "C" int index_topk(const csa2_fp4_cache* cache, const uint16_t* q_idx, const float* w, int32_t Hi,
                          const int32_t* seq_of_query, const int32_t* n_visible, const int32_t* block_table,
                          int32_t max_pages, int32_t nq, float* scores, int64_t ld, int32_t k, int32_t* topk_idx,
                          void* ws, size_t ws_bytes, hipStream_t stream) {
  int st = check_args(cache, q_idx, w, Hi, n_visible, block_table, max_pages, nq, scores, ld);
  if (st != CSA2_OK) return st;
  if (k < 1 || k > CSA2_MAX_K || ld >= ((int64_t)1 << 31)) return CSA2_ERR_SHAPE;
  if (nq == 0) return CSA2_OK;
  if (!topk_idx) return CSA2_ERR_NULL;
  if (!ws || ws_bytes < topk_select_workspace_size(nq, ld, k)) return CSA2_ERR_WORKSPACE;
  // the counting pass folds into the scan when every workgroup serves one query
  const bool fuse = ld > 0 && query_tile(seq_of_query, nq, 0) == 1;
  int copies = 1;
  if (ld > 0) {
    uint32_t* hist = fuse ? topk_digit1_hist(ws, nq, ld) : nullptr;
    st = launch_hi(cache, q_idx, w, Hi, seq_of_query, n_visible, block_table, max_pages, nq, scores, ld, hist, k,
                   &copies, stream);
    if (st != CSA2_OK) return st;
  }
  return topk_enqueue(scores, ld, n_visible, nq, k, topk_idx, ws, stream, fuse, copies, nullptr, 0);
}

// ---- index_topk as two calls: the counting scan, then the selection --------------
// index_score_counted leaves the selection's first-digit histogram (always in all
// kTopkHistCopies copies, so that topk_select_counted needs no knowledge of how it was
// counted) in the top-k workspace; with one query per workgroup the scan counts as it
// scores, as inside index_topk, otherwise a counting pass follows the scan.
extern "C" int index_score_counted(const csa2_fp4_cache* cache, const uint16_t* q_idx, const float* w, int32_t Hi,
                                   const int32_t* seq_of_query, const int32_t* n_visible, const int32_t* block_table,
                                   int32_t max_pages, int32_t nq, float* scores, int64_t ld, int32_t k, void* ws,
                                   size_t ws_bytes, hipStream_t stream) {
  int st = check_args(cache, q_idx, w, Hi, n_visible, block_table, max_pages, nq, scores, ld);
  if (st != CSA2_OK) return st;
  if (k < 1 || k > CSA2_MAX_K || ld >= ((int64_t)1 << 31)) return CSA2_ERR_SHAPE;
  if (nq == 0 || ld == 0) return CSA2_OK;
  if (!ws || ws_bytes < topk_select_workspace_size(nq, ld, k)) return CSA2_ERR_WORKSPACE;
  if (query_tile(seq_of_query, nq, 0) == 1)
    return launch_hi(cache, q_idx, w, Hi, seq_of_query, n_visible, block_table, max_pages, nq, scores, ld,
                     topk_digit1_hist(ws, nq, ld), k, nullptr, stream, PoolArgs(), nullptr, kTopkHistCopies);
  st = launch_hi(cache, q_idx, w, Hi, seq_of_query, n_visible, block_table, max_pages, nq, scores, ld, nullptr, k,
                 nullptr, stream);
  if (st != CSA2_OK) return st;
  return topk_count(scores, ld, n_visible, nq, k, ws, kTopkHistCopies, stream);
}

// ---- index_topk without allocation: the workspace in a static device array --------
// For callers that cannot allocate (code under graph capture, serving loops).  Each
// device holds its own copy of `scratch` for the life of the process; its device
// address comes from hipGetSymbolAddress, once per device, and only that address is
// handed to kernels (the array's name in host code is a host-side stand-in).
static __device__ __align__(256) unsigned char scratch[CSA2_NOALLOC_SCRATCH_BYTES];

static int scratch_address(void** out) {
  static std::mutex mu;
  static void* addr[64] = {};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return CSA2_ERR_LAUNCH;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return CSA2_ERR_LAUNCH;
    addr[dev] = p;
  }
  *out = addr[dev];
  return CSA2_OK;
}

extern "C" int index_topk_noalloc(const csa2_fp4_cache* cache, const uint16_t* q_idx, const float* w, int32_t Hi,
                                  const int32_t* seq_of_query, const int32_t* n_visible, const int32_t* block_table,
                                  int32_t max_pages, int32_t nq, float* scores, int64_t ld, int32_t k,
                                  int32_t* topk_idx, hipStream_t stream) {
  int st = check_args(cache, q_idx, w, Hi, n_visible, block_table, max_pages, nq, scores, ld);
  if (st != CSA2_OK) return st;
  if (k < 1 || k > CSA2_MAX_K || ld >= ((int64_t)1 << 31)) return CSA2_ERR_SHAPE;
  if (nq == 0) return CSA2_OK;
  if (!topk_idx) return CSA2_ERR_NULL;
  const size_t need = topk_select_workspace_size(nq, ld, k);
  if (need > (size_t)CSA2_NOALLOC_SCRATCH_BYTES) return CSA2_ERR_WORKSPACE;
  void* ws = nullptr;
  st = scratch_address(&ws);
  if (st != CSA2_OK) return st;
  // the array keeps the last call's bytes: its counters and histograms start at zero
  st = zero_fill(ws, topk_zero_bytes(nq, ld), stream);
  if (st != CSA2_OK) return st;
  return index_topk(cache, q_idx, w, Hi, seq_of_query, n_visible, block_table, max_pages, nq, scores, ld, k,
                    topk_idx, ws, need, stream);
}

extern "C" size_t index_topk_pool_build_workspace_size(int32_t nq, int64_t ld, int32_t k, int32_t npool) {
  if (nq <= 0) return 256;
  return ((topk_select_workspace_size(nq, ld, k) + 255) & ~(size_t)255) +
         index_pool_build_workspace_size(nq, ld, npool);
}

extern "C" int index_topk_pool_build(const csa2_fp4_cache* cache, const uint16_t* q_idx, const float* w, int32_t Hi,
                                     const int32_t* seq_of_query, const int32_t* n_visible,
                                     const int32_t* block_table, int32_t max_pages, int32_t nq, float* scores,
                                     int64_t ld, int32_t k, int32_t* topk_idx, int32_t npool, int32_t* pool, void* ws,
                                     size_t ws_bytes, hipStream_t stream) {
  int st = check_args(cache, q_idx, w, Hi, n_visible, block_table, max_pages, nq, scores, ld);
  if (st != CSA2_OK) return st;
  if (k < 1 || k > CSA2_MAX_K || npool < 1 || npool > CSA2_MAX_K || ld >= ((int64_t)1 << 31)) return CSA2_ERR_SHAPE;
  if (nq == 0) return CSA2_OK;
  if (!topk_idx || !pool) return CSA2_ERR_NULL;
  if (!ws || ws_bytes < index_topk_pool_build_workspace_size(nq, ld, k, npool)) return CSA2_ERR_WORKSPACE;
  const size_t topk_bytes = (topk_select_workspace_size(nq, ld, k) + 255) & ~(size_t)255;
  void* ws_pool = static_cast<char*>(ws) + topk_bytes;
  const size_t pool_bytes = ws_bytes - topk_bytes;
  if (ld == 0 || query_tile(seq_of_query, nq, 0) != 1) {  // the two calls in turn
    st = index_topk(cache, q_idx, w, Hi, seq_of_query, n_visible, block_table, max_pages, nq, scores, ld, k, topk_idx,
                    ws, topk_bytes, stream);
    if (st != CSA2_OK) return st;
    return index_pool_build(scores, ld, n_visible, nq, npool, pool, ws_pool, pool_bytes, stream);
  }
  // one query per workgroup: the scan also writes the block maxima and counts their
  // first digit, so neither selection needs a counting launch
  const PoolWs pw = pool_ws_carve(ws_pool, nq, ld);
  PoolBuildArgs pb;
  pb.bmax = pw.bmax;
  pb.ldb = pw.ldb;
  pb.bhist = topk_digit1_hist(pw.ws_topk, nq, pw.ldb);
  pb.nblocks = pw.nblocks;
  pb.npool = npool;
  int copies = 1;
  st = launch_hi(cache, q_idx, w, Hi, seq_of_query, n_visible, block_table, max_pages, nq, scores, ld,
                 topk_digit1_hist(ws, nq, ld), k, &copies, stream, PoolArgs(), &pb);
  if (st != CSA2_OK) return st;
  // the top-k of the scores and the top npool blocks, one selection launch for both
  return topk_enqueue_pair(scores, ld, n_visible, nq, k, topk_idx, ws, copies, pw.bmax, pw.ldb, pw.nblocks, nq, npool,
                           pool, pw.ws_topk, copies, stream);
}

// the pool workspace: visible pool positions per query, then the selection's workspace
static size_t pool_nvis_bytes(int32_t nq) { return ((size_t)nq * sizeof(int32_t) + 255) & ~(size_t)255; }

extern "C" size_t index_topk_pool_workspace_size(int32_t nq, int32_t npool, int32_t k) {
  if (nq <= 0 || npool < 1) return 0;
  return pool_nvis_bytes(nq) + topk_select_workspace_size(nq, (int64_t)npool * kPoolBlock, k);
}

extern "C" int index_topk_pool(const csa2_fp4_cache* cache, const uint16_t* q_idx, const float* w, int32_t Hi,
                               const int32_t* seq_of_query, const int32_t* n_visible, const int32_t* pool,
                               int32_t npool, const int32_t* block_table, int32_t max_pages, int32_t nq,
                               float* scores_pool, int32_t k, int32_t* topk_idx, void* ws, size_t ws_bytes,
                               hipStream_t stream) {
  if (!cache_ok(cache)) return CSA2_ERR_NULL;
  if (!cache_shape_ok(cache) || nq < 0 || max_pages < 1) return CSA2_ERR_SHAPE;
  if (Hi < 16 || Hi > 128 || Hi % 16 != 0) return CSA2_ERR_SHAPE;
  if (npool < 1 || npool > CSA2_MAX_K || k < 1 || k > CSA2_MAX_K) return CSA2_ERR_SHAPE;
  if (nq == 0) return CSA2_OK;
  if (!q_idx || !w || !n_visible || !pool || !block_table || !scores_pool || !topk_idx) return CSA2_ERR_NULL;
  if (!ws || ws_bytes < index_topk_pool_workspace_size(nq, npool, k)) return CSA2_ERR_WORKSPACE;
  const int64_t ld = (int64_t)npool * kPoolBlock;
  int32_t* pool_nvis = reinterpret_cast<int32_t*>(ws);
  void* ws_topk = reinterpret_cast<char*>(ws) + pool_nvis_bytes(nq);
  PoolArgs pa;
  pa.pool = pool;
  pa.npool = npool;
  pa.nvis = pool_nvis;
  int copies = 1;
  // one query per workgroup: the selection's first counting pass runs inside the scan
  const int st = launch_hi(cache, q_idx, w, Hi, seq_of_query, n_visible, block_table, max_pages, nq, scores_pool,
                           ld, topk_digit1_hist(ws_topk, nq, ld), k, &copies, stream, pa);
  if (st != CSA2_OK) return st;
  return topk_enqueue(scores_pool, ld, pool_nvis, nq, k, topk_idx, ws_topk, stream, true, copies, pool, npool);
}
