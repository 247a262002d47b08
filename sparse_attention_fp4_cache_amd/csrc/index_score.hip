// index_score.hip -- lightning-indexer scores over MXFP4 keys with gfx950 scaled MFMA.
//
// Source: "DeepSeek-V4.1-Flash, expliqué pas à pas", CSA2 section (the indexer scores
// each cache entry from the query's indexer query and the entry's indexer key) and
// FP4 KV cache section (indexer queries and keys are OCP MXFP4).
//
// score[q][j] = fma-chain over h = 0..Hi-1 of w[q][h] * max(d_h, 0), starting at +0,
// d_h = exact dot(qhat_h, khat_j) rounded once to fp32.
//
// Layout of the work.  A wavefront takes one page (64 consecutive entries) at a time
// and, for each query of its tile, issues Hi/16 x 4 MFMAs
//   V_MFMA_SCALE_F32_16X16X128_F8F6F4 (A = 16 query heads, B = 16 keys, K = 128)
// with E8M0 block scales, so one instruction produces 16x16 complete dot products.
// Operand lane l holds row l%16 and the 32-channel block l/16: that is exactly one
// 16-byte slice of a packed key row plus its E8M0 byte, so each key row is fetched
// with four coalesced 16-byte loads per lane group.
// Measured on MI355X: the instruction returns the round-once exact dot whenever the
// four per-block exponent sums (u_q + u_k) span at most 14; it loses low bits beyond
// that.  Entries whose scales could exceed a span of 12 (or reach the fp32 subnormal
// or overflow range) take an exact integer/fp64 path instead, so results are always
// bit-identical to the definition.
// The query heads are permuted across MFMA rows so that lane group g ends up holding
// a contiguous run of Hi/4 heads; a 4x4 transpose across lane groups with
// v_permlane32_swap / v_permlane16_swap then leaves every lane with one entry and
// all Hi heads in ascending order, and the fma chain runs with all 64 lanes busy.
#include "common.hpp"
#include "host_common.hpp"

namespace csa2 {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kMaxSpread = 12;   // exponent-sum span accepted on the MFMA path
constexpr int kMinExpSum = 130;  // keeps every nonzero dot >= 2^-126 (fp32 normal)
constexpr int kMaxExpSum = 360;  // keeps every dot far below fp32 overflow
constexpr int kMaxPagesPerWave = 16;  // pages (of 64 entries) one wavefront scans

// per-query staging record in LDS, for Hi = 16*MT heads
template <int MT>
struct QStage {
  uint4 codes[MT][64];            // A operand of M-tile mt for lane l
  uint32_t scale[(MT + 3) / 4][64];  // byte (mt%4) of word mt/4: E8M0 of lane l in tile mt
  uint8_t u[16 * MT][4];          // E8M0 of head h, block b (plain order, exact path)
  float w[16 * MT];
  int row;
  int nvis;
  int ok_spread;  // largest per-head block-exponent span of the query
  int umin, umax;  // smallest / largest block exponent of the query
};

// Head held by row rho of M-tile mt: lane group rho/4 owns heads [(rho/4)*4MT, +4MT).
template <int MT>
CSA2_DEV int head_of(int mt, int rho) { return (rho >> 2) * 4 * MT + 4 * mt + (rho & 3); }

// MX32 quantisation of one 32-channel block held by one thread -> 16 packed bytes.
// For a normal power-of-two scale X the hardware V_CVT_SCALEF32_PK_FP4_F32 computes
// round-to-nearest-even(x / X) with saturation and a copied sign bit, which is the
// element rule exactly (checked on gfx950 against every bf16 value); blocks whose
// shared exponent is near the ends of the range take the compare-based rule.
CSA2_DEV void mx32_block(const uint16_t* __restrict__ src, uint4& out, uint32_t& u_out) {
  uint32_t raw[16];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint4 t = reinterpret_cast<const uint4*>(src)[i];
    raw[4 * i] = t.x;
    raw[4 * i + 1] = t.y;
    raw[4 * i + 2] = t.z;
    raw[4 * i + 3] = t.w;
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
  if (u >= 4u && u <= 250u) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {  // element pair (2i, 2i+1) -> byte i
      const uint32_t c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, bf16_to_f32(raw[i] & 0xFFFFu),
                                                                   __uint_as_float(raw[i] & 0xFFFF0000u), X, 0);
      word[i >> 2] |= (c & 0xFFu) << (8 * (i & 3));
    }
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      uint32_t c = e2m1_code(bf16_to_f32(raw[i] & 0xFFFFu), X) | (e2m1_code(bf16_to_f32(raw[i] >> 16), X) << 4);
      word[i >> 2] |= c << (8 * (i & 3));
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
  uint32_t sc[4];   // its E8M0 byte
  uint32_t own;     // the 4 E8M0 bytes of entry `lane` of the page
};

CSA2_DEV void load_keys(KeyTile& t, const uint8_t* __restrict__ idx_codes, const uint8_t* __restrict__ idx_scales,
                        int64_t slot0, int lane) {
  const int g = lane >> 4, n = lane & 15;
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    const int64_t s = slot0 + 16 * nt + n;
    t.codes[nt] = *reinterpret_cast<const uint4*>(idx_codes + s * kIdxRowBytes + 16 * g);
    t.sc[nt] = idx_scales[s * kIdxScaleBytes + g];
  }
  t.own = *reinterpret_cast<const uint32_t*>(idx_scales + (slot0 + lane) * kIdxScaleBytes);
}

template <int MT>
__global__ __launch_bounds__(256) void index_score_kernel(const uint8_t* __restrict__ idx_codes,
                                                          const uint8_t* __restrict__ idx_scales,
                                                          const uint16_t* __restrict__ q_idx,
                                                          const float* __restrict__ w,
                                                          const int32_t* __restrict__ seq_of_query,
                                                          const int32_t* __restrict__ n_visible,
                                                          const int32_t* __restrict__ block_table, int max_pages,
                                                          int nq, float* __restrict__ scores, int64_t ld, int qt,
                                                          int groups_per_wave, int total_groups) {
  constexpr int HI = 16 * MT;
  extern __shared__ __align__(16) unsigned char smem[];
  QStage<MT>* st = reinterpret_cast<QStage<MT>*>(smem);
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int q0 = blockIdx.y * qt;
  const int gfirst = (blockIdx.x * 4 + wid) * groups_per_wave;
  const int gend = min(gfirst + groups_per_wave, total_groups);
  const int first_row = (q0 < nq) ? (seq_of_query ? seq_of_query[q0] : q0) : 0;

  // ---- physical pages of this wavefront (one table read), and the first two pages
  // of keys in flight while the queries are staged
  int pages[kMaxPagesPerWave];
#pragma unroll
  for (int i = 0; i < kMaxPagesPerWave; ++i)
    pages[i] = (gfirst + i < gend) ? block_table[(int64_t)first_row * max_pages + gfirst + i] : 0;
  KeyTile t0, t1, t2;
  int cur_row = first_row;
  if (gfirst < gend) load_keys(t0, idx_codes, idx_scales, (int64_t)pages[0] * kPage, lane);
  if (gfirst + 1 < gend) load_keys(t1, idx_codes, idx_scales, (int64_t)pages[1] * kPage, lane);

  // ---- stage the tile's queries: MXFP4 operands, scales, weights
  for (int item = tid; item < qt * MT * 64; item += 256) {
    const int qi = item / (MT * 64), rem = item % (MT * 64), mt = rem >> 6, l = rem & 63;
    const int g = l >> 4, rho = l & 15, h = head_of<MT>(mt, rho), q = q0 + qi;
    uint4 codes = make_uint4(0, 0, 0, 0);
    uint32_t u = 127;
    if (q < nq) mx32_block(q_idx + ((int64_t)q * HI + h) * kIndexDim + 32 * g, codes, u);
    st[qi].codes[mt][l] = codes;
    st[qi].u[h][g] = (uint8_t)u;
    reinterpret_cast<uint8_t*>(&st[qi].scale[mt >> 2][l])[mt & 3] = (uint8_t)u;
  }
  for (int item = tid; item < qt * HI; item += 256) {
    const int qi = item / HI, h = item % HI, q = q0 + qi;
    st[qi].w[h] = (q < nq) ? w[(int64_t)q * HI + h] : 0.0f;
  }
  if (tid < qt) {
    const int q = q0 + tid;
    st[tid].row = (q < nq) ? (seq_of_query ? seq_of_query[q] : q) : 0;
    st[tid].nvis = (q < nq) ? n_visible[q] : 0;
    st[tid].ok_spread = 0;  // largest per-head span until the reduction below is done
    st[tid].umin = 255;
    st[tid].umax = 0;
  }
  lds_barrier();
  for (int item = tid; item < qt * HI; item += 256) {  // per-head block-exponent span
    const int qi = item / HI, h = item % HI;
    int lo = 255, hi = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int u = st[qi].u[h][b];
      lo = u < lo ? u : lo;
      hi = u > hi ? u : hi;
    }
    atomicMax(&st[qi].ok_spread, hi - lo);
    atomicMin(&st[qi].umin, lo);
    atomicMax(&st[qi].umax, hi);
  }
  lds_barrier();
  if (gfirst >= gend) return;
  const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};

#pragma unroll 1
  for (int i = 0; gfirst + i < gend; ++i) {
    const int G = gfirst + i;
    if (G + 2 < gend)  // two pages ahead stay in flight
      load_keys(t2, idx_codes, idx_scales, (int64_t)pages[(i + 2) & (kMaxPagesPerWave - 1)] * kPage, lane);
    KeyTile& cur = t0;
    for (int qi = 0; qi < qt; ++qi) {
      const QStage<MT>& s = st[qi];
      if (G * kPage >= s.nvis) continue;  // uniform
      if (s.row != cur_row) {  // a query of another sequence in this tile: load its page
        load_keys(cur, idx_codes, idx_scales, (int64_t)block_table[(int64_t)s.row * max_pages + G] * kPage, lane);
        cur_row = s.row;
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
      const bool exact_needed = (j < s.nvis) & (((kmax - kmin) + s.ok_spread > kMaxSpread) |
                                                (s.umin + kmin < kMinExpSum) | (s.umax + kmax > kMaxExpSum));
      float acc = 0.0f;
#pragma unroll
      for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc = fmaf(s.w[b * 4 * MT + 4 * mt + r], relu(d[mt][b][r]), acc);
      if (exact_needed) {  // rare: recompute this entry exactly
        const int64_t slot = (int64_t)block_table[(int64_t)s.row * max_pages + G] * kPage + lane;
        const uint8_t* krow = idx_codes + slot * kIdxRowBytes;
        acc = 0.0f;
        for (int h = 0; h < HI; ++h) acc = fmaf(s.w[h], relu(exact_dot<MT>(s, h, krow, own)), acc);
      }
      if (j < s.nvis) scores[(int64_t)(q0 + qi) * ld + j] = acc;
    }
    t0 = t1;  // t1 and t2 always hold this wavefront's own (first-row) pages
    t1 = t2;
    cur_row = first_row;
  }
}

template <int MT>
static int launch_mt(const csa2_fp4_cache* c, const uint16_t* q_idx, const float* w, const int32_t* soq,
                     const int32_t* nvis, const int32_t* bt, int32_t max_pages, int32_t nq, float* scores, int64_t ld,
                     hipStream_t stream) {
  const int total_groups = (int)ceil_div(ld, kPage);
  if (total_groups == 0 || nq == 0) return CSA2_OK;
  // queries per workgroup: share each loaded page among several queries when there are many
  int qt = nq >= 64 ? 8 : 1;
  while (qt > 1 && sizeof(QStage<MT>) * qt > 48 * 1024) qt >>= 1;
  // pages per wavefront: enough wavefronts to cover the chip about twice
  const long long qtiles = ceil_div(nq, qt);
  const long long want_waves = qtiles >= 512 ? 4 * qtiles : 2048;
  int gpw = (int)ceil_div(total_groups * qtiles, want_waves);
  if (gpw < 1) gpw = 1;
  if (gpw > kMaxPagesPerWave) gpw = kMaxPagesPerWave;
  const unsigned gx = ceil_div(total_groups, 4LL * gpw);
  const size_t lds = sizeof(QStage<MT>) * qt;
  hipLaunchKernelGGL(index_score_kernel<MT>, dim3(gx, (unsigned)qtiles), dim3(256), lds, stream, c->idx_codes,
                     c->idx_scales, q_idx, w, soq, nvis, bt, max_pages, nq, scores, ld, qt, gpw, total_groups);
  return launch_status();
}

}  // namespace csa2

using namespace csa2;

extern "C" int index_score(const csa2_fp4_cache* cache, const uint16_t* q_idx, const float* w, int32_t Hi,
                           const int32_t* seq_of_query, const int32_t* n_visible, const int32_t* block_table,
                           int32_t max_pages, int32_t nq, float* scores, int64_t ld, hipStream_t stream) {
  if (!cache_ok(cache)) return CSA2_ERR_NULL;
  if (!cache_shape_ok(cache) || nq < 0 || ld < 0 || max_pages < 0) return CSA2_ERR_SHAPE;
  if (Hi < 16 || Hi > 128 || Hi % 16 != 0) return CSA2_ERR_SHAPE;
  if (nq == 0 || ld == 0) return CSA2_OK;
  if (!q_idx || !w || !n_visible || !block_table || !scores) return CSA2_ERR_NULL;
  if (max_pages < (ld + CSA2_PAGE_SIZE - 1) / CSA2_PAGE_SIZE) return CSA2_ERR_SHAPE;
  if (ld > (int64_t)1 << 30) return CSA2_ERR_SHAPE;
  switch (Hi / 16) {
    case 1: return launch_mt<1>(cache, q_idx, w, seq_of_query, n_visible, block_table, max_pages, nq, scores, ld, stream);
    case 2: return launch_mt<2>(cache, q_idx, w, seq_of_query, n_visible, block_table, max_pages, nq, scores, ld, stream);
    case 3: return launch_mt<3>(cache, q_idx, w, seq_of_query, n_visible, block_table, max_pages, nq, scores, ld, stream);
    case 4: return launch_mt<4>(cache, q_idx, w, seq_of_query, n_visible, block_table, max_pages, nq, scores, ld, stream);
    case 5: return launch_mt<5>(cache, q_idx, w, seq_of_query, n_visible, block_table, max_pages, nq, scores, ld, stream);
    case 6: return launch_mt<6>(cache, q_idx, w, seq_of_query, n_visible, block_table, max_pages, nq, scores, ld, stream);
    case 7: return launch_mt<7>(cache, q_idx, w, seq_of_query, n_visible, block_table, max_pages, nq, scores, ld, stream);
    default: return launch_mt<8>(cache, q_idx, w, seq_of_query, n_visible, block_table, max_pages, nq, scores, ld, stream);
  }
}
