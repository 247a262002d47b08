// sparse_attn.hip -- attention over the selected FP4 cache entries plus the
// sliding window, one shared softmax (decode and prefill chunk).
//
// Source: "DeepSeek-V4.1-Flash, expliqué pas à pas", CSA2 section (the main query
// reads the selected entries and the layer's own sliding-window KV), FP4 KV cache
// section (FP4 is a storage format: entries are dequantised before attention),
// attention forms (the window is the last 128 tokens), intro (softmax-weighted
// mean of the values); "La lignée DeepSeek" (one latent vector shared by all heads,
// so every entry and window row is both key and value for all heads).
//
// Work decomposition.  A workgroup (8 wavefronts, two halves of 4) owns one query,
// 16 heads and a contiguous range of candidate rows (selected entries first, then
// window rows).  The two halves walk alternate tiles of 32 rows at the same time,
// each with its own LDS tile and online softmax, and combine their states at the end:
//   gather   : a thread loads 64 channels of one tile row with 16-byte loads (only
//              the kinds of row the tile holds: FP4 entry or bf16 window row) and
//              dequantises them into LDS as row-major X[32][512] (bf16; E2M1 x E4M3
//              has at most 6 significant bits in [2^-10, 2688], so the bf16 value is
//              exact).  16-byte chunks are XOR-swizzled per row block against bank
//              conflicts.  The bytes of the next tile are loaded into registers while
//              the current tile is computed.
//   logits   : S^T = X Q^T with V_MFMA_F32_16X16X32_BF16; each wavefront covers a
//              quarter of the 512 channels and the four partial tiles are summed in
//              LDS in a fixed order.  The rows are permuted across the two 16-row
//              M-tiles so that lane group g holds rows 8g .. 8g+7.
//   softmax  : per head, running max / sum in fp32 (exp2 of log2e-scaled logits).
//   values   : O^T += X^T P^T; each wavefront owns 128 output channels.  The X^T
//              operand is read from row-major X with DS_READ_B64_TR_B16 (a transposing
//              LDS read), the P operand comes straight from the logits accumulator
//              registers (the K index of the MFMA is permuted to match), split into a
//              bf16 high part and a bf16 remainder so P keeps ~16 significant bits.
// With several row ranges per query the unnormalised partial (O, m, l) goes to the
// workspace and a merge kernel combines the ranges with their log-sum-exp weights.
// Both halves run the same number of tile steps (a half past the end of the range
// computes an empty tile), so every workgroup barrier is reached by all wavefronts.
#include "common.hpp"
#include "host_common.hpp"

#include <type_traits>

namespace csa2 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));

constexpr int kRT = 32;              // rows per tile
constexpr int kXStride = 512 + 8;    // bf16 elements per row of X in LDS (padding vs bank conflicts)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLazyMax = 8.0f;  // one-range kernel: largest weight 2^8 before the reference maximum moves

// 2^x with V_EXP_F32 alone: exact where the library exp2f is (results of normal
// magnitude), it only skips the library's rescaling for results below 2^-126, which
// weigh nothing here.
CSA2_DEV float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

struct AttnArgs {
  const uint8_t* main_codes;
  const uint8_t* main_scales;
  const uint16_t* q;         // [nq][H][512]
  int H;
  const int32_t* topk_idx;   // [nq][k]
  int k;
  const int32_t* block_table;
  int max_pages;
  const uint16_t* swa;       // bf16 window rows [.][512], or
  const uint8_t* swa8;       // FP8 window rows: E4M3FN codes [.][512] ...
  const uint8_t* swa8_scale; // ... and one E8M0 scale per row
  const int32_t* swa_len;    // decode: valid window rows per query
  int window;
  int prefill;               // 1: window rows of query i are swa rows i .. i+window-1
  int swa_first_valid;
  float scale_log2;          // softmax_scale * log2(e)
  int nq;
  int nsplit;                // row ranges per query
  int rows_per_split;        // multiple of kRT
  float* out;                // [nq][H][512]
  float* lse;                // [nq][H]
  float* part_o;             // [nq][nsplit][H][512]
  float* part_ml;            // [nq][nsplit][H][2]
};

constexpr int kSeg = 512;  // rows whose sources are resolved into LDS at a time
constexpr int kThreads = 512;  // two halves of 4 wavefronts

struct __align__(16) HalfSmem {
  uint16_t x[kRT * kXStride];    // X[row][ch], 16-byte chunks swizzled by xchunk()
  float red[4][2][4][64];        // partial logits [wave][mtile][r][lane]
};
struct __align__(16) AttnSmem {
  HalfSmem h[2];
  int src[kSeg];  // row source: slot >= 0, window row -2-r, or -1 (none, also the padding)
};
static_assert(sizeof(AttnSmem) <= 160 * 1024, "attention LDS exceeds 160 KB");
// the second half's tile area holds its softmax state for the final combine
// at the end each half's tile area holds its O as [16 heads][kOStride floats], and
// the first half's logit area the (m, l) of both halves
constexpr int kOStride = kLatentDim + 4;  // floats per head row (rows start 4 banks apart)
static_assert(16 * kOStride * sizeof(float) <= sizeof(HalfSmem::x), "combine area");
static_assert(2 * 16 * 2 * sizeof(float) <= sizeof(HalfSmem::red), "combine (m, l) area");

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
// two fp32 -> packed bf16 (V_CVT_PK_BF16_F32, round to nearest even; exact for values
// that fit bf16, such as every dequantised E2M1 x E4M3 product)
CSA2_DEV uint32_t pack_bf16(float lo, float hi) {
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

CSA2_DEV uint32_t bf16_rne_bits(float f) {  // fp32 -> bf16 bits, round to nearest even (finite f)
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Physical 16-byte chunk of logical chunk c (8 channels) within a row of X: chunk
// c of the 8-chunk block c/8 is moved to (c % 8) ^ (c / 8), so the eight threads that
// write one row block per instruction hit different banks.
CSA2_DEV int xchunk(int c) { return c ^ ((c >> 3) & 7); }

// Raw bytes of this thread's share of one tile, as loaded from HBM.  Thread t of a
// half owns tile row t/8 and channels 64*(t%8) .. +63.  Only the kinds of row the
// tile can hold are loaded (a uniform branch); an address of a missing row is
// clamped to row 0 and its value masked out.
struct TileRegs {
  uint4 code[2];  // FP4 entry: 32 code bytes (64 channels)
  uint32_t sc;    // FP4 entry: the E4M3 scale bytes of channels 16j .. 16j+15, j = 0..3
  uint4 win[8];   // window row: 64 bf16 (FP8 window: 64 code bytes in win[0..3])
  uint32_t wsc;   // FP8 window row: its E8M0 scale byte
  int kind;       // 1: FP4 entry, 2: window row, 0: no row
};

// 8 E4M3FN codes (two dwords) times a power-of-two scale as 8 bf16, exact (4
// significant bits times 2^e), via V_CVT_PK_F32_FP8 (OCP E4M3FN on gfx950).
CSA2_DEV uint4 dequant_fp8x8(uint32_t lo, uint32_t hi, float X) {
  const v2f a = __builtin_amdgcn_cvt_pk_f32_fp8((int)lo, false), b = __builtin_amdgcn_cvt_pk_f32_fp8((int)lo, true);
  const v2f c = __builtin_amdgcn_cvt_pk_f32_fp8((int)hi, false), d = __builtin_amdgcn_cvt_pk_f32_fp8((int)hi, true);
  return make_uint4(pack_bf16(a[0] * X, a[1] * X), pack_bf16(b[0] * X, b[1] * X), pack_bf16(c[0] * X, c[1] * X),
                    pack_bf16(d[0] * X, d[1] * X));
}

// Channels 8i .. 8i+7 of a thread's window share as bf16: loaded bf16, or dequantised
// from the FP8 codes (byte 8i of the share is in win[i / 2]).
template <bool W8>
CSA2_DEV uint4 win_chunk(const uint4* win, int i, float X) {
  if (!W8) return win[i];
  const uint4 v = win[i >> 1];
  return (i & 1) ? dequant_fp8x8(v.z, v.w, X) : dequant_fp8x8(v.x, v.y, X);
}

CSA2_DEV float e8m0_scale(uint32_t u) { return ldexpf(1.0f, (int)(u & 0xFFu) - 127); }

template <bool W8>
CSA2_DEV void issue_tile(const AttnArgs& a, const int* src_rows, int tid, int tile_row0, bool has_main, bool has_win,
                         TileRegs& t) {
  const int row = tid >> 3, c8 = tid & 7;
  const int src = src_rows[tile_row0 + row];
  t.kind = src >= 0 ? 1 : (src <= -2 ? 2 : 0);
  if (has_main) {
    const int64_t slot = src >= 0 ? src : 0;
    const uint4* cp = reinterpret_cast<const uint4*>(a.main_codes + slot * kMainRowBytes) + 2 * c8;
    t.code[0] = cp[0];
    t.code[1] = cp[1];
    t.sc = reinterpret_cast<const uint32_t*>(a.main_scales + slot * kMainScaleBytes)[c8];
  } else {
    t.code[0] = t.code[1] = make_uint4(0u, 0u, 0u, 0u);
    t.sc = 0u;
  }
  t.wsc = 0u;
  if (has_win && W8) {
    const int64_t wrow = src <= -2 ? (int64_t)(-2 - src) : 0;
    const uint4* wp = reinterpret_cast<const uint4*>(a.swa8 + wrow * kLatentDim) + 4 * c8;
#pragma unroll
    for (int i = 0; i < 4; ++i) t.win[i] = wp[i];
#pragma unroll
    for (int i = 4; i < 8; ++i) t.win[i] = make_uint4(0u, 0u, 0u, 0u);
    t.wsc = a.swa8_scale[wrow];
  } else if (has_win) {
    const int64_t wrow = src <= -2 ? (int64_t)(-2 - src) : 0;
    const uint4* wp = reinterpret_cast<const uint4*>(a.swa + wrow * kLatentDim) + 8 * c8;
#pragma unroll
    for (int i = 0; i < 8; ++i) t.win[i] = wp[i];
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) t.win[i] = make_uint4(0u, 0u, 0u, 0u);
  }
}

CSA2_DEV uint4 and4(uint4 v, uint32_t m) { return make_uint4(v.x & m, v.y & m, v.z & m, v.w & m); }
CSA2_DEV uint4 or4(uint4 a, uint4 b) { return make_uint4(a.x | b.x, a.y | b.y, a.z | b.z, a.w | b.w); }

// E2M1 x E4M3 of 8 channels (one code dword) as 8 bf16, exact.
CSA2_DEV uint4 dequant8(uint32_t c, float s) {
  const v2f d0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 0);
  const v2f d1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 1);
  const v2f d2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 2);
  const v2f d3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 3);
  return make_uint4(pack_bf16(d0[0] * s, d0[1] * s), pack_bf16(d1[0] * s, d1[1] * s),
                    pack_bf16(d2[0] * s, d2[1] * s), pack_bf16(d3[0] * s, d3[1] * s));
}

// Dequantise the loaded bytes into X (row-major, swizzled chunks) in LDS.
// Branch-free within a tile: E4M3 scale via V_CVT_F32_FP8 (OCP E4M3FN on gfx950),
// E2M1 pairs via V_CVT_SCALEF32_PK_F32_FP4 with a unit scale, product exact in
// fp32 and in bf16.
template <bool W8>
CSA2_DEV void store_tile(HalfSmem& sm, int tid, const TileRegs& t, bool has_main) {
  const int row = tid >> 3, c8 = tid & 7;
  uint4* xr = reinterpret_cast<uint4*>(sm.x + row * kXStride);
  const uint32_t wmask = t.kind == 2 ? ~0u : 0u;
  const float X = W8 ? e8m0_scale(t.wsc) : 1.0f;
  if (has_main) {
    const uint32_t mmask = t.kind == 1 ? ~0u : 0u;
    const uint32_t cw[8] = {t.code[0].x, t.code[0].y, t.code[0].z, t.code[0].w,
                            t.code[1].x, t.code[1].y, t.code[1].z, t.code[1].w};
    const float sc[4] = {__builtin_amdgcn_cvt_f32_fp8((int)t.sc, 0), __builtin_amdgcn_cvt_f32_fp8((int)t.sc, 1),
                         __builtin_amdgcn_cvt_f32_fp8((int)t.sc, 2), __builtin_amdgcn_cvt_f32_fp8((int)t.sc, 3)};
#pragma unroll
    for (int i = 0; i < 8; ++i)  // chunk i (8 channels) of this thread's 64 uses scale byte i / 2
      xr[xchunk(8 * c8 + i)] = or4(and4(dequant8(cw[i], sc[i >> 1]), mmask), and4(win_chunk<W8>(t.win, i, X), wmask));
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) xr[xchunk(8 * c8 + i)] = and4(win_chunk<W8>(t.win, i, X), wmask);
  }
}

CSA2_DEV bf16x8 as_bf16x8(uint4 v) {
  bf16x8 r;
  __builtin_memcpy(&r, &v, 16);
  return r;
}

template <bool W8>
__global__ __launch_bounds__(kThreads) void sparse_attn_kernel(AttnArgs a) {
  __shared__ AttnSmem smem;
  const int half = threadIdx.x >> 8;
  const int tid = threadIdx.x & 255, lane = tid & 63, wid = tid >> 6;  // within the half
  HalfSmem& sm = smem.h[half];
  const int g = lane >> 4, n16 = lane & 15;
  const int hg = blockIdx.y;          // head group of 16
  const int qrow = blockIdx.z;        // query
  const int split = blockIdx.x;
  const int bt_row = a.prefill ? 0 : qrow;
  const int total_rows = a.k + a.window;
  const int r_begin = split * a.rows_per_split;
  const int r_end = min(r_begin + a.rows_per_split, total_rows);
  const int nrows = r_end - r_begin;
  const int head = hg * 16 + n16;  // head owned by this lane in every accumulator

  // Q^T operand for this wavefront's 128 channels: lane holds head n16, channels
  // 128*wid + 32*ks + 8*g .. +7
  uint4 qop[4];
  const uint16_t* qp = a.q + ((int64_t)qrow * a.H + head) * kLatentDim + 128 * wid + 8 * g;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) qop[ks] = *reinterpret_cast<const uint4*>(qp + 32 * ks);

  v4f acc[8];  // O^T: M-tile mt covers channels 128*wid + 16*mt + 4*g + r, column = head
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) acc[mt] = v4f{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.0f;

  for (int seg0 = 0; seg0 < nrows; seg0 += kSeg) {
  const int seg_n = min(kSeg, nrows - seg0);
  lds_barrier();  // the previous segment's sources are no longer read
  // where every row of this segment comes from (one round of index loads); rows
  // past the segment up to the next tile pair are padding (-1)
  const int seg_pad = (seg_n + 2 * kRT - 1) / (2 * kRT) * (2 * kRT);
  for (int rl = (int)threadIdx.x; rl < seg_pad; rl += kThreads) {
    const int r = r_begin + seg0 + rl;
    int src = -1;
    if (rl >= seg_n) {
    } else if (r < a.k) {
      const int j = a.topk_idx[(int64_t)qrow * a.k + r];
      if (j >= 0) src = a.block_table[(int64_t)bt_row * a.max_pages + (j >> 6)] * kPage + (j & 63);
    } else {
      const int wr = r - a.k;
      if (a.prefill) {
        if (qrow + wr >= a.swa_first_valid) src = -2 - (qrow + wr);
      } else if (wr < a.swa_len[qrow]) {
        src = -2 - (qrow * a.window + wr);
      }
    }
    smem.src[rl] = src;
  }
  lds_barrier();
  // kinds of row in the tile at segment row rl0: FP4 entries below k, window rows above
  auto has_main = [&](int rl0) { return r_begin + seg0 + rl0 < a.k; };
  auto has_win = [&](int rl0) { return a.window > 0 && r_begin + seg0 + rl0 + kRT > a.k; };
  TileRegs cur;
  issue_tile<W8>(a, smem.src, tid, half * kRT, has_main(half * kRT), has_win(half * kRT), cur);
  for (int pair0 = 0; pair0 < seg_n; pair0 += 2 * kRT) {
    const int row0 = pair0 + half * kRT;  // may lie past seg_n: an empty tile
    lds_barrier();  // previous tile fully consumed
    store_tile<W8>(sm, tid, cur, has_main(row0));
    const int next0 = row0 + 2 * kRT;  // inside the padded sources whenever another pair follows
    if (pair0 + 2 * kRT < seg_n) issue_tile<W8>(a, smem.src, tid, next0, has_main(next0), has_win(next0), cur);
    lds_barrier();
    // ---- partial logits over this wavefront's 128 channels, two 16-row M-tiles
    v4f s[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      s[t] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        // M row n16 of tile t is tile row 8*(n16/4) + 4t + n16%4, so that lane group g
        // ends up holding the logits of rows 8g .. 8g+7
        const int xrow = 8 * (n16 >> 2) + 4 * t + (n16 & 3);
        const uint4 xa = reinterpret_cast<const uint4*>(sm.x + xrow * kXStride)[xchunk(16 * wid + 4 * ks + g)];
        s[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xa), as_bf16x8(qop[ks]), s[t], 0, 0, 0);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) sm.red[wid][t][r][lane] = s[t][r];
    }
    lds_barrier();
    // full logits (same fixed summation order in every wavefront), scaled to log2 units
    float z[2][4];
    float tmax = -INFINITY;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float v = ((sm.red[0][t][r][lane] + sm.red[1][t][r][lane]) + sm.red[2][t][r][lane]) + sm.red[3][t][r][lane];
        const int rl = row0 + 8 * g + 4 * t + r;
        const bool valid = (rl < seg_n) & (smem.src[rl & (kSeg - 1)] != -1);  // no short-circuit branch
        z[t][r] = valid ? v * a.scale_log2 : -INFINITY;
        tmax = fmaxf(tmax, z[t][r]);
      }
    tmax = max_rows(tmax);
    const float m_new = fmaxf(m_run, tmax);
    const float alpha = (m_new == -INFINITY) ? 1.0f : fast_exp2(m_run - m_new);
    float p[2][4];
    float psum = 0.0f;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        p[t][r] = fast_exp2(z[t][r] - (m_new == -INFINITY ? 0.0f : m_new));  // exp2(-inf) = 0
        psum += p[t][r];
      }
    psum = sum_rows(psum);
    l_run = l_run * alpha + psum;
    m_run = m_new;
    // P^T operand: K slot 8g+i <-> tile row 8g+i = this lane's p[i/4][i%4]
    uint32_t phi[4], plo[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float a0 = p[i >> 1][2 * (i & 1)], a1 = p[i >> 1][2 * (i & 1) + 1];
      const uint32_t h0 = bf16_rne_bits(a0), h1 = bf16_rne_bits(a1);
      phi[i] = h0 | (h1 << 16);
      const float r0 = a0 - __uint_as_float(h0 << 16), r1 = a1 - __uint_as_float(h1 << 16);
      plo[i] = bf16_rne_bits(r0) | (bf16_rne_bits(r1) << 16);
    }
    const bf16x8 Bhi = as_bf16x8(make_uint4(phi[0], phi[1], phi[2], phi[3]));
    const bf16x8 Blo = as_bf16x8(make_uint4(plo[0], plo[1], plo[2], plo[3]));
    // X^T operand of M-tile mt: lane (n16, g) needs channel 128*wid + 16*mt + n16 of
    // tile rows 8g .. 8g+7.  In a transposing read, lane 4r + c of each 16-lane group
    // addresses channels 4c .. 4c+3 of row r and receives channel n16 of rows 0..3.
    const int tr_c = n16 & 3;
    const uint16_t* tr_row = sm.x + (8 * g + (n16 >> 2)) * kXStride + 4 * (tr_c & 1);
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
      acc[mt] *= alpha;
      const uint16_t* tp = tr_row + 8 * xchunk(16 * wid + 2 * mt + (tr_c >> 1));
      const bf16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)tp);
      const bf16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(tp + 4 * kXStride));
      const bf16x8 A = __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
      acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, Bhi, acc[mt], 0, 0, 0);
      acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, Blo, acc[mt], 0, 0, 0);
    }
  }

  }  // segments

  // ---- combine the halves and write.  Each half leaves its O in its own tile area
  // as [head][channel] and its (m, l) per head next to it; then all 512 threads
  // rescale both halves to the larger running maximum, add them and write whole
  // 2 KB rows of the output.
  lds_barrier();  // every tile consumed
  float* o_mine = reinterpret_cast<float*>(sm.x);
  float* ml = reinterpret_cast<float*>(smem.h[0].red);  // [half][16 heads][m, l]
#pragma unroll
  for (int mt = 0; mt < 8; ++mt)
    *reinterpret_cast<float4*>(o_mine + n16 * kOStride + 128 * wid + 16 * mt + 4 * g) =
        make_float4(acc[mt][0], acc[mt][1], acc[mt][2], acc[mt][3]);
  if (wid == 0 && g == 0) {
    ml[(half * 16 + n16) * 2] = m_run;
    ml[(half * 16 + n16) * 2 + 1] = l_run;
  }
  lds_barrier();
  const float* o0 = reinterpret_cast<const float*>(smem.h[0].x);
  const float* o1 = reinterpret_cast<const float*>(smem.h[1].x);
  // thread t: float4 c4 = t % 128 of heads hq, hq + 4, hq + 8, hq + 12 (hq = t / 128);
  // every LDS read first, then the arithmetic and the stores
  const int hq = (int)threadIdx.x >> 7, c4 = (int)threadIdx.x & 127;
  float2 s0[4], s1[4];
  float4 x0[4], x1[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int hh = hq + 4 * i;
    s0[i] = *reinterpret_cast<const float2*>(ml + hh * 2);
    s1[i] = *reinterpret_cast<const float2*>(ml + (16 + hh) * 2);
    x0[i] = *reinterpret_cast<const float4*>(o0 + hh * kOStride + 4 * c4);
    x1[i] = *reinterpret_cast<const float4*>(o1 + hh * kOStride + 4 * c4);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float m0 = s0[i].x, l0 = s0[i].y, m1 = s1[i].x, l1 = s1[i].y;
    const float M = fmaxf(m0, m1);
    const float a0 = (m0 == -INFINITY) ? 0.0f : fast_exp2(m0 - M);
    const float a1 = (m1 == -INFINITY) ? 0.0f : fast_exp2(m1 - M);
    const float L = l0 * a0 + l1 * a1;
    const float4 o = make_float4(x0[i].x * a0 + x1[i].x * a1, x0[i].y * a0 + x1[i].y * a1,
                                 x0[i].z * a0 + x1[i].z * a1, x0[i].w * a0 + x1[i].w * a1);
    const int hd = hg * 16 + hq + 4 * i;
    if (a.nsplit == 1) {
      const float inv = (L > 0.0f) ? __builtin_amdgcn_rcpf(L) : 0.0f;
      reinterpret_cast<float4*>(a.out + ((int64_t)qrow * a.H + hd) * kLatentDim)[c4] =
          make_float4(o.x * inv, o.y * inv, o.z * inv, o.w * inv);
      if (c4 == 0) a.lse[(int64_t)qrow * a.H + hd] = (L > 0.0f) ? (M + __builtin_amdgcn_logf(L)) * kLn2 : -INFINITY;
    } else {
      const int64_t pidx = ((int64_t)qrow * a.nsplit + split) * a.H + hd;
      // streaming (nt) stores: the partials are read once, by the merge on other
      // compute units, so they need not stay in this L2 (the kernel's end then has
      // fewer dirty lines to write back: 11.6 -> 11.0 us per decode call at 1M)
      __builtin_nontemporal_store(v4f{o.x, o.y, o.z, o.w}, reinterpret_cast<v4f*>(a.part_o + pidx * kLatentDim) + c4);
      if (c4 == 0) {
        a.part_ml[2 * pidx] = M;
        a.part_ml[2 * pidx + 1] = L;
      }
    }
  }
}

// ---- one row range per query: one workgroup per (query, 64 heads) ----------------
// With many queries (a prefill chunk) every query gets one workgroup, and it takes 64
// heads, so each gathered and dequantised tile of 32 rows serves 64 heads instead of
// 16.  Eight wavefronts on one tile at a time: wavefront w owns heads 16*(w%4)..+15
// of the group and, for the values, channels 256*(w/4)..+255; the logits of its heads
// are the sum (in a fixed order) of the halves computed by the two wavefronts that
// share them, so both keep the same softmax state.  A thread gathers 32 channels of
// one tile row (16 code bytes + 2 scale bytes, or 64 bytes of a window row).
constexpr int kWideHeads = 64;
constexpr int kWideMaxRows = CSA2_MAX_K + CSA2_MAX_WINDOW;
constexpr int kWStride = kLatentDim;  // bf16 per X row: unpadded, wchunk() spreads the banks
// Physical 16-byte chunk of logical chunk c in row r of a wide-kernel tile: xchunk's
// spread of one row's chunks, then a row term, so that every LDS access pattern of the
// kernel reaches distinct banks: the 8 rows {0..3, 8..11} of one chunk that a logits
// read serves per pass, the 4 rows x 32 bytes of a transposing read, and the 8 chunks
// of one row a dequantising store writes.  (With the padded stride and xchunk the
// first two patterns met 2-way conflicts; the kernel gained about 1%: 2.60 against
// 2.63 ms for a 4096-query chunk, so the bank conflicts were not what bounds it.)
CSA2_DEV int wchunk(int r, int c) {
  const int f = (2 * (r & 3)) | ((r >> 3) & 1) | ((((r >> 3) ^ (r >> 4)) & 1) << 3);
  return c ^ ((c >> 3) & 7) ^ f;
}
struct __align__(16) WideSmem {
  uint16_t x[3][kRT * kWStride];  // X[row][ch] of three tiles, 16-byte chunks swizzled by wchunk()
  float red[2][4][2][2][4][64];   // partial logits [tile parity][head group][channel half][mtile][r][lane]
  int src[kWideMaxRows];          // source of every row of the query
};
static_assert(sizeof(WideSmem) <= 160 * 1024, "attention LDS exceeds 160 KB");

struct WideRegs {
  uint4 code;     // FP4 entry: 16 code bytes (32 channels)
  uint32_t sc;    // FP4 entry: the two E4M3 scale bytes of those channels
  uint4 win[4];   // window row: 32 bf16 (FP8 window: 32 code bytes in win[0..1])
  uint32_t wsc;   // FP8 window row: its E8M0 scale byte
  int kind;       // 1: FP4 entry, 2: window row, 0: no row
};

template <bool W8>
CSA2_DEV void issue_wide(const AttnArgs& a, const int* src_rows, int tid, int tile_row0, bool has_main, bool has_win,
                         WideRegs& t) {
  const int row = tid >> 4, c16 = tid & 15;
  const int src = src_rows[tile_row0 + row];
  t.kind = src >= 0 ? 1 : (src <= -2 ? 2 : 0);
  if (has_main) {
    const int64_t slot = src >= 0 ? src : 0;
    t.code = reinterpret_cast<const uint4*>(a.main_codes + slot * kMainRowBytes)[c16];
    t.sc = reinterpret_cast<const uint16_t*>(a.main_scales + slot * kMainScaleBytes)[c16];
  } else {
    t.code = make_uint4(0u, 0u, 0u, 0u);
    t.sc = 0u;
  }
  t.wsc = 0u;
  if (has_win && W8) {
    const int64_t wrow = src <= -2 ? (int64_t)(-2 - src) : 0;
    const uint4* wp = reinterpret_cast<const uint4*>(a.swa8 + wrow * kLatentDim) + 2 * c16;
    t.win[0] = wp[0];
    t.win[1] = wp[1];
    t.win[2] = t.win[3] = make_uint4(0u, 0u, 0u, 0u);
    t.wsc = a.swa8_scale[wrow];
  } else if (has_win) {
    const int64_t wrow = src <= -2 ? (int64_t)(-2 - src) : 0;
    const uint4* wp = reinterpret_cast<const uint4*>(a.swa + wrow * kLatentDim) + 4 * c16;
#pragma unroll
    for (int i = 0; i < 4; ++i) t.win[i] = wp[i];
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) t.win[i] = make_uint4(0u, 0u, 0u, 0u);
  }
}

template <bool W8>
CSA2_DEV void store_wide(uint16_t* x, int tid, const WideRegs& t, bool has_main, bool has_win) {
  const int row = tid >> 4, c16 = tid & 15;
  uint4* xr = reinterpret_cast<uint4*>(x + row * kWStride);
  const uint32_t wmask = t.kind == 2 ? ~0u : 0u;
  const float X = W8 ? e8m0_scale(t.wsc) : 1.0f;
  if (has_main && !has_win) {
    // FP4 rows only: a row that is not an entry dequantises code 0 with scale 0 (the
    // loaded bytes of its stand-in slot are not used), which is +0 in every channel
    const bool m = t.kind == 1;
    const uint32_t sc = m ? t.sc : 0u;
    const float s0 = __builtin_amdgcn_cvt_f32_fp8((int)sc, 0), s1 = __builtin_amdgcn_cvt_f32_fp8((int)sc, 1);
    const uint32_t cw[4] = {m ? t.code.x : 0u, m ? t.code.y : 0u, m ? t.code.z : 0u, m ? t.code.w : 0u};
#pragma unroll
    for (int i = 0; i < 4; ++i) xr[wchunk(row, 4 * c16 + i)] = dequant8(cw[i], i < 2 ? s0 : s1);
  } else if (has_main) {
    const uint32_t mmask = t.kind == 1 ? ~0u : 0u;
    const float s0 = __builtin_amdgcn_cvt_f32_fp8((int)t.sc, 0), s1 = __builtin_amdgcn_cvt_f32_fp8((int)t.sc, 1);
    const uint32_t cw[4] = {t.code.x, t.code.y, t.code.z, t.code.w};
#pragma unroll
    for (int i = 0; i < 4; ++i)  // chunk i (8 channels) of this thread's 32 uses scale byte i / 2
      xr[wchunk(row, 4 * c16 + i)] =
          or4(and4(dequant8(cw[i], i < 2 ? s0 : s1), mmask), and4(win_chunk<W8>(t.win, i, X), wmask));
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) xr[wchunk(row, 4 * c16 + i)] = and4(win_chunk<W8>(t.win, i, X), wmask);
  }
}

template <bool W8>
__global__ __launch_bounds__(kThreads) void sparse_attn_wide_kernel(AttnArgs a) {
  __shared__ WideSmem smem;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int g = lane >> 4, n16 = lane & 15;
  const int hg = wid & 3, kh = wid >> 2;  // head group of 16 within the 64, channel half
  const int qrow = blockIdx.x;
  const int bt_row = a.prefill ? 0 : qrow;
  const int nrows = a.k + a.window;
  const int head = kWideHeads * blockIdx.y + 16 * hg + n16;  // head of this lane in every accumulator

  // Q^T operand for the logits over this wavefront's 256 channels: lane holds head n16
  // of its group, channels 256*kh + 32*ks + 8*g .. +7
  uint4 qop[8];
  const uint16_t* qp = a.q + ((int64_t)qrow * a.H + head) * kLatentDim + 256 * kh + 8 * g;
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) qop[ks] = *reinterpret_cast<const uint4*>(qp + 32 * ks);

  v4f acc[16];  // O^T: M-tile mt covers channels 256*kh + 16*mt + 4*g + r, column = head
#pragma unroll
  for (int mt = 0; mt < 16; ++mt) acc[mt] = v4f{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.0f;

  // sources of every row (FP4 slot, -2 - window row, or -1 for none), padded to tiles
  const int nrows_pad = (nrows + kRT - 1) / kRT * kRT;
  for (int r = tid; r < nrows_pad; r += kThreads) {
    int src = -1;
    if (r >= nrows) {
    } else if (r < a.k) {
      const int j = a.topk_idx[(int64_t)qrow * a.k + r];
      if (j >= 0) src = a.block_table[(int64_t)bt_row * a.max_pages + (j >> 6)] * kPage + (j & 63);
    } else {
      const int wr = r - a.k;
      if (a.prefill) {
        if (qrow + wr >= a.swa_first_valid) src = -2 - (qrow + wr);
      } else if (wr < a.swa_len[qrow]) {
        src = -2 - (qrow * a.window + wr);
      }
    }
    smem.src[r] = src;
  }
  lds_barrier();
  auto has_main = [&](int r0) { return r0 < a.k; };
  auto has_win = [&](int r0) { return a.window > 0 && r0 + kRT > a.k; };
  const int ntiles = nrows_pad / kRT;

  // One barrier per tile.  Iteration t: partial logits of tile t (X buffer t%3) into
  // red[t%2]; dequantise tile t+1 (loaded during iteration t-1) into X buffer (t+1)%3;
  // issue the loads of tile t+2; barrier; then the softmax and P.X of tile t.  The
  // buffer written in iteration t was last read in iteration t-2, and red[t%2] in
  // iteration t-2, both before the barrier of iteration t-1.
  WideRegs cur;
  issue_wide<W8>(a, smem.src, tid, 0, has_main(0), has_win(0), cur);
  store_wide<W8>(smem.x[0], tid, cur, has_main(0), has_win(0));
  // the Q operand is complete before the tile loop, whose waits then cover only the
  // tile loads in flight
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) asm volatile("" ::"v"(qop[ks].x), "v"(qop[ks].y), "v"(qop[ks].z), "v"(qop[ks].w));
  if (ntiles > 1) issue_wide<W8>(a, smem.src, tid, kRT, has_main(kRT), has_win(kRT), cur);
  lds_barrier();
  // The loop is unrolled by the three X buffers, so that each step's buffer is a
  // compile-time constant and its LDS addresses take immediate offsets instead of
  // per-read address arithmetic.
  auto tile_step = [&](const int t, auto bsel) __attribute__((always_inline)) {
    constexpr int B = decltype(bsel)::value;
    const int row0 = t * kRT;
    const uint16_t* xt = smem.x[B];  // a constant buffer: LDS offsets fold into the instructions
    float(&red)[4][2][2][4][64] = smem.red[t & 1];
    // ---- partial logits over this wavefront's 256 channels, two 16-row M-tiles whose
    // MFMA chains alternate (no MFMA waits on the one just before it)
    {
      v4f sl[2] = {v4f{0.f, 0.f, 0.f, 0.f}, v4f{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          const int xrow = 8 * (n16 >> 2) + 4 * tt + (n16 & 3);  // lane group g gets rows 8g .. 8g+7
          const uint4 xa = reinterpret_cast<const uint4*>(xt + xrow * kWStride)[wchunk(xrow, 32 * kh + 4 * ks + g)];
          sl[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xa), as_bf16x8(qop[ks]), sl[tt], 0, 0, 0);
        }
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int r = 0; r < 4; ++r) red[hg][kh][tt][r][lane] = sl[tt][r];
    }
    if (t + 1 < ntiles) store_wide<W8>(smem.x[(B + 1) % 3], tid, cur, has_main(row0 + kRT), has_win(row0 + kRT));
    if (t + 2 < ntiles)
      issue_wide<W8>(a, smem.src, tid, row0 + 2 * kRT, has_main(row0 + 2 * kRT), has_win(row0 + 2 * kRT), cur);
    lds_barrier();
    float z[2][4];
    float tmax = -INFINITY;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float v = red[hg][0][tt][r][lane] + red[hg][1][tt][r][lane];
        const int rl = row0 + 8 * g + 4 * tt + r;
        const bool valid = smem.src[rl] != -1;
        // v * scale once rounded (+ 0), or -inf for a row with no source: a select of
        // constants, so the logit loads stay unconditional (no branch per row)
        z[tt][r] = __builtin_fmaf(v, a.scale_log2, valid ? 0.0f : -INFINITY);
        tmax = fmaxf(tmax, z[tt][r]);
      }
    tmax = max_rows(tmax);
    // the reference maximum moves only when a tile's maximum passes it by more than
    // kLazyMax (log2 units), so the weights stay <= 2^kLazyMax and O is rescaled on a
    // few tiles per query instead of on most
    const float m_new = (tmax > m_run + kLazyMax) ? tmax : m_run;
    const float alpha = (m_new == -INFINITY) ? 1.0f : fast_exp2(m_run - m_new);
    float p[2][4];
    float psum = 0.0f;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        p[tt][r] = fast_exp2(z[tt][r] - (m_new == -INFINITY ? 0.0f : m_new));
        psum += p[tt][r];
      }
    psum = sum_rows(psum);
    l_run = l_run * alpha + psum;
    m_run = m_new;
    uint32_t phi[4], plo[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float a0 = p[i >> 1][2 * (i & 1)], a1 = p[i >> 1][2 * (i & 1) + 1];
      phi[i] = pack_bf16(a0, a1);
      plo[i] = pack_bf16(a0 - __uint_as_float(phi[i] << 16), a1 - __uint_as_float(phi[i] & 0xFFFF0000u));
    }
    const bf16x8 Bhi = as_bf16x8(make_uint4(phi[0], phi[1], phi[2], phi[3]));
    const bf16x8 Blo = as_bf16x8(make_uint4(plo[0], plo[1], plo[2], plo[3]));
    // rescale O only when some head's running maximum moved (alpha == 1 leaves it as is)
    if (__builtin_amdgcn_ballot_w64(alpha != 1.0f) != 0ull) {
#pragma unroll
      for (int mt = 0; mt < 16; ++mt) acc[mt] *= alpha;
    }
    // X^T operand of M-tile mt (channels 256*kh + 16*mt + ..), transposing LDS reads
    // (rows 8g + n16/4 and 4 below it share wchunk's row term)
    const int tr_c = n16 & 3, tr_r = 8 * g + (n16 >> 2);
    const uint16_t* tr_row = xt + tr_r * kWStride + 4 * (tr_c & 1);
    // two M-tiles at a time, so that each accumulator's second MFMA (P's remainder)
    // is not issued right behind its first
#pragma unroll
    for (int mt = 0; mt < 16; mt += 2) {
      bf16x8 A[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const uint16_t* tp = tr_row + 8 * wchunk(tr_r, 32 * kh + 2 * (mt + u) + (tr_c >> 1));
        const bf16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)tp);
        const bf16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(tp + 4 * kWStride));
        A[u] = __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) acc[mt + u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[u], Bhi, acc[mt + u], 0, 0, 0);
#pragma unroll
      for (int u = 0; u < 2; ++u) acc[mt + u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[u], Blo, acc[mt + u], 0, 0, 0);
    }
  };
  for (int t = 0; t < ntiles; t += 3) {  // ntiles is uniform: every wavefront takes the same steps
    tile_step(t, std::integral_constant<int, 0>{});
    if (t + 1 < ntiles) tile_step(t + 1, std::integral_constant<int, 1>{});
    if (t + 2 < ntiles) tile_step(t + 2, std::integral_constant<int, 2>{});
  }

  // ---- write: lane holds head `head`, channels 256*kh + 16*mt + 4*g + r
  const float inv = (l_run > 0.0f) ? __builtin_amdgcn_rcpf(l_run) : 0.0f;
  float* op = a.out + ((int64_t)qrow * a.H + head) * kLatentDim + 256 * kh + 4 * g;
#pragma unroll
  for (int mt = 0; mt < 16; ++mt)
    *reinterpret_cast<float4*>(op + 16 * mt) =
        make_float4(acc[mt][0] * inv, acc[mt][1] * inv, acc[mt][2] * inv, acc[mt][3] * inv);
  if (kh == 0 && g == 0)
    a.lse[(int64_t)qrow * a.H + head] = (l_run > 0.0f) ? (m_run + __builtin_amdgcn_logf(l_run)) * kLn2 : -INFINITY;
}

// Combine the row ranges of one (query, head): out = sum_s 2^(m_s-M) O_s / L.
// One wavefront per workgroup, kMergeSlices workgroups per (query, head), each owning
// 64 channels (one per lane): a workgroup then reads ns * 256 bytes of partials, where
// one per (query, head) read ns * 2 KB and was held back by how many loads one
// compute unit keeps in flight.  With at most B <= 64 ranges the wavefront issues the
// loads of every range's O_s at once (unconditional: addresses past the last range
// are clamped to it, weight 0) together with lane s's (m_s, l_s), takes M and L with
// wave reductions, and sums the ranges in index order with one fma chain per channel:
// one round of loads, no LDS, no barrier.  More ranges take rounds of B.
constexpr int kMergeThreads = 64;
constexpr int kMergeSlices = kLatentDim / kMergeThreads;
template <int B>
__global__ __launch_bounds__(kMergeThreads) void attn_merge_kernel(AttnArgs a) {
  const int head = blockIdx.x / kMergeSlices, slice = blockIdx.x % kMergeSlices, qrow = blockIdx.y;
  const int lane = threadIdx.x;
  const int ns = a.nsplit;
  const int64_t base = (int64_t)qrow * ns * a.H + head;  // + s * H
  const float* po = a.part_o + kMergeThreads * slice + lane;  // + pidx * 512
  auto ml_of = [&](int s) { return *reinterpret_cast<const float2*>(a.part_ml + 2 * (base + (int64_t)s * a.H)); };
  float o = 0.0f;
  float M, L = 0.0f;
  auto accumulate = [&](const float (&v)[B], float w) {
#pragma unroll
    for (int u = 0; u < B; ++u) o = fmaf(v[u], __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), u)), o);
  };
  if (ns <= B) {
    float v[B];
#pragma unroll
    for (int u = 0; u < B; ++u) v[u] = po[(base + (int64_t)min(u, ns - 1) * a.H) * kLatentDim];
    const float2 ml = lane < ns ? ml_of(lane) : make_float2(-INFINITY, 0.0f);
    M = wave_max(ml.x);
    const float w = (ml.x == -INFINITY) ? 0.0f : fast_exp2(ml.x - M);
    L = wave_sum(ml.y * w);
    accumulate(v, w);
  } else {
    M = -INFINITY;
    for (int s0 = 0; s0 < ns; s0 += 64)
      if (s0 + lane < ns) M = fmaxf(M, ml_of(s0 + lane).x);
    M = wave_max(M);
    for (int s0 = 0; s0 < ns; s0 += B) {
      float v[B];
#pragma unroll
      for (int u = 0; u < B; ++u) v[u] = po[(base + (int64_t)min(s0 + u, ns - 1) * a.H) * kLatentDim];
      const float2 ml = (lane < B && s0 + lane < ns) ? ml_of(s0 + lane) : make_float2(-INFINITY, 0.0f);
      const float w = (ml.x == -INFINITY) ? 0.0f : fast_exp2(ml.x - M);
      L += wave_sum(ml.y * w);
      accumulate(v, w);
    }
  }
  const float inv = (L > 0.0f) ? __builtin_amdgcn_rcpf(L) : 0.0f;
  a.out[((int64_t)qrow * a.H + head) * kLatentDim + kMergeThreads * slice + lane] = o * inv;
  if (slice == 0 && lane == 0)
    a.lse[(int64_t)qrow * a.H + head] = (L > 0.0f) ? (M + __builtin_amdgcn_logf(L)) * kLn2 : -INFINITY;
}

static void launch_merge(const AttnArgs& a, hipStream_t stream) {
  const dim3 grid((unsigned)(a.H * kMergeSlices), (unsigned)a.nq), block(kMergeThreads);
  const int ns = a.nsplit;
  if (ns <= 8) hipLaunchKernelGGL(attn_merge_kernel<8>, grid, block, 0, stream, a);
  else if (ns <= 16) hipLaunchKernelGGL(attn_merge_kernel<16>, grid, block, 0, stream, a);
  else if (ns <= 24) hipLaunchKernelGGL(attn_merge_kernel<24>, grid, block, 0, stream, a);
  else if (ns <= 32) hipLaunchKernelGGL(attn_merge_kernel<32>, grid, block, 0, stream, a);
  else if (ns <= 40) hipLaunchKernelGGL(attn_merge_kernel<40>, grid, block, 0, stream, a);
  else if (ns <= 48) hipLaunchKernelGGL(attn_merge_kernel<48>, grid, block, 0, stream, a);
  else hipLaunchKernelGGL(attn_merge_kernel<64>, grid, block, 0, stream, a);
}

// Row ranges per query: enough workgroups to spread a small batch over the chip,
// one range when there are many queries.
static void plan_splits(int nq, int H, int k, int window, int* nsplit, int* rows_per_split) {
  const int total = k + window;
  const int tiles = (total + kRT - 1) / kRT;
  const long long groups = (long long)nq * (H / 16);
  int want = (int)((256 + groups - 1) / groups);  // one 512-thread workgroup per CU
  if (want < 1) want = 1;
  int tiles_per = (tiles + want - 1) / want;
  if (tiles_per < 2 && tiles >= 2) tiles_per = 2;
  *rows_per_split = tiles_per * kRT;
  *nsplit = (total + *rows_per_split - 1) / *rows_per_split;
}

static size_t part_bytes(int nq, int H, int nsplit) {
  if (nsplit <= 1) return 0;
  return (size_t)nq * nsplit * H * (kLatentDim + 2) * sizeof(float);
}

static int run_attention(AttnArgs a, void* ws, size_t ws_bytes, hipStream_t stream) {
  plan_splits(a.nq, a.H, a.k, a.window, &a.nsplit, &a.rows_per_split);
  const size_t need = part_bytes(a.nq, a.H, a.nsplit);
  if (need > 0) {
    if (!ws || ws_bytes < need) return CSA2_ERR_WORKSPACE;
    a.part_o = reinterpret_cast<float*>(ws);
    a.part_ml = a.part_o + (size_t)a.nq * a.nsplit * a.H * kLatentDim;
  }
  const bool w8 = a.swa8 != nullptr;
  if (a.nsplit == 1 && a.H % kWideHeads == 0) {  // many queries: a workgroup takes 64 heads
    const dim3 grid((unsigned)a.nq, (unsigned)(a.H / kWideHeads));
    if (w8) hipLaunchKernelGGL(sparse_attn_wide_kernel<true>, grid, dim3(kThreads), 0, stream, a);
    else hipLaunchKernelGGL(sparse_attn_wide_kernel<false>, grid, dim3(kThreads), 0, stream, a);
    return launch_status();
  }
  const dim3 grid((unsigned)a.nsplit, (unsigned)(a.H / 16), (unsigned)a.nq);
  if (w8) hipLaunchKernelGGL(sparse_attn_kernel<true>, grid, dim3(kThreads), 0, stream, a);
  else hipLaunchKernelGGL(sparse_attn_kernel<false>, grid, dim3(kThreads), 0, stream, a);
  if (a.nsplit > 1) launch_merge(a, stream);
  return launch_status();
}

static size_t attn_ws_size(int nq, int H, int k, int window) {
  int nsplit, rps;
  if (nq <= 0 || H <= 0) return 256;
  plan_splits(nq, H, k, window, &nsplit, &rps);
  const size_t b = part_bytes(nq, H, nsplit);
  return b > 0 ? b : 256;
}

// swa: the window rows' storage (bf16 rows, or the FP8 codes; the FP8 scales are
// checked by the caller)
static int check_common(const csa2_fp4_cache* cache, const uint16_t* q, int32_t H, const int32_t* topk_idx, int32_t k,
                        const int32_t* block_table, int32_t max_pages, const void* swa, int32_t window,
                        float scale, float* out, float* lse) {
  if (!cache_ok(cache)) return CSA2_ERR_NULL;
  if (!cache_shape_ok(cache)) return CSA2_ERR_SHAPE;
  if (H < 16 || H > 128 || H % 16 != 0) return CSA2_ERR_SHAPE;
  if (k < 0 || k > CSA2_MAX_K || window < 0 || window > CSA2_MAX_WINDOW || max_pages < 0) return CSA2_ERR_SHAPE;
  if (!(scale == scale)) return CSA2_ERR_SHAPE;
  if (!q || !out || !lse) return CSA2_ERR_NULL;
  if (k > 0 && (!topk_idx || !block_table)) return CSA2_ERR_NULL;
  if (window > 0 && !swa) return CSA2_ERR_NULL;
  return CSA2_OK;
}

}  // namespace csa2

using namespace csa2;

extern "C" size_t sparse_attn_decode_workspace_size(int32_t B, int32_t H, int32_t k, int32_t window) {
  return attn_ws_size(B, H, k, window);
}

extern "C" size_t sparse_attn_prefill_chunk_workspace_size(int32_t T, int32_t H, int32_t k, int32_t window) {
  return attn_ws_size(T, H, k, window);
}

namespace csa2 {

static int decode_impl(const csa2_fp4_cache* cache, const uint16_t* q, int32_t H, const int32_t* topk_idx, int32_t k,
                       const int32_t* block_table, int32_t max_pages, const uint16_t* swa, const uint8_t* swa8,
                       const uint8_t* swa8_scale, const int32_t* swa_len, int32_t window, float softmax_scale,
                       int32_t B, float* out, float* lse, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (B < 0) return CSA2_ERR_SHAPE;
  const void* win = swa8 ? static_cast<const void*>(swa8) : static_cast<const void*>(swa);
  const int st = check_common(cache, q, H, topk_idx, k, block_table, max_pages, win, window, softmax_scale, out, lse);
  if (st != CSA2_OK) return st;
  if (window > 0 && (!swa_len || (swa8 && !swa8_scale))) return CSA2_ERR_NULL;
  if (B == 0) return CSA2_OK;
  AttnArgs a{};
  a.main_codes = cache->main_codes;
  a.main_scales = cache->main_scales;
  a.q = q;
  a.H = H;
  a.topk_idx = topk_idx;
  a.k = k;
  a.block_table = block_table;
  a.max_pages = max_pages;
  a.swa = swa8 ? nullptr : swa;
  a.swa8 = window > 0 ? swa8 : nullptr;
  a.swa8_scale = swa8_scale;
  a.swa_len = swa_len;
  a.window = window;
  a.prefill = 0;
  a.swa_first_valid = 0;
  a.scale_log2 = softmax_scale * kLog2e;
  a.nq = B;
  a.out = out;
  a.lse = lse;
  return run_attention(a, ws, ws_bytes, stream);
}

static int prefill_impl(const csa2_fp4_cache* cache, const uint16_t* q, int32_t H, const int32_t* topk_idx, int32_t k,
                        const int32_t* block_table, int32_t max_pages, int64_t chunk_start, int32_t T,
                        const uint16_t* swa, const uint8_t* swa8, const uint8_t* swa8_scale, int32_t swa_first_valid,
                        int32_t window, float softmax_scale, float* out, float* lse, void* ws, size_t ws_bytes,
                        hipStream_t stream) {
  if (T < 0 || chunk_start < 0 || swa_first_valid < 0) return CSA2_ERR_SHAPE;
  const void* win = swa8 ? static_cast<const void*>(swa8) : static_cast<const void*>(swa);
  const int st = check_common(cache, q, H, topk_idx, k, block_table, max_pages, win, window, softmax_scale, out, lse);
  if (st != CSA2_OK) return st;
  if (window > 0 && swa8 && !swa8_scale) return CSA2_ERR_NULL;
  if (T == 0) return CSA2_OK;
  AttnArgs a{};
  a.main_codes = cache->main_codes;
  a.main_scales = cache->main_scales;
  a.q = q;
  a.H = H;
  a.topk_idx = topk_idx;
  a.k = k;
  a.block_table = block_table;
  a.max_pages = max_pages;
  a.swa = swa8 ? nullptr : swa;
  a.swa8 = window > 0 ? swa8 : nullptr;
  a.swa8_scale = swa8_scale;
  a.swa_len = nullptr;
  a.window = window;
  a.prefill = 1;
  a.swa_first_valid = swa_first_valid;
  a.scale_log2 = softmax_scale * kLog2e;
  a.nq = T;
  a.out = out;
  a.lse = lse;
  return run_attention(a, ws, ws_bytes, stream);
}

}  // namespace csa2

extern "C" int sparse_attn_decode(const csa2_fp4_cache* cache, const uint16_t* q, int32_t H, const int32_t* topk_idx,
                                  int32_t k, const int32_t* block_table, int32_t max_pages, const uint16_t* swa,
                                  const int32_t* swa_len, int32_t window, float softmax_scale, int32_t B, float* out,
                                  float* lse, void* ws, size_t ws_bytes, hipStream_t stream) {
  return decode_impl(cache, q, H, topk_idx, k, block_table, max_pages, swa, nullptr, nullptr, swa_len, window,
                     softmax_scale, B, out, lse, ws, ws_bytes, stream);
}

extern "C" int sparse_attn_decode_fp8win(const csa2_fp4_cache* cache, const uint16_t* q, int32_t H,
                                         const int32_t* topk_idx, int32_t k, const int32_t* block_table,
                                         int32_t max_pages, const uint8_t* swa_codes, const uint8_t* swa_scales,
                                         const int32_t* swa_len, int32_t window, float softmax_scale, int32_t B,
                                         float* out, float* lse, void* ws, size_t ws_bytes, hipStream_t stream) {
  return decode_impl(cache, q, H, topk_idx, k, block_table, max_pages, nullptr, swa_codes, swa_scales, swa_len,
                     window, softmax_scale, B, out, lse, ws, ws_bytes, stream);
}

extern "C" int sparse_attn_prefill_chunk(const csa2_fp4_cache* cache, const uint16_t* q, int32_t H,
                                         const int32_t* topk_idx, int32_t k, const int32_t* block_table,
                                         int32_t max_pages, int64_t chunk_start, int32_t T, const uint16_t* swa,
                                         int32_t swa_first_valid, int32_t window, float softmax_scale, float* out,
                                         float* lse, void* ws, size_t ws_bytes, hipStream_t stream) {
  return prefill_impl(cache, q, H, topk_idx, k, block_table, max_pages, chunk_start, T, swa, nullptr, nullptr,
                      swa_first_valid, window, softmax_scale, out, lse, ws, ws_bytes, stream);
}

extern "C" int sparse_attn_prefill_chunk_fp8win(const csa2_fp4_cache* cache, const uint16_t* q, int32_t H,
                                                const int32_t* topk_idx, int32_t k, const int32_t* block_table,
                                                int32_t max_pages, int64_t chunk_start, int32_t T,
                                                const uint8_t* swa_codes, const uint8_t* swa_scales,
                                                int32_t swa_first_valid, int32_t window, float softmax_scale,
                                                float* out, float* lse, void* ws, size_t ws_bytes,
                                                hipStream_t stream) {
  return prefill_impl(cache, q, H, topk_idx, k, block_table, max_pages, chunk_start, T, nullptr, swa_codes,
                      swa_scales, swa_first_valid, window, softmax_scale, out, lse, ws, ws_bytes, stream);
}
