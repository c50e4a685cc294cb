// pkv_decode_mfma.hip -- split-KV paged decode kernel for CDNA4 (gfx950),
// matrix-core path, used when the rows that share a kv head (G query heads x
// q_len tokens) fill a 16-row MFMA tile.
//
// Method as in pkv_decode.hip (AstrAI commit d565d44, "attn_paged_decode.cu"
// commit notes: the MMA split-KV paged decode kernel packs the query heads of
// one kv head into tensor-core tiles and resolves the page table once per key
// tile).  gfx950 mapping:
//  * a workgroup covers one key split of up to 32 rows (two 16-row blocks)
//    of each of hpb kv heads (1, 2 or 4); wave w works on head w % hpb and
//    takes every (NW / hpb)-th 16-key tile; the waves of a head merge their
//    (m, l, O) once at the end through LDS;
//  * K and V tiles are fetched with full-row 128-bit loads into registers
//    (double-buffered, so the next tile's loads fly during this tile's math)
//    and written to a per-wave LDS slice with an XOR chunk swizzle;
//  * S^T = K Q^T with v_mfma_f32_16x16x32_bf16: the K operand is a
//    ds_read_b128 per lane, Q stays in registers; the S^T accumulator leaves
//    each lane one query row and four keys, so the online-softmax max, exp
//    and rescale are in-lane apart from two permlane swaps;
//  * O^T = V^T P^T with v_mfma_f32_16x16x16_bf16: V^T comes straight from
//    the row-major V tile through ds_read_b64_tr_b16 (the gfx950 transposing
//    LDS read), P^T is the S^T register layout itself; P is split into a bf16
//    high part and a bf16 remainder (two MFMAs, both converted with the
//    gfx950 v_cvt_pk_bf16_f32) so the probabilities keep about 16
//    significant bits, and the row sums l use the fp32 values;
//  * exclusion (tail, causal, -inf mask) is a select; scores are in base 2.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

using namespace dev;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

// Two probabilities as bf16 high parts (round to nearest even, one
// v_cvt_pk_bf16_f32 for the pair) and the bf16 roundings of what remains of
// each.  The high parts' fp32 values come back from the packed word by a
// shift and a mask, not by converting each value on its own.
__device__ __forceinline__ void split_pair(float x, float y, bf16x2_t &hi, bf16x2_t &lo) {
  hi = __builtin_convertvector(f32x2_t{x, y}, bf16x2_t);
  const uint32_t u = __builtin_bit_cast(uint32_t, hi);
  lo = __builtin_convertvector(f32x2_t{x - __uint_as_float(u << 16), y - __uint_as_float(u & 0xffff0000u)},
                               bf16x2_t);
}

constexpr int kBtCap = 1024;
constexpr int KT = 16;  // keys per wave tile
constexpr float kRescaleLog2 = 8.f;  // lazy-rescale threshold (base-2 score units)

template <int D>
struct MLay {
  static constexpr int NW = kWavesPerBlock;
  static constexpr int NCH = D / 8;          // 16-byte chunks per row
  static constexpr int LPR = D / 8;          // lanes per row in a coalesced load
  static constexpr int RPI = 64 / LPR;       // rows per load instruction
  static constexpr int NLD = KT / RPI;       // load instructions per 16-key tile (K or V)
  static constexpr int TILE_ELEMS = KT * D;  // bf16 per K (or V) tile
  static constexpr int MASK_BYTES = 2 * 64 * 16;      // mask values: [row block][lane] float4
  static constexpr int WAVE_LDS = 2 * TILE_ELEMS * 2 + MASK_BYTES;  // bytes: K + V tile, mask
  static constexpr int BT_BYTES = (kBtCap + 4) * 4;
  static constexpr int OB_STRIDE = D + 4;    // merge-buffer row stride (floats), padded against bank conflicts
  // merge phase: per-wave O rows and (m, l)
  static constexpr int MERGE_BYTES = NW * 16 * OB_STRIDE * 4 + NW * 16 * 2 * 4;
  static constexpr int MAIN_BYTES = BT_BYTES + NW * WAVE_LDS;
  static constexpr int SMEM_BYTES = MAIN_BYTES > MERGE_BYTES ? MAIN_BYTES : MERGE_BYTES;
  // swizzles (16-byte chunk index within a row)
  __device__ static int swk(int ch, int row) { return ch ^ (row & (NCH - 1)); }
  __device__ static int swv(int ch, int row) { return ch ^ ((2 * row) & (NCH - 2)); }
};

template <int D, int NRB, bool MASK>
struct MTile {
  uint4 k[MLay<D>::NLD];
  uint4 v[MLay<D>::NLD];
  float mk[MASK ? NRB : 1][4];  // additive mask of this lane's 4 keys (per row block for 3D masks)
};

struct MCtx {
  const uint16_t *kbase, *vbase;
  const int *bt;
  int p0, page_shift, pmask;
  int64_t page_stride;
  int row_stride;
  int ke;
  int R;     // packed rows of the sequence per kv head
  int kvis;  // keys every row of this wave that exists sees (a tile below it needs no visibility select)
};

// The smallest key limit over a wave's rows that exist (rows past the
// sequence's rows see nothing and are never written, so they do not count).
template <int NRB>
__device__ __forceinline__ int wave_min_limit(const int (&lim)[NRB], int r0, int R, int lane) {
  int v = INT_MAX;
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb)
    if (r0 + (lane & 15) + 16 * rb < R) v = lim[rb] < v ? lim[rb] : v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_xor(v, d, 64);
    v = o < v ? o : v;
  }
  return v;
}

// Loads of one 16-key tile: full K/V rows, 128 bits per lane.  Rows past the
// end are clamped to the last valid key (finite data, zero weight); when a
// page holds the whole tile its page is resolved once, in scalar registers.
template <int D, int NRB, bool MASK, bool UPAGE, bool PREFILL = false>
__device__ __forceinline__ void mload(const DecodeArgs &a, const MCtx &c, int b, int r0, int base, int lane,
                                      MTile<D, NRB, MASK> &t) {
  using L = MLay<D>;
  const int ch = lane % L::LPR;
  const int jlast = c.ke - 1;
  if constexpr (UPAGE) {
    // a tile past the window end (an unconditional prefetch) reads the last key's page
    const int bj = base < jlast ? base : jlast;
    const int page = __builtin_amdgcn_readfirstlane(c.bt[(bj >> c.page_shift) - c.p0]);
    // the tile's first key in the scalar offset; keys j of the tile are j - bj < T rows further
    const int64_t pofs = (int64_t)page * c.page_stride + (int64_t)(bj & c.pmask) * c.row_stride;
    const uint16_t *kp = c.kbase + pofs;
    const uint16_t *vp = c.vbase + pofs;
    if (D == 128 && !PREFILL && base + KT - 1 <= jlast) {
      // every key of the tile exists (bj = base): row ii * RPI + lane / LPR of
      // the tile, one multiply for the lane and a wave-uniform step per load
      // (in the 32-row kernel at D = 128 only: 1.5-2% on 16 x 4096 keys at
      // G = 4 and 8; no gain at D = 64 or in the prefill-shaped kernel,
      // register spills at D = 256)
      const uint32_t o0 = (uint32_t)((lane / L::LPR) * c.row_stride);
      const uint32_t step = (uint32_t)(L::RPI * c.row_stride);
#pragma unroll
      for (int ii = 0; ii < L::NLD; ++ii) {
        const uint32_t off = o0 + ii * step;
        t.k[ii] = load_stream(reinterpret_cast<const uint4 *>(kp + off) + ch);
        __builtin_amdgcn_sched_barrier(0);  // fixed issue order (see mtile_loop)
        t.v[ii] = load_stream(reinterpret_cast<const uint4 *>(vp + off) + ch);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
#pragma unroll
      for (int ii = 0; ii < L::NLD; ++ii) {
        int j = base + ii * L::RPI + lane / L::LPR;
        j = j < jlast ? j : jlast;
        const uint32_t off = (uint32_t)((j - bj) * c.row_stride);
        t.k[ii] = load_stream(reinterpret_cast<const uint4 *>(kp + off) + ch);
        __builtin_amdgcn_sched_barrier(0);
        t.v[ii] = load_stream(reinterpret_cast<const uint4 *>(vp + off) + ch);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  } else {
#pragma unroll
    for (int ii = 0; ii < L::NLD; ++ii) {
      int j = base + ii * L::RPI + lane / L::LPR;
      j = j < jlast ? j : jlast;
      const int page = c.bt[(j >> c.page_shift) - c.p0];
      const int64_t off = (int64_t)page * c.page_stride + (int64_t)(j & c.pmask) * c.row_stride;
      t.k[ii] = load_stream(reinterpret_cast<const uint4 *>(c.kbase + off) + ch);
      __builtin_amdgcn_sched_barrier(0);  // fixed issue order (see mtile_loop)
      t.v[ii] = load_stream(reinterpret_cast<const uint4 *>(c.vbase + off) + ch);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  if constexpr (MASK) {
    const int q = lane >> 4;
    const int cc = lane & 15;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int j = base + 4 * q + i;
      j = j < jlast ? j : jlast;
      const float *mrow = a.mask + (int64_t)b * a.mask_sb + j;
      // one load per row block on every path (2D masks, mask_sq = 0, load the
      // same entry): a branch-dependent load count makes the compiler wait for
      // all loads at the loop header
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
        const int rr = r0 + cc + 16 * rb < c.R ? r0 + cc + 16 * rb : c.R - 1;
        t.mk[rb][i] = mrow[(int64_t)(rr / a.G) * a.mask_sq];
      }
    }
  }
}

template <int D, int NRB>
struct MState {
  float m[NRB];           // running max of this lane's row (base 2), equal across its 4 lanes
  float l[NRB];           // this lane's share of the row sum
  f32x4_t o[NRB][D / 16]; // O^T: d = 16*nb + 4q + i, row c
};

// Registers of one tile -> the wave's LDS slice (rows XOR-swizzled by chunk;
// each lane's mask values at [row block][lane]).  The mask goes through LDS
// too, although each lane reads back its own values: kept in registers past
// the reload of the tile, they would need a copy, and a copy of registers
// whose loads are in flight makes the compiler wait for every load.
template <int D, int NRB, bool MASK>
__device__ __forceinline__ void mstore(const MTile<D, NRB, MASK> &t, uint16_t *kt, uint16_t *vt, float *mkt,
                                       int lane) {
  using L = MLay<D>;
#pragma unroll
  for (int ii = 0; ii < L::NLD; ++ii) {
    const int row = ii * L::RPI + lane / L::LPR;
    const int ch = lane % L::LPR;
    reinterpret_cast<uint4 *>(kt + row * D)[L::swk(ch, row)] = t.k[ii];
    reinterpret_cast<uint4 *>(vt + row * D)[L::swv(ch, row)] = t.v[ii];
  }
  if constexpr (MASK) {
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb)
      reinterpret_cast<float4 *>(mkt)[rb * 64 + lane] = make_float4(t.mk[rb][0], t.mk[rb][1], t.mk[rb][2], t.mk[rb][3]);
  }
  __builtin_amdgcn_wave_barrier();
}

template <int D, int NRB, bool CAUSAL, bool MASK>
__device__ __forceinline__ void mcompute(const DecodeArgs &a, const MCtx &c, int base,
                                         const float *mkt, const uint4 (&qb)[NRB][D / 32],
                                         const int (&lim)[NRB], const uint16_t *kt, const uint16_t *vt,
                                         int lane, MState<D, NRB> &st) {
  using L = MLay<D>;
  const int cc = lane & 15;
  const int q = lane >> 4;
  // S^T[key][row] = K Q^T : A = K[key cc][d 32s+8q..], B = Q^T
  f32x4_t s4[NRB];
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) s4[rb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int stp = 0; stp < D / 32; ++stp) {
    const uint4 kv = reinterpret_cast<const uint4 *>(kt + cc * D)[L::swk(4 * stp + q, cc)];
    const bf16x8_t ka = __builtin_bit_cast(bf16x8_t, kv);
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb)
      s4[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, __builtin_bit_cast(bf16x8_t, qb[rb][stp]), s4[rb], 0, 0, 0);
  }

  // scale, mask, visibility; lane holds keys base+4q+i of row r0+cc+16rb
  float sv[NRB][4];
  float dmax = -INFINITY;   // NaN (-inf - -inf) is ignored by fmaxf
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    float mk[4] = {0.f, 0.f, 0.f, 0.f};
    if constexpr (MASK) {
      const float4 m4 = reinterpret_cast<const float4 *>(mkt)[rb * 64 + lane];
      mk[0] = m4.x;
      mk[1] = m4.y;
      mk[2] = m4.z;
      mk[3] = m4.w;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      sv[rb][i] = MASK ? fmaf(s4[rb][i], a.scale_log2, mk[i] * kLog2e) : s4[rb][i] * a.scale_log2;
  }
  // a tile inside every row's window (wave-uniform) needs no visibility select
  if (!(base + KT <= c.ke && base + KT <= c.kvis)) {
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = base + 4 * q + i;
        sv[rb][i] = (j < c.ke && j < lim[rb]) ? sv[rb][i] : -INFINITY;
      }
  }
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb)
    dmax = fmaxf(dmax, fmaxf(fmaxf(sv[rb][0], sv[rb][1]), fmaxf(sv[rb][2], sv[rb][3])) - st.m[rb]);
  // lazy reference max: move it (and rescale O, l) only when a score exceeds
  // it by more than kRescaleLog2; the branch is wave-uniform
  if (__builtin_amdgcn_ballot_w64(dmax > kRescaleLog2) != 0) {
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      float mt = fmaxf(fmaxf(sv[rb][0], sv[rb][1]), fmaxf(sv[rb][2], sv[rb][3]));
      mt = xor32<OpMax>(xor16<OpMax>(mt));
      const float mnew = fmaxf(st.m[rb], mt);
      const float alpha = mnew == -INFINITY ? 1.f : fast_exp2(st.m[rb] - mnew);
      st.m[rb] = mnew;
      st.l[rb] *= alpha;
#pragma unroll
      for (int nb = 0; nb < D / 16; ++nb) st.o[rb][nb] *= alpha;
    }
  }
  bf16x4_t ph[NRB], pl[NRB];
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    const float use = st.m[rb] == -INFINITY ? 0.f : st.m[rb];
    float lsum = 0.f;
#pragma unroll
    for (int i = 0; i < 4; i += 2) {
      const float p0 = fast_exp2(sv[rb][i] - use);
      const float p1 = fast_exp2(sv[rb][i + 1] - use);
      lsum += p0;
      lsum += p1;
      bf16x2_t hi, lo;
      split_pair(p0, p1, hi, lo);
      ph[rb][i] = hi[0];
      ph[rb][i + 1] = hi[1];
      pl[rb][i] = lo[0];
      pl[rb][i + 1] = lo[1];
    }
    st.l[rb] += lsum;
  }

  // O^T[d][row] += V^T P^T : A = V^T via the transposing LDS read
  const int srow = 4 * q + (cc >> 2);      // V row this lane addresses for the transposing read
  const int sd = 4 * (cc & 3);             // its d offset within the 16-column block
#pragma unroll
  for (int nb = 0; nb < D / 16; ++nb) {
    const int d0 = 16 * nb + sd;
    const int ch = d0 >> 3;
    const int half = (d0 >> 2) & 1;
    // vt points into LDS: the C cast is an address-space cast to the LDS offset
    lds_i16x4_t *src = (lds_i16x4_t *)(reinterpret_cast<const char *>(vt) + srow * D * 2 + L::swv(ch, srow) * 16 +
                                       half * 8);
    const i16x4_t vraw = __builtin_amdgcn_ds_read_tr16_b64_v4i16(src);
    const bf16x4_t va = __builtin_bit_cast(bf16x4_t, vraw);
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      st.o[rb][nb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, ph[rb], st.o[rb][nb], 0, 0, 0);
      st.o[rb][nb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pl[rb], st.o[rb][nb], 0, 0, 0);
    }
  }
  __builtin_amdgcn_wave_barrier();
}

// Two 16-key tiles at once (keys base .. base + 31, the second tile at
// kt1 / vt1): the same scores, mask, visibility and online softmax as
// mcompute over eight keys per lane, and O^T += V^T P^T as one
// v_mfma_f32_16x16x32_bf16 per 16 columns (per P half) instead of two
// 16x16x16 ones.  The k index of that product runs over the lane's own keys:
// k slots 8q .. 8q + 3 are keys 4q + i of the first tile and slots 8q + 4 ..
// 8q + 7 keys 16 + 4q + i of the second, in the P operand (the lane's
// probabilities) and in the V^T operand (two transposing reads, one per
// tile) alike.
template <int D, int NRB, bool CAUSAL, bool MASK>
__device__ __forceinline__ void mcompute2(const DecodeArgs &a, const MCtx &c, int base, const float *mkt0,
                                          const float *mkt1, const uint4 (&qb)[NRB][D / 32], const int (&lim)[NRB],
                                          const uint16_t *kt0, const uint16_t *vt0, const uint16_t *kt1,
                                          const uint16_t *vt1, int lane, MState<D, NRB> &st) {
  using L = MLay<D>;
  const int cc = lane & 15;
  const int q = lane >> 4;
  f32x4_t s4[2][NRB];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) s4[h][rb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int stp = 0; stp < D / 32; ++stp) {
    const bf16x8_t ka0 =
        __builtin_bit_cast(bf16x8_t, reinterpret_cast<const uint4 *>(kt0 + cc * D)[L::swk(4 * stp + q, cc)]);
    const bf16x8_t ka1 =
        __builtin_bit_cast(bf16x8_t, reinterpret_cast<const uint4 *>(kt1 + cc * D)[L::swk(4 * stp + q, cc)]);
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      const bf16x8_t qv = __builtin_bit_cast(bf16x8_t, qb[rb][stp]);
      s4[0][rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka0, qv, s4[0][rb], 0, 0, 0);
      s4[1][rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka1, qv, s4[1][rb], 0, 0, 0);
    }
  }

  float sv[NRB][8];
  float dmax = -INFINITY;
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      float mk[4] = {0.f, 0.f, 0.f, 0.f};
      if constexpr (MASK) {
        const float4 m4 = reinterpret_cast<const float4 *>(h ? mkt1 : mkt0)[rb * 64 + lane];
        mk[0] = m4.x;
        mk[1] = m4.y;
        mk[2] = m4.z;
        mk[3] = m4.w;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
        sv[rb][4 * h + i] = MASK ? fmaf(s4[h][rb][i], a.scale_log2, mk[i] * kLog2e) : s4[h][rb][i] * a.scale_log2;
    }
  }
  if (!(base + 2 * KT <= c.ke && base + 2 * KT <= c.kvis)) {
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int j = base + 16 * h + 4 * q + i;
          sv[rb][4 * h + i] = (j < c.ke && j < lim[rb]) ? sv[rb][4 * h + i] : -INFINITY;
        }
  }
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    float mt = sv[rb][0];
#pragma unroll
    for (int i = 1; i < 8; ++i) mt = fmaxf(mt, sv[rb][i]);
    dmax = fmaxf(dmax, mt - st.m[rb]);
  }
  if (__builtin_amdgcn_ballot_w64(dmax > kRescaleLog2) != 0) {
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      float mt = sv[rb][0];
#pragma unroll
      for (int i = 1; i < 8; ++i) mt = fmaxf(mt, sv[rb][i]);
      mt = xor32<OpMax>(xor16<OpMax>(mt));
      const float mnew = fmaxf(st.m[rb], mt);
      const float alpha = mnew == -INFINITY ? 1.f : fast_exp2(st.m[rb] - mnew);
      st.m[rb] = mnew;
      st.l[rb] *= alpha;
#pragma unroll
      for (int nb = 0; nb < D / 16; ++nb) st.o[rb][nb] *= alpha;
    }
  }
  bf16x8_t ph[NRB], pl[NRB];
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    const float use = st.m[rb] == -INFINITY ? 0.f : st.m[rb];
    float lsum = 0.f;
#pragma unroll
    for (int i = 0; i < 8; i += 2) {
      const float p0 = fast_exp2(sv[rb][i] - use);
      const float p1 = fast_exp2(sv[rb][i + 1] - use);
      lsum += p0;
      lsum += p1;
      bf16x2_t hi, lo;
      split_pair(p0, p1, hi, lo);
      ph[rb][i] = hi[0];
      ph[rb][i + 1] = hi[1];
      pl[rb][i] = lo[0];
      pl[rb][i + 1] = lo[1];
    }
    st.l[rb] += lsum;
  }

  const int srow = 4 * q + (cc >> 2);
  const int sd = 4 * (cc & 3);
#pragma unroll
  for (int nb = 0; nb < D / 16; ++nb) {
    const int d0 = 16 * nb + sd;
    const int ch = d0 >> 3;
    const int half = (d0 >> 2) & 1;
    const int ofs = srow * D * 2 + L::swv(ch, srow) * 16 + half * 8;
    // vt0 / vt1 point into LDS: the C casts are address-space casts to LDS offsets
    const i16x4_t v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t *)(reinterpret_cast<const char *>(vt0) + ofs));
    const i16x4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t *)(reinterpret_cast<const char *>(vt1) + ofs));
    const bf16x4_t va0 = __builtin_bit_cast(bf16x4_t, v0);
    const bf16x4_t va1 = __builtin_bit_cast(bf16x4_t, v1);
    const bf16x8_t va = bf16x8_t{va0[0], va0[1], va0[2], va0[3], va1[0], va1[1], va1[2], va1[3]};
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      st.o[rb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, ph[rb], st.o[rb][nb], 0, 0, 0);
      st.o[rb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pl[rb], st.o[rb][nb], 0, 0, 0);
    }
  }
  __builtin_amdgcn_wave_barrier();
}

// One pipeline step: tile tt (in registers tr) -> LDS; issue the loads of
// tile tnext into tr; compute tile tt from LDS.
template <int D, int NRB, bool CAUSAL, bool MASK, bool UPAGE>
__device__ __forceinline__ void mstep(const DecodeArgs &a, const MCtx &c, int b, int r0, int wb, int tt,
                                      int tnext, MTile<D, NRB, MASK> &tr, const uint4 (&qb)[NRB][D / 32],
                                      const int (&lim)[NRB], uint16_t *kt, uint16_t *vt, int lane,
                                      MState<D, NRB> &st) {
  float *mkt = reinterpret_cast<float *>(vt + MLay<D>::TILE_ELEMS);
  mstore<D, NRB, MASK>(tr, kt, vt, mkt, lane);
  // unconditional (a tile past the end loads the last key again, clamped in
  // mload): the loads in flight are then the same on every path, and the
  // wait before the next tile leaves this prefetch in flight
  mload<D, NRB, MASK, UPAGE>(a, c, b, r0, wb + tnext * KT, lane, tr);
  mcompute<D, NRB, CAUSAL, MASK>(a, c, wb + tt * KT, mkt, qb, lim, kt, vt, lane, st);
}

// Register tiles per wave, as measured on MI355X (B = 16 x 4096 keys and
// B = 4 x 32768 keys, Hkv = 8): one, so that each wave keeps a single tile's
// loads in flight while it computes the previous tile -- at D <= 64 (two
// workgroups per CU) that is 8-11% faster than two, and at D = 128 without a
// mask 7-9% faster; two at D = 128 with a mask (5% faster there); one at
// D = 256, where two would spill.  More bytes in flight per CU than that
// made the random-page K/V stream slower, not faster (four tiles: up to 60%).
template <int D, int NRB, bool MASK>
constexpr int mfma_nbuf() { return (D == 128 && MASK) ? 2 : 1; }

// The key-tile loop of one wave: tiles t0, t0 + tstep, ...
template <int D, int NRB, bool CAUSAL, bool MASK, bool UPAGE, int NBUF = mfma_nbuf<D, NRB, MASK>()>
__device__ __forceinline__ void mtile_loop(const DecodeArgs &a, const MCtx &c, int b, int r0, int wb, int t0,
                                           int tstep, int ntiles, const uint4 (&qb)[NRB][D / 32],
                                           const int (&lim)[NRB], uint16_t *kt, uint16_t *vt, int lane,
                                           MState<D, NRB> &st) {
  // NBUF register tiles in a ring: tile t sits in buffer (t / tstep) % NBUF; a
  // tile goes to LDS, then the loads of the tile NBUF steps ahead are issued
  // into the freed registers
  if (t0 >= ntiles) return;
  MTile<D, NRB, MASK> tr[NBUF];
  // issue the tiles in order, not interleaved by the scheduler, so that the
  // wait for tile i leaves the loads of tiles i+1.. in flight
#pragma unroll
  for (int i = 0; i < NBUF; ++i) {
    mload<D, NRB, MASK, UPAGE>(a, c, b, r0, wb + (t0 + i * tstep) * KT, lane, tr[i]);
    __builtin_amdgcn_sched_barrier(0);
  }
  // no early exit inside a round: a step past the last tile computes a tile
  // whose keys are all past the window end (weight 0); an exit there would
  // give the loop a second path into its header and the compiler would then
  // wait for all loads at the header
  for (int t = t0; t < ntiles; t += NBUF * tstep) {
#pragma unroll
    for (int i = 0; i < NBUF; ++i) {
      const int tt = t + i * tstep;
      mstep<D, NRB, CAUSAL, MASK, UPAGE>(a, c, b, r0, wb, tt, tt + NBUF * tstep, tr[i], qb, lim, kt, vt, lane,
                                         st);
    }
  }
}

// Two resident workgroups per CU (2 waves per SIMD) where the registers allow:
// not with two row blocks at D = 256, nor at D = 128 with a mask (which spills
// within 256 registers).
template <int D, int NRB, bool MASK>
constexpr int mfma_min_blocks() { return (NRB == 2 && (D >= 256 || (D == 128 && MASK))) ? 1 : 2; }

template <int D, int NRB, bool CAUSAL, bool MASK, bool UPAGE>
__global__ __launch_bounds__(kWavesPerBlock * 64, (mfma_min_blocks<D, NRB, MASK>())) void split_decode_mfma(
    const DecodeArgs a) {
  using L = MLay<D>;
  constexpr int NW = L::NW;
  constexpr int RW = 16 * NRB;
  __shared__ __attribute__((aligned(16))) unsigned char smem_raw[L::SMEM_BYTES];
  // output row of packed row rr of head slot hh of the block, at rr * hpb + hh
  __shared__ int64_t rowtab[RW * kMaxHeadsPerBlock];

  Work wk0;
  if (!work_of<CAUSAL>(a, wk0)) return;
  const int b = wk0.b, s = wk0.s, hg = wk0.hg, rg = wk0.rg;

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int hw = w & (a.hpb - 1);   // this wave's head slot in the group
  const int wk = w >> a.lhpb;       // its index among the waves of that head
  const int wph = NW >> a.lhpb;     // waves per head
  const int g = hg * a.hpb + hw;
  const int cc = lane & 15;
  const int q = lane >> 4;
  const int r0 = rg * RW;

  const int kvlen = wk0.L;
  const SeqRows sr = wk0.sr;
  if (r0 >= sr.R) return;  // a row block past the sequence's tokens (varlen batches)
  int lim[NRB];
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) lim[rb] = row_keys(a, sr, kvlen, r0 + cc + 16 * rb);
  const int rlast = (r0 + RW < sr.R ? r0 + RW : sr.R) - 1;
  const int kmax = row_keys(a, sr, kvlen, rlast);   // the last row sees the most keys

  // splits past the unit's keys: no work; outside the in-kernel merge they
  // leave (m, l) = (-inf, 0) for the combine step
  const int nact = active_splits(a, kmax);
  const int nrt = (sr.R - r0 < RW ? sr.R - r0 : RW) * a.hpb;  // output rows of the block
  if (s >= nact) {
    if (!a.fused) empty_partials(a, sr.tok0, hg, r0, s, nrt);
    return;
  }
  // the unit's only split with keys writes the output itself
  const bool direct = !a.partials || (a.fused && nact == 1);

  int *bt_lds = reinterpret_cast<int *>(smem_raw);
  uint16_t *kt = reinterpret_cast<uint16_t *>(smem_raw + L::BT_BYTES + w * L::WAVE_LDS);
  uint16_t *vt = kt + L::TILE_ELEMS;

  MCtx c;
  c.kbase = a.k + g * a.head_stride;
  c.vbase = a.v + g * a.head_stride;
  c.bt = bt_lds;
  c.page_shift = a.page_shift;
  c.pmask = (1 << a.page_shift) - 1;
  c.page_stride = a.page_stride;
  c.row_stride = a.row_stride;
  c.R = sr.R;
  c.kvis = wave_min_limit<NRB>(lim, r0, sr.R, lane);
  const int kb = s * a.chunk;
  int kend = kb + a.chunk;
  if (kend > kmax) kend = kmax;

  // q operand: lane supplies Q[row cc+16rb][d 32*stp + 8q .. +8]
  uint4 qb[NRB][D / 32];
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    const int rr = r0 + cc + 16 * rb;
    if (rr < sr.R) {
      const uint4 *src = reinterpret_cast<const uint4 *>(a.q + out_row(a, sr.tok0, g, rr) * D);
#pragma unroll
      for (int stp = 0; stp < D / 32; ++stp) qb[rb][stp] = src[4 * stp + q];
    } else {
#pragma unroll
      for (int stp = 0; stp < D / 32; ++stp) qb[rb][stp] = make_uint4(0u, 0u, 0u, 0u);
    }
  }

  const int *bt_row = a.block_table + (int64_t)b * a.max_pages;
  const int win_keys = window_keys(kBtCap, a.page_shift, NW * KT);
  const int cap_keys = a.max_pages << a.page_shift;
  auto load_bt = [&](int from) {
    if (a.contig) {  // contiguous K/V: sequence b is page b
      if (threadIdx.x == 0) bt_lds[0] = b;
      return;
    }
    int to = from + win_keys;
    if (to > kb + a.chunk) to = kb + a.chunk;
    if (to > cap_keys) to = cap_keys;
    const int p0 = from >> a.page_shift;
    const int np = to > from ? ((to - 1) >> a.page_shift) - p0 + 1 : 0;
    for (int i = threadIdx.x; i < np; i += NW * 64) bt_lds[i] = bt_row[p0 + i];
  };

  MState<D, NRB> st;
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    st.m[rb] = -INFINITY;
    st.l[rb] = 0.f;
#pragma unroll
    for (int nb = 0; nb < D / 16; ++nb) st.o[rb][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  if ((int)threadIdx.x < RW * a.hpb) {
    const int rr = r0 + (threadIdx.x >> a.lhpb);
    rowtab[threadIdx.x] = rr < sr.R ? out_row(a, sr.tok0, hg * a.hpb + (threadIdx.x & (a.hpb - 1)), rr) : 0;
  }
  load_bt(kb);
  __syncthreads();
  for (int wb = kb; wb < kend; wb += win_keys) {
    const int we = wb + win_keys < kend ? wb + win_keys : kend;
    if (wb != kb) {
      __syncthreads();
      load_bt(wb);
      __syncthreads();
    }
    c.p0 = wb >> a.page_shift;
    c.ke = we;
    const int ntiles = (we - wb + KT - 1) / KT;
    mtile_loop<D, NRB, CAUSAL, MASK, UPAGE>(a, c, b, r0, wb, wk, wph, ntiles, qb, lim, kt, vt, lane, st);
  }

  // row sums over the four lanes of each row
  float ltot[NRB];
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) ltot[rb] = xor32<OpSum>(xor16<OpSum>(st.l[rb]));

  // merge the waves of each head, one 16-row block at a time.  Row slot
  // u = wk * HR + cc * hpb + hw: the block-local row index ri = cc * hpb + hw
  // (matching rowtab), once per wave of a head.
  const int HR = 16 * a.hpb;
  float *ob = reinterpret_cast<float *>(smem_raw);        // [NW * 16][OB_STRIDE]
  float *mlb = ob + NW * 16 * L::OB_STRIDE;               // [NW * 16][2]
  const int u = wk * HR + cc * a.hpb + hw;
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    __syncthreads();
#pragma unroll
    for (int nb = 0; nb < D / 16; ++nb) {
      // lane holds O^T[d = 16nb + 4q + i][row cc]
      float4 *dst = reinterpret_cast<float4 *>(ob + u * L::OB_STRIDE + 16 * nb + 4 * q);
      dst[0] = make_float4(st.o[rb][nb][0], st.o[rb][nb][1], st.o[rb][nb][2], st.o[rb][nb][3]);
    }
    if (q == 0) *reinterpret_cast<float2 *>(mlb + u * 2) = make_float2(st.m[rb], ltot[rb]);
    const int rs = r0 + 16 * rb;
    const int nrows = (sr.R - rs < 16 ? sr.R - rs : 16) * a.hpb;
    __syncthreads();
    auto item = [&](int ri, int d, float &M, float &W, float &vx, float &vy) {
      merge_waves<NW, L::OB_STRIDE>(mlb, ob, HR, wph, ri, d, M, W, vx, vy);
    };
    write_rows<D>(a, s, direct, rowtab + 16 * rb * a.hpb, nrows, item, NW * 64);
  }
  if (a.fused && !direct)
    fused_tail<D>(a, wk0.unit, nact, rowtab, nrt, reinterpret_cast<float *>(smem_raw), NW * 64);
}

// ---- prefill-shaped workgroup ----------------------------------------------
// Four waves of 32 rows each (128 packed rows of one kv head) over the same
// keys.  A shared tile of 64 keys is four 16-key subtiles, wave w fetching
// subtile w (the same loads and swizzled LDS layout as above); every wave
// then computes all four subtiles for its own rows.  Shared tiles are
// double-buffered in LDS with one barrier per tile: the next tile's loads
// fly while this one computes, and go to LDS after it.  A wave's rows are
// its own, so it writes them (or its split's partials) from registers with
// no merge between waves.  With a mask, each wave stages its rows' mask
// values of the next tile in its own LDS slice after computing the current
// one (single-buffered: only that wave reads it).
template <int D, bool MASK>
struct PLay {
  static constexpr int NW = kWavesPerBlock;
  static constexpr int SUB = NW;                      // 16-key subtiles per shared tile
  static constexpr int KTC = SUB * KT;                // keys per shared tile
  static constexpr int SUB_ELEMS = KT * D;            // bf16 per K (or V) subtile
  static constexpr int BUF_BYTES = 2 * SUB * SUB_ELEMS * 2;
  static constexpr int MASK_SUB = 2 * 64 * 4;         // floats per subtile: [row block][lane] float4
  static constexpr int MASK_WAVE = MASK ? SUB * MASK_SUB * 4 : 0;
  static constexpr int BT_BYTES = (kBtCap + 4) * 4;
  static constexpr int SMEM_BYTES = BT_BYTES + 2 * BUF_BYTES + NW * MASK_WAVE;
};

// Mask values of a wave's rows for the four subtiles of the shared tile at
// key tb: lane (cc, q) takes keys tb + 16 sub + 4q + i of rows rw + cc + 16 rb
// (keys and rows clamped into range; one load per entry on every path).
template <int NRB>
__device__ __forceinline__ void pmask_load(const DecodeArgs &a, const MCtx &c, int b, int rw, int tb, int lane,
                                           float (&pm)[kWavesPerBlock][NRB][4]) {
  const int q = lane >> 4;
  const int cc = lane & 15;
  const int jlast = c.ke - 1;
#pragma unroll
  for (int sub = 0; sub < kWavesPerBlock; ++sub) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int j = tb + KT * sub + 4 * q + i;
      j = j < jlast ? j : jlast;
      const float *mrow = a.mask + (int64_t)b * a.mask_sb + j;
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
        const int rr = rw + cc + 16 * rb < c.R ? rw + cc + 16 * rb : c.R - 1;
        pm[sub][rb][i] = mrow[(int64_t)(rr / a.G) * a.mask_sq];
      }
    }
  }
}

template <int NRB>
__device__ __forceinline__ void pmask_store(const float (&pm)[kWavesPerBlock][NRB][4], float *mw, int lane) {
#pragma unroll
  for (int sub = 0; sub < kWavesPerBlock; ++sub)
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb)
      reinterpret_cast<float4 *>(mw + sub * 2 * 64 * 4)[rb * 64 + lane] =
          make_float4(pm[sub][rb][0], pm[sub][rb][1], pm[sub][rb][2], pm[sub][rb][3]);
  __builtin_amdgcn_wave_barrier();
}

template <int D, bool CAUSAL, bool MASK, bool UPAGE>
__global__ __launch_bounds__(kWavesPerBlock * 64, (MASK && D == 128) ? 1 : 2) void split_prefill_mfma(
    const DecodeArgs a) {
  using P = PLay<D, MASK>;
  constexpr int NW = P::NW;
  constexpr int NRB = 2;                 // 32 rows per wave
  constexpr int RWG = NW * 16 * NRB;     // rows per workgroup
  __shared__ __attribute__((aligned(16))) unsigned char smem_raw[P::SMEM_BYTES];
  __shared__ int64_t rowtab[RWG];

  Work wk0;
  if (!work_of<CAUSAL>(a, wk0)) return;
  const int b = wk0.b, s = wk0.s, g = wk0.hg, rg = wk0.rg;  // one kv head per workgroup: group = head
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int cc = lane & 15;
  const int q = lane >> 4;
  const int kvlen = wk0.L;
  const SeqRows sr = wk0.sr;
  const int r0 = rg * RWG;
  if (r0 >= sr.R) return;  // a row block past the sequence's tokens (varlen batches)
  const int rw = r0 + 32 * w;  // this wave's first row
  int lim[NRB];
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) lim[rb] = row_keys(a, sr, kvlen, rw + cc + 16 * rb);
  const int rlast = (r0 + RWG < sr.R ? r0 + RWG : sr.R) - 1;
  const int kmax = row_keys(a, sr, kvlen, rlast);
  const int wlast = (rw + 32 < sr.R ? rw + 32 : sr.R) - 1;
  const int wkmax = wlast >= rw ? row_keys(a, sr, kvlen, wlast) : 0;  // keys this wave's rows see

  const int nact = active_splits(a, kmax);
  const int nrt = sr.R - r0 < RWG ? sr.R - r0 : RWG;
  if (s >= nact) {
    if (!a.fused) empty_partials(a, sr.tok0, g, r0, s, nrt);
    return;
  }
  const bool direct = !a.partials || (a.fused && nact == 1);

  int *bt_lds = reinterpret_cast<int *>(smem_raw);
  unsigned char *bufs = smem_raw + P::BT_BYTES;
  auto ktile = [&](int buf, int sub) {
    return reinterpret_cast<uint16_t *>(bufs + buf * P::BUF_BYTES) + sub * P::SUB_ELEMS;
  };
  auto vtile = [&](int buf, int sub) {
    return reinterpret_cast<uint16_t *>(bufs + buf * P::BUF_BYTES) + (P::SUB + sub) * P::SUB_ELEMS;
  };
  float *mw = reinterpret_cast<float *>(bufs + 2 * P::BUF_BYTES + w * P::MASK_WAVE);

  MCtx c;
  c.kbase = a.k + g * a.head_stride;
  c.vbase = a.v + g * a.head_stride;
  c.bt = bt_lds;
  c.page_shift = a.page_shift;
  c.pmask = (1 << a.page_shift) - 1;
  c.page_stride = a.page_stride;
  c.row_stride = a.row_stride;
  c.R = sr.R;
  c.kvis = wave_min_limit<NRB>(lim, rw, sr.R, lane);
  const int kb = s * a.chunk;
  int kend = kb + a.chunk;
  if (kend > kmax) kend = kmax;

  uint4 qb[NRB][D / 32];
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    const int rr = rw + cc + 16 * rb;
    if (rr < sr.R) {
      const uint4 *src = reinterpret_cast<const uint4 *>(a.q + out_row(a, sr.tok0, g, rr) * D);
#pragma unroll
      for (int stp = 0; stp < D / 32; ++stp) qb[rb][stp] = src[4 * stp + q];
    } else {
#pragma unroll
      for (int stp = 0; stp < D / 32; ++stp) qb[rb][stp] = make_uint4(0u, 0u, 0u, 0u);
    }
  }

  const int *bt_row = a.block_table + (int64_t)b * a.max_pages;
  const int win_keys = window_keys(kBtCap, a.page_shift, P::KTC);
  const int cap_keys = a.max_pages << a.page_shift;
  auto load_bt = [&](int from) {
    if (a.contig) {  // contiguous K/V: sequence b is page b
      if (threadIdx.x == 0) bt_lds[0] = b;
      return;
    }
    int to = from + win_keys;
    if (to > kb + a.chunk) to = kb + a.chunk;
    if (to > cap_keys) to = cap_keys;
    const int p0 = from >> a.page_shift;
    const int np = to > from ? ((to - 1) >> a.page_shift) - p0 + 1 : 0;
    for (int i = threadIdx.x; i < np; i += NW * 64) bt_lds[i] = bt_row[p0 + i];
  };

  MState<D, NRB> st;
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    st.m[rb] = -INFINITY;
    st.l[rb] = 0.f;
#pragma unroll
    for (int nb = 0; nb < D / 16; ++nb) st.o[rb][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  if (threadIdx.x < RWG) {
    const int rr = r0 + threadIdx.x;
    rowtab[threadIdx.x] = rr < sr.R ? out_row(a, sr.tok0, g, rr) : 0;
  }
  load_bt(kb);
  __syncthreads();
  for (int wb = kb; wb < kend; wb += win_keys) {
    const int we = wb + win_keys < kend ? wb + win_keys : kend;
    if (wb != kb) {
      __syncthreads();
      load_bt(wb);
      __syncthreads();
    }
    c.p0 = wb >> a.page_shift;
    c.ke = we;
    const int ntiles = (we - wb + P::KTC - 1) / P::KTC;
    MTile<D, NRB, false> tr;
    float pm[MASK ? NW : 1][NRB][4];
    mload<D, NRB, false, UPAGE, true>(a, c, b, rw, wb + KT * w, lane, tr);
    if constexpr (MASK) pmask_load<NRB>(a, c, b, rw, wb, lane, pm);
    mstore<D, NRB, false>(tr, ktile(0, w), vtile(0, w), nullptr, lane);
    if constexpr (MASK) pmask_store<NRB>(pm, mw, lane);
    __syncthreads();
    for (int t = 0; t < ntiles; ++t) {
      const int buf = t & 1;
      const int tb = wb + t * P::KTC;
      // the next shared tile (unconditional: past the window end, mload and
      // pmask_load clamp to its last key)
      mload<D, NRB, false, UPAGE, true>(a, c, b, rw, tb + P::KTC + KT * w, lane, tr);
      if constexpr (MASK) pmask_load<NRB>(a, c, b, rw, tb + P::KTC, lane, pm);
#pragma unroll
      for (int sub = 0; sub < P::SUB; sub += 2) {
        const int base = tb + KT * sub;
        if (base < wkmax)  // wave-uniform: some row of this wave sees a key of the subtile pair
          mcompute2<D, NRB, CAUSAL, MASK>(a, c, base, mw + sub * P::MASK_SUB, mw + (sub + 1) * P::MASK_SUB, qb, lim,
                                          ktile(buf, sub), vtile(buf, sub), ktile(buf, sub + 1),
                                          vtile(buf, sub + 1), lane, st);
      }
      mstore<D, NRB, false>(tr, ktile(buf ^ 1, w), vtile(buf ^ 1, w), nullptr, lane);
      if constexpr (MASK) pmask_store<NRB>(pm, mw, lane);
      __syncthreads();
    }
  }

  // each wave writes its own rows: lane (cc, q) holds O^T[16nb + 4q + i][row cc]
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    const float W = xor32<OpSum>(xor16<OpSum>(st.l[rb]));
    const int rr = rw + 16 * rb + cc;
    if (rr < sr.R) {
      const int64_t row = out_row(a, sr.tok0, g, rr);
      const float inv = W > 0.f ? 1.f / W : 0.f;
#pragma unroll
      for (int nb = 0; nb < D / 16; ++nb) {
        const int d0 = 16 * nb + 4 * q;
        const f32x4_t v = st.o[rb][nb] * inv;
        if (direct) {
          const uint32_t lo = (uint32_t)f32_to_bf16_rne(v[0]) | ((uint32_t)f32_to_bf16_rne(v[1]) << 16);
          const uint32_t hi = (uint32_t)f32_to_bf16_rne(v[2]) | ((uint32_t)f32_to_bf16_rne(v[3]) << 16);
          *reinterpret_cast<uint2 *>(a.out + row * D + d0) = make_uint2(lo, hi);
          if (a.out_f32) *reinterpret_cast<float4 *>(a.out_f32 + row * D + d0) = make_float4(v[0], v[1], v[2], v[3]);
        } else if (W > 0.f) {
          float *po = a.o_part + (row * a.S + s) * D + d0;
          if (a.fused) {  // merged by another workgroup of this launch
            store_dev2(po, v[0], v[1]);
            store_dev2(po + 2, v[2], v[3]);
          } else {
            *reinterpret_cast<float4 *>(po) = make_float4(v[0], v[1], v[2], v[3]);
          }
        }
      }
      if (!direct && q == 0) {
        float *pm2 = a.ml_part + (row * a.S + s) * 2;
        const float mx = W > 0.f ? st.m[rb] * kLn2 : -INFINITY;
        if (a.fused)
          store_dev2(pm2, mx, W);
        else
          *reinterpret_cast<float2 *>(pm2) = make_float2(mx, W);
      }
    }
  }
  if (a.fused && !direct)
    fused_tail<D>(a, wk0.unit, nact, rowtab, nrt, reinterpret_cast<float *>(smem_raw), NW * 64);
}

template <int D, bool C, bool M, bool U>
hipError_t plaunch_t(const DecodeArgs &a, hipStream_t stream) {
  hipLaunchKernelGGL((split_prefill_mfma<D, C, M, U>), dim3((unsigned)split_grid(a)), dim3(kWavesPerBlock * 64), 0,
                     stream, a);
  return hipGetLastError();
}

template <int D, bool C, bool M>
hipError_t plaunch_u(const DecodeArgs &a, hipStream_t s) {
  return a.page_shift >= 4 ? plaunch_t<D, C, M, true>(a, s) : plaunch_t<D, C, M, false>(a, s);
}

template <int D>
hipError_t plaunch_d(const DecodeArgs &a, bool causal, bool mask, hipStream_t s) {
  if (causal) return mask ? plaunch_u<D, true, true>(a, s) : plaunch_u<D, true, false>(a, s);
  return mask ? plaunch_u<D, false, true>(a, s) : plaunch_u<D, false, false>(a, s);
}

template <int D, int NRB, bool C, bool M, bool U>
hipError_t mlaunch_t(const DecodeArgs &a, hipStream_t stream) {
  const int64_t grid = split_grid(a);
  hipLaunchKernelGGL((split_decode_mfma<D, NRB, C, M, U>), dim3((unsigned)grid), dim3(kWavesPerBlock * 64), 0,
                     stream, a);
  return hipGetLastError();
}

template <int D, int NRB, bool C, bool M>
hipError_t mlaunch_u(const DecodeArgs &a, hipStream_t s) {
  // a 16-key tile's page is wave-uniform when pages hold at least 16 keys
  return a.page_shift >= 4 ? mlaunch_t<D, NRB, C, M, true>(a, s) : mlaunch_t<D, NRB, C, M, false>(a, s);
}

template <int D, int NRB>
hipError_t mlaunch_nrb(const DecodeArgs &a, bool causal, bool mask, hipStream_t s) {
  if (causal) return mask ? mlaunch_u<D, NRB, true, true>(a, s) : mlaunch_u<D, NRB, true, false>(a, s);
  return mask ? mlaunch_u<D, NRB, false, true>(a, s) : mlaunch_u<D, NRB, false, false>(a, s);
}

template <int D>
hipError_t mlaunch_d(const DecodeArgs &a, int nrb16, bool causal, bool mask, hipStream_t s) {
  return nrb16 == 1 ? mlaunch_nrb<D, 1>(a, causal, mask, s) : mlaunch_nrb<D, 2>(a, causal, mask, s);
}

}  // namespace

int launch_split_prefill(const DecodeArgs &a, int head_dim, bool causal, bool has_mask, hipStream_t stream) {
  switch (head_dim) {
    case 32: return plaunch_d<32>(a, causal, has_mask, stream);
    case 64: return plaunch_d<64>(a, causal, has_mask, stream);
    default: return plaunch_d<128>(a, causal, has_mask, stream);
  }
}

int launch_split_mfma(const DecodeArgs &a, int head_dim, int nrb16, bool causal, bool has_mask,
                      hipStream_t stream) {
  switch (head_dim) {
    case 32: return mlaunch_d<32>(a, nrb16, causal, has_mask, stream);
    case 64: return mlaunch_d<64>(a, nrb16, causal, has_mask, stream);
    case 128: return mlaunch_d<128>(a, nrb16, causal, has_mask, stream);
    default: return mlaunch_d<256>(a, nrb16, causal, has_mask, stream);
  }
}

}  // namespace pkv
