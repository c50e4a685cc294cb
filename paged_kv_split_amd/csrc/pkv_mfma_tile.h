// pkv_mfma_tile.h -- matrix-core building blocks of the split kernels for
// CDNA4 (gfx950): 16-key K/V tile loads, the swizzled LDS tile layout, and
// one tile's scores, online softmax and PV product on the matrix cores (not
// part of the public ABI).
//
//  * S^T = K Q^T with v_mfma_f32_16x16x32_bf16: the K operand is a
//    ds_read_b128 per lane, Q stays in registers; the S^T accumulator leaves
//    each lane one query row and four keys, so the online-softmax max, exp
//    and rescale are in-lane apart from two permlane swaps;
//  * O^T = V^T P^T with v_mfma_f32_16x16x16_bf16 (or 16x16x32 over a pair of
//    tiles): V^T comes straight from the row-major V tile through
//    ds_read_b64_tr_b16 (the gfx950 transposing LDS read), P^T is the S^T
//    register layout itself; P is split into a bf16 high part and a bf16
//    remainder (two MFMAs, both converted with the gfx950 v_cvt_pk_bf16_f32)
//    so the probabilities keep about 16 significant bits, and the row sums l
//    use the fp32 values;
//  * exclusion (tail, causal, -inf mask) is a select; scores are in base 2.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {
namespace mt {

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
  // merge phase, per 16-row block: per-wave O rows and (m, l)
  static constexpr int MERGE_BYTES = NW * 16 * OB_STRIDE * 4 + NW * 16 * 2 * 4;
  static constexpr int MAIN_BYTES = BT_BYTES + NW * WAVE_LDS;
  // swizzles (16-byte chunk index within a row).  K: row r's chunks XOR
  // r mod NCH (at D = 32: (r >> 1) mod NCH), so that the eight lanes of one LDS pass of a
  // key-major read (rows 8i .. 8i + 7, one chunk each) hit distinct banks
  // (at D = 32 four chunks per row make a plain XOR with r repeat every four
  // rows, which 128-byte passes cover twice).  V: the
  // transposing read gives each lane 8 bytes of one row; four lanes cover one
  // 32-byte segment of a row, and one pass serves 8 rows.  Segment s of row r
  // moves to s XOR ((r >> SSH) mod NSEG), SSH chosen so that those 8 rows
  // land on 8 distinct 32-byte bank groups (the pass covers 256 bytes of
  // banks): measured on MI355X at D = 64, an XOR with r mod 4 left rows r and
  // r + 4 on the same banks (12% of LDS cycles in bank conflicts).
  static constexpr int NSEG = NCH / 2;  // 32-byte segments per row
  static constexpr int SSH = NSEG >= 8 ? 0 : (NSEG == 4 ? 1 : 2);
  // (written as before the D <= 64 forms were added where those reduce to the
  // plain XOR: at D = 256 the kernels sit at the register limit, and
  // equivalent but differently written indices spilled twice as much)
  __device__ static int swk(int ch, int row) {
    return NCH >= 8 ? ch ^ (row & (NCH - 1)) : ch ^ ((row >> 1) & (NCH - 1));
  }
  __device__ static int swv(int ch, int row) {
    return NSEG >= 8 ? ch ^ ((2 * row) & (NCH - 2)) : ch ^ (2 * ((row >> SSH) & (NSEG - 1)));
  }
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
// Wave priority around the matrix-core sections (PRIO, the prefill-shaped
// kernel): a wave raises its issue priority while it issues its products and
// drops it for the softmax, so of two waves sharing a SIMD that reach their
// products together one goes first and moves on to its vector work while the
// other's products run, instead of both alternating through the products
// and then both through the softmax.  Measured on MI355X (4 x 512-token
// prefill chunks over 4096 keys, D = 128): 205.1 -> 198.5 us; priority on the
// score products alone 204.6, on the PV products alone 203.5, on the softmax
// instead 206.8; the mixed varlen batch unchanged (84.5 us).
__device__ __forceinline__ void set_issue_prio(bool high) {
  __builtin_amdgcn_sched_barrier(0);
  if (high)
    __builtin_amdgcn_s_setprio(1);
  else
    __builtin_amdgcn_s_setprio(0);
  __builtin_amdgcn_sched_barrier(0);
}

template <int D, int NRB, bool CAUSAL, bool MASK, bool PRIO = false>
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
  if constexpr (PRIO) set_issue_prio(true);
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

  if constexpr (PRIO) set_issue_prio(false);
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

  if constexpr (PRIO) set_issue_prio(true);
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
  if constexpr (PRIO) set_issue_prio(false);
  __builtin_amdgcn_wave_barrier();
}


}  // namespace mt
}  // namespace pkv
