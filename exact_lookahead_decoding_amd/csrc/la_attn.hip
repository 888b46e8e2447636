// Lookahead-mask attention over the committed prefix and the packed rows.
//
// "M7.3 - Lookahead Decoding", 0x04A / 0x04B / 0x07A: every packed row sees
// the whole committed prefix plus the rows of its own branch; an ordinary
// causal kernel cannot express this, and a dense additive mask costs
// B*H*Q*(K_in+Q) elements.  Here the mask never exists as a tensor: row i
// sees exactly logical positions 0 .. pos_i, position t taken from the
// cache when t < shared_end and through the row's branch path otherwise.
//
// Reduction tree (a function of key positions, the cache capacity and the
// model's head counts only, so a row gets the same bits whether it is alone
// in an autoregressive step or packed with a whole lookahead round):
//   * keys are cut into chunks of 32 positions and the chunks into key
//     splits of `spl` chunks (la_attention_spl);
//   * inside a split the chunks are taken in decreasing position with the
//     online softmax: the reference maximum m' moves to the chunk's exact
//     maximum only when fma(max, scale, -m) exceeds RESCALE (a row that has
//     seen nothing keeps the finite M_NONE), p = 2^(s - m'), each of a row's
//     four lanes keeps its own running sum l' = l * 2^(m - m') + its p in a
//     fixed order (the row's sum is the four lanes' sum at the end), and
//     O' = O * 2^(m - m') + V^T P^T accumulated by MFMA over a fixed key ->
//     slot assignment;
//   * the splits' states are folded in split order by a small merge
//     kernel, then O / l.
// A chunk's scores are the same numbers whichever rows share the MFMA, and
// a row's probabilities and products sit in the same MFMA slots whether the
// chunk's keys came from the cache or from the row's branch (other
// branches add exact zeros).
//
// Work decomposition (gfx950, wave64):
//   * one workgroup per (KV head, key split, row group); a row group is
//     eight waves x one tile of 16 query rows (two waves per SIMD, so one
//     wave's vector ALU work overlaps the other's MFMAs and LDS waits).
//     Tiles are row-tile major over the query heads of a KV head
//     (grouped-query attention), every wave holds its tile's Q in registers
//     and walks every chunk of the split, so each K/V byte of the split
//     reaches the workgroup once;
//   * K and V of committed chunks arrive through a ring of D chunk slots in
//     LDS by global_load_lds DMA (16-byte pieces XOR-swizzled by row), one
//     barrier per chunk.  The DMA is issued as inline asm and the LDS reads
//     are ordinary loads, so the compiler places only LDS waits on them and
//     the ring orders the DMA with explicit vmcnt waits.  Software
//     pipelined: the QK^T MFMAs of chunk i + 1 are issued beside chunk i's
//     softmax (one set of K and one of V fragment registers);
//   * QK: S^T = K Q^T with 16x16x32 bf16 MFMA (one query row per lane
//     column, softmax statistics stay in-lane); PV: O^T += V^T P^T, the V^T
//     operand read straight from the row-major chunk with ds_read_b64_tr_b16
//     (the 64 halves a 16-lane group names are dealt out so that lane i
//     receives items i, i+16, i+32, i+48);
//   * chunks reaching past shared_end (at most three) are the highest
//     positions of their split, so they come first: the committed rows of
//     the first of them and every packed row's K/V are staged in LDS once,
//     and each wave walks the distinct branches of its tiles (the row
//     builder's tables), indexing the staged rows through the branch path;
//   * the block -> work map keeps every workgroup of one KV head on one XCD
//     (blockIdx % 8), so the head's K/V shared by its row groups and its
//     split states are fetched from that XCD's L2.
#include <algorithm>
#include <type_traits>

#include "la_common.h"
#include "la_dev.h"
#include "la_kernels.h"

#define CH 32          // keys per chunk
#define NEG_INF (-__builtin_inff())
#define RESCALE 8.0f   // log2 units: the reference maximum moves only past this
#define M_NONE (-1e30f) // reference maximum of a row that has seen no key (finite: 2^(s - M_NONE) never overflows to NaN)

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

// a*wa + b*wb as fma(a, wa, b*wb): the one rounding sequence of the split fold
__device__ __forceinline__ float lin2(float a, float wa, float b, float wb) {
#pragma clang fp contract(off)
  return __builtin_fmaf(a, wa, b * wb);
}

// MFMA k-slot e (0..7) of lane group g <-> key offset inside the chunk.
__device__ __forceinline__ int slot_key(int g, int e) { return 16 * (e >> 2) + 4 * g + (e & 3); }

template <int W> struct alignas(4 * W) Words { uint32_t w[W]; };

// The 16-byte pieces of an LDS chunk row r are XOR-swizzled: position p
// holds piece p ^ piece_swz(r).  With 16 pieces (256-byte rows, which span
// the 64 banks once) the swizzle is a bijection of r mod 16 chosen for both
// fragment reads: a K read (16 B a lane, 16 rows at one piece) sees 16
// distinct positions, and a transposed V read (8 B a lane, a lane's row pair
// of pieces 2i, 2i + 1) gives the rows a lane group reads together distinct
// piece pairs -- rows 0-7 (and 8-15) as well as rows 0-3 with 8-11 (and 4-7
// with 12-15): a row's partner on its piece pair is row r ^ 12.
template <int PIECES> __device__ __forceinline__ int piece_swz(int r) {
  if constexpr (PIECES == 16) {
    const int x = r & 15, h = x >> 2;
    return ((x & 3) << 1) | (((h ^ (h >> 1)) & 1) << 3) | (x >> 3);
  } else {
    return r % PIECES;
  }
}
// LDS address of 16-byte piece q of chunk row r
template <int ROWB> __device__ __forceinline__ uint32_t piece_addr(uint32_t base, int r, int q) {
  constexpr int PIECES = ROWB / 16;
  return base + (uint32_t)(r * ROWB + 16 * (q ^ piece_swz<PIECES>(r)));
}

// LDS reads are ordinary loads (the compiler places their lgkmcnt waits);
// the DMA into LDS is inline asm, so the compiler sees no pending LDS write
// and never waits for DMA before an LDS read -- the ring orders the DMA with
// its own vmcnt waits and barriers.  The DMA has no register results.
template <typename V> __device__ __forceinline__ V lds_get(uint32_t addr) {
  return *(const __attribute__((address_space(3))) V*)addr;
}
typedef short i16x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ LdsT<8>::T lds_get_tr16(uint32_t addr) {
  const i16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4_t*)addr);
  return __builtin_bit_cast(LdsT<8>::T, v);
}
// lane l's 16 (4) bytes of src land at LDS offset lds_off + 16 l (4 l); m0 is restored
__device__ __forceinline__ void dma16(const void* src, uint32_t lds_off) {
  uint32_t keep;
  lds_off = __builtin_amdgcn_readfirstlane(lds_off);   // wave-uniform by construction; an SGPR for m0
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off\n\ts_mov_b32 m0, %0"
               : "=&s"(keep) : "v"(src), "s"(lds_off) : "memory");
}
__device__ __forceinline__ void dma4(const void* src, uint32_t lds_off) {
  uint32_t keep;
  lds_off = __builtin_amdgcn_readfirstlane(lds_off);
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %1, off\n\ts_mov_b32 m0, %0"
               : "=&s"(keep) : "v"(src), "s"(lds_off) : "memory");
}
// uniform base + per-lane offset as one VALU add the compiler keeps as is
// (left alone, it hoists every base-independent offset into its own register)
__device__ __forceinline__ uint32_t add_sv(uint32_t sbase, uint32_t voff) {
  uint32_t a;
  sbase = __builtin_amdgcn_readfirstlane(sbase);
  asm("v_add_u32 %0, %1, %2" : "=v"(a) : "s"(sbase), "v"(voff));
  return a;
}
// s_waitcnt vmcnt(N) for the asm DMA (an asm statement the compiler keeps as written)
template <int N> __device__ __forceinline__ void dma_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

template <typename T, int DH> struct AttnT;

// bf16: 16x16x32 MFMA; lane (g, c) = (lane / 16, lane % 16).
typedef LdsT<16>::T V4u;

template <int DH> struct AttnT<bf16_t, DH> {
  static constexpr int ROWB = DH * 2, KS = DH / 32, NDT = DH / 16;
  static constexpr int QKN = KS;                      // QK^T MFMAs per 16 keys
  struct QF { V4u p[KS]; };                           // Q[row c][32 s + 8 g ..]
  struct KF { V4u p[2][KS]; };                        // K[key 16 kg + .][32 s + 8 g ..]
  struct VF { LdsT<8>::T p[NDT][2]; };                // V^T operand halves (transposed reads)
  static constexpr int NVR = 2;                      // V rows a lane reads per chunk
  // Q fragments of lane (g, c) from its row
  static __device__ __forceinline__ void load_q(QF& q, const char* row, int g) {
#pragma unroll
    for (int s = 0; s < KS; ++s) q.p[s] = *(const V4u*)(row + 16 * (4 * s + g));
  }
  // chunk key offset of V row j of lane (g, c)
  static __device__ __forceinline__ int vkey(int g, int c, int j) { return 16 * j + 4 * g + (c >> 2); }
  // K fragments of lane (g, c): key rows rk[kg] of the chunk at base
  static __device__ __forceinline__ void load_k(KF& k, uint32_t base, const int (&rk)[2], int g) {
#pragma unroll
    for (int kg = 0; kg < 2; ++kg)
#pragma unroll
      for (int s = 0; s < KS; ++s) k.p[kg][s] = lds_get<V4u>(piece_addr<ROWB>(base, rk[kg], 4 * s + g));
  }
  // V^T operand of tile dt: lane (g, c) names row rv[h] (slot keys 4g + c/4 and 16 + 4g + c/4) and dims
  // 16 dt + 4 (c % 4) .. +3; after the transposed read it holds dim 16 dt + c of slot keys slot_key(g, e)
  static __device__ __forceinline__ void load_v(VF& v, uint32_t base, const int (&rv)[2], int c) {
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t a = piece_addr<ROWB>(base, rv[h], 2 * dt + ((c & 3) >> 1)) + 8 * (c & 1);
        v.p[dt][h] = lds_get_tr16(a);
      }
  }
  static __device__ __forceinline__ void load_vr(VF& v, uint32_t base, const int (&rv)[NVR], int c) {
    load_v(v, base, rv, c);
  }
  // the lower 16 keys only: K of key group 0, V of keys 0-15 (the upper half's V reads as zeros)
  static __device__ __forceinline__ void load_k_lo(KF& k, uint32_t base, const int (&rk)[2], int g) {
#pragma unroll
    for (int s = 0; s < KS; ++s) k.p[0][s] = lds_get<V4u>(piece_addr<ROWB>(base, rk[0], 4 * s + g));
  }
  static __device__ __forceinline__ void load_vr_lo(VF& v, uint32_t base, const int (&rv)[NVR], int c) {
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      v.p[dt][0] = lds_get_tr16(piece_addr<ROWB>(base, rv[0], 2 * dt + ((c & 3) >> 1)) + 8 * (c & 1));
      v.p[dt][1] = LdsT<8>::T{0, 0};
    }
  }
  // A chunk slot's fragments at fixed per-lane offsets (the second 16-row
  // half of a chunk adds 16 rows, an immediate offset of the LDS read)
  struct Lofs { uint32_t k[KS], v[NDT]; };
  static __device__ __forceinline__ Lofs lane_ofs(int g, int c) {
    constexpr int P = ROWB / 16;
    Lofs o;
#pragma unroll
    for (int s = 0; s < KS; ++s) o.k[s] = c * ROWB + 16 * ((4 * s + g) ^ piece_swz<P>(c));
    const int r = 4 * g + (c >> 2);
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
      o.v[dt] = r * ROWB + 16 * ((2 * dt + ((c & 3) >> 1)) ^ piece_swz<P>(r)) + 8 * (c & 1);
    return o;
  }
  static __device__ __forceinline__ void load_k_at(KF& k, uint32_t base, const Lofs& o, int, int) {
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const uint32_t a = add_sv(base, o.k[s]);
#pragma unroll
      for (int kg = 0; kg < 2; ++kg) k.p[kg][s] = lds_get<V4u>(a + kg * 16 * ROWB);
    }
  }
  static __device__ __forceinline__ void load_v_at(VF& v, uint32_t base, const Lofs& o, int, int) {
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const uint32_t a = add_sv(base, o.v[dt]);
#pragma unroll
      for (int h = 0; h < 2; ++h) v.p[dt][h] = lds_get_tr16(a + h * 16 * ROWB);
    }
  }
  static __device__ __forceinline__ f32x4 qk(const KF& k, int kg, const QF& q) {
    f32x4 acc = {0, 0, 0, 0};
#pragma unroll
    for (int s = 0; s < KS; ++s)
      acc = mfma_bf16_32(__builtin_bit_cast(bf16x8, k.p[kg][s]), __builtin_bit_cast(bf16x8, q.p[s]), acc);
    return acc;
  }
  // both 16-key halves, their accumulation chains interleaved (each in the order of qk)
  static __device__ __forceinline__ void qk2(const KF& k, const QF& q, f32x4& a0, f32x4& a1) {
    a0 = f32x4{0, 0, 0, 0};
    a1 = f32x4{0, 0, 0, 0};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      a0 = mfma_bf16_32(__builtin_bit_cast(bf16x8, k.p[0][s]), __builtin_bit_cast(bf16x8, q.p[s]), a0);
      a1 = mfma_bf16_32(__builtin_bit_cast(bf16x8, k.p[1][s]), __builtin_bit_cast(bf16x8, q.p[s]), a1);
    }
  }
  typedef bf16x8 PP;
  // P^T operand: p of slot e rounded to bf16 (nearest even)
  static __device__ __forceinline__ PP prep(const float* ps) {
    typedef float f2 __attribute__((ext_vector_type(2)));
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    uint32_t bh[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f2 v = {ps[2 * j], ps[2 * j + 1]};
      bh[j] = __builtin_bit_cast(uint32_t, __builtin_convertvector(v, b2));
    }
    return __builtin_bit_cast(bf16x8, bh);
  }
  static __device__ __forceinline__ f32x4 pv(const VF& v, int dt, const PP& pp, f32x4 o) {
    const uint32_t w[4] = {v.p[dt][0].x, v.p[dt][0].y, v.p[dt][1].x, v.p[dt][1].y};
    return mfma_bf16_32(__builtin_bit_cast(bf16x8, w), pp, o);
  }
  // head dimension of accumulator row i (0..15) of output tile dt
  static __device__ __forceinline__ int dim(int dt, int i) { return 16 * dt + i; }
};

// fp32: 16x16x4 MFMA; lane (g, c) holds 16-byte pieces LP*g .. of its rows.
template <int DH> struct AttnT<float, DH> {
  static constexpr int ROWB = DH * 4, PIECES = ROWB / 16, LP = PIECES / 4, NDT = DH / 16, VB = NDT * 4;
  static constexpr int QKN = 4 * LP;                  // QK^T MFMAs per 16 keys
  struct QF { V4u p[LP]; };
  struct KF { V4u p[2][LP]; };
  typedef Words<NDT> VV;
  struct VF { VV v[8]; };
  static constexpr int NVR = 8;
  static __device__ __forceinline__ void load_q(QF& q, const char* row, int g) {
#pragma unroll
    for (int s = 0; s < LP; ++s) q.p[s] = *(const V4u*)(row + 16 * (LP * g + s));
  }
  static __device__ __forceinline__ int vkey(int g, int c, int j) { return slot_key(g, j); }
  static __device__ __forceinline__ void load_k(KF& k, uint32_t base, const int (&rk)[2], int g) {
#pragma unroll
    for (int kg = 0; kg < 2; ++kg)
#pragma unroll
      for (int s = 0; s < LP; ++s) k.p[kg][s] = lds_get<V4u>(piece_addr<ROWB>(base, rk[kg], LP * g + s));
  }
  // slot e of lane (g, c): key row rvs[e]; the lane reads the NDT dims NDT*c .. of it
  static __device__ __forceinline__ void load_v8(VF& v, uint32_t base, const int (&rvs)[8], int c) {
    const int off = VB * c;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t a = piece_addr<ROWB>(base, rvs[e], off / 16) + off % 16;
      if constexpr (NDT == 1) {
        v.v[e].w[0] = lds_get<uint32_t>(a);
      } else {
        v.v[e] = __builtin_bit_cast(VV, lds_get<V4u>(a));
      }
    }
  }
  static __device__ __forceinline__ void load_vr(VF& v, uint32_t base, const int (&rv)[NVR], int c) {
    load_v8(v, base, rv, c);
  }
  static __device__ __forceinline__ void load_k_lo(KF& k, uint32_t base, const int (&rk)[2], int g) {
#pragma unroll
    for (int s = 0; s < LP; ++s) k.p[0][s] = lds_get<V4u>(piece_addr<ROWB>(base, rk[0], LP * g + s));
  }
  static __device__ __forceinline__ void load_vr_lo(VF& v, uint32_t base, const int (&rv)[NVR], int c) {
    const int off = VB * c;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if (e >= 4) {
        v.v[e] = VV{};
        continue;
      }
      const uint32_t a = piece_addr<ROWB>(base, rv[e], off / 16) + off % 16;
      if constexpr (NDT == 1) {
        v.v[e].w[0] = lds_get<uint32_t>(a);
      } else {
        v.v[e] = __builtin_bit_cast(VV, lds_get<V4u>(a));
      }
    }
  }
  struct Lofs {};
  static __device__ __forceinline__ Lofs lane_ofs(int, int) { return Lofs{}; }
  static __device__ __forceinline__ void load_k_at(KF& k, uint32_t base, const Lofs&, int g, int c) {
    const int rk[2] = {c, 16 + c};
    load_k(k, base, rk, g);
  }
  static __device__ __forceinline__ void load_v_at(VF& v, uint32_t base, const Lofs&, int g, int c) {
    int rv[NVR];
#pragma unroll
    for (int j = 0; j < NVR; ++j) rv[j] = vkey(g, c, j);
    load_v8(v, base, rv, c);
  }
  static __device__ __forceinline__ f32x4 qk(const KF& k, int kg, const QF& q) {
    f32x4 acc = {0, 0, 0, 0};
#pragma unroll
    for (int s = 0; s < LP; ++s)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc = mfma_f32_4(__uint_as_float(k.p[kg][s][j]), __uint_as_float(q.p[s][j]), acc);
    return acc;
  }
  static __device__ __forceinline__ void qk2(const KF& k, const QF& q, f32x4& a0, f32x4& a1) {
    a0 = f32x4{0, 0, 0, 0};
    a1 = f32x4{0, 0, 0, 0};
#pragma unroll
    for (int s = 0; s < LP; ++s)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        a0 = mfma_f32_4(__uint_as_float(k.p[0][s][j]), __uint_as_float(q.p[s][j]), a0);
        a1 = mfma_f32_4(__uint_as_float(k.p[1][s][j]), __uint_as_float(q.p[s][j]), a1);
      }
  }
  struct PP { float p[8]; };
  static __device__ __forceinline__ PP prep(const float* ps) {
    PP r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r.p[e] = ps[e];
    return r;
  }
  static __device__ __forceinline__ f32x4 pv(const VF& v, int dt, const PP& pp, f32x4 o) {
#pragma unroll
    for (int e = 0; e < 8; ++e) o = mfma_f32_4(__uint_as_float(v.v[e].w[dt]), pp.p[e], o);
    return o;
  }
  static __device__ __forceinline__ int dim(int dt, int i) { return NDT * i + dt; }
};

// Maximum / minimum over the 16 lanes of each DPP row (row rotations by 8,
// 4, 2 and 1): the rows of a tile sit in lanes c = 0..15 of every 16-lane group.
__device__ __forceinline__ int row16_max(int x) {
  x = max(x, __builtin_amdgcn_update_dpp(x, x, 0x128, 0xf, 0xf, false));
  x = max(x, __builtin_amdgcn_update_dpp(x, x, 0x124, 0xf, 0xf, false));
  x = max(x, __builtin_amdgcn_update_dpp(x, x, 0x122, 0xf, 0xf, false));
  return max(x, __builtin_amdgcn_update_dpp(x, x, 0x121, 0xf, 0xf, false));
}
__device__ __forceinline__ int row16_min(int x) {
  x = min(x, __builtin_amdgcn_update_dpp(x, x, 0x128, 0xf, 0xf, false));
  x = min(x, __builtin_amdgcn_update_dpp(x, x, 0x124, 0xf, 0xf, false));
  x = min(x, __builtin_amdgcn_update_dpp(x, x, 0x122, 0xf, 0xf, false));
  return min(x, __builtin_amdgcn_update_dpp(x, x, 0x121, 0xf, 0xf, false));
}

// Reductions over the 4 lanes of a row (lanes l, l^16, l^32, l^48) with the
// cross-row swaps: both results of a swap hold the pair (low lane, high lane),
// so op(r[0], r[1]) gives every lane of the pair the same value.
__device__ __forceinline__ float row4_max(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float row4_sum(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Softmax half of one online chunk step for the lane's row.  s[e]: raw QK
// score of slot e (-inf: not visible).  The reference m (the same in the
// row's four lanes) moves to the chunk's row maximum only when that exceeds
// it by more than RESCALE; p = 2^(s sl2 - m'); the lane keeps its own
// running sum l' = l 2^(m - m') + sum of its p (fixed order), the row's sum
// being the four lanes' sum at the end.  Leaves p in s and returns the factor
// 2^(m - m') the running O must be scaled by before P V is added (exactly 1
// when m stays; a row that has seen no key keeps m = M_NONE and p = 0).
__device__ __forceinline__ float row_max8(const float (&s)[8]) {
  return fmaxf(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])), fmaxf(fmaxf(s[4], s[5]), fmaxf(s[6], s[7])));
}
// The reference moves when fma(max, sl2, -m) > RESCALE, a test monotone in
// the maximum, so a row moves exactly when one of its lanes' own
// maxima passes it: the ring's usual-case test and this one agree row by row.
__device__ __forceinline__ bool ref_moves(float mx, float sl2, float m) {
  return __builtin_fmaf(mx, sl2, -m) > RESCALE;
}
__device__ __forceinline__ float chunk_softmax(float (&s)[8], float sl2, float& m, float& l) {
  const float mr = row4_max(row_max8(s));
  const float mn = ref_moves(mr, sl2, m) ? mr * sl2 : m;
  const float wa = ex2(m - mn);
#pragma unroll
  for (int e = 0; e < 8; ++e) s[e] = ex2(__builtin_fmaf(s[e], sl2, -mn));
  float ls = s[0];
#pragma unroll
  for (int e = 1; e < 8; ++e) ls += s[e];
  l = __builtin_fmaf(l, wa, ls);
  m = mn;
  return wa;
}

// keep a P^T operand where it is computed (an empty asm the compiler must
// see its value at)
__device__ __forceinline__ void tie_pp(bf16x8& p) { asm volatile("" : "+v"(p)); }
template <typename PPT> __device__ __forceinline__ void tie_pp(PPT& p) {
#pragma unroll
  for (int e = 0; e < 8; ++e) asm volatile("" : "+v"(p.p[e]));
}

template <int NDT> __device__ __forceinline__ void scale_o(f32x4* O, float wa) {
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int r = 0; r < 4; ++r) O[dt][r] *= wa;
}

// Tail stage addressing.  Stage row of position x on a branch: committed
// positions (below shared_end) sit at x - tbase; later ones at ncom + the
// branch's workspace row for x, read from the staged path table (word w of
// path_read).  Positions the branch does not reach are never visible to its
// rows; they read staged row 0.
template <int NR> __device__ __forceinline__ void path_read(uint32_t (&w)[NR], uint32_t pst, int b,
                                                            const int (&x)[NR], int se, int maxp) {
#pragma unroll
  for (int j = 0; j < NR; ++j) w[j] = lds_get<uint32_t>(pst + 4 * (uint32_t)(b * maxp + min(max(x[j] - se, 0), maxp - 1)));
}
template <int NR> __device__ __forceinline__ void path_rows(int (&r)[NR], const uint32_t (&w)[NR], const int (&x)[NR],
                                                            int se, int tbase, int ncom, int nws) {
#pragma unroll
  for (int j = 0; j < NR; ++j) r[j] = x[j] < se ? x[j] - tbase : (w[j] < (unsigned)nws ? ncom + (int)w[j] : 0);
}

// Wait until at most k of the wave's chunk loads (pw loads each) are in flight, 0 <= k < KMAX.
template <int PW, int KMAX, int K = 0> __device__ __forceinline__ void ring_wait(int k) {
  if constexpr (K + 1 >= KMAX) {
    dma_wait<K * PW>();
  } else {
    if (k <= K) dma_wait<K * PW>();
    else ring_wait<PW, KMAX, K + 1>(k);
  }
}

// One workgroup per (KV head, key split, row group of NW x TPW tiles); a
// ring of D chunk slots.
template <typename T, int DH, int NW, int TPW, int D>
__device__ __forceinline__ void attn_body(const LaAttnArgs& a, const unsigned blk) {
  typedef AttnT<T, DH> AT;
  constexpr int ROWB = AT::ROWB, NDT = AT::NDT, NVR = AT::NVR;
  constexpr int CHB = CH * ROWB;                 // K (or V) of one chunk
  constexpr int SLOT = 2 * CHB;                  // one ring slot: K then V
  constexpr int NI = SLOT / 1024;                // 1 KB DMA instructions per chunk
  constexpr int PW = NI >= NW ? NI / NW : 1;     // per wave (waves past NI repeat wave w % NI's load)
  static_assert(NI % NW == 0 || NW % NI == 0, "DMA split");
  static_assert(D >= 2 && (D - 1) * PW < 64, "ring depth within the vmcnt range");
  constexpr int RPB = 1024 / ROWB;               // rows per DMA instruction
  constexpr int PIECES = ROWB / 16;
  // with four or more slots the ring refills a chunk's slot one step late,
  // so the per-chunk barrier need not wait for the LDS reads just issued
  constexpr bool LAG = D >= 4;
  extern __shared__ __attribute__((aligned(1024))) char lds[];

  ARGS_READY("s"(a.Hkv), "s"(a.wg_head), "s"(a.rgroups), "s"(a.nsplit), "s"(a.spl), "s"(a.ring_end), "s"(a.tail0),
             "s"(a.n_tail), "s"(a.shared_end), "s"(a.scale_log2), "s"(a.T_cap), "s"(a.kc), "s"(a.vc), "s"(a.H),
             "s"(a.Q), "s"(a.q), "s"(a.pos), "s"(a.st_bytes), "s"(a.tile_meta), "s"(a.branch), "s"(a.kw), "s"(a.vw),
             "s"(a.ws_cap), "s"(a.st_rows), "s"(a.st_half), "s"(a.path), "s"(a.nb), "s"(a.maxp), "s"(a.n_ws));
  // block -> (XCD, KV head, split, row group); the highest splits (tail chunks) first
  const int xcd = blk & 7, bi = blk >> 3;
  const int g_kv = xcd + 8 * (bi / a.wg_head);
  if (g_kv >= a.Hkv) return;
  const int li = bi % a.wg_head;
  const int sp = a.nsplit - 1 - li / a.rgroups;
  const int rg = li % a.rgroups;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, c16 = lane & 15;
  const int se = a.shared_end;
  const float sl2 = a.scale_log2;
  const char* kc = (const char*)a.kc + (size_t)g_kv * a.T_cap * ROWB;
  const char* vc = (const char*)a.vc + (size_t)g_kv * a.T_cap * ROWB;

  // this split's chunks: ring chunks [r_lo, r_hi), tail chunks [t_lo, t_hi), all taken in decreasing order
  const int s_lo = sp * a.spl, s_hi = s_lo + a.spl;
  const int r_lo = s_lo, r_hi = min(s_hi, a.ring_end);
  const int t_lo = max(s_lo, a.tail0), t_hi = min(s_hi, a.tail0 + a.n_tail);
  const bool has_tail = t_lo < t_hi;              // uniform over the workgroup
  const int nring = max(0, r_hi - r_lo);

  // the wave's tiles, row-tile major: tile t = rows 16 (t / group) .., query
  // head g_kv * group + t % group (a wave's tiles share their rows when the
  // group is at least TPW, and so their branches).  Rows past Q (and tiles
  // past the last) compute on row Q - 1's data and store nothing.  Nothing
  // is computed from the loads until they are needed: the compiler does not
  // count the asm DMA, so its wait for them also waits for the DMA issued
  // before that point.
  const int group = a.H / a.Hkv;
  const int rtiles = (a.Q + 15) >> 4;
  bool tv[TPW], rvalid[TPW];
  int hh[TPW], row[TPW], pos[TPW];
  typename AT::QF qf[TPW];
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    const int tile = (rg * NW + wave) * TPW + u;
    tv[u] = tile < group * rtiles;
    hh[u] = g_kv * group + (tv[u] ? tile % group : 0);
    row[u] = (tv[u] ? tile / group : 0) * 16 + c16;
    rvalid[u] = tv[u] && row[u] < a.Q;
    const int rr = min(row[u], a.Q - 1);
    AT::load_q(qf[u], (const char*)a.q + ((size_t)rr * a.H + hh[u]) * ROWB, g);
    pos[u] = a.pos[rr];
  }

  // LDS: [tail stage (K rows, V rows, path table)] [ring of D slots]
  const int st_bytes = has_tail ? a.st_bytes : 0;
  char* const ring = lds + st_bytes;

  // ring chunk i (0 = the split's last ring chunk, i < nring) into slot
  // i % D.  A chunk wholly below shared_end is one affine run of rows; in
  // the last chunk of a call without tail, rows past shared_end - 1 repeat
  // it (never visible).
  uint32_t lsrc[PW];                              // the lane's byte offset inside a chunk, per load
#pragma unroll
  for (int j = 0; j < PW; ++j) {
    const int ins = (wave * PW + j) % NI;
    const int r = (ins % (NI / 2)) * RPB + lane / PIECES;
    lsrc[j] = r * ROWB + 16 * ((lane % PIECES) ^ piece_swz<PIECES>(r));
  }
  auto issue = [&](int i) __attribute__((always_inline)) {
    const int cidx = r_hi - 1 - i;
    const uint32_t slot = lds_addr(ring) + (uint32_t)(i % D) * SLOT;
    if (CH * cidx + CH <= se) {
#pragma unroll
      for (int j = 0; j < PW; ++j) {
        const int ins = (wave * PW + j) % NI;     // 0 .. NI-1: K blocks, then V blocks
        const int half = ins / (NI / 2), blk = ins % (NI / 2);
        dma16((half ? vc : kc) + (size_t)cidx * CHB + lsrc[j], slot + half * CHB + blk * 1024);
      }
    } else {
#pragma unroll
      for (int j = 0; j < PW; ++j) {
        const int ins = (wave * PW + j) % NI;
        const int half = ins / (NI / 2), blk = ins % (NI / 2);
        const int r = blk * RPB + lane / PIECES;
        const int src_row = min(CH * cidx + r, se - 1);
        dma16((half ? vc : kc) + (size_t)src_row * ROWB + 16 * ((lane % PIECES) ^ piece_swz<PIECES>(r)),
              slot + half * CHB + blk * 1024);
      }
    }
  };

  // tail WGs: each tile's distinct branches (lane i < 16: the i-th) and each row's branch, loaded with Q
  int nbr[TPW], bid[TPW], br[TPW];
  const int ncom = se - CH * a.tail0;
  float M[TPW], L[TPW];
  f32x4 O[TPW][NDT];
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    M[u] = M_NONE;
    L[u] = 0.f;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) O[u][dt] = f32x4{0, 0, 0, 0};
  }

  // committed chunks through the ring, in decreasing position, software
  // pipelined: step i issues the QK^T MFMAs of chunk i + 1 (its K fragments
  // were read in step i - 1) ahead of chunk i's softmax, so the products run
  // while the vector ALU works; then chunk i's P V.  One set of K and one of V
  // fragment registers.  One barrier per chunk: chunk i + 2 has landed and
  // every wave has read chunk i + 1 (K and V), whose slot is then refilled.
  const typename AT::Lofs lofs = AT::lane_ofs(g, c16);
  auto slot_base = [&](int i) __attribute__((always_inline)) {
    return (uint32_t)__builtin_amdgcn_readfirstlane(lds_addr(ring) + (uint32_t)(i % D) * SLOT);
  };
  auto ring_part = [&]() __attribute__((always_inline)) {
    if (nring <= 0) return;
    typename AT::KF kf;
    typename AT::VF vf;
    ring_wait<PW, D - 1>(min(D - 2, nring - 1));   // chunk 0 landed (chunks 1 .. D - 2 may be in flight)
    ring_barrier();
    // first use of Q and the positions where nothing used them yet: the
    // compiler's wait for them (which also waits for the chunks issued so
    // far) falls here, once, and not inside the loop
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
#pragma unroll
      for (int s = 0; s < (int)(sizeof(qf[u].p) / sizeof(qf[u].p[0])); ++s) asm volatile("" : "+v"(qf[u].p[s]));
      asm volatile("" : "+v"(pos[u]));
    }
    int pmin = 0x7fffffff;                          // smallest row position of the wave
#pragma unroll
    for (int u = 0; u < TPW; ++u) pmin = min(pmin, pos[u]);
    pmin = __builtin_amdgcn_readfirstlane(row16_min(pmin));
    // chunks 0 .. jm - 1 hold a key past some row of the wave: only they are masked
    const int jm = min(nring, max(0, r_hi - (pmin + 1) / CH));
    if (D - 1 < nring) issue(D - 1);
    AT::load_k_at(kf, slot_base(0), lofs, g, c16);
    AT::load_v_at(vf, slot_base(0) + CHB, lofs, g, c16);
    float sc[TPW][8];
    auto qk_all = [&](float (&s)[TPW][8]) __attribute__((always_inline)) {
#pragma unroll
      for (int u = 0; u < TPW; ++u) {
        f32x4 s0, s1;
        AT::qk2(kf, qf[u], s0, s1);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          s[u][r] = s0[r];
          s[u][4 + r] = s1[r];
        }
      }
    };
    qk_all(sc);
    if (nring > 1) {
      ring_wait<PW, D - 1>(min(D - 2, nring - 2));  // chunk 1 landed
      ring_barrier();                               // every wave has read chunk 0: its slot is free
      if (!LAG && D < nring) issue(D);
      AT::load_k_at(kf, slot_base(1), lofs, g, c16);
    }
    auto step = [&](int i, auto masked, auto last) __attribute__((always_inline)) {
      float sn[TPW][8];
      if constexpr (!decltype(last)::value) qk_all(sn);   // chunk i + 1, in flight during the softmax
      if constexpr (decltype(masked)::value) {
        const int x0 = CH * (r_hi - 1 - i);
#pragma unroll
        for (int u = 0; u < TPW; ++u)
#pragma unroll
          for (int e = 0; e < 8; ++e) sc[u][e] = x0 + slot_key(g, e) <= pos[u] ? sc[u][e] : NEG_INF;
      }
      // the usual case first: no row's maximum moves (p against the current
      // reference, the sums grow by the chunk's); if some row's would, the
      // chunk goes through chunk_softmax instead (same arithmetic where the
      // reference stays, so a row's bits do not depend on the other rows)
      typename AT::PP pp[TPW];
      float ps[TPW][8], lsum[TPW];
      bool moves = false;
#pragma unroll
      for (int u = 0; u < TPW; ++u) {
        // the exponents s sl2 - m; their maximum is fma(max s, sl2, -m) (a
        // monotone map), so the test is ref_moves' on this lane's scores
        float t[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) t[e] = __builtin_fmaf(sc[u][e], sl2, -M[u]);
        moves |= row_max8(t) > RESCALE;
#pragma unroll
        for (int e = 0; e < 8; ++e) ps[u][e] = ex2(t[e]);
        float ls = ps[u][0];                        // = 0 + p0 (p >= +0)
#pragma unroll
        for (int e = 1; e < 8; ++e) ls += ps[u][e];
        lsum[u] = L[u] + ls;
        pp[u] = AT::prep(ps[u]);
      }
      if constexpr (!decltype(last)::value) {
        // one QK^T MFMA, then a share of the softmax's vector instructions
#pragma unroll
        for (int k = 0; k < 2 * TPW * AT::QKN; ++k) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
        }
      }
      // computed here, before the branch, in both cases (the compiler would
      // otherwise sink them past it, away from the QK^T MFMAs)
#pragma unroll
      for (int u = 0; u < TPW; ++u) {
        tie_pp(pp[u]);
        asm volatile("" : "+v"(lsum[u]));
      }
      auto pv_all = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
          for (int u = 0; u < TPW; ++u) O[u][dt] = AT::pv(vf, dt, pp[u], O[u][dt]);
      };
      if (__ballot(moves) != 0ull) {                // some reference maximum moves: the full step, O * wa
#pragma unroll
        for (int u = 0; u < TPW; ++u) {
          const float wa = chunk_softmax(sc[u], sl2, M[u], L[u]);
          pp[u] = AT::prep(sc[u]);
          scale_o<NDT>(O[u], wa);
        }
        pv_all();
      } else {
#pragma unroll
        for (int u = 0; u < TPW; ++u) L[u] = lsum[u];
        pv_all();
      }
      if constexpr (!decltype(last)::value) {
        AT::load_v_at(vf, slot_base(i + 1) + CHB, lofs, g, c16);
        if (i + 2 < nring) {
          if constexpr (LAG) {
            // chunks up to i - 1 + D issued; chunk i's reads were used before the barrier
            ring_wait<PW, D - 1>(min(D - 3, nring - 3 - i));   // chunk i + 2 landed
            slot_barrier();                         // every wave has used chunk i: its slot is free
            if (i + D < nring) issue(i + D);
          } else {
            ring_wait<PW, D - 1>(min(D - 2, nring - 3 - i));   // chunk i + 2 landed
            ring_barrier();                         // every wave has read chunk i + 1: its slot is free
            if (i + 1 + D < nring) issue(i + 1 + D);
          }
          AT::load_k_at(kf, slot_base(i + 2), lofs, g, c16);
        }
#pragma unroll
        for (int u = 0; u < TPW; ++u)
#pragma unroll
          for (int e = 0; e < 8; ++e) sc[u][e] = sn[u][e];
      }
    };
    using T_ = std::true_type;
    using F_ = std::false_type;
    int i = 0;
    for (; i < min(jm, nring - 1); ++i) step(i, T_{}, F_{});
    for (; i < nring - 1; ++i) step(i, F_{}, F_{});
    if (jm >= nring) step(nring - 1, T_{}, T_{});
    else step(nring - 1, F_{}, T_{});
  };
  // chunks past shared_end, from the tail stage (the highest positions of the split: they come first)
  auto tail_part = [&]() __attribute__((always_inline)) {
    ring_barrier();                               // every wave's part of the stage is visible
    int pmax[TPW];                                // largest row position of each tile
#pragma unroll
    for (int u = 0; u < TPW; ++u) pmax[u] = __builtin_amdgcn_readfirstlane(row16_max(pos[u]));
    // the distinct branches of the wave's tiles: lane k < nu holds the k-th
    int ub = -1, nu = 0;
    if constexpr (TPW == 1) {
      // one tile: the row builder's list of its branches is distinct already
      nu = __builtin_amdgcn_readfirstlane(nbr[0]);
      ub = lane < nu ? bid[0] : -1;
    } else {
#pragma unroll
      for (int u = 0; u < TPW; ++u) {
        const int n = __builtin_amdgcn_readfirstlane(nbr[u]);
        for (int i = 0; i < n; ++i) {
          const int b = __builtin_amdgcn_readlane(bid[u], i);
          if (__ballot(ub == b) == 0ull) {
            ub = lane == nu ? b : ub;
            ++nu;
          }
        }
      }
    }
    const uint32_t kst = lds_addr(lds), vst = kst + a.st_half, pst = kst + 2 * a.st_half;
    const int maxp = a.maxp, nws = a.n_ws, tbase = CH * a.tail0;
    for (int cidx = t_hi - 1; cidx >= t_lo; --cidx) {
      const int x0 = CH * cidx;
      bool tl[TPW];                               // tiles with a row reaching the chunk (uniform)
      int pm = -1;
#pragma unroll
      for (int u = 0; u < TPW; ++u) {
        tl[u] = tv[u] && pmax[u] >= x0;
        pm = tl[u] ? max(pm, pmax[u]) : pm;
      }
      // whether some row reaches the chunk's upper 16 keys (uniform); if not,
      // that half's K, V and QK^T are skipped: its scores stay -inf and its
      // V reads as zeros, so p = 0 there as before
      const bool hi = pm >= x0 + 16;
      auto ldk = [&](typename AT::KF& kf, const int (&rk)[2]) __attribute__((always_inline)) {
        if (hi) AT::load_k(kf, kst, rk, g);
        else AT::load_k_lo(kf, kst, rk, g);
      };
      const int xk[2] = {x0 + c16, x0 + 16 + c16};
      int xv[NVR];
#pragma unroll
      for (int j = 0; j < NVR; ++j) xv[j] = x0 + AT::vkey(g, c16, j);

      // QK^T, branch by branch: branch k's K fragments are read while the
      // MFMAs of branch k - 1 run; a row keeps the scores of its own branch
      float sc[TPW][8];
#pragma unroll
      for (int u = 0; u < TPW; ++u)
#pragma unroll
        for (int e = 0; e < 8; ++e) sc[u][e] = NEG_INF;
      auto qk_branch = [&](const typename AT::KF& kf, int b) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < TPW; ++u) {
          const bool mine = br[u] == b;
          if (!tl[u] || __ballot(mine) == 0ull) continue;
#pragma unroll
          for (int kg = 0; kg < 2; ++kg) {
            if (kg == 1 && !hi) break;
            const f32x4 s4 = AT::qk(kf, kg, qf[u]);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float v = (x0 + 16 * kg + 4 * g + r <= pos[u]) ? s4[r] : NEG_INF;
              sc[u][4 * kg + r] = mine ? v : sc[u][4 * kg + r];
            }
          }
        }
      };
      if (nu > 0) {
        typename AT::KF ka, kb;
        uint32_t w[2];
        int rk[2];
        path_read(w, pst, __builtin_amdgcn_readlane(ub, 0), xk, se, maxp);
        path_rows(rk, w, xk, se, tbase, ncom, nws);
        ldk(ka, rk);
        if (nu > 1) path_read(w, pst, __builtin_amdgcn_readlane(ub, 1), xk, se, maxp);
        for (int k = 0; k < nu; k += 2) {
          // ka: branch k; w: path words of branch k + 1
          if (k + 1 < nu) {
            path_rows(rk, w, xk, se, tbase, ncom, nws);
            ldk(kb, rk);
            if (k + 2 < nu) path_read(w, pst, __builtin_amdgcn_readlane(ub, k + 2), xk, se, maxp);
          }
          qk_branch(ka, __builtin_amdgcn_readlane(ub, k));
          if (k + 1 >= nu) break;
          if (k + 2 < nu) {
            path_rows(rk, w, xk, se, tbase, ncom, nws);
            ldk(ka, rk);
            if (k + 3 < nu) path_read(w, pst, __builtin_amdgcn_readlane(ub, k + 3), xk, se, maxp);
          }
          qk_branch(kb, __builtin_amdgcn_readlane(ub, k + 1));
        }
      }
      float wa[TPW];
      bool rescale = false;
#pragma unroll
      for (int u = 0; u < TPW; ++u) {
        wa[u] = chunk_softmax(sc[u], sl2, M[u], L[u]);
        rescale |= tl[u] && wa[u] != 1.f;
      }
      if (__ballot(rescale) != 0ull) {
#pragma unroll
        for (int u = 0; u < TPW; ++u) scale_o<NDT>(O[u], wa[u]);
      }
      // P V, branch by branch: a row's probabilities enter only its own
      // branch's product (the other branches add exact zeros)
      auto pv_branch = [&](const typename AT::VF& vf, int b) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < TPW; ++u) {
          const bool mine = br[u] == b;
          if (!tl[u] || __ballot(mine) == 0ull) continue;
          float ps[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) ps[e] = mine ? sc[u][e] : 0.f;
          const typename AT::PP pp = AT::prep(ps);
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) O[u][dt] = AT::pv(vf, dt, pp, O[u][dt]);
        }
      };
      auto ldv = [&](typename AT::VF& vf, const int (&rv)[NVR]) __attribute__((always_inline)) {
        if (hi) AT::load_vr(vf, vst, rv, c16);
        else AT::load_vr_lo(vf, vst, rv, c16);
      };
      if (nu > 0) {
        typename AT::VF va, vb;
        uint32_t w[NVR];
        int rv[NVR];
        path_read(w, pst, __builtin_amdgcn_readlane(ub, 0), xv, se, maxp);
        path_rows(rv, w, xv, se, tbase, ncom, nws);
        ldv(va, rv);
        if (nu > 1) path_read(w, pst, __builtin_amdgcn_readlane(ub, 1), xv, se, maxp);
        for (int k = 0; k < nu; k += 2) {
          if (k + 1 < nu) {
            path_rows(rv, w, xv, se, tbase, ncom, nws);
            ldv(vb, rv);
            if (k + 2 < nu) path_read(w, pst, __builtin_amdgcn_readlane(ub, k + 2), xv, se, maxp);
          }
          pv_branch(va, __builtin_amdgcn_readlane(ub, k));
          if (k + 1 >= nu) break;
          if (k + 2 < nu) {
            path_rows(rv, w, xv, se, tbase, ncom, nws);
            ldv(va, rv);
            if (k + 3 < nu) path_read(w, pst, __builtin_amdgcn_readlane(ub, k + 3), xv, se, maxp);
          }
          pv_branch(vb, __builtin_amdgcn_readlane(ub, k + 1));
        }
      }
    }
  };

  // The two kinds of workgroup run separate copies of the code, so that the
  // compiler's waits for Q and the positions fall where each needs them.
  if (has_tail) {
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      const int* meta = a.tile_meta + (size_t)(row[u] >> 4) * 64;
      nbr[u] = meta[0];
      bid[u] = meta[1 + (lane & 15)];
      br[u] = a.branch[min(row[u], a.Q - 1)];
    }
    // the stage: committed rows [32 tail0, shared_end), then every packed
    // row's K/V (workspace rows), K rows then V rows, then the row builder's
    // branch path table [nb][maxp]; it lands before the ring is issued
    const char* kw = (const char*)a.kw + (size_t)g_kv * a.ws_cap * ROWB;
    const char* vw = (const char*)a.vw + (size_t)g_kv * a.ws_cap * ROWB;
    const int st_rows = a.st_rows;
    const int nblk = (st_rows + RPB - 1) / RPB;
    for (int ins = wave; ins < 2 * nblk; ins += NW) {
      const int half = ins / nblk, blk = ins % nblk;
      const int r = blk * RPB + lane / PIECES;
      const char* src;
      if (r < ncom) src = (half ? vc : kc) + (size_t)(CH * a.tail0 + r) * ROWB;
      else if (r < st_rows) src = (half ? vw : kw) + (size_t)(r - ncom) * ROWB;
      else src = (half ? vc : kc) + (size_t)(se - 1) * ROWB;
      dma16(src + 16 * ((lane % PIECES) ^ piece_swz<PIECES>(r)), lds_addr(lds + half * a.st_half + blk * 1024));
    }
    const int npath = a.nb * a.maxp;
    for (int ins = wave; ins * 64 < npath; ins += NW)
      dma4(a.path + min(ins * 64 + lane, npath - 1), lds_addr(lds + 2 * a.st_half + ins * 256));
    dma_wait<0>();                                // stage and this wave's loads landed
    // the compiler does not count the DMA: tie the loaded values here, so
    // that its own wait for them falls here and not after the ring's issue
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
#pragma unroll
      for (int s = 0; s < (int)(sizeof(qf[u].p) / sizeof(qf[u].p[0])); ++s) asm volatile("" : "+v"(qf[u].p[s]));
      asm volatile("" : "+v"(pos[u]), "+v"(nbr[u]), "+v"(bid[u]), "+v"(br[u]));
      nbr[u] = tv[u] ? min(nbr[u], 16) : 0;
      bid[u] = lane < 16 ? bid[u] : -1;
    }
    // the ring's first D - 1 chunks
#pragma unroll
    for (int i = 0; i < D - 1; ++i)
      if (i < nring) issue(i);
    tail_part();
    ring_part();
  } else {
#pragma unroll
    for (int i = 0; i < D - 1; ++i)
      if (i < nring) issue(i);
    ring_part();
  }
  dma_wait<0>();                                   // no DMA may land after the workgroup has left

  // results: lane (g, c) holds rows c, accumulator rows 4 g + r of every output tile
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    L[u] = row4_sum(L[u]);
    if (M[u] == M_NONE) M[u] = NEG_INF;
  }
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    if (!rvalid[u]) continue;
    if (a.nsplit > 1) {
      const size_t base = ((size_t)sp * a.H + hh[u]) * a.Q + row[u];
      if (g == 0) *(float2*)(a.part_ml + base * 2) = make_float2(M[u], L[u]);
      float* po = a.part_o + base * DH;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        if constexpr (std::is_same<T, bf16_t>::value) {
          *(float4*)(po + AT::dim(dt, 4 * g)) = make_float4(O[u][dt][0], O[u][dt][1], O[u][dt][2], O[u][dt][3]);
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) po[AT::dim(dt, 4 * g + r)] = O[u][dt][r];
        }
      }
      continue;
    }
    T* dst = (T*)a.o + ((size_t)row[u] * a.H + hh[u]) * DH;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      if constexpr (std::is_same<T, bf16_t>::value) {
        const uint32_t w0 = (uint32_t)f2bf(O[u][dt][0] / L[u]) | ((uint32_t)f2bf(O[u][dt][1] / L[u]) << 16);
        const uint32_t w1 = (uint32_t)f2bf(O[u][dt][2] / L[u]) | ((uint32_t)f2bf(O[u][dt][3] / L[u]) << 16);
        *(uint2*)(dst + AT::dim(dt, 4 * g)) = make_uint2(w0, w1);
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) dst[AT::dim(dt, 4 * g + r)] = O[u][dt][r] / L[u];
      }
    }
  }
}

template <typename T, int DH, int NW, int TPW, int D>
__global__ void __launch_bounds__(64 * NW) la_attn_kernel(LaAttnArgs a) {
  attn_body<T, DH, NW, TPW, D>(a, blockIdx.x);
}

// Several requests in one launch: block b belongs to the last entry whose
// first workgroup is at or below b (every request's block count is a
// multiple of 8, so b % 8 is also the block's XCD inside the request).
template <typename T, int DH, int NW, int TPW, int D>
__global__ void __launch_bounds__(64 * NW) la_attn_multi_kernel(const LaAttnSeg* __restrict__ segs, int n,
                                                               int layer) {
  const int b = blockIdx.x;
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (segs[mid].blk0 <= b) lo = mid;
    else hi = mid - 1;
  }
  LaAttnArgs a = segs[lo].a;
  const long long kvo = layer * segs[lo].kv_layer, wso = layer * segs[lo].ws_layer;
  a.kc = (const char*)a.kc + kvo;
  a.vc = (const char*)a.vc + kvo;
  a.kw = (const char*)a.kw + wso;
  a.vw = (const char*)a.vw + wso;
  attn_body<T, DH, NW, TPW, D>(a, (unsigned)(b - segs[lo].blk0));
}

// Fold of the key splits' states in split order (m, l, O), then O / l.  One
// thread per 4 head dimensions of a (row, head).
template <typename T, int DH>
__device__ __forceinline__ void merge_body(const LaAttnArgs& a, const unsigned blk) {
  constexpr int V4 = DH / 4, MS = 8;            // splits whose loads are all issued before the fold
  ARGS_READY("s"(a.H), "s"(a.Hkv), "s"(a.Q), "s"(a.nsplit), "s"(a.part_ml), "s"(a.part_o), "s"(a.o));
  // block -> (XCD, KV head): the head's split states were written on that
  // XCD (the attention kernel's mapping), so they are read from its L2
  const int group = a.H / a.Hkv;
  const int per = a.Q * group * V4;               // (row, q-head, 4 dims) items of one KV head
  const int wpk = (per + 255) / 256;
  const int g_kv = (blk & 7) + 8 * ((blk >> 3) / wpk);
  const int item = ((blk >> 3) % wpk) * 256 + threadIdx.x;
  if (g_kv >= a.Hkv || item >= per) return;
  const int d4 = item % V4, r2 = item / V4;
  const int row = r2 / group, hh = g_kv * group + r2 % group;
  float ma = NEG_INF, la = 0.f;
  float oa[4] = {0.f, 0.f, 0.f, 0.f};
  auto fold = [&](float2 ml, float4 ob) __attribute__((always_inline)) {
    if (ml.x == NEG_INF) return;
    const float mn = fmaxf(ma, ml.x);
    const float wa = ex2(ma - mn), wb = ex2(ml.x - mn);
    la = lin2(la, wa, ml.y, wb);
    oa[0] = lin2(oa[0], wa, ob.x, wb);
    oa[1] = lin2(oa[1], wa, ob.y, wb);
    oa[2] = lin2(oa[2], wa, ob.z, wb);
    oa[3] = lin2(oa[3], wa, ob.w, wb);
    ma = mn;
  };
  for (int s0 = 0; s0 < a.nsplit; s0 += MS) {
    float2 ml[MS];
    float4 ob[MS];
#pragma unroll
    for (int k = 0; k < MS; ++k) {
      const int s = s0 + k;
      if (s < a.nsplit) {
        const size_t base = ((size_t)s * a.H + hh) * a.Q + row;
        ml[k] = *(const float2*)(a.part_ml + base * 2);
        ob[k] = *(const float4*)(a.part_o + base * DH + 4 * d4);
      }
    }
#pragma unroll
    for (int k = 0; k < MS; ++k)
      if (s0 + k < a.nsplit) fold(ml[k], ob[k]);
  }
  T* dst = (T*)a.o + ((size_t)row * a.H + hh) * DH + 4 * d4;
  if constexpr (sizeof(T) == 2) {
    const uint32_t w0 = (uint32_t)f2bf(oa[0] / la) | ((uint32_t)f2bf(oa[1] / la) << 16);
    const uint32_t w1 = (uint32_t)f2bf(oa[2] / la) | ((uint32_t)f2bf(oa[3] / la) << 16);
    *(uint2*)dst = make_uint2(w0, w1);
  } else {
    *(float4*)dst = make_float4(oa[0] / la, oa[1] / la, oa[2] / la, oa[3] / la);
  }
}

template <typename T, int DH>
__global__ void __launch_bounds__(256) la_attn_merge_kernel(LaAttnArgs a) {
  merge_body<T, DH>(a, blockIdx.x);
}

// several requests: block b belongs to the last entry whose first merge
// workgroup is at or below b (requests of a single split have none)
template <typename T, int DH>
__global__ void __launch_bounds__(256) la_attn_merge_multi_kernel(const LaAttnSeg* __restrict__ segs, int n) {
  const int b = blockIdx.x;
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (segs[mid].mblk0 <= b) lo = mid;
    else hi = mid - 1;
  }
  merge_body<T, DH>(segs[lo].a, (unsigned)(b - segs[lo].mblk0));
}

// Chunks per key split: a function of the cache capacity and the model's head
// counts only (never of the rows of a call), so every call on one cache cuts
// its keys the same way.  About `target` splits when the cache is full --
// eight up to 40 query heads, fewer for more (their row tiles already give
// many workgroups: 64 heads take five, which keeps a 90-row round of 64
// query heads on 8 KV heads within one workgroup per CU with the shortest
// splits) -- and at least 4 chunks.
static int spl_for(int t_cap, int H, int Hkv) {
  const int nch = (std::max(t_cap, 1) + CH - 1) / CH;
  const int target = std::max(1, std::min(8, 320 / std::max(1, H)));
  return std::max(4, (nch + target - 1) / target);
}
int la_attention_spl(int t_cap, int H, int Hkv) { return spl_for(t_cap, H, Hkv); }
// upper bound over head counts (the smallest split length is the one of 8 splits)
int la_attention_parts(int max_pos, int t_cap) {
  const int nch = (std::max(t_cap, 1) + CH - 1) / CH;
  const int spl = std::max(4, (nch + 7) / 8);
  return max_pos < 0 ? 1 : max_pos / (CH * spl) + 1;
}

// The tail stage holds the committed part of the first tail chunk (< 32
// rows) and every packed row but the ordinary one, K and V, and the branch
// path table, beside a ring of at least two chunk slots.
int la_attention_fits(int dh, int esz, int q_max, int nb_max, int maxp_max) {
  const size_t rowb = (size_t)dh * esz, ring2 = 2 * 2 * CH * rowb;
  const size_t rows = (size_t)(CH - 1) + std::max(q_max - 1, 0);
  const size_t half = (rows * rowb + 1023) / 1024 * 1024;
  const size_t paths = ((size_t)nb_max * maxp_max * 4 + 1023) / 1024 * 1024;
  return 2 * half + paths + ring2 <= LDS_BYTES;
}

// What one launch runs: one request's arguments (by value), or a table of
// requests in device memory for a given layer.
struct AttnLaunch {
  const LaAttnArgs* a;
  const LaAttnSeg* segs;
  int n, layer;
};

template <typename T, int DH, int NW, int TPW, int D>
static void launch_cfg(const AttnLaunch& L, int grid, size_t lds, hipStream_t st) {
  if (L.segs) {
    static const bool attr = hipFuncSetAttribute((const void*)&la_attn_multi_kernel<T, DH, NW, TPW, D>,
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, LDS_BYTES) == hipSuccess;
    (void)attr;
    hipLaunchKernelGGL((la_attn_multi_kernel<T, DH, NW, TPW, D>), dim3(grid), dim3(64 * NW), lds, st, L.segs, L.n,
                       L.layer);
  } else {
    static const bool attr = hipFuncSetAttribute((const void*)&la_attn_kernel<T, DH, NW, TPW, D>,
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, LDS_BYTES) == hipSuccess;
    (void)attr;
    hipLaunchKernelGGL((la_attn_kernel<T, DH, NW, TPW, D>), dim3(grid), dim3(64 * NW), lds, st, *L.a);
  }
}

// ring depth: 6 chunk slots where the LDS holds them beside the tail stage
// (bf16), else 4, else 2; a single wave issues a whole chunk's 16 loads, so it
// keeps at most 4 slots (the vmcnt counter holds 63 loads)
template <typename T, int DH, int NW, int TPW>
static void launch_depth(const AttnLaunch& L, int depth, int grid, size_t lds, hipStream_t st) {
  constexpr bool deep = std::is_same<T, bf16_t>::value && NW > 1;
  if (deep && depth == 6) launch_cfg<T, DH, NW, TPW, deep ? 6 : 4>(L, grid, lds, st);
  else if (depth == 4) launch_cfg<T, DH, NW, TPW, 4>(L, grid, lds, st);
  else launch_cfg<T, DH, NW, TPW, 2>(L, grid, lds, st);
}

template <typename T, int DH>
static void launch_shape(const AttnLaunch& L, int nw, int depth, int grid, size_t lds, hipStream_t st) {
  if (nw == 8) launch_depth<T, DH, 8, 1>(L, depth, grid, lds, st);
  else if (nw == 4) launch_depth<T, DH, 4, 1>(L, depth, grid, lds, st);
  else if (nw == 2) launch_depth<T, DH, 2, 1>(L, depth, grid, lds, st);
  else launch_depth<T, DH, 1, 1>(L, depth, grid, lds, st);
}

static int kv_slots(int Hkv) { return 8 * ((Hkv + 7) / 8); }       // KV heads rounded up to the 8 XCDs
static int attn_tiles(const LaAttnArgs& a) { return (a.H / a.Hkv) * ((a.Q + 15) / 16); }  // 16-row tiles of a KV head
static int merge_wpk(const LaAttnArgs& a, int dh) { return (a.Q * (a.H / a.Hkv) * (dh / 4) + 255) / 256; }

// Validation, and the key ranges and splits of one call.
static int attn_prep(LaAttnArgs& a) {
  if (a.H <= 0 || a.Hkv <= 0 || a.H % a.Hkv != 0 || a.shared_end < 1 || a.shared_end > a.T_cap) return -2;
  if (a.n_ws < 0 || a.n_ws > a.ws_cap || a.maxp < 1) return -2;
  const int se = a.shared_end;
  const bool tail = a.max_pos >= se;
  // ring chunks: every chunk below the first one that reaches past shared_end
  // (or up to the largest row position when nothing does); tail chunks after it
  a.tail0 = se / CH;
  a.ring_end = tail ? a.tail0 : a.max_pos / CH + 1;
  a.n_tail = tail ? a.max_pos / CH - a.tail0 + 1 : 0;
  // a branch reaches at most 64 positions past shared_end (the row builder's path table)
  if (tail && a.max_pos - se >= 64) return -2;
  a.scale_log2 = a.scale * 1.4426950408889634f;
  a.spl = spl_for(a.T_cap, a.H, a.Hkv);
  const int last_chunk = a.max_pos / CH;
  a.nsplit = last_chunk / a.spl + 1;
  if (a.nsplit > 1 && (a.part_o == nullptr || a.part_ml == nullptr || a.nsplit > a.max_splits)) return -2;
  return 0;
}

// Tiles per workgroup, for calls of tiles[i] tiles per KV head cut in
// nsplit[i] key splits: the most (up to 8) that still leave 128 workgroups
// (half the CUs) in all, one wave per tile (eight waves: two per SIMD, so one
// wave's vector ALU work overlaps the other's MFMAs and LDS waits, and one
// workgroup streams each K/V chunk for all its tiles).  Fewer waves per
// workgroup to fill more CUs lose more than they gain: a workgroup with a
// tail stage often leaves room for only one per CU, so four-wave workgroups
// then run one wave per SIMD.
static int pick_nw(const LaAttnArgs* a, int stride_bytes, int n) {
  auto at = [&](int i) -> const LaAttnArgs& { return *(const LaAttnArgs*)((const char*)a + (size_t)i * stride_bytes); };
  int tmax = 0;
  for (int i = 0; i < n; ++i) tmax = std::max(tmax, attn_tiles(at(i)));
  int nw = 1;
  for (const int c : {8, 4, 2, 1}) {
    if (c > tmax && c != 1) continue;
    long wgs = 0;
    for (int i = 0; i < n; ++i)
      wgs += (long)kv_slots(at(i).Hkv) * at(i).nsplit * ((attn_tiles(at(i)) + c - 1) / c);
    nw = c;
    if (wgs >= 128) break;
  }
  return nw;
}

// The tail stage (committed rows of the first tail chunk + every packed row,
// K and V, 1 KB aligned, then the path table) before the ring; its bytes
static size_t attn_stage(LaAttnArgs& a, int rowb) {
  size_t st_bytes = 0;
  if (a.n_tail > 0) {
    const int rows = (a.shared_end - CH * a.tail0) + a.n_ws;
    const int rpb = 1024 / rowb;
    a.st_rows = rows;
    a.st_half = ((rows + rpb - 1) / rpb) * 1024;
    st_bytes = 2 * (size_t)a.st_half + ((size_t)a.nb * a.maxp * 4 + 1023) / 1024 * 1024;
    a.st_bytes = (int)st_bytes;
  }
  return st_bytes;
}

// the deepest ring (6, 4 or 2 slots) beside a tail stage of st_bytes; 0 if none fits
static int ring_depth_for(bool bf16, int nw, int rowb, size_t st_bytes) {
  const size_t slot = 2 * (size_t)CH * rowb;
  int depth = bf16 && nw > 1 ? 6 : 4;
  while (depth > 2 && st_bytes + depth * slot > LDS_BYTES) depth -= 2;
  return st_bytes + depth * slot > LDS_BYTES ? 0 : depth;
}

static bool dh_supported(int dtype, int dh) {
  return dtype == LA_DT_BF16 ? (dh == 128 || dh == 64) : (dh == 16 || dh == 64);
}

template <typename T, int DH>
static void launch_merge(const AttnLaunch& L, int grid, hipStream_t st) {
  if (L.segs) hipLaunchKernelGGL((la_attn_merge_multi_kernel<T, DH>), dim3(grid), dim3(256), 0, st, L.segs, L.n);
  else hipLaunchKernelGGL((la_attn_merge_kernel<T, DH>), dim3(grid), dim3(256), 0, st, *L.a);
}

static void launch_any(int dtype, int dh, const AttnLaunch& L, int nw, int depth, int grid, size_t lds, int mgrid,
                       hipStream_t st) {
  if (dtype == LA_DT_BF16) {
    if (dh == 128) { launch_shape<bf16_t, 128>(L, nw, depth, grid, lds, st); if (mgrid) launch_merge<bf16_t, 128>(L, mgrid, st); }
    else { launch_shape<bf16_t, 64>(L, nw, depth, grid, lds, st); if (mgrid) launch_merge<bf16_t, 64>(L, mgrid, st); }
  } else {
    if (dh == 16) { launch_shape<float, 16>(L, nw, depth, grid, lds, st); if (mgrid) launch_merge<float, 16>(L, mgrid, st); }
    else { launch_shape<float, 64>(L, nw, depth, grid, lds, st); if (mgrid) launch_merge<float, 64>(L, mgrid, st); }
  }
}

int la_attention_launch(int dtype, const LaAttnArgs& a0, hipStream_t st) {
  LaAttnArgs a = a0;
  if (a.Q <= 0) return 0;
  if (!dh_supported(dtype, a.dh)) return -2;
  if (int rc = attn_prep(a)) return rc;
  const bool bf16 = dtype == LA_DT_BF16;
  const int rowb = a.dh * (bf16 ? 2 : 4);
  const int nw = pick_nw(&a, sizeof a, 1);
  a.rgroups = (attn_tiles(a) + nw - 1) / nw;
  a.wg_head = a.rgroups * a.nsplit;
  const size_t st_bytes = attn_stage(a, rowb);
  const int depth = ring_depth_for(bf16, nw, rowb, st_bytes);
  if (!depth) return -2;
  a.ring_depth = depth;
  const size_t lds = st_bytes + depth * 2 * (size_t)CH * rowb;
  const int kv = kv_slots(a.Hkv);
  const AttnLaunch L{&a, nullptr, 1, 0};
  launch_any(dtype, a.dh, L, nw, depth, kv * a.wg_head, lds, a.nsplit > 1 ? kv * merge_wpk(a, a.dh) : 0, st);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int la_attention_multi_plan(int dtype, LaAttnSeg* segs, int n, LaAttnMulti* m) {
  if (n <= 0 || !segs || !m) return -2;
  const int dh = segs[0].a.dh;
  if (!dh_supported(dtype, dh)) return -2;
  const bool bf16 = dtype == LA_DT_BF16;
  const int rowb = dh * (bf16 ? 2 : 4);
  for (int i = 0; i < n; ++i) {
    LaAttnArgs& a = segs[i].a;
    if (a.Q <= 0 || a.dh != dh) return -2;
    if (int rc = attn_prep(a)) return rc;
  }
  const int nw = pick_nw(&segs[0].a, sizeof(LaAttnSeg), n);
  size_t st_max = 0;
  for (int i = 0; i < n; ++i) {
    LaAttnArgs& a = segs[i].a;
    a.rgroups = (attn_tiles(a) + nw - 1) / nw;
    a.wg_head = a.rgroups * a.nsplit;
    st_max = std::max(st_max, attn_stage(a, rowb));
  }
  const int depth = ring_depth_for(bf16, nw, rowb, st_max);
  if (!depth) return -2;
  int grid = 0, mgrid = 0;
  for (int i = 0; i < n; ++i) {
    LaAttnArgs& a = segs[i].a;
    const int kv = kv_slots(a.Hkv);
    a.ring_depth = depth;
    segs[i].blk0 = grid;
    segs[i].mblk0 = mgrid;
    grid += kv * a.wg_head;
    if (a.nsplit > 1) mgrid += kv * merge_wpk(a, dh);
  }
  m->nw = nw;
  m->depth = depth;
  m->dh = dh;
  m->grid = grid;
  m->mgrid = mgrid;
  m->lds = st_max + depth * 2 * (size_t)CH * rowb;
  return 0;
}

int la_attention_multi_launch(int dtype, const LaAttnMulti& m, const LaAttnSeg* segs, int n, int layer,
                              hipStream_t st) {
  if (m.grid <= 0) return 0;
  if (!dh_supported(dtype, m.dh) || !segs || n <= 0) return -2;
  const AttnLaunch L{nullptr, segs, n, layer};
  launch_any(dtype, m.dh, L, m.nw, m.depth, m.grid, m.lds, m.mgrid, st);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}
