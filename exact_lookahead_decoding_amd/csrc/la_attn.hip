// Lookahead-mask attention over the committed prefix and the packed rows.
//
// "M7.3 - Lookahead Decoding", 0x04A / 0x04B / 0x07A: every packed row sees
// the whole committed prefix plus the rows of its own branch; an ordinary
// causal kernel cannot express this, and a dense additive mask costs
// B*H*Q*(K_in+Q) elements.  Here the mask never exists as a tensor: row i
// sees exactly logical positions 0 .. pos_i, position t taken from the
// cache when t < shared_end and through the row's branch path otherwise.
//
// Reduction tree (a function of logical positions only, so a row gets the
// same bits whether it is alone in an autoregressive step or packed with a
// whole lookahead round):
//   * keys are cut into chunks of 32 positions; chunk c belongs to class
//     c % 4;
//   * inside a class the chunks are taken in increasing position with the
//     online softmax: the chunk's exact maximum gives the new running maximum
//     m', the running sums are scaled by 2^(m - m'), p = 2^(s - m'),
//     l' = l * 2^(m - m') + sum p (fixed lane order), and O' = O * 2^(m - m')
//     + V^T P^T accumulated by MFMA over a fixed key -> slot assignment;
//   * the 4 class states are folded in class order (fold_state), then O / l.
//
// Work decomposition (gfx950, wave64; a wave owns one tile of 16 query rows
// of one q-head):
//   * class kernel: a workgroup (KV head, class, row group) of up to 8 tiles
//     streams its class's committed chunks once from HBM: K and V of a chunk
//     land in LDS through global_load_lds_dwordx4 (16-byte pieces XOR-swizzled
//     by row, so the QK and the PV fragment reads are bank-conflict free) in a
//     4-stage ring shared by all tiles of the workgroup; the row positions and
//     the tile's Q come in the same way, so the only waits are the ring's own;
//     each row's class state goes to the workspace;
//   * QK: S^T = K Q^T, 16x16x32 bf16 MFMA (16x16x4 fp32): one query row per
//     lane column, so the softmax statistics stay in-lane;
//   * PV: O^T += V^T P^T; output tile dt holds head dimensions NDT*m + dt, so
//     a lane reads NDT contiguous elements of each key row and transposes
//     them in registers; bf16 P enters as a hi + lo pair (fp32-level P);
//   * tail + merge kernel: one wave per tile folds the class states in order;
//     the class owning a chunk that reaches past shared_end (at most a few per
//     call) gets that chunk applied first, computed right there by gathering
//     each key's K/V row from the cache or, through the branch path, from the
//     packed rows' workspace, once per branch in the tile (rows of other
//     branches get p = 0 in that pass, which leaves their sums unchanged).
// The block -> work mapping keeps every class workgroup of one KV head on one
// XCD (blockIdx % 8), so the head's Q and the row groups' shared K/V chunks
// are fetched from HBM once.
#include <algorithm>
#include <type_traits>

#include "la_common.h"
#include "la_dev.h"
#include "la_kernels.h"

#define CH 32         // keys per chunk
#define NCLS 4        // chunk classes
#define NTAIL 4       // most chunks per call that reach past shared_end
#define TAIL_ROWS 128 // key rows the tail + merge kernel stages in LDS at once
#define NEG_INF (-__builtin_inff())



// Stages of the class workgroup's LDS ring: as many 2*CHB-byte stages as fit
// next to the Q tiles (at most 8), and no more than the vmcnt field (63) can
// wait on (CW DMA instructions per stage and wave).
constexpr int ring_depth(int chb, int tl, int rowb, int cw) {
  const int fit = (LDS_BYTES - tl * (16 * rowb + 256)) / (2 * chb);
  const int cnt = 1 + 63 / cw;
  const int d = fit < cnt ? fit : cnt;
  return d < 8 ? d : 8;
}


template <int W> struct alignas(4 * W) Words { uint32_t w[W]; };

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

// a*wa + b*wb as fma(a, wa, b*wb): the one rounding sequence of the class fold
__device__ __forceinline__ float lin2(float a, float wa, float b, float wb) {
#pragma clang fp contract(off)
  return __builtin_fmaf(a, wa, b * wb);
}

// MFMA k-slot e (0..7) of lane group g <-> key offset inside the chunk.
__device__ __forceinline__ int slot_key(int g, int e) { return 16 * (e >> 2) + 4 * g + (e & 3); }

template <typename T, int DH> struct AttnT;

template <int DH> struct AttnT<bf16_t, DH> {
  static constexpr int ROWB = DH * 2;         // bytes per key row
  static constexpr int PIECES = ROWB / 16;    // 16-byte pieces per row
  static constexpr int LP = PIECES / 4;       // pieces a lane group supplies for QK (one per MFMA step)
  static constexpr int NDT = DH / 16;         // output tiles
  static constexpr int VB = NDT * 2;          // bytes of one key row a lane supplies for PV
  typedef Words<VB / 4> VV;
  struct QF { u32x4 p[LP]; };
  static __device__ __forceinline__ f32x4 qk(const QF& k, const QF& q) {
    f32x4 acc = {0, 0, 0, 0};
#pragma unroll
    for (int s = 0; s < LP; ++s)
      acc = mfma_bf16_32(__builtin_bit_cast(bf16x8, k.p[s]), __builtin_bit_cast(bf16x8, q.p[s]), acc);
    return acc;
  }
  // P^T operand of one chunk: p of slot e as a hi + lo bf16 pair
  struct PP { bf16x8 hi, lo; };
  static __device__ __forceinline__ PP prep(const float* ps) {
    typedef float f2 __attribute__((ext_vector_type(2)));
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    uint32_t bh[4], bl[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f2 v = {ps[2 * j], ps[2 * j + 1]};
      const uint32_t hw = __builtin_bit_cast(uint32_t, __builtin_convertvector(v, b2));   // nearest even
      const f2 r = {v[0] - __uint_as_float(hw << 16), v[1] - __uint_as_float(hw & 0xffff0000u)};
      bh[j] = hw;
      bl[j] = __builtin_bit_cast(uint32_t, __builtin_convertvector(r, b2));
    }
    return PP{__builtin_bit_cast(bf16x8, bh), __builtin_bit_cast(bf16x8, bl)};
  }
  // o += V^T(dt) P^T over the chunk's 8 slots; vv[e] holds the lane's elements of slot e
  template <typename V>
  static __device__ __forceinline__ f32x4 pv(int dt, const V* vv, const PP& pp, f32x4 o) {
    uint32_t w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t lo = vv[2 * j].w[dt >> 1], hi = vv[2 * j + 1].w[dt >> 1];
      // element dt of key slot 2j (low half) and of key slot 2j + 1 (high half)
      w[j] = __builtin_amdgcn_perm(hi, lo, (dt & 1) ? 0x07060302u : 0x05040100u);
    }
    const bf16x8 A = __builtin_bit_cast(bf16x8, w);
    return mfma_bf16_32(A, pp.lo, mfma_bf16_32(A, pp.hi, o));
  }
};

template <int DH> struct AttnT<float, DH> {
  static constexpr int ROWB = DH * 4;
  static constexpr int PIECES = ROWB / 16;
  static constexpr int LP = PIECES / 4;       // pieces = 4*LP floats = DH/4 MFMA steps
  static constexpr int NDT = DH / 16;
  static constexpr int VB = NDT * 4;
  typedef Words<NDT> VV;
  struct QF { u32x4 p[LP]; };
  static __device__ __forceinline__ f32x4 qk(const QF& k, const QF& q) {
    f32x4 acc = {0, 0, 0, 0};
#pragma unroll
    for (int s = 0; s < LP; ++s) {
      acc = mfma_f32_4(__uint_as_float(k.p[s].x), __uint_as_float(q.p[s].x), acc);
      acc = mfma_f32_4(__uint_as_float(k.p[s].y), __uint_as_float(q.p[s].y), acc);
      acc = mfma_f32_4(__uint_as_float(k.p[s].z), __uint_as_float(q.p[s].z), acc);
      acc = mfma_f32_4(__uint_as_float(k.p[s].w), __uint_as_float(q.p[s].w), acc);
    }
    return acc;
  }
  struct PP { float p[8]; };
  static __device__ __forceinline__ PP prep(const float* ps) {
    PP r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r.p[e] = ps[e];
    return r;
  }
  template <typename V>
  static __device__ __forceinline__ f32x4 pv(int dt, const V* vv, const PP& pp, f32x4 o) {
#pragma unroll
    for (int e = 0; e < 8; ++e) o = mfma_f32_4(__uint_as_float(vv[e].w[dt]), pp.p[e], o);
    return o;
  }
};

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

// Rescale threshold of the running reference (log2 units): the reference m
// moves to a chunk's maximum only when that maximum exceeds it by more than
// this, so p = 2^(s - m) stays below 2^RESCALE and O is rarely rescaled.
#define RESCALE 8.0f

// Softmax half of one online chunk step for the lane's row.  s[e]: raw QK
// score of slot e (-inf: not visible).  Updates the reference m and l, leaves
// p in s and returns the factor the running O must be scaled by before P V is
// added.  A row that has seen no key yet keeps its state (factor 1, p = 0).
__device__ __forceinline__ float chunk_softmax(float (&s)[8], float sl2, float& m, float& l) {
  float mx = s[0];
#pragma unroll
  for (int e = 1; e < 8; ++e) mx = fmaxf(mx, s[e]);
  const float mc = row4_max(mx) * sl2;
  const float mn = (m == NEG_INF || mc > m + RESCALE) ? mc : m;
  const bool live = mn != NEG_INF;
  const float wa = (live && mn != m) ? ex2(m - mn) : 1.f;
  float ls = 0.f;
  if (__ballot(!live) == 0ull) {                  // every row has a visible key (the usual case)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float p = ex2(__builtin_fmaf(s[e], sl2, -mn));
      s[e] = p;
      ls += p;
    }
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float p = live ? ex2(__builtin_fmaf(s[e], sl2, -mn)) : 0.f;
      s[e] = p;
      ls += p;
    }
  }
  l = __builtin_fmaf(l, wa, row4_sum(ls));
  m = live ? mn : m;
  return wa;
}

template <int NDT> __device__ __forceinline__ void scale_o(f32x4* O, float wa) {
  if (__ballot(wa != 1.f) == 0ull) return;       // running maximum unchanged everywhere: O * 1 = O
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int r = 0; r < 4; ++r) O[dt][r] *= wa;
}

// Fold the class state (mb, lb, ob) into (ma, la, oa); an empty state has
// m = -inf (an empty ma gives wa = 2^-inf = 0).
template <int NDT>
__device__ __forceinline__ void fold_state(float& ma, float& la, f32x4* oa, float mb, float lb, const f32x4* ob) {
  if (mb == NEG_INF) return;
  const float mn = fmaxf(ma, mb);
  const float wa = ex2(ma - mn), wb = ex2(mb - mn);
  la = lin2(la, wa, lb, wb);
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int r = 0; r < 4; ++r) oa[dt][r] = lin2(oa[dt][r], wa, ob[dt][r], wb);
  ma = mn;
}


// Store one row's state.  The lane holds output tiles dt0 .. dt0 + NT - 1 of
// head dimension NDT*(4g + r) + dt; (m, l) is written by the owner of dt0 = 0.
template <int NDT, int NT>
__device__ __forceinline__ void store_state(float* po, float* pml, int g, int dt0, float m, float l, const f32x4* o) {
  if (g == 0 && dt0 == 0) *(float2*)pml = make_float2(m, l);
  if (m == NEG_INF) return;
  float* dst = po + 4 * NDT * g + dt0;
  if constexpr (NT % 4 == 0) {
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int q = 0; q < NT; q += 4)
        *(float4*)(dst + NDT * r + q) = make_float4(o[q][r], o[q + 1][r], o[q + 2][r], o[q + 3][r]);
  } else if constexpr (NT == 2) {
#pragma unroll
    for (int r = 0; r < 4; ++r) *(float2*)(dst + NDT * r) = make_float2(o[0][r], o[1][r]);
  } else {
    static_assert(NT == 1 && NDT == 1, "output tiles");
    *(float4*)dst = make_float4(o[0][0], o[0][1], o[0][2], o[0][3]);
  }
}

// Class workgroup: KV head g_kv, class cls, row group rg of TL tiles.  Its
// TL * DHS waves share one LDS ring: wave w owns tile w % TL and output tiles
// (head dimensions) slice w / TL of DHS; the DHS waves of a tile compute the
// same scores and softmax (the same bits) and each accumulates its slice of O.
template <typename T, int DH, int TL, int DHS>
__global__ void __launch_bounds__(64 * TL * DHS) la_attn_kernel(LaAttnArgs a) {
  typedef AttnT<T, DH> AT;
  typedef typename AT::QF QF;
  constexpr int NW = TL * DHS;
  constexpr int ROWB = AT::ROWB, PIECES = AT::PIECES, LP = AT::LP, NDT = AT::NDT, VB = AT::VB;
  constexpr int NT = NDT / DHS;                 // output tiles of a wave
  constexpr int VBW = VB / DHS;                 // bytes of one key row a wave's lane reads for PV
  static_assert(NDT % DHS == 0 && VBW % 4 == 0, "head-dimension split");
  typedef Words<VBW / 4> VV;
  constexpr int CHB = CH * ROWB;               // bytes of K (or V) of one chunk
  constexpr int NBLK = 2 * CHB / 1024;         // 1 KB DMA blocks per chunk, K then V
  constexpr int CW = NBLK >= NW ? NBLK / NW : 1;
  static_assert(NBLK % NW == 0 || NW > NBLK, "DMA blocks per wave");
  constexpr int DEPTH = ring_depth(CHB, TL, ROWB, CW);
  static_assert(DEPTH >= 2, "ring stages");
  // dynamic LDS: DEPTH ring stages of K and V, then each tile's Q, then each
  // tile's 16 row positions.  Every global load of this kernel is a DMA into
  // LDS read back with inline asm.
  extern __shared__ __attribute__((aligned(1024))) char lds[];

  // block -> (XCD, KV head, class, row group)
  const int xcd = blockIdx.x & 7, bi = blockIdx.x >> 3;
  const int hpx = (a.Hkv + 7) >> 3;
  const int rg = bi % a.rgroups;
  const int hl = (bi / a.rgroups) % hpx;
  const int cls = bi / (a.rgroups * hpx);
  const int g_kv = xcd + 8 * hl;
  if (g_kv >= a.Hkv || cls >= NCLS) return;
  const int n = a.class_last >= cls ? (a.class_last - cls) / NCLS + 1 : 0;
  if (n == 0) return;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int tslot = wave % TL, half = wave / TL;
  const int g = lane >> 4, c16 = lane & 15;
  const int se = a.shared_end;
  const float sl2 = a.scale_log2;
  const char* kc = (const char*)a.kc + (size_t)g_kv * a.T_cap * ROWB;
  const char* vc = (const char*)a.vc + (size_t)g_kv * a.T_cap * ROWB;

  // the wave's tile: 16 rows of q-head hh (rows past Q load row Q - 1 and stay unused)
  const int group = a.H / a.Hkv;
  const int rtiles = (a.Q + 15) >> 4;
  const int tile = rg * TL + tslot;
  const bool tv = tile < group * rtiles;
  const int hh = g_kv * group + (tv ? tile / rtiles : 0);
  const int row0 = (tv ? tile % rtiles : 0) * 16;
  const bool rvalid = tv && row0 + c16 < a.Q;
  char* const qa = lds + DEPTH * 2 * CHB + tslot * 16 * ROWB;
  char* const pa = lds + DEPTH * 2 * CHB + TL * 16 * ROWB + tslot * 256;
  constexpr int RPB = 1024 / ROWB;              // rows per 1 KB DMA block
  if (half == 0) {
    __builtin_amdgcn_global_load_lds((const void*)(a.pos + min(row0 + (lane & 15), a.Q - 1)), (lds_void_t*)pa, 4, 0,
                                     0);
#pragma unroll
    for (int j = 0; j < 16 / RPB; ++j) {
      const int r = min(row0 + j * RPB + lane / PIECES, a.Q - 1);
      const char* src = (const char*)a.q + ((size_t)r * a.H + hh) * ROWB + 16 * (lane % PIECES);
      __builtin_amdgcn_global_load_lds((const void*)src, (lds_void_t*)(qa + j * 1024), 16, 0, 0);
    }
  }

  // chunk k of the class into a ring stage.  Every step issues exactly one
  // stage, so the number of DMA operations in flight is the same on every path
  // and the waits are static; past the last chunk all lanes load one 16-byte
  // piece (a dummy that nobody reads).
  auto issue = [&](char* stage, int k) {
    const int c = cls + NCLS * k;
#pragma unroll
    for (int j = 0; j < CW; ++j) {
      const int b = wave + NW * j;
      if (b < NBLK) {
        const bool isv = b >= NBLK / 2;
        const int bb = isv ? b - NBLK / 2 : b;
        const int L = bb * 1024 + 16 * lane;
        const int r = L / ROWB, slot = (L % ROWB) / 16;
        const int piece = slot ^ (r % PIECES);
        const char* src = k < n ? (isv ? vc : kc) + (size_t)min(CH * c + r, se - 1) * ROWB + 16 * piece
                                : kc + (size_t)(se - 1) * ROWB;
        __builtin_amdgcn_global_load_lds((const void*)src, (lds_void_t*)(stage + (isv ? CHB : 0) + bb * 1024), 16,
                                         0, 0);
      }
    }
  };
#pragma unroll
  for (int k = 0; k < DEPTH; ++k) issue(lds + k * 2 * CHB, k);
  wait_vm<(CW * DEPTH < 63 ? CW * DEPTH : 63)>();  // this wave's Q and positions (issued first) have landed
  ring_barrier();                                   // ... and those of the other waves
  QF qf;
  int pos;
  {
    typename LdsT<16>::T qraw[LP];
    const uint32_t qaddr = lds_addr(qa + c16 * ROWB + 16 * LP * g);
    if constexpr (LP >= 1) qraw[0] = lds_read<16, 0>(qaddr);
    if constexpr (LP >= 2) qraw[1] = lds_read<16, 16>(qaddr);
    if constexpr (LP >= 3) qraw[2] = lds_read<16, 32>(qaddr);
    if constexpr (LP >= 4) qraw[3] = lds_read<16, 48>(qaddr);
    unsigned int praw[1] = {lds_read<4, 0>(lds_addr(pa + 4 * c16))};
    lds_wait(qraw);
    lds_wait(praw);
#pragma unroll
    for (int s = 0; s < LP; ++s) qf.p[s] = rvalid ? __builtin_bit_cast(u32x4, qraw[s]) : u32x4{0, 0, 0, 0};
    pos = rvalid ? (int)praw[0] : -1;
  }
  // smallest position among the wave's rows: chunks ending at or below it need no mask
  int pmin = rvalid ? pos : 0x7fffffff;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) pmin = min(pmin, __shfl_xor(pmin, o, 64));
  pmin = __builtin_amdgcn_readfirstlane(pmin);

  // lane parts of the fragment addresses (stage, group and slot-half offsets are immediates)
  uint32_t koff[LP], voff[4];
#pragma unroll
  for (int s = 0; s < LP; ++s) koff[s] = lds_addr(lds + c16 * ROWB + 16 * ((LP * g + s) ^ (c16 % PIECES)));
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int kk = 4 * g + e;                   // slot_key(g, e); slot e + 4 is 16 rows further
    const int off = VB * c16 + VBW * half;
    voff[e] = lds_addr(lds + CHB + kk * ROWB + 16 * ((off / 16) ^ (kk % PIECES)) + off % 16);
  }

  float M = NEG_INF, L = 0.f;
  f32x4 O[NT];
#pragma unroll
  for (int dt = 0; dt < NT; ++dt) O[dt] = f32x4{0, 0, 0, 0};

  auto step = [&](auto SI, int k) {
    constexpr int S = decltype(SI)::value;
    constexpr int SB = S * 2 * CHB;             // stage base
    constexpr int SBH = SB & ~65535, SBL = SB & 65535;   // ds offsets reach 64 KB
    wait_vm<CW * (DEPTH - 1)>();                // chunk k landed (DEPTH - 1 later stages may be in flight)
    ring_barrier();
    if (k < n) {
      const int x0 = CH * (cls + NCLS * k);
      typename LdsT<16>::T kraw[2 * LP];
#pragma unroll
      for (int s = 0; s < LP; ++s) {
        kraw[s] = lds_read<16, SBL>(koff[s] + SBH);
        kraw[LP + s] = lds_read<16, SBL + 16 * ROWB>(koff[s] + SBH);
      }
      typename LdsT<VBW>::T vraw[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        vraw[e] = lds_read<VBW, SBL>(voff[e] + SBH);
        vraw[e + 4] = lds_read<VBW, SBL + 16 * ROWB>(voff[e] + SBH);
      }
      lds_wait(kraw);
      float sc[8];
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        QF kf;
#pragma unroll
        for (int s = 0; s < LP; ++s) kf.p[s] = __builtin_bit_cast(u32x4, kraw[LP * jj + s]);
        const f32x4 s4 = AT::qk(kf, qf);
#pragma unroll
        for (int r = 0; r < 4; ++r) sc[4 * jj + r] = s4[r];
      }
      if (x0 + CH - 1 > pmin) {                 // some key of the chunk lies past some row
#pragma unroll
        for (int e = 0; e < 8; ++e) sc[e] = x0 + slot_key(g, e) <= pos ? sc[e] : NEG_INF;
      }
      const float wa = chunk_softmax(sc, sl2, M, L);
      lds_wait(vraw);
      VV vv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) vv[e] = __builtin_bit_cast(VV, vraw[e]);
      ring_barrier();                           // every wave has read the stage
      scale_o<NT>(O, wa);
      const typename AT::PP pp = AT::prep(sc);
#pragma unroll
      for (int dt = 0; dt < NT; ++dt) O[dt] = AT::pv(dt, vv, pp, O[dt]);
      issue(lds + SB, k + DEPTH);
    } else {                                    // past the last chunk: keep the DMA rhythm only
      ring_barrier();
      issue(lds + SB, k + DEPTH);
    }
  };
  for (int k0 = 0; k0 < n; k0 += DEPTH)
    static_for<0, DEPTH>([&](auto SI) { step(SI, k0 + decltype(SI)::value); });
  wait_vm<0>();                                   // no DMA may land after the workgroup has left
  if (rvalid) {
    const size_t base = ((size_t)cls * a.H + hh) * a.Q + row0 + c16;
    store_state<NDT, NT>(a.part_o + base * DH, a.part_ml + base * 2, g, half * NT, M, L, O);
  }
}

// Chunks that reach past shared_end and the final fold.  One wave per tile of
// 16 rows: for each class it takes the class state, applies the class's tail
// chunk with the online step (computed here from the tile's tail keys, staged
// in LDS: each lane reads its key's K/V row through the branch path, once per
// branch present in the tile), folds the classes in order and stores O / l.
template <typename T, int DH>
__global__ void __launch_bounds__(64) la_attn_tail_merge_kernel(LaAttnArgs a) {
  typedef AttnT<T, DH> AT;
  typedef typename AT::QF QF;
  typedef typename AT::VV VV;
  constexpr int ROWB = AT::ROWB, LP = AT::LP, NDT = AT::NDT, VB = AT::VB;
  __shared__ int spath[16][64];                 // the tile's branches: workspace row of position shared_end + e
  extern __shared__ __attribute__((aligned(1024))) char tls[];   // staged tail K rows, then V rows
  const int lane = threadIdx.x, g = lane >> 4, c16 = lane & 15;
  const int group = a.H / a.Hkv;
  const int rtiles = (a.Q + 15) >> 4;
  const int tiles_kv = group * rtiles;
  const int g_kv = blockIdx.x / tiles_kv;
  if (g_kv >= a.Hkv) return;
  const int tile = blockIdx.x % tiles_kv;
  const int hh = g_kv * group + tile / rtiles;
  const int row = (tile % rtiles) * 16 + c16;
  const bool rvalid = row < a.Q;
  const int se = a.shared_end;
  const float sl2 = a.scale_log2;

  // class states of the lane's row, all loads issued up front
  float cm[NCLS], cl[NCLS];
  f32x4 co[NCLS][NDT];
#pragma unroll
  for (int cls = 0; cls < NCLS; ++cls) {
    cm[cls] = NEG_INF;
    cl[cls] = 0.f;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) co[cls][dt] = f32x4{0, 0, 0, 0};
    if (cls <= a.class_last && rvalid) {
      const size_t base = ((size_t)cls * a.H + hh) * a.Q + row;
      const float2 ml = *(const float2*)(a.part_ml + base * 2);
      cm[cls] = ml.x;
      cl[cls] = ml.y;
      const float* src = a.part_o + base * DH + 4 * NDT * g;
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) co[cls][dt][r] = src[NDT * r + dt];
    }
  }

  if (a.n_tail > 0) {
    const int pos = rvalid ? a.pos[row] : -1;
    const int br = rvalid ? a.branch[row] : -1;
    const char* kc = (const char*)a.kc + (size_t)g_kv * a.T_cap * ROWB;
    const char* vc = (const char*)a.vc + (size_t)g_kv * a.T_cap * ROWB;
    const char* kw = (const char*)a.kw + (size_t)g_kv * a.ws_cap * ROWB;
    const char* vw = (const char*)a.vw + (size_t)g_kv * a.ws_cap * ROWB;
    QF qf;
    {
      const char* qrow = (const char*)a.q + ((size_t)(rvalid ? row : 0) * a.H + hh) * ROWB + 16 * LP * g;
#pragma unroll
      for (int s = 0; s < LP; ++s) qf.p[s] = rvalid ? *(const u32x4*)(qrow + 16 * s) : u32x4{0, 0, 0, 0};
    }
    // the tile's branches that reach a tail chunk (at most 16 rows, so at most 16)
    const bool need0 = rvalid && pos >= CH * a.tail0;
    int nbr = 0;
    int bl = -1;                                  // lane i < nbr: branch i
    unsigned long long pend = __ballot(need0 && g == 0);
    while (pend) {
      const int b = __builtin_amdgcn_readfirstlane(__shfl(br, __ffsll((long long)pend) - 1, 64));
      pend &= ~__ballot(need0 && g == 0 && br == b);
      if (lane == nbr) bl = b;
      ++nbr;
    }
    // their paths into LDS: spath[i][e] = workspace row of position se + e on
    // branch i, -1 when that position is not on the path.  Lane i reads branch
    // i's path length, then every lane reads entry e = lane of every branch
    // (all loads of a round issued together)
    const int plen = lane < nbr ? min(a.path_len[bl], a.maxp) : 0;
    int wv[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int b = __shfl(bl, i, 64), pl = __shfl(plen, i, 64);
      wv[i] = (i < nbr && lane < pl) ? a.path[(size_t)b * a.maxp + lane] : -1;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (i < nbr) spath[i][lane] = (unsigned)wv[i] < (unsigned)a.n_ws ? wv[i] : -1;
    __syncthreads();
    // The tail keys of the tile's branches are gathered into LDS with one round
    // of DMA (16-byte pieces XOR-swizzled by staged row): first the committed
    // rows [X0, se) shared by every branch, then EP rows per branch for the
    // positions se .. max_pos (a clamped committed row where a position is not
    // on the branch's path; it is never visible to the branch's rows).
    const int X0 = CH * a.tail0;
    const int ncom = se - X0;                       // 0 .. 31
    const int EP = a.max_pos - se + 1;              // 1 .. 63
    const int bb = min(nbr, (TAIL_ROWS - ncom) / EP);   // branches staged at once (>= 1)
    constexpr int RPB = 1024 / ROWB, PIECES = AT::PIECES;
    char* const ks = tls;
    char* const vs = tls + TAIL_ROWS * ROWB;
    auto stage = [&](int i0, int nb) {
      const int nr = ncom + nb * EP;
      for (int blk = 0; blk * RPB < nr; ++blk) {
        const int j = blk * RPB + lane / PIECES;
        const int piece = (lane % PIECES) ^ (j % PIECES);
        int crow = se - 1, wrow = -1;
        if (j < ncom) crow = X0 + j;
        else if (j < nr) wrow = spath[i0 + (j - ncom) / EP][(j - ncom) % EP];
        const size_t off = (size_t)(wrow >= 0 ? wrow : crow) * ROWB + 16 * piece;
        __builtin_amdgcn_global_load_lds((const void*)((wrow >= 0 ? kw : kc) + off), (lds_void_t*)(ks + blk * 1024), 16,
                                         0, 0);
        __builtin_amdgcn_global_load_lds((const void*)((wrow >= 0 ? vw : vc) + off), (lds_void_t*)(vs + blk * 1024), 16,
                                         0, 0);
      }
      wait_vm<0>();
    };
    // staged row of key x on batch branch bi (x >= X0)
    auto srow = [&](int x, int bi) -> int {
      if (x < se) return x - X0;
      const int e = x - se;
      return e < EP ? ncom + bi * EP + e : 0;
    };
    const bool one = nbr <= bb;
    if (one) stage(0, nbr);
    // the online step of tail chunk x0 on top of a class state (m, l, o)
    auto tail_step = [&](int x0, float& m, float& l, f32x4* o) {
      const bool need = rvalid && pos >= x0;
      if (__ballot(need) == 0ull) return;
      float sc[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) sc[e] = NEG_INF;
      for (int i0 = 0; i0 < nbr; i0 += bb) {
        const int nb = min(bb, nbr - i0);
        if (!one) stage(i0, nb);
        for (int bi = 0; bi < nb; ++bi) {
          const int b = __shfl(bl, i0 + bi, 64);
          const bool mine = need && br == b;
          if (__ballot(mine) == 0ull) continue;
#pragma unroll
          for (int jj = 0; jj < 2; ++jj) {
            const int r = srow(x0 + 16 * jj + c16, bi);
            QF kf;
#pragma unroll
            for (int s = 0; s < LP; ++s) kf.p[s] = *(const u32x4*)(ks + r * ROWB + 16 * ((LP * g + s) ^ (r % PIECES)));
            const f32x4 s4 = AT::qk(kf, qf);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const float v = (x0 + 16 * jj + 4 * g + q <= pos) ? s4[q] : NEG_INF;
              sc[4 * jj + q] = mine ? v : sc[4 * jj + q];
            }
          }
        }
      }
      // softmax part and rescale, then P V once per branch (the other rows add exact zeros)
      const float wa = chunk_softmax(sc, sl2, m, l);
      scale_o<NDT>(o, wa);
      for (int i0 = 0; i0 < nbr; i0 += bb) {
        const int nb = min(bb, nbr - i0);
        if (!one) stage(i0, nb);
        for (int bi = 0; bi < nb; ++bi) {
          const int b = __shfl(bl, i0 + bi, 64);
          const bool mine = need && br == b;
          if (__ballot(mine) == 0ull) continue;
          VV vv[8];
          float ps[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int r = srow(x0 + slot_key(g, e), bi);
            const int off = VB * c16;
            vv[e] = *(const VV*)(vs + r * ROWB + 16 * ((off / 16) ^ (r % PIECES)) + off % 16);
            ps[e] = mine ? sc[e] : 0.f;
          }
          const typename AT::PP pp = AT::prep(ps);
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) o[dt] = AT::pv(dt, vv, pp, o[dt]);
        }
      }
    };
    // each tail chunk belongs to its own class (at most NCLS of them)
#pragma unroll
    for (int cls = 0; cls < NCLS; ++cls) {
      const int tau = (cls - a.tail0 % NCLS + NCLS) % NCLS;
      if (tau < a.n_tail) tail_step(CH * (a.tail0 + tau), cm[cls], cl[cls], co[cls]);
    }
  }

  float M = NEG_INF, L = 0.f;
  f32x4 O[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) O[dt] = f32x4{0, 0, 0, 0};
#pragma unroll
  for (int cls = 0; cls < NCLS; ++cls) fold_state<NDT>(M, L, O, cm[cls], cl[cls], co[cls]);
  if (rvalid) {
    // lane holds head dimensions NDT*(4g + r) + dt: 4*NDT contiguous values
    T* dst = (T*)a.o + ((size_t)row * a.H + hh) * DH + 4 * NDT * g;
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) st<T>(dst + NDT * r + dt, O[dt][r] / L);
  }
}

int la_attention_parts() { return NCLS; }

template <typename T, int DH, int TL, int DHS>
static void launch_cls(const LaAttnArgs& a, int grid, hipStream_t st) {
  constexpr int ROWB = AttnT<T, DH>::ROWB;
  constexpr int NBLK = 2 * CH * ROWB / 1024, NW = TL * DHS;
  constexpr int DEPTH = ring_depth(CH * ROWB, TL, ROWB, NBLK >= NW ? NBLK / NW : 1);
  constexpr size_t lds = (size_t)DEPTH * 2 * CH * ROWB + (size_t)TL * 16 * ROWB + (size_t)TL * 256;
  static_assert(lds <= LDS_BYTES, "LDS");
  static const bool attr = hipFuncSetAttribute((const void*)&la_attn_kernel<T, DH, TL, DHS>,
                                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) == hipSuccess;
  (void)attr;
  hipLaunchKernelGGL((la_attn_kernel<T, DH, TL, DHS>), dim3(grid), dim3(64 * TL * DHS), lds, st, a);
}

template <typename T, int DH>
static void launch_dh(LaAttnArgs a, hipStream_t st) {
  constexpr int NDT = AttnT<T, DH>::NDT;
  const int group = a.H / a.Hkv;
  const int tiles = group * ((a.Q + 15) / 16);
  // tiles per class workgroup: at most 8, fewer while that keeps the grid under
  // 256 workgroups; with 4 tiles or fewer each tile gets two waves (two halves
  // of the head dimensions) so that every SIMD has two waves to interleave
  int tl = 8;
  while (tl > 1 && (tl / 2 >= tiles || a.Hkv * NCLS * ((tiles + tl - 1) / tl) < 256)) tl /= 2;
  a.rgroups = (tiles + tl - 1) / tl;
  if (a.class_last >= 0) {
    const int hpx = (a.Hkv + 7) / 8;
    const int grid = 8 * hpx * NCLS * a.rgroups;
    if constexpr (NDT % 2 == 0) {
      switch (tl) {
        case 8: launch_cls<T, DH, 8, 1>(a, grid, st); break;
        case 4: launch_cls<T, DH, 4, 2>(a, grid, st); break;
        case 2: launch_cls<T, DH, 2, 2>(a, grid, st); break;
        default: launch_cls<T, DH, 1, 2>(a, grid, st); break;
      }
    } else {
      switch (tl) {
        case 8: launch_cls<T, DH, 8, 1>(a, grid, st); break;
        case 4: launch_cls<T, DH, 4, 1>(a, grid, st); break;
        case 2: launch_cls<T, DH, 2, 1>(a, grid, st); break;
        default: launch_cls<T, DH, 1, 1>(a, grid, st); break;
      }
    }
  }
  constexpr size_t tlds = (size_t)2 * TAIL_ROWS * AttnT<T, DH>::ROWB;
  static const bool tattr = hipFuncSetAttribute((const void*)&la_attn_tail_merge_kernel<T, DH>,
                                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)tlds) == hipSuccess;
  (void)tattr;
  hipLaunchKernelGGL((la_attn_tail_merge_kernel<T, DH>), dim3(a.Hkv * tiles), dim3(64), a.n_tail > 0 ? tlds : 0, st,
                     a);
}

int la_attention_launch(int dtype, const LaAttnArgs& a0, hipStream_t st) {
  LaAttnArgs a = a0;
  if (a.Q <= 0) return 0;
  if (a.H % a.Hkv != 0 || a.shared_end < 1 || a.shared_end > a.T_cap) return -2;
  if (a.n_ws < 0 || a.n_ws > a.ws_cap || a.maxp < 1) return -2;
  const int se = a.shared_end;
  const bool tail = a.max_pos >= se;
  a.class_last = tail ? se / CH - 1 : a.max_pos / CH;
  a.tail0 = se / CH;
  a.n_tail = tail ? a.max_pos / CH - se / CH + 1 : 0;
  // tail positions are read through a 64-entry path table per branch
  if (a.n_tail > NTAIL || (tail && a.max_pos - se >= 64)) return -2;
  a.scale_log2 = a.scale * 1.4426950408889634f;
  if (dtype == LA_DT_BF16) {
    if (a.dh == 128) launch_dh<bf16_t, 128>(a, st);
    else if (a.dh == 64) launch_dh<bf16_t, 64>(a, st);
    else return -2;
  } else {
    if (a.dh == 16) launch_dh<float, 16>(a, st);
    else if (a.dh == 64) launch_dh<float, 64>(a, st);
    else return -2;
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}
