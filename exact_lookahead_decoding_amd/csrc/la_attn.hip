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
//     c % 8;
//   * every chunk yields its own softmax state for the row: exact chunk
//     maximum m, p = 2^(s - m), l = sum p in a fixed lane order, and
//     O = sum p v from MFMA with a fixed key -> slot assignment;
//   * inside a class the chunk states are folded in increasing position,
//     then the 8 class states are folded in class order, then O / l.
// The fold is one function (no contraction), so it gives the same bits
// whichever kernel applies it.
//
// Work decomposition (gfx950, wave64; a wave owns one tile of 16 query
// rows of one q-head):
//   * class kernel: a workgroup (KV head, class, row group) of up to 8 tiles
//     streams its class's committed chunks once from HBM: K and V of a chunk
//     land in LDS through global_load_lds_dwordx4 (16-byte pieces
//     XOR-swizzled by row, so the QK and the PV fragment reads are bank
//     conflict free) in a 4-stage ring shared by all tiles of the workgroup;
//     each row's class state goes to the workspace;
//   * QK: S^T = K Q^T, 16x16x32 bf16 MFMA (16x16x4 fp32): one query row per
//     lane column, so the softmax statistics stay in-lane;
//   * PV: V^T P^T; output tile dt holds head dimensions NDT*m + dt, so a
//     lane reads NDT contiguous elements of each key row and transposes them
//     in registers; bf16 P enters as a hi + lo pair (fp32-level P);
//   * tail + merge kernel: one wave per tile folds the class states in
//     order; the class of a chunk that reaches past shared_end (at most a
//     few per call) gets that chunk folded in first, computed right there by
//     gathering each key's K/V row from the cache or, through the branch
//     path, from the packed rows' workspace, once per branch in the tile.
// The block -> work mapping keeps every class workgroup of one KV head on
// one XCD (blockIdx % 8), so a head's Q is fetched from HBM once.
#include <algorithm>

#include "la_common.h"
#include "la_kernels.h"

#define CH 32         // keys per chunk
#define NCLS 8        // chunk classes
#define NTAIL 4       // most tail chunks per call
#define DEPTH 4       // LDS ring stages of a class workgroup
#define NEG_INF (-__builtin_inff())

typedef __attribute__((address_space(3))) void lds_void_t;

template <int W> struct alignas(4 * W) Words { uint32_t w[W]; };

// a*wa + b*wb as fma(a, wa, b*wb): the one rounding sequence every fold
// of softmax states uses.
__device__ __forceinline__ float lin2(float a, float wa, float b, float wb) {
#pragma clang fp contract(off)
  return __builtin_fmaf(a, wa, b * wb);
}

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

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
      const b2 h = __builtin_convertvector(v, b2);          // round to nearest even
      const uint32_t hw = __builtin_bit_cast(uint32_t, h);
      const f2 r = {v[0] - __uint_as_float(hw << 16), v[1] - __uint_as_float(hw & 0xffff0000u)};
      bh[j] = hw;
      bl[j] = __builtin_bit_cast(uint32_t, __builtin_convertvector(r, b2));
    }
    return PP{__builtin_bit_cast(bf16x8, bh), __builtin_bit_cast(bf16x8, bl)};
  }
  // output tile dt of V^T P^T over the chunk, from zero
  static __device__ __forceinline__ f32x4 pv(int dt, const VV* vv, const PP& pp) {
    uint32_t w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t lo = vv[2 * j].w[dt >> 1], hi = vv[2 * j + 1].w[dt >> 1];
      w[j] = (dt & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
    }
    const bf16x8 A = __builtin_bit_cast(bf16x8, w);
    const f32x4 acc = mfma_bf16_32(A, pp.hi, f32x4{0, 0, 0, 0});
    return mfma_bf16_32(A, pp.lo, acc);
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
  static __device__ __forceinline__ f32x4 pv(int dt, const VV* vv, const PP& pp) {
    f32x4 o = {0, 0, 0, 0};
#pragma unroll
    for (int e = 0; e < 8; ++e) o = mfma_f32_4(__uint_as_float(vv[e].w[dt]), pp.p[e], o);
    return o;
  }
};

// Chunk softmax of one row from its 8 in-lane scores (log2 units, -inf =
// not visible): exact maximum m, p = 2^(s - m) in place, l = sum p.
__device__ __forceinline__ void chunk_softmax(float (&sc)[2][4], float& m, float& l) {
  float mx = NEG_INF;
#pragma unroll
  for (int jj = 0; jj < 2; ++jj)
#pragma unroll
    for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sc[jj][r]);
  mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
  mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
  float ls = 0.f;
#pragma unroll
  for (int jj = 0; jj < 2; ++jj)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float p = sc[jj][r] == NEG_INF ? 0.f : ex2(sc[jj][r] - mx);
      sc[jj][r] = p;
      ls += p;
    }
  ls += __shfl_xor(ls, 16, 64);
  ls += __shfl_xor(ls, 32, 64);
  m = mx;
  l = ls;
}

// Fold the state (mb, lb, ob) into (ma, la, oa); an empty state has m = -inf
// (an empty ma gives wa = 2^-inf = 0).
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

template <int N> __device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// Workgroup barrier that leaves outstanding global loads in flight (the
// ring waits for its own stages with wait_vm): LDS reads of this wave are
// complete before the barrier, and the compiler may not move memory
// accesses across it.
__device__ __forceinline__ void ring_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// LDS reads of the ring stages are issued as inline asm: the compiler then
// sees no LDS load that could alias an in-flight stage DMA (it would wait for
// all of them), and the ring's own waits order everything.  lds_wait() waits
// for every outstanding LDS read and ties the values to the wait.
template <int B> struct LdsT;
template <> struct LdsT<16> { typedef uint32_t T __attribute__((ext_vector_type(4))); };
template <> struct LdsT<8> { typedef uint32_t T __attribute__((ext_vector_type(2))); };
template <> struct LdsT<4> { typedef uint32_t T; };
template <int B> __device__ __forceinline__ typename LdsT<B>::T lds_read(const char* p) {
  typename LdsT<B>::T v;
  const uint32_t a = (uint32_t)(uintptr_t)p;        // low half of a flat LDS address = LDS offset
  if constexpr (B == 16) asm volatile("ds_read_b128 %0, %1" : "=v"(v) : "v"(a));
  else if constexpr (B == 8) asm volatile("ds_read_b64 %0, %1" : "=v"(v) : "v"(a));
  else asm volatile("ds_read_b32 %0, %1" : "=v"(v) : "v"(a));
  return v;
}
template <typename T, int N> __device__ __forceinline__ void lds_wait(T (&v)[N]) {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
  for (int i = 0; i < N; ++i) asm volatile("" : "+v"(v[i]));
}

// Store one row's state: O^T tiles hold head dimension NDT*(4g + r) + dt.
template <int NDT>
__device__ __forceinline__ void store_state(float* po, float* pml, int g, float m, float l, const f32x4* o) {
  if (g == 0) *(float2*)pml = make_float2(m, l);
  if (m == NEG_INF) return;
  float* dst = po + 4 * NDT * g;
  if constexpr (NDT % 4 == 0) {
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int q = 0; q < NDT; q += 4)
        *(float4*)(dst + NDT * r + q) = make_float4(o[q][r], o[q + 1][r], o[q + 2][r], o[q + 3][r]);
  } else {
    static_assert(NDT == 1, "head dimension");
    *(float4*)dst = make_float4(o[0][0], o[0][1], o[0][2], o[0][3]);
  }
}

// Tile of 16 query rows of one q-head owned by a wave: lane (g, c16) holds row c16.
struct TileRows {
  int hh, row, pos;
  bool valid;
};
__device__ __forceinline__ TileRows tile_rows(const LaAttnArgs& a, int g_kv, int tile, int c16) {
  const int group = a.H / a.Hkv;
  const int rtiles = (a.Q + 15) >> 4;
  const bool tv = tile < group * rtiles;
  TileRows t;
  t.hh = g_kv * group + (tv ? tile / rtiles : 0);
  t.row = (tv ? tile % rtiles : 0) * 16 + c16;
  t.valid = tv && t.row < a.Q;
  t.pos = t.valid ? a.pos[t.row] : -1;
  return t;
}

template <typename QF, int LP>
__device__ __forceinline__ QF load_q(const LaAttnArgs& a, const TileRows& t, int g, int rowb) {
  QF qf;
  const char* qrow = (const char*)a.q + ((size_t)t.row * a.H + t.hh) * rowb + 16 * LP * g;
#pragma unroll
  for (int s = 0; s < LP; ++s) qf.p[s] = t.valid ? *(const u32x4*)(qrow + 16 * s) : u32x4{0, 0, 0, 0};
  return qf;
}

// Class workgroup: KV head g_kv, class cls, row group rg.  Streams the class's
// committed chunks through the LDS ring and leaves each row's class state.
template <typename T, int DH, int NW>
__global__ void __launch_bounds__(64 * NW) la_attn_kernel(LaAttnArgs a) {
  typedef AttnT<T, DH> AT;
  typedef typename AT::QF QF;
  typedef typename AT::VV VV;
  constexpr int ROWB = AT::ROWB, PIECES = AT::PIECES, LP = AT::LP, NDT = AT::NDT, VB = AT::VB;
  constexpr int CHB = CH * ROWB;               // bytes of K (or V) of one chunk
  constexpr int NBLK = 2 * CHB / 1024;         // 1 KB DMA blocks per chunk, K then V
  constexpr int CW = NBLK >= NW ? NBLK / NW : 1;
  static_assert(NBLK % NW == 0 || NW > NBLK, "DMA blocks per wave");
  // dynamic LDS: DEPTH ring stages of K and V, then each wave's Q tile, then
  // each wave's 16 row positions.  Every global load of this kernel is a DMA
  // into LDS read back with inline asm, so the only waits are the ring's own.
  extern __shared__ __attribute__((aligned(1024))) char lds[];
  char* const st0 = lds;
  char* const st1 = lds + 2 * CHB;
  char* const st2 = lds + 4 * CHB;
  char* const st3 = lds + 6 * CHB;
  static_assert(DEPTH == 4, "ring stages");

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
  const int g = lane >> 4, c16 = lane & 15;
  const int se = a.shared_end;
  const float sl2 = a.scale_log2;
  const char* kc = (const char*)a.kc + (size_t)g_kv * a.T_cap * ROWB;
  const char* vc = (const char*)a.vc + (size_t)g_kv * a.T_cap * ROWB;

  // the wave's tile: 16 rows of q-head hh (rows past Q load row Q - 1 and stay unused)
  const int group = a.H / a.Hkv;
  const int rtiles = (a.Q + 15) >> 4;
  const int tile = rg * NW + wave;
  const bool tv = tile < group * rtiles;
  const int hh = g_kv * group + (tv ? tile / rtiles : 0);
  const int row0 = (tv ? tile % rtiles : 0) * 16;
  const bool rvalid = tv && row0 + c16 < a.Q;
  char* const qa = lds + DEPTH * 2 * CHB + wave * 16 * ROWB;
  char* const pa = lds + DEPTH * 2 * CHB + NW * 16 * ROWB + wave * 256;
  __builtin_amdgcn_global_load_lds((const void*)(a.pos + min(row0 + (lane & 15), a.Q - 1)), (lds_void_t*)pa, 4, 0, 0);
  constexpr int RPB = 1024 / ROWB;              // rows per 1 KB DMA block
#pragma unroll
  for (int j = 0; j < 16 / RPB; ++j) {
    const int r = min(row0 + j * RPB + lane / PIECES, a.Q - 1);
    const char* src = (const char*)a.q + ((size_t)r * a.H + hh) * ROWB + 16 * (lane % PIECES);
    __builtin_amdgcn_global_load_lds((const void*)src, (lds_void_t*)(qa + j * 1024), 16, 0, 0);
  }

  QF qf;
  int pos = -1, pmin = 0;

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

  float M = NEG_INF, L = 0.f;
  f32x4 O[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) O[dt] = f32x4{0, 0, 0, 0};

  auto step = [&](char* sk, int k) {
    wait_vm<CW * (DEPTH - 1)>();                // chunk k landed (DEPTH - 1 later stages may be in flight)
    ring_barrier();
    if (k >= n) {                                 // past the last chunk: keep the DMA rhythm only
      ring_barrier();
      issue(sk, k + DEPTH);
      return;
    }
    const char* sv = sk + CHB;
    const int x0 = CH * (cls + NCLS * k);
    const bool full = x0 + CH - 1 <= pmin;      // every key of the chunk visible to every row
    typedef typename LdsT<16>::T R16;
    R16 kraw[2 * LP];
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      const int kr = 16 * jj + c16;
#pragma unroll
      for (int s = 0; s < LP; ++s) kraw[LP * jj + s] = lds_read<16>(sk + kr * ROWB + 16 * ((LP * g + s) ^ (kr % PIECES)));
    }
    lds_wait(kraw);
    float sc[2][4];
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      QF kf;
#pragma unroll
      for (int s = 0; s < LP; ++s) kf.p[s] = __builtin_bit_cast(u32x4, kraw[LP * jj + s]);
      const f32x4 s4 = AT::qk(kf, qf);
#pragma unroll
      for (int r = 0; r < 4; ++r)
        sc[jj][r] = (full || x0 + 16 * jj + 4 * g + r <= pos) ? s4[r] * sl2 : NEG_INF;
    }
    typedef typename LdsT<VB>::T RV;
    RV vraw[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int kk = slot_key(g, e);
      const int off = VB * c16;
      vraw[e] = lds_read<VB>(sv + kk * ROWB + 16 * ((off / 16) ^ (kk % PIECES)) + off % 16);
    }
    float mc, lc;
    chunk_softmax(sc, mc, lc);
    float ps[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) ps[e] = sc[e >> 2][e & 3];
    lds_wait(vraw);
    VV vv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) vv[e] = __builtin_bit_cast(VV, vraw[e]);
    ring_barrier();
    issue(sk, k + DEPTH);
    // fold the chunk state into the running state with fold_state's arithmetic,
    // one output tile at a time; MFMA runs for the whole wave, so rows without
    // a visible key keep their state through selects
    const bool has = mc != NEG_INF;
    const unsigned long long hv = __ballot(has);
    if (hv != 0ull) {
      const typename AT::PP pp = AT::prep(ps);
      const float mn = fmaxf(M, mc);
      const float wa = ex2(M - mn), wb = ex2(mc - mn);
      if (__ballot(has || !rvalid) == ~0ull) {
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const f32x4 oc = AT::pv(dt, vv, pp);
#pragma unroll
          for (int r = 0; r < 4; ++r) O[dt][r] = lin2(O[dt][r], wa, oc[r], wb);
        }
        L = lin2(L, wa, lc, wb);
        M = mn;
      } else {
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const f32x4 oc = AT::pv(dt, vv, pp);
#pragma unroll
          for (int r = 0; r < 4; ++r) O[dt][r] = has ? lin2(O[dt][r], wa, oc[r], wb) : O[dt][r];
        }
        L = has ? lin2(L, wa, lc, wb) : L;
        M = has ? mn : M;
      }
    }
  };

  issue(st0, 0);
  issue(st1, 1);
  issue(st2, 2);
  issue(st3, 3);
  wait_vm<(CW * DEPTH < 63 ? CW * DEPTH : 63)>();  // the row positions and Q (issued first) have landed
  {
    typename LdsT<16>::T qraw[LP];
#pragma unroll
    for (int s = 0; s < LP; ++s) qraw[s] = lds_read<16>(qa + c16 * ROWB + 16 * (LP * g + s));
    unsigned int praw[1] = {lds_read<4>(pa + 4 * c16)};
    lds_wait(qraw);
    lds_wait(praw);
#pragma unroll
    for (int s = 0; s < LP; ++s) qf.p[s] = rvalid ? __builtin_bit_cast(u32x4, qraw[s]) : u32x4{0, 0, 0, 0};
    pos = rvalid ? (int)praw[0] : -1;
  }
  // smallest position among the wave's rows: chunks ending at or below it need no mask
  pmin = rvalid ? pos : 0x7fffffff;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) pmin = min(pmin, __shfl_xor(pmin, o, 64));
  for (int k0 = 0; k0 < n; k0 += DEPTH) {
    step(st0, k0);
    step(st1, k0 + 1);
    step(st2, k0 + 2);
    step(st3, k0 + 3);
  }
  wait_vm<0>();                                   // no DMA may land after the workgroup has left
  if (rvalid) {
    const size_t base = ((size_t)cls * a.H + hh) * a.Q + row0 + c16;
    store_state<NDT>(a.part_o + base * DH, a.part_ml + base * 2, g, M, L, O);
  }
}

// Chunks that reach past shared_end (at most NTAIL per call) and the final
// fold.  A wave owns one tile of 16 rows: for class 0..7 it takes the class
// state, folds in the class's tail chunk (computed here: each lane gathers its
// key's K/V row from the cache or, through the branch path, from the
// workspace, once per branch present in the tile; rows of other branches get
// p = 0 in that pass), folds the class into the total, and finally stores
// O / l.
template <typename T, int DH>
__global__ void __launch_bounds__(256) la_attn_tail_merge_kernel(LaAttnArgs a) {
  typedef AttnT<T, DH> AT;
  typedef typename AT::QF QF;
  typedef typename AT::VV VV;
  constexpr int ROWB = AT::ROWB, LP = AT::LP, NDT = AT::NDT, VB = AT::VB;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int group = a.H / a.Hkv;
  const int tiles_kv = group * ((a.Q + 15) >> 4);
  const int gt = blockIdx.x * 4 + wave;
  const int g_kv = gt / tiles_kv;
  if (g_kv >= a.Hkv) return;
  const TileRows tr = tile_rows(a, g_kv, gt % tiles_kv, c16);
  if (__ballot(tr.valid) == 0ull) return;
  const int pos = tr.pos;
  const int se = a.shared_end;
  const float sl2 = a.scale_log2;
  const char* kc = (const char*)a.kc + (size_t)g_kv * a.T_cap * ROWB;
  const char* vc = (const char*)a.vc + (size_t)g_kv * a.T_cap * ROWB;
  const char* kw = (const char*)a.kw + (size_t)g_kv * a.ws_cap * ROWB;
  const char* vw = (const char*)a.vw + (size_t)g_kv * a.ws_cap * ROWB;
  const int br = tr.valid ? a.branch[tr.row] : -1;
  QF qf;
  if (a.n_tail > 0) qf = load_q<QF, LP>(a, tr, g, ROWB);

  // row address of key x on a branch (a clamped committed row when x is not on its path)
  auto src_row = [&](int x, const int* pth, int plen, const char* cbase, const char* wbase) -> const char* {
    if (x < se) return cbase + (size_t)x * ROWB;
    const int e = x - se;
    const int w = e < plen ? pth[e] : -1;
    if ((unsigned)w < (unsigned)a.n_ws) return wbase + (size_t)w * ROWB;
    return cbase + (size_t)(se - 1) * ROWB;
  };

  float M = NEG_INF, L = 0.f;
  f32x4 O[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) O[dt] = f32x4{0, 0, 0, 0};
  for (int cls = 0; cls < NCLS; ++cls) {
    float m = NEG_INF, l = 0.f;
    f32x4 o[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) o[dt] = f32x4{0, 0, 0, 0};
    if (cls <= a.class_last && tr.valid) {
      const size_t base = ((size_t)cls * a.H + tr.hh) * a.Q + tr.row;
      const float2 ml = *(const float2*)(a.part_ml + base * 2);
      m = ml.x;
      l = ml.y;
      if (m != NEG_INF) {
        const float* src = a.part_o + base * DH + 4 * NDT * g;
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) o[dt][r] = src[NDT * r + dt];
      }
    }
    const int tau = (cls - a.tail0 % NCLS + NCLS) % NCLS;
    if (tau < a.n_tail) {
      const int x0 = CH * (a.tail0 + tau);
      const bool need = tr.valid && pos >= x0;
      const unsigned long long all = __ballot(need && g == 0);
      float sc[2][4];
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
#pragma unroll
        for (int r = 0; r < 4; ++r) sc[jj][r] = NEG_INF;
      unsigned long long pend = all;
      while (pend) {
        const int b = __builtin_amdgcn_readfirstlane(__shfl(br, __ffsll((long long)pend) - 1, 64));
        const bool mine = need && br == b;
        pend &= ~__ballot(mine && g == 0);
        const int plen = min(a.path_len[b], a.maxp);
        const int* pth = a.path + (size_t)b * a.maxp;
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
          const char* kr = src_row(x0 + 16 * jj + c16, pth, plen, kc, kw) + 16 * LP * g;
          QF kf;
#pragma unroll
          for (int s = 0; s < LP; ++s) kf.p[s] = *(const u32x4*)(kr + 16 * s);
          const f32x4 s4 = AT::qk(kf, qf);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float v = (x0 + 16 * jj + 4 * g + r <= pos) ? s4[r] * sl2 : NEG_INF;
            sc[jj][r] = mine ? v : sc[jj][r];
          }
        }
      }
      float mc, lc;
      chunk_softmax(sc, mc, lc);
      f32x4 oc[NDT];
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) oc[dt] = f32x4{0, 0, 0, 0};
      pend = all;
      while (pend) {
        const int b = __builtin_amdgcn_readfirstlane(__shfl(br, __ffsll((long long)pend) - 1, 64));
        const bool mine = need && br == b;
        pend &= ~__ballot(mine && g == 0);
        const int plen = min(a.path_len[b], a.maxp);
        const int* pth = a.path + (size_t)b * a.maxp;
        VV vv[8];
        float ps[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          vv[e] = *(const VV*)(src_row(x0 + slot_key(g, e), pth, plen, vc, vw) + VB * c16);
          ps[e] = mine ? sc[e >> 2][e & 3] : 0.f;
        }
        const typename AT::PP pp = AT::prep(ps);
        // rows of branch b take this pass (their keys in every slot)
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const f32x4 ob = AT::pv(dt, vv, pp);
#pragma unroll
          for (int r = 0; r < 4; ++r) oc[dt][r] = mine ? ob[r] : oc[dt][r];
        }
      }
      fold_state<NDT>(m, l, o, mc, lc, oc);
    }
    fold_state<NDT>(M, L, O, m, l, o);
  }
  if (tr.valid) {
    // lane holds head dimensions NDT*(4g + r) + dt: 4*NDT contiguous values
    T* dst = (T*)a.o + ((size_t)tr.row * a.H + tr.hh) * DH + 4 * NDT * g;
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) st<T>(dst + NDT * r + dt, O[dt][r] / L);
  }
}

int la_attention_parts() { return NCLS; }

template <typename T, int DH, int NW>
static void launch_nw(const LaAttnArgs& a, int grid, hipStream_t st) {
  constexpr int ROWB = AttnT<T, DH>::ROWB;
  constexpr size_t lds = (size_t)DEPTH * 2 * CH * ROWB + (size_t)NW * 16 * ROWB + (size_t)NW * 256;
  static const bool attr = hipFuncSetAttribute((const void*)&la_attn_kernel<T, DH, NW>,
                                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) == hipSuccess;
  (void)attr;
  hipLaunchKernelGGL((la_attn_kernel<T, DH, NW>), dim3(grid), dim3(64 * NW), lds, st, a);
}

template <typename T, int DH>
static void launch_dh(LaAttnArgs a, hipStream_t st) {
  const int group = a.H / a.Hkv;
  const int tiles = group * ((a.Q + 15) / 16);
  const int nw = tiles >= 8 ? 8 : tiles >= 4 ? 4 : tiles >= 2 ? 2 : 1;
  a.rgroups = (tiles + nw - 1) / nw;
  if (a.class_last >= 0) {
    const int hpx = (a.Hkv + 7) / 8;
    const int grid = 8 * hpx * NCLS * a.rgroups;
    switch (nw) {
      case 8: launch_nw<T, DH, 8>(a, grid, st); break;
      case 4: launch_nw<T, DH, 4>(a, grid, st); break;
      case 2: launch_nw<T, DH, 2>(a, grid, st); break;
      default: launch_nw<T, DH, 1>(a, grid, st); break;
    }
  }
  const int waves = a.Hkv * tiles;
  hipLaunchKernelGGL((la_attn_tail_merge_kernel<T, DH>), dim3((waves + 3) / 4), dim3(256), 0, st, a);
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
  if (a.n_tail > NTAIL) return -2;
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
