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
//   * keys are cut into chunks of 32 positions and the chunks into key
//     splits of a fixed number of chunks (set by the cache capacity); chunk
//     c belongs to class c % 4;
//   * inside a split, a class takes its chunks in decreasing position with
//     the online softmax: the reference maximum m' moves to the chunk's
//     exact maximum only when that exceeds it by more than RESCALE, the
//     running sums are scaled by 2^(m - m'), p = 2^(s - m'),
//     l' = l * 2^(m - m') + sum p (fixed lane order), and O' = O * 2^(m - m')
//     + V^T P^T accumulated by MFMA over a fixed key -> slot assignment;
//   * a split's 4 class states are folded in class order, the splits' states
//     in split order, then O / l.
//
// Work decomposition (gfx950, wave64; a wave owns one class of one tile of
// 16 query rows of one q-head):
//   * one workgroup per (KV head, row group of up to 4 tiles, key split of
//     a fixed number of 128-position stages), 4 class waves per tile pair
//     (a wave computes two tiles from one read of the chunk's K and V); K
//     and V of every committed chunk
//     land in LDS through global_load_lds_dwordx4 (16-byte pieces
//     XOR-swizzled by row, so the QK and the PV fragment reads are
//     bank-conflict free) in a ring of 128-key stages shared by all tiles and
//     classes of the workgroup; the row positions and the tiles' Q come in
//     the same way, so the only waits are the ring's own;
//   * QK: S^T = K Q^T, 16x16x32 bf16 MFMA (16x16x4 fp32): one query row per
//     lane column, so the softmax statistics stay in-lane;
//   * PV: O^T += V^T P^T; output tile dt holds head dimensions NDT*m + dt, so
//     a lane reads NDT contiguous elements of each key row and transposes
//     them in registers; P enters rounded to bf16 (fp32 accumulation);
//   * the chunks that reach past shared_end (at most one per class) are
//     applied last in their class, from rows gathered out of the cache or,
//     through each branch's path, out of the packed rows' workspace, once per
//     branch in the tile (rows of other branches get p = 0 in that pass,
//     which leaves their sums unchanged);
//   * the class states are folded in class order inside the workgroup; with
//     several key splits a small kernel folds the splits' states in order.
// The block -> work mapping keeps every workgroup of one KV head on one XCD
// (blockIdx % 8), so the head's Q and the K/V chunks shared by its row groups
// are fetched from HBM once.
#include <algorithm>
#include <type_traits>

#include "la_common.h"
#include "la_dev.h"
#include "la_kernels.h"

#define CH 32         // keys per chunk
#define NCLS 4        // chunk classes
#define NTAIL 4       // most chunks per call that reach past shared_end
#define NEG_INF (-__builtin_inff())



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
  // P^T operand of one chunk: p of slot e rounded to bf16 (nearest even)
  typedef bf16x8 PP;
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
  // V^T(dt) operand of the chunk's 8 slots; vv[e] holds the lane's elements of slot e
  typedef bf16x8 VA;
  template <typename V> static __device__ __forceinline__ VA va(int dt, const V* vv) {
    uint32_t w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t lo = vv[2 * j].w[dt >> 1], hi = vv[2 * j + 1].w[dt >> 1];
      // element dt of key slot 2j (low half) and of key slot 2j + 1 (high half)
      w[j] = __builtin_amdgcn_perm(hi, lo, (dt & 1) ? 0x07060302u : 0x05040100u);
    }
    return __builtin_bit_cast(bf16x8, w);
  }
  // o += V^T(dt) P^T
  static __device__ __forceinline__ f32x4 pva(const VA& A, const PP& pp, f32x4 o) { return mfma_bf16_32(A, pp, o); }
  template <typename V>
  static __device__ __forceinline__ f32x4 pv(int dt, const V* vv, const PP& pp, f32x4 o) {
    return pva(va(dt, vv), pp, o);
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
  struct VA { float v[8]; };
  template <typename V> static __device__ __forceinline__ VA va(int dt, const V* vv) {
    VA r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r.v[e] = __uint_as_float(vv[e].w[dt]);
    return r;
  }
  static __device__ __forceinline__ f32x4 pva(const VA& A, const PP& pp, f32x4 o) {
#pragma unroll
    for (int e = 0; e < 8; ++e) o = mfma_f32_4(A.v[e], pp.p[e], o);
    return o;
  }
  template <typename V>
  static __device__ __forceinline__ f32x4 pv(int dt, const V* vv, const PP& pp, f32x4 o) {
    return pva(va(dt, vv), pp, o);
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

// One workgroup per (KV head, row group, key split); a row group is NT =
// TP * TPW tiles of 16 query rows; wave w is class c = w / TP of tile pair
// slot w % TP, which holds TPW tiles: the K and V fragments a wave reads
// from the ring serve all its tiles.  A key split is a fixed run of spb ring
// stages (spb is a function of the cache capacity only); several splits
// leave one folded state per row each, and a merge kernel folds them in
// split order (a split's chunks, tail chunks included, are fixed by
// position, so the tree still depends on positions only).
// Three phases per workgroup:
//   1. tail (splits that hold one): the chunks reaching past shared_end (at
//      most one per class, the highest positions of the split, so the first
//      in their class): the ring's space is used to stage, per tile, the
//      committed rows [32 tail0, shared_end) and, for each branch in the
//      tile, its workspace rows of positions shared_end .. max_pos (read
//      through the branch path); the scores come per branch and P V runs once
//      per branch (rows of other branches add exact zeros);
//   2. prefix: ring stage s holds keys [128 s, 128 s + 128) of the head (the
//      class-c chunk 4 s + c, K and V, 16-byte pieces XOR-swizzled by row)
//      for every chunk below shared_end (or up to the largest row position
//      when nothing reaches past it), stages taken from the split's last to
//      its first; each class wave takes its chunk of the stage with the
//      online step, so a stage is read from HBM once for all the workgroup's
//      tiles and classes;
//   3. fold: every class wave hands its states over through LDS and folds,
//      for one accumulator row of each tile, classes 0, 1, 2, 3 in order,
//      then stores O / l (or the split's state).
// Every global load of the ring is a DMA into LDS read back with inline asm;
// the waits are static vmcnt counts (every wave issues the same DMA count per
// stage).
// Whether key split s holds chunks that reach past shared_end (a chunk
// belongs to the split of its position).
__host__ __device__ __forceinline__ bool split_has_tail(const LaAttnArgs& a, int s) {
  const int per = a.spb * NCLS;
  return max(a.tail0, s * per) < min(a.tail0 + a.n_tail, (s + 1) * per);
}

template <typename T, int DH, int TP, int TPW>
__global__ void __launch_bounds__(64 * NCLS * TP) __attribute__((amdgpu_waves_per_eu(1, TP)))
la_attn_kernel(LaAttnArgs a) {
  typedef AttnT<T, DH> AT;
  typedef typename AT::QF QF;
  typedef typename AT::VV VV;
  constexpr int NW = NCLS * TP;                 // waves
  constexpr int NT = TP * TPW;                  // tiles per workgroup
  constexpr int ROWB = AT::ROWB, PIECES = AT::PIECES, LP = AT::LP, NDT = AT::NDT, VB = AT::VB;
  constexpr int CHB = CH * ROWB;                // K (or V) of one chunk
  constexpr int BLKB = NCLS * 2 * CHB;          // one ring stage: 4 chunks, K then V each
  constexpr int NDMA = BLKB / 1024;
  constexpr int CW = NDMA / NW;                 // DMA instructions per stage and wave
  static_assert(NDMA % NW == 0 && CW >= 1, "DMA blocks per wave");
  constexpr int DEPTH = 2;
  constexpr int RPB = 1024 / ROWB;              // key rows per 1 KB DMA block
  // Q tiles and row positions (one DMA of 64 lanes per tile); the ring starts 1 KB aligned
  constexpr int FIX = (NT * (16 * ROWB + 256) + 1023) & ~1023;
  extern __shared__ __attribute__((aligned(1024))) char lds[];
  char* const ring = lds + FIX;                 // ring stages, later the tail rows, then the fold states

  // block -> (XCD, KV head, key split, row group): the workgroups of one
  // head share an XCD (and its L2).  A split holding tail chunks gets two
  // workgroups per row group when a wave has two tiles (each takes one tile
  // of every tile pair), so the tail work of a tile pair runs in parallel.
  const int xcd = blockIdx.x & 7, bi = blockIdx.x >> 3;
  const int g_kv = xcd + 8 * (bi / a.wg_head);
  if (g_kv >= a.Hkv) return;
  int li = bi % a.wg_head, sp = 0, hf = -1;
  for (; sp < a.nsplit; ++sp) {
    const bool half = TPW == 2 && a.tail_half && split_has_tail(a, sp);
    const int n = a.rgroups * (half ? 2 : 1);
    if (li < n) {
      if (half) {
        hf = li % 2;
        li /= 2;
      }
      break;
    }
    li -= n;
  }
  if (sp == a.nsplit) return;
  const int rg = li;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int cls = wave / TP, pslot = wave % TP;
  const int g = lane >> 4, c16 = lane & 15;
  const int se = a.shared_end;
  const float sl2 = a.scale_log2;
  const char* kc = (const char*)a.kc + (size_t)g_kv * a.T_cap * ROWB;
  const char* vc = (const char*)a.vc + (size_t)g_kv * a.T_cap * ROWB;

  // the wave's tiles: 16 rows of q-head hh each (rows past Q load row Q - 1
  // and stay unused; a tile past the head group is skipped)
  const int group = a.H / a.Hkv;
  const int rtiles = (a.Q + 15) >> 4;
  bool tv[TPW], rvalid[TPW];
  int hh[TPW], row[TPW];
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    const int tile = rg * NT + pslot * TPW + (hf >= 0 ? hf : u);
    tv[u] = (hf < 0 || u == 0) && tile < group * rtiles;
    hh[u] = g_kv * group + (tv[u] ? tile / rtiles : 0);
    row[u] = (tv[u] ? tile % rtiles : 0) * 16 + c16;
    rvalid[u] = tv[u] && row[u] < a.Q;
  }
  auto qa = [&](int u) __attribute__((always_inline)) { return lds + (pslot * TPW + u) * 16 * ROWB; };
  auto pa = [&](int u) __attribute__((always_inline)) { return lds + NT * 16 * ROWB + (pslot * TPW + u) * 256; };
  // Chunks of a class are taken in decreasing position, so a split's tail
  // chunks (the highest positions) come first: a workgroup with tail chunks
  // applies them before its ring starts (the ring's space holds the tiles'
  // branch tables and staged rows meanwhile), and the ring then walks its
  // stages from the last to the first.
  const int t_lo = max(a.tail0, sp * a.spb * NCLS), t_hi = min(a.tail0 + a.n_tail, (sp + 1) * a.spb * NCLS);
  const bool has_tail = t_lo < t_hi;              // split_has_tail(a, sp): uniform over the workgroup
  int* const spath0 = (int*)ring;                 // tail: [NT][16 branches][64 positions] workspace rows
  int* const meta0 = (int*)(ring + NT * 16 * 64 * 4);   // tail: [NT][64] branch count, branch ids
  if (cls == 0) {
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      const int row0 = row[u] - c16;
      __builtin_amdgcn_global_load_lds((const void*)(a.pos + min(row0 + (lane & 15), a.Q - 1)), (lds_void_t*)pa(u), 4,
                                       0, 0);
#pragma unroll
      for (int j = 0; j < 16 / RPB; ++j) {
        const int r = min(row0 + j * RPB + lane / PIECES, a.Q - 1);
        const char* src = (const char*)a.q + ((size_t)r * a.H + hh[u]) * ROWB + 16 * (lane % PIECES);
        __builtin_amdgcn_global_load_lds((const void*)src, (lds_void_t*)(qa(u) + j * 1024), 16, 0, 0);
      }
      if (has_tail && tv[u]) {                    // the tile's branch tables (row builder)
        const int rt = row0 >> 4;
        __builtin_amdgcn_global_load_lds((const void*)(a.tile_meta + (size_t)rt * 64 + lane),
                                         (lds_void_t*)(meta0 + (pslot * TPW + u) * 64), 4, 0, 0);
#pragma unroll
        for (int j = 0; j < 4; ++j)
          __builtin_amdgcn_global_load_lds((const void*)(a.tile_path + (size_t)rt * 1024 + j * 256 + 4 * lane),
                                           (lds_void_t*)(spath0 + (pslot * TPW + u) * 1024 + j * 256), 16, 0, 0);
      }
    }
  }

  // ring stage s: chunks 4 s .. 4 s + 3; outside the split's stages every
  // lane loads one 16-byte piece (a dummy that nobody reads), so every wave
  // issues CW DMA instructions per stage on every path
  const int nblk = (a.class_last + NCLS) / NCLS;   // stages of the whole prefix (class_last = -1: none)
  const int s_begin = sp * a.spb;                     // this split's stages
  const int s_end = min(s_begin + a.spb, nblk);
  // wave w brings the DMA blocks w*CW .. w*CW + CW - 1 of a stage (a
  // contiguous run inside its chunk cw of the stage: CW divides the 1 KB
  // blocks of a chunk half or is a multiple of them).  The lane's source
  // offset inside a chunk is the same for every stage; only stages that
  // reach past shared_end clamp rows.
  constexpr int HB = CHB / 1024;                // 1 KB blocks in a chunk's K (or V)
  static_assert(HB % CW == 0 || CW % HB == 0, "DMA runs");
  const int b0 = wave * CW;
  const int cw = b0 / (2 * HB);
  // K or V of block j: one half for the whole run when CW <= HB, else the
  // run is a whole chunk (K blocks, then V blocks)
  constexpr bool WHOLE = CW > HB;
  const char* const half0 = ((b0 / HB) & 1) ? vc : kc;
  auto kv_of = [&](int j) __attribute__((always_inline)) -> const char* { return WHOLE ? ((j / HB) ? vc : kc) : half0; };
  int oj[CW];
#pragma unroll
  for (int j = 0; j < CW; ++j) {
    const int r = ((b0 + j) % HB) * RPB + lane / PIECES;
    oj[j] = r * ROWB + 16 * ((lane % PIECES) ^ (r % PIECES));
  }
  auto issue = [&](char* stage, int s) __attribute__((always_inline)) {
    const int x0 = CH * (NCLS * s + cw);
    const bool in = s >= s_begin && s < s_end;
    if (in && x0 + CH <= se) {                  // the whole chunk lies below shared_end
#pragma unroll
      for (int j = 0; j < CW; ++j) {
        const char* base = kv_of(j);
        __builtin_amdgcn_global_load_lds((const void*)(base + (size_t)x0 * ROWB + oj[j]),
                                         (lds_void_t*)(stage + (b0 + j) * 1024), 16, 0, 0);
      }
    } else if (in) {                            // rows past shared_end - 1 repeat it (never visible)
#pragma unroll
      for (int j = 0; j < CW; ++j) {
        const char* base = kv_of(j);
        const int r = ((b0 + j) % HB) * RPB + lane / PIECES;
        const int off = oj[j] - r * ROWB;
        __builtin_amdgcn_global_load_lds((const void*)(base + (size_t)min(x0 + r, se - 1) * ROWB + off),
                                         (lds_void_t*)(stage + (b0 + j) * 1024), 16, 0, 0);
      }
    } else {                                    // outside the split: one valid 16-byte piece
#pragma unroll
      for (int j = 0; j < CW; ++j)
        __builtin_amdgcn_global_load_lds((const void*)(kc + (size_t)(se - 1) * ROWB),
                                         (lds_void_t*)(stage + (b0 + j) * 1024), 16, 0, 0);
    }
  };
  // the rows' branches (read now, used by the tail phase)
  int br[TPW];
#pragma unroll
  for (int u = 0; u < TPW; ++u) br[u] = (a.n_tail > 0 && rvalid[u]) ? a.branch[row[u]] : -1;
  // Without tail chunks the ring's first stage goes out with Q and is waited
  // for here; its second stage follows once Q is read, so the first stage
  // is not held up behind every workgroup's second one.
  if (!has_tail) issue(ring, s_end - 1);
  wait_vm<0>();                                      // this wave's Q, positions, branches (and first stage)
  ring_barrier();                                    // ... and those of the other waves
  QF qf[TPW];
  int pos[TPW], pmin[TPW];
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    typename LdsT<16>::T qraw[LP];
    const uint32_t qaddr = lds_addr(qa(u) + c16 * ROWB + 16 * LP * g);
    if constexpr (LP >= 1) qraw[0] = lds_read<16, 0>(qaddr);
    if constexpr (LP >= 2) qraw[1] = lds_read<16, 16>(qaddr);
    if constexpr (LP >= 3) qraw[2] = lds_read<16, 32>(qaddr);
    if constexpr (LP >= 4) qraw[3] = lds_read<16, 48>(qaddr);
    unsigned int praw[1] = {lds_read<4, 0>(lds_addr(pa(u) + 4 * c16))};
    lds_wait(qraw);
    lds_wait(praw);
#pragma unroll
    for (int s = 0; s < LP; ++s) qf[u].p[s] = rvalid[u] ? __builtin_bit_cast(u32x4, qraw[s]) : u32x4{0, 0, 0, 0};
    pos[u] = rvalid[u] ? (int)praw[0] : -1;
    // smallest position among the tile's rows: chunks ending at or below it need no mask
    int pm = rvalid[u] ? pos[u] : 0x7fffffff;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) pm = min(pm, __shfl_xor(pm, o, 64));
    pmin[u] = __builtin_amdgcn_readfirstlane(pm);
  }

  float M[TPW], L[TPW];
  f32x4 O[TPW][NDT];
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    M[u] = NEG_INF;
    L[u] = 0.f;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) O[u][dt] = f32x4{0, 0, 0, 0};
  }

  if (has_tail) {
    const int X0 = CH * a.tail0;
    const int ncom = se - X0;                       // 0 .. 31
    const int EP = a.max_pos - se + 1;              // 1 .. 64
    // staged rows of each tile pair slot, after the branch tables
    char* const ks = ring + NT * (16 * 64 + 64) * 4 + pslot * 2 * a.trows * ROWB;
    char* const vs = ks + a.trows * ROWB;
    // the tiles' distinct branches (lane i < nbr: branch i)
    int nbr[TPW], bl[TPW];
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      const int* mt = meta0 + (pslot * TPW + u) * 64;
      nbr[u] = tv[u] ? min(mt[0], 16) : 0;
      bl[u] = (tv[u] && lane < 16) ? mt[1 + lane] : -1;
    }
    // branches staged at once per tile (the committed rows, then EP rows per
    // branch), and the batches every tile of the workgroup goes through
    const int bb = (a.trows - ncom) / EP;           // >= 1 (the launcher sizes trows)
    int* const nbat = (int*)(lds + NT * 16 * ROWB);   // the row positions' space, free since they were read
    if (cls == 0 && lane == 0) {
#pragma unroll
      for (int u = 0; u < TPW; ++u) nbat[pslot * TPW + u] = (nbr[u] + bb - 1) / bb;
    }
    __syncthreads();
    int nbatch = 0;
#pragma unroll
    for (int t = 0; t < NT; ++t) nbatch = max(nbatch, nbat[t]);
    const char* kw = (const char*)a.kw + (size_t)g_kv * a.ws_cap * ROWB;
    const char* vw = (const char*)a.vw + (size_t)g_kv * a.ws_cap * ROWB;
    const int tau = (cls - a.tail0 % NCLS + NCLS) % NCLS;   // the class's tail chunk (at most one)
    const bool mine_chunk = tau < a.n_tail && a.tail0 + tau >= t_lo && a.tail0 + tau < t_hi;
    // With a single tail chunk in the split its branches are spread over the
    // four class waves (wave c takes the batch branches i with i % 4 == c);
    // every wave starts from the empty state (the tail comes first), and the
    // chunk's class wave then collects each row's state from the wave that
    // handled the row's branch, through the staging space.
    constexpr int SF = 2 + 4 * NDT;                 // floats of one lane's state
    const bool spread = t_hi - t_lo == 1 && 2 * a.trows * ROWB >= NCLS * SF * 64 * 4;
    const int cstar = t_lo % NCLS;
    const int x0 = CH * (spread ? t_lo : a.tail0 + tau);
    const bool work = spread || mine_chunk;
    auto srow = [&](int x, int bi) -> int {
      if (x < se) return x - X0;
      const int e = x - se;
      return e < EP ? ncom + bi * EP + e : 0;
    };
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      if (hf >= 0 && u > 0) break;                // one tile per pair slot (uniform over the workgroup)
      const int* const spath = spath0 + (pslot * TPW + u) * 1024;
      const bool need = work && rvalid[u] && pos[u] >= x0;
      bool own = false;                           // a branch this wave handled holds the lane's row
      for (int bt = 0; bt < nbatch; ++bt) {
        const int i0 = bt * bb;
        const int nb = max(0, min(bb, nbr[u] - i0));
        // staged row of key x on batch branch bi (x >= X0); a clamped committed
        // row where a position is not on the branch's path (never visible to it)
        const int nr = nb > 0 ? ncom + nb * EP : 0;
        for (int blk = cls; blk * RPB < nr; blk += NCLS) {
          const int j = blk * RPB + lane / PIECES;
          const int piece = (lane % PIECES) ^ (j % PIECES);
          int crow = se - 1, wrow = -1;
          if (j < ncom) crow = X0 + j;
          else if (j < nr) {
            wrow = spath[(i0 + (j - ncom) / EP) * 64 + (j - ncom) % EP];
            if ((unsigned)wrow >= (unsigned)a.n_ws) wrow = -1;
          }
          const size_t off = (size_t)(wrow >= 0 ? wrow : crow) * ROWB + 16 * piece;
          __builtin_amdgcn_global_load_lds((const void*)((wrow >= 0 ? kw : kc) + off), (lds_void_t*)(ks + blk * 1024),
                                           16, 0, 0);
          __builtin_amdgcn_global_load_lds((const void*)((wrow >= 0 ? vw : vc) + off), (lds_void_t*)(vs + blk * 1024),
                                           16, 0, 0);
        }
        wait_vm<0>();
        __syncthreads();
        // rows of this batch's branches: the chunk's online step (for the
        // wave's other rows every score stays -inf, which leaves their state
        // exactly as it is, and P V adds exact zeros)
        if (nb > 0 && __ballot(need) != 0ull) {
          float sc[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) sc[e] = NEG_INF;
          for (int bi = 0; bi < nb; ++bi) {
            if (spread && (i0 + bi) % NCLS != cls) continue;
            const int b = __shfl(bl[u], i0 + bi, 64);
            const bool mine = need && br[u] == b;
            own |= mine;
            if (__ballot(mine) == 0ull) continue;
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
              const int r = srow(x0 + 16 * jj + c16, bi);
              QF kf;
#pragma unroll
              for (int q = 0; q < LP; ++q)
                kf.p[q] = *(const u32x4*)(ks + r * ROWB + 16 * ((LP * g + q) ^ (r % PIECES)));
              const f32x4 s4 = AT::qk(kf, qf[u]);
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                const float v = (x0 + 16 * jj + 4 * g + q <= pos[u]) ? s4[q] : NEG_INF;
                sc[4 * jj + q] = mine ? v : sc[4 * jj + q];
              }
            }
          }
          const float wa = chunk_softmax(sc, sl2, M[u], L[u]);
          scale_o<NDT>(O[u], wa);
          for (int bi = 0; bi < nb; ++bi) {
            if (spread && (i0 + bi) % NCLS != cls) continue;
            const int b = __shfl(bl[u], i0 + bi, 64);
            const bool mine = need && br[u] == b;
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
            for (int dt = 0; dt < NDT; ++dt) O[u][dt] = AT::pv(dt, vv, pp, O[u][dt]);
          }
        }
        __syncthreads();                          // the staged rows are no longer read
      }
      if (spread) {
        float* const sl = (float*)ks;             // [NCLS][SF][64] lane states, in the staging space
        unsigned long long* const om = (unsigned long long*)(lds + NT * 16 * ROWB + 64) + pslot * NCLS;
        const unsigned long long ownm = __ballot(own);
        float* const my = sl + (size_t)cls * SF * 64;
        my[lane] = M[u];
        my[64 + lane] = L[u];
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
          for (int r = 0; r < 4; ++r) my[(2 + 4 * dt + r) * 64 + lane] = O[u][dt][r];
        if (lane == 0) om[cls] = ownm;
        __syncthreads();
        if (cls == cstar) {
#pragma unroll
          for (int w = 0; w < NCLS; ++w) {
            if (w == cls || ((om[w] >> lane) & 1ull) == 0ull) continue;
            const float* src = sl + (size_t)w * SF * 64;
            M[u] = src[lane];
            L[u] = src[64 + lane];
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
              for (int r = 0; r < 4; ++r) O[u][dt][r] = src[(2 + 4 * dt + r) * 64 + lane];
          }
        } else {                                  // this class has no chunk in the tail
          M[u] = NEG_INF;
          L[u] = 0.f;
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) O[u][dt] = f32x4{0, 0, 0, 0};
        }
        __syncthreads();                          // the states are no longer read
      }
    }
    // the tail is done with the ring's space: the ring starts
    issue(ring, s_end - 1);
  }
  static_assert(DEPTH == 2, "ring start");
  issue(ring + BLKB, s_end - 2);                   // the first step waits for the first stage only

  // lane parts of the fragment addresses of the class's chunk (stage offsets are immediates)
  uint32_t koff[LP], voff[4];
#pragma unroll
  for (int s = 0; s < LP; ++s)
    koff[s] = lds_addr(ring + cls * 2 * CHB + c16 * ROWB + 16 * ((LP * g + s) ^ (c16 % PIECES)));
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int kk = 4 * g + e;                   // slot_key(g, e); slot e + 4 is 16 rows further
    const int off = VB * c16;
    voff[e] = lds_addr(ring + cls * 2 * CHB + CHB + kk * ROWB + 16 * ((off / 16) ^ (kk % PIECES)) + off % 16);
  }

  auto step = [&](auto SI, int s) __attribute__((always_inline)) {
    constexpr int S = decltype(SI)::value;
    constexpr int SB = S * BLKB;                // stage base
    constexpr int SBH = SB & ~65535, SBL = SB & 65535;   // ds offsets reach 64 KB
    wait_vm<CW * (DEPTH - 1)>();                // stage s landed (the next one may be in flight)
    ring_barrier();
    const int k = NCLS * s + cls;               // the class's chunk
    const bool live = k <= a.class_last;
    // the chunk's K and V go to registers first, so the stage is released
    // (and the stage two steps ahead issued) before any arithmetic
    typename LdsT<16>::T kraw[2 * LP];
    typename LdsT<VB>::T vraw[8];
    if (live) {
#pragma unroll
      for (int q = 0; q < LP; ++q) {
        kraw[q] = lds_read<16, SBL>(koff[q] + SBH);
        kraw[LP + q] = lds_read<16, SBL + 16 * ROWB>(koff[q] + SBH);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        vraw[e] = lds_read<VB, SBL>(voff[e] + SBH);
        vraw[e + 4] = lds_read<VB, SBL + 16 * ROWB>(voff[e] + SBH);
      }
      lds_wait(kraw);
      lds_wait(vraw);
    }
    ring_barrier();                             // every wave has read the stage
    issue(ring + SB, s - DEPTH);
    if (live) {
      const int x0 = CH * k;
      float sc[TPW][8];
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        QF kf;
#pragma unroll
        for (int q = 0; q < LP; ++q) kf.p[q] = __builtin_bit_cast(u32x4, kraw[LP * jj + q]);
#pragma unroll
        for (int u = 0; u < TPW; ++u) {
          if (!tv[u]) continue;
          const f32x4 s4 = AT::qk(kf, qf[u]);
#pragma unroll
          for (int r = 0; r < 4; ++r) sc[u][4 * jj + r] = s4[r];
        }
      }
      typename AT::PP pp[TPW];
#pragma unroll
      for (int u = 0; u < TPW; ++u) {
        if (!tv[u]) continue;
        if (x0 + CH - 1 > pmin[u]) {            // some key of the chunk lies past some row
#pragma unroll
          for (int e = 0; e < 8; ++e) sc[u][e] = x0 + slot_key(g, e) <= pos[u] ? sc[u][e] : NEG_INF;
        }
        const float wa = chunk_softmax(sc[u], sl2, M[u], L[u]);
        pp[u] = AT::prep(sc[u]);
        scale_o<NDT>(O[u], wa);
      }
      VV vv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) vv[e] = __builtin_bit_cast(VV, vraw[e]);
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const typename AT::VA A = AT::va(dt, vv);
#pragma unroll
        for (int u = 0; u < TPW; ++u)
          if (tv[u]) O[u][dt] = AT::pva(A, pp[u], O[u][dt]);
      }
    }
  };
  for (int s0 = s_end - 1; s0 >= s_begin; s0 -= DEPTH)
    static_for<0, DEPTH>([&](auto SI) {
      if (decltype(SI)::value == 0 || s0 - decltype(SI)::value >= s_begin) step(SI, s0 - decltype(SI)::value);
    });

  wait_vm<0>();                                   // the dummy stages have landed: the ring is free
  ring_barrier();

  // fold: every class wave hands (m, l, O) over through LDS; class wave c
  // then folds accumulator row c (head dimensions NDT*(4g + c) + dt, NDT
  // contiguous values) of every tile of its pair slot, classes 0, 1, 2, 3 in
  // order, and stores them
  constexpr int FS = 64 * (2 + 4 * NDT);          // floats of one wave's state: (m, l) per lane, then O by row
  auto xf = [&](int u, int c) __attribute__((always_inline)) {
    return (float*)ring + (size_t)((pslot * TPW + u) * NCLS + c) * FS;
  };
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    if (!tv[u]) continue;
    float* d = xf(u, cls);
    *(float2*)(d + 2 * lane) = make_float2(M[u], L[u]);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float* dr = d + 128 + (r * 64 + lane) * NDT;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) dr[dt] = O[u][dt][r];
    }
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    if (!tv[u] || !rvalid[u]) continue;
    float Mf = NEG_INF, Lf = 0.f;
    float Of[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) Of[dt] = 0.f;
#pragma unroll
    for (int c = 0; c < NCLS; ++c) {
      const float* d = xf(u, c);
      const float2 ml = *(const float2*)(d + 2 * lane);
      if (ml.x == NEG_INF) continue;
      const float* dr = d + 128 + (cls * 64 + lane) * NDT;
      const float mn = fmaxf(Mf, ml.x);
      const float wa = ex2(Mf - mn), wb = ex2(ml.x - mn);
      Lf = lin2(Lf, wa, ml.y, wb);
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) Of[dt] = lin2(Of[dt], wa, dr[dt], wb);
      Mf = mn;
    }
    const int d0 = NDT * (4 * g + cls);             // first of the NDT contiguous head dimensions
    if (a.nsplit > 1) {
      // the split's state: (m, l) and O in natural dimension order
      const size_t base = ((size_t)sp * a.H + hh[u]) * a.Q + row[u];
      if (g == 0 && cls == 0) *(float2*)(a.part_ml + base * 2) = make_float2(Mf, Lf);
      float* po = a.part_o + base * DH + d0;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) po[dt] = Of[dt];
      continue;
    }
    T* dst = (T*)a.o + ((size_t)row[u] * a.H + hh[u]) * DH + d0;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) st<T>(dst + dt, Of[dt] / Lf);
  }
}

// Fold of the key splits' states in split order (the same sequence of
// roundings as the class fold), then O / l.  One thread per 4 head dimensions of
// a (row, head).
template <typename T, int DH>
__global__ void __launch_bounds__(256) la_attn_merge_kernel(LaAttnArgs a) {
  constexpr int V4 = DH / 4, MS = 8;            // splits whose loads are all issued before the fold
  // block -> (XCD, KV head): the head's split states were written on that
  // XCD (the attention kernel's mapping), so they are read from its L2
  const int group = a.H / a.Hkv;
  const int per = a.Q * group * V4;               // (row, q-head, 4 dims) items of one KV head
  const int wpk = (per + 255) / 256;
  const int g_kv = (blockIdx.x & 7) + 8 * ((blockIdx.x >> 3) / wpk);
  const int item = ((blockIdx.x >> 3) % wpk) * 256 + threadIdx.x;
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

// Ring stages (128 positions each) per key split: a function of the cache
// capacity only, so every call on one cache cuts its keys the same way: one
// stage per split up to 8 stages (short caches: more, shorter workgroups),
// else about four splits when the cache is full.
int la_attention_spb(int t_cap) {
  const int stages = (std::max(t_cap, 1) + CH * NCLS - 1) / (CH * NCLS);
  if (stages <= 8) return 1;
  return std::max(1, (stages + 3) / 4);
}
int la_attention_parts(int max_pos, int t_cap) {
  return max_pos < 0 ? 1 : max_pos / (CH * NCLS * la_attention_spb(t_cap)) + 1;
}

// dynamic LDS of the kernel: the fixed part, then the largest of the ring,
// the tail (branch paths of NT tiles, rows of TP tiles: trows each, K and V)
// and the fold states
template <typename T, int DH, int TP, int TPW>
static size_t attn_lds(int trows) {
  constexpr int ROWB = AttnT<T, DH>::ROWB, NDT = AttnT<T, DH>::NDT, NT = TP * TPW;
  const size_t fix = ((size_t)NT * (16 * ROWB + 256) + 1023) & ~(size_t)1023;
  const size_t ring = (size_t)2 * NCLS * 2 * CH * ROWB;
  const size_t tail = (size_t)NT * (16 * 64 + 64) * 4 + (size_t)TP * 2 * trows * ROWB;
  const size_t fold = (size_t)NT * NCLS * 64 * (4 * NDT + 2) * 4;
  return fix + std::max(ring, std::max(tail, fold));
}

template <typename T, int DH, int TP, int TPW>
static void launch_cfg(const LaAttnArgs& a, int grid, size_t lds, hipStream_t st) {
  static const bool attr = hipFuncSetAttribute((const void*)&la_attn_kernel<T, DH, TP, TPW>,
                                               hipFuncAttributeMaxDynamicSharedMemorySize, LDS_BYTES) == hipSuccess;
  (void)attr;
  hipLaunchKernelGGL((la_attn_kernel<T, DH, TP, TPW>), dim3(grid), dim3(64 * NCLS * TP), lds, st, a);
}

// compute units of the current device (cached per device)
static int cu_count() {
  static int cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cache[dev] == 0) {
    int n = 0;
    cache[dev] = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0 ? n : 256;
  }
  return cache[dev];
}

template <typename T, int DH>
static int launch_dh(LaAttnArgs a, hipStream_t st) {
  const int group = a.H / a.Hkv;
  const int tiles = group * ((a.Q + 15) / 16);
  // staged tail rows per tile (K and V): what the LDS left after the fixed
  // part and the branch paths holds, at least the committed rows of a tail
  // chunk (< 32) and the EP positions of one branch; at most those of 16
  // branches
  constexpr int ROWB = AttnT<T, DH>::ROWB, RPB = 1024 / ROWB;
  const int EP = a.n_tail > 0 ? a.max_pos - a.shared_end + 1 : 0;
  auto rows_for = [&](int tp, int nt) {
    const size_t fix = (((size_t)nt * (16 * ROWB + 256)) + 1023) & ~(size_t)1023;
    const size_t paths = (size_t)nt * (16 * 64 + 64) * 4;
    const int fit = (int)((LDS_BYTES - fix - paths) / ((size_t)tp * 2 * ROWB)) / RPB * RPB;
    const int want = ((CH - 1 + 16 * EP) + RPB - 1) / RPB * RPB;
    return std::min(fit, want);
  };
  const int need_rows = ((CH - 1 + EP) + RPB - 1) / RPB * RPB;
  // tiles per workgroup: 4 (two tile pairs) while that still gives about 160
  // workgroups, else 2, or 1 for a single tile
  const int kv = 8 * ((a.Hkv + 7) / 8);
  auto wgs = [&](int nt) { return kv * ((tiles + nt - 1) / nt) * a.nsplit; };
  int nt = tiles == 1 ? 1 : (tiles >= 3 && wgs(4) >= 160) ? 4 : 2;
  // two tiles: two pair slots of one tile each (8 waves, two per SIMD)
  const int tp = nt == 1 ? 1 : 2;
  const int tpw = nt / tp;
  if (a.n_tail > 0 && rows_for(tp, nt) < need_rows) return -2;
  a.trows = a.n_tail > 0 ? rows_for(tp, nt) : 0;
  a.rgroups = (tiles + nt - 1) / nt;
  // Two workgroups per row group in the tail's split, unless that adds a
  // round of workgroups to the grid (one workgroup fits a CU at a time).
  auto per_head = [&](bool half) {
    int n = 0;
    for (int s = 0; s < a.nsplit; ++s) n += a.rgroups * (half && split_has_tail(a, s) ? 2 : 1);
    return n;
  };
  const int ncu = cu_count();
  const int single = per_head(false), doubled = per_head(tpw == 2);
  a.tail_half = tpw == 2 && (kv * doubled + ncu - 1) / ncu <= (kv * single + ncu - 1) / ncu;
  a.wg_head = a.tail_half ? doubled : single;
  const int grid = kv * a.wg_head;
  size_t lds;
  if (nt == 4) lds = attn_lds<T, DH, 2, 2>(a.trows);
  else if (nt == 2) lds = attn_lds<T, DH, 2, 1>(a.trows);
  else lds = attn_lds<T, DH, 1, 1>(a.trows);
  if (lds > LDS_BYTES) return -2;
  if (nt == 4) launch_cfg<T, DH, 2, 2>(a, grid, lds, st);
  else if (nt == 2) launch_cfg<T, DH, 2, 1>(a, grid, lds, st);
  else launch_cfg<T, DH, 1, 1>(a, grid, lds, st);
  if (a.nsplit > 1) {
    const int wpk = (a.Q * group * (DH / 4) + 255) / 256;
    hipLaunchKernelGGL((la_attn_merge_kernel<T, DH>), dim3(kv * wpk), dim3(256), 0, st, a);
  }
  return 0;
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
  // at most one tail chunk per class; tail positions come from a 64-entry path table per branch
  if (a.n_tail > NTAIL || (tail && a.max_pos - se >= 64)) return -2;
  a.scale_log2 = a.scale * 1.4426950408889634f;
  // key splits: the split of the last chunk any row reaches, plus one
  const int last_chunk = tail ? a.tail0 + a.n_tail - 1 : a.class_last;
  a.spb = la_attention_spb(a.T_cap);
  a.nsplit = last_chunk / (NCLS * a.spb) + 1;
  if (a.nsplit > 1 && (a.part_o == nullptr || a.part_ml == nullptr || a.nsplit > a.max_splits)) return -2;
  int rc;
  if (dtype == LA_DT_BF16) {
    if (a.dh == 128) rc = launch_dh<bf16_t, 128>(a, st);
    else if (a.dh == 64) rc = launch_dh<bf16_t, 64>(a, st);
    else return -2;
  } else {
    if (a.dh == 16) rc = launch_dh<float, 16>(a, st);
    else if (a.dh == 64) rc = launch_dh<float, 64>(a, st);
    else return -2;
  }
  if (rc) return rc;
  return hipGetLastError() == hipSuccess ? 0 : -1;
}
