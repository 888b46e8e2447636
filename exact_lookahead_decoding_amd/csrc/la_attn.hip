// Lookahead-mask attention over the committed prefix and the packed rows.
//
// "M7.3 - Lookahead Decoding", 0x04A / 0x04B / 0x07A: every packed row sees
// the whole committed prefix plus the rows of its own branch; an ordinary
// causal kernel cannot express this, and a dense additive mask costs
// B*H*Q*(K_in+Q) elements.  Here the mask never exists as a tensor: row i
// sees exactly logical positions 0 .. pos_i, position t taken from the
// cache when t < shared_end and through the row's branch path otherwise.
//
// Work decomposition (gfx950, wave64):
//   * grid = (KV head x row split, key span of 128 positions), 4 waves; a
//     wave owns up to TPW tiles of 16 query rows (one q-head each; the GQA
//     group's q-heads share the staged K/V);
//   * phase A: the span's committed K (row-major) and V (transposed) are
//     staged once in LDS; every 16-key group that lies entirely below
//     shared_end is folded with S^T = K Q^T (16x16x32 bf16 MFMA: one query
//     row per lane column, so softmax statistics stay in-lane) and
//     O^T += V^T P^T (16x16x16 bf16 MFMA, P as a hi + lo bf16 pair);
//   * phase B (only spans that reach the packed rows): the straddling
//     committed keys and every packed row's K/V (the workspace) are staged
//     in the same LDS in one bulk load; groups that reach past shared_end
//     are folded once per branch present in the tile, each lane addressing
//     its key's LDS row through the branch path; rows of other branches see
//     the group fully masked, which leaves their state bit-for-bit unchanged;
//   * each span writes (m, l, O) per row; a second kernel folds the spans in
//     increasing order and normalises.
// The reduction tree (16-key groups folded in order inside 128-key spans,
// spans folded in order) depends only on logical positions, so a row gets
// the same bits whether it is alone (autoregressive step) or packed.
#include <algorithm>

#include "la_common.h"
#include "la_kernels.h"

#define SPAN 128
#define GK 16
#define NEG_INF (-__builtin_inff())
#define PATH_LDS 1024

template <typename T, int DH> struct AttnT;

template <int DH> struct AttnT<bf16_t, DH> {
  static constexpr int QK_STEPS = DH / 32;
  static constexpr int KROW = DH + 8;
  static constexpr int PIECES = DH / 8;       // 16-byte pieces per row
  typedef bf16x8 qfrag;
  static __device__ __forceinline__ qfrag load_q(const bf16_t* qrow, int g, int s) {
    return *(const bf16x8*)(qrow + 32 * s + 8 * g);
  }
  static __device__ __forceinline__ f32x4 qk(const bf16_t* krow, int g, const qfrag* qf) {
    f32x4 acc = {0, 0, 0, 0};
#pragma unroll
    for (int s = 0; s < QK_STEPS; ++s) acc = mfma_bf16_32(*(const bf16x8*)(krow + 32 * s + 8 * g), qf[s], acc);
    return acc;
  }
  static __device__ __forceinline__ void split_p(const float* p, i16x4& bh, i16x4& bl) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bf16_t hi = f2bf(p[i]);
      bh[i] = (short)hi;
      bl[i] = (short)f2bf(p[i] - bf2f(hi));
    }
  }
  // O^T[16dt + 4g + i][row] += V^T rows of the 4 keys of lane group g (contiguous from r0) times P^T
  static __device__ __forceinline__ void pv_contig(f32x4* o, const bf16_t* vt, int vrow, int r0, int c16,
                                                   const float* p) {
    i16x4 bh, bl;
    split_p(p, bh, bl);
#pragma unroll
    for (int dt = 0; dt < DH / 16; ++dt) {
      const i16x4 a = *(const i16x4*)(vt + (16 * dt + c16) * vrow + r0);
      o[dt] = mfma_bf16_16(a, bh, o[dt]);
      o[dt] = mfma_bf16_16(a, bl, o[dt]);
    }
  }
  // same with the 4 keys at arbitrary LDS rows r[0..3]
  static __device__ __forceinline__ void pv_rows(f32x4* o, const bf16_t* vt, int vrow, const int* r, int c16,
                                                 const float* p) {
    i16x4 bh, bl;
    split_p(p, bh, bl);
#pragma unroll
    for (int dt = 0; dt < DH / 16; ++dt) {
      const bf16_t* col = vt + (16 * dt + c16) * vrow;
      i16x4 a;
      a[0] = (short)col[r[0]];
      a[1] = (short)col[r[1]];
      a[2] = (short)col[r[2]];
      a[3] = (short)col[r[3]];
      o[dt] = mfma_bf16_16(a, bh, o[dt]);
      o[dt] = mfma_bf16_16(a, bl, o[dt]);
    }
  }
  // stage one 16-byte piece of a key's K row and V row (V transposed)
  static __device__ __forceinline__ void put(bf16_t* k, bf16_t* v, int vrow, int row, const bf16_t* ksrc,
                                             const bf16_t* vsrc, int piece) {
    *(u32x4*)(k + row * KROW + 8 * piece) = ksrc ? *(const u32x4*)(ksrc + 8 * piece) : u32x4{0, 0, 0, 0};
    u32x4 vv = vsrc ? *(const u32x4*)(vsrc + 8 * piece) : u32x4{0, 0, 0, 0};
    const bf16_t* ve = (const bf16_t*)&vv;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[(8 * piece + e) * vrow + row] = ve[e];
  }
  static __device__ __forceinline__ void put_regs(bf16_t* k, bf16_t* v, int vrow, int row, const u32x4& kk,
                                                  const u32x4& vv, int piece) {
    *(u32x4*)(k + row * KROW + 8 * piece) = kk;
    const bf16_t* ve = (const bf16_t*)&vv;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[(8 * piece + e) * vrow + row] = ve[e];
  }
  static constexpr int v_elems(int rows) { return DH * (rows + 8); }
  static constexpr int v_row_len(int rows) { return rows + 8; }
};

template <int DH> struct AttnT<float, DH> {
  static constexpr int QK_STEPS = DH / 4;
  static constexpr int KROW = DH + 4;
  static constexpr int PIECES = DH / 4;
  typedef float qfrag;
  static __device__ __forceinline__ qfrag load_q(const float* qrow, int g, int s) { return qrow[4 * s + g]; }
  static __device__ __forceinline__ f32x4 qk(const float* krow, int g, const qfrag* qf) {
    f32x4 acc = {0, 0, 0, 0};
#pragma unroll
    for (int s = 0; s < QK_STEPS; ++s) acc = mfma_f32_4(krow[4 * s + g], qf[s], acc);
    return acc;
  }
  static __device__ __forceinline__ void pv_contig(f32x4* o, const float* v, int vrow, int r0, int c16,
                                                   const float* p) {
#pragma unroll
    for (int dt = 0; dt < DH / 16; ++dt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) o[dt] = mfma_f32_4(v[(r0 + i) * vrow + 16 * dt + c16], p[i], o[dt]);
    }
  }
  static __device__ __forceinline__ void pv_rows(f32x4* o, const float* v, int vrow, const int* r, int c16,
                                                 const float* p) {
#pragma unroll
    for (int dt = 0; dt < DH / 16; ++dt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) o[dt] = mfma_f32_4(v[r[i] * vrow + 16 * dt + c16], p[i], o[dt]);
    }
  }
  static __device__ __forceinline__ void put(float* k, float* v, int vrow, int row, const float* ksrc,
                                             const float* vsrc, int piece) {
    *(u32x4*)(k + row * KROW + 4 * piece) = ksrc ? *(const u32x4*)(ksrc + 4 * piece) : u32x4{0, 0, 0, 0};
    *(u32x4*)(v + row * vrow + 4 * piece) = vsrc ? *(const u32x4*)(vsrc + 4 * piece) : u32x4{0, 0, 0, 0};
  }
  static __device__ __forceinline__ void put_regs(float* k, float* v, int vrow, int row, const u32x4& kk,
                                                  const u32x4& vv, int piece) {
    *(u32x4*)(k + row * KROW + 4 * piece) = kk;
    *(u32x4*)(v + row * vrow + 4 * piece) = vv;
  }
  static constexpr int v_elems(int rows) { return rows * (DH + 4); }
  static constexpr int v_row_len(int) { return DH + 4; }
};

// One online-softmax step of tile I over the keys [K0, K0 + 16).  Rows not in
// MINE see the group fully masked: m stays, the scale is exactly 1, P is 0,
// so their state does not change.
#define LA_STEP(I, SRAW, K0, MINE, PVCALL)                                                  \
  do {                                                                                      \
    float sv[4];                                                                            \
    float gm = NEG_INF;                                                                     \
    _Pragma("unroll") for (int q4 = 0; q4 < 4; ++q4) {                                      \
      const int t_ = (K0) + 4 * g + q4;                                                     \
      sv[q4] = ((MINE) && t_ <= pos[I]) ? (SRAW)[q4] * sl2 : NEG_INF;                       \
      gm = fmaxf(gm, sv[q4]);                                                               \
    }                                                                                       \
    gm = fmaxf(gm, __shfl_xor(gm, 16, 64));                                                 \
    gm = fmaxf(gm, __shfl_xor(gm, 32, 64));                                                 \
    const float mn = fmaxf(m[I], gm);                                                       \
    float p[4];                                                                             \
    float sc;                                                                               \
    if (mn == NEG_INF) {                                                                    \
      sc = 1.f;                                                                             \
      p[0] = p[1] = p[2] = p[3] = 0.f;                                                      \
    } else {                                                                                \
      sc = (m[I] == NEG_INF) ? 0.f : exp2f(m[I] - mn);                                      \
      _Pragma("unroll") for (int q4 = 0; q4 < 4; ++q4) p[q4] =                              \
          (sv[q4] == NEG_INF) ? 0.f : exp2f(sv[q4] - mn);                                   \
    }                                                                                       \
    float ps = (p[0] + p[1]) + (p[2] + p[3]);                                               \
    ps += __shfl_xor(ps, 16, 64);                                                           \
    ps += __shfl_xor(ps, 32, 64);                                                           \
    l[I] = l[I] * sc + ps;                                                                  \
    m[I] = mn;                                                                              \
    _Pragma("unroll") for (int dt = 0; dt < DH / 16; ++dt) o[I][dt] *= sc;                  \
    PVCALL;                                                                                 \
  } while (0)

template <typename T, int DH, int QB, int TPW>
__global__ void __launch_bounds__(256) la_attn_kernel(LaAttnArgs a) {
  typedef AttnT<T, DH> AT;
  constexpr int KROW = AT::KROW;
  constexpr int A_ELEMS = SPAN * KROW + AT::v_elems(SPAN);
  constexpr int B_ELEMS = QB * KROW + AT::v_elems(QB);
  constexpr int ELEMS = A_ELEMS > B_ELEMS ? A_ELEMS : B_ELEMS;
  __shared__ __attribute__((aligned(16))) T lds[ELEMS];
  __shared__ int pth_lds[PATH_LDS];
  __shared__ int plen_lds[256];

  const int g_kv = blockIdx.x / a.rsplit;
  const int rsp = blockIdx.x % a.rsplit;
  const int span = blockIdx.y;
  const int t0s = span * SPAN;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int group = a.H / a.Hkv;
  const T* kc = (const T*)a.kc + (size_t)g_kv * a.T_cap * DH;
  const T* vc = (const T*)a.vc + (size_t)g_kv * a.T_cap * DH;
  const T* kw = (const T*)a.kw + (size_t)g_kv * a.ws_cap * DH;
  const T* vw = (const T*)a.vw + (size_t)g_kv * a.ws_cap * DH;
  const float sl2 = a.scale * 1.4426950408889634f;          // scores in log2 units
  const int rtiles = (a.Q + 15) / 16;
  const int ntiles = group * rtiles;

  // ---- phase A staging: committed keys [t0s, shared_hi) of the span ----
  T* ka = lds;
  T* va = lds + SPAN * KROW;
  constexpr int VA_ROW = AT::v_row_len(SPAN);
  const int shared_hi = min(t0s + SPAN, a.shared_end);
  const int nA = max(0, shared_hi - t0s);
  {
    // every thread issues all of its loads before its first LDS store
    constexpr int PER = (SPAN * AT::PIECES + 255) / 256;
    u32x4 kr[PER], vr[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int idx = threadIdx.x + 256 * j;
      const int key = idx / AT::PIECES, piece = idx % AT::PIECES;
      if (key < nA) {
        const size_t off = (size_t)(t0s + key) * DH + piece * (16 / sizeof(T));
        kr[j] = *(const u32x4*)(kc + off);
        vr[j] = *(const u32x4*)(vc + off);
      }
    }
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int idx = threadIdx.x + 256 * j;
      const int key = idx / AT::PIECES, piece = idx % AT::PIECES;
      if (key < nA) AT::put_regs(ka, va, VA_ROW, key, kr[j], vr[j], piece);
    }
  }

  // ---- per-tile state ----
  typename AT::qfrag qf[TPW][AT::QK_STEPS];
  float m[TPW], l[TPW];
  f32x4 o[TPW][DH / 16];
  int pos[TPW], br[TPW], hh[TPW], row[TPW], tmax[TPW];
  bool rvalid[TPW];
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    const int tile = (rsp * 4 + wave) * TPW + i;
    const bool tv = tile < ntiles;
    hh[i] = tv ? g_kv * group + tile / rtiles : 0;
    row[i] = tv ? (tile % rtiles) * 16 + c16 : a.Q;
    rvalid[i] = tv && row[i] < a.Q;
    pos[i] = rvalid[i] ? a.pos[row[i]] : -1;
    br[i] = rvalid[i] ? a.branch[row[i]] : -1;
    int t = pos[i];
    for (int s = 32; s > 0; s >>= 1) t = max(t, __shfl_xor(t, s, 64));
    tmax[i] = t;
    const T* qrow = (const T*)a.q + ((size_t)(rvalid[i] ? row[i] : 0) * a.H + hh[i]) * DH;
#pragma unroll
    for (int s = 0; s < AT::QK_STEPS; ++s) {
      qf[i][s] = AT::load_q(qrow, g, s);
      if (!rvalid[i]) qf[i][s] = typename AT::qfrag{};
    }
    m[i] = NEG_INF;
    l[i] = 0.f;
#pragma unroll
    for (int dt = 0; dt < DH / 16; ++dt) o[i][dt] = f32x4{0, 0, 0, 0};
  }
  __syncthreads();

  // ---- phase A: groups entirely below shared_end ----
  const int g0 = (a.shared_end / GK) * GK;                  // first group holding a key >= shared_end
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    const int kend = min(min(t0s + SPAN, tmax[i] + 1), g0);
    for (int k0 = t0s; k0 < kend; k0 += GK) {
      const f32x4 s = AT::qk(ka + (k0 - t0s + c16) * KROW, g, qf[i]);
      LA_STEP(i, s, k0, true, AT::pv_contig(o[i], va, VA_ROW, k0 - t0s + 4 * g, c16, p));
    }
  }

  // ---- phase B: groups reaching the packed rows ----
  const int b0 = max(t0s, g0);
  if (a.max_pos >= b0 && b0 < t0s + SPAN) {
    __syncthreads();                                        // phase A is done with the staging area
    T* kb = lds;
    T* vb = lds + QB * KROW;
    constexpr int VB_ROW = AT::v_row_len(QB);
    const int zero_row = GK + a.n_ws;                       // all-zero row: keys past a branch's path
    const int nrows = zero_row + 1;
    constexpr int PERB = 8;                                 // pieces per thread per batch
    for (int base = 0; base < nrows * AT::PIECES; base += 256 * PERB) {
      u32x4 kr[PERB], vr[PERB];
#pragma unroll
      for (int j = 0; j < PERB; ++j) {
        const int idx = base + threadIdx.x + 256 * j;
        const int r = idx / AT::PIECES, piece = idx % AT::PIECES;
        const T* ksrc = nullptr;
        const T* vsrc = nullptr;
        if (r < GK) {
          const int t = g0 + r;
          if (t < a.shared_end) {
            ksrc = kc + (size_t)t * DH;
            vsrc = vc + (size_t)t * DH;
          }
        } else if (r < zero_row) {
          ksrc = kw + (size_t)(r - GK) * DH;
          vsrc = vw + (size_t)(r - GK) * DH;
        }
        const int off = piece * (16 / sizeof(T));
        kr[j] = (r < nrows && ksrc) ? *(const u32x4*)(ksrc + off) : u32x4{0, 0, 0, 0};
        vr[j] = (r < nrows && vsrc) ? *(const u32x4*)(vsrc + off) : u32x4{0, 0, 0, 0};
      }
#pragma unroll
      for (int j = 0; j < PERB; ++j) {
        const int idx = base + threadIdx.x + 256 * j;
        const int r = idx / AT::PIECES, piece = idx % AT::PIECES;
        if (r < nrows) AT::put_regs(kb, vb, VB_ROW, r, kr[j], vr[j], piece);
      }
    }
    const int ptot = a.nb * a.maxp;
    const bool path_in_lds = ptot <= PATH_LDS && a.nb <= 256;
    if (path_in_lds) {
      for (int idx = threadIdx.x; idx < ptot; idx += 256) pth_lds[idx] = a.path[idx];
      for (int idx = threadIdx.x; idx < a.nb; idx += 256) plen_lds[idx] = a.path_len[idx];
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int kend = min(t0s + SPAN, tmax[i] + 1);
      for (int k0 = b0; k0 < kend; k0 += GK) {
        bool pending = rvalid[i] && pos[i] >= k0;
        while (true) {
          const unsigned long long bal = __ballot(pending);
          if (bal == 0ull) break;
          const int b = __shfl(br[i], __ffsll((long long)bal) - 1, 64);
          const int* pth = path_in_lds ? pth_lds + b * a.maxp : a.path + (size_t)b * a.maxp;
          const int plen = path_in_lds ? plen_lds[b] : a.path_len[b];
          auto key_row = [&](int t) -> int {
            if (t < a.shared_end) return t - g0;
            const int e = t - a.shared_end;
            return e < plen ? GK + pth[e] : zero_row;
          };
          const f32x4 s = AT::qk(kb + key_row(k0 + c16) * KROW, g, qf[i]);
          int rr[4];
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) rr[q4] = key_row(k0 + 4 * g + q4);
          const bool mine = rvalid[i] && br[i] == b;
          LA_STEP(i, s, k0, mine, AT::pv_rows(o[i], vb, VB_ROW, rr, c16, p));
          pending = pending && br[i] != b;
        }
      }
    }
  }

  // ---- span partials ----
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    if (!rvalid[i]) continue;
    const size_t base = ((size_t)span * a.H + hh[i]) * a.Q + row[i];
    if (g == 0) {
      a.part_ml[base * 2] = m[i];
      a.part_ml[base * 2 + 1] = l[i];
    }
    float* po = a.part_o + base * DH;
#pragma unroll
    for (int dt = 0; dt < DH / 16; ++dt) *(f32x4*)(po + 16 * dt + 4 * g) = o[i][dt];
  }
}

// fold the span partials in increasing span order, normalise, store
template <typename T>
__global__ void la_attn_merge_kernel(LaAttnArgs a) {
  const int row = blockIdx.x, h = blockIdx.y, d = threadIdx.x;
  float M = NEG_INF, L = 0.f, O = 0.f;
  for (int s = 0; s < a.n_spans; ++s) {
    const float* ml = a.part_ml + (((size_t)s * a.H + h) * a.Q + row) * 2;
    const float ms = ml[0];
    if (ms == NEG_INF) continue;
    const float ls = ml[1];
    const float os = a.part_o[(((size_t)s * a.H + h) * a.Q + row) * a.dh + d];
    const float mn = fmaxf(M, ms);
    const float wa = (M == NEG_INF) ? 0.f : exp2f(M - mn);
    const float wb = exp2f(ms - mn);
    L = L * wa + ls * wb;
    O = O * wa + os * wb;
    M = mn;
  }
  st<T>((T*)a.o + ((size_t)row * a.H + h) * a.dh + d, O / L);
}

int la_attention_spans(int max_pos) { return max_pos / SPAN + 1; }

template <typename T, int DH, int QB, int TPW>
static void launch_one(const LaAttnArgs& a, hipStream_t st) {
  hipLaunchKernelGGL((la_attn_kernel<T, DH, QB, TPW>), dim3(a.Hkv * a.rsplit, a.n_spans), dim3(256), 0, st, a);
  hipLaunchKernelGGL((la_attn_merge_kernel<T>), dim3(a.Q, a.H), dim3(DH), 0, st, a);
}

template <typename T, int DH>
static int launch_dh(LaAttnArgs a, hipStream_t st) {
  // split the query tiles over workgroups so that the grid fills the chip; a wave owns 1 or 4 tiles
  const int group = a.H / a.Hkv;
  const int ntiles = group * ((a.Q + 15) / 16);
  const int units = a.Hkv * a.n_spans;
  int rsplit = std::max(1, std::min((512 + units - 1) / units, (ntiles + 3) / 4));
  int tpw = (ntiles + 4 * rsplit - 1) / (4 * rsplit);
  if (tpw > 1) {
    tpw = 4;
    rsplit = (ntiles + 15) / 16;
  }
  a.rsplit = rsplit;
  if (a.n_ws < 0 || a.n_ws > a.ws_cap) return -2;
  const int rows_b = GK + a.n_ws + 1;                       // straddle keys + workspace rows + zero row
  if (rows_b <= 128) {
    if (tpw == 1) launch_one<T, DH, 128, 1>(a, st);
    else launch_one<T, DH, 128, 4>(a, st);
  } else if (rows_b <= 256) {
    if (tpw == 1) launch_one<T, DH, 256, 1>(a, st);
    else launch_one<T, DH, 256, 4>(a, st);
  } else {
    return -2;
  }
  return 0;
}

int la_attention_launch(int dtype, const LaAttnArgs& a, hipStream_t st) {
  if (a.Q <= 0) return 0;
  if (a.H % a.Hkv != 0) return -2;
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
