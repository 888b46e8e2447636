// Lookahead-mask attention over the committed prefix and the packed rows.
//
// "M7.3 - Lookahead Decoding", 0x04A / 0x04B / 0x07A: every packed row sees
// the whole committed prefix plus the rows of its own branch; an ordinary
// causal kernel cannot express this, and a dense additive mask costs
// B*H*Q*(K_in+Q) elements.  Here the mask never exists as a tensor: row i
// sees exactly logical positions 0 .. pos_i, position t taken from the
// cache when t < shared_end and from the row's branch path otherwise.
//
// Work decomposition (gfx950, wave64):
//   * grid = (KV head, key span of 128 positions); 4 waves per workgroup;
//   * the span's cache K (row-major) and V (transposed) are staged once in
//     LDS and shared by every query row of every q-head of the GQA group;
//   * a wave owns a 16-row tile of one q-head; S^T = K Q^T on MFMA (the
//     16x16 result holds one query row per lane column), then an online
//     softmax step and O^T += V^T P^T on MFMA, per 16-key group;
//   * groups that reach past shared_end are rebuilt per branch from the
//     branch path (cache rows below shared_end, workspace rows above) in a
//     per-wave LDS tile; rows of other branches see that group fully masked,
//     which leaves their state bit-for-bit unchanged;
//   * each span writes (m, l, O) per row; a second kernel merges spans in
//     increasing order.
// The reduction tree (16-key groups folded in order inside 128-key spans,
// spans folded in order) depends only on logical positions, so a row gets
// the same bits whether it is alone (autoregressive step) or packed.
#include "la_common.h"
#include "la_kernels.h"

#define SPAN 128
#define GK 16
#define NEG_INF (-__builtin_inff())

template <typename T, int DH> struct AttnT;

template <int DH> struct AttnT<bf16_t, DH> {
  static constexpr int QK_STEPS = DH / 32;
  static constexpr int KROW = DH + 8;         // K tile row (elements)
  static constexpr int VROW = SPAN + 8;       // V^T row for the span (elements)
  static constexpr int VBROW = GK + 8;        // V^T row for a branch group
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
  // O^T[16dt + 4g + i][row] += sum_k V[key0 + k][16dt + c16] P[row][key0 + k]
  // P enters the bf16 MFMA as a hi + lo pair (about 16 significant bits), so
  // the probabilities are not truncated to bf16 precision.
  static __device__ __forceinline__ void pv(f32x4* o, const bf16_t* vt, int vrow, int key0, int g, int c16,
                                            const float* p) {
    i16x4 bh, bl;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bf16_t hi = f2bf(p[i]);
      bh[i] = (short)hi;
      bl[i] = (short)f2bf(p[i] - bf2f(hi));
    }
#pragma unroll
    for (int dt = 0; dt < DH / 16; ++dt) {
      const i16x4 a = *(const i16x4*)(vt + (16 * dt + c16) * vrow + key0 + 4 * g);
      o[dt] = mfma_bf16_16(a, bh, o[dt]);
      o[dt] = mfma_bf16_16(a, bl, o[dt]);
    }
  }
  // stage one key's K row and V column into LDS
  static __device__ __forceinline__ void put(bf16_t* kdst, bf16_t* vt, int vrow, int key, const bf16_t* ksrc,
                                             const bf16_t* vsrc, int piece) {
    *(u32x4*)(kdst + 8 * piece) = ksrc ? *(const u32x4*)(ksrc + 8 * piece) : u32x4{0, 0, 0, 0};
    u32x4 v = vsrc ? *(const u32x4*)(vsrc + 8 * piece) : u32x4{0, 0, 0, 0};
    const bf16_t* ve = (const bf16_t*)&v;
#pragma unroll
    for (int e = 0; e < 8; ++e) vt[(8 * piece + e) * vrow + key] = ve[e];
  }
  static constexpr int PIECES = DH / 8;
};

template <int DH> struct AttnT<float, DH> {
  static constexpr int QK_STEPS = DH / 4;
  static constexpr int KROW = DH + 4;
  static constexpr int VROW = DH + 4;         // V kept row-major [key][dh] for fp32
  static constexpr int VBROW = DH + 4;
  typedef float qfrag;
  static __device__ __forceinline__ qfrag load_q(const float* qrow, int g, int s) { return qrow[4 * s + g]; }
  static __device__ __forceinline__ f32x4 qk(const float* krow, int g, const qfrag* qf) {
    f32x4 acc = {0, 0, 0, 0};
#pragma unroll
    for (int s = 0; s < QK_STEPS; ++s) acc = mfma_f32_4(krow[4 * s + g], qf[s], acc);
    return acc;
  }
  static __device__ __forceinline__ void pv(f32x4* o, const float* v, int vrow, int key0, int g, int c16,
                                            const float* p) {
#pragma unroll
    for (int dt = 0; dt < DH / 16; ++dt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) o[dt] = mfma_f32_4(v[(key0 + 4 * g + i) * vrow + 16 * dt + c16], p[i], o[dt]);
    }
  }
  static __device__ __forceinline__ void put(float* kdst, float* v, int vrow, int key, const float* ksrc,
                                             const float* vsrc, int piece) {
    *(u32x4*)(kdst + 4 * piece) = ksrc ? *(const u32x4*)(ksrc + 4 * piece) : u32x4{0, 0, 0, 0};
    *(u32x4*)(v + key * vrow + 4 * piece) = vsrc ? *(const u32x4*)(vsrc + 4 * piece) : u32x4{0, 0, 0, 0};
  }
  static constexpr int PIECES = DH / 4;
};

__device__ __forceinline__ void wave_lds_sync() {
  __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_wave_barrier();
}

template <typename T, int DH>
__global__ void __launch_bounds__(256) la_attn_kernel(LaAttnArgs a) {
  typedef AttnT<T, DH> AT;
  constexpr int KROW = AT::KROW, VROW = AT::VROW, VBROW = AT::VBROW;
  constexpr bool VT = sizeof(T) == 2;                  // V transposed in LDS (bf16)
  constexpr int VSPAN = VT ? DH * VROW : SPAN * VROW;  // elements
  constexpr int VBR = VT ? DH * VBROW : GK * VBROW;
  __shared__ __attribute__((aligned(16))) T ks[SPAN * KROW];
  __shared__ __attribute__((aligned(16))) T vs[VSPAN];
  __shared__ __attribute__((aligned(16))) T kb_all[4][GK * KROW];
  __shared__ __attribute__((aligned(16))) T vb_all[4][VBR];

  const int g_kv = blockIdx.x;
  const int span = blockIdx.y;
  const int t0s = span * SPAN;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int group = a.H / a.Hkv;
  const T* kc = (const T*)a.kc + (size_t)g_kv * a.T_cap * DH;
  const T* vc = (const T*)a.vc + (size_t)g_kv * a.T_cap * DH;
  const T* kw = (const T*)a.kw + (size_t)g_kv * a.ws_cap * DH;
  const T* vw = (const T*)a.vw + (size_t)g_kv * a.ws_cap * DH;
  const int shared_hi = min(t0s + SPAN, a.shared_end);      // cache keys of this span: [t0s, shared_hi)

  // ---- stage the span's cache keys (all waves) ----
  for (int idx = threadIdx.x; idx < SPAN * AT::PIECES; idx += 256) {
    const int key = idx / AT::PIECES, piece = idx % AT::PIECES;
    const int t = t0s + key;
    const bool ok = t < shared_hi;
    AT::put(ks + key * KROW, vs, VT ? VROW : VROW, key, ok ? kc + (size_t)t * DH : nullptr,
            ok ? vc + (size_t)t * DH : nullptr, piece);
  }
  __syncthreads();

  T* kb = kb_all[wave];
  T* vb = vb_all[wave];
  const int rtiles = (a.Q + 15) / 16;
  const int ntiles = group * rtiles;
  const float sl2 = a.scale * 1.4426950408889634f;           // scores in log2 units

  for (int tile = wave; tile < ntiles; tile += 4) {
    const int h = g_kv * group + tile / rtiles;
    const int row = (tile % rtiles) * 16 + c16;
    const bool rvalid = row < a.Q;
    const int pos = rvalid ? a.pos[row] : -1;
    const int br = rvalid ? a.branch[row] : -1;
    int tmax = pos;
    for (int o = 32; o > 0; o >>= 1) tmax = max(tmax, __shfl_xor(tmax, o, 64));
    if (tmax < t0s) {
      // no row of this tile reaches the span: empty partials
      if (rvalid && g == 0) {
        float* ml = a.part_ml + (((size_t)span * a.H + h) * a.Q + row) * 2;
        ml[0] = NEG_INF;
        ml[1] = 0.f;
      }
      if (rvalid) {
        float* po = a.part_o + (((size_t)span * a.H + h) * a.Q + row) * DH;
        for (int dt = 0; dt < DH / 16; ++dt) *(f32x4*)(po + 16 * dt + 4 * g) = f32x4{0, 0, 0, 0};
      }
      continue;
    }
    typename AT::qfrag qf[AT::QK_STEPS];
    {
      const T* qrow = (const T*)a.q + ((size_t)(rvalid ? row : 0) * a.H + h) * DH;
#pragma unroll
      for (int s = 0; s < AT::QK_STEPS; ++s) {
        qf[s] = AT::load_q(qrow, g, s);
        if (!rvalid) qf[s] = typename AT::qfrag{};
      }
    }
    float m = NEG_INF, l = 0.f;
    f32x4 o[DH / 16];
#pragma unroll
    for (int dt = 0; dt < DH / 16; ++dt) o[dt] = f32x4{0, 0, 0, 0};

    // one online-softmax step over the 16 keys [k0, k0 + 16) for rows in `mine`
    auto step = [&](const f32x4& sraw, int k0, bool mine, const T* vsrc, int vrow, int vkey0) {
      float sv[4];
      float gm = NEG_INF;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = k0 + 4 * g + i;
        sv[i] = (mine && t <= pos) ? sraw[i] * sl2 : NEG_INF;
        gm = fmaxf(gm, sv[i]);
      }
      gm = fmaxf(gm, __shfl_xor(gm, 16, 64));
      gm = fmaxf(gm, __shfl_xor(gm, 32, 64));
      const float mn = fmaxf(m, gm);
      float p[4];
      float sc;
      if (mn == NEG_INF) {
        sc = 1.f;
        p[0] = p[1] = p[2] = p[3] = 0.f;
      } else {
        sc = (m == NEG_INF) ? 0.f : exp2f(m - mn);
#pragma unroll
        for (int i = 0; i < 4; ++i) p[i] = (sv[i] == NEG_INF) ? 0.f : exp2f(sv[i] - mn);
      }
      float ps = (p[0] + p[1]) + (p[2] + p[3]);
      ps += __shfl_xor(ps, 16, 64);
      ps += __shfl_xor(ps, 32, 64);
      l = l * sc + ps;
      m = mn;
#pragma unroll
      for (int dt = 0; dt < DH / 16; ++dt) o[dt] *= sc;
      AT::pv(o, vsrc, vrow, vkey0, g, c16, p);
    };

    const int kend = min(t0s + SPAN, tmax + 1);
    for (int k0 = t0s; k0 < kend; k0 += GK) {
      if (k0 + GK <= a.shared_end) {
        // every key of the group is in the cache: shared LDS tile
        const f32x4 s = AT::qk(ks + (k0 - t0s + c16) * KROW, g, qf);
        step(s, k0, true, vs, VROW, k0 - t0s);
      } else {
        // group reaches the packed rows: one pass per branch present in the tile
        bool pending = rvalid && pos >= k0;
        while (true) {
          const unsigned long long bal = __ballot(pending);
          if (bal == 0ull) break;
          const int src_lane = __ffsll((long long)bal) - 1;
          const int b = __shfl(br, src_lane, 64);
          const int32_t* pth = a.path + (size_t)b * a.maxp;
          const int plen = a.path_len[b];
          wave_lds_sync();
          for (int idx = lane; idx < GK * AT::PIECES; idx += 64) {
            const int key = idx / AT::PIECES, piece = idx % AT::PIECES;
            const int t = k0 + key;
            const T* ksrc = nullptr;
            const T* vsrc = nullptr;
            if (t < a.shared_end) {
              ksrc = kc + (size_t)t * DH;
              vsrc = vc + (size_t)t * DH;
            } else if (t - a.shared_end < plen) {
              const int wr = pth[t - a.shared_end];
              ksrc = kw + (size_t)wr * DH;
              vsrc = vw + (size_t)wr * DH;
            }
            AT::put(kb + key * KROW, vb, VBROW, key, ksrc, vsrc, piece);
          }
          wave_lds_sync();
          const bool mine = rvalid && br == b;
          const f32x4 s = AT::qk(kb + c16 * KROW, g, qf);
          step(s, k0, mine, vb, VBROW, 0);
          pending = pending && br != b;
        }
      }
    }
    if (rvalid) {
      if (g == 0) {
        float* ml = a.part_ml + (((size_t)span * a.H + h) * a.Q + row) * 2;
        ml[0] = m;
        ml[1] = l;
      }
      float* po = a.part_o + (((size_t)span * a.H + h) * a.Q + row) * DH;
#pragma unroll
      for (int dt = 0; dt < DH / 16; ++dt) *(f32x4*)(po + 16 * dt + 4 * g) = o[dt];
    }
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

template <typename T, int DH>
static void launch_dh(const LaAttnArgs& a, hipStream_t st) {
  hipLaunchKernelGGL((la_attn_kernel<T, DH>), dim3(a.Hkv, a.n_spans), dim3(256), 0, st, a);
  hipLaunchKernelGGL((la_attn_merge_kernel<T>), dim3(a.Q, a.H), dim3(DH), 0, st, a);
}

int la_attention_launch(int dtype, const LaAttnArgs& a, hipStream_t st) {
  if (a.Q <= 0) return 0;
  if (a.H % a.Hkv != 0) return -2;
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
