// Skinny GEMM Y = X W^T for the packed rows (M <= 256), HBM-bound on W.
//
// The target forward of one packed round multiplies a few dozen rows by
// every weight matrix ("M7.3 - Lookahead Decoding", 0x05C row and FLOP
// ledger: token-wise target work over Q rows), so the round's cost is one
// pass over the weights and the kernel's only job is to keep HBM busy:
//   * a workgroup (4 waves) owns 4*NTW output tiles of 16 columns (SwiGLU:
//     4 gate/up tile pairs) and one split of K;
//   * W is stored packed (la_gemm_pack_launch): the MFMA B fragments of one
//     workgroup step lie in one contiguous run of 4*NTW*NKB KB, in the order
//     the DMA instructions read them, so every instruction reads 1 KB
//     contiguous and a workgroup streams one contiguous region; the weight
//     loads are non-temporal, so the single-use stream does not evict the
//     activation rows every workgroup re-reads from L2;
//   * W and X reach LDS through global_load_lds, one 1 KB MFMA fragment per
//     DMA instruction (lane l's 16 bytes at 16 l, read back with
//     conflict-free ds_read_b128), in a ring of DW+1 stages: each wave brings
//     its own W fragments and a quarter of the X fragments shared by all
//     four, DW steps ahead of the MFMAs;
//   * per step: wait for this wave's step (a static vmcnt: every step is the
//     same G loads per wave, steps past the end load 16 bytes of a valid
//     address), a barrier that leaves the later steps in flight, issue step
//     i + DW into the stage step i - 1 used, then the MFMAs.
// The K partition (chunk size, split count) depends on (N, K) only; every
// output element is the same chunk-ordered MFMA sequence (and, with splits,
// the same fixed-order sum of split partials) whatever M is and whichever
// tile slot its row occupies, so a row gets identical bits in a one-row
// autoregressive step and inside a packed lookahead round.
#include <algorithm>

#include "la_common.h"
#include "la_dev.h"
#include "la_kernels.h"

typedef LdsT<16>::T v4u;

#define CPOL_NT 2   // cache policy of a load: non-temporal (streamed once)

template <typename T> struct GT;
template <> struct GT<bf16_t> {
  static constexpr int KC = 128;   // K per chunk: 4 k-blocks of 32
  static constexpr int EPL = 8;    // K elements in a lane's 16-byte piece
};
template <> struct GT<float> {
  static constexpr int KC = 64;    // 4 k-blocks of 16
  static constexpr int EPL = 4;
};

// One k-block: every lane holds 16 bytes of its A row / B column.
//   bf16: one 16x16x32 MFMA; lane group g = l/16 holds k = 8g .. 8g+7.
//   fp32: four 16x16x4 MFMAs; MFMA j takes k = 4g + j of lane group g.
template <typename T> __device__ __forceinline__ f32x4 kblock(v4u a, v4u b, f32x4 c) {
  if constexpr (sizeof(T) == 2) {
    return mfma_bf16_32(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c);
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) c = mfma_f32_4(__uint_as_float(a[j]), __uint_as_float(b[j]), c);
    return c;
  }
}

// A ring step is NKB k-blocks (4 for narrow stages, 2 once the X and W
// fragments of a k-block reach 12 KB); the ring holds DW+1 stages, at most
// 4 (three steps in flight per wave measured fastest on the round's shapes:
// deeper rings only lengthen the queues), and the per-step wait may not
// exceed vmcnt's 63.
constexpr int gemm_nkb(int mt, int ntw) { return mt + 4 * ntw >= 12 ? 2 : 4; }
constexpr int gemm_stage(int mt, int ntw) { return (mt + 4 * ntw) * gemm_nkb(mt, ntw) * 1024; }
constexpr int gemm_loads(int mt, int ntw) { return (ntw + mt / 4) * gemm_nkb(mt, ntw) + (mt % 4) * gemm_nkb(mt, ntw) / 4; }
constexpr int gemm_depth(int mt, int ntw) {
  int d = 3;
  while (d > 1 && (d + 1) * gemm_stage(mt, ntw) > LDS_BYTES) --d;
  while (d > 1 && (d - 1) * gemm_loads(mt, ntw) > 63) --d;
  return d;
}

__device__ __forceinline__ float silu_f(float g) { return g / (1.0f + expf(-g)); }

template <typename T, int EPI>
__device__ __forceinline__ void gemm_store(const LaGemmArgs& a, int m, int n, float v0, float v1) {
  if (EPI == LA_EPI_STORE) {
    st<T>((T*)a.Y + (size_t)m * a.ldy + n, v0);
  } else if (EPI == LA_EPI_RESID) {
    float r = ld<T>((const T*)a.R + (size_t)m * a.ldy + n);
    st<T>((T*)a.Y + (size_t)m * a.ldy + n, v0 + r);
  } else if (EPI == LA_EPI_SWIGLU) {
    st<T>((T*)a.Y + (size_t)m * a.ldy + n, silu_f(v0) * v1);
  } else if (EPI == LA_EPI_F32) {
    ((float*)a.Y)[(size_t)m * a.ldy + n] = v0;
  }
}

// Fused QKV epilogue of packed column n (pair-major inside each head) of row
// m: the value is rounded to the storage type, as a stored projection would
// be; q and k are rotated at the row's logical position with the rotation
// partner from lane ^ 8 (same row, same tile), then written where the
// attention reads them.  Every lane of the wave calls it (the partner
// exchange is a wave operation); rows past M are not stored.
// (cos, sin) of packed column n at row m (1, 0 for v columns and dead lanes)
__device__ __forceinline__ float2 qkv_rope(const LaQkvOut& o, int m, int n, bool live) {
  const int hb = n >> o.lg_dh, j = n & (o.dh - 1);
  if (!live || hb >= o.H + o.Hkv) return make_float2(1.f, 0.f);
  return o.rope[((size_t)o.pos[m] << (o.lg_dh - 1)) + 8 * (j >> 4) + (j & 7)];
}

template <typename T>
__device__ __forceinline__ void qkv_store(const LaQkvOut& o, int m, int n, float v, bool live, float2 cs) {
  const float x = StoreT<T>::round(v);
  const float xp = __shfl_xor(x, 8, 64);
  if (!live) return;
  const int dh = o.dh, half = dh / 2;
  const int hb = n >> o.lg_dh, j = n & (dh - 1), k = j >> 4, c = j & 15;
  const int i = 8 * k + (c & 7);                  // rotation index
  const int d = c < 8 ? i : half + i;             // natural head dimension
  T* dst;
  bool rot = true;
  if (hb < o.H) {
    dst = (T*)o.q + ((size_t)m * o.H + hb) * dh;
  } else {
    const bool isk = hb < o.H + o.Hkv;
    const int g = isk ? hb - o.H : hb - o.H - o.Hkv;
    rot = isk;
    if (m < o.n_direct) dst = (T*)(isk ? o.kc : o.vc) + ((size_t)g * o.T_cap + o.cache_row0 + m) * dh;
    else dst = (T*)(isk ? o.kw : o.vw) + ((size_t)g * o.ws_cap + (m - o.n_direct)) * dh;
  }
  float y = x;
  if (rot) y = c < 8 ? x * cs.x - xp * cs.y : x * cs.x + xp * cs.y;
  st<T>(dst + d, y);
}

template <typename T, int MT, int NTW, int EPI>
__global__ void __launch_bounds__(256) la_gemm_kernel(LaGemmArgs a) {
  constexpr int KC = GT<T>::KC, EPL = GT<T>::EPL, KB = KC / 4;
  constexpr int NKB = gemm_nkb(MT, NTW);         // k-blocks per ring step
  constexpr int DW = gemm_depth(MT, NTW);
  constexpr int R = DW + 1;                      // ring stages
  constexpr int STAGE = gemm_stage(MT, NTW);
  constexpr int WOFF = MT * NKB * 1024;          // W fragments after the X fragments
  constexpr int XF = MT * NKB / 4;               // X fragments per step and wave
  constexpr int G = NTW * NKB + XF;              // DMA instructions per step and wave
  static_assert((MT * NKB) % 4 == 0, "X fragments split evenly over the waves");
  static_assert(G == gemm_loads(MT, NTW), "load count");
  extern __shared__ __attribute__((aligned(1024))) char lds[];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const bool swiglu = (EPI == LA_EPI_SWIGLU) || (a.swiglu_partial != 0);
  const int split = blockIdx.y;
  const int c_begin = (int)(((long)split * a.nchunks) / a.splits);
  const int nc = (int)(((long)(split + 1) * a.nchunks) / a.splits) - c_begin;   // >= 1 (splits <= nchunks)
  const int n = nc * (4 / NKB);                                                  // ring steps

  // tile t of this wave: output columns colw + 16 t (SwiGLU: gate columns
  // colw and their up rows); its fragment for k-block kb sits at packed
  // fragment ((blockIdx.x * nkb + kb) * 4 + wave) * NTW + t
  const int colw = (blockIdx.x * 4 + wave) * 16 * (swiglu ? 1 : NTW);
  const size_t nkb = (size_t)(a.K / KB);
  const T* W = (const T*)a.W;
  const T* X = (const T*)a.X;
  const T* wp[NTW];
#pragma unroll
  for (int t = 0; t < NTW; ++t)
    wp[t] = W + ((((size_t)blockIdx.x * nkb + (size_t)c_begin * 4) * 4 + wave) * NTW + t) * 64 * EPL + lane * EPL;
  // X fragments this wave brings in: f = wave + 4 j is (row tile f / NKB,
  // k-block f % NKB); rows past M load row M - 1 and are never stored
  const T* xp = X + (size_t)c_begin * KC + EPL * g;
  int xoff[XF];
#pragma unroll
  for (int j = 0; j < XF; ++j) {
    const int f = wave + 4 * j;
    xoff[j] = min((f / NKB) * 16 + c16, a.M - 1) * a.ldx + (f % NKB) * KB;
  }

  f32x4 acc[MT][NTW];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int t = 0; t < NTW; ++t) acc[i][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // step i (relative to the split) into stage SL; past the split's last step
  // every lane loads the same valid 16 bytes into a stage nobody reads
  auto issue = [&](auto SL, int i) {
    constexpr int sl = decltype(SL)::value;
    const bool live = i < n;
    const size_t k0 = (size_t)i * (NKB * KB);
    char* stage = lds + sl * STAGE;
#pragma unroll
    for (int t = 0; t < NTW; ++t) {
#pragma unroll
      for (int s = 0; s < NKB; ++s) {
        const T* src = live ? wp[t] + ((size_t)i * NKB + s) * (4 * NTW * 64 * EPL) : W;
        __builtin_amdgcn_global_load_lds((const void*)src,
                                         (lds_void_t*)(stage + WOFF + ((wave * NTW + t) * NKB + s) * 1024), 16, 0,
                                         CPOL_NT);
      }
    }
#pragma unroll
    for (int j = 0; j < XF; ++j) {
      const T* src = live ? xp + xoff[j] + k0 : X;
      __builtin_amdgcn_global_load_lds((const void*)src, (lds_void_t*)(stage + (wave + 4 * j) * 1024), 16, 0, 0);
    }
  };

  // X fragment (mt, s) sits at (mt * NKB + s) KB of the stage, W fragment
  // (wave, t, s) at WOFF + ((wave * NTW + t) * NKB + s) KB; lane l's 16 bytes
  // are at 16 l in both
  auto compute = [&](auto SL) {
    constexpr int sl = decltype(SL)::value;
    const uint32_t xb = lds_addr(lds + sl * STAGE) + 16 * lane;
    const uint32_t wb = xb + WOFF + wave * NTW * NKB * 1024;
    v4u A[2][MT], B[2][NTW];
    auto fetch = [&](auto S, auto BUF) {
      constexpr int s = decltype(S)::value, b = decltype(BUF)::value;
      static_for<0, MT>([&](auto J) { A[b][J] = lds_read<16, (decltype(J)::value * NKB + s) * 1024>(xb); });
      static_for<0, NTW>([&](auto J) { B[b][J] = lds_read<16, (decltype(J)::value * NKB + s) * 1024>(wb); });
    };
    fetch(std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{});
    lds_wait(A[0]);
    lds_wait(B[0]);
    static_for<0, NKB>([&](auto S) {
      constexpr int s = decltype(S)::value, cur = s & 1, nxt = (s + 1) & 1;
      if constexpr (s + 1 < NKB) fetch(std::integral_constant<int, s + 1>{}, std::integral_constant<int, nxt>{});
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int t = 0; t < NTW; ++t) acc[mt][t] = kblock<T>(A[cur][mt], B[cur][t], acc[mt][t]);
      if constexpr (s + 1 < NKB) {
        lds_wait(A[nxt]);
        lds_wait(B[nxt]);
      }
    });
  };

  // fused QKV epilogue: the rotation factors of the lane's outputs are
  // fetched before the ring starts (few rows), so their latency hides
  // behind the weight stream
  constexpr bool QPRE = EPI == LA_EPI_QKV && MT <= 4;
  float2 qcs[QPRE ? MT : 1][4][NTW];
  if constexpr (QPRE) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int t = 0; t < NTW; ++t) {
          const int m = mt * 16 + 4 * g + r, col = colw + 16 * t;
          qcs[mt][r][t] = qkv_rope(a.qo, m, col + c16, m < a.M && col < a.N);
        }
  }
  static_for<0, DW>([&](auto J) { issue(J, decltype(J)::value); });
  for (int i0 = 0; i0 < n; i0 += R) {
    static_for<0, R>([&](auto J) {
      constexpr int j = decltype(J)::value;
      const int i = i0 + j;
      if (i < n) {
        wait_vm<(DW - 1) * G>();   // step i landed (steps i+1 .. i+DW-1 may be in flight)
        ring_barrier();            // ... for every wave; stage (i-1) % R is no longer read
        issue(std::integral_constant<int, (j + DW) % R>{}, i + DW);
        compute(J);
      }
    });
  }
  wait_vm<0>();   // no DMA may land after the workgroup has left

  // D lane l holds rows 4*g + r, column c16 of each 16x16 tile
  if constexpr (EPI == LA_EPI_QKV) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int t = 0; t < NTW; ++t) {
          const int m = mt * 16 + 4 * g + r, col = colw + 16 * t;
          const bool live = m < a.M && col < a.N;
          float2 cs;
          if constexpr (QPRE) cs = qcs[mt][r][t];
          else cs = qkv_rope(a.qo, m, col + c16, live);
          qkv_store<T>(a.qo, m, col + c16, acc[mt][t][r], live, cs);
        }
    return;
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = mt * 16 + 4 * g + r;
      if (m >= a.M) continue;
      if (swiglu) {
        if (colw >= a.N) continue;
        const float v0 = acc[mt][0][r], v1 = acc[mt][NTW - 1][r];
        if (EPI == LA_EPI_PARTIAL) {
          float* P = a.P + ((size_t)split * a.M + m) * a.pcols;
          P[colw + c16] = v0;
          P[a.up_off + colw + c16] = v1;
        } else {
          gemm_store<T, EPI>(a, m, colw + c16, v0, v1);
        }
      } else {
#pragma unroll
        for (int t = 0; t < NTW; ++t) {
          const int col = colw + 16 * t;
          if (col >= a.N) continue;
          if (EPI == LA_EPI_PARTIAL) a.P[((size_t)split * a.M + m) * a.pcols + col + c16] = acc[mt][t][r];
          else gemm_store<T, EPI>(a, m, col + c16, acc[mt][t][r], 0.f);
        }
      }
    }
  }
}

// Fixed-order reduction of split partials (split 0 first), then the
// epilogue; a thread takes four adjacent columns (N is a multiple of 16).
template <typename T, int EPI>
__global__ void __launch_bounds__(256) la_gemm_reduce_kernel(LaGemmArgs a) {
  constexpr int MS = 8;                           // splits whose loads are all issued before the sums
  ARGS_READY("s"(a.P), "s"(a.Y), "s"(a.M), "s"(a.N), "s"(a.splits), "s"(a.pcols), "s"(a.up_off), "s"(a.ldy));
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  const int n4 = a.N / 4;
  if (idx >= (size_t)a.M * n4) return;
  const int m = (int)(idx / n4), n = 4 * (int)(idx % n4);
  float4 s0 = make_float4(0.f, 0.f, 0.f, 0.f), s1 = s0;
  for (int s00 = 0; s00 < a.splits; s00 += MS) {
    float4 v[MS], u[MS];
#pragma unroll
    for (int k = 0; k < MS; ++k) {
      if (s00 + k < a.splits) {
        const float* P = a.P + ((size_t)(s00 + k) * a.M + m) * a.pcols;
        v[k] = *(const float4*)(P + n);
        if (EPI == LA_EPI_SWIGLU) u[k] = *(const float4*)(P + a.up_off + n);
      }
    }
#pragma unroll
    for (int k = 0; k < MS; ++k) {
      if (s00 + k < a.splits) {
        s0.x += v[k].x; s0.y += v[k].y; s0.z += v[k].z; s0.w += v[k].w;
        if (EPI == LA_EPI_SWIGLU) { s1.x += u[k].x; s1.y += u[k].y; s1.z += u[k].z; s1.w += u[k].w; }
      }
    }
  }
  gemm_store<T, EPI>(a, m, n, s0.x, s1.x);
  gemm_store<T, EPI>(a, m, n + 1, s0.y, s1.y);
  gemm_store<T, EPI>(a, m, n + 2, s0.z, s1.z);
  gemm_store<T, EPI>(a, m, n + 3, s0.w, s1.w);
}

// ---------------------------------------------------------------------------
// bf16: 32x32x16 MFMA kernel.
//
// A wave owns CW = 2 column tiles of 32 (SwiGLU: the gate and the up tile of
// the same 32 output columns) over every row tile of 32, so a workgroup of
// NWV waves (4, 3 or 2, a function of the weight shape: the fewer that fill
// clearly more CUs in one round of workgroups) covers 64 NWV columns (SwiGLU:
// 32 NWV outputs).  Per k16 block a wave reads RT X fragments (shared by the
// workgroup's waves) and its 2 W fragments from LDS for 2 RT MFMAs of 32
// cycles: 64 bytes of LDS reads per clock and CU at full MFMA rate, where
// 16x16x32 tiles would need four times as much.
//   * W packed (la_gemm_pack_launch): fragment (tile pair p, k16 block kb,
//     tile t) is 1 KB, lane l's 16 bytes = W[32 c + l % 32][16 kb + 8 (l / 32)
//     .. +7] of column tile c = 2 p + t (SwiGLU: the gate (t = 0) or up (t =
//     1) rows of output tile p), ordered [p][kb][t], the B operand layout of
//     the MFMA: a wave's two tiles are one contiguous stream (two streams a
//     tile apart read measurably slower); tiles past N are zero;
//   * X and W reach LDS by global_load_lds DMA (issued as inline asm, so
//     the compiler places only LDS waits on the reads; the ring waits for
//     its own stages with exact vmcnt counts), a ring of NS stages of SK k16
//     blocks; X rows are stored row-major per 32-row tile with their 16-byte
//     pieces XOR-swizzled by row, so the A-operand reads (one row per lane)
//     are conflict-free and the DMA reads each row's run contiguously;
//   * the K partition: units of 64 (four k16 blocks), a split count that is a
//     function of (N, K) only; inside a split the k16 blocks are taken in
//     order, so an output element gets the same bits whatever M and row tile.
// D of a 32x32 tile: lane l, value v holds row 8 (v / 4) + 4 (l / 32) + v % 4,
// column l % 32.

__device__ __forceinline__ f32x16 mfma_bf16_32x32(v4u a, v4u b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                 0, 0);
}

template <typename V> __device__ __forceinline__ V g2_lds(uint32_t addr) {
  return *(const __attribute__((address_space(3))) V*)addr;
}
// uniform base + per-lane offset as one VALU add the compiler keeps as written
__device__ __forceinline__ uint32_t g2_add(uint32_t sbase, uint32_t voff) {
  uint32_t r;
  sbase = __builtin_amdgcn_readfirstlane(sbase);
  asm("v_add_u32 %0, %1, %2" : "=v"(r) : "s"(sbase), "v"(voff));
  return r;
}
// lane l's 16 bytes of src land at LDS offset lds_off + 16 l; m0 is restored
__device__ __forceinline__ void g2_dma(const void* src, uint32_t lds_off) {
  uint32_t keep;
  lds_off = __builtin_amdgcn_readfirstlane(lds_off);
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off\n\ts_mov_b32 m0, %0"
               : "=&s"(keep) : "v"(src), "s"(lds_off) : "memory");
}
// the same, non-temporal: the weight stream is read once and so does not
// displace the activation rows every workgroup re-reads from L2
__device__ __forceinline__ void g2_dma_nt(const void* src, uint32_t lds_off) {
  uint32_t keep;
  lds_off = __builtin_amdgcn_readfirstlane(lds_off);
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off nt\n\ts_mov_b32 m0, %0"
               : "=&s"(keep) : "v"(src), "s"(lds_off) : "memory");
}
template <int N> __device__ __forceinline__ void g2_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// at most k (< KMAX) of the wave's stages (PW loads each) still in flight
template <int PW, int KMAX, int K = 0> __device__ __forceinline__ void g2_ring_wait(int k) {
  if constexpr (K + 1 >= KMAX) {
    g2_wait<K * PW>();
  } else {
    if (k <= K) g2_wait<K * PW>();
    else g2_ring_wait<PW, KMAX, K + 1>(k);
  }
}

constexpr int G2_CW = 2;
constexpr int g2_sk(int rt) { return rt <= 4 ? 4 : 2; }                      // k16 blocks per stage
constexpr int g2_xi(int rt, int nwv) { return (rt * g2_sk(rt) + nwv - 1) / nwv; }   // X DMA per wave and stage
constexpr int g2_stage(int rt, int nwv) { return (rt + nwv * G2_CW) * g2_sk(rt) * 1024; }
// ring slots: as many stages as the LDS holds, at most 6, and few enough that
// the DMA of the stages in flight stays within the vmcnt counter (63)
constexpr int g2_slots(int rt, int nwv) {
  const int by_lds = LDS_BYTES / g2_stage(rt, nwv) < 6 ? LDS_BYTES / g2_stage(rt, nwv) : 6;
  const int by_cnt = 63 / (G2_CW * g2_sk(rt) + g2_xi(rt, nwv)) + 1;
  return by_lds < by_cnt ? by_lds : by_cnt;
}

template <int RT, int EPI, int NWV>
__global__ void __launch_bounds__(64 * NWV) la_gemm2_kernel(LaGemmArgs a) {
  constexpr int CW = G2_CW, SK = g2_sk(RT), NS = g2_slots(RT, NWV);
  constexpr int XB = RT * SK * 1024;              // X bytes of a stage (row tile rt at rt * SK KB)
  constexpr int STAGE = g2_stage(RT, NWV);
  constexpr int XI = g2_xi(RT, NWV);              // X DMA instructions per wave and stage (the last may repeat)
  constexpr int G = CW * SK + XI;                 // DMA instructions per wave and stage
  constexpr int ROWB = SK * 32;                   // bytes of an X row in a stage
  constexpr int PP = ROWB / 16;                   // its 16-byte pieces
  constexpr int RPW = 256 / ROWB;                 // rows per 256-byte bank window
  constexpr int RPI = 1024 / ROWB;                // rows per 1 KB DMA instruction
  static_assert(NS >= 3 && (NS - 1) * G < 64, "ring shape");
  extern __shared__ __attribute__((aligned(1024))) char lds[];

  ARGS_READY("s"(a.X), "s"(a.W), "s"(a.M), "s"(a.N), "s"(a.K), "s"(a.ldx), "s"(a.splits), "s"(a.swiglu_partial));
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const bool sw = (EPI == LA_EPI_SWIGLU) || (a.swiglu_partial != 0);
  const int split = blockIdx.y;
  const int nu = a.K / 64;                        // K units of four k16 blocks
  const int u0 = (int)((long)split * nu / a.splits), u1 = (int)((long)(split + 1) * nu / a.splits);
  const int n = (u1 - u0) * (4 / SK);             // ring stages of the split
  const int kb0 = u0 * 4;                         // first k16 block of the split
  const int nkb = a.K / 16;
  const int tw = blockIdx.x * NWV + wave;         // the wave's tile pair
  const char* W = (const char*)a.W;
  const bf16_t* X = (const bf16_t*)a.X;
  const uint32_t lds0 = (uint32_t)(uintptr_t)lds;

  // the wave's W fragment (t, k16 block kb) in the packed order; pairs past
  // the last (a ragged N) read the last pair and store nothing
  const int ntile = (a.N + 31) / 32, npair = sw ? ntile : (ntile + 1) / 2;
  auto wfrag = [&](int t, int kb) -> const char* {
    const size_t f = ((size_t)min(tw, npair - 1) * nkb + kb) * 2 + t;
    return W + f * 1024 + 16 * lane;
  };
  // the lane's X source row and piece per X instruction of a stage (row tile rt = q / SK, part ii = q % SK)
  const bf16_t* xsrc[XI];
  uint32_t xdst[XI];
#pragma unroll
  for (int x = 0; x < XI; ++x) {
    // the stage's RT SK X blocks dealt to the waves; a wave's slot past the
    // last repeats the last block (the same bytes to the same LDS place)
    const int q = min(wave * XI + x, RT * SK - 1), rt = q / SK, ii = q % SK;
    const int r = ii * RPI + lane / PP;           // row inside the 32-row tile
    const int p = lane % PP, lq = p ^ ((r / RPW) % PP);
    const int m = min(rt * 32 + r, a.M - 1);      // rows past M repeat row M - 1 (never stored)
    xsrc[x] = X + (size_t)m * a.ldx + 8 * lq;
    xdst[x] = (uint32_t)(rt * SK + ii) * 1024;
  }
  auto issue = [&](int i) __attribute__((always_inline)) {
    const uint32_t slot = lds0 + (uint32_t)(i % NS) * STAGE;
    const int kb = kb0 + i * SK;
#pragma unroll
    for (int t = 0; t < CW; ++t)
#pragma unroll
      for (int j = 0; j < SK; ++j) g2_dma_nt(wfrag(t, kb + j), slot + XB + ((wave * CW + t) * SK + j) * 1024);
#pragma unroll
    for (int x = 0; x < XI; ++x) g2_dma(xsrc[x] + (size_t)kb * 16, slot + xdst[x]);
  };

  // LDS offsets of the lane's fragments: A (X row l % 32, piece 2 j + l / 32 swizzled), B (16 l)
  uint32_t xo[SK];
  {
    const int r = lane % 32, sel = lane / 32, gsw = (r / RPW) % PP;
#pragma unroll
    for (int j = 0; j < SK; ++j) xo[j] = r * ROWB + 16 * ((2 * j + sel) ^ gsw);
  }
  const uint32_t wo = 16 * lane;

  f32x16 acc[RT][CW];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int t = 0; t < CW; ++t)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[rt][t][v] = 0.f;

#pragma unroll
  for (int i = 0; i < NS - 1; ++i)
    if (i < n) issue(i);
  for (int i = 0; i < n; ++i) {
    g2_ring_wait<G, NS - 1>(min(NS - 2, n - 1 - i));   // stage i landed (later ones may be in flight)
    ring_barrier();                                  // ... for every wave; stage i - 1's slot is free
    if (i + NS - 1 < n) issue(i + NS - 1);
    const uint32_t slot = lds0 + (uint32_t)(i % NS) * STAGE;
    const uint32_t wb = slot + XB + (uint32_t)wave * CW * SK * 1024;
#pragma unroll
    for (int j = 0; j < SK; ++j) {
      const uint32_t xa = g2_add(slot, xo[j]), wa = g2_add(wb, wo);
      v4u A[RT], B[CW];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) A[rt] = g2_lds<v4u>(xa + rt * SK * 1024);
#pragma unroll
      for (int t = 0; t < CW; ++t) B[t] = g2_lds<v4u>(wa + (t * SK + j) * 1024);
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int t = 0; t < CW; ++t) acc[rt][t] = mfma_bf16_32x32(A[rt], B[t], acc[rt][t]);
    }
  }
  g2_wait<0>();   // no DMA may land after the workgroup has left

  const int c32 = lane % 32, rq = 4 * (lane / 32);
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int m = rt * 32 + 8 * (v / 4) + rq + (v % 4);
      if (m >= a.M) continue;
      if (sw) {
        const int col = tw * 32 + c32;
        if (col >= a.N) continue;
        if (EPI == LA_EPI_PARTIAL) {
          float* P = a.P + ((size_t)split * a.M + m) * a.pcols;
          P[col] = acc[rt][0][v];
          P[a.up_off + col] = acc[rt][1][v];
        } else {
          gemm_store<bf16_t, EPI>(a, m, col, acc[rt][0][v], acc[rt][1][v]);
        }
      } else {
#pragma unroll
        for (int t = 0; t < CW; ++t) {
          const int col = (2 * tw + t) * 32 + c32;
          if (col >= a.N) continue;
          if (EPI == LA_EPI_PARTIAL) a.P[((size_t)split * a.M + m) * a.pcols + col] = acc[rt][t][v];
          else gemm_store<bf16_t, EPI>(a, m, col, acc[rt][t][v], 0.f);
        }
      }
    }
}

// Packed bf16 W for la_gemm2_kernel: thread idx writes lane idx % 64 of fragment idx / 64.
__global__ void __launch_bounds__(256) la_gemm2_pack_kernel(const bf16_t* W, bf16_t* P, int N, int K, int up_off,
                                                            int swiglu, size_t pieces) {
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= pieces) return;
  const int lane = (int)(idx & 63);
  const size_t f = idx >> 6;
  const size_t nkb = (size_t)(K / 16);
  // f = (p * nkb + kb) * 2 + t: tile pair p (SwiGLU: output tile p, gate t = 0 / up t = 1)
  const int t = (int)(f & 1);
  const size_t rest = f >> 1;
  const int p = (int)(rest / nkb), kb = (int)(rest % nkb);
  const int col = (swiglu ? p : 2 * p + t) * 32 + lane % 32;
  u32x4 v = {0, 0, 0, 0};
  if (col < N) {
    const int row = (swiglu && t ? up_off : 0) + col;
    v = *(const u32x4*)(W + (size_t)row * K + (size_t)kb * 16 + 8 * (lane / 32));
  }
  *(u32x4*)(P + idx * 8) = v;
}

template <int RT, int EPI, int NWV>
static void launch_g2(const LaGemmArgs& a, dim3 grid, hipStream_t st) {
  constexpr int lds = g2_slots(RT, NWV) * g2_stage(RT, NWV);
  static_assert(lds <= LDS_BYTES, "LDS");
  auto kern = la_gemm2_kernel<RT, EPI, NWV>;
  static bool attr = false;   // idempotent, so a race between threads only repeats it
  if (!attr) {
    hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    attr = true;
  }
  hipLaunchKernelGGL(kern, grid, dim3(64 * NWV), lds, st, a);
}

template <int EPI, int NWV>
static void launch_g2_rt(const LaGemmArgs& a, dim3 grid, hipStream_t st) {
  const int rt = (a.M + 31) / 32;
  if (rt <= 1) launch_g2<1, EPI, NWV>(a, grid, st);
  else if (rt <= 2) launch_g2<2, EPI, NWV>(a, grid, st);
  else if (rt <= 3) launch_g2<3, EPI, NWV>(a, grid, st);
  else if (rt <= 4) launch_g2<4, EPI, NWV>(a, grid, st);
  else if (rt <= 6) launch_g2<6, EPI, NWV>(a, grid, st);
  else launch_g2<8, EPI, NWV>(a, grid, st);
}

// Waves per workgroup for N output columns in `splits` K splits: four, or
// fewer where that fills clearly more of the 256 CUs in one round of
// workgroups (each CU streams its share of the weights, and a CU's own load
// rate is bounded).  A function of the weight shape only; a column's
// arithmetic is its wave's whatever the workgroup size.
static int g2_waves(int N, int swiglu, int splits) {
  int best = 4;
  long best_wgs = 0;
  for (const int w : {4, 3, 2}) {
    const int per = swiglu ? w * 32 : w * 32 * G2_CW;
    const long wgs = (long)((N + per - 1) / per) * splits;
    if (wgs > 256) continue;
    if (wgs > best_wgs + 16) { best = w; best_wgs = wgs; }
  }
  return best;
}

template <int EPI, int NWV>
static void launch_g2_s(const LaGemmArgs& a, hipStream_t st) {
  const int per = EPI == LA_EPI_SWIGLU ? NWV * 32 : NWV * 32 * G2_CW;   // output columns per workgroup
  dim3 grid((a.N + per - 1) / per, a.splits);
  if (a.splits > 1) launch_g2_rt<LA_EPI_PARTIAL, NWV>(a, grid, st);
  else launch_g2_rt<EPI, NWV>(a, grid, st);
}

template <int EPI>
static int launch_g2_t(LaGemmArgs a, hipStream_t st) {
  const bool swiglu = EPI == LA_EPI_SWIGLU;
  a.swiglu_partial = swiglu ? 1 : 0;
  const int nwv = g2_waves(a.N, swiglu, a.splits);
  if (nwv == 2) launch_g2_s<EPI, 2>(a, st);
  else if (nwv == 3) launch_g2_s<EPI, 3>(a, st);
  else launch_g2_s<EPI, 4>(a, st);
  if (a.splits > 1 && !a.defer_reduce) {
    const size_t total = (size_t)a.M * (a.N / 4);
    hipLaunchKernelGGL((la_gemm_reduce_kernel<bf16_t, EPI>), dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st,
                       a);
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// ---------------------------------------------------------------------------

// Tiles per wave: a function of the weight shape only (it fixes the packed
// layout); two when that still leaves ~200 workgroups, and always for SwiGLU
// (its gate and up tiles).
int la_gemm_ntw(int N, int swiglu) { return swiglu ? 2 : (N >= 25600 ? 2 : 1); }

static size_t pack_blocks(int N, int swiglu) {
  const int per = swiglu ? 4 : 4 * la_gemm_ntw(N, swiglu);   // output tiles per workgroup
  return (size_t)((N / 16 + per - 1) / per);
}

size_t la_gemm_packed_elems(int dtype, int N, int K, int swiglu) {
  // bf16: tile pairs (SwiGLU: an output tile's gate and up tiles) of 32 x K
  if (dtype == LA_DT_BF16) return (size_t)(swiglu ? (N + 31) / 32 : ((N + 31) / 32 + 1) / 2) * 2 * 32 * (size_t)K;
  return pack_blocks(N, swiglu) * 4 * la_gemm_ntw(N, swiglu) * 16 * (size_t)K;
}

// Natural column of packed column n under the pair-major order of the fused
// QKV epilogue: inside each dh-wide head, tile k holds dims 8k .. 8k+7 in
// its lanes 0..7 and their rotation partners dh/2 + 8k .. in lanes 8..15.
__host__ __device__ __forceinline__ int qkv_natural(int n, int dh) {
  const int j = n % dh, k = j / 16, c = j % 16;
  return n - j + (c < 8 ? 8 * k + c : dh / 2 + 8 * k + c - 8);
}

// Packed W: fragment f = ((b * nkb + kb) * 4 + w) * NTW + t holds, lane l
// after lane, the 16 bytes of W row (tile row0 + l % 16), k = kb * KB +
// EPL * (l / 16) .. +EPL-1; rows of tiles past N are zero.
template <typename T>
__global__ void __launch_bounds__(256) la_gemm_pack_kernel(const T* W, T* P, int N, int K, int up_off, int ntw,
                                                           int swiglu, int rope_dh, size_t pieces) {
  constexpr int KB = GT<T>::KC / 4, EPL = GT<T>::EPL;
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= pieces) return;
  const int lane = (int)(idx & 63);
  const size_t f = idx >> 6;
  const size_t nkb = (size_t)(K / KB);
  const int t = (int)(f % ntw);
  const int w = (int)((f / ntw) % 4);
  const int kb = (int)((f / (4 * ntw)) % nkb);
  const size_t b = f / (4 * ntw * nkb);
  const int col = swiglu ? (int)(b * 4 + w) * 16 : (int)(b * 4 + w) * 16 * ntw + 16 * t;
  u32x4 v = {0, 0, 0, 0};
  if (col < N) {
    int row = (swiglu ? col + t * up_off : col) + (lane & 15);
    if (rope_dh > 0) row = qkv_natural(row, rope_dh);
    v = *(const u32x4*)(W + (size_t)row * K + (size_t)kb * KB + EPL * (lane >> 4));
  }
  *(u32x4*)(P + idx * EPL) = v;
}

int la_gemm_pack_launch(int dtype, const void* W, void* P, int N, int K, int swiglu, hipStream_t st, int rope_dh) {
  const int kc = dtype == LA_DT_BF16 ? GT<bf16_t>::KC : GT<float>::KC;
  if (N % 16 != 0 || K % kc != 0 || N <= 0) return -2;
  if (rope_dh > 0 && (swiglu || rope_dh % 16 != 0 || N % rope_dh != 0)) return -2;
  const int ntw = la_gemm_ntw(N, swiglu);
  const size_t pieces = la_gemm_packed_elems(dtype, N, K, swiglu) / (dtype == LA_DT_BF16 ? 8 : 4);
  const unsigned grid = (unsigned)((pieces + 255) / 256);
  if (dtype == LA_DT_BF16) {
    if (rope_dh > 0) return -2;                  // the pair-major QKV layout is fp32-only
    hipLaunchKernelGGL(la_gemm2_pack_kernel, dim3(grid), dim3(256), 0, st, (const bf16_t*)W, (bf16_t*)P, N, K, N,
                       swiglu, pieces);
  } else
    hipLaunchKernelGGL(la_gemm_pack_kernel<float>, dim3(grid), dim3(256), 0, st, (const float*)W, (float*)P, N, K, N,
                       ntw, swiglu, rope_dh, pieces);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int la_gemm_splits(int N, int K, int dtype, int swiglu) {
  // a function of the weight shape only (never of M)
  if (dtype == LA_DT_BF16) {
    // bf16: as many K splits (units of 64, at most 8) as keep the workgroups
    // within one per CU of the 256
    const int groups = (N + (swiglu ? 128 : 256) - 1) / (swiglu ? 128 : 256);
    const int units = K / 64;
    return std::max(1, std::min(std::min(8, units), 256 / std::max(groups, 1)));
  }
  // fp32: split K only when there are too few column tiles to give every CU
  // a workgroup, up to 4 ways
  const int kc = GT<float>::KC;
  const int nchunks = K / kc;
  const int blocks = (N / 16 + 3) / 4;
  if (swiglu || blocks >= 128 || nchunks < 2) return 1;
  int s = (256 + blocks - 1) / blocks;
  s = std::min(s, 4);
  s = std::min(s, nchunks);
  return std::max(s, 1);
}

template <typename T, int MT, int NTW, int EPI>
static void launch_k(const LaGemmArgs& a, dim3 grid, hipStream_t st) {
  constexpr int lds = (gemm_depth(MT, NTW) + 1) * gemm_stage(MT, NTW);
  static_assert(lds <= LDS_BYTES, "LDS");
  auto kern = la_gemm_kernel<T, MT, NTW, EPI>;
  static bool attr = false;   // idempotent, so a race between threads only repeats it
  if (!attr) {
    hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    attr = true;
  }
  hipLaunchKernelGGL(kern, grid, dim3(256), lds, st, a);
}

template <typename T, int EPI, int MT>
static void launch_mt(const LaGemmArgs& a, int ntw, hipStream_t st) {
  const int tiles = a.N / 16;
  const int per = a.swiglu_partial ? 4 : 4 * ntw;
  dim3 grid((tiles + per - 1) / per, a.splits);
  const bool part = a.splits > 1;
  if (ntw == 2) {
    if (part) launch_k<T, MT, 2, LA_EPI_PARTIAL>(a, grid, st);
    else launch_k<T, MT, 2, EPI>(a, grid, st);
  } else {
    if (part) launch_k<T, MT, 1, LA_EPI_PARTIAL>(a, grid, st);
    else launch_k<T, MT, 1, EPI>(a, grid, st);
  }
}

template <typename T, int EPI>
static int launch_t(LaGemmArgs a, hipStream_t st) {
  const int mt = (a.M + 15) / 16;
  const bool swiglu = EPI == LA_EPI_SWIGLU;
  a.swiglu_partial = swiglu ? 1 : 0;
  const int ntw = la_gemm_ntw(a.N, swiglu);
  if constexpr (EPI == LA_EPI_SWIGLU) {
    if (mt <= 1) launch_mt<T, EPI, 1>(a, 2, st);
    else if (mt <= 2) launch_mt<T, EPI, 2>(a, 2, st);
    else if (mt <= 4) launch_mt<T, EPI, 4>(a, 2, st);
    else if (mt <= 8) launch_mt<T, EPI, 8>(a, 2, st);
    else if (mt <= 12) launch_mt<T, EPI, 12>(a, 2, st);
    else launch_mt<T, EPI, 16>(a, 2, st);
  } else {
    if (mt <= 1) launch_mt<T, EPI, 1>(a, ntw, st);
    else if (mt <= 2) launch_mt<T, EPI, 2>(a, ntw, st);
    else if (mt <= 4) launch_mt<T, EPI, 4>(a, ntw, st);
    else if (mt <= 8) launch_mt<T, EPI, 8>(a, ntw, st);
    else if (mt <= 12) launch_mt<T, EPI, 12>(a, ntw, st);
    else launch_mt<T, EPI, 16>(a, ntw, st);
  }
  if (a.splits > 1 && !a.defer_reduce) {
    const size_t total = (size_t)a.M * (a.N / 4);
    hipLaunchKernelGGL((la_gemm_reduce_kernel<T, EPI>), dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, a);
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int la_gemm_launch(int dtype, int epi, LaGemmArgs a, hipStream_t st) {
  const int kc = dtype == LA_DT_BF16 ? GT<bf16_t>::KC : GT<float>::KC;
  if (a.M < 1 || a.M > 256 || a.K % kc != 0 || a.N % 16 != 0 || a.ldx % (16 / (dtype == LA_DT_BF16 ? 2 : 4)))
    return -2;
  // K units a split is made of (bf16: 64, fp32: one chunk)
  a.nchunks = dtype == LA_DT_BF16 ? a.K / 64 : a.K / kc;
  if (a.splits < 1) a.splits = 1;
  if (a.splits > a.nchunks) return -2;
  if (a.splits > 1 && a.P == nullptr) return -2;
  if (a.defer_reduce && (a.splits < 2 || (epi != LA_EPI_RESID && epi != LA_EPI_STORE))) return -2;
  if (epi == LA_EPI_QKV) {
    if (a.splits != 1 || a.qo.dh < 16 || (a.qo.dh & (a.qo.dh - 1)) != 0 || a.N % a.qo.dh != 0) return -2;
    a.qo.lg_dh = __builtin_ctz((unsigned)a.qo.dh);
  }
  if (dtype == LA_DT_BF16) {
    switch (epi) {
      case LA_EPI_STORE: return launch_g2_t<LA_EPI_STORE>(a, st);
      case LA_EPI_RESID: return launch_g2_t<LA_EPI_RESID>(a, st);
      case LA_EPI_SWIGLU: return launch_g2_t<LA_EPI_SWIGLU>(a, st);
      case LA_EPI_F32: return launch_g2_t<LA_EPI_F32>(a, st);
      case LA_EPI_QKV: return -2;                // bf16 QKV: stored, then rotated and placed by la_qkv_post_launch
    }
  } else {
    switch (epi) {
      case LA_EPI_STORE: return launch_t<float, LA_EPI_STORE>(a, st);
      case LA_EPI_RESID: return launch_t<float, LA_EPI_RESID>(a, st);
      case LA_EPI_SWIGLU: return launch_t<float, LA_EPI_SWIGLU>(a, st);
      case LA_EPI_F32: return launch_t<float, LA_EPI_F32>(a, st);
      case LA_EPI_QKV: return launch_t<float, LA_EPI_QKV>(a, st);
    }
  }
  return -2;
}
