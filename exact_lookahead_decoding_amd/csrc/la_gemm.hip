// Skinny GEMM Y = X W^T for the packed rows (M <= 256), HBM-bound on W.
//
// The target forward of one packed round multiplies a few hundred rows by
// every weight matrix ("M7.3 - Lookahead Decoding", 0x05C row and FLOP
// ledger: token-wise target work over Q rows), so W is streamed once per
// round and the rows stay on chip:
//   * a workgroup (4 waves) owns a block of output columns and one split of
//     the K dimension; each wave owns two 16-column MFMA tiles and all M rows;
//   * W fragments go global -> registers, one K chunk ahead;
//   * the X chunk is staged through LDS (double buffered) and shared by the
//     four waves.
// Batch invariance: the K partition (chunk size, split count) depends only
// on (N, K), never on M, and every output element is produced by the same
// MFMA sequence and the same fixed-order split reduction whatever row slot
// it occupies.  A row therefore gets bit-identical results in a 1-row
// autoregressive step and in a packed lookahead round.
#include "la_common.h"
#include "la_kernels.h"

template <typename T> struct MM;
template <> struct MM<bf16_t> {
  static constexpr int KC = 128;     // K elements per chunk
  static constexpr int KSTEP = 32;   // K per MFMA
  static constexpr int VEC = 8;      // elements per lane per fragment
  static constexpr int PAD = 8;
  typedef bf16x8 frag;
  static __device__ __forceinline__ frag ld(const bf16_t* p) { return *(const bf16x8*)p; }
  static __device__ __forceinline__ f32x4 mma(frag a, frag b, f32x4 c) { return mfma_bf16_32(a, b, c); }
};
template <> struct MM<float> {
  static constexpr int KC = 64;
  static constexpr int KSTEP = 4;
  static constexpr int VEC = 1;
  static constexpr int PAD = 4;
  typedef float frag;
  static __device__ __forceinline__ frag ld(const float* p) { return *p; }
  static __device__ __forceinline__ f32x4 mma(frag a, frag b, f32x4 c) { return mfma_f32_4(a, b, c); }
};

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

template <typename T, int MT, int EPI>
__global__ void __launch_bounds__(256) la_gemm_kernel(LaGemmArgs a) {
  typedef MM<T> mm;
  constexpr int KC = mm::KC;
  constexpr int NKS = KC / mm::KSTEP;        // k-steps per chunk
  constexpr int LROW = KC + mm::PAD;         // LDS row length (elements)
  constexpr int ROWS = MT * 16;
  constexpr int EPP = 16 / sizeof(T);        // elements per 16-byte piece
  constexpr int PPR = KC / EPP;              // pieces per row (16)
  __shared__ __attribute__((aligned(16))) T xs[2][ROWS * LROW];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g = lane >> 4;
  const int c16 = lane & 15;
  const bool swiglu = (EPI == LA_EPI_SWIGLU) || (a.swiglu_partial != 0);
  const int r0 = swiglu ? blockIdx.x * 64 + wave * 16 : blockIdx.x * 128 + wave * 32;
  const int r1 = swiglu ? r0 + a.up_off : r0 + 16;
  const bool active = r0 < a.N;
  const int split = blockIdx.y;
  const int c_begin = (int)(((long)split * a.nchunks) / a.splits);
  const int c_end = (int)(((long)(split + 1) * a.nchunks) / a.splits);

  const T* X = (const T*)a.X;
  const T* W = (const T*)a.W;
  const T* w0p = W + (size_t)(active ? r0 + c16 : 0) * a.K + mm::VEC * g;
  const T* w1p = W + (size_t)(active ? r1 + c16 : 0) * a.K + mm::VEC * g;

  f32x4 acc[MT][2];
#pragma unroll
  for (int i = 0; i < MT; ++i) { acc[i][0] = f32x4{0, 0, 0, 0}; acc[i][1] = f32x4{0, 0, 0, 0}; }

  typename mm::frag bcur[NKS][2], bnxt[NKS][2];
  u32x4 xreg[MT];

  auto load_b = [&](int c, typename mm::frag (&b)[NKS][2]) {
    const size_t k0 = (size_t)c * KC;
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
      b[s][0] = mm::ld(w0p + k0 + s * mm::KSTEP);
      b[s][1] = mm::ld(w1p + k0 + s * mm::KSTEP);
    }
  };
  auto load_x = [&](int c) {
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      const int piece = threadIdx.x + 256 * i;
      const int row = piece / PPR, col = (piece % PPR) * EPP;
      if (row < a.M) xreg[i] = *(const u32x4*)(X + (size_t)row * a.ldx + (size_t)c * KC + col);
      else xreg[i] = u32x4{0, 0, 0, 0};
    }
  };
  auto store_x = [&](int buf) {
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      const int piece = threadIdx.x + 256 * i;
      const int row = piece / PPR, col = (piece % PPR) * EPP;
      *(u32x4*)(&xs[buf][row * LROW + col]) = xreg[i];
    }
  };

  if (c_begin < c_end) {
    if (active) load_b(c_begin, bcur);
    load_x(c_begin);
    store_x(0);
    __syncthreads();
    int buf = 0;
    for (int c = c_begin; c < c_end; ++c) {
      const bool more = c + 1 < c_end;
      if (more) {
        if (active) load_b(c + 1, bnxt);
        load_x(c + 1);
      }
      if (active) {
#pragma unroll
        for (int s = 0; s < NKS; ++s) {
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
            typename mm::frag af = mm::ld(&xs[buf][(mt * 16 + c16) * LROW + s * mm::KSTEP + mm::VEC * g]);
            acc[mt][0] = mm::mma(af, bcur[s][0], acc[mt][0]);
            acc[mt][1] = mm::mma(af, bcur[s][1], acc[mt][1]);
          }
        }
      }
      if (more) {
        store_x(buf ^ 1);
#pragma unroll
        for (int s = 0; s < NKS; ++s) { bcur[s][0] = bnxt[s][0]; bcur[s][1] = bnxt[s][1]; }
      }
      __syncthreads();
      buf ^= 1;
    }
  }
  if (!active) return;

  // epilogue: D lane l holds rows 4*g + r, column c16 of each 16x16 tile
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = mt * 16 + 4 * g + r;
      if (m >= a.M) continue;
      const float v0 = acc[mt][0][r], v1 = acc[mt][1][r];
      if (EPI == LA_EPI_PARTIAL) {
        float* P = a.P + ((size_t)split * a.M + m) * a.pcols;
        if (swiglu) {
          P[r0 + c16] = v0;
          P[a.up_off + r0 + c16] = v1;
        } else {
          P[r0 + c16] = v0;
          P[r0 + 16 + c16] = v1;
        }
      } else if (EPI == LA_EPI_SWIGLU) {
        gemm_store<T, EPI>(a, m, r0 + c16, v0, v1);
      } else {
        gemm_store<T, EPI>(a, m, r0 + c16, v0, 0.f);
        gemm_store<T, EPI>(a, m, r0 + 16 + c16, v1, 0.f);
      }
    }
  }
}

// Fixed-order reduction of split partials, then the epilogue.
template <typename T, int EPI>
__global__ void __launch_bounds__(256) la_gemm_reduce_kernel(LaGemmArgs a) {
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t total = (size_t)a.M * a.N;
  if (idx >= total) return;
  const int m = (int)(idx / a.N), n = (int)(idx % a.N);
  float s0 = 0.f, s1 = 0.f;
  for (int s = 0; s < a.splits; ++s) {
    const float* P = a.P + ((size_t)s * a.M + m) * a.pcols;
    s0 += P[n];
    if (EPI == LA_EPI_SWIGLU) s1 += P[a.up_off + n];
  }
  gemm_store<T, EPI>(a, m, n, s0, s1);
}

// ---------------------------------------------------------------------------

int la_gemm_splits(int N, int K, int dtype, int swiglu) {
  // depends on the weight shape only (never on M): aim at ~384 workgroups
  const int kc = dtype == LA_DT_BF16 ? MM<bf16_t>::KC : MM<float>::KC;
  const int nblk = swiglu ? (N + 63) / 64 : (N + 127) / 128;
  const int nchunks = K / kc;
  int s = (384 + nblk - 1) / nblk;
  if (s > nchunks / 2) s = nchunks / 2;
  if (s < 1) s = 1;
  return s;
}

template <typename T, int EPI, int MT>
static void launch_mt(const LaGemmArgs& a, dim3 grid, hipStream_t st) {
  if (a.splits > 1) {
    hipLaunchKernelGGL((la_gemm_kernel<T, MT, LA_EPI_PARTIAL>), grid, dim3(256), 0, st, a);
  } else {
    hipLaunchKernelGGL((la_gemm_kernel<T, MT, EPI>), grid, dim3(256), 0, st, a);
  }
}

template <typename T, int EPI>
static int launch_t(LaGemmArgs a, hipStream_t st) {
  const int mt = (a.M + 15) / 16;
  const bool swiglu = EPI == LA_EPI_SWIGLU;
  a.swiglu_partial = swiglu ? 1 : 0;
  const int nblk = swiglu ? (a.N + 63) / 64 : (a.N + 127) / 128;
  dim3 grid(nblk, a.splits);
  if (mt <= 1) launch_mt<T, EPI, 1>(a, grid, st);
  else if (mt <= 2) launch_mt<T, EPI, 2>(a, grid, st);
  else if (mt <= 4) launch_mt<T, EPI, 4>(a, grid, st);
  else if (mt <= 8) launch_mt<T, EPI, 8>(a, grid, st);
  else if (mt <= 12) launch_mt<T, EPI, 12>(a, grid, st);
  else launch_mt<T, EPI, 16>(a, grid, st);
  if (a.splits > 1) {
    const size_t total = (size_t)a.M * a.N;
    hipLaunchKernelGGL((la_gemm_reduce_kernel<T, EPI>), dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, a);
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int la_gemm_launch(int dtype, int epi, LaGemmArgs a, hipStream_t st) {
  const int kc = dtype == LA_DT_BF16 ? MM<bf16_t>::KC : MM<float>::KC;
  if (a.M < 1 || a.M > 256 || a.K % kc != 0 || a.N % 16 != 0) return -2;
  if (epi != LA_EPI_SWIGLU && a.N % 32 != 0) return -2;
  a.nchunks = a.K / kc;
  if (a.splits < 1) a.splits = 1;
  if (a.splits > a.nchunks) return -2;
  if (a.splits > 1 && a.P == nullptr) return -2;
  if (dtype == LA_DT_BF16) {
    switch (epi) {
      case LA_EPI_STORE: return launch_t<bf16_t, LA_EPI_STORE>(a, st);
      case LA_EPI_RESID: return launch_t<bf16_t, LA_EPI_RESID>(a, st);
      case LA_EPI_SWIGLU: return launch_t<bf16_t, LA_EPI_SWIGLU>(a, st);
      case LA_EPI_F32: return launch_t<bf16_t, LA_EPI_F32>(a, st);
    }
  } else {
    switch (epi) {
      case LA_EPI_STORE: return launch_t<float, LA_EPI_STORE>(a, st);
      case LA_EPI_RESID: return launch_t<float, LA_EPI_RESID>(a, st);
      case LA_EPI_SWIGLU: return launch_t<float, LA_EPI_SWIGLU>(a, st);
      case LA_EPI_F32: return launch_t<float, LA_EPI_F32>(a, st);
    }
  }
  return -2;
}
