// Token-wise pieces of the target forward: embedding gather, RMSNorm, RoPE
// at each row's logical position, and placement of each row's K/V.
//
// "M7.3 - Lookahead Decoding", 0x04: every packed row carries a logical
// position (positions are not packed indices); 0x07: the ordinary row's K/V
// is the start of the new frontier while every other packed row's K/V is
// temporary workspace until publication.
//
// Every kernel here computes each row independently with a fixed reduction
// order, so a row's values do not depend on which other rows share the call.
#include "la_common.h"
#include "la_kernels.h"

// Rows are moved as 16-byte vectors; a thread issues all of its loads before
// using any of them.
template <typename T, int VPT>
__global__ void __launch_bounds__(256) embed_kernel(const T* E, const int32_t* tok, T* x, int d) {
  const int m = blockIdx.x;
  const int nv = d * (int)sizeof(T) / 16;
  const u32x4* src = (const u32x4*)(E + (size_t)tok[m] * d);
  u32x4* dst = (u32x4*)(x + (size_t)m * d);
  u32x4 r[VPT];
#pragma unroll
  for (int j = 0; j < VPT; ++j) {
    const int v = threadIdx.x + 256 * j;
    if (v < nv) r[j] = src[v];
  }
#pragma unroll
  for (int j = 0; j < VPT; ++j) {
    const int v = threadIdx.x + 256 * j;
    if (v < nv) dst[v] = r[j];
  }
}

static int vpt_for(int d, int esz) {
  const int nv = d * esz / 16;
  const int v = (nv + 255) / 256;
  return v <= 1 ? 1 : v <= 2 ? 2 : v <= 4 ? 4 : 8;
}

template <typename T, int VPT>
static void embed_t(const void* E, const int32_t* tok, void* x, int M, int d, hipStream_t st) {
  hipLaunchKernelGGL((embed_kernel<T, VPT>), dim3(M), dim3(256), 0, st, (const T*)E, tok, (T*)x, d);
}

void la_embed_launch(int dtype, const void* E, const int32_t* tok, void* x, int M, int d, hipStream_t st) {
  if (M <= 0) return;
  const int esz = dtype == LA_DT_BF16 ? 2 : 4;
  switch (vpt_for(d, esz) * 2 + (dtype == LA_DT_BF16)) {
    case 2: embed_t<float, 1>(E, tok, x, M, d, st); break;
    case 3: embed_t<bf16_t, 1>(E, tok, x, M, d, st); break;
    case 4: embed_t<float, 2>(E, tok, x, M, d, st); break;
    case 5: embed_t<bf16_t, 2>(E, tok, x, M, d, st); break;
    case 8: embed_t<float, 4>(E, tok, x, M, d, st); break;
    case 9: embed_t<bf16_t, 4>(E, tok, x, M, d, st); break;
    case 16: embed_t<float, 8>(E, tok, x, M, d, st); break;
    default: embed_t<bf16_t, 8>(E, tok, x, M, d, st); break;
  }
}

// Residual fold + RMSNorm.  x' = x[src], or, with NS split partials of the
// residual GEMM pending, x' = T(((P_0 + P_1) + ...) + x[src]) (the same sum
// and rounding as that GEMM's own epilogue), written back to x when write_x;
// y[m] = T(x' * rs * w), rs = 1/sqrt(mean(x'^2) + eps), src = rows ? rows[m] : m.
// The sum of squares has one fixed order for every row: each thread's
// elements in index order, then a butterfly within the wave, then the wave
// sums in a fixed pairwise grouping.  All loads of a thread are issued first;
// NTH threads per row (512 once a row needs two 16-byte vectors per thread
// at 256, so its loads come from twice as many waves).
template <typename T, int VPT, int NS, int NTH>
__global__ void __launch_bounds__(NTH) addnorm_kernel(T* x, const float* P, size_t pstride, int write_x, const T* w,
                                                      T* y, const int32_t* rows, int d, float eps) {
  constexpr int E = 16 / sizeof(T);
  __shared__ float red[NTH / 64];
  ARGS_READY("s"(x), "s"(P), "s"(pstride), "s"(write_x), "s"(w), "s"(y), "s"(rows), "s"(d), "s"(eps));
  const int m = blockIdx.x;
  const int src = rows ? rows[m] : m;
  const int nv = d / E;
  u32x4* xr = (u32x4*)(x + (size_t)src * d);
  const u32x4* wr = (const u32x4*)w;
  u32x4 xv[VPT], wv[VPT];
  float4 pv[NS > 0 ? NS : 1][VPT][E / 4];
#pragma unroll
  for (int j = 0; j < VPT; ++j) {
    const int v = threadIdx.x + NTH * j;
    if (v < nv) {
      xv[j] = xr[v];
      wv[j] = wr[v];
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const float4* pp = (const float4*)(P + s * pstride + (size_t)src * d + (size_t)v * E);
#pragma unroll
        for (int q = 0; q < E / 4; ++q) pv[s][j][q] = pp[q];
      }
    }
  }
  float xf[VPT][E];
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < VPT; ++j) {
    const int v = threadIdx.x + NTH * j;
    if (v < nv) {
      const T* e = (const T*)&xv[j];
#pragma unroll
      for (int q = 0; q < E; ++q) {
        float f = ld<T>(e + q);
        if constexpr (NS > 0) {
          float acc = 0.f;
#pragma unroll
          for (int s = 0; s < NS; ++s) acc += ((const float*)&pv[s][j][0])[q];
          f = StoreT<T>::round(acc + f);
        }
        xf[j][q] = f;
        ss += f * f;
      }
      if constexpr (NS > 0) {
        if (write_x) {
          u32x4 ov;
          T* oe = (T*)&ov;
#pragma unroll
          for (int q = 0; q < E; ++q) st<T>(oe + q, xf[j][q]);
          xr[v] = ov;
        }
      }
    }
  }
  for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  float tot = (red[0] + red[1]) + (red[2] + red[3]);
  if constexpr (NTH == 512) tot = tot + ((red[4] + red[5]) + (red[6] + red[7]));
  const float rs = 1.0f / sqrtf(tot / (float)d + eps);
  u32x4* yr = (u32x4*)(y + (size_t)m * d);
#pragma unroll
  for (int j = 0; j < VPT; ++j) {
    const int v = threadIdx.x + NTH * j;
    if (v < nv) {
      const T* we = (const T*)&wv[j];
      u32x4 ov;
      T* oe = (T*)&ov;
#pragma unroll
      for (int q = 0; q < E; ++q) st<T>(oe + q, xf[j][q] * rs * ld<T>(we + q));
      yr[v] = ov;
    }
  }
}

template <typename T, int VPT, int NS, int NTH>
static void an_t(void* x, const float* P, size_t pstride, int write_x, const void* w, void* y, const int32_t* rows,
                 int M, int d, float eps, hipStream_t st) {
  hipLaunchKernelGGL((addnorm_kernel<T, VPT, NS, NTH>), dim3(M), dim3(NTH), 0, st, (T*)x, P, pstride, write_x,
                     (const T*)w, (T*)y, rows, d, eps);
}

template <typename T, int VPT, int NTH>
static void an_s(int S, void* x, const float* P, size_t pstride, int write_x, const void* w, void* y,
                 const int32_t* rows, int M, int d, float eps, hipStream_t st) {
  switch (S) {
    case 0: an_t<T, VPT, 0, NTH>(x, P, pstride, write_x, w, y, rows, M, d, eps, st); break;
    case 1: an_t<T, VPT, 1, NTH>(x, P, pstride, write_x, w, y, rows, M, d, eps, st); break;
    case 2: an_t<T, VPT, 2, NTH>(x, P, pstride, write_x, w, y, rows, M, d, eps, st); break;
    case 3: an_t<T, VPT, 3, NTH>(x, P, pstride, write_x, w, y, rows, M, d, eps, st); break;
    case 4: an_t<T, VPT, 4, NTH>(x, P, pstride, write_x, w, y, rows, M, d, eps, st); break;
    case 5: an_t<T, VPT, 5, NTH>(x, P, pstride, write_x, w, y, rows, M, d, eps, st); break;
    case 6: an_t<T, VPT, 6, NTH>(x, P, pstride, write_x, w, y, rows, M, d, eps, st); break;
    case 7: an_t<T, VPT, 7, NTH>(x, P, pstride, write_x, w, y, rows, M, d, eps, st); break;
    default: an_t<T, VPT, 8, NTH>(x, P, pstride, write_x, w, y, rows, M, d, eps, st); break;
  }
}

int la_addnorm_launch(int dtype, void* x, const float* P, int S, size_t pstride, int write_x, const void* w, void* y,
                      const int32_t* rows, int M, int d, float eps, hipStream_t st) {
  if (M <= 0) return 0;
  if (!P) S = 0;
  if (S < 0 || S > LA_ADDNORM_MAX_SPLITS) return -2;
  const int esz = dtype == LA_DT_BF16 ? 2 : 4;
  switch (vpt_for(d, esz) * 2 + (dtype == LA_DT_BF16)) {
    case 2: an_s<float, 1, 256>(S, x, P, pstride, write_x, w, y, rows, M, d, eps, st); break;
    case 3: an_s<bf16_t, 1, 256>(S, x, P, pstride, write_x, w, y, rows, M, d, eps, st); break;
    case 4: an_s<float, 1, 512>(S, x, P, pstride, write_x, w, y, rows, M, d, eps, st); break;
    case 5: an_s<bf16_t, 1, 512>(S, x, P, pstride, write_x, w, y, rows, M, d, eps, st); break;
    case 8: an_s<float, 2, 512>(S, x, P, pstride, write_x, w, y, rows, M, d, eps, st); break;
    case 9: an_s<bf16_t, 2, 512>(S, x, P, pstride, write_x, w, y, rows, M, d, eps, st); break;
    case 16: an_s<float, 4, 512>(S, x, P, pstride, write_x, w, y, rows, M, d, eps, st); break;
    default: an_s<bf16_t, 4, 512>(S, x, P, pstride, write_x, w, y, rows, M, d, eps, st); break;
  }
  return 0;
}

void la_rmsnorm_launch(int dtype, const void* x, const void* w, void* y, const int32_t* rows, int M, int d,
                       float eps, hipStream_t st) {
  (void)la_addnorm_launch(dtype, (void*)x, nullptr, 0, 0, 0, w, y, rows, M, d, eps, st);
}

// cos/sin of t * theta^(-2i/dh), evaluated in fp64 and stored as fp32
__global__ void rope_table_kernel(float2* tab, int T, int half, int dh, double theta) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= T * half) return;
  const int t = idx / half, i = idx % half;
  const double inv = pow(theta, -2.0 * (double)i / (double)dh);
  const double ang = (double)t * inv;
  tab[idx] = make_float2((float)cos(ang), (float)sin(ang));
}

void la_rope_table_launch(float2* tab, int T, int dh, float theta, hipStream_t st) {
  const int half = dh / 2;
  const int n = T * half;
  hipLaunchKernelGGL(rope_table_kernel, dim3((n + 255) / 256), dim3(256), 0, st, tab, T, half, dh, (double)theta);
}

// qkv [M][(H + 2 Hkv) dh] -> q [M][H][dh] with RoPE; k (RoPE) and v to the
// cache for the first n_direct rows (cache row cache_row0 + m), to the
// workspace (row m - n_direct) for the others.  One block per (row, head).
// With RED the row's values are the fixed-order sums of the projection's S
// K-split partials (sstride floats apart) rounded to the storage type (what
// the split reduction stores); without, the stored values.

// where head hh (q heads, then k, then v) of the request's row m goes; qrow is the row's q
template <typename T>
__device__ inline T* post_dst(int m, int hh, int H, int Hkv, int dh, T* qrow, T* kc, T* vc, int T_cap,
                              int cache_row0, int n_direct, T* kw, T* vw, int ws_cap) {
  if (hh < H) return qrow + (size_t)hh * dh;
  const int g = hh < H + Hkv ? hh - H : hh - H - Hkv;
  const bool isk = hh < H + Hkv;
  if (m < n_direct) return (isk ? kc : vc) + ((size_t)g * T_cap + cache_row0 + m) * dh;
  return (isk ? kw : vw) + ((size_t)g * ws_cap + (m - n_direct)) * dh;
}

// one (row, head): src is the head's first value (RED: in the first partial)
template <typename T, bool RED>
__device__ inline void post_head(const void* src0, int S, size_t sstride, const float2* rope, int p, bool rot, int dh,
                                 T* dst) {
  const int half = dh / 2;
  for (int i = threadIdx.x; i < half; i += 64) {
    float x1, x2;
    if constexpr (RED) {
      const float* src = (const float*)src0;
      float a1 = 0.f, a2 = 0.f;
      for (int s = 0; s < S; ++s) {
        a1 += src[s * sstride + i];
        a2 += src[s * sstride + i + half];
      }
      x1 = StoreT<T>::round(a1);
      x2 = StoreT<T>::round(a2);
    } else {
      const T* src = (const T*)src0;
      x1 = ld<T>(src + i);
      x2 = ld<T>(src + i + half);
    }
    if (rot) {
      const float2 cs = rope[(size_t)p * half + i];
      st<T>(dst + i, x1 * cs.x - x2 * cs.y);
      st<T>(dst + i + half, x2 * cs.x + x1 * cs.y);
    } else {
      st<T>(dst + i, x1);
      st<T>(dst + i + half, x2);
    }
  }
}

template <typename T, bool RED>
__global__ void __launch_bounds__(64) qkv_post_kernel(const void* src, int S, int Prows, const float2* rope,
                                                      const int32_t* pos, int H, int Hkv, int dh, T* q, T* kc, T* vc,
                                                      int T_cap, int cache_row0, int n_direct, T* kw, T* vw,
                                                      int ws_cap) {
  ARGS_READY("s"(src), "s"(S), "s"(Prows), "s"(rope), "s"(pos), "s"(H), "s"(Hkv), "s"(dh), "s"(q), "s"(kc), "s"(vc),
             "s"(T_cap), "s"(cache_row0), "s"(n_direct), "s"(kw), "s"(vw), "s"(ws_cap));
  const int m = blockIdx.x;
  const int hh = blockIdx.y;
  const int pcols = (H + 2 * Hkv) * dh;
  const size_t off = (size_t)m * pcols + (size_t)hh * dh;
  const void* s0 = RED ? (const void*)((const float*)src + off) : (const void*)((const T*)src + off);
  T* dst = post_dst<T>(m, hh, H, Hkv, dh, q + (size_t)m * H * dh, kc, vc, T_cap, cache_row0, n_direct, kw, vw,
                       ws_cap);
  post_head<T, RED>(s0, S, (size_t)Prows * pcols, rope, pos[m], hh < H + Hkv, dh, dst);
}

// the same over the stacked rows of several requests: block x is stacked row
// m, owned by the last entry whose r0 <= m
template <typename T, bool RED>
__global__ void __launch_bounds__(64) qkv_post_multi_kernel(const void* src, int S, int M,
                                                            const LaPostSeg* __restrict__ segs, int n, int layer,
                                                            int H, int Hkv, int dh, T* q) {
  ARGS_READY("s"(src), "s"(S), "s"(M), "s"(segs), "s"(n), "s"(layer), "s"(H), "s"(Hkv), "s"(dh), "s"(q));
  const int m = blockIdx.x;
  const int hh = blockIdx.y;
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (segs[mid].r0 <= m) lo = mid;
    else hi = mid - 1;
  }
  const LaPostSeg& g = segs[lo];
  const int mr = m - g.r0;
  const int pcols = (H + 2 * Hkv) * dh;
  const size_t off = (size_t)m * pcols + (size_t)hh * dh;
  const void* s0 = RED ? (const void*)((const float*)src + off) : (const void*)((const T*)src + off);
  T* kc = (T*)((char*)g.kc + layer * g.kv_layer);
  T* vc = (T*)((char*)g.vc + layer * g.kv_layer);
  T* kw = (T*)((char*)g.kw + layer * g.ws_layer);
  T* vw = (T*)((char*)g.vw + layer * g.ws_layer);
  T* dst = post_dst<T>(mr, hh, H, Hkv, dh, q + (size_t)m * H * dh, kc, vc, g.T_cap, g.cache_row0, g.n_direct, kw, vw,
                       g.ws_cap);
  post_head<T, RED>(s0, S, (size_t)M * pcols, g.rope, g.pos[mr], hh < H + Hkv, dh, dst);
}

void la_qkv_reduce_post_launch(int dtype, const float* P, int S, int Prows, int M, const float2* rope,
                               const int32_t* pos, int H, int Hkv, int dh, void* q, void* kc, void* vc, int T_cap,
                               int cache_row0, int n_direct, void* kw, void* vw, int ws_cap, hipStream_t st) {
  if (M <= 0) return;
  dim3 grid(M, H + 2 * Hkv);
  if (dtype == LA_DT_BF16)
    hipLaunchKernelGGL((qkv_post_kernel<bf16_t, true>), grid, dim3(64), 0, st, (const void*)P, S, Prows, rope, pos, H,
                       Hkv, dh, (bf16_t*)q, (bf16_t*)kc, (bf16_t*)vc, T_cap, cache_row0, n_direct, (bf16_t*)kw,
                       (bf16_t*)vw, ws_cap);
  else
    hipLaunchKernelGGL((qkv_post_kernel<float, true>), grid, dim3(64), 0, st, (const void*)P, S, Prows, rope, pos, H,
                       Hkv, dh, (float*)q, (float*)kc, (float*)vc, T_cap, cache_row0, n_direct, (float*)kw,
                       (float*)vw, ws_cap);
}

void la_qkv_post_launch(int dtype, const void* qkv, const float2* rope, const int32_t* pos, int M, int H, int Hkv,
                        int dh, void* q, void* kc, void* vc, int T_cap, int cache_row0, int n_direct, void* kw,
                        void* vw, int ws_cap, hipStream_t st) {
  if (M <= 0) return;
  dim3 grid(M, H + 2 * Hkv);
  if (dtype == LA_DT_BF16)
    hipLaunchKernelGGL((qkv_post_kernel<bf16_t, false>), grid, dim3(64), 0, st, qkv, 0, 0, rope, pos, H, Hkv, dh,
                       (bf16_t*)q, (bf16_t*)kc, (bf16_t*)vc, T_cap, cache_row0, n_direct, (bf16_t*)kw, (bf16_t*)vw,
                       ws_cap);
  else
    hipLaunchKernelGGL((qkv_post_kernel<float, false>), grid, dim3(64), 0, st, qkv, 0, 0, rope, pos, H, Hkv, dh,
                       (float*)q, (float*)kc, (float*)vc, T_cap, cache_row0, n_direct, (float*)kw, (float*)vw,
                       ws_cap);
}

void la_qkv_post_multi_launch(int dtype, const float* P, int S, const void* qkv, int M, const LaPostSeg* segs, int n,
                              int layer, int H, int Hkv, int dh, void* q, hipStream_t st) {
  if (M <= 0 || n <= 0) return;
  dim3 grid(M, H + 2 * Hkv);
  const void* src = S > 0 ? (const void*)P : qkv;
  if (dtype == LA_DT_BF16) {
    if (S > 0)
      hipLaunchKernelGGL((qkv_post_multi_kernel<bf16_t, true>), grid, dim3(64), 0, st, src, S, M, segs, n, layer, H,
                         Hkv, dh, (bf16_t*)q);
    else
      hipLaunchKernelGGL((qkv_post_multi_kernel<bf16_t, false>), grid, dim3(64), 0, st, src, 0, M, segs, n, layer, H,
                         Hkv, dh, (bf16_t*)q);
  } else {
    if (S > 0)
      hipLaunchKernelGGL((qkv_post_multi_kernel<float, true>), grid, dim3(64), 0, st, src, S, M, segs, n, layer, H,
                         Hkv, dh, (float*)q);
    else
      hipLaunchKernelGGL((qkv_post_multi_kernel<float, false>), grid, dim3(64), 0, st, src, 0, M, segs, n, layer, H,
                         Hkv, dh, (float*)q);
  }
}

__global__ void fill_i32_kernel(int32_t* p, int n, int v) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = v;
}
void la_fill_i32_launch(int32_t* p, int n, int v, hipStream_t st) {
  if (n <= 0) return;
  hipLaunchKernelGGL(fill_i32_kernel, dim3((n + 255) / 256), dim3(256), 0, st, p, n, v);
}
