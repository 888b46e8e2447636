// Verify-and-accept: greedy survivor matching and exact one-hot sampling.
//
// "M7.3 - Lookahead Decoding", 0x05A: the first emitted token is the
// ordinary row's argmax; candidate c's hit length is the longest a with
// g_(1..a) = z^(c)_(1..a), z^(c) = (argmax out, argmax guess^(c)_1, ...);
// the accepted length h is the maximum hit, and every candidate reaching it
// exposes the same conditionals, so the lowest-index one is committed.  A
// full match emits S + 1 tokens; under the capped convention (the page's
// implementation-side max_hit count) hits stop at S - 1 and a round emits at
// most S tokens.  Ties in argmax go to the lowest token id.
//
// 0x05B: at each offset the distinct tokens offered by the surviving
// candidates are tested in candidate order as point masses -- token c is
// accepted with probability p(c) / (1 - sum p(rejected)); a rejection
// removes c's mass; acceptance filters the survivors; when every offered
// token is rejected the output is drawn from the residual.  The arithmetic
// is fixed IEEE fp64 so that the decisions are reproducible:
//   e_v = expneg((double(l_v) - double(l_max)) / T)  (Cody-Waite reduction
//   with a two-part ln2, degree-13 Taylor polynomial evaluated inner-first,
//   ldexp), sums blocked by 256 ids in id order, acceptance test
//   u * remaining < e_c, residual inverse-CDF over blocked cumulative sums.
// Randomness: Philox4x32-10 (Salmon et al., SC'11) keyed by the seed,
// counter (round, offset, draw, 0), u = ((x0>>5)*2^26 + (x1>>6)) * 2^-53.
#include "la_common.h"
#include "la_kernels.h"

// ---------------------------------------------------------------- argmax
// One 1024-thread block per row; each thread keeps 8 float4 loads in flight
// and scans its elements in index order (first maximum kept), then the block
// reduces with ties going to the lower index.
__global__ void __launch_bounds__(1024) argmax_kernel(const float* logits, int V, int32_t* out) {
  __shared__ float bv[1024];
  __shared__ int bi[1024];
  const float* x = logits + (size_t)blockIdx.x * V;
  float best = -__builtin_inff();
  int idx = 0x7fffffff;
  const int nv = V / 4;
  for (int base = 0; base < nv; base += 1024 * 8) {
    float4 r[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int v = base + threadIdx.x + 1024 * j;
      if (v < nv) r[j] = ((const float4*)x)[v];
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int v = base + threadIdx.x + 1024 * j;
      if (v < nv) {
        if (r[j].x > best) { best = r[j].x; idx = 4 * v; }
        if (r[j].y > best) { best = r[j].y; idx = 4 * v + 1; }
        if (r[j].z > best) { best = r[j].z; idx = 4 * v + 2; }
        if (r[j].w > best) { best = r[j].w; idx = 4 * v + 3; }
      }
    }
  }
  for (int i = 4 * nv + threadIdx.x; i < V; i += 1024) {       // tail when V is not a multiple of 4
    const float f = x[i];
    if (f > best || (f == best && i < idx)) { best = f; idx = i; }
  }
  bv[threadIdx.x] = best;
  bi[threadIdx.x] = idx;
  __syncthreads();
  for (int s = 512; s > 0; s >>= 1) {
    if (threadIdx.x < s) {
      const float v2 = bv[threadIdx.x + s];
      const int i2 = bi[threadIdx.x + s];
      if (v2 > bv[threadIdx.x] || (v2 == bv[threadIdx.x] && i2 < bi[threadIdx.x])) {
        bv[threadIdx.x] = v2;
        bi[threadIdx.x] = i2;
      }
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) out[blockIdx.x] = bi[0] == 0x7fffffff ? 0 : bi[0];
}

void la_argmax_launch(const float* logits, int rows, int V, int32_t* out, hipStream_t st) {
  if (rows <= 0) return;
  hipLaunchKernelGGL(argmax_kernel, dim3(rows), dim3(1024), 0, st, logits, V, out);
}

// ---------------------------------------------------------------- greedy
__global__ void greedy_accept_kernel(const int32_t* amax, int n_inp, const int32_t* cand, int C, int S, int hmax,
                                     LaAcceptDev* acc, int32_t* z) {
  __shared__ int hits[64];
  const int t = threadIdx.x;
  const int gbase = 1 + n_inp;
  for (int c = t; c < 64; c += blockDim.x) {
    int a = 0;
    if (c < C) {
      while (a < hmax) {
        const int za = a == 0 ? amax[0] : amax[gbase + c * S + a - 1];
        if (cand[c * S + a] != za) break;
        ++a;
      }
    }
    hits[c] = c < C ? a : -1;
  }
  for (int j = t; j < n_inp; j += blockDim.x) z[j] = amax[1 + j];
  __syncthreads();
  if (t == 0) {
    int h = 0, w = -1;
    for (int c = 0; c < C; ++c)
      if (hits[c] > h) { h = hits[c]; w = c; }
    acc->h = h;
    acc->winner = h > 0 ? w : -1;
    acc->n_emit = h + 1;
    acc->emitted[0] = amax[0];
    for (int k = 1; k <= h; ++k) acc->emitted[k] = amax[gbase + w * S + k - 1];
  }
}

void la_greedy_accept_launch(const int32_t* amax, int n_inp, const int32_t* cand, int C, int S, int hmax,
                             LaAcceptDev* acc, int32_t* z, hipStream_t st) {
  hipLaunchKernelGGL(greedy_accept_kernel, dim3(1), dim3(64), 0, st, amax, n_inp, cand, C, S, hmax, acc, z);
}

// ---------------------------------------------------------------- sampling
__device__ __forceinline__ void philox4x32_10(uint32_t c[4], uint32_t k0, uint32_t k1) {
  for (int r = 0; r < 10; ++r) {
    if (r) { k0 += 0x9E3779B9u; k1 += 0xBB67AE85u; }
    const uint32_t lo0 = 0xD2511F53u * c[0], hi0 = __umulhi(0xD2511F53u, c[0]);
    const uint32_t lo1 = 0xCD9E8D57u * c[2], hi1 = __umulhi(0xCD9E8D57u, c[2]);
    const uint32_t n0 = hi1 ^ c[1] ^ k0, n2 = hi0 ^ c[3] ^ k1;
    c[0] = n0; c[1] = lo1; c[2] = n2; c[3] = lo0;
  }
}

__device__ double la_uniform(uint64_t seed, uint32_t round, uint32_t offset, uint32_t draw) {
  uint32_t c[4] = {round, offset, draw, 0u};
  philox4x32_10(c, (uint32_t)seed, (uint32_t)(seed >> 32));
  return ((double)(c[0] >> 5) * 67108864.0 + (double)(c[1] >> 6)) * (1.0 / 9007199254740992.0);
}

#pragma clang fp contract(off)
__device__ double la_expneg(double a) {
  const double LN2_HI = 0x1.62e42fee00000p-1;
  const double LN2_LO = 0x1.a39ef35793c76p-33;
  const double INV_LN2 = 0x1.71547652b82fep+0;
  if (a < -745.0) return 0.0;
  const double k = __builtin_rint(a * INV_LN2);
  const double r = (a - k * LN2_HI) - k * LN2_LO;
  double p = 1.0;
  for (int n = 13; n >= 1; --n) p = 1.0 + (r / (double)n) * p;
  return ldexp(p, (int)k);
}

#define SBLK 256
#define MAXBLK 256
#define VT 1024        // threads of the sampling workgroup

// This thread's share of a row's maximum: 16-byte loads, eight in flight
// (the maximum of a set does not depend on the order it is taken in).
__device__ float row_max_part(const float* x, int V) {
  const int nt = blockDim.x;
  const int n4 = ((uintptr_t)x & 15) ? 0 : V / 4;  // a caller's row may start off 16 bytes: plain loads then
  const float4* x4 = (const float4*)x;
  float mx = -__builtin_inff();
  for (int i0 = threadIdx.x; i0 < n4; i0 += 8 * nt) {
    float4 v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int i = i0 + j * nt;
      v[j] = i < n4 ? x4[i] : make_float4(-__builtin_inff(), -__builtin_inff(), -__builtin_inff(), -__builtin_inff());
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) mx = fmaxf(mx, fmaxf(fmaxf(v[j].x, v[j].y), fmaxf(v[j].z, v[j].w)));
  }
  for (int i = 4 * n4 + (int)threadIdx.x; i < V; i += nt) mx = fmaxf(mx, x[i]);
  return mx;
}

// masses of one row into e[], block sums into bs[] (shared).  Every thread
// evaluates masses at a stride of the workgroup (the costly part: the fp64
// polynomial with its exact divisions); then one thread per block of SBLK ids
// sums that block in id order.
__device__ void row_masses(const float* x, int V, double T, double* e, double* bs, float* red) {
  red[threadIdx.x] = row_max_part(x, V);
  __syncthreads();
  for (int s = blockDim.x / 2; s > 0; s >>= 1) {
    if (threadIdx.x < s) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + s]);
    __syncthreads();
  }
  const double lmax = (double)red[0];
  for (int i = threadIdx.x; i < V; i += blockDim.x) e[i] = la_expneg(((double)x[i] - lmax) / T);
  __syncthreads();                                // every mass is visible to the workgroup
  const int nb = (V + SBLK - 1) / SBLK;
  for (int b = threadIdx.x; b < nb; b += blockDim.x) {
    // eight loads ahead of their adds; ids past V add +0.0, which leaves a
    // sum of non-negative masses unchanged
    double s = 0.0;
    const int end = min(V, (b + 1) * SBLK);
    for (int i = b * SBLK; i < end; i += 8) {
      double v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = i + j < end ? e[i + j] : 0.0;
#pragma unroll
      for (int j = 0; j < 8; ++j) s = s + v[j];
    }
    bs[b] = s;
  }
  __syncthreads();
}

// The same masses and block sums for one row, spread over the GPU: one
// workgroup per block of SBLK ids (every workgroup takes the whole row's
// maximum itself, so all use the same one); thread 0 sums the block in id
// order.  Block sums land in bs_g (global).
__global__ void __launch_bounds__(SBLK) sample_masses_kernel(const float* x, int V, double T, double* e,
                                                              double* bs_g) {
  __shared__ float red[SBLK];
  __shared__ double eb[SBLK];
  red[threadIdx.x] = row_max_part(x, V);
  __syncthreads();
  for (int s = SBLK / 2; s > 0; s >>= 1) {
    if (threadIdx.x < s) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + s]);
    __syncthreads();
  }
  const double lmax = (double)red[0];
  const int b = blockIdx.x, i = b * SBLK + (int)threadIdx.x;
  double ev = 0.0;
  if (i < V) {
    ev = la_expneg(((double)x[i] - lmax) / T);
    e[i] = ev;
  }
  eb[threadIdx.x] = ev;
  __syncthreads();
  if (threadIdx.x == 0) {
    double sum = 0.0;
    const int n = min(SBLK, V - b * SBLK);
    for (int j = 0; j < n; ++j) sum = sum + eb[j];
    bs_g[b] = sum;
  }
}

// block sums of row masses computed by sample_masses_kernel, into shared bs
__device__ void load_block_sums(const double* bs_g, int V, double* bs) {
  const int nb = (V + SBLK - 1) / SBLK;
  for (int b = threadIdx.x; b < nb; b += blockDim.x) bs[b] = bs_g[b];
  __syncthreads();
}

// Residual inverse-CDF draw (tokens rejected already excluded from e / bs),
// by the whole workgroup: thread 0 finds the block the target falls in, the
// workgroup stages that block's masses in LDS (eb), and thread 0 walks them
// -- the serial walk over the same sums.  A block that yields nothing (which
// the sums' equality rules out) resumes the walk from global memory.  The
// result is valid in thread 0.
__device__ int residual_draw(const double* e, const double* bs, int V, double u, int amax_tok, double* eb,
                             int* blk_s, double* walk_s) {
  const int nb = (V + SBLK - 1) / SBLK;
  if (threadIdx.x == 0) {
    double R = 0.0;
    for (int b = 0; b < nb; ++b) R = R + bs[b];
    int blk = -1;                                 // -1: no positive mass
    double acc = 0.0, target = 0.0;
    if (R > 0.0) {
      target = u * R;
      blk = nb;                                   // nb: no block reaches the target
      for (int b = 0; b < nb; ++b) {
        if (acc + bs[b] > target) {
          blk = b;
          break;
        }
        acc = acc + bs[b];
      }
    }
    *blk_s = blk;
    walk_s[0] = acc;
    walk_s[1] = target;
  }
  __syncthreads();
  const int blk = *blk_s;
  if (blk >= 0 && blk < nb) {
    const int i = blk * SBLK + (int)threadIdx.x;
    if (threadIdx.x < SBLK) eb[threadIdx.x] = i < V ? e[i] : 0.0;
    __syncthreads();
  }
  if (threadIdx.x != 0 || blk < 0) return amax_tok;
  double acc = walk_s[0];
  const double target = walk_s[1];
  if (blk < nb) {
    double local = 0.0;
    const int end = min(V, (blk + 1) * SBLK);
    for (int i = blk * SBLK; i < end; ++i) {
      local = local + eb[i - blk * SBLK];
      if (acc + local > target) return i;
    }
    acc = acc + bs[blk];
    for (int b = blk + 1; b < nb; ++b) {
      if (acc + bs[b] > target) {
        local = 0.0;
        const int e2 = min(V, (b + 1) * SBLK);
        for (int i = b * SBLK; i < e2; ++i) {
          local = local + e[i];
          if (acc + local > target) return i;
        }
      }
      acc = acc + bs[b];
    }
  }
  for (int i = V - 1; i >= 0; --i)
    if (e[i] > 0.0) return i;
  return amax_tok;
}

// zero the masses of the rejected tokens, then recompute their blocks' sums
// in id order; thread k < nrej takes rejection k (two rejections in one block
// write the same sum)
__device__ void exclude(double* e, double* bs, int V, const int* rej, int nrej) {
  if ((int)threadIdx.x < nrej) e[rej[threadIdx.x]] = 0.0;
  __syncthreads();
  if ((int)threadIdx.x < nrej) {
    const int b = rej[threadIdx.x] / SBLK;
    double s = 0.0;
    const int end = min(V, (b + 1) * SBLK);
    for (int i = b * SBLK; i < end; ++i) s = s + e[i];
    bs[b] = s;
  }
  __syncthreads();
}

__global__ void __launch_bounds__(VT) sample_accept_kernel(const float* logits, int V, int n_inp,
                                                           const int32_t* amax, const int32_t* cand, int C, int S,
                                                           int hmax, double T, uint64_t seed, int round_id,
                                                           double* e, LaAcceptDev* acc, int32_t* z) {
  __shared__ double bs[MAXBLK];
  __shared__ float red[VT];
  __shared__ int surv[64];
  __shared__ int nsurv;
  __shared__ int done, accepted, nrej_s;
  __shared__ int rej[64];
  __shared__ int ctok[64];                        // offered tokens of the survivors, their masses and draws
  __shared__ double cm[64], cu[64];
  __shared__ double eb[SBLK], walk_s[2];
  __shared__ int blk_s;
  const int gbase = 1 + n_inp;
  for (int j = threadIdx.x; j < n_inp; j += blockDim.x) z[j] = amax[1 + j];
  if (threadIdx.x == 0) {
    nsurv = C;
    for (int c = 0; c < C; ++c) surv[c] = c;
    done = 0;
  }
  __syncthreads();
  int n_emit = 0;
  for (int a = 0; a <= hmax; ++a) {
    const int row = a == 0 ? 0 : gbase + surv[0] * S + a - 1;
    if (a == 0) load_block_sums(e + V, V, bs);   // row 0's masses: sample_masses_kernel, launched first
    else row_masses(logits + (size_t)row * V, V, T, e, bs, red);
    // survivor si offers its token at offset a; the k-th distinct test uses draw k (k < nsurv)
    if (a < hmax && (int)threadIdx.x < nsurv) {
      const int tok = cand[surv[threadIdx.x] * S + a];
      ctok[threadIdx.x] = tok;
      cm[threadIdx.x] = e[tok];
      cu[threadIdx.x] = la_uniform(seed, (uint32_t)round_id, (uint32_t)a, threadIdx.x);
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      const int nb = (V + SBLK - 1) / SBLK;
      double Z = 0.0;
      for (int b = 0; b < nb; ++b) Z = Z + bs[b];
      double remaining = Z;
      int nrej = 0;
      accepted = -1;
      if (a < hmax) {
        int k = 0;
        for (int si = 0; si < nsurv && accepted < 0; ++si) {
          const int tok = ctok[si];
          bool seen = false;
          for (int q = 0; q < nrej; ++q) seen |= rej[q] == tok;
          if (seen) continue;
          const double u = cu[k];
          ++k;
          if (u * remaining < cm[si]) {
            accepted = tok;
          } else {
            remaining = remaining - cm[si];
            rej[nrej++] = tok;
          }
        }
      }
      nrej_s = nrej;
      if (accepted >= 0) {
        acc->emitted[a] = accepted;
        int ns = 0;
        for (int si = 0; si < nsurv; ++si)
          if (cand[surv[si] * S + a] == accepted) surv[ns++] = surv[si];
        nsurv = ns;
      }
    }
    __syncthreads();
    if (accepted < 0) {                           // every offered token rejected: the residual draw
      exclude(e, bs, V, rej, nrej_s);
      const double u = la_uniform(seed, (uint32_t)round_id, (uint32_t)a, 1024u);
      const int tok = residual_draw(e, bs, V, u, amax[row], eb, &blk_s, walk_s);
      if (threadIdx.x == 0) {
        acc->emitted[a] = tok;
        done = 1;
      }
    }
    __syncthreads();
    n_emit = a + 1;
    if (done) break;
  }
  if (threadIdx.x == 0) {
    const int h = n_emit - 1;
    acc->h = h;
    acc->n_emit = n_emit;
    acc->winner = h > 0 ? surv[0] : -1;
  }
}

void la_sample_accept_launch(const float* logits, int V, int n_inp, const int32_t* amax, const int32_t* cand,
                               int C, int S, int hmax, double T, uint64_t seed, int round_id, double* scratch,
                               LaAcceptDev* acc, int32_t* z, hipStream_t st) {
  hipLaunchKernelGGL(sample_masses_kernel, dim3((V + SBLK - 1) / SBLK), dim3(SBLK), 0, st, logits, V, T, scratch,
                     scratch + V);
  hipLaunchKernelGGL(sample_accept_kernel, dim3(1), dim3(VT), 0, st, logits, V, n_inp, amax, cand, C, S, hmax, T,
                     seed, round_id, scratch, acc, z);
}

// plain target sample of row 0 (first token after prefill; autoregressive sampling)
__global__ void __launch_bounds__(VT) sample_row_kernel(const float* logits, int V, double T, uint64_t seed,
                                                        int round_id, const int32_t* amax, double* e, int32_t* out) {
  __shared__ double bs[MAXBLK];
  __shared__ double eb[SBLK], walk_s[2];
  __shared__ int blk_s;
  load_block_sums(e + V, V, bs);                 // the masses: sample_masses_kernel, launched first
  const double u = la_uniform(seed, (uint32_t)round_id, 0u, 1024u);
  const int tok = residual_draw(e, bs, V, u, amax[0], eb, &blk_s, walk_s);
  if (threadIdx.x == 0) out[0] = tok;
}

void la_sample_row_launch(const float* logits, int V, double T, uint64_t seed, int round_id, const int32_t* amax,
                          double* scratch, int32_t* out, hipStream_t st) {
  hipLaunchKernelGGL(sample_masses_kernel, dim3((V + SBLK - 1) / SBLK), dim3(SBLK), 0, st, logits, V, T, scratch,
                     scratch + V);
  hipLaunchKernelGGL(sample_row_kernel, dim3(1), dim3(VT), 0, st, logits, V, T, seed, round_id, amax, scratch, out);
}
