// Per-request proposal state on the device: keyed n-gram pool, trajectory
// window, and publication of accepted K/V rows.
//
// Pool ("M7.3 - Lookahead Decoding", 0x03 / 0x03B): a map from a first token
// to at most G suffixes of S = N - 1 tokens, least-recently-used first.
// Keys are token ids, so the table is direct-addressed by key (an identity
// hash): cnt[V] and ent[V][G][S].  An upsert moves an existing suffix to the
// most-recent end, evicts entry 0 of a full list, or appends.  One wavefront
// performs the upserts of a round one after another in extraction order:
// lane e compares list entry e with the suffix, a ballot finds the match,
// and the list is shifted in registers.  Extraction: column j's key is x_t
// (j = 0) or level-0 cell j-1, its suffix is levels 1..R-1 at column j and
// the new output z_j.
//
// Window (0x03A / 0x03C): warmup fills shift every level left by one and
// append the deepest level's outputs (dropping the first when the source
// level is >= 1); the steady ALWAYS_FWD_ONE advance is
// [level1[1:], level2, ..., z].
//
// Publication (0x06B / 0x06C / 0x07): the winning candidate's first h rows
// hold the K/V of the accepted candidate inputs; they are copied right
// after the ordinary row's K/V (already at cache row K_in), everything else
// in the workspace is dropped.
#include "la_common.h"
#include "la_kernels.h"

#define POOL_MAX_S 16

__device__ void pool_upsert_one(int32_t* cnt, int32_t* ent, int key, const int* suf, int G, int S) {
  const int lane = threadIdx.x;
  int32_t* bucket = ent + (size_t)key * G * S;
  const int c = cnt[key];
  int mine[POOL_MAX_S];
  bool match = false;
  if (lane < c) {
    match = true;
    for (int s = 0; s < S; ++s) {
      mine[s] = bucket[lane * S + s];
      match = match && mine[s] == suf[s];
    }
  }
  const unsigned long long bal = __ballot(match);
  int shift_from, slot;
  if (bal) {
    shift_from = __ffsll((long long)bal);      // entries after the match move down one
    slot = c - 1;
  } else if (c == G) {
    shift_from = 1;                            // evict entry 0
    slot = G - 1;
  } else {
    shift_from = c;                            // nothing moves
    slot = c;
  }
  __asm__ volatile("" ::: "memory");
  if (lane >= shift_from && lane < c)
    for (int s = 0; s < S; ++s) bucket[(lane - 1) * S + s] = mine[s];
  if (lane < S) bucket[slot * S + lane] = suf[lane];
  if (lane == 0 && !bal && c < G) cnt[key] = c + 1;
  // the next upsert is this wavefront's own: workgroup scope orders it (no L2 write-back)
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
}

__global__ void __launch_bounds__(64) pool_upsert_kernel(int32_t* cnt, int32_t* ent, const int32_t* keys,
                                                         const int32_t* sufs, int n, int G, int S) {
  int suf[POOL_MAX_S];
  for (int i = 0; i < n; ++i) {
    for (int s = 0; s < S; ++s) suf[s] = sufs[i * S + s];
    pool_upsert_one(cnt, ent, keys[i], suf, G, S);
  }
}

void la_pool_upsert_launch(int32_t* cnt, int32_t* ent, const int32_t* keys, const int32_t* sufs, int n, int G,
                           int S, hipStream_t st) {
  if (n <= 0) return;
  hipLaunchKernelGGL(pool_upsert_kernel, dim3(1), dim3(64), 0, st, cnt, ent, keys, sufs, n, G, S);
}

// extraction of the W keyed n-grams from the pre-shift window and z, then
// upsert in column order.  Workgroup j owns key k_j when no earlier column
// has the same key, and applies every column with that key in column order:
// different keys touch different buckets, so the per-key order (all the LRU
// rule depends on) is the serial one and the keys proceed in parallel.
__global__ void __launch_bounds__(64) pool_collect_kernel(int32_t* cnt, int32_t* ent, int x_t, const int32_t* win,
                                                          int stride, int R, int W, const int32_t* z, int G) {
  const int S = R;
  const int j0 = blockIdx.x;
  auto key_of = [&](int j) { return j == 0 ? x_t : win[j - 1]; };
  const int key = key_of(j0);
  for (int j = 0; j < j0; ++j)
    if (key_of(j) == key) return;               // an earlier column owns this key
  int suf[POOL_MAX_S];
  for (int j = j0; j < W; ++j) {
    if (j > j0 && key_of(j) != key) continue;
    for (int r = 1; r < R; ++r) suf[r - 1] = win[r * stride + j];
    suf[R - 1] = z[j];
    pool_upsert_one(cnt, ent, key, suf, G, S);
  }
}

void la_pool_collect_launch(int32_t* cnt, int32_t* ent, int x_t, const int32_t* win, int win_stride, int R, int W,
                            const int32_t* z, int G, hipStream_t st) {
  if (W <= 0) return;
  hipLaunchKernelGGL(pool_collect_kernel, dim3(W), dim3(64), 0, st, cnt, ent, x_t, win, win_stride, R, W, z, G);
}

__global__ void __launch_bounds__(64) pool_lookup_kernel(const int32_t* cnt, const int32_t* ent, int key, int G,
                                                         int S, int32_t* out, int32_t* n) {
  const int c = min(cnt[key], G);
  const int32_t* bucket = ent + (size_t)key * G * S;
  for (int i = threadIdx.x; i < c * S; i += 64) out[i] = bucket[i];
  if (threadIdx.x == 0) *n = c;
}

void la_pool_lookup_launch(const int32_t* cnt, const int32_t* ent, int key, int G, int S, int32_t* out, int32_t* n,
                           hipStream_t st) {
  hipLaunchKernelGGL(pool_lookup_kernel, dim3(1), dim3(64), 0, st, cnt, ent, key, G, S, out, n);
}

void la_pool_clear_launch(int32_t* cnt, int V, hipStream_t st) { la_fill_i32_launch(cnt, V, 0, st); }

// ---------------------------------------------------------------- window
struct WinArgs {
  int so[16], sn[16];
};

// steady state: entry i of the advanced level r is entry i + shift of the
// pinned advance (level 0 <- level 1 from its second entry, level r <- r + 1,
// the deepest <- z), or `fill` past its end (shift 0: the pinned advance)
__global__ void window_next_kernel(const int32_t* win, int32_t* out, int stride, int R, WinArgs sz, int deepest,
                                   int warm, const int32_t* z, int nz, int shift, int fill) {
  for (int idx = threadIdx.x; idx < R * stride; idx += blockDim.x) {
    const int r = idx / stride, i = idx % stride;
    int v = 0;
    if (i < sz.sn[r]) {
      if (warm) {
        const int k = i + shift;
        if (k >= sz.sn[r]) v = fill;
        else if (r == 0) v = win[1 * stride + k + 1];
        else if (r < R - 1) v = win[(r + 1) * stride + k];
        else v = z[k];
      } else {
        if (r <= deepest) v = win[r * stride + i + 1];
        else if (r == deepest + 1) v = deepest >= 1 ? z[i + 1] : z[i];
      }
    }
    out[idx] = v;
  }
}

void la_window_next_launch(const int32_t* win, int32_t* out, int stride, int R, const int* sizes_old,
                           const int* sizes_new, int deepest, int warm, const int32_t* z, int nz, int shift,
                           int fill, hipStream_t st) {
  WinArgs a;
  for (int r = 0; r < 16; ++r) {
    a.so[r] = r < R ? sizes_old[r] : 0;
    a.sn[r] = r < R ? sizes_new[r] : 0;
  }
  hipLaunchKernelGGL(window_next_kernel, dim3(1), dim3(256), 0, st, win, out, stride, R, a, deepest, warm, z, nz,
                     warm ? shift : 0, fill);
}

// ---------------------------------------------------------------- K/V commit
template <typename T>
__global__ void kv_commit_kernel(T* kc, T* vc, const T* kw, const T* vw, int Hkv, int dh, int T_cap, int ws_cap,
                                 int dst_row0, int src_row0) {
  const int lg = blockIdx.x;             // layer * Hkv + kv head
  const int j = blockIdx.y;              // accepted row
  const size_t cbase = ((size_t)lg * T_cap + dst_row0 + j) * dh;
  const size_t wbase = ((size_t)lg * ws_cap + src_row0 + j) * dh;
  for (int i = threadIdx.x; i < dh; i += blockDim.x) {
    kc[cbase + i] = kw[wbase + i];
    vc[cbase + i] = vw[wbase + i];
  }
}

void la_kv_commit_launch(int dtype, void* kc, void* vc, const void* kw, const void* vw, int L, int Hkv, int dh,
                         int T_cap, int ws_cap, int dst_row0, int src_row0, int h, hipStream_t st) {
  if (h <= 0) return;
  dim3 grid(L * Hkv, h);
  if (dtype == LA_DT_BF16)
    hipLaunchKernelGGL(kv_commit_kernel<bf16_t>, grid, dim3(64), 0, st, (bf16_t*)kc, (bf16_t*)vc, (const bf16_t*)kw,
                       (const bf16_t*)vw, Hkv, dh, T_cap, ws_cap, dst_row0, src_row0);
  else
    hipLaunchKernelGGL(kv_commit_kernel<float>, grid, dim3(64), 0, st, (float*)kc, (float*)vc, (const float*)kw,
                       (const float*)vw, Hkv, dh, T_cap, ws_cap, dst_row0, src_row0);
}
