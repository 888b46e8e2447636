// Packed-row builder: one immutable row manifest per round.
//
// "M7.3 - Lookahead Decoding", 0x04 and 0x04A: one ordinary row, the
// lookahead trajectory rows and C candidate suffixes of S rows are packed
// into one call; a shared row record (role, level, column, candidate,
// offset, logical position, requested logit) feeds tokens, positions, the
// branch mask and the output slices; the visibility sets are
//   Vis(b_j) = {b_k : k <= j},  Vis(u_(r,j)) = {b_k : k <= j} U {u_(q,j) : q <= r},
//   Vis(v_(c,s)) = {b_0} U {v_(c,q) : q <= s},
// plus the committed prefix for everyone.  Logical positions:
// pos(b_j) = p + j, pos(u_(r,j)) = p + j + r, pos(v_(c,s)) = p + 1 + s.
//
// Physical order here is branch-major (the pages' dense path is level-major;
// their specialised attention path uses its own permutation as well):
// column j contributes [b_j, u_(1,j), ..., u_(d_j,j)] (b_0 is the ordinary
// row, packed row 0), then candidate c contributes [v_(c,0..S-1)].
//
// Under these sets a row at position t sees exactly one row at each
// logical position p .. t, so the mask is stored as a *path* per branch:
// path[b][k] is the workspace row holding logical position p + 1 + k on
// branch b (column j: b_1..b_j then u_(1..d_j, j); candidate c:
// v_(c,0..S-1)).  Row i sees row k iff k is the ordinary row, or
// pos_k <= pos_i and path[branch_i][pos_k - p - 1] is k's workspace row.
// The attention kernel gathers keys through the path; the bit mask is the
// same relation written out (for auditing against the dense definition).
#include "la_common.h"
#include "la_dev.h"
#include "la_kernels.h"

static int level_at(const LaLayout* L, int r, int j) {
  return L->sizes[r] > 0 && j >= L->starts[r] && j < L->starts[r] + L->sizes[r];
}

int la_layout_finish(LaLayout* L) {
  if (L->R < 1 || L->R > 16 || L->sizes[0] < 0 || L->S < 1 || L->C < 0) return -1;
  L->starts[0] = 1;
  const int ncols = L->sizes[0] + 1;
  L->n_cols = ncols;
  int Q = 0, maxp = L->S;
  for (int j = 0; j < ncols; ++j) {
    int depth = 0;
    for (int r = 1; r < L->R; ++r) {
      if (level_at(L, r, j)) {
        if (depth != r - 1) return -1;            // levels at a column must be nested 1..d
        depth = r;
      }
    }
    Q += 1 + depth;
    if (j + depth > maxp) maxp = j + depth;
  }
  for (int r = 1; r < L->R; ++r)
    if (L->sizes[r] > 0 && (L->starts[r] < 0 || L->starts[r] + L->sizes[r] > ncols)) return -1;
  Q += L->C * L->S;
  L->Q = Q;
  L->NB = ncols + L->C;
  L->maxp = maxp;
  int deepest = 0;
  for (int r = 0; r < L->R; ++r)
    if (L->sizes[r] > 0) deepest = r;
  L->n_inp = L->sizes[deepest];
  L->n_logit = 1 + L->n_inp + L->C * L->S;
  L->mask_words = (Q + 31) / 32;
  return 0;
}

__device__ static int d_level_at(const LaLayout& L, int r, int j) {
  return L.sizes[r] > 0 && j >= L.starts[r] && j < L.starts[r] + L.sizes[r];
}
__device__ static int d_depth(const LaLayout& L, int j) {
  int d = 0;
  for (int r = 1; r < L.R; ++r)
    if (d_level_at(L, r, j)) d = r;
  return d;
}
#define LA_MAX_COLS 128   // window columns the builder's tables hold (W + N - 2 <= 64 + 14)

// LDS mirrors of what the later phases read back (positions, branches,
// paths, tile tables), so the mask and tile phases do no global loads
__host__ __device__ static size_t rows_lds_bytes(const LaLayout& L) {
  const int ntiles = (L.Q + 15) / 16;
  return ((size_t)2 * L.Q + L.NB + (size_t)L.NB * L.maxp + (size_t)ntiles * 64) * 4;
}

__global__ void __launch_bounds__(256) build_rows_kernel(LaLayout L, int x_t, const int32_t* win, int win_stride,
                                                         const int32_t* cands, LaRowsDev o) {
  extern __shared__ int32_t sm[];
  const int ntiles = (L.Q + 15) / 16;
  int32_t* const s_pos = sm;                       // [Q]
  int32_t* const s_br = s_pos + L.Q;               // [Q]
  int32_t* const s_plen = s_br + L.Q;              // [NB]
  int32_t* const s_path = s_plen + L.NB;           // [NB][maxp]
  int32_t* const s_meta = s_path + (size_t)L.NB * L.maxp;   // [ntiles][64]
  const int t = threadIdx.x;
  const int p = L.p;
  const int cand_start = L.Q - L.C * L.S;
  // column depths and first rows, once (the layout's level table is read per column here only)
  __shared__ int s_depth[LA_MAX_COLS], s_cs[LA_MAX_COLS + 1];
  for (int j = t; j < L.n_cols; j += blockDim.x) s_depth[j] = d_depth(L, j);
  __syncthreads();
  if (t == 0) {
    int acc = 0;
    for (int j = 0; j < L.n_cols; ++j) {
      s_cs[j] = acc;
      acc += 1 + s_depth[j];
    }
    s_cs[L.n_cols] = acc;
  }
  __syncthreads();
  auto put_row = [&](int row, int tok, int pos, int role, int level, int col, int cand, int off, int br) {
    o.tok[row] = tok;
    o.pos[row] = pos;
    o.role[row] = role;
    o.level[row] = level;
    o.col[row] = col;
    o.cand[row] = cand;
    o.off[row] = off;
    o.branch[row] = br;
    s_pos[row] = pos;
    s_br[row] = br;
  };
  auto put_path = [&](int b, int e, int v) {
    o.path[(size_t)b * L.maxp + e] = v;
    s_path[(size_t)b * L.maxp + e] = v;
  };
  // columns
  for (int j = t; j < L.n_cols; j += blockDim.x) {
    const int cs = s_cs[j];
    const int depth = s_depth[j];
    put_row(cs, j == 0 ? x_t : win[j - 1], p + j, j == 0 ? 0 : 1, 0, j, -1, -1, j);   // b_j
    for (int r = 1; r <= depth; ++r)
      put_row(cs + r, win[r * win_stride + (j - L.starts[r])], p + j + r, 1, r, j, -1, -1, j);
    for (int k = 0; k < j; ++k) put_path(j, k, s_cs[k + 1] - 1);
    for (int r = 1; r <= depth; ++r) put_path(j, j + r - 1, cs + r - 1);
    o.path_len[j] = j + depth;
    s_plen[j] = j + depth;
  }
  // candidates
  for (int c = t; c < L.C; c += blockDim.x) {
    const int b = L.n_cols + c;
    for (int s = 0; s < L.S; ++s) {
      const int row = cand_start + c * L.S + s;
      put_row(row, cands[c * L.S + s], p + 1 + s, 2, -1, -1, c, s, b);
      put_path(b, s, row - 1);
    }
    o.path_len[b] = L.S;
    s_plen[b] = L.S;
  }
  // logit rows: out, inp (deepest level, column order), guess ((c, s) order)
  int deepest = 0;
  for (int r = 0; r < L.R; ++r)
    if (L.sizes[r] > 0) deepest = r;
  if (t == 0) o.logit_rows[0] = 0;
  for (int i = t; i < L.n_inp; i += blockDim.x) {
    const int j = deepest == 0 ? 1 + i : L.starts[deepest] + i;
    o.logit_rows[1 + i] = s_cs[j] + deepest;
  }
  for (int i = t; i < L.C * L.S; i += blockDim.x) o.logit_rows[1 + L.n_inp + i] = cand_start + i;
  __syncthreads();
  // compact visibility mask, derived from the paths: one bit per lane (row
  // i, word w, bit b at index (i * nw + w) * 32 + b), the wave's ballot gives
  // two whole words (the loop steps whole waves, so words never straddle)
  const int nw = L.mask_words;
  const int nbits = L.Q * nw * 32;
  for (int base = t - (t & 63); base < nbits; base += blockDim.x) {
    const int idx = base + (t & 63);
    bool vis = false;
    if (idx < nbits) {
      const int i = idx / (nw * 32), k = idx % (nw * 32);
      if (k == 0) vis = true;
      else if (k < L.Q) {
        const int pk = s_pos[k], e = pk - p - 1;
        const int bi = s_br[i];
        vis = pk <= s_pos[i] && e >= 0 && e < s_plen[bi] && s_path[(size_t)bi * L.maxp + e] == k - 1;
      }
    }
    const unsigned long long m = __ballot(vis);
    if ((t & 31) == 0 && idx < nbits) o.mask[idx / 32] = (uint32_t)(m >> (t & 32));
  }
  // per 16-row tile: its distinct branches in row order (rows are branch
  // major, so a tile holds a few consecutive runs) and their paths, which
  // the attention kernel stages for the keys past the committed prefix
  for (int tt = t; tt < ntiles; tt += blockDim.x) {
    int32_t* meta = s_meta + (size_t)tt * 64;
    int nb = 0;
    for (int i = 16 * tt; i < 16 * tt + 16 && i < L.Q; ++i) {
      const int b = s_br[i];
      bool seen = false;
      for (int k = 0; k < nb; ++k) seen |= meta[1 + k] == b;
      if (!seen) meta[1 + nb++] = b;
    }
    meta[0] = nb;
    for (int k = 1 + nb; k < 64; ++k) meta[k] = -1;
  }
  __syncthreads();
  for (int idx = t; idx < ntiles * 64; idx += blockDim.x) o.tile_meta[idx] = s_meta[idx];
  for (int idx = t; idx < ntiles * 1024; idx += blockDim.x) {
    const int tt = idx / 1024, i = (idx / 64) % 16, e = idx % 64;
    const int32_t* meta = s_meta + (size_t)tt * 64;
    int v = -1;
    if (i < meta[0]) {
      const int b = meta[1 + i];
      if (e < s_plen[b] && e < L.maxp) v = s_path[(size_t)b * L.maxp + e];
      if (v < 0 || v >= L.Q - 1) v = -1;
    }
    o.tile_path[idx] = v;
  }
}

int la_build_rows_fits(const LaLayout& L) {
  return rows_lds_bytes(L) <= (size_t)(LDS_BYTES - 2048) && L.n_cols <= LA_MAX_COLS;
}

int la_build_rows_launch(const LaLayout& L, int x_t, const int32_t* win, int win_stride, const int32_t* cands,
                         LaRowsDev rows, hipStream_t st) {
  const size_t lds = rows_lds_bytes(L);
  constexpr int DYN_MAX = LDS_BYTES - 2048;       // beside the static column tables
  if (lds > DYN_MAX || L.n_cols > LA_MAX_COLS) return -2;
  if (lds > 65536) {                              // above the default dynamic limit
    static const bool attr = hipFuncSetAttribute((const void*)&build_rows_kernel,
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, DYN_MAX) == hipSuccess;
    if (!attr) return -2;
  }
  hipLaunchKernelGGL(build_rows_kernel, dim3(1), dim3(256), lds, st, L, x_t, win, win_stride, cands, rows);
  return 0;
}
