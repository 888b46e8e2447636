// Internal launch interface between the host orchestrator and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

enum { LA_DT_F32 = 0, LA_DT_BF16 = 1 };
enum { LA_EPI_STORE = 0, LA_EPI_RESID = 1, LA_EPI_SWIGLU = 2, LA_EPI_F32 = 3, LA_EPI_PARTIAL = 4, LA_EPI_QKV = 5 };
// Fused QKV epilogue: the projection's columns are packed pair-major (la_gemm_pack_launch with rope_dh = dh), each
// value is rounded to the storage type, rotated at its row's logical position (q and k) and written to q [M][H][dh]
// and to the K/V cache (the first n_direct rows, at cache row cache_row0 + m) or the workspace (row m - n_direct).
struct LaQkvOut {
  const float2* rope;   // [positions][dh/2] (cos, sin)
  const int32_t* pos;   // [M]
  void *q, *kc, *vc, *kw, *vw;   // one layer's K/V cache [Hkv][T_cap][dh] and workspace [Hkv][ws_cap][dh]
  int H, Hkv, dh, T_cap, cache_row0, n_direct, ws_cap;
  int lg_dh;            // log2(dh) (set by the launcher)
};

struct LaGemmArgs {
  const void* X;      // [M][ldx] storage dtype
  const void* W;      // packed weights (la_gemm_pack_launch) of the [rows][K] nn.Linear matrix
  void* Y;            // output [M][ldy]
  const void* R;      // residual [M][ldy] (RESID), may alias Y
  float* P;           // split partials [splits][M][pcols]
  int M, N, K;        // N = output columns (SWIGLU: F)
  int ldx, ldy;
  int splits, nchunks;
  int up_off;         // SWIGLU: first row of the "up" half of W (= F)
  int pcols;          // partial row length (SWIGLU: 2F, else N)
  int swiglu_partial; // set by the launcher
  int defer_reduce;   // RESID with splits > 1: leave the partials for la_addnorm_launch
  LaQkvOut qo;        // QKV epilogue only
};
int la_gemm_splits(int N, int K, int dtype, int swiglu);
int la_gemm_ntw(int N, int swiglu);
size_t la_gemm_packed_elems(int dtype, int N, int K, int swiglu);   // elements of the packed copy of W
// W [rows][K] (SwiGLU: gate rows 0..N-1, up rows N..2N-1) -> packed P; rope_dh > 0 (fp32 only) packs the
// columns of each dh-wide head pair-major (tile k of a head holds dims 8k..8k+7 and dh/2+8k..dh/2+8k+7) for
// LA_EPI_QKV
int la_gemm_pack_launch(int dtype, const void* W, void* P, int N, int K, int swiglu, hipStream_t st, int rope_dh = 0);
int la_gemm_launch(int dtype, int epi, LaGemmArgs a, hipStream_t st);

// row metadata produced by the packed-row builder (device int32 arrays)
struct LaRowsDev {
  int32_t* tok;        // [Q] input token of each packed row
  int32_t* pos;        // [Q] logical position
  int32_t* role;       // [Q] 0 ordinary, 1 lookahead, 2 verify
  int32_t* level;      // [Q] trajectory level (-1 verify)
  int32_t* col;        // [Q] window column (-1 verify)
  int32_t* cand;       // [Q] candidate (-1 otherwise)
  int32_t* off;        // [Q] suffix offset (-1 otherwise)
  int32_t* branch;     // [Q] branch id
  int32_t* path;       // [NB][maxp] workspace row of logical position shared_end + k
  int32_t* path_len;   // [NB]
  int32_t* logit_rows; // [n_logit]: out, inp (column order), guess ((c, s) order)
  uint32_t* mask;      // [Q][mask_words] visibility bits among current rows
  int32_t* tile_meta;  // [ceil(Q/16)][64]: distinct branches of each 16-row tile (count, then ids)
  int32_t* tile_path;  // [ceil(Q/16)][16][64]: their paths (-1: none)
};

struct LaLayout {        // host-side description of one round's rows
  int p;                 // logical position of the ordinary row
  int R;                 // number of trajectory levels
  int sizes[16];         // cells per level (0 = not materialised)
  int starts[16];        // first column of each level (level 0 starts at 1)
  int C, S;              // candidates, suffix length
  int Q, NB, maxp, n_logit, n_inp, n_cols, mask_words;
};
int la_layout_finish(LaLayout* L);   // fills Q, NB, ... ; returns 0 or -1 if inconsistent
// whether the builder's LDS tables hold the round (la_build_rows_launch returns -2 otherwise)
int la_build_rows_fits(const LaLayout& L);
// returns -2 when the round's tables exceed the builder's LDS
int la_build_rows_launch(const LaLayout& L, int x_t, const int32_t* win, int win_stride,
                         const int32_t* cands, LaRowsDev rows, hipStream_t st);

// attention
struct LaAttnArgs {
  const void* q;        // [Q][H][dh]
  const void* kc;       // cache K [Hkv][T_cap][dh] (one layer)
  const void* vc;
  const void* kw;       // workspace K [Hkv][ws_cap][dh] (one layer), packed row k -> ws row k-1
  const void* vw;
  void* o;              // [Q][H][dh]
  float* part_o;        // [splits][H][Q][dh] softmax states of the key splits (several splits only)
  float* part_ml;       // [splits][H][Q][2]  (m, l) of those states
  int max_splits;       // splits part_o / part_ml hold (la_attention_parts(max_pos, T_cap))
  const int32_t* pos;
  const int32_t* branch;
  const int32_t* path;
  const int32_t* path_len;
  const int32_t* tile_meta;   // per 16-row tile: branch count and ids (row builder)
  const int32_t* tile_path;   // per 16-row tile: [16][64] workspace rows of positions shared_end + k
  int Q, H, Hkv, dh, T_cap, ws_cap, maxp;
  int shared_end;       // keys [0, shared_end) come from the cache, later ones from the row's path
  int max_pos;          // largest row position (an upper bound is fine)
  int nb;               // branches in the path table
  int n_ws;             // workspace rows written by this call (packed rows other than the ordinary row)
  float scale;          // softmax scale (1/sqrt(dh))
  // set by the launcher
  int tail0, n_tail;    // first chunk and number of chunks reaching past shared_end
  int ring_end;         // chunks below it are read from the cache through the ring
  int spl;              // chunks per key split (la_attention_spl)
  int nsplit;           // key splits
  int rgroups;          // row groups per KV head
  int wg_head;          // workgroups per KV head (all splits)
  int ring_depth;       // ring slots of one chunk each
  int st_rows, st_half, st_bytes;  // tail stage: rows (committed part of the first tail chunk + packed rows),
                                   // bytes of its K (and of its V) part, bytes with the path table
  float scale_log2;     // scale * log2(e)
};
int la_attention_launch(int dtype, const LaAttnArgs& a, hipStream_t st);
int la_attention_spl(int t_cap, int H, int Hkv); // chunks of 32 positions per key split
int la_attention_parts(int max_pos, int t_cap);   // upper bound on the key splits of a call reaching max_pos
// whether a round of q_max rows (nb_max branches reaching maxp_max positions) fits the tail stage's LDS
int la_attention_fits(int dh, int esz, int q_max, int nb_max, int maxp_max);

// Several requests' attention in one launch (each against its own cache).
// One entry per request: its arguments with layer 0's cache and workspace
// pointers, and the bytes from one layer's K (or V) to the next one's.
struct LaAttnSeg {
  LaAttnArgs a;
  long long kv_layer, ws_layer;
  int blk0, mblk0;      // the request's first attention / merge workgroup (set by the plan)
  int pad[2];
};
struct LaAttnMulti {    // the launch shape every request of the launch shares
  int nw, depth, dh, grid, mgrid;
  size_t lds;
};
// Completes each entry's arguments for one common workgroup shape and ring
// depth (the shape never changes a row's arithmetic); -2 if a request cannot
// run.  Layer-independent: the same plan serves every layer.
int la_attention_multi_plan(int dtype, LaAttnSeg* segs, int n, LaAttnMulti* m);
// segs: the planned entries in device memory
int la_attention_multi_launch(int dtype, const LaAttnMulti& m, const LaAttnSeg* segs, int n, int layer,
                              hipStream_t st);

// model pieces
void la_embed_launch(int dtype, const void* E, const int32_t* tok, void* x, int M, int d, hipStream_t st);
void la_rmsnorm_launch(int dtype, const void* x, const void* w, void* y, const int32_t* rows, int M, int d,
                       float eps, hipStream_t st);
// Residual fold + RMSNorm: x' = T(((P_0 + P_1) + ...) + x) for the split
// partials P_s = P + s * pstride ([M][d] fp32 each; none when S == 0), written
// back to x when write_x; y[m] = RMSNorm(x'[src]) with src = rows ? rows[m] : m.
#define LA_ADDNORM_MAX_SPLITS 8   // partials the fold takes (the GEMM's K split never exceeds it); -2 beyond
int la_addnorm_launch(int dtype, void* x, const float* P, int S, size_t pstride, int write_x, const void* w, void* y,
                      const int32_t* rows, int M, int d, float eps, hipStream_t st);
void la_rope_table_launch(float2* tab, int T, int dh, float theta, hipStream_t st);
// la_qkv_post_launch from the S K-split partials [S][Prows][(H + 2 Hkv) dh] of the projection (fixed-order
// sum, rounded) for its rows 0..M-1 (P may point at a later row of a larger partial buffer)
void la_qkv_reduce_post_launch(int dtype, const float* P, int S, int Prows, int M, const float2* rope,
                               const int32_t* pos, int H, int Hkv, int dh, void* q, void* kc, void* vc, int T_cap,
                               int cache_row0, int n_direct, void* kw, void* vw, int ws_cap, hipStream_t st);
void la_qkv_post_launch(int dtype, const void* qkv, const float2* rope, const int32_t* pos, int M, int H, int Hkv,
                        int dh, void* q, void* kc, void* vc, int T_cap, int cache_row0, int n_direct, void* kw,
                        void* vw, int ws_cap, hipStream_t st);
// Both over the stacked rows of several requests in one launch: entry i
// owns rows r0 .. (next entry's r0) - 1 (entries in row order), q goes to the
// stacked q [M][H][dh], k and v to the request's own cache and workspace of
// the layer (layer 0's pointers + layer * the layer distance in bytes).
struct LaPostSeg {
  const int32_t* pos;   // the request's row positions
  const float2* rope;
  void *kc, *vc, *kw, *vw;
  long long kv_layer, ws_layer;
  int r0, T_cap, cache_row0, n_direct, ws_cap, pad;
};
// S > 0: from the partials P [S][M][(H + 2 Hkv) dh]; S == 0: from the stored qkv [M][(H + 2 Hkv) dh]
void la_qkv_post_multi_launch(int dtype, const float* P, int S, const void* qkv, int M, const LaPostSeg* segs, int n,
                              int layer, int H, int Hkv, int dh, void* q, hipStream_t st);

// verification
void la_argmax_launch(const float* logits, int rows, int V, int32_t* out, hipStream_t st);
struct LaAcceptDev {     // device image of one verification result
  int32_t h, winner, n_emit, pad;
  int32_t emitted[32];
};
// hmax: most candidate tokens accepted (S, or S - 1 when a full match is capped)
void la_greedy_accept_launch(const int32_t* amax, int n_inp, const int32_t* cand, int C, int S, int hmax,
                             LaAcceptDev* acc, int32_t* z, hipStream_t st);
// scratch: V + 256 doubles (the masses of a row, then its block sums)
void la_sample_accept_launch(const float* logits, int V, int n_inp, const int32_t* amax, const int32_t* cand,
                             int C, int S, int hmax, double T, uint64_t seed, int round_id, double* scratch,
                             LaAcceptDev* acc, int32_t* z, hipStream_t st);
void la_sample_row_launch(const float* logits, int V, double T, uint64_t seed, int round_id, const int32_t* amax,
                          double* scratch, int32_t* out, hipStream_t st);

// pool
void la_pool_clear_launch(int32_t* cnt, int V, hipStream_t st);
void la_pool_lookup_launch(const int32_t* cnt, const int32_t* ent, int key, int G, int S, int32_t* out,
                           int32_t* n, hipStream_t st);
void la_pool_upsert_launch(int32_t* cnt, int32_t* ent, const int32_t* keys, const int32_t* sufs, int n, int G,
                           int S, hipStream_t st);
void la_pool_collect_launch(int32_t* cnt, int32_t* ent, int x_t, const int32_t* win, int win_stride, int R,
                            int W, const int32_t* z, int G, hipStream_t st);

// window and commit
// warm: shift > 0 slices every advanced level by shift and refills its tail with fill (ALWAYS_FWD_ONE=False)
void la_window_next_launch(const int32_t* win, int32_t* out, int stride, int R, const int* sizes_old,
                           const int* sizes_new, int deepest, int warm, const int32_t* z, int nz, int shift, int fill,
                           hipStream_t st);
void la_kv_commit_launch(int dtype, void* kc, void* vc, const void* kw, const void* vw, int L, int Hkv, int dh,
                         int T_cap, int ws_cap, int dst_row0, int src_row0, int h, hipStream_t st);
void la_fill_i32_launch(int32_t* p, int n, int v, hipStream_t st);
