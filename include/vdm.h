/*
 * vdm.h -- C ABI of the MI355X (gfx950) vecset SDF decoder library (libvdm.so).
 *
 * What the calls compute follows the FlashVDM pages:
 *   - "Unleashing Vecset Diffusion Model for Fast Shape Generation" (aipaper.cc
 *     summary), section 3: a vecset is an unordered set of latent tokens; the
 *     decoder cross-attends from any query point to the tokens and yields the
 *     SDF there.
 *   - same page, section 4.1 "Lightning Vecset Decoder":
 *       item 1, Hierarchical Volume Decoding (coarse volume, sign-change voxels,
 *       truncated-SDF band for thin parts, one dilation, refine only selected
 *       voxels, repeat to the target resolution);
 *       item 2, Adaptive KV Selection (per sub-volume, probe queries attend to
 *       all tokens, the top-K tokens serve every query of that sub-volume,
 *       queries of different sub-volumes packed together);
 *       item 3, the slim decoder (narrow width, low MLP ratio, no LayerNorm).
 *   - the techwalker article on FlashVDM, parts 2 and 5 (same three pieces;
 *     regions wholly inside/outside keep their label without detailed queries).
 *
 * Decoder (readings of details the pages leave open are listed where they apply):
 *   e(p)  = [x, y, z, sin(f_k x).., sin(f_k y).., sin(f_k z).., cos(..same..)],
 *           f_k = 2^k * pi, k = 0..7; 51 features; the argument is the float32
 *           product f_k * c
 *   q     = Wq e;   k_j = Wk z_j;   v_j = Wv z_j        (no biases)
 *   o_h   = softmax_j(q_h . k_hj / 8) v_hj, heads of 64 columns
 *   a     = Wo o;   y = a + W2 GELU(W1 a) (exact-erf GELU);   net = w_head . y
 *   SDF   = analytic(p) + net_scale * net, analytic = min over primitives of the
 *           sphere / box signed distance.
 *
 * Conventions for every call:
 *   - Tensor pointers are DEVICE pointers owned by the caller, row-major, and
 *     16-byte aligned (xyz and list: 4-byte aligned). The library keeps no
 *     pointer after a call returns.
 *   - Scratch memory is a caller-provided device workspace of at least the size
 *     the matching vdm_*_workspace_size() returns (256-byte aligned). Nothing is
 *     allocated by the library.
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL = the default
 *     stream) and never synchronises it.
 *   - Every call returns a vdm_status and never aborts; on failure,
 *     vdm_last_error() (thread-local) describes it and no kernel was launched
 *     (VDM_ERR_HIP: a launch failed; earlier launches of that call may have run).
 *   - N = 0 queries is a successful no-op.
 *   - Supported decoders: n_freq = 8; dtype BF16 with D = 64 or 256, or F32 with
 *     D = 64; H = D / 64; F a multiple of 256 (BF16, D = 256) or 64 (D = 64),
 *     at most 4096; M >= 1 tokens.
 *   - NaN/Inf in inputs propagate to the affected outputs; a NaN SDF value never
 *     makes a voxel active (every comparison with NaN is false).
 */
#ifndef VDM_H
#define VDM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define VDM_VERSION 1
#define VDM_MAX_PRIMS 16
#define VDM_MAX_LEVELS 6
#define VDM_E_DIM 51

typedef void* vdm_stream; /* hipStream_t */

typedef enum {
  VDM_OK = 0,
  VDM_ERR_INVALID_ARG = -1, /* null pointer, bad size, misalignment, bad parameter */
  VDM_ERR_UNSUPPORTED = -2, /* decoder dims / dtype outside the supported set */
  VDM_ERR_WORKSPACE = -3,   /* workspace missing or smaller than required */
  VDM_ERR_HIP = -4          /* a HIP runtime call or kernel launch failed */
} vdm_status;

typedef enum { VDM_F32 = 0, VDM_BF16 = 1 } vdm_dtype;

typedef enum { VDM_PRIM_SPHERE = 0, VDM_PRIM_BOX = 1 } vdm_prim_kind;

/* One analytic primitive of the SDF prior.
 * SPHERE: size[0] = radius (size[1..2] ignored).  BOX: size = half extents. */
typedef struct {
  int32_t kind;
  float centre[3];
  float size[3];
} vdm_prim;

/* A decoder instance. Weight pointers are device pointers in `dtype`,
 * row-major [out, in]; w_head is float32 [D]. */
typedef struct {
  int32_t D;        /* width = 64 * H */
  int32_t H;        /* attention heads of 64 columns */
  int32_t F;        /* MLP hidden width */
  int32_t n_freq;   /* Fourier frequencies per axis; must be 8 */
  int32_t dtype;    /* vdm_dtype of weights, latents, Q, K and V */
  float net_scale;  /* SDF = analytic + net_scale * net */
  const void* Wq;   /* [D, 51] */
  const void* Wk;   /* [D, D]  */
  const void* Wv;   /* [D, D]  */
  const void* Wo;   /* [D, D]  */
  const void* W1;   /* [F, D]  */
  const void* W2;   /* [D, F]  */
  const float* w_head; /* [D], float32 */
  int32_t n_prims;  /* 1 .. VDM_MAX_PRIMS */
  vdm_prim prims[VDM_MAX_PRIMS];
} vdm_decoder;

/* Where the queries are.
 * Grid point (i, j, k) of an R-cell grid (R + 1 points per axis) over [-1, 1]^3
 * has coordinates c = float32((2i - R) / R) per axis and row-major linear index
 * (i * (R + 1) + j) * (R + 1) + k (x slowest, z fastest). */
typedef enum {
  VDM_Q_POINTS = 0,    /* xyz[N, 3] float32 */
  VDM_Q_GRID = 1,      /* every grid point in linear order; N must be (R + 1)^3 */
  VDM_Q_GRID_LIST = 2  /* list[N] int32 linear grid indices */
} vdm_qmode;

typedef struct {
  int32_t mode;          /* vdm_qmode */
  int32_t R;             /* grid modes: cells per axis, 1 .. 4096 */
  int64_t N;             /* number of queries */
  const float* xyz;      /* VDM_Q_POINTS */
  const int32_t* list;   /* VDM_Q_GRID_LIST */
} vdm_queries;

/* Per-block token sets for decoding with adaptive KV selection.
 * Block b of an R-cell grid groups points whose indices lie in
 * [block*bi, block*bi + block - 1] per axis (clipped to R); blocks are numbered
 * b = (bi * NB + bj) * NB + bk with NB = ceil((R + 1) / block). */
typedef struct {
  int32_t block;            /* block edge in grid points (8) */
  int32_t cap;              /* row stride of sel_idx */
  const int32_t* sel_idx;   /* [rows, cap] ascending token ids (first sel_cnt valid) */
  const int32_t* sel_cnt;   /* [rows], 1 .. cap (0 gives a zero attention output) */
  const int32_t* block_row; /* [NB^3] block id -> row of sel_idx, or NULL (row = block id) */
  int32_t heads;            /* 0: one set per row; 1: per-head sets (vdm_select_kv_heads): head h of
                               row r attends to set r * H + h of sel_idx / sel_cnt */
} vdm_kvsel;

/* Hierarchical decoding parameters. Level L has R0 * 2^L cells per axis. */
typedef struct {
  int32_t R0;        /* coarse cells per axis (75) */
  int32_t levels;    /* 1 .. VDM_MAX_LEVELS (3: 75 -> 150 -> 300) */
  int32_t dilation;  /* 3x3x3 dilations applied to the active cells (1) */
  float tau;         /* band: a tested cell is active if min |SDF| over its corners < tau */
  int32_t use_kvsel; /* 0: full attention; 1: adaptive KV selection at every level */
  int32_t block;     /* KV selection block edge in points (8) */
  int32_t k;         /* tokens kept per probe (64) */
  int32_t cap;       /* token cap per block (512) */
  int32_t probes;    /* 0: corner probes; 1: random probes (see vdm_select_kv), level L seeded with seed + R0 * 2^L */
  uint64_t seed;     /* random probes: SplitMix64 seed */
  int32_t heads;     /* KV selection: 0 = one token set per block; 1 = one per (block, head) */
} vdm_hier_params;

/* Per-level counters written by vdm_decode_hier to a DEVICE array of int64:
 * stats[L * VDM_STAT_FIELDS + field]. */
enum {
  VDM_STAT_R = 0,       /* cells per axis */
  VDM_STAT_TESTED = 1,  /* cells whose 8 corners were all computed */
  VDM_STAT_ACTIVE = 2,  /* tested cells with a sign change or min |s| < tau */
  VDM_STAT_KEPT = 3,    /* cells after dilation (0 on the last level) */
  VDM_STAT_QUERIES = 4, /* points decoded at this level */
  VDM_STAT_BLOCKS = 5,  /* blocks holding at least one query */
  VDM_STAT_ITEMS = 6,   /* decode work items (block, query chunk) */
  VDM_STAT_SELECTED = 7,/* sum over blocks of selected tokens (KV selection) */
  VDM_STAT_FIELDS = 8
};

/* Optional DEVICE outputs of vdm_decode_hier for inspection (NULL = skip).
 * Level L: R = R0 * 2^L, P = R + 1, NB = ceil(P / block). */
typedef struct {
  float* vol[VDM_MAX_LEVELS];       /* [P^3] volume after level L's decode */
  uint8_t* active[VDM_MAX_LEVELS];  /* [R^3] 1 = active cell */
  uint8_t* kept[VDM_MAX_LEVELS];    /* [R^3] 1 = kept after dilation */
  int32_t* list[VDM_MAX_LEVELS];    /* [P^3] level L's query list (blocked order) */
  int32_t* sel_blocks[VDM_MAX_LEVELS]; /* [NB^3] occupied block ids, ascending */
  int32_t* sel_cnt[VDM_MAX_LEVELS];    /* [NB^3] selected tokens per occupied block */
  int32_t* sel_idx[VDM_MAX_LEVELS];    /* [NB^3, cap] selected token ids */
} vdm_hier_debug;

/* ---------------------------------------------------------------- calls */

/* Fused Fourier embedding + query projection (FlashVDM summary section 3; the
 * decoder's first step). Q[n, :] = Wq e(xyz[n]) rounded to `dtype`.
 * xyz: [N, 3] float32. Q: [N, D] in dtype. */
vdm_status vdm_embed_queries(const vdm_decoder* dec, const float* xyz, int64_t N, void* Q,
                             vdm_stream stream);

/* Key/value projection of the vecset, once per shape (section 3: the tokens
 * are projected for cross-attention). K = Z Wk^T, V = Z Wv^T rounded to dtype.
 * Z, K, V: [M, D] in dtype. */
vdm_status vdm_project_kv(const vdm_decoder* dec, const void* Z, int64_t M, void* K, void* V,
                          vdm_stream stream);

/* SDF at N query points (section 3; dense decoding, or with the token subsets of
 * adaptive KV selection, section 4.1 item 2).
 * K, V: [M, D] in dtype (from vdm_project_kv). sdf: [N] float32, sdf[n] for the
 * n-th query. sel: NULL = full attention; otherwise queries must be
 * VDM_Q_GRID_LIST entries sorted by blocked key (block id, then row-major inside
 * the block; as vdm_decode_hier produces) and each query attends to its block's
 * token set. Preconditions with sel: list entries are unique grid points; for
 * every block holding a query, block_row (or the block id) names a row of
 * sel_idx / sel_cnt; sel_cnt of that row lies in 1 .. cap. Outside them the
 * results are defined but not meaningful: an entry outside [0, (R+1)^3) gets
 * sdf = NaN, a repeated entry is decoded once per occurrence, token ids are
 * clamped into [0, M), sel_cnt is clamped into [0, cap], and an empty set
 * (sel_cnt = 0) gives a zero attention output. Workspace:
 * vdm_dense_workspace_size(dec, M, N, sel != NULL), asked with the device that
 * runs the call current: with full attention over M >= 8192 tokens (bf16, D = 256)
 * the tiles of a last round of the decode grid that would be at most half full
 * are split over token ranges (split-KV), and the size includes the partial
 * results of that split, planned for the current device's compute units. The
 * split changes only the fp32 order of the attention sums; results stay the same
 * from run to run. */
vdm_status vdm_decode_dense(const vdm_decoder* dec, const vdm_queries* q, const void* K,
                            const void* V, int64_t M, const vdm_kvsel* sel, float* sdf, void* ws,
                            size_t ws_bytes, vdm_stream stream);

/* Bytes of the device scratch array that vdm_decode_dense_noalloc uses on each
 * GPU (48 MiB): enough for the 1024-wide bf16 decoder up to about 47,000 tokens. */
#define VDM_NOALLOC_SCRATCH_BYTES (48u << 20)

/* For callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): vdm_decode_dense with
 * full attention (sel = NULL) and no workspace argument. The packed K/V, packed
 * epilogue weights and key norms live in a library-owned device array of
 * VDM_NOALLOC_SCRATCH_BYTES per GPU, held until the process ends; the call
 * allocates nothing. It needs vdm_dense_workspace_size(dec, M, N, 0) bytes of
 * that array and returns VDM_ERR_WORKSPACE (launching nothing) when that exceeds
 * VDM_NOALLOC_SCRATCH_BYTES. Results equal vdm_decode_dense's bit for bit. Every
 * call on one GPU shares that GPU's array (the key norms are cleared on each
 * call; the rest is overwritten): calls that overlap on one GPU, on different
 * streams or host threads, race and must be ordered by the caller. The first
 * call on a device looks up the array's address on that device. */
vdm_status vdm_decode_dense_noalloc(const vdm_decoder* dec, const vdm_queries* q, const void* K,
                                    const void* V, int64_t M, float* sdf, vdm_stream stream);

/* Dense decoding of a batch of B vecsets (shapes) at the same N query points:
 * one decode launch for the whole batch (the packing of each shape's K/V is one
 * launch per shape). K, V: [B, M, D] in dtype, shape b at byte offset
 * b * M * D * element size (which must keep 16-byte alignment); sdf: [B, N]
 * float32. Shape b's results equal, bit for bit, those of vdm_decode_dense on
 * that shape alone. No token selection. Requires 1 <= B <= 4096. Workspace:
 * vdm_dense_batch_workspace_size(dec, B, M). */
vdm_status vdm_decode_dense_batch(const vdm_decoder* dec, const vdm_queries* q, int32_t B,
                                  const void* K, const void* V, int64_t M, float* sdf, void* ws,
                                  size_t ws_bytes, vdm_stream stream);

/* Adaptive KV selection (section 4.1 item 2) for blocks of an R-cell grid.
 * For each listed block 8 probe points: probes = 0, its 8 corners (indices
 * block*b and min(block*b + block - 1, R) per axis); probes = 1, 8 random grid
 * points of the block, as the pages sample them: probe n of block id b takes
 * along axis a (0 = x) the index lo_a + (u mod e_a), where lo_a is the block's
 * first index, e_a its number of points along a, and u the c-th output (counted
 * from 0, c = (8 b + n) * 3 + a) of the SplitMix64 stream seeded with `seed`
 * (Steele, Lea and Flood 2014: state += 0x9E3779B97F4A7C15, then the mix of
 * Vigna's reference splitmix64.c). A token's score for a probe
 * is the head-mean softmax probability; each probe keeps its top-k tokens (equal
 * scores: lower index first); the block keeps their union, reduced to the `cap`
 * tokens of largest max-over-probes score when larger (ties: lower index).
 * Output row r (for blocks[r], or block r when blocks == NULL and
 * nblk = NB^3): sel_idx[r, 0 .. sel_cnt[r]) ascending, rest -1.
 * Requires 1 <= k <= M, k <= cap and M <= 65536 (VDM_ERR_UNSUPPORTED beyond).
 * Rows of more than 4096 tokens are searched in 4096-token chunks, which keep
 * up to 1024 candidates per probe and 1024 union members per block, so there
 * k * ceil(M / 4096) <= 1024 and, unless cap >= 8 k, 8 k <= 1024 (else
 * VDM_ERR_UNSUPPORTED); the result is the same top-k. Workspace:
 * vdm_select_workspace_size(dec, M): 32 score rows of M floats for each of up
 * to 256 workgroups (1 GiB at M = 32768), plus a packed copy of K. */
vdm_status vdm_select_kv(const vdm_decoder* dec, int32_t R, int32_t block, int32_t k, int32_t cap,
                         int32_t probes, uint64_t seed, const void* K, int64_t M,
                         const int32_t* blocks, int64_t nblk, int32_t* sel_idx, int32_t* sel_cnt,
                         void* ws, size_t ws_bytes, vdm_stream stream);

/* Adaptive KV selection with one token set per (block, head): the alternative
 * reading of the multi-head score in section 4.1 item 2. Head h ranks the tokens
 * by its own softmax probability (not the head mean); each head keeps its own
 * union of the probes' top-k and its own cap (by the head's max-over-probes
 * probability). Arguments and limits as vdm_select_kv, except M <= 16384 (the
 * workspace holds H score rows per probe); output rows are [nblk][H]: set h of
 * block row r is sel_idx[(r * H + h) * cap ..], sel_cnt[r * H + h]. Workspace:
 * vdm_select_heads_workspace_size(dec, M). Decode with a vdm_kvsel whose heads = 1. */
vdm_status vdm_select_kv_heads(const vdm_decoder* dec, int32_t R, int32_t block, int32_t k, int32_t cap,
                               int32_t probes, uint64_t seed, const void* K, int64_t M,
                               const int32_t* blocks, int64_t nblk, int32_t* sel_idx, int32_t* sel_cnt,
                               void* ws, size_t ws_bytes, vdm_stream stream);

/* Hierarchical volume decoding (section 4.1 item 1), optionally with adaptive KV
 * selection at every level (item 2). Writes the final (R0*2^(levels-1) + 1)^3
 * float32 volume `vol` (vol_elems must be at least that), per-level counters to
 * the device array `stats` ([levels * VDM_STAT_FIELDS] int64, may be NULL) and
 * the optional inspection outputs `dbg` (may be NULL).
 * Level 0 decodes every point. At each level, tested cells are active when their
 * corner SDFs include both s < 0 and s >= 0 or min |s| < tau; active cells are
 * dilated `dilation` times with the 3x3x3 stencil; every corner of every child of
 * a kept cell that was not decoded before is decoded at the next level; every
 * other point takes its nearest ancestor's value (the point (i/2, j/2, k/2) of the
 * previous level, integer division). No host synchronisation. Workspace:
 * vdm_hier_workspace_size(dec, params, M). */
vdm_status vdm_decode_hier(const vdm_decoder* dec, const vdm_hier_params* params, const void* K,
                           const void* V, int64_t M, float* vol, int64_t vol_elems,
                           int64_t* stats, const vdm_hier_debug* dbg, void* ws, size_t ws_bytes,
                           vdm_stream stream);

/* Hierarchical decoding of a batch of B vecsets (shapes) with the same params:
 * shape b runs the level loop of vdm_decode_hier on K, V at byte offset
 * b * M * D * element size (which must keep 16-byte alignment), writes
 * vol + b * (R+1)^3 (R the finest grid; vol_elems covers all B volumes) and, when
 * stats is not NULL, stats + b * levels * VDM_STAT_FIELDS, with workspace slice b
 * of vdm_hier_batch_workspace_size(dec, params, B, M) / B bytes. Every mask stage
 * of a level (cell test, dilation, marking, scans, list emission, fill) is one
 * launch for all B shapes, and so are each level's KV selection and decode: their
 * groups of blocks, tiles or work items run shape after shape in one persistent
 * launch, found from a device-side prefix of the shapes' counts (no host sync). Shape b's volume and counters equal, bit for bit, those of
 * vdm_decode_hier on that shape alone. No inspection outputs. Requires
 * 1 <= B <= 4096. */
vdm_status vdm_decode_hier_batch(const vdm_decoder* dec, const vdm_hier_params* params, int32_t B,
                                 const void* K, const void* V, int64_t M, float* vol, int64_t vol_elems,
                                 int64_t* stats, void* ws, size_t ws_bytes, vdm_stream stream);

/* Surface extraction: the stage that follows VAE decoding in a vecset diffusion
 * pipeline (techwalker article on FlashVDM, part 1, the four stages). The pages
 * leave the method open; it is read here as marching cubes at SDF = 0 on the
 * decoded grid.
 * vol: [(R+1)^3] float32 values at the grid points x_i = -1 + 2 i / R, row-major
 * (x slowest), as vdm_decode_hier writes them. cell_mask: optional [R^3] uint8,
 * row-major cells (cell (i,j,k) has corners i..i+1, j..j+1, k..k+1); nonzero =
 * extract the cell; NULL = every cell.
 * - A point is inside when its value is < 0 (0 and NaN are outside).
 * - Every grid edge whose end points differ in that test and that belongs to an
 *   extracted cell carries one vertex, at the zero of the linear interpolant
 *   along the edge (t = v0 / (v0 - v1) from the lower end point). Vertices are
 *   numbered by ascending edge id a * (R+1)^3 + point index (a = 0, 1, 2 for
 *   edges along x, y, z; point index = (i * (R+1) + j) * (R+1) + k).
 * - A cell's surface is built face by face: a face with two crossing edges gets
 *   one segment between them, a face with four (inside corners on a diagonal)
 *   gets two segments that each cut off one inside corner. Segments are directed
 *   so that the normal points from inside corners to outside ones, and chain
 *   into loops. Each loop is split into a fan around the loop vertex of smallest
 *   edge id among those that share no cube face with a loop vertex other than
 *   their two loop neighbours; loops of a cell in order of their smallest edge
 *   id; cells in row-major order.
 * - Triangle normals (right-hand rule) point towards positive values; the mesh
 *   is closed wherever the surface does not reach the volume's boundary or the
 *   edge of the cell mask.
 * Outputs (device): verts [max_verts][3] float32 world coordinates; tris
 * [max_tris][3] int32 vertex ids; vert_edges [max_verts] int64 edge ids (may be
 * NULL); counts [2] int64 = vertices and triangles of the whole mesh. Entries
 * past max_verts / max_tris are not written: compare counts with the maxima
 * once the stream has run (verts / tris may be NULL when their maximum is 0).
 * Requires 1 <= R <= 893 (vertex ids fit int32). Workspace:
 * vdm_surface_workspace_size(R). */
vdm_status vdm_extract_surface(const float* vol, int32_t R, const uint8_t* cell_mask, float* verts,
                               int64_t max_verts, int32_t* tris, int64_t max_tris, int64_t* vert_edges,
                               int64_t* counts, void* ws, size_t ws_bytes, vdm_stream stream);

/* ---------------------------------------------------------------- helpers */

/* ---------------------------------------------------------------- local KNN decoder */

/* A local (K-nearest-neighbour) decoder: the AVS-Conv operator of the MSVS-VAE
 * page (kwkr.cn), section 1.1, followed by the slim head of the vecset decoder.
 * For a query x, its K nearest supports j (support positions p_j, features f_j)
 * give offsets delta_j = p_j - x, dynamic weights w_j = B GELU(A delta_j + a)
 * (one per feature channel, exact-erf GELU) and the fused feature
 *   h = (1/K) sum_j w_j * f_j + (1/K) sum_j f_j    (weighted mean + mean-pool residual);
 * then y = h + W2 GELU(W1 h), net = w_head . y, SDF = analytic(x) + net_scale * net.
 * Neighbours: the K supports of smallest float32 squared distance
 * fl(fl(fl(dx*dx) + fl(dy*dy)) + fl(dz*dz)), dx = fl(p_jx - x_x) etc. (no fused
 * multiply-add), equal distances to the lower support index.
 * Supported: C = 256, K = 16, hidden = 32, bf16 features and B, W1, W2;
 * F a multiple of 256 up to 4096. Device pointers, row-major [out, in]. */
typedef struct {
  int32_t C;           /* feature width */
  int32_t F;           /* head MLP width */
  int32_t K;           /* neighbours per query */
  int32_t hidden;      /* width of the offset MLP */
  float net_scale;     /* SDF = analytic + net_scale * net */
  const float* A;      /* [hidden, 3] float32 */
  const float* a;      /* [hidden] float32 */
  const void* B;       /* [C, hidden] bf16 */
  const void* W1;      /* [F, C] bf16 */
  const void* W2;      /* [C, F] bf16 */
  const float* w_head; /* [C] float32 */
  int32_t n_prims;     /* 1 .. VDM_MAX_PRIMS */
  vdm_prim prims[VDM_MAX_PRIMS];
} vdm_local_decoder;

/* SDF of the local decoder at N query points (MSVS-VAE page section 1.1; the
 * 200K-query batch of its section 3.3). sup_xyz: [M, 3] float32 support
 * positions; feats: [M, C] bf16 support features; xyz: [N, 3] float32 queries;
 * sdf: [N] float32. nbr: optional [N, K] int32 output, each query's neighbours
 * nearest first (NULL: not written). The supports are bucketed into a 32^3 grid
 * of cells over [-1, 1]^3 (positions outside are bucketed into the border cells
 * and still found). A query with a NaN coordinate has no neighbours (its nbr
 * entries are 2^31 - 1) and a NaN SDF. Requires K <= M. Workspace:
 * vdm_local_workspace_size(dec, M, N). */
vdm_status vdm_decode_local(const vdm_local_decoder* dec, const float* sup_xyz, const void* feats, int64_t M,
                            const float* xyz, int64_t N, float* sdf, int32_t* nbr, void* ws, size_t ws_bytes,
                            vdm_stream stream);

/* Workspace bytes for the calls above (0 with vdm_last_error set on bad args). */
size_t vdm_dense_workspace_size(const vdm_decoder* dec, int64_t M, int64_t N, int32_t with_sel);
size_t vdm_select_workspace_size(const vdm_decoder* dec, int64_t M);
size_t vdm_select_heads_workspace_size(const vdm_decoder* dec, int64_t M);
size_t vdm_hier_workspace_size(const vdm_decoder* dec, const vdm_hier_params* params, int64_t M);
size_t vdm_surface_workspace_size(int32_t R);
size_t vdm_dense_batch_workspace_size(const vdm_decoder* dec, int32_t B, int64_t M);
size_t vdm_hier_batch_workspace_size(const vdm_decoder* dec, const vdm_hier_params* params, int32_t B,
                                     int64_t M);
size_t vdm_local_workspace_size(const vdm_local_decoder* dec, int64_t M, int64_t N);

/* ---------------------------------------------------------------- kernel timing */

/* Kinds of launches the library can time. */
enum {
  VDM_TIME_DECODE = 0,      /* fused decode over the whole token set (dense, hierarchical levels) */
  VDM_TIME_DECODE_GATHERED, /* fused decode over per-block token sets (adaptive KV selection) */
  VDM_TIME_SELECT,          /* probe scoring, top-k and union (vdm_select_kv, hierarchical levels) */
  VDM_TIME_EMBED,           /* vdm_embed_queries */
  VDM_TIME_PROJECT_KV,      /* vdm_project_kv */
  /* per-level bookkeeping of vdm_decode_hier: */
  VDM_TIME_CELL_TEST,       /* sign-change / band test of the tested cells */
  VDM_TIME_DILATE,          /* 3x3x3 dilation of the active cells */
  VDM_TIME_MARK,            /* candidate points of the next level, minus computed ones */
  VDM_TIME_SCAN,            /* prefix sums of per-block counts (three launches per level) */
  VDM_TIME_EMIT,            /* query list, work items and occupied blocks */
  VDM_TIME_FILL,            /* nearest-ancestor fill of the next level's volume */
  VDM_TIME_SURFACE,         /* vdm_extract_surface (all of its launches) */
  /* vdm_decode_local: */
  VDM_TIME_LOCAL_GRID,      /* bucketing of the supports into cells (count, scan, scatter) */
  VDM_TIME_LOCAL_KNN,       /* K nearest supports of every query */
  VDM_TIME_LOCAL_FUSE,      /* offset MLP, dynamic weights, weighted sum and mean residual */
  VDM_TIME_LOCAL_HEAD,      /* head MLP, SDF */
  VDM_TIME_KINDS
};

/* Launch timing with HIP events: while on, every launch of the kinds above is
 * bracketed by two events recorded on the call's stream (host-side state shared
 * by all threads; nothing is synchronised when recording).
 * mode: 1 = on, 0 = off (records kept), 2 = drop all records (state unchanged).
 * vdm_timing_read waits for the recorded events of one kind and returns how many
 * launches were recorded and their summed durations in milliseconds. */
vdm_status vdm_timing(int32_t mode);
vdm_status vdm_timing_read(int32_t kind, int64_t* launches, double* total_ms);

/* VDM_VERSION of the built library. */
int32_t vdm_version(void);

/* The current HIP device's compute units and peak shader clock in kHz, as the
 * runtime reports them (the figures the bf16 MFMA peak is quoted at). Either
 * pointer may be NULL. VDM_ERR_HIP when the runtime has no device. */
vdm_status vdm_device_info(int32_t* compute_units, int32_t* peak_clock_khz);

/* Description of the last failure on the calling thread ("" if none). */
const char* vdm_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* VDM_H */
