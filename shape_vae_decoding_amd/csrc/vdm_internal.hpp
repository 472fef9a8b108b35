// Internal argument structs shared by the host API layer and the kernels, and
// the host-side launchers each kernel file provides.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/vdm.h"

namespace vdm {

// ------------------------------------------------------------------ bounds-checked builds
// Built with -DVDM_DEBUG=1, the kernels check every data-dependent index
// (token ids, selection rows, work items, block ids, list and item slots,
// support indices) with VDM_BOUND(cond, id): a false condition records `id` in
// its source file's debug word (the first failure is kept) and the guarded
// access is skipped or clamped. Every entry point of such a build synchronises
// its stream, reads and clears the words, and fails with VDM_ERR_HIP naming the
// check. Release builds compile VDM_BOUND to `true`.
#ifndef VDM_DEBUG
#define VDM_DEBUG 0
#endif

enum BoundCheck : unsigned {
  BC_DECODE_ITEM = 1,  // a work item's queries [q0, q1): 0 <= q0 <= q1 <= N, at most one tile
  BC_DECODE_ROW,       // a work item's selection row >= 0
  BC_DECODE_SET,       // a selection row's count within [0, cap]
  BC_DECODE_TOKEN,     // a selected token id within [0, M)
  BC_LIST_ROW,         // a block's selection row (block_row) >= 0
  BC_SELECT_BLOCK,     // a block id of the selection within [0, NB^3)
  BC_SELECT_OUT,       // a compacted token set within its cap
  BC_EMIT_LIST,        // a list slot within the list's capacity
  BC_EMIT_ITEM,        // a work-item slot within the item array's capacity
  BC_SCAN_OCC,         // an occupied-block slot within the block count
  BC_LOCAL_SCATTER,    // a support's slot in cell order within [0, M)
  BC_LOCAL_RANGE,      // a cell's support range within [0, M]
  BC_LOCAL_QUERY,      // a query index in cell order within [0, N)
  BC_SELECT_CAND,      // a chunk winner's slot within a wave's candidate list
  BC_CHECKS
};

#if VDM_DEBUG
// one per source file (static): each file reads its own with debug_take_word
static __device__ unsigned debug_word;
__device__ __forceinline__ bool bound_ok(bool ok, unsigned id) {
  if (!ok) atomicCAS(&debug_word, 0u, id);
  return ok;
}
#define VDM_BOUND(cond, id) ::vdm::bound_ok((cond), (id))
// this file's debug word, cleared; defines the file's reader `fn`
#define VDM_DEBUG_READER(fn)                                                        \
  hipError_t fn(unsigned* w) {                                                      \
    hipError_t e = hipMemcpyFromSymbol(w, HIP_SYMBOL(debug_word), sizeof(unsigned)); \
    if (e != hipSuccess) return e;                                                  \
    const unsigned z = 0;                                                           \
    return hipMemcpyToSymbol(HIP_SYMBOL(debug_word), &z, sizeof(unsigned));         \
  }
#else
#define VDM_BOUND(cond, id) true
#define VDM_DEBUG_READER(fn) \
  hipError_t fn(unsigned* w) {   \
    *w = 0;                      \
    return hipSuccess;           \
  }
#endif
// the readers of the kernel files
hipError_t debug_take_decode(unsigned* w);
hipError_t debug_take_select(unsigned* w);
hipError_t debug_take_hvd(unsigned* w);
hipError_t debug_take_local(unsigned* w);
hipError_t debug_take_prep(unsigned* w);
hipError_t debug_take_surface(unsigned* w);

struct PrimDev {
  int kind;
  float c[3];
  float s[3];
};

struct PrimSet {
  int n;
  PrimDev p[VDM_MAX_PRIMS];
};

// Where a tile's queries come from.
//   mode 0: xyz[3q..3q+2]; 1: grid point with linear index q; 2: grid point list[q];
//   3: corner probe q % 8 of block q / 8 (block id list[q / 8], or q / 8 when list
//      is null) of an R-cell grid split into blocks of `block` points per axis.
struct QuerySrc {
  int mode;
  int R;
  const float* xyz;
  const int32_t* list;
  int block;
  int probes = 0;          // mode 3: 0 = corner probes, 1 = random probes (SplitMix64 stream of `seed`)
  unsigned long long seed = 0;
};

// A decode work item: queries [q0, q1) of the query source, attending to token
// row `row` of the selection (gathered mode) or to every token (row < 0).
struct Item {
  int32_t q0, q1, row, pad;
};

struct DecodeArgs {
  QuerySrc qs;
  int64_t N;            // number of queries (dense tiles)
  const void* Wq;       // [D][51]
  const void* Kp;       // dense: packed K tiles [Mpad/32][H][chunk][64 lanes][16 B]; gathered: K [M][D]
  const void* Vt;       // dense: packed V^T tiles [Mpad/32][H][chunk][64 lanes][16 B]; gathered: V [M][D]
  const float* kmax;    // [H] max over tokens of ||k_h|| (softmax shift bound)
  int M;                // tokens (dense)
  // bf16: fragment-packed copies (launch_pack_w); fp32: the row-major weights
  const void* Wo;
  const void* W1;
  const void* W2;
  const float* w_head;
  int F;
  float net_scale;
  PrimSet prims;
  float* out;           // sdf
  int scatter;          // 1: out[linear grid index] (grid modes), 0: out[q]
  // tiles: items == null -> tiles of BQ consecutive queries of N (or *d_N) queries;
  //        items != null -> n_tiles (or *d_n_items) work items
  const int32_t* d_N;       // device query count, or null (use N)
  int64_t n_tiles;          // host item count
  const int32_t* d_n_items; // device item count, or null (use n_tiles)
  const Item* items;
  // gathered
  const int32_t* sel_idx;
  const int32_t* sel_cnt;
  int cap;
  int heads;  // gathered: 1 = per-head sets (row r's set for head h is selection row r * H + h)
  // dense batch of vecsets (0 or 1: one): tile t belongs to shape t / tiles-per-shape,
  // whose packed K/V start kv_stride bytes after the previous shape's, kmax at
  // [shape][H], and outputs at out + shape * out_stride
  int batch;
  int64_t kv_stride;
  int64_t out_stride;
  // ragged batch (batch > 1 and tile_prefix set): shape b has its own device count,
  // *(d_N + b * cnt_stride) queries (dense tiles of BQ) or *(d_n_items + b *
  // cnt_stride) work items; tile_prefix[b] = the tiles or items of shapes before b
  // (tile_prefix[batch] = all of them). Shape b's query list is at qs.list +
  // b * list_stride bytes, its items at items + b * items_stride bytes, its
  // selection at sel_idx and sel_cnt + b * sel_stride bytes (each), its key norms at
  // kmax + b * kmax_stride floats; K/V and outputs use kv_stride and out_stride.
  const int64_t* tile_prefix = nullptr;
  int64_t cnt_stride = 0;
  int64_t list_stride = 0;
  int64_t items_stride = 0;
  int64_t sel_stride = 0;
  int64_t kmax_stride = 0;
  // dense split of the tail (decode_split_plan): the last split_tiles tiles are each
  // cut into `split` ranges of token tiles, one work unit per range; each unit
  // writes its partial O and row sums to part, and the unit that arrives last at a
  // tile (part_cnt, zeroed before the launch) adds them in range order and runs the
  // epilogue. split = 1: no split.
  int split = 1;
  int64_t split_tiles = 0;
  float* part = nullptr;
  int32_t* part_cnt = nullptr;
  // a counter, zero before the launch, from which workgroups take their work units
  // in order (required in gathered mode; null: dense units go round-robin)
  unsigned long long* queue = nullptr;
};

// The tail split of a dense full-attention launch of n_tiles tiles over M tokens:
// when the last round of the persistent grid would be at most half full and the
// token set is long (M >= 8192), the leftover tiles are split into `parts` token
// ranges (of at least 512 tokens) so that the last round is filled. parts = 1: no
// split. part_bytes / cnt_bytes: the scratch the split needs.
struct SplitPlan {
  int parts = 1;
  int64_t tiles = 0;
  size_t part_bytes = 0, cnt_bytes = 0;
};
SplitPlan decode_split_plan(int dtype, int D, int64_t M, int64_t n_tiles);

struct DevInfo {
  int cus;
  int max_lds;
};

DevInfo dev_info();

// ------------------------------------------------------------------ launchers
// Each returns hipSuccess or the launch error.

// K, V [M][D] -> per-(32-token tile, head) operand runs of 64 lanes x 32 elements,
// stored chunk-major (see k_prep.hip); V and Vt may be null (K only)
// B shapes: K/V at byte stride in_stride, Kp/Vt at out_stride (one launch)
hipError_t launch_pack_kv(int dtype, const void* K, const void* V, int M, int D, int Mpad, void* Kp,
                          void* Vt, hipStream_t s, int B = 1, int64_t in_stride = 0, int64_t out_stride = 0);
// bf16 W [rows][cols] -> MFMA A-operand fragments: block (rb, ks) of 32 rows x 16
// columns is 64 lanes x 8 elements, lane l holding W[32rb + l%32][16ks + 8(l/32) + 0..7];
// blocks in (rb, ks) order. rows % 32 == 0, cols % 16 == 0.
hipError_t launch_pack_w(const void* W, int rows, int cols, void* Wp, hipStream_t s);
// kmax[h] = max_m ||K[m][64h .. 64h+63]||_2 (kmax must be zeroed first)
// B shapes: K at byte stride k_stride, kmax at kmax_stride (one launch)
hipError_t launch_key_norms(int dtype, const void* K, int M, int H, float* kmax, hipStream_t s, int B = 1,
                            int64_t k_stride = 0, int64_t kmax_stride = 0);
// K = Z Wk^T, V = Z Wv^T
hipError_t launch_project_kv(int dtype, const void* Z, const void* Wk, const void* Wv, int M, int D,
                             void* K, void* V, hipStream_t s);
// Q [N][D] = Wq e(xyz)
hipError_t launch_embed(int dtype, int D, const QuerySrc& qs, int64_t N, const void* Wq, void* Q,
                        hipStream_t s);
// the decoder over tiles (dense) or items (list/gathered)
hipError_t launch_decode(int dtype, int D, bool gathered, const DecodeArgs& a, hipStream_t s);
int decode_tile_queries(int dtype, int D);
int decode_f_chunk(int dtype, int D);

// KV selection for blocks; blocks == null: block id = row. n_blocks from host or *d_n_blocks.
struct SelectArgs {
  int R, block, k, cap, M, H, D;
  int probes;          // 0: the 8 corners of a block; 1: 8 random points (SplitMix64 stream of seed)
  unsigned long long seed;
  const void* Wq;  // [D][51]
  const void* K;   // [M][D]
  const void* Kp;  // bf16: K packed like the dense decoder's tiles (launch_pack_kv), else unused
  const int32_t* blocks;
  int64_t n_blocks;
  const int32_t* d_n_blocks;
  int32_t* sel_idx;
  int32_t* sel_cnt;
  int64_t* stat_selected;  // optional: += sum of sel_cnt
  float* scores;           // scratch of select_scratch_bytes(M, per_head ? H : 1)
  int per_head;            // 1: one set per (block, head), rows [block][H]; 0: one per block
  // ragged batch (batch > 1): shape b has *(d_n_blocks + b * cnt_stride) blocks;
  // grp_prefix[b] = the groups of SEL_GB blocks of shapes before b (grp_prefix[batch]
  // = all). Shape b's block list, K, packed K, selection (sel_idx and sel_cnt each)
  // and counter are at byte offsets b * blocks_stride, b * k_stride, b * kp_stride,
  // b * sel_stride and b * stat_stride; the score scratch is per workgroup.
  int batch = 1;
  const int64_t* grp_prefix = nullptr;
  int64_t cnt_stride = 0, blocks_stride = 0, k_stride = 0, kp_stride = 0, sel_stride = 0, stat_stride = 0;
};
hipError_t launch_select(int dtype, const SelectArgs& a, hipStream_t s);
int select_blocks_per_group();  // blocks one workgroup of the selection takes at a time
size_t select_scratch_bytes(int M, int sets);
// largest token count of a selection; whether (M, k, cap) fits the kernel's lists
int select_max_tokens(bool per_head);
bool select_fits(int64_t M, int k, int cap, bool per_head);

// ------------------------------------------------------------------ local KNN decoder
// Supports are bucketed into LOCAL_G^3 cells over [-1, 1]^3.
constexpr int LOCAL_G = 32;
constexpr int LOCAL_K = 16;
constexpr int LOCAL_HIDDEN = 32;
constexpr int LOCAL_C = 256;

// Bucketing of n points into the cells: counts (zeroed by the caller), starts
// [LOCAL_G^3 + 1], fill (zeroed), cell_of [n]; then, in cell order, spos (x, y, z,
// index bits) and/or order (index) when not null; occ [LOCAL_G^2] occupancy words
// (bit k of word i * LOCAL_G + j: cell (i, j, k) holds a point) when not null.
hipError_t launch_local_grid(const float* xyz, int64_t n, int32_t* counts, int32_t* starts, int32_t* fill,
                             int32_t* cell_of, float4* spos, int32_t* order, uint32_t* occ, hipStream_t s);
// nbr [N][LOCAL_K]: each query's nearest supports, nearest first; queries taken
// in the given order (a permutation of 0 .. N-1)
hipError_t launch_local_knn(const float* xyz, int64_t N, const int32_t* order, const int32_t* starts,
                            const uint32_t* occ, const float4* spos, int32_t* nbr, hipStream_t s);

struct LocalFuseArgs {
  const float* sup_xyz;   // [M][3]
  const void* feats;      // [M][C] bf16
  int M;
  const float* xyz;       // [N][3]
  int64_t N;
  const int32_t* nbr;     // [N][K]
  const float* A;         // [hidden][3]
  const float* a;         // [hidden]
  const void* B;          // [C][hidden] bf16
  void* h;                // [N][C] bf16 out
};
hipError_t launch_local_fuse(const LocalFuseArgs& a, hipStream_t s);

// y = h + W2 GELU(W1 h), net = w_head . y, out[q] = analytic(x_q) + net_scale net
struct HeadArgs {
  const float* xyz;    // [N][3]
  int64_t N;
  const void* h;       // [N][256] bf16
  const void* W1;      // fragment-packed (launch_pack_w)
  const void* W2;      // fragment-packed
  const float* w_head; // [256]
  int F;
  float net_scale;
  PrimSet prims;
  float* out;
};
hipError_t launch_local_head(const HeadArgs& a, hipStream_t s);

// Surface extraction (marching cubes at SDF = 0) workspace: crossing-edge bit
// planes, inside bits, per-word vertex prefixes, per-piece triangle counts and
// their prefixes, per-block partial sums.
struct SurfaceWs {
  int64_t nwa;     // 64-bit words per plane (one per piece of 63 points of a row)
  int64_t nwords;  // 3 * nwa
  int64_t nwb;     // blocks of the word scan
  int64_t ncb;     // blocks of the triangle-count scan
  size_t off_words, off_ins, off_prefix, off_tcnt, off_tpre, off_wpart, off_cpart, bytes;
};
SurfaceWs surface_ws_layout(int R);
// counts[0] = vertices, counts[1] = triangles (device); entries past the maxima are not written
hipError_t launch_surface(const float* vol, int R, const uint8_t* mask, float* verts, int64_t max_verts,
                          int32_t* tris, int64_t max_tris, int64_t* vert_edges, int64_t* counts, char* ws,
                          hipStream_t s);

}  // namespace vdm
