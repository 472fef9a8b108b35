// Internal argument structs shared by the host API layer and the kernels, and
// the host-side launchers each kernel file provides.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/vdm.h"

namespace vdm {

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
  // dense batch of vecsets (0 or 1: one): tile t belongs to shape t / tiles-per-shape,
  // whose packed K/V start kv_stride bytes after the previous shape's, kmax at
  // [shape][H], and outputs at out + shape * out_stride
  int batch;
  int64_t kv_stride;
  int64_t out_stride;
};

struct DevInfo {
  int cus;
  int max_lds;
};

DevInfo dev_info();

// ------------------------------------------------------------------ launchers
// Each returns hipSuccess or the launch error.

// K, V [M][D] -> per-(32-token tile, head) operand runs of 64 lanes x 32 elements,
// stored chunk-major (see k_prep.hip); V and Vt may be null (K only)
hipError_t launch_pack_kv(int dtype, const void* K, const void* V, int M, int D, int Mpad, void* Kp,
                          void* Vt, hipStream_t s);
// bf16 W [rows][cols] -> MFMA A-operand fragments: block (rb, ks) of 32 rows x 16
// columns is 64 lanes x 8 elements, lane l holding W[32rb + l%32][16ks + 8(l/32) + 0..7];
// blocks in (rb, ks) order. rows % 32 == 0, cols % 16 == 0.
hipError_t launch_pack_w(const void* W, int rows, int cols, void* Wp, hipStream_t s);
// kmax[h] = max_m ||K[m][64h .. 64h+63]||_2 (kmax must be zeroed first)
hipError_t launch_key_norms(int dtype, const void* K, int M, int H, float* kmax, hipStream_t s);
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
  float* scores;           // scratch of select_scratch_bytes(M)
};
hipError_t launch_select(int dtype, const SelectArgs& a, hipStream_t s);
size_t select_scratch_bytes(int M);

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
