// Launchers of the hierarchical-decoding mask stages (k_hvd.hip).
#pragma once

#include "vdm_internal.hpp"

namespace vdm {

__host__ __device__ inline int nblocks8(int P) { return (P + 7) / 8; }
// 64-bit words of a blocked bit mask for P points (or cells) per axis
inline int64_t mask_words(int P) {
  const int64_t NB = nblocks8(P);
  return NB * NB * NB * 8;
}

// A device pointer of a batch of B shapes: shape b's copy starts `stride` bytes
// after shape b-1's (stride 0: one shared copy, or B = 1). Kernels launched with
// gridDim.y = B take shape blockIdx.y's pointer with at().
template <typename T>
struct BP {
  T* p;
  int64_t stride;
  __device__ __forceinline__ T* at() const {
    return reinterpret_cast<T*>(reinterpret_cast<char*>(const_cast<void*>(static_cast<const void*>(p))) +
                                (int64_t)blockIdx.y * stride);
  }
};
template <typename T>
inline BP<T> bp(T* p, int64_t stride = 0) {
  return BP<T>{p, stride};
}

hipError_t launch_zero(void* p, size_t bytes, hipStream_t s);
// B copies, stride bytes apart
hipError_t launch_zero_b(BP<void> p, size_t bytes, int B, hipStream_t s);
// Every launcher below runs B shapes at once (gridDim.y = B), each on its own
// copies of the buffers (BP strides).
hipError_t launch_stats_init(BP<int64_t> stats, int levels, int R0, int B, hipStream_t s);
// part: stat_part_words() zero-initialised partial counters (left zero on return)
inline int64_t stat_part_words() { return 256 * 8; }
hipError_t launch_cell_test(BP<const float> vol, int R, BP<const uint64_t> kept_prev, float tau, BP<uint64_t> active,
                            BP<int64_t> part, BP<int64_t> stat_tested, BP<int64_t> stat_active, int B, hipStream_t s);
// identity = 1: copy (and count) without dilating; stat.p may be null (no count)
hipError_t launch_dilate(BP<const uint64_t> in, BP<uint64_t> out, int R, int identity, BP<int64_t> part,
                         BP<int64_t> stat, int B, hipStream_t s);
hipError_t launch_mark(BP<const uint64_t> kept, int R, BP<const uint64_t> comp_prev, int all_new, int Rn,
                       BP<uint64_t> newmask, BP<uint64_t> comp_next, BP<int32_t> counts, int B, hipStream_t s);
// occ: occupied blocks (count > 0) in block order
hipError_t launch_scan(BP<const int32_t> counts, int64_t n, int bq, BP<int4> partial, BP<int4> offs, BP<int32_t> occ,
                       BP<int32_t> tot, BP<int64_t> stats_level, int B, hipStream_t s);
inline int64_t scan_partials(int64_t n) { return (n + 2047) / 2048; }
// reads the occupied-block list and its count tot[2] written by launch_scan
// list_cap, item_cap: capacities of one shape's list and item array (checked in
// bounds-checked builds)
hipError_t launch_emit(BP<const uint64_t> newmask, BP<const int32_t> counts, BP<const int4> offs,
                       BP<const int32_t> occ, BP<const int32_t> tot, int Rn, int bq, BP<int32_t> list,
                       int64_t list_cap, BP<Item> items, int64_t item_cap, int B, hipStream_t s);
hipError_t launch_fill(BP<const float> prev, int Pp, BP<float> next, int Pn, int B, hipStream_t s);
// prefix[b] = sum over shapes b' < b of ceil(max(cnt[b' * stride], 0) / per), b = 0 .. B
// (the tiles or work items of a ragged batched decode); one workgroup, B <= 4096
hipError_t launch_batch_prefix(const int32_t* cnt, int64_t stride, int B, int per, int64_t* prefix, hipStream_t s);
hipError_t launch_bits_to_bytes(const uint64_t* m, int n, int NB, uint8_t* out, hipStream_t s);
hipError_t launch_items_from_list(const int32_t* list, int64_t N, int R, int block, const int32_t* block_row, int bq,
                                  Item* items, int32_t* n_items, float* out, hipStream_t s);

}  // namespace vdm
