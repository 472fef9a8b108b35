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

hipError_t launch_zero(void* p, size_t bytes, hipStream_t s);
hipError_t launch_stats_init(int64_t* stats, int levels, int R0, hipStream_t s);
// part: stat_part_words() zero-initialised partial counters (left zero on return)
inline int64_t stat_part_words() { return 256 * 8; }
hipError_t launch_cell_test(const float* vol, int R, const uint64_t* kept_prev, float tau, uint64_t* active,
                            int64_t* part, int64_t* stat_tested, int64_t* stat_active, hipStream_t s);
// identity = 1: copy (and count) without dilating; stat may be null (no count)
hipError_t launch_dilate(const uint64_t* in, uint64_t* out, int R, int identity, int64_t* part, int64_t* stat,
                         hipStream_t s);
hipError_t launch_mark(const uint64_t* kept, int R, const uint64_t* comp_prev, int all_new, int Rn,
                       uint64_t* newmask, uint64_t* comp_next, int32_t* counts, hipStream_t s);
// occ: occupied blocks (count > 0) in block order
hipError_t launch_scan(const int32_t* counts, int64_t n, int bq, int4* partial, int4* offs, int32_t* occ, int32_t* tot,
                       int64_t* stats_level, hipStream_t s);
inline int64_t scan_partials(int64_t n) { return (n + 2047) / 2048; }
// reads the occupied-block list and its count tot[2] written by launch_scan
hipError_t launch_emit(const uint64_t* newmask, const int32_t* counts, const int4* offs, const int32_t* occ,
                       const int32_t* tot, int Rn, int bq, int32_t* list, Item* items, hipStream_t s);
hipError_t launch_fill(const float* prev, int Pp, float* next, int Pn, hipStream_t s);
hipError_t launch_bits_to_bytes(const uint64_t* m, int n, int NB, uint8_t* out, hipStream_t s);
hipError_t launch_items_from_list(const int32_t* list, int64_t N, int R, int block, const int32_t* block_row, int bq,
                                  Item* items, int32_t* n_items, float* out, hipStream_t s);

}  // namespace vdm
