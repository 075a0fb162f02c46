// Index maps between MFMA lanes, keys / head dims and LDS positions.
// Host+device so that tests can check them on the CPU (bijectivity and
// bank-conflict freedom) without a GPU.
//
// Key order inside one 32-key step.  The S^T = K Q^T product uses two 16x16
// M-tiles per step; row m of half h (= M-tile parity) is key
//     32*(mt/2) + 8*(m/4) + 4*h + m%4.
// With the C layout (lane group g holds rows 4g..4g+3) this puts keys
// 8g..8g+7 of the step in lane group g, i.e. exactly the 8 contraction slots
// the following P.V MFMA (16x16x32) expects from that lane group, so the
// probabilities go from accumulators to operands without any data movement.
// The P.V output rows (head dims) use the same map, which gives every lane
// eight consecutive output columns (16-byte stores).
//
// LDS swizzles: a 16-byte chunk c of a row r is stored at chunk position
// c ^ swz(r); swz only touches the low 4 (or 3, 2) bits, so a row's chunks
// are permuted within aligned groups.  The maps are chosen so that the 16
// lanes of one lane group read 16 distinct 16-byte bank slots.
#pragma once

#if defined(__HIPCC__)
#define MQA_HD __host__ __device__ __forceinline__
#else
#define MQA_HD inline
#endif

namespace mqa {
namespace layout {

// key (within the tile) of row m of S^T M-tile mt
MQA_HD constexpr int st_row_key(int mt, int m) {
    return 32 * (mt >> 1) + 8 * (m >> 2) + 4 * (mt & 1) + (m & 3);
}
// key held by accumulator element i of lane group g in S^T M-tile mt
MQA_HD constexpr int st_c_key(int mt, int g, int i) {
    return 32 * (mt >> 1) + 8 * g + 4 * (mt & 1) + i;
}
// head dim of row m of P.V M-tile mt, and of accumulator element i of group g
MQA_HD constexpr int pv_row_d(int mt, int m) { return st_row_key(mt, m); }
MQA_HD constexpr int pv_c_d(int mt, int g, int i) { return st_c_key(mt, g, i); }

// Row-major key tile (>= 16 chunks per row): chunk position = c ^ kswz(row).
MQA_HD constexpr int kswz(int row) { return (((row >> 3) & 3) << 2) | (row & 3); }

// Rows of 8 chunks (128 bytes): chunk position = c ^ swz8(row).
MQA_HD constexpr int swz8(int row) { return ((row >> 1) & 1) | (((row >> 3) & 3) << 1); }
// Rows of 4 chunks (64 bytes): chunk position = c ^ swz4(row).
MQA_HD constexpr int swz4(int row) { return (row >> 3) & 3; }

// Swizzle for a transposed V tile row (head dim d) holding rl chunks of keys.
MQA_HD constexpr int vswz(int d, int rl) { return rl == 4 ? swz4(d) : swz8(d); }

}  // namespace layout
}  // namespace mqa
