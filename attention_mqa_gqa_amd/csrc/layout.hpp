// Index maps between MFMA lanes, keys / head dims and LDS positions.
// Host+device so that tests can check them on the CPU (bijectivity and
// bank-conflict freedom) without a GPU.
//
// LDS swizzles: a 16-byte chunk c of a row r is stored at chunk position
// c ^ swz(r); a swizzle only permutes chunks within aligned groups, and the
// maps are chosen so that the lanes served together read distinct 16-byte
// bank slots.
#pragma once

#if defined(__HIPCC__)
#define MQA_HD __host__ __device__ __forceinline__
#else
#define MQA_HD inline
#endif

namespace mqa {
namespace layout {

// ---------------------------------------------------------------------------
// Maps for v_mfma_f32_32x32x16_bf16 (A/B: lane l holds row/column l % 32 and
// 8 contraction elements of lane half l / 32; C: accumulator i of lane l is
// row 8*(i/4) + 4*(l/32) + i%4, column l % 32).
//
// Row m of a 32-row A operand is mapped to key / head dim swap23(m) (bits 2
// and 3 exchanged).  Then the 16 accumulators of lane half h are the keys
// 8h..8h+7 (i = 0..7) and 16+8h..16+8h+7 (i = 8..15): the scores of a lane
// are directly the two 16-key P operands of the next MFMA, and a P.V output
// lane holds two runs of 8 consecutive head dims.
MQA_HD constexpr int swap23(int m) { return (m & ~12) | (((m >> 2) & 1) << 3) | (((m >> 3) & 1) << 2); }
// key (head dim) held by accumulator i of lane half h
MQA_HD constexpr int c32_index(int h, int i) { return 16 * (i >> 3) + 8 * h + (i & 7); }

// Swizzles for 32-row operand reads (16 lanes -> 16 distinct 16-byte slots
// per 256 bytes and 8 lanes -> 8 distinct slots per 128 bytes):
//   rows of >= 16 chunks, rows of 8 chunks, rows of 4 chunks.
MQA_HD constexpr int swz32_16(int r) { return swap23(r & 15); }
MQA_HD constexpr int swz32_8(int r) { return ((r >> 1) & 1) | (((r >> 3) & 1) << 1) | (((r ^ (r >> 2)) & 1) << 2); }
MQA_HD constexpr int swz32_4(int r) { return ((r >> 3) & 1) | ((((r >> 1) ^ (r >> 2)) & 1) << 1); }
// Rows of an odd multiple of 8 chunks (24: a 192-wide bf16 row).  Row r
// starts at chunk 24r, i.e. 8 (r & 1) modulo 16, so the row parity already
// separates two halves of a 256-byte bank window; the swizzle permutes
// chunks within aligned groups of 8 and must be one-to-one on the rows of
// one parity (16-lane groups) and on the rows of one 8-lane group (rows
// {0-3, 8-11} or {4-7, 12-15} after swap23).
MQA_HD constexpr int swz32_x8(int r) { return ((r ^ (r >> 2)) & 1) | (r & 2) | (((r >> 3) & 1) << 2); }
MQA_HD constexpr int swz32(int r, int row_chunks) {
    return row_chunks % 16 == 0 ? swz32_16(r)
         : row_chunks == 8      ? swz32_8(r)
         : row_chunks % 16 == 8 ? swz32_x8(r)
                                : swz32_4(r);
}
// chunks per swizzle group of a 32-row operand row (the swizzle keeps a
// chunk inside its aligned group of this many chunks)
MQA_HD constexpr int swz32_group(int row_chunks) { return row_chunks % 16 == 0 ? 16 : (row_chunks % 8 == 0 ? 8 : 4); }

// Rows that are one 1 KB copy each (K rows at D = 512, MLA latent rows) are
// stored with 16 bytes of padding, key row r at row position swap23(r): the
// lane that reads key swap23(n) reads position n, and 8 (16) consecutive
// lanes hit 8 (16) distinct bank slots without any swizzle.
MQA_HD constexpr int padded_row_bytes(int row_bytes) { return row_bytes + 16; }
MQA_HD constexpr int padded_row_pos(int key_row) { return swap23(key_row & 31) | (key_row & ~31); }

// Bytes of one prefill K tile of kt keys as stored in the workspace tile
// stream and in LDS: padded 1 KB rows (d_qk = 512) or plain swizzled rows.
MQA_HD constexpr int prefill_k_tile_bytes(int kt, int d_qk) {
    return 2 * d_qk == 1024 ? kt * padded_row_bytes(1024) : kt * 2 * d_qk;
}

// MLA-absorbed decode tiles (32 cache rows).
// Latent rows (1 KB + 16 B padding): row k of the tile sits at row position
// 8(k/8) + 2(k%4) + (k/4)%2.  Score reads (lane n reads row n) then hit
// distinct bank slots over 8 and 16 lanes, and a transposing 64-bit read of
// four consecutive rows (one 16-lane group) touches 4 x 32 distinct bytes
// of every 128-byte bank window.
MQA_HD constexpr int mla_lat_pos(int k) { return (k & ~7) | ((k & 3) << 1) | ((k >> 2) & 1); }
// RoPE rows (128 B = 8 chunks): chunk c of row r at position c ^ mla_rope_swz(r).
MQA_HD constexpr int mla_rope_swz(int r) { return (r ^ (r >> 3)) & 7; }
// P tile (one 64-byte row of 32 keys per head): chunk c at c ^ ptile_swz(h).
MQA_HD constexpr int ptile_swz(int h) { return ((h >> 1) ^ (h >> 2)) & 3; }

}  // namespace layout
}  // namespace mqa
