// Causal / full prefill attention for query heads sharing key/value heads.
//
// 16-bit path, bf16 or fp16 inputs (flash-style, one pass over K/V, scores
// never materialised --
// the tiling idea of "GQA和MLA详解" (lzwjava.github.io) §4 applied to the
// (T,T) score matrix as that page's §1 describes):
//   * one workgroup = one (batch, KV head) and a block of query tokens for
//     ALL G query heads of that KV head, so every K/V tile staged in LDS is
//     reused by the whole head group (the MQA/GQA saving; heads are indexed,
//     never copied -- lzwjava §2);
//   * per wave: 32*NR query rows; S^T = K Q^T and O^T += V^T P^T on
//     v_mfma_f32_32x32x16_bf16 with fp32 accumulation; Q stays in VGPRs,
//     the O^T accumulator for the full value width stays in AGPRs;
//   * online softmax per row in registers (exp2 domain, lazy rescale);
//   * K tiles (from K itself, or pre-padded at d = 512) and pre-transposed
//     V tiles are copied global->LDS with asynchronous direct-to-LDS loads,
//     double buffered;
//   * causal: key tiles past the block's last token are never visited, the
//     diagonal tile is masked per element, and the heaviest blocks start
//     first.
// Queries and keys may differ in number (T_q <= T_kv when causal: the
// queries are the last T_q tokens of the sequence) and the value width may
// differ from the query/key width (expanded MLA prefill: 192 / 128).
// fp32 path: a plain fp32 VALU kernel (no reduced-precision operands).
#include <type_traits>

#include "common.hpp"
#include "layout.hpp"
#include "kernels.hpp"

namespace mqa {

// ---------------------------------------------------------------------------
// K [B*Hkv, T, DK], V [B*Hkv, T, DV] -> tile stream
// [B*Hkv, n_tiles, (K tile | V^T tile)] for DK = 512, [B*Hkv, n_tiles,
// V^T tile] otherwise.
// Each 32-key tile is stored exactly as the prefill kernel keeps it in LDS:
// the V^T tile (row = value dim, 32 keys per row, swizzled chunks), zero
// past T, and for 1 KB rows the K tile (row-major, plain chunk order with 16
// bytes of padding per row, key layout::padded_row_pos(p) at row position
// p).  V's contraction index (the key) is its row index, so the P.V operand
// needs it transposed; doing that here once turns every V copy of the main
// kernel into a straight 16-byte stream (uniform base + 16 * lane).  Narrower
// K rows need no packing: the main kernel copies them from K itself, the
// chunk swizzle folded into its per-lane source offsets.
// ---------------------------------------------------------------------------
template <int DK, int DV, int KT>
__global__ __launch_bounds__(256) void kv_pack_kernel(const bf16* __restrict__ K, const bf16* __restrict__ V,
                                                      bf16* __restrict__ KVt, int T, int n_tiles) {
    constexpr int RL = KT / 8;           // 16-byte chunks per V^T row
    constexpr int ROW_CHUNKS = DK / 8;   // 16-byte chunks per K row
    constexpr int NB = RL * (DV / 8);    // 8x8 blocks per V tile
    constexpr bool KPAD = (2 * DK == 1024);
    constexpr int KTILE_B = KPAD ? layout::prefill_k_tile_bytes(KT, DK) : 0;   // packed K bytes per tile
    constexpr int KROW_B = layout::prefill_k_tile_bytes(KT, DK) / KT;
    constexpr int TILE_V = KT * DV;
    const int tile = blockIdx.x;
    const size_t bh = blockIdx.y;
    const bf16* ksrc = K + bh * (size_t)T * DK;
    const bf16* vsrc = V + bh * (size_t)T * DV;
    char* kdst = (char*)KVt + (bh * n_tiles + tile) * (size_t)(KTILE_B + 2 * TILE_V);
    bf16* vdst = (bf16*)(kdst + KTILE_B);
    // blockIdx.z: 0 packs the K tile (1 KB rows only), 1 the V^T tile (a
    // grid of depth 1 packs only V^T)
    const int part = KPAD ? (int)blockIdx.z : 1;
    // K tile: chunk position p of row position kk holds global chunk
    // p ^ swz(kk) of key kk, or (1 KB rows) chunk p of key padded_row_pos(kk)
#pragma unroll 8
    for (int q = threadIdx.x; part == 0 && q < KT * ROW_CHUNKS; q += 256) {
        const int kk = q / ROW_CHUNKS;
        const int p = q % ROW_CHUNKS;
        const int c = KPAD ? p : (p ^ layout::swz32(kk, ROW_CHUNKS));
        const int key = tile * KT + (KPAD ? layout::padded_row_pos(kk) : kk);
        const u32x4 val = key < T ? ldg16(ksrc + (size_t)key * DK + c * 8) : u32x4{0, 0, 0, 0};
        *(u32x4*)(kdst + kk * KROW_B + p * 16) = val;
    }
    // V^T tile: 8x8 blocks transposed with byte permutes
    for (int blk = threadIdx.x; part == 1 && blk < NB; blk += 256) {
        const int kb = blk % RL;
        const int db = blk / RL;
        u32x4 r[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int key = tile * KT + kb * 8 + j;
            if (key < T) r[j] = ldg16(vsrc + (size_t)key * DV + db * 8);
            else r[j] = u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const int d = db * 8 + t;
            const uint32_t sel = (t & 1) ? kSelHiHalves : kSelLoHalves;
            const int w = t >> 1;
            u32x4 o;
            o.x = perm(r[1][w], r[0][w], sel);
            o.y = perm(r[3][w], r[2][w], sel);
            o.z = perm(r[5][w], r[4][w], sel);
            o.w = perm(r[7][w], r[6][w], sel);
            const int pos = kb ^ layout::swz32(d, RL);
            *(u32x4*)(vdst + (size_t)(d * RL + pos) * 8) = o;
        }
    }
}

// ---------------------------------------------------------------------------
// 16-bit flash prefill on v_mfma_f32_32x32x16_bf16 (F16: _f16, fp16 inputs,
// P and a 16-bit output rounded to fp16).
//   DK  query/key width (128, 192 or 512)   DV  value width (128 or 512)
//   NR  32-row N-tiles per wave             NW  waves per workgroup
//   KT  keys per tile (32)
// Each wave owns 32*NR query rows with the full widths: Q^T operands and
// the O^T accumulator stay in registers for the whole key loop (one wave per
// SIMD at 512).  Rows of a workgroup: r = 0 .. NW*32*NR-1, head = r % G,
// token = t0 + r / G.  Keys inside a tile follow layout::swap23 so that the
// score accumulators are the P operands of the P.V MFMA as they stand.
// Causal: query token i (of Tq) sees keys j <= i + q_off, q_off = Tkv - Tq.
// ---------------------------------------------------------------------------
template <int DK, int DV, int NR, int NW, int KT, bool CAUSAL, bool OUT_F32, bool F16>
__global__ __launch_bounds__(NW * 64, (DK == 512 ? 1 : 8 / NW)) void prefill_bf16_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ KVt,
    void* __restrict__ Out, float* __restrict__ Lse, int Hq, int Hkv, int Tq, int Tkv, int q_off,
    int G, int tok_per_wg, int n_tok_blocks, int n_kv_tiles, int xcd_map, float scale_log2) {
    constexpr int RW = 32 * NR;           // rows per wave
    constexpr int KS = DK / 16;           // QK^T contraction steps
    constexpr int MT_O = DV / 32;         // O^T M-tiles (value dims)
    constexpr int KSP = KT / 16;          // P.V contraction steps
    constexpr int RL = KT / 8;            // chunks per V^T row
    constexpr int TILE_K = KT * DK;       // elements per K tile
    constexpr int TILE_V = KT * DV;       // elements per V^T tile
    constexpr int ROW_CHUNKS = DK / 8;
    // 1 KB copies per tile; a K tile that does not split evenly over the
    // waves ends with one round in which every wave copies PLK lanes' worth
    // (so every wave issues the same number of copy instructions)
    constexpr int CK = TILE_K * 2 / 1024;
    constexpr int CV = TILE_V * 2 / 1024;
    constexpr int FK = CK / NW;                            // full K copy rounds
    constexpr int PLK = (CK % NW) * 64 / NW;               // lanes per wave in the last round
    constexpr int LHK = FK + (PLK ? 1 : 0);                // copy instructions per wave per K tile
    constexpr int LHV = CV / NW;                           // ... per V^T tile
    // K rows of 1 KB (DK = 512) are one copy instruction each, so in LDS each
    // row can start 16 bytes after the previous one ends (and rows can be
    // placed in any order): the 8 or 16 lanes served together then read
    // distinct bank slots without any swizzle, and a lane reads every
    // contraction step of its row from one address register plus an
    // immediate offset.  Narrower rows are swizzled instead.
    constexpr bool KPAD = (2 * DK == 1024);
    constexpr int KSTAGE_B = layout::prefill_k_tile_bytes(KT, DK);   // LDS bytes per K stage
    constexpr int KROW_B = KSTAGE_B / KT;                            // LDS bytes per K row
    constexpr int VSTAGE_B = 2 * TILE_V;                   // LDS bytes per V^T stage
    static_assert(KT == 32, "key tile");
    static_assert(CV % NW == 0, "V^T tile must split evenly over the waves");
    static_assert((CK % NW) * 64 % NW == 0 && (!KPAD || (PLK == 0 && FK % 4 == 0)), "K tile split");

    // 16-bit outputs leave through LDS (rows of 2 DV + 16 bytes, reusing the
    // stages once the loop is done)
    constexpr int OROW_B = 2 * DV + 16;
    constexpr int OUT_LDS_B = OUT_F32 ? 0 : NW * RW * OROW_B;
    constexpr int SMEM_B = 2 * KSTAGE_B + 2 * VSTAGE_B > OUT_LDS_B ? 2 * KSTAGE_B + 2 * VSTAGE_B : OUT_LDS_B;
    __shared__ __attribute__((aligned(16))) char smem[SMEM_B];

    const int lane = lane_id();
    const int w = wave_id();
    const int h2 = lane >> 5;             // lane half
    const int n = lane & 31;              // row (column of the 32x32 tile)
    // Workgroup -> (batch, KV head, token block).  Workgroups are dealt to
    // the XCDs round-robin by flat index f (XCD f % 8, its slot-th one).  The
    // maps keep the K/V tiles an XCD re-reads in its own L2:
    //   xcd_map 1 (pairs P = B*Hkv a multiple of 8): every XCD takes whole
    //     (batch, KV head) pairs, blocks of a pair heaviest first;
    //   xcd_map 2 (8 a multiple of P, blocks a multiple of 8/P): each pair
    //     gets 8/P XCDs and their slots deal its blocks heaviest first;
    //   otherwise the launch grid's own order.
    int blk, hk, b;
    if (xcd_map != 0) {
        const int f = (int)(blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z));
        const int x = f % kNumXcd, slot = f / kNumXcd;
        int pair;
        if (xcd_map == 1) {
            pair = (slot / n_tok_blocks) * kNumXcd + x;
            blk = slot % n_tok_blocks;
        } else {
            const int P = (int)(gridDim.y * gridDim.z);
            pair = x % P;
            blk = slot * (kNumXcd / P) + x / P;
        }
        hk = pair % Hkv;
        b = pair / Hkv;
    } else {
        blk = blockIdx.x;
        hk = blockIdx.y;
        b = blockIdx.z;
    }
    const int tb = CAUSAL ? (n_tok_blocks - 1 - blk) : blk;     // heaviest blocks first
    const int t0 = tb * tok_per_wg;
    const int rows_used = tok_per_wg * G;

    int row_tok[NR];
    int row_head[NR];
    bool row_ok[NR];
#pragma unroll
    for (int nt = 0; nt < NR; ++nt) {
        const int r = w * RW + 32 * nt + n;
        row_tok[nt] = t0 + r / G;
        row_head[nt] = hk * G + r % G;
        row_ok[nt] = (r < rows_used) && (row_tok[nt] < Tq);
    }

    // Q^T operands: lane half h2 holds head dims 16ks + 8h2 .. +7 of row n.
    bf16x8 qb[NR][KS];
#pragma unroll
    for (int nt = 0; nt < NR; ++nt) {
        const bf16* qrow = Q + (((size_t)b * Hq + row_head[nt]) * Tq + (row_ok[nt] ? row_tok[nt] : 0)) * DK;
        const u32x4 zero = {0, 0, 0, 0};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const u32x4 v = ldg16(qrow + 16 * ks + 8 * h2);
            qb[nt][ks] = __builtin_bit_cast(bf16x8, row_ok[nt] ? v : zero);
        }
    }

    const size_t bh = (size_t)b * Hkv + hk;
    // tile stream: (padded K tile |) V^T tile; narrower K rows come from K
    constexpr int KSTREAM_B = KPAD ? KSTAGE_B : 0;
    constexpr int TILE_B = KSTREAM_B + 2 * TILE_V;     // bytes per tile in the stream
    const char* KVbh = (const char*)KVt + bh * (size_t)n_kv_tiles * TILE_B;
    const uint64_t Kg = (uint64_t)(uintptr_t)(K + bh * (size_t)Tkv * DK);

    const int t_last = min(Tq, t0 + tok_per_wg) - 1;
    const int n_tiles = CAUSAL ? ((t_last + q_off) / KT + 1) : n_kv_tiles;

    // LDS: K stages 0/1, then V^T stages 0/1; tile j lives in stage j & 1.
    // Iteration t starts with one barrier (K(t+1) and V(t) have landed; every
    // wave is done with S(t), which read K(t), and with P(t-1).V(t-1)), then
    // computes S(t+1) next to softmax(t) while copying K(t+2) into the stage
    // of K(t), then P(t).V(t); V(t+1) goes into the stage of V(t-1) at the
    // start of one of the two phases.  With one wave per SIMD (d_qk = 512)
    // the copies are split over both phases (measured 3.7 % faster); with two
    // waves per SIMD both go in phase A (6 % faster at d_qk = 192).
    constexpr bool V_IN_B = KPAD;
    static_assert(!V_IN_B || LHV % 4 == 0, "V copies in phase B go by groups of four");
    const uint32_t lds_base = lds_addr(smem);
    const uint32_t lane16 = (uint32_t)lane * 16u;
    // copy group g (of FK / 4) of a padded K tile: four padded 1 KB rows,
    // identical in the stream and in LDS, four copies per M0 write.  The
    // grouped copies (padded K, V^T) sit inside the MFMA chains and are
    // issued on every iteration, also for tiles past the last one: those
    // read the last tile again into a stage that nothing reads afterwards
    // (bit-identical results; a branch would cut the chain into separate
    // scheduling regions, 1.2 % slower at d_qk = 512)
    auto issue_k_group = [&](int tile, int g) {
        const char* src = KVbh + (size_t)min(tile, n_tiles - 1) * TILE_B;
        const uint32_t dst = lds_base + (uint32_t)((tile & 1) * KSTAGE_B);
        const int row = (g * NW + w) * 4;
        if constexpr (KPAD) copy4_to_lds_async<KROW_B>(src + row * KROW_B, lane16, dst + (uint32_t)(row * KROW_B));
    };
    // Unpadded K tiles are copied from K itself: LDS byte o of a tile is
    // chunk (o % row) / 16 of row r = o / row, which holds chunk
    // c ^ swz32(r) of key r; k_src gives that chunk's byte offset from the
    // tile's first key row (rows at or past the tile's row_lim valid rows
    // read the last valid one, masked later).
    auto k_src = [&](int o, int row_lim) -> uint32_t {
        const int r = o / (2 * DK), c = (o % (2 * DK)) / 16;
        return (uint32_t)(min(r, row_lim - 1) * (2 * DK) + ((c ^ layout::swz32(r, ROW_CHUNKS)) * 16));
    };
    auto k_copy_byte = [&](int i) {      // LDS byte of this lane in K copy i
        return i < FK ? (i * NW + w) * 1024 + lane * 16 : FK * NW * 1024 + w * PLK * 16 + lane * 16;
    };
    auto issue_k = [&](int tile) {
        const uint32_t dst = lds_base + (uint32_t)((tile & 1) * KSTAGE_B);
        if constexpr (KPAD) {
#pragma unroll
            for (int g = 0; g < FK / 4; ++g) issue_k_group(tile, g);
        } else {
            const void* src = (const void*)(uintptr_t)(Kg + (uint64_t)tile * (KT * 2 * DK));
            const int row_lim = min(Tkv - tile * KT, KT);    // valid rows of this tile (wave-uniform)
#pragma unroll
            for (int i = 0; i < FK; ++i) {
                const int inst = i * NW + w;               // wave-uniform
                const uint32_t off = k_src(k_copy_byte(i), row_lim);
                copy16_to_lds_async(src, off, dst + (uint32_t)inst * 1024u);
            }
            if constexpr (PLK != 0) {
                // last round: wave w copies bytes [FK NW 1 KB + 16 PLK w, +16 PLK)
                // of the tile with its first PLK lanes
                const uint32_t lds_off = (uint32_t)(FK * NW * 1024 + w * PLK * 16);
                const uint32_t off = k_src(min(k_copy_byte(FK), TILE_K * 2 - 16), row_lim);
                if (lane < PLK) copy16_to_lds_async(src, off, dst + lds_off);
            }
        }
    };
    // copy group g (of LHV / 4) of a V^T tile: V^T tiles are contiguous in
    // both places, so each wave copies runs of 4 KB, four copies per M0 write
    auto issue_v_group = [&](int tile, int g) {
        const char* src = KVbh + (size_t)min(tile, n_tiles - 1) * TILE_B + KSTREAM_B;
        const uint32_t dst = lds_base + (uint32_t)(2 * KSTAGE_B + (tile & 1) * VSTAGE_B);
        const int inst = (g * NW + w) * 4;
        copy4_to_lds_async<1024>(src + inst * 1024, lane16, dst + (uint32_t)inst * 1024u);
    };
    auto issue_v = [&](int tile) {
        const char* src = KVbh + (size_t)tile * TILE_B + KSTREAM_B;
        const uint32_t dst = lds_base + (uint32_t)(2 * KSTAGE_B + (tile & 1) * VSTAGE_B);
        if constexpr (LHV % 4 == 0) {
#pragma unroll
            for (int g = 0; g < LHV / 4; ++g) issue_v_group(tile, g);
        } else {
#pragma unroll
            for (int i = 0; i < LHV; ++i) {
                const int inst = i * NW + w;
                copy16_to_lds_async(src + inst * 1024, lane16, dst + (uint32_t)inst * 1024u);
            }
        }
    };

    f32x16 o[MT_O][NR];
#pragma unroll
    for (int mt = 0; mt < MT_O; ++mt)
#pragma unroll
        for (int nt = 0; nt < NR; ++nt) o[mt][nt] = f32x16{};
    float m_run[NR], l_run[NR];
#pragma unroll
    for (int nt = 0; nt < NR; ++nt) { m_run[nt] = -INFINITY; l_run[nt] = 0.f; }

    // K operand of contraction step ks for this lane (key row swap23(n),
    // dims 16ks + 8h2 .. +7), as a byte offset into a K stage.  Padded rows:
    // one base plus 32 ks.  Swizzled rows: the swizzle only permutes chunks
    // within aligned groups of GS (16, or 8 for 24-chunk rows), so GS/2 lane
    // offsets plus an immediate stride of 16 GS bytes per GS/2 steps cover
    // every step.
    const int krow = layout::swap23(n);
    const uint32_t kpad_off = (uint32_t)(n * KROW_B + h2 * 16);
    constexpr int GS = layout::swz32_group(ROW_CHUNKS);
    constexpr int NKO = GS / 2;
    uint32_t koff[KPAD ? 1 : NKO];
    if constexpr (!KPAD) {
        const int k_swz = layout::swz32(krow, ROW_CHUNKS);
#pragma unroll
        for (int v = 0; v < NKO; ++v) koff[v] = (uint32_t)(krow * 2 * DK + (((2 * v + h2) ^ k_swz) * 16));
    }
    auto kread = [&](const char* kst, int ks) {
        if constexpr (KPAD) return *(const bf16x8*)(kst + kpad_off + ks * 32);
        else return *(const bf16x8*)(kst + koff[ks % NKO] + (ks / NKO) * (GS * 16));
    };
    constexpr int PF = 4;

    // full S^T of one tile into acc (prologue only)
    auto s_all = [&](f32x16 (&acc)[NR], const char* kst) {
        bf16x8 abuf[PF];
#pragma unroll
        for (int j = 0; j < PF; ++j) abuf[j] = kread(kst, j);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const bf16x8 a = abuf[ks % PF];
            if (ks + PF < KS) abuf[ks % PF] = kread(kst, ks + PF);
#pragma unroll
            for (int nt = 0; nt < NR; ++nt) acc[nt] = mfma_32x32x16_t<F16>(a, qb[nt][ks], acc[nt]);
        }
    };

    // Softmax pieces on one tile's scores (raw S^T accumulators; the scale
    // is > 0, so row maxima are taken on raw scores and the scale folds
    // into the exponent).  Key of accumulator i of lane half h2 within the
    // tile: layout::c32_index(h2, i); row nt of this lane: token row_tok[nt].
    auto mask_tile = [&](f32x16 (&sc)[NR], int tile) {
        const int j0 = tile * KT;
#pragma unroll
        for (int nt = 0; nt < NR; ++nt) {
            const int lim = (CAUSAL ? min(row_tok[nt] + q_off, Tkv - 1) : Tkv - 1) - j0;
#pragma unroll
            for (int i = 0; i < 16; ++i)
                if (layout::c32_index(h2, i) > lim) sc[nt][i] = -INFINITY;
        }
    };
    // does any row of this wave see a masked key in `tile`?
    const int wave_tok_min = t0 + (w * RW) / G;
    auto tile_masked = [&](int tile) {
        const int last_key = tile * KT + KT - 1;
        return last_key >= Tkv || (CAUSAL && last_key > wave_tok_min + q_off);
    };
    const float c = scale_log2;

    // prologue: copies K(0), K(1), V(0); S(0).
    issue_k(0);
    if (n_tiles > 1) issue_k(1);
    issue_v(0);
    wait_vmcnt_of<LHK, LHV>(n_tiles > 1 ? LHK + LHV : LHV);   // K(0) has landed
    __syncthreads();
    f32x16 sA[NR], sB[NR];
#pragma unroll
    for (int nt = 0; nt < NR; ++nt) sA[nt] = f32x16{};
    s_all(sA, smem);
    if (tile_masked(0)) mask_tile(sA, 0);
#pragma unroll
    for (int nt = 0; nt < NR; ++nt) {
        float mloc = -INFINITY;
#pragma unroll
        for (int i = 0; i < 8; ++i) mloc = max3f(mloc, sA[nt][2 * i], sA[nt][2 * i + 1]);
        m_run[nt] = max_over_halves(mloc) * c;
    }

    // Iteration t (scores of tile t in sc, masked, row max folded into m_run):
    //   barrier;
    //   phase A: copies of K(t+2) (and V(t+1)); S(t+1) MFMAs, with the
    //            exponentials, row sums and bf16 packing of P(t) placed
    //            between them;
    //   phase B: (copies of V(t+1)); P(t).V(t) MFMAs, with the masking and
    //            row max of S(t+1) between them; then the (rare) lazy
    //            rescale for tile t+1.
    // Each phase is a fixed sequence of chunks separated by scheduling
    // fences, so MFMA latency is filled with this wave's VALU work.  The
    // copies issued at iteration t are the only ones in flight and must
    // land before iteration t+1, so the wait is for all of them.
    // The score buffers alternate between sA and sB (loop unrolled by 2).
    constexpr int NSTEP_PV = KSP * MT_O;
    auto body = [&](int it, f32x16 (&sc)[NR], f32x16 (&sn)[NR]) {
        const bool has_next = it + 1 < n_tiles;
        // K(it+1) and V(it) have landed
        wait_vmcnt<0>();
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();

        // ---- phase A: S(it+1) (unconditionally: on the last tile it reads a
        // stale but valid K stage and is discarded) | exp of S(it) ----------
        // The first K operand reads go out before the copies, whose issue
        // then covers their latency.
        const char* kst = smem + ((it + 1) & 1) * KSTAGE_B;
#pragma unroll
        for (int nt = 0; nt < NR; ++nt) sn[nt] = f32x16{};
        // Row sums of P(t): at d_qk = 512 the fp32 probabilities are added
        // up next to the exponentials.  Elsewhere they are taken from the
        // packed 16-bit probabilities (the values the MFMAs use), a pair per
        // v_dot2c, half the VALU instructions: at 128 in phase B, whose
        // phase A is the most exponential-heavy (≈1 % faster), at 192 right
        // after the packing in phase A (3 % faster; at 512 neither form
        // gains, and the phase-B one spills)
        constexpr bool SUM_IN_B = DK == 128;
        constexpr bool SUM_PACKED_A = DK == 192;
        float lsum[NR];
#pragma unroll
        for (int nt = 0; nt < NR; ++nt) lsum[nt] = 0.f;
        {
            bf16x8 abuf[PF];
#pragma unroll
            for (int j = 0; j < PF; ++j) abuf[j] = kread(kst, j);
            if (!KPAD && it + 2 < n_tiles) issue_k(it + 2);
            if (!V_IN_B && has_next) issue_v(it + 1);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                // padded K: the copy groups spread evenly over the phase
                if constexpr (KPAD) {
                    if (ks % (KS / (FK / 4)) == 0) issue_k_group(it + 2, ks / (KS / (FK / 4)));
                }
                const bf16x8 a = abuf[ks % PF];
                if (ks + PF < KS) abuf[ks % PF] = kread(kst, ks + PF);
#pragma unroll
                for (int nt = 0; nt < NR; ++nt) sn[nt] = mfma_32x32x16_t<F16>(a, qb[nt][ks], sn[nt]);
#pragma unroll
                for (int i = ks * 16 / KS; i < (ks + 1) * 16 / KS; ++i) {
#pragma unroll
                    for (int nt = 0; nt < NR; ++nt) {
                        // pinned to this step: otherwise the exponentials
                        // are sunk past the copy-group branch and bunch up
                        // between two MFMAs
                        float pr = fast_exp2(fmaf(sc[nt][i], c, -m_run[nt]));
                        asm volatile("" : "+v"(pr));
                        sc[nt][i] = pr;
                        if constexpr (!SUM_IN_B && !SUM_PACKED_A) lsum[nt] += pr;
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        bf16x8 pb[NR][KSP];
#pragma unroll
        for (int nt = 0; nt < NR; ++nt) {
            if constexpr (!SUM_IN_B && !SUM_PACKED_A) {
                l_run[nt] += lsum[nt];
                asm volatile("" : "+v"(l_run[nt]));
            }
#pragma unroll
            for (int kp = 0; kp < KSP; ++kp) {
                f32x4 lo = {sc[nt][8 * kp + 0], sc[nt][8 * kp + 1], sc[nt][8 * kp + 2], sc[nt][8 * kp + 3]};
                f32x4 hi = {sc[nt][8 * kp + 4], sc[nt][8 * kp + 5], sc[nt][8 * kp + 6], sc[nt][8 * kp + 7]};
                pb[nt][kp] = pack8_t<F16>(lo, hi);
                // keeps the exponentials in phase A: without a use here the
                // compiler sinks them into phase B, next to the P.V MFMAs
                asm volatile("" : "+v"(pb[nt][kp]));
                if constexpr (SUM_PACKED_A) {
                    const u32x4 wv = __builtin_bit_cast(u32x4, pb[nt][kp]);
#pragma unroll
                    for (int q = 0; q < 4; ++q) l_run[nt] = add_pair_t<F16>(wv[q], l_run[nt]);
                }
            }
        }

        // ---- phase B: O^T += V^T P^T (contraction step outer, head-dim tile
        // inner, V^T reads PF steps ahead) | row max of S(it+1) --------------
        float mloc[NR];
#pragma unroll
        for (int nt = 0; nt < NR; ++nt) mloc[nt] = -INFINITY;
        {
            const char* vl = smem + 2 * KSTAGE_B + (it & 1) * VSTAGE_B;
            bf16x8 vbuf[PF];
            auto vaddr = [&](int step) {
                const int kp = step / MT_O, mt = step % MT_O;
                const int d = 32 * mt + krow;
                return vl + (d * RL + ((2 * kp + h2) ^ layout::swz32(d, RL))) * 16;
            };
#pragma unroll
            for (int st = 0; st < PF; ++st) vbuf[st] = *(const bf16x8*)vaddr(st);
            if (has_next && tile_masked(it + 1)) mask_tile(sn, it + 1);
#pragma unroll
            for (int st = 0; st < NSTEP_PV; ++st) {
                // V(t+1) in this phase: the copy groups spread evenly over it
                if constexpr (V_IN_B) {
                    if (st % (NSTEP_PV / (LHV / 4)) == 0) issue_v_group(it + 1, st / (NSTEP_PV / (LHV / 4)));
                }
                const bf16x8 a = vbuf[st % PF];
                if (st + PF < NSTEP_PV) vbuf[st % PF] = *(const bf16x8*)vaddr(st + PF);
                const int kp = st / MT_O, mt = st % MT_O;
#pragma unroll
                for (int nt = 0; nt < NR; ++nt) mfma_32x32x16_acc_t<F16>(a, pb[nt][kp], o[mt][nt]);
                if constexpr (SUM_IN_B) {
#pragma unroll
                    for (int wd = st * 4 * KSP / NSTEP_PV; wd < (st + 1) * 4 * KSP / NSTEP_PV; ++wd) {
#pragma unroll
                        for (int nt = 0; nt < NR; ++nt)
                            l_run[nt] = add_pair_t<F16>(__builtin_bit_cast(u32x4, pb[nt][wd / 4])[wd % 4], l_run[nt]);
                    }
                }
                // two scores per max3
#pragma unroll
                for (int i = st * 8 / NSTEP_PV; i < (st + 1) * 8 / NSTEP_PV; ++i) {
#pragma unroll
                    for (int nt = 0; nt < NR; ++nt) mloc[nt] = max3f(mloc[nt], sn[nt][2 * i], sn[nt][2 * i + 1]);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        // lazy rescale for tile it+1: only when a row max grew by more than
        // 2^kRescaleSlack (after the P.V MFMAs of this tile have drained)
        float mx[NR];
        bool need = false;
#pragma unroll
        for (int nt = 0; nt < NR; ++nt) {
            mx[nt] = max_over_halves(mloc[nt]) * c;
            need |= mx[nt] > m_run[nt] + kRescaleSlack;
        }
        if (__any(need && has_next)) {
            mfma_acc_drain();
#pragma unroll
            for (int nt = 0; nt < NR; ++nt) {
                const float mnew = fmaxf(m_run[nt], mx[nt]);
                const float alpha = fast_exp2(m_run[nt] - mnew);
                m_run[nt] = mnew;
                l_run[nt] *= alpha;
#pragma unroll
                for (int mt = 0; mt < MT_O; ++mt) scale_acc(o[mt][nt], alpha);
            }
        }
    };
    for (int it = 0; it < n_tiles; it += 2) {
        body(it, sA, sB);
        if (it + 1 < n_tiles) body(it + 1, sB, sA);
    }
    wait_vmcnt<0>();    // the copies past the last tile

    // ---- epilogue: normalise, store ------------------------------------------
    // Accumulators 8 half .. 8 half + 7 of tile (mt, nt) are 8 consecutive
    // value dims of this lane's row.  fp32 rows are stored from registers.
    // 16-bit rows go through LDS first, so that every store instruction
    // writes whole rows (1 KB contiguous at d_v = 512, four 256-byte rows at
    // 128) instead of 16 bytes of each of 32 rows: at d_v = 512 a
    // workgroup's epilogue takes 4.3 us this way, 5.2 us storing 16-byte
    // pieces straight from the accumulators.
    mfma_acc_drain();
    if constexpr (!OUT_F32) __syncthreads();    // every wave is done with the last V^T stage
#pragma unroll
    for (int nt = 0; nt < NR; ++nt) {
        const float l = sum_over_halves(l_run[nt]);
        const float inv = 1.f / l;
        const size_t row = ((size_t)b * Hq + row_head[nt]) * Tq + row_tok[nt];
        char* orow = smem + (w * RW + 32 * nt + n) * OROW_B;
        if (!OUT_F32 || row_ok[nt]) {
#pragma unroll
            for (int mt = 0; mt < MT_O; ++mt) {
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    const f32x16& acc = o[mt][nt];
                    const f32x4 lo = f32x4{acc[8 * half + 0], acc[8 * half + 1], acc[8 * half + 2], acc[8 * half + 3]} * inv;
                    const f32x4 hi = f32x4{acc[8 * half + 4], acc[8 * half + 5], acc[8 * half + 6], acc[8 * half + 7]} * inv;
                    const int d0 = 32 * mt + layout::c32_index(h2, 8 * half);
                    if constexpr (OUT_F32) {
                        float* dst = (float*)Out + row * DV + d0;
                        *(f32x4*)dst = lo;
                        *(f32x4*)(dst + 4) = hi;
                    } else {
                        *(bf16x8*)(orow + 2 * d0) = pack8_t<F16>(lo, hi);
                    }
                }
            }
        }
        if (Lse != nullptr && h2 == 0 && row_ok[nt]) Lse[row] = m_run[nt] * kLn2 + __logf(l);
    }
    if constexpr (!OUT_F32) {
        __syncthreads();
        // 16-byte chunk q of row r: a wave instruction covers RPW whole rows,
        // and a wave's rows are r0, r0 + STEP, ...  All of a wave's LDS reads
        // go out before its stores (one wait instead of one per row), and
        // row r = token offset * G + head offset is stepped without divides.
        constexpr int CPR = DV / 8;                   // chunks per row
        constexpr int RPW = 64 / CPR;                 // rows per wave instruction
        constexpr int STEP = NW * RPW;
        constexpr int ITER = RW * NR / RPW;           // instructions per wave
        static_assert(64 % CPR == 0 && (RW * NR) % RPW == 0, "row split");
        const int q = lane % CPR;
        const int r0 = w * RPW + lane / CPR;
        u32x4 vals[ITER];
#pragma unroll
        for (int k = 0; k < ITER; ++k) vals[k] = *(const u32x4*)(smem + (r0 + k * STEP) * OROW_B + 16 * q);
        int tok_off = r0 / G, head_off = r0 - tok_off * G;
        const int dq = STEP / G, dr = STEP - dq * G;
        // the output pointer moves by one of two strides per step: the head
        // offset grows by dr (and the token by dq), wrapping past G
        const long long head_el = (long long)Tq * DV;
        const long long d_step = dr * head_el + (long long)dq * DV;
        const long long d_wrap = d_step - G * head_el + DV;
        bf16* optr = (bf16*)Out + (((size_t)b * Hq + (size_t)hk * G + head_off) * Tq + t0 + tok_off) * DV + 8 * q;
#pragma unroll
        for (int k = 0; k < ITER; ++k) {
            if (r0 + k * STEP < rows_used && t0 + tok_off < Tq) *(u32x4*)optr = vals[k];
            head_off += dr;
            tok_off += dq;
            const bool wrap = head_off >= G;
            head_off -= wrap ? G : 0;
            tok_off += wrap ? 1 : 0;
            optr += wrap ? d_wrap : d_step;
        }
    }
}

// ---------------------------------------------------------------------------
// fp32 prefill on the fp32 MFMA (v_mfma_f32_16x16x4_f32: fp32 products and
// fp32 accumulation), fp32 exp2.  One workgroup = 16 consecutive rows of one
// (batch, KV head), row rho = token * G + head within the group (any G), so
// every K/V tile staged in LDS serves all the group's heads.  Key tiles of
// 16.  The four waves split the widths: wave w holds dims
// [w DK/4, (w+1) DK/4) of Q^T (the contraction slice of its partial scores)
// and value dims [w DV/4, (w+1) DV/4) of O^T.  The partial scores are summed
// through LDS in wave order, so every wave holds the same full scores and
// runs the same online softmax on them.
// 16x16x4 f32 layouts (wave64): A[m][k] in lane 16k + m, B[k][n] in lane
// 16k + n, D[m][n] accumulator i of lane 16(m/4) + n with i = m % 4.
// Scores are S^T (m = key, n = row).  Row m of the A operand carries key
// 4(m%4) + m/4 of the tile, so accumulator i of lane group g holds key
// 4i + g: the B operand (P^T, k = g) of P.V step i, with no data movement.
// K rows are padded by 16 bytes and V rows by 64 in LDS, which spreads both
// operand read patterns over distinct banks.
// ---------------------------------------------------------------------------
constexpr int kF32Rows = 16;   // rows per workgroup
constexpr int kF32Kt = 16;     // keys per tile

template <int DK, int DV, bool CAUSAL>
__global__ __launch_bounds__(256) void prefill_f32_kernel(const float* __restrict__ Q, const float* __restrict__ K,
                                                          const float* __restrict__ V, float* __restrict__ Out,
                                                          float* __restrict__ Lse, int Hq, int Tq, int Tkv,
                                                          int q_off, int G, int n_blk, float scale_log2) {
    constexpr int QS = DK / 4;            // contraction slice per wave
    constexpr int KSW = QS / 4;           // MFMA steps of a partial score
    constexpr int VS = DV / 4;            // value dims per wave
    constexpr int MTV = VS / 16;          // O^T tiles per wave
    constexpr int KROW = DK + 4;          // LDS row strides (floats)
    constexpr int VROW = DV + 16;
    constexpr int KTILE = kF32Kt * KROW;
    constexpr int VTILE = kF32Kt * VROW;
    constexpr int CK = DK / 64;           // 16-byte chunks per thread per K tile
    constexpr int CV = DV / 64;
    static_assert(DK % 64 == 0 && DV % 64 == 0, "widths are multiples of 64");
    __shared__ __attribute__((aligned(16))) float lds[2 * KTILE + 2 * VTILE + 4 * 64 * 4];
    float* const kst = lds;                              // [2][KTILE]
    float* const vst = lds + 2 * KTILE;                  // [2][VTILE]
    float* const xs = lds + 2 * KTILE + 2 * VTILE;       // partial scores [wave][lane][4]

    const int tid = (int)threadIdx.x;
    const int lane = lane_id();
    const int w = wave_id();
    const int g = lane >> 4, n = lane & 15;
    const int hk = blockIdx.y, b = blockIdx.z;
    const int blk = CAUSAL ? (n_blk - 1 - (int)blockIdx.x) : (int)blockIdx.x;   // heaviest first
    const long long rho0 = (long long)blk * kF32Rows;
    const long long rho = rho0 + n;
    const int tok = (int)(rho / G);
    const int head = hk * G + (int)(rho % G);
    const bool row_ok = tok < Tq;
    const int t_last = (int)min((long long)Tq - 1, (rho0 + kF32Rows - 1) / G);
    const int n_kv = (Tkv + kF32Kt - 1) / kF32Kt;
    const int n_tiles = CAUSAL ? min((t_last + q_off) / kF32Kt + 1, n_kv) : n_kv;
    const int Hkv = (int)gridDim.y;

    // B operands of the partial scores: lane (g, n) holds Q[row n][w QS + 4s + g]
    float qv[KSW];
    {
        const float* qrow = Q + (((size_t)b * Hq + head) * Tq + (row_ok ? tok : 0)) * DK + w * QS + g;
#pragma unroll
        for (int s = 0; s < KSW; ++s) qv[s] = row_ok ? qrow[4 * s] : 0.f;
    }
    const float* Kbh = K + ((size_t)b * Hkv + hk) * (size_t)Tkv * DK;
    const float* Vbh = V + ((size_t)b * Hkv + hk) * (size_t)Tkv * DV;
    // tile t through registers: thread chunk c = tid + 256 r is key c / (D/4),
    // 16-byte column c % (D/4); keys past the end read the last key (masked)
    u32x4 kr[CK], vr[CV];
    auto load_tile = [&](int t) {
#pragma unroll
        for (int r = 0; r < CK; ++r) {
            const int c = tid + 256 * r;
            const int j = min(t * kF32Kt + c / (DK / 4), Tkv - 1);
            kr[r] = ldg16(Kbh + (size_t)j * DK + (c % (DK / 4)) * 4);
        }
#pragma unroll
        for (int r = 0; r < CV; ++r) {
            const int c = tid + 256 * r;
            const int j = min(t * kF32Kt + c / (DV / 4), Tkv - 1);
            vr[r] = ldg16(Vbh + (size_t)j * DV + (c % (DV / 4)) * 4);
        }
    };
    auto store_tile = [&](int stage) {
#pragma unroll
        for (int r = 0; r < CK; ++r) {
            const int c = tid + 256 * r;
            *(u32x4*)(kst + stage * KTILE + (c / (DK / 4)) * KROW + (c % (DK / 4)) * 4) = kr[r];
        }
#pragma unroll
        for (int r = 0; r < CV; ++r) {
            const int c = tid + 256 * r;
            *(u32x4*)(vst + stage * VTILE + (c / (DV / 4)) * VROW + (c % (DV / 4)) * 4) = vr[r];
        }
    };

    f32x4 o[MTV];
#pragma unroll
    for (int mt = 0; mt < MTV; ++mt) o[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;
    const int ksig = 4 * (n & 3) + (n >> 2);     // key carried by A-operand row n

    load_tile(0);
    store_tile(0);
    __syncthreads();
    for (int t = 0; t < n_tiles; ++t) {
        const int st = t & 1;
        if (t + 1 < n_tiles) load_tile(t + 1);     // in flight during this tile
        // partial S^T over this wave's contraction slice
        f32x4 sp = {0.f, 0.f, 0.f, 0.f};
        const float* ka = kst + st * KTILE + ksig * KROW + w * QS + g;
#pragma unroll
        for (int s = 0; s < KSW; ++s) sp = __builtin_amdgcn_mfma_f32_16x16x4f32(ka[4 * s], qv[s], sp, 0, 0, 0);
        *(f32x4*)(xs + (w * 64 + lane) * 4) = sp;
        __syncthreads();
        f32x4 sc = *(const f32x4*)(xs + lane * 4);
#pragma unroll
        for (int v = 1; v < 4; ++v) sc += *(const f32x4*)(xs + (v * 64 + lane) * 4);
        // online softmax of rows n over keys 16t + 4i + g
        float mx = -INFINITY;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int key = t * kF32Kt + 4 * i + g;
            if (key >= Tkv || (CAUSAL && key > tok + q_off)) sc[i] = -INFINITY;
            mx = fmaxf(mx, sc[i]);
        }
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float mnew = fmaxf(m_run, mx * scale_log2);
        const float alpha = m_run == -INFINITY ? 0.f : fast_exp2(m_run - mnew);
        const float mu = mnew == -INFINITY ? 0.f : mnew;
        float p[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) p[i] = fast_exp2(fmaf(sc[i], scale_log2, -mu));
        l_run = l_run * alpha + ((p[0] + p[1]) + (p[2] + p[3]));
        m_run = mnew;
        // O^T += V^T P^T over this wave's value dims
        const float* va = vst + st * VTILE + g * VROW + w * VS + n;
#pragma unroll
        for (int mt = 0; mt < MTV; ++mt) {
            o[mt] *= alpha;
#pragma unroll
            for (int s = 0; s < 4; ++s)
                o[mt] = __builtin_amdgcn_mfma_f32_16x16x4f32(va[4 * s * VROW + 16 * mt], p[s], o[mt], 0, 0, 0);
        }
        if (t + 1 < n_tiles) store_tile(st ^ 1);
        __syncthreads();
    }

    float l = l_run + __shfl_xor(l_run, 16);      // row sum over the four lane groups
    l += __shfl_xor(l, 32);
    if (!row_ok) return;
    const size_t row = ((size_t)b * Hq + head) * Tq + tok;
    const float inv = 1.f / l;
#pragma unroll
    for (int mt = 0; mt < MTV; ++mt)
        *(f32x4*)(Out + row * DV + w * VS + 16 * mt + 4 * g) = o[mt] * inv;
    if (Lse != nullptr && w == 0 && g == 0) Lse[row] = m_run * kLn2 + __logf(l);
}

template <int DK, int DV, int NR, int NW, int KT, bool F16>
static hipError_t launch_16(const PrefillArgs& a) {
    const int R = NW * 32 * NR;
    const int tok = R / a.G;
    const int n_tok_blocks = (a.Tq + tok - 1) / tok;
    const int n_kv_tiles = (a.Tkv + KT - 1) / KT;
    const int q_off = a.Tkv - a.Tq;
    bf16* kvt = (bf16*)a.workspace;
    hipLaunchKernelGGL((kv_pack_kernel<DK, DV, KT>), dim3(n_kv_tiles, a.B * a.Hkv, 2 * DK == 1024 ? 2 : 1), dim3(256),
                       0, a.stream,
                       (const bf16*)a.k, (const bf16*)a.v, kvt, a.Tkv, n_kv_tiles);
    const dim3 grid(n_tok_blocks, a.Hkv, a.B);
    const float sl2 = a.scale * kLog2e;
    const int P = a.B * a.Hkv;
    const int xcd_map = P % kNumXcd == 0 ? 1 : (kNumXcd % P == 0 && n_tok_blocks % (kNumXcd / P) == 0 ? 2 : 0);
#define MQA_PREFILL_LAUNCH(C, F)                                                                              \
    hipLaunchKernelGGL((prefill_bf16_kernel<DK, DV, NR, NW, KT, C, F, F16>), grid, dim3(NW * 64), 0, a.stream, \
                       (const bf16*)a.q, (const bf16*)a.k, (const bf16*)kvt, a.out, a.lse, a.Hq, a.Hkv, a.Tq, a.Tkv, q_off, a.G, \
                       tok, n_tok_blocks, n_kv_tiles, xcd_map, sl2)
    if (a.causal) {
        if (a.out_f32) MQA_PREFILL_LAUNCH(true, true); else MQA_PREFILL_LAUNCH(true, false);
    } else {
        if (a.out_f32) MQA_PREFILL_LAUNCH(false, true); else MQA_PREFILL_LAUNCH(false, false);
    }
#undef MQA_PREFILL_LAUNCH
    return hipGetLastError();
}

template <int DK, int DV>
static hipError_t launch_f32(const PrefillArgs& a) {
    const long long rows = (long long)a.Tq * a.G;
    const int n_blk = (int)((rows + kF32Rows - 1) / kF32Rows);
    const dim3 grid(n_blk, a.Hkv, a.B);
    const float sl2 = a.scale * kLog2e;
    const int q_off = a.Tkv - a.Tq;
    if (a.causal)
        hipLaunchKernelGGL((prefill_f32_kernel<DK, DV, true>), grid, dim3(256), 0, a.stream, (const float*)a.q,
                           (const float*)a.k, (const float*)a.v, (float*)a.out, a.lse, a.Hq, a.Tq, a.Tkv, q_off, a.G,
                           n_blk, sl2);
    else
        hipLaunchKernelGGL((prefill_f32_kernel<DK, DV, false>), grid, dim3(256), 0, a.stream, (const float*)a.q,
                           (const float*)a.k, (const float*)a.v, (float*)a.out, a.lse, a.Hq, a.Tq, a.Tkv, q_off, a.G,
                           n_blk, sl2);
    return hipGetLastError();
}

template <int DK, int DV, int NR, int NW, int KT>
static hipError_t launch_bf16(const PrefillArgs& a) {
    return a.f16 ? launch_16<DK, DV, NR, NW, KT, true>(a) : launch_16<DK, DV, NR, NW, KT, false>(a);
}

PrefillPlan prefill_plan(int d_qk, int d_v, int in16) {
    PrefillPlan p{};
    if (!in16) {
        // fp32: equal widths (multiples of 64 up to 512) or the 192 / 128 pair
        const bool ok = d_qk % 64 == 0 && d_v % 64 == 0 && d_qk <= 512 && d_v <= 512 &&
                        (d_qk == d_v || (d_qk == 192 && d_v == 128));
        p.rows_per_wg = ok ? (1 << 30) : 0;
        p.kt = 0;
        return p;
    }
    if (d_qk == 512 && d_v == 512) { p.rows_per_wg = 4 * 32 * 1; p.kt = 32; }
    else if (d_qk == 128 && d_v == 128) { p.rows_per_wg = 8 * 32 * 1; p.kt = 32; }
    // two independent 4-wave workgroups per CU: their score phases (heavy
    // on exponentials) and P.V phases drift apart instead of running in
    // lock step behind one barrier (measured 3-4 % faster than one 8-wave
    // workgroup; no gain at 128)
    else if (d_qk == 192 && d_v == 128) { p.rows_per_wg = 4 * 32 * 1; p.kt = 32; }
    return p;
}

hipError_t prefill_launch(const PrefillArgs& a) {
    if (!a.in16) {
        if (a.DK == 192 && a.DV == 128) return launch_f32<192, 128>(a);
        if (a.DK != a.DV) return hipErrorInvalidValue;
        switch (a.DK) {
            case 64: return launch_f32<64, 64>(a);
            case 128: return launch_f32<128, 128>(a);
            case 192: return launch_f32<192, 192>(a);
            case 256: return launch_f32<256, 256>(a);
            case 320: return launch_f32<320, 320>(a);
            case 384: return launch_f32<384, 384>(a);
            case 448: return launch_f32<448, 448>(a);
            case 512: return launch_f32<512, 512>(a);
            default: return hipErrorInvalidValue;
        }
    }
    if (a.DK == 512 && a.DV == 512) return launch_bf16<512, 512, 1, 4, 32>(a);
    // 128 and 192 / 128: eight waves of one 32-row tile each (at most 256
    // registers, two waves per SIMD, so one wave's softmax overlaps the
    // other's MFMAs)
    if (a.DK == 128 && a.DV == 128) return launch_bf16<128, 128, 1, 8, 32>(a);
    if (a.DK == 192 && a.DV == 128) return launch_bf16<192, 128, 1, 4, 32>(a);
    return hipErrorInvalidValue;
}

}  // namespace mqa
