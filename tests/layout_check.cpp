// CPU check of the lane/LDS index maps in csrc/layout.hpp (built with g++).
// Prints "ok" or the first violated property and exits non-zero.
#include <cstdio>
#include <set>
#include <vector>
#include "../attention_mqa_gqa_amd/csrc/layout.hpp"
using namespace mqa::layout;

static int fail(const char* what, int a, int b) { std::printf("FAIL %s (%d, %d)\n", what, a, b); return 1; }

int main() {
    // 1. 32x32x16 maps: accumulator (h, i) is row 8(i/4)+4h+i%4 of the A operand,
    //    i.e. key swap23(row); the two lane halves cover each 16-key step.
    for (int h = 0; h < 2; ++h)
        for (int i = 0; i < 16; ++i)
            if (c32_index(h, i) != swap23(8 * (i / 4) + 4 * h + (i % 4))) return fail("c32", h, i);
    for (int ks = 0; ks < 2; ++ks) {
        std::set<int> keys;
        for (int h = 0; h < 2; ++h)
            for (int j = 0; j < 8; ++j) keys.insert(c32_index(h, 8 * ks + j));
        if ((int)keys.size() != 16 || *keys.begin() != 16 * ks) return fail("c32 kstep", ks, 0);
    }
    // 2. 32-row operand reads: 8-lane groups hit 8 distinct slots of 128 B and
    //    16-lane groups 16 distinct slots of 256 B.
    auto grp_ok = [](auto addr) {
        for (int grp : {8, 16}) {
            for (int base = 0; base < 64; base += grp) {
                std::set<long> s;
                for (int l = base; l < base + grp; ++l) s.insert((addr(l) / 16) % grp);
                if ((int)s.size() != grp) return false;
            }
        }
        return true;
    };
    for (int rc : {4, 8, 16, 24, 64}) {
        for (int blk = 0; blk < 16; ++blk)
            for (int ks = 0; ks < rc / 2; ++ks) {
                auto addr = [&](int l) {
                    int r = 32 * blk + swap23(l % 32);
                    int c = 2 * ks + l / 32;
                    return ((long)r * rc + (c ^ swz32(r, rc))) * 16;
                };
                if (!grp_ok(addr)) return fail("32-row reads", rc, ks);
            }
        for (int r = 0; r < 512; ++r) {
            std::set<int> s;
            for (int c = 0; c < rc; ++c) s.insert(c ^ swz32(r, rc));
            if ((int)s.size() != rc || *s.rbegin() != rc - 1) return fail("swz32 bijection", rc, r);
            // each chunk stays inside its aligned swizzle group
            const int gs = swz32_group(rc);
            for (int c = 0; c < rc; ++c)
                if ((c ^ swz32(r, rc)) / gs != c / gs) return fail("swz32 group", rc, r);
        }
    }
    // 3. Padded 1 KB rows: lane l reads row position l % 32 (key
    //    swap23(l % 32)), chunk 2 ks + l / 32.
    for (int ks = 0; ks < 32; ++ks) {
        auto addr = [&](int l) { return (long)(l % 32) * padded_row_bytes(1024) + (2 * ks + l / 32) * 16; };
        if (!grp_ok(addr)) return fail("padded reads", ks, 0);
    }
    for (int r = 0; r < 64; ++r)
        if (padded_row_pos(padded_row_pos(r)) != r || padded_row_pos(r) / 32 != r / 32) return fail("padded pos", r, 0);
    // 4. MLA tiles: latent score reads (lane l: row l % 32, chunk 2 ks + l / 32),
    //    RoPE reads, P^T operand reads (row = head 32 nt + l % 32) and the
    //    transposing 64-bit V^T reads (16-lane groups: 4 rows x 32 bytes).
    {
        std::set<int> pos;
        for (int k = 0; k < 32; ++k) pos.insert(mla_lat_pos(k));
        if ((int)pos.size() != 32 || *pos.rbegin() != 31) return fail("mla_lat_pos bijection", 0, 0);
        for (int r = 0; r < 32; ++r) {
            std::set<int> c8, c4;
            for (int c = 0; c < 8; ++c) c8.insert(c ^ mla_rope_swz(r));
            for (int c = 0; c < 4; ++c) c4.insert(c ^ ptile_swz(r));
            if (c8.size() != 8 || *c8.rbegin() != 7 || c4.size() != 4 || *c4.rbegin() != 3) return fail("mla swz bijection", r, 0);
        }
        for (int ks = 0; ks < 32; ++ks) {
            auto addr = [&](int l) { return (long)mla_lat_pos(l % 32) * padded_row_bytes(1024) + (2 * ks + l / 32) * 16; };
            if (!grp_ok(addr)) return fail("mla latent reads", ks, 0);
        }
        for (int j = 0; j < 4; ++j) {
            auto addr = [&](int l) { int r = l % 32; return (long)r * 128 + (((2 * j + l / 32) ^ mla_rope_swz(r)) * 16); };
            if (!grp_ok(addr)) return fail("mla rope reads", j, 0);
        }
        for (int nt = 0; nt < 4; ++nt)
            for (int kp = 0; kp < 2; ++kp) {
                auto addr = [&](int l) { int h = 32 * nt + l % 32; return (long)h * 64 + (((2 * kp + l / 32) ^ ptile_swz(h)) * 16); };
                if (!grp_ok(addr)) return fail("P reads", nt, kp);
            }
        // tr reads: group q, lane j = 4s + a reads row 16kp + 8(q/2) + 4r + s,
        // bytes 2 (128 w + 32 mt + 16 (q % 2) + 4 a) .. +8; the 16 lanes of a
        // group must cover 32 distinct 4-byte banks (of 32)
        for (int w = 0; w < 4; ++w)
            for (int mt = 0; mt < 4; ++mt)
                for (int kp = 0; kp < 2; ++kp)
                    for (int r = 0; r < 2; ++r)
                        for (int q = 0; q < 4; ++q) {
                            std::set<int> banks;
                            for (int j = 0; j < 16; ++j) {
                                int srow = j >> 2, a = j & 3;
                                int key = 16 * kp + 8 * (q >> 1) + 4 * r + srow;
                                long addr = (long)mla_lat_pos(key) * padded_row_bytes(1024) + 2 * (128 * w + 32 * mt + 16 * (q & 1) + 4 * a);
                                banks.insert((int)((addr / 4) % 32));
                                banks.insert((int)((addr / 4 + 1) % 32));
                            }
                            if (banks.size() != 32) return fail("tr reads", mt, q);
                        }
    }
    std::printf("ok\n");
    return 0;
}
