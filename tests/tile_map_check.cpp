// Host check of the tiled kernel's work split and LDS layout (tile_split and
// tile_word in ecmd_tape.h), for the tile shapes given on the command line as
// TM TN TB triples.  For each shape it checks:
//   * the output-chunk split and the staging split each cover every 4-element
//     group of the tile exactly once and stay inside the tile;
//   * tile_word maps the tile's TM x TN elements one to one onto TM * TN words;
//   * under gfx950's LDS model for wave64 four-byte accesses (32 banks, each
//     half-wavefront served on its own, bank = word mod 32) no half-wavefront
//     of the staging writes or of the chunk reads has two lanes on one bank
//     with different words.
// Prints one line per shape and exits non-zero on the first failure.
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "ecmd_tape.h"

using ecmd::tile_split;
using ecmd::tile_word;

static int fail(int tm, int tn, int tb, const char *what)
{
    std::printf("FAIL %dx%dx%d: %s\n", tm, tn, tb, what);
    return 1;
}

// Largest number of distinct words that share one bank within any
// half-wavefront, for words[item] (item = work-item + TB * j).
static int worst_conflict(const std::vector<int> &words)
{
    int worst = 1;
    const int items = (int)words.size();
    for (int base = 0; base < items; base += 32) {
        // items base..base+31 are one half-wavefront when TB is a multiple of 64
        std::vector<std::vector<int>> bank(32);
        for (int l = 0; l < 32 && base + l < items; ++l) {
            const int w = words[base + l];
            auto &b = bank[w & 31];
            bool seen = false;
            for (int x : b) seen = seen || x == w;   // one word read by two lanes is a broadcast
            if (!seen) b.push_back(w);
        }
        for (auto &b : bank)
            if ((int)b.size() > worst) worst = (int)b.size();
    }
    return worst;
}

static int check(int tm, int tn, int tb)
{
    const int vecs = tm * tn / 4;
    if (tm % 32 || tn % 32 || tb % 64 || vecs % tb) return fail(tm, tn, tb, "shape not supported by the split");
    // Splits: (row, 4 columns) chunks and (column, 4 rows) staging vectors.
    std::vector<int> seen_chunk(vecs, 0), seen_stage(vecs, 0), seen_word(tm * tn, 0);
    for (int v = 0; v < vecs; ++v) {
        int r, c;
        tile_split(v, tn, r, c);
        if (r < 0 || r >= tm || c < 0 || c + 3 >= tn || c % 4) return fail(tm, tn, tb, "chunk outside the tile");
        ++seen_chunk[r * (tn / 4) + c / 4];
        int sc, sr;
        tile_split(v, tm, sc, sr);
        if (sc < 0 || sc >= tn || sr < 0 || sr + 3 >= tm || sr % 4) return fail(tm, tn, tb, "staging vector outside the tile");
        ++seen_stage[sc * (tm / 4) + sr / 4];
    }
    for (int k = 0; k < vecs; ++k)
        if (seen_chunk[k] != 1 || seen_stage[k] != 1) return fail(tm, tn, tb, "split not one to one");
    for (int c = 0; c < tn; ++c)
        for (int r = 0; r < tm; ++r) {
            const int w = tile_word(tm, c, r);
            if (w < 0 || w >= tm * tn) return fail(tm, tn, tb, "LDS word out of range");
            ++seen_word[w];
        }
    for (int w = 0; w < tm * tn; ++w)
        if (seen_word[w] != 1) return fail(tm, tn, tb, "LDS layout not one to one");
    // Bank conflicts.  Item order: work-item t of pass j is item t + TB * j;
    // a pass is one instruction of every wavefront, so half-wavefronts are
    // 32-aligned runs of items.
    int worst_w = 0, worst_r = 0;
    for (int e = 0; e < 4; ++e) {
        std::vector<int> wr(vecs), rd(vecs);
        for (int v = 0; v < vecs; ++v) {
            int sc, sr, r, c;
            tile_split(v, tm, sc, sr);
            wr[v] = tile_word(tm, sc, sr + e);
            tile_split(v, tn, r, c);
            rd[v] = tile_word(tm, c + e, r);
        }
        const int a = worst_conflict(wr), b = worst_conflict(rd);
        worst_w = a > worst_w ? a : worst_w;
        worst_r = b > worst_r ? b : worst_r;
    }
    std::printf("%dx%dx%d: staging writes %d-way, chunk reads %d-way\n", tm, tn, tb, worst_w, worst_r);
    if (worst_w != 1 || worst_r != 1) return fail(tm, tn, tb, "bank conflict");
    return 0;
}

// The bank model itself, on the layout the tiled kernel used before the
// swizzle: a whole-wavefront row or column run per split and a column pitch
// of TM + 1 words.  rocprofv3 measured SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE
// at 50% for 64 x 64 tiles and 60% for 32 x 256 ones on that layout; the
// model must give the conflict degrees that explain those figures: 2-way
// writes and reads (1 extra cycle of 2), and conflict-free writes with 4-way
// reads (3 extra cycles of 5).
static int check_model()
{
    struct Case { int tm, tn, want_w, want_r; } cases[] = {{64, 64, 2, 2}, {32, 256, 1, 4}};
    for (const Case &k : cases) {
        const int vecs = k.tm * k.tn / 4;
        int ww = 0, wr = 0;
        for (int e = 0; e < 4; ++e) {
            std::vector<int> w(vecs), r(vecs);
            for (int v = 0; v < vecs; ++v) {
                const int sc = v / (k.tm / 4), sr = 4 * (v % (k.tm / 4));
                w[v] = sc * (k.tm + 1) + sr + e;
                const int rr = v / (k.tn / 4), cc = 4 * (v % (k.tn / 4));
                r[v] = (cc + e) * (k.tm + 1) + rr;
            }
            const int a = worst_conflict(w), b = worst_conflict(r);
            ww = a > ww ? a : ww;
            wr = b > wr ? b : wr;
        }
        std::printf("model, padded pitch %dx%d: writes %d-way, reads %d-way\n", k.tm, k.tn, ww, wr);
        if (ww != k.want_w || wr != k.want_r) return fail(k.tm, k.tn, 0, "bank model disagrees with the measured layout");
    }
    return 0;
}

int main(int argc, char **argv)
{
    if (check_model()) return 1;
    if (argc < 4 || (argc - 1) % 3) {
        std::fprintf(stderr, "usage: %s TM TN TB [TM TN TB ...]\n", argv[0]);
        return 2;
    }
    for (int i = 1; i < argc; i += 3)
        if (check(std::atoi(argv[i]), std::atoi(argv[i + 1]), std::atoi(argv[i + 2]))) return 1;
    return 0;
}
