// Host check of the tiled kernel's work split and LDS layout (tile_split and
// tile_word in ecmd_tape.h; for 16-bit tiles tile_split8 and tile_pair_word,
// two elements per word), for the tile shapes given on the command line as
// TM TN TB triples (after "-8": shapes of 8-element vectors).  For each shape
// it checks:
//   * the output-chunk split and the staging split each cover every 4-element
//     (8-element) group of the tile exactly once and stay inside the tile;
//   * the layout maps the tile's TM x TN elements (TM x TN / 2 pairs) one to
//     one onto TM * TN (TM * TN / 2) words;
//   * under gfx950's LDS model for wave64 four-byte accesses (32 banks, each
//     half-wavefront served on its own, bank = word mod 32) no half-wavefront
//     of the staging writes or of the chunk reads has two lanes on one bank
//     with different words.
// Prints one line per shape and exits non-zero on the first failure.
#include <cstdio>
#include <cstdlib>
#include <string>
#include <vector>

#include "ecmd_tape.h"

// The split and layout for vectors of V elements.
template <int V>
static void split(int v, int minor_len, int &major, int &minor)
{
    if constexpr (V == 4) ecmd::tile_split(v, minor_len, major, minor);
    else ecmd::tile_split8(v, minor_len, major, minor);
}

// The LDS word holding element (column c, row r), for the element layout
// (V = 4) or the pair layout (V = 8).
template <int V>
static int word(int tm, int c, int r)
{
    if constexpr (V == 4) return ecmd::tile_word(tm, c, r);
    else return ecmd::tile_pair_word(tm, c, r >> 1);
}

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

template <int V>
static int check(int tm, int tn, int tb)
{
    const int vecs = tm * tn / V;
    const int unit = 8 * V;      // minor extent of a half-wavefront
    if (tm % unit || tn % unit || tb % 64 || vecs % tb) return fail(tm, tn, tb, "shape not supported by the split");
    // Splits: (row, V columns) chunks and (column, V rows) staging vectors.
    const int per_word = V == 8 ? 2 : 1, words = tm * tn / per_word;
    std::vector<int> seen_chunk(vecs, 0), seen_stage(vecs, 0), seen_word(words, 0);
    for (int v = 0; v < vecs; ++v) {
        int r, c;
        split<V>(v, tn, r, c);
        if (r < 0 || r >= tm || c < 0 || c + V - 1 >= tn || c % V) return fail(tm, tn, tb, "chunk outside the tile");
        ++seen_chunk[r * (tn / V) + c / V];
        int sc, sr;
        split<V>(v, tm, sc, sr);
        if (sc < 0 || sc >= tn || sr < 0 || sr + V - 1 >= tm || sr % V)
            return fail(tm, tn, tb, "staging vector outside the tile");
        ++seen_stage[sc * (tm / V) + sr / V];
    }
    for (int k = 0; k < vecs; ++k)
        if (seen_chunk[k] != 1 || seen_stage[k] != 1) return fail(tm, tn, tb, "split not one to one");
    for (int c = 0; c < tn; ++c)
        for (int r = 0; r < tm; r += per_word) {
            const int w = word<V>(tm, c, r);
            if (w < 0 || w >= words) return fail(tm, tn, tb, "LDS word out of range");
            if (per_word == 2 && word<V>(tm, c, r + 1) != w) return fail(tm, tn, tb, "a pair split over two words");
            ++seen_word[w];
        }
    for (int w = 0; w < words; ++w)
        if (seen_word[w] != 1) return fail(tm, tn, tb, "LDS layout not one to one");
    // Bank conflicts.  Item order: work-item t of pass j is item t + TB * j;
    // a pass is one instruction of every wavefront, so half-wavefronts are
    // 32-aligned runs of items.
    // Staging writes: one word per element (V = 4) or per pair of rows (V = 8:
    // word e holds rows 2e, 2e + 1 of the vector); chunk reads: one word per
    // element either way.
    int worst_w = 0, worst_r = 0;
    for (int e = 0; e < V; ++e) {
        std::vector<int> wr(vecs), rd(vecs);
        for (int v = 0; v < vecs; ++v) {
            int sc, sr, r, c;
            split<V>(v, tm, sc, sr);
            wr[v] = word<V>(tm, sc, sr + (V == 8 ? 2 * (e % 4) : e));
            split<V>(v, tn, r, c);
            rd[v] = word<V>(tm, c + e, r);
        }
        const int a = worst_conflict(wr), b = worst_conflict(rd);
        worst_w = a > worst_w ? a : worst_w;
        worst_r = b > worst_r ? b : worst_r;
    }
    std::printf("%s%dx%dx%d: staging writes %d-way, chunk reads %d-way\n", V == 8 ? "8-element " : "", tm, tn, tb,
                worst_w, worst_r);
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
    bool eight = false;
    int shapes = 0;
    for (int i = 1; i < argc;) {
        if (std::string(argv[i]) == "-8") {
            eight = true;
            ++i;
            continue;
        }
        if (i + 2 >= argc) break;
        const int tm = std::atoi(argv[i]), tn = std::atoi(argv[i + 1]), tb = std::atoi(argv[i + 2]);
        if (eight ? check<8>(tm, tn, tb) : check<4>(tm, tn, tb)) return 1;
        ++shapes;
        i += 3;
    }
    if (shapes == 0) {
        std::fprintf(stderr, "usage: %s TM TN TB [TM TN TB ...] [-8 TM TN TB ...]\n", argv[0]);
        return 2;
    }
    return 0;
}
