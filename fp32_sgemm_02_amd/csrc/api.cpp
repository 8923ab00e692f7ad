// api.cpp -- the C ABI of include/fp32_sgemm.h: argument validation, the
// special cases, choice of kernel family and tile, and the launch.
//
// The operation and its argument list follow the SGEMM definition and kernel
// signature of "a CUDA matmul" (plasmient.com labs) sections 00 and 02,
// extended with BLAS leading dimensions and a stream.  Launch geometry is the
// ceiling-division grid of that page's section 02, so shapes that are not tile
// multiples are covered, with edge guards in the kernels ("The 1% kernel"
// section 6: idle threads past the matrix).
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "gemm_internal.hpp"

namespace sg {
namespace {

constexpr int kVersion = 500;   // 0.5.0
constexpr int kBadConfig = -13;
constexpr int kBadTransA = -21;
constexpr int kBadTransB = -22;
constexpr int kBadOrder = -23;
constexpr int kBadBias = -24;
constexpr int kBadAct = -25;
constexpr int kBadStrideA = -26;
constexpr int kBadStrideB = -27;
constexpr int kBadStrideC = -28;
constexpr int kBadBatch = -29;
constexpr int kBadDtype = -30;
constexpr int kBadScratch = -31;

// A status of the row-major call that serves a column-major one (operands
// swapped, M and N swapped), renamed after the caller's arguments.
int colmajor_status(int st) {
    switch (st) {
    case -1: return -2;
    case -2: return -1;
    case -5: return -7;
    case -6: return -8;
    case -7: return -5;
    case -8: return -6;
    case kBadTransA: return kBadTransB;
    case kBadTransB: return kBadTransA;
    default: return st;
    }
}

bool aligned4(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// 16-byte vector I/O needs every row start of A, B and C (of every batch
// entry) on a 16-byte boundary ("The GEMM Scrapbook", vectorisation chapter:
// 128-bit accesses need 16-byte alignment).
bool vector_io_ok(const Problem &p) {
    return rows_aligned(p.A, p.lda, p.stride_a, p.batch, 4) &&
           rows_aligned(p.B, p.ldb, p.stride_b, p.batch, 4) &&
           rows_aligned(p.C, p.ldc, p.stride_c, p.batch, 4);
}

struct Tuned {
    int variant, tile, group_m;
};

#include "tuned_table.inc"

long long tiles_for(const TileEntry &t, int M, int N) {
    return (long long)((M + t.desc.bm - 1) / t.desc.bm) * ((N + t.desc.bn - 1) / t.desc.bn);
}

// The MFMA family: the general tiles, then the direct-load tiles for
// untransposed A, then those for transposed A, in one table; the direct-load
// tiles get their fused-epilogue and stream-K launchers (compiled separately,
// same order).
const TileEntry *mfma_family(int *count) {
    static const std::vector<TileEntry> all = [] {
        std::vector<TileEntry> v;
        int n = 0, nf = 0;
        const TileEntry *t = mfma_tiles(&n);
        v.insert(v.end(), t, t + n);
        const LaunchFn *f = nullptr;
        t = mfma_direct_tiles(&n);
        f = mfma_direct_epi_launchers(&nf);
        int nsk = 0;
        const LaunchFn *sk = mfma_direct_sk_launchers(&nsk);
        for (int i = 0; i < n; ++i) {
            v.push_back(t[i]);
            if (nf == n) v.back().fused = f[i];
            if (nsk == n && sk[i]) {
                v.back().streamk = sk[i];
                v.back().desc.flags |= SGEMM_TILE_STREAMK;
            }
        }
        t = mfma_direct_ta_tiles(&n);
        f = mfma_direct_ta_epi_launchers(&nf);
        sk = mfma_direct_ta_sk_launchers(&nsk);
        for (int i = 0; i < n; ++i) {
            v.push_back(t[i]);
            if (nf == n) v.back().fused = f[i];
            if (nsk == n && sk[i]) {
                v.back().streamk = sk[i];
                v.back().desc.flags |= SGEMM_TILE_STREAMK;
            }
        }
        return v;
    }();
    *count = (int)all.size();
    return all.data();
}

// Whether tile t can run this problem: whole-tile tiles need whole tiles and
// 16-byte I/O for every operand (io_ok), direct-load tiles need their 31-bit
// panel offsets to fit.
bool tile_applies(const TileEntry &t, const Problem &p, bool io_ok) {
    if ((p.trans_a != 0) != ((t.desc.flags & SGEMM_TILE_TRANS_A) != 0)) return false;
    if (p.trans_b && !(t.desc.flags & SGEMM_TILE_TRANS_B)) return false;
    if (t.desc.flags & SGEMM_TILE_WHOLE)
        return io_ok && direct_applies(p, t.desc.bm, t.desc.bn, t.desc.bk, false);
    if (t.desc.flags & SGEMM_TILE_DIRECT)
        return direct_applies(p, t.desc.bm, t.desc.bn, t.desc.bk, true);
    return true;
}

const TileEntry *family(int variant, int *count) {
    switch (variant) {
    case SGEMM_VARIANT_MFMA: return mfma_family(count);
    case SGEMM_VARIANT_VALU: return valu_tiles(count);
    case SGEMM_VARIANT_SKINNY: return skinny_tiles(count);
    case SGEMM_VARIANT_SMALL: return small_tiles(count);
    default: *count = 0; return nullptr;
    }
}

// Argument checks; codes follow sgemm's parameter list (a transposed operand
// is stored K x M (A) or N x K (B), so its leading dimension covers M or K).
int validate(int M, int N, int K, float alpha, const float *A, int lda, const float *B, int ldb,
             float *C, int ldc, int trans_a = 0, int trans_b = 0) {
    if (M < 0) return -1;
    if (N < 0) return -2;
    if (K < 0) return -3;
    const int a_cols = trans_a ? M : K, b_cols = trans_b ? K : N;
    if (lda < (a_cols > 1 ? a_cols : 1)) return -6;
    if (ldb < (b_cols > 1 ? b_cols : 1)) return -8;
    if (ldc < (N > 1 ? N : 1)) return -11;
    if (M == 0 || N == 0) return 0;
    const bool reads_ab = (alpha != 0.f) && K > 0;
    if (reads_ab && (!A || !aligned4(A))) return -5;
    if (reads_ab && (!B || !aligned4(B))) return -7;
    if (!C || !aligned4(C)) return -10;
    return 0;
}

int to_status(hipError_t e) { return e == hipSuccess ? 0 : static_cast<int>(e); }

// The general MFMA tile for a shape: the largest tile that still yields
// about one workgroup per CU.  The fallback when a chosen direct-load tile
// cannot run (it always can).
int general_mfma_tile(int M, int N) {
    int count = 0;
    const TileEntry *tiles = mfma_tiles(&count);
    const int order[] = {2, 5, 7};
    for (int idx : order)
        if (idx < count && tiles_for(tiles[idx], M, N) >= 200) return idx;
    return 7;
}

constexpr int kCUs = 256;
constexpr double kPeakFlops = 157.3e12;   // fp32 MFMA, dense

// A tile of one k-group whose waves own fewer than 64 x 128 outputs each,
// running alone on its CU (at most one workgroup per CU: two waves per SIMD),
// covers less of its loads' latency than at 4096^3, where its efficiency was
// measured with several workgroups per CU.  Graph-replayed, the 8-wave
// 128 x 128 tile of 32 x 64 wave tiles ran 3.4-6.5 % behind the k-group tiles
// on products that give it exactly one round (4096 x 1000 x 3001, 4096 x
// 1024 x 4096, 2048 x 2048 x 4096, 1024 x 4096 x 4096, 4096 x 1000 x 1000)
// and ahead of them from two rounds on (4096 x 2048 x 4096, 2816^3).
constexpr double kLoneWorkgroupPenalty = 1.05;

// Estimated time of tile t on `batch` M x N outputs: rounds of workgroups
// over the 256 CUs, each round costing one tile's work at the tile's measured
// efficiency.  Rounding up to whole rounds is what makes a 4097-row product
// with 256-row tiles cost as much as a 4352-row one.
double tile_cost(const TileEntry &t, int M, int N, int batch = 1) {
    const long long n = tiles_for(t, M, N) * batch;
    const long long rounds = (n + kCUs - 1) / kCUs;
    double c = (double)rounds * t.desc.bm * t.desc.bn / (t.eff_pct > 0 ? t.eff_pct : 50);
    const sgemm_tile_desc &d = t.desc;
    if (n <= kCUs && d.wm > 0 && d.wn > 0 && d.wm * d.wn < 64 * 128 &&
        d.threads / 64 == (d.bm / d.wm) * (d.bn / d.wn))   // one k-group
        c *= kLoneWorkgroupPenalty;
    return c;
}

// Edge strips.  When a tile leaves at most 16 rows (or columns) past its last
// whole tile row (column) and those cost a whole extra round of workgroups,
// the strip can go to the skinny family instead (few rows: the MFMA strip
// kernel; few columns: the row-streaming kernel).  Returns the rows / columns
// split off (0: none).
struct Strips {
    int rows, cols;
};

Strips edge_strips(const Problem &p, const TileEntry &t) {
    Strips s{0, 0};
    const int bm = t.desc.bm, bn = t.desc.bn;
    const int mr = p.M % bm, nr = p.N % bn;
    const long long tn = (p.N + bn - 1) / bn, tm = (p.M + bm - 1) / bm;
    auto rounds = [](long long tiles) { return (tiles + kCUs - 1) / kCUs; };
    if (mr > 0 && mr <= 16 && p.M > bm && rounds(tm * tn) > rounds((tm - 1) * tn)) s.rows = mr;
    const long long tm2 = (p.M - s.rows + bm - 1) / bm;
    if (nr > 0 && nr <= 16 && p.N > bn && rounds(tm2 * tn) > rounds(tm2 * (tn - 1))) s.cols = nr;
    return s;
}

Problem main_part(const Problem &p, Strips s) {
    Problem m = p;
    m.M -= s.rows;
    m.N -= s.cols;
    return m;
}

// Stream-K (the tile's persistent runs over evenly split k-iterations, plus
// a fixup; for a batch, persistent runs over the whole tiles of all entries):
// its launcher serves A and B that take dwordx4 loads.  Estimated time, in the units of tile_cost: the whole rounds before
// the split wave plus each workgroup's share of the split iterations, and the
// partial sums (written and read once, at about 4 TB/s) with the second
// launch (about 4 us).
bool streamk_ok(const Problem &p) {
    return rows_aligned(p.A, p.lda, p.stride_a, p.batch, 4) &&
           rows_aligned(p.B, p.ldb, p.stride_b, p.batch, 4) &&
           (p.trans_a ? p.M : p.K) % 4 == 0 && (p.trans_b ? p.K : p.N) % 4 == 0;
}

// Workspace bytes (after the counters) of a stream-K launch of tile t: two
// tile accumulators for each of the 256 persistent workgroups (none for a
// batch, which runs whole tiles only).
size_t streamk_workspace_bytes(const TileEntry &t, const Problem &p) {
    return p.batch > 1 ? 0 : (size_t)2 * 256 * 4 * t.desc.bm * t.desc.bn;
}

double streamk_cost(const TileEntry &t, const Problem &p) {
    const long long tiles = tiles_for(t, p.M, p.N);
    const long long iters = (p.K + t.desc.bk - 1) / t.desc.bk;
    const long long dp = tiles >= kCUs ? (tiles / kCUs - 1) * kCUs : 0;
    const long long sk = tiles - dp;
    const long long share = (sk * iters + kCUs - 1) / kCUs;
    const double eff = t.eff_pct > 0 ? t.eff_pct : 50;
    const double rounds = (double)dp / kCUs + (double)share / iters;
    // seconds per cost unit: one round of tiles at `eff` % of the peak
    const double unit_s = 2.0 * p.K * kCUs * 100.0 / kPeakFlops;
    const long long partials = sk < kCUs ? sk + kCUs : 2 * kCUs;
    const double extra_s = 2.0 * partials * t.desc.bm * t.desc.bn * 4 / 4e12 + 4e-6;
    return rounds * t.desc.bm * t.desc.bn / eff + extra_s / unit_s;
}

// The MFMA tile for a shape that is not in the tuned table: the applicable
// tile of least estimated time (ties: the earlier, i.e. general, tile),
// counting for each tile the option of handing its edge strips to the skinny
// family (`strips`, when not null, receives the chosen tile's strips; a strip
// is charged 5 % of the main part, far below the round it saves) and, where
// the tile offers it, stream-K (`*streamk` set when chosen).
int default_mfma_tile(const Problem &p, bool io_ok, Strips *strips = nullptr,
                      bool *streamk = nullptr) {
    int count = 0;
    const TileEntry *tiles = mfma_family(&count);
    const bool trans = p.trans_a || p.trans_b;
    int best = trans ? -1 : general_mfma_tile(p.M, p.N);   // -1: nothing applies
    double best_cost = trans ? 1e300 : tile_cost(tiles[best], p.M, p.N, p.batch);
    Strips best_strips{0, 0};
    if (p.trans_a) strips = nullptr;   // the few-columns strip kernel reads A untransposed
    for (int i = 0; i < count; ++i) {
        const Strips sp = strips ? edge_strips(p, tiles[i]) : Strips{0, 0};
        const Problem m = main_part(p, sp);
        if (!tile_applies(tiles[i], m, io_ok)) continue;
        double c = tile_cost(tiles[i], m.M, m.N, p.batch);
        if (sp.rows || sp.cols) c *= 1.05;
        if (c < best_cost) {
            best = i;
            best_cost = c;
            best_strips = sp;
            if (streamk) *streamk = false;
        }
        // (with a caller's scratch: only where its workspace fits)
        if (streamk && tiles[i].streamk && io_ok && streamk_ok(p) &&
            tile_applies(tiles[i], p, io_ok) &&
            (!p.scratch || streamk_workspace_bytes(tiles[i], p) <= p.scratch_bytes) &&
            (p.batch == 1 || (p.K <= 256 && tiles_for(tiles[i], p.M, p.N) * p.batch >= 2 * kCUs))) {
            // a batch runs persistent whole tiles: measured 3-5 % faster than
            // one workgroup per tile when K is short and tiles span several
            // waves (a tile's stores drain under the next tile's loads)
            const double cs = p.batch == 1 ? streamk_cost(tiles[i], p)
                                           : 0.96 * tile_cost(tiles[i], p.M, p.N, p.batch);
            if (cs < best_cost) {
                best = i;
                best_cost = cs;
                best_strips = Strips{0, 0};
                *streamk = true;
            }
        }
    }
    // Short K (at most 256) with A untransposed, C at least 256 x 256 and two
    // or more rounds of 128 x 128 tiles that fill at least 85 % of their last
    // round and of their area: the 8-wave 128 x 128 tile, measured fastest there (batched attention scores
    // 32 x 2048 x 2048 x 128: 308 us against 321 for the cost model's pick;
    // 8192^2 x 64..256: 3-13 %; 5632^2 x 256: 2-4 %).  At short K the
    // per-workgroup cost of the first loads and of the C store weighs more
    // than the 4096^3 efficiencies of the table.  (The 4-wave 128 x 128 tile
    // of 64 x 64 wave tiles measures within 4 % of it either way at K <= 64.)
    if (!p.trans_a && p.K <= 256) {
        for (int i = 0; i < count; ++i) {
            const sgemm_tile_desc &d = tiles[i].desc;
            if (!((d.flags & SGEMM_TILE_DIRECT) && !(d.flags & SGEMM_TILE_TRANS_A) && d.bm == 128 &&
                  d.bn == 128 && d.bk == 16 && d.wm == 32 && d.wn == 64))
                continue;
            const long long n = tiles_for(tiles[i], p.M, p.N) * p.batch;
            const long long rounds = (n + kCUs - 1) / kCUs;
            const double fill = (double)p.M * p.N * p.batch / ((double)n * 128 * 128);
            if (tile_applies(tiles[i], p, io_ok) && p.M >= 256 && p.N >= 256 && rounds >= 2 &&
                n * 100 >= 85 * rounds * kCUs && fill >= 0.85) {
                best = i;
                best_strips = Strips{0, 0};
                if (streamk) *streamk = false;
                break;
            }
        }
    }
    if (strips) *strips = best_strips;
    return best;
}

// Automatic choice (in resolve): the measured best configuration for this
// exact shape (tuned_table.inc; single products only), else the skinny family
// for memory-bound shapes, else the MFMA tile of least estimated time,
// possibly with edge strips split off.  A choice that cannot run on the
// actual operands falls back to the general rule.

// The configuration a call runs with: explicit (sgemm_ex) or automatic, with
// an automatic choice that cannot run on these operands replaced by the
// general rule.  `vec` selects the tile's 16-byte-capable launcher (general
// tiles: every operand allows 16-byte I/O; direct-load tiles decide per
// operand themselves) unless 4-byte I/O is asked for.  Returns 0 or kBadConfig.
struct Choice {
    int variant, tile, group_m;
    bool vec;
    bool streamk = false;
};

int resolve(const Problem &p, const sgemm_config *cfg, Choice &out, Strips *strips = nullptr) {
    const int flags = cfg ? cfg->flags : 0;
    const bool want_vec = !(flags & SGEMM_FLAG_SCALAR_IO);
    const bool io_ok = want_vec && vector_io_ok(p);
    int variant = cfg ? cfg->variant : SGEMM_VARIANT_AUTO;
    int tile = cfg ? cfg->tile : -1;
    int group_m = cfg ? cfg->group_m : 0;
    if (variant < 0 || variant >= SGEMM_VARIANT_COUNT) return kBadConfig;
    const bool explicit_tile = (variant != SGEMM_VARIANT_AUTO) && tile >= 0;
    if (strips) *strips = Strips{0, 0};
    const bool trans = p.trans_a || p.trans_b;
    if (trans && variant == SGEMM_VARIANT_VALU) return kBadConfig;   // VALU reads untransposed
    bool streamk = (flags & SGEMM_FLAG_STREAMK) != 0;
    if (streamk && !explicit_tile) return kBadConfig;   // stream-K is asked for with a tile
    if (variant == SGEMM_VARIANT_AUTO) {
        Tuned a;
        if (trans || (flags & SGEMM_FLAG_UNTUNED) || p.batch > 1 ||
            !lookup_tuned(p.M, p.N, p.K, a)) {
            const int small = small_pick(p);
            if (small >= 0 && small_tiny_batch(p))
                a = Tuned{SGEMM_VARIANT_SMALL, small, 0};
            else if (skinny_pick(p) >= 0)
                a = Tuned{SGEMM_VARIANT_SKINNY, -1, 0};
            else if (small >= 0)
                a = Tuned{SGEMM_VARIANT_SMALL, small, 0};
            else
                a = Tuned{SGEMM_VARIANT_MFMA, default_mfma_tile(p, io_ok, strips, &streamk), 0};
            if (a.tile < 0 && a.variant == SGEMM_VARIANT_MFMA) return kBadConfig;
        }
        variant = a.variant;
        tile = a.tile;
        if (group_m <= 0) group_m = a.group_m;
    }
    const Problem pm = strips ? main_part(p, *strips) : p;
    int count = 0;
    const TileEntry *tiles = family(variant, &count);
    if (!tiles) return kBadConfig;
    if (variant == SGEMM_VARIANT_SKINNY) {
        if (tile < 0) tile = skinny_pick(p);
        if (!skinny_fits(tile, p)) return kBadConfig;   // shape is not skinny
    } else if (variant == SGEMM_VARIANT_SMALL) {
        if (!small_fits(p)) return kBadConfig;
        if (tile < 0) tile = small_choice(p);
    } else if (tile < 0) {
        tile = (variant == SGEMM_VARIANT_MFMA) ? default_mfma_tile(p, io_ok) : 0;
    }
    if (tile < 0) return kBadConfig;
    if (tile >= count) {
        if (explicit_tile || variant != SGEMM_VARIANT_MFMA || trans) return kBadConfig;
        tile = general_mfma_tile(p.M, p.N);   // a tuned row naming a tile that is not compiled
    }
    // (skinny and small tiles were checked by skinny_fits / small_fits; they
    // serve any transposition of B)
    if (variant != SGEMM_VARIANT_SKINNY && variant != SGEMM_VARIANT_SMALL &&
        !tile_applies(tiles[tile], pm, io_ok)) {
        if (explicit_tile || trans) return kBadConfig;
        tile = general_mfma_tile(p.M, p.N);   // automatic choice that cannot run here
        if (strips) *strips = Strips{0, 0};
        streamk = false;
    }
    if (streamk && (variant != SGEMM_VARIANT_MFMA || !tiles[tile].streamk)) return kBadConfig;
    // direct-load and skinny tiles pick 16-byte paths per operand themselves
    const bool per_operand = (tiles[tile].desc.flags & SGEMM_TILE_DIRECT) ||
                             variant == SGEMM_VARIANT_SKINNY || variant == SGEMM_VARIANT_SMALL;
    const bool vec = per_operand ? want_vec : io_ok;
    if (!(vec ? tiles[tile].vec : tiles[tile].scalar)) return kBadConfig;
    if (streamk && (!vec || !streamk_ok(p))) return kBadConfig;   // (automatic: never so)
    out = Choice{variant, tile, group_m, vec, streamk};
    return 0;
}


// One kernel launch per chunk of at most kMaxBatchPerLaunch batch entries.
// With an epilogue (bias / activation), the tile's fused launcher applies it
// in the kernel's own epilogue when it serves these operands; otherwise the
// product is stored first and an elementwise pass applies it (beta = 1).
int launch(const Problem &p, const Choice &ch, hipStream_t stream) {
    int count = 0;
    const TileEntry &t = family(ch.variant, &count)[ch.tile];
    static const bool log = std::getenv("FP32_SGEMM_LOG") != nullptr;
    const LaunchFn plain = ch.vec ? t.vec : t.scalar;
    const LaunchFn fused = (ch.vec && p.has_epilogue()) ? t.fused : nullptr;
    for (int b0 = 0; b0 < p.batch; b0 += kMaxBatchPerLaunch) {
        Problem q = p;
        q.batch = p.batch - b0 < kMaxBatchPerLaunch ? p.batch - b0 : kMaxBatchPerLaunch;
        q.A += b0 * p.stride_a;
        q.B += b0 * p.stride_b;
        q.C += b0 * p.stride_c;
        hipError_t e = hipErrorNotSupported;
        bool sk_ran = false;
        if (ch.streamk && t.streamk) {
            // stream-K stores the product; an epilogue then takes the elementwise pass
            Problem g = q;
            g.bias = nullptr;
            g.act = SGEMM_ACT_NONE;
            e = t.streamk(g, ch.group_m, stream);   // hipErrorNotSupported: operands it cannot take
            sk_ran = (e != hipErrorNotSupported);
            if (sk_ran && e == hipSuccess && q.has_epilogue()) e = launch_elementwise(q, 1.f, stream);
        }
        if (!sk_ran && fused) e = fused(q, ch.group_m, stream);   // NotSupported: cannot fuse
        const bool done = sk_ran || (fused && e != hipErrorNotSupported);
        if (log)
            std::fprintf(stderr,
                         "sgemm M=%d N=%d K=%d batch=%d variant=%d tile=%d (%dx%dx%d) group_m=%d "
                         "%s%s%s\n",
                         q.M, q.N, q.K, q.batch, ch.variant, ch.tile, t.desc.bm, t.desc.bn,
                         t.desc.bk, ch.group_m, ch.vec ? "vec16" : "scalar",
                         sk_ran ? " stream-k" : "",
                         !q.has_epilogue() ? "" : (done && !sk_ran) ? " fused-epilogue"
                                                                    : " epilogue-pass");
        if (!done) {
            Problem g = q;
            g.bias = nullptr;
            g.act = SGEMM_ACT_NONE;
            e = plain(g, ch.group_m, stream);
            if (e == hipSuccess && q.has_epilogue()) e = launch_elementwise(q, 1.f, stream);
        }
        if (e != hipSuccess) return to_status(e);
    }
    return 0;
}

// Argument checks shared by every entry point, in sgemm's numbering (a
// transposed operand is stored K x M (A) or N x K (B), so its leading
// dimension covers M or K), then those of the batched and epilogue forms.
int validate(const Problem &p) {
    if (p.trans_a != 0 && p.trans_a != 1) return kBadTransA;
    if (p.trans_b != 0 && p.trans_b != 1) return kBadTransB;
    if (p.act < SGEMM_ACT_NONE || p.act > SGEMM_ACT_GELU_TANH) return kBadAct;
    if (p.batch < 0) return kBadBatch;
    if (p.stride_a < 0) return kBadStrideA;
    if (p.stride_b < 0) return kBadStrideB;
    const int st = validate(p.M, p.N, p.K, p.alpha, p.A, (int)p.lda, p.B, (int)p.ldb, p.C,
                            (int)p.ldc, p.trans_a, p.trans_b);
    if (st != 0) return st;
    if (p.M == 0 || p.N == 0 || p.batch == 0) return 0;
    if (p.batch > 1 && p.stride_c < (long long)(p.M - 1) * p.ldc + p.N) return kBadStrideC;
    if (p.bias && !aligned4(p.bias)) return kBadBias;
    return 0;
}

// Workspace bytes (after the counters) that launching choice ch on p takes.
size_t choice_workspace(const Problem &p, const Choice &ch) {
    int count = 0;
    const TileEntry *t = family(ch.variant, &count);
    if (ch.variant == SGEMM_VARIANT_SKINNY) return skinny_workspace_bytes(ch.tile, p, ch.group_m);
    if (ch.streamk && t && ch.tile < count) return streamk_workspace_bytes(t[ch.tile], p);
    return 0;
}

// Validates and runs one call.  The special cases of the reference BLAS:
// nothing to do for an empty C or batch; alpha == 0 or K == 0 leaves
// C = beta * C (plus the epilogue), without reading A or B.  With
// `noalloc`, partial sums take the static scratch array instead of the
// library's workspace: plans are chosen among those whose partial sums fit
// it, and a call whose plan (an explicit configuration) needs more is
// rejected before anything is launched.
int run(Problem p, hipStream_t stream, const sgemm_config *cfg, bool noalloc = false) {
    const int v = validate(p);
    if (v != 0) return v;
    if (p.M == 0 || p.N == 0 || p.batch == 0) return 0;
    if (p.batch == 1) p.stride_a = p.stride_b = p.stride_c = 0;

    if (p.alpha == 0.f || p.K == 0) {
        if (p.beta == 1.f && !p.has_epilogue()) return 0;
        return to_status(launch_elementwise(p, p.beta, stream));
    }
    if (noalloc) {
        const hipError_t e = static_scratch(&p.scratch, &p.scratch_bytes);
        if (e != hipSuccess) return to_status(e);
    }

    Choice ch;
    Strips sp;
    int st = resolve(p, cfg, ch, &sp);
    if (st != 0) return st;
    // the parts of the plan: the main part, the column strip beside it, the
    // row strip below it
    const int m1 = p.M - sp.rows, n1 = p.N - sp.cols;
    Problem cols = p, rows = p;
    Choice ch_cols, ch_rows;
    if (sp.cols) {
        cols.M = m1;
        cols.N = sp.cols;
        cols.B = p.trans_b ? p.B + (long long)n1 * p.ldb : p.B + n1;
        cols.C = p.C + n1;
        if (p.bias) cols.bias = p.bias + n1;
        st = resolve(cols, nullptr, ch_cols);
        if (st != 0) return st;
    }
    if (sp.rows) {
        rows.M = sp.rows;
        rows.A = p.A + (long long)m1 * p.lda;
        rows.C = p.C + (long long)m1 * p.ldc;
        st = resolve(rows, nullptr, ch_rows);
        if (st != 0) return st;
    }
    const Problem main = main_part(p, sp);
    if (p.scratch) {
        if (choice_workspace(main, ch) > p.scratch_bytes ||
            (sp.cols && choice_workspace(cols, ch_cols) > p.scratch_bytes) ||
            (sp.rows && choice_workspace(rows, ch_rows) > p.scratch_bytes))
            return kBadScratch;
    }
    st = launch(main, ch, stream);
    if (st == 0 && sp.cols) st = launch(cols, ch_cols, stream);
    if (st == 0 && sp.rows) st = launch(rows, ch_rows, stream);
    return st;
}

// ---- 16-bit inputs -----------------------------------------------------------
// The 16-bit tile of least estimated time for the word problem pw (the fp32
// cost model over the 16-bit tile list), or -1.
int pick_tile16(const Problem &pw) {
    int best = -1;
    double best_cost = 1e300;
    for (int t = 0; t < tiles16_count(); ++t) {
        const sgemm_tile_desc &d = *tile16_desc(t);
        if (!direct_applies(pw, d.bm, d.bn, d.bk / 2, true)) continue;
        const long long tiles = (long long)((pw.M + d.bm - 1) / d.bm) * ((pw.N + d.bn - 1) / d.bn);
        const double c = (double)((tiles * pw.batch + kCUs - 1) / kCUs) * d.bm * d.bn /
                         tile16_eff(t);
        if (c < best_cost) {
            best = t;
            best_cost = c;
        }
    }
    return best;
}

// C = alpha * op(A) * op(B) + beta * C with A, B 16-bit (dtype) and C fp32.
// Argument checks as sgemm_op's (A and B need 2-byte alignment), -30 for an
// unknown dtype.  The matrix-core tiles serve A untransposed with B
// transposed when K, lda, ldb are even and A, B 4-byte aligned (the operands
// are then word matrices along k), and so does the few-rows skinny kernel
// for M <= 8, or M <= 16 with 16-byte rows of A and B (automatic choice
// only); everything else runs the generic kernel.
int run16(int dtype, int trans_a, int trans_b, int M, int N, int K, float alpha, const void *A,
          int lda, const void *B, int ldb, float beta, float *C, int ldc, hipStream_t stream,
          const sgemm_config *cfg) {
    if (dtype != SGEMM_DTYPE_BF16 && dtype != SGEMM_DTYPE_F16) return kBadDtype;
    if (trans_a != 0 && trans_a != 1) return kBadTransA;
    if (trans_b != 0 && trans_b != 1) return kBadTransB;
    if (M < 0) return -1;
    if (N < 0) return -2;
    if (K < 0) return -3;
    const int a_cols = trans_a ? M : K, b_cols = trans_b ? K : N;
    if (lda < (a_cols > 1 ? a_cols : 1)) return -6;
    if (ldb < (b_cols > 1 ? b_cols : 1)) return -8;
    if (ldc < (N > 1 ? N : 1)) return -11;
    if (M == 0 || N == 0) return 0;
    const bool reads_ab = (alpha != 0.f) && K > 0;
    auto aligned2 = [](const void *q) { return (reinterpret_cast<uintptr_t>(q) & 1u) == 0; };
    if (reads_ab && (!A || !aligned2(A))) return -5;
    if (reads_ab && (!B || !aligned2(B))) return -7;
    if (!C || !aligned4(C)) return -10;
    if (!reads_ab) {
        if (beta == 1.f) return 0;
        Problem p{M, N, K, alpha, beta, nullptr, 1, nullptr, 1, C, ldc};
        return to_status(launch_elementwise(p, beta, stream));
    }
    int variant = cfg ? cfg->variant : SGEMM_VARIANT_AUTO;
    int tile = cfg ? cfg->tile : -1;
    const int group_m = cfg ? cfg->group_m : 0;
    const bool mfma_ok = !trans_a && trans_b && K % 2 == 0 && lda % 2 == 0 && ldb % 2 == 0 &&
                         aligned4(A) && aligned4(B);
    Problem pw{M,   N,   K / 2, alpha, beta, static_cast<const float *>(A), lda / 2,
               static_cast<const float *>(B), ldb / 2, C, ldc};
    pw.trans_b = 1;
    if (variant == SGEMM_VARIANT_AUTO) {
        // few rows in word form: the skinny kernel streams W once; up to 8
        // rows with any word layout, up to 16 where A and W rows take
        // 16-byte loads (the LDS-staged kernel; with 4-byte loads the 64 x 64
        // k-group tile was measured faster at 16 rows)
        const bool staged = pw.K % 4 == 0 && rows_aligned(pw.A, pw.lda, 0, 1, 4) &&
                            rows_aligned(pw.B, pw.ldb, 0, 1, 4);
        if (mfma_ok && (M <= 8 || (M <= 16 && staged)))
            return to_status(launch_skinny16(dtype, pw, stream));
        variant = (mfma_ok && pick_tile16(pw) >= 0) ? SGEMM_VARIANT_MFMA16
                                                    : SGEMM_VARIANT_GENERIC16;
    }
    if (variant == SGEMM_VARIANT_MFMA16) {
        if (!mfma_ok) return kBadConfig;
        if (tile < 0) tile = pick_tile16(pw);
        if (tile < 0 || tile >= tiles16_count()) return kBadConfig;
        const sgemm_tile_desc &d = *tile16_desc(tile);
        if (!direct_applies(pw, d.bm, d.bn, d.bk / 2, true)) return kBadConfig;
        return to_status(launch_tile16(tile, dtype, pw, group_m, stream));
    }
    if (variant == SGEMM_VARIANT_GENERIC16 && tile <= 0) {
        Problem16 q{M,   N,   K, alpha, beta, static_cast<const unsigned short *>(A), lda,
                    static_cast<const unsigned short *>(B), ldb, C, ldc};
        q.trans_a = trans_a;
        q.trans_b = trans_b;
        return to_status(launch_generic16(dtype, q, stream));
    }
    return kBadConfig;
}

// The descriptor of the generic 16-bit kernel (one configuration).
const sgemm_tile_desc kGeneric16Desc{64, 64, 16, 64, 64, 4, 4, 256, 2 * 16 * 65 * 4, 1, 0};

Problem make_problem(int trans_a, int trans_b, int M, int N, int K, float alpha, const float *A,
                     int lda, const float *B, int ldb, float beta, float *C, int ldc) {
    Problem p{M, N, K, alpha, beta, A, lda, B, ldb, C, ldc};
    p.trans_a = trans_a;
    p.trans_b = trans_b;
    return p;
}

}  // namespace
}  // namespace sg

extern "C" {

int sgemm(int M, int N, int K, float alpha, const float *A, int lda, const float *B, int ldb,
          float beta, float *C, int ldc, hipStream_t stream) {
    return sg::run(sg::make_problem(0, 0, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc), stream,
                   nullptr);
}

int sgemm_ex(int M, int N, int K, float alpha, const float *A, int lda, const float *B, int ldb,
             float beta, float *C, int ldc, hipStream_t stream, const sgemm_config *cfg) {
    return sg::run(sg::make_problem(0, 0, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc), stream,
                   cfg);
}

int sgemm_op(int trans_a, int trans_b, int M, int N, int K, float alpha, const float *A,
             int lda, const float *B, int ldb, float beta, float *C, int ldc, hipStream_t stream) {
    return sg::run(sg::make_problem(trans_a, trans_b, M, N, K, alpha, A, lda, B, ldb, beta, C,
                                    ldc),
                   stream, nullptr);
}

int sgemm_op_ex(int trans_a, int trans_b, int M, int N, int K, float alpha, const float *A,
                int lda, const float *B, int ldb, float beta, float *C, int ldc,
                hipStream_t stream, const sgemm_config *cfg) {
    return sg::run(sg::make_problem(trans_a, trans_b, M, N, K, alpha, A, lda, B, ldb, beta, C,
                                    ldc),
                   stream, cfg);
}

int sgemm_op_ex_noalloc(int trans_a, int trans_b, int M, int N, int K, float alpha,
                        const float *A, int lda, const float *B, int ldb, float beta, float *C,
                        int ldc, hipStream_t stream, const sgemm_config *cfg) {
    return sg::run(sg::make_problem(trans_a, trans_b, M, N, K, alpha, A, lda, B, ldb, beta, C,
                                    ldc),
                   stream, cfg, true);
}

int sgemm_epilogue_ex(int trans_a, int trans_b, int M, int N, int K, float alpha,
                      const float *A, int lda, const float *B, int ldb, float beta, float *C,
                      int ldc, const float *bias, int act, hipStream_t stream,
                      const sgemm_config *cfg) {
    sg::Problem p = sg::make_problem(trans_a, trans_b, M, N, K, alpha, A, lda, B, ldb, beta, C,
                                     ldc);
    p.bias = bias;
    p.act = act;
    return sg::run(p, stream, cfg);
}

int sgemm_epilogue(int trans_a, int trans_b, int M, int N, int K, float alpha, const float *A,
                   int lda, const float *B, int ldb, float beta, float *C, int ldc,
                   const float *bias, int act, hipStream_t stream) {
    return sgemm_epilogue_ex(trans_a, trans_b, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, bias,
                             act, stream, nullptr);
}

int sgemm_strided_batched_ex(int trans_a, int trans_b, int M, int N, int K, float alpha,
                             const float *A, int lda, long long stride_a, const float *B,
                             int ldb, long long stride_b, float beta, float *C, int ldc,
                             long long stride_c, int batch, hipStream_t stream,
                             const sgemm_config *cfg) {
    sg::Problem p = sg::make_problem(trans_a, trans_b, M, N, K, alpha, A, lda, B, ldb, beta, C,
                                     ldc);
    p.batch = batch;
    p.stride_a = stride_a;
    p.stride_b = stride_b;
    p.stride_c = stride_c;
    return sg::run(p, stream, cfg);
}

int sgemm_strided_batched(int trans_a, int trans_b, int M, int N, int K, float alpha,
                          const float *A, int lda, long long stride_a, const float *B, int ldb,
                          long long stride_b, float beta, float *C, int ldc, long long stride_c,
                          int batch, hipStream_t stream) {
    return sgemm_strided_batched_ex(trans_a, trans_b, M, N, K, alpha, A, lda, stride_a, B, ldb,
                                    stride_b, beta, C, ldc, stride_c, batch, stream, nullptr);
}

int sgemm_op_plan(int trans_a, int trans_b, int M, int N, int K, const float *A, int lda,
                  const float *B, int ldb, const float *C, int ldc, sgemm_config *out,
                  int *edge_rows, int *edge_cols) {
    if (!out) return -14;
    if (trans_a != 0 && trans_a != 1) return sg::kBadTransA;
    if (trans_b != 0 && trans_b != 1) return sg::kBadTransB;
    if (M < 0) return -1;
    if (N < 0) return -2;
    if (K < 0) return -3;
    const sg::Problem p{M,   N,   K, 1.f, 0.f, A, lda, B, ldb, const_cast<float *>(C),
                        ldc, trans_a, trans_b};
    sg::Choice ch;
    sg::Strips sp{0, 0};
    const int st = sg::resolve(p, nullptr, ch, &sp);
    if (st != 0) return st;
    out->variant = ch.variant;
    out->tile = ch.tile;
    // a few-rows skinny plan reports the K slices it splits into (none when
    // its one row runs as the one-column product)
    out->group_m = (ch.variant == SGEMM_VARIANT_SKINNY && sg::skinny_kind(ch.tile) == 0)
                       ? (sg::skinny_one_row_column(p, ch.group_m, ch.vec)
                              ? 1
                              : sg::skinny_slices(ch.tile, p, ch.group_m))
                       : ch.group_m;
    out->flags = (ch.vec ? 0 : SGEMM_FLAG_SCALAR_IO) | (ch.streamk ? SGEMM_FLAG_STREAMK : 0);
    if (edge_rows) *edge_rows = sp.rows;
    if (edge_cols) *edge_cols = sp.cols;
    return 0;
}

int sgemm_plan(int M, int N, int K, const float *A, int lda, const float *B, int ldb,
               const float *C, int ldc, sgemm_config *out, int *edge_rows, int *edge_cols) {
    return sgemm_op_plan(0, 0, M, N, K, A, lda, B, ldb, C, ldc, out, edge_rows, edge_cols);
}

int sgemm_cblas(int order, int trans_a, int trans_b, int M, int N, int K, float alpha,
                const float *A, int lda, const float *B, int ldb, float beta, float *C, int ldc,
                hipStream_t stream) {
    auto op = [](int t) { return t == 111 ? 0 : (t == 112 || t == 113) ? 1 : -1; };
    const int ta = op(trans_a), tb = op(trans_b);
    if (order != 101 && order != 102) return sg::kBadOrder;
    if (ta < 0) return sg::kBadTransA;
    if (tb < 0) return sg::kBadTransB;
    if (order == 101)
        return sg::run(sg::make_problem(ta, tb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc),
                       stream, nullptr);
    // column-major C = op(A) op(B) is row-major C^T = op(B)^T op(A)^T over the
    // same memory: B's storage takes A's place and the transposition flags carry over
    const int st = sg::run(sg::make_problem(tb, ta, N, M, K, alpha, B, ldb, A, lda, beta, C, ldc),
                           stream, nullptr);
    return sg::colmajor_status(st);
}

int sgemm_select(int M, int N, int K, const float *A, int lda, const float *B, int ldb,
                 const float *C, int ldc, sgemm_config *out) {
    return sgemm_plan(M, N, K, A, lda, B, ldb, C, ldc, out, nullptr, nullptr);
}

int sgemm_mixed_ex(int dtype, int trans_a, int trans_b, int M, int N, int K, float alpha,
                   const void *A, int lda, const void *B, int ldb, float beta, float *C, int ldc,
                   hipStream_t stream, const sgemm_config *cfg) {
    return sg::run16(dtype, trans_a, trans_b, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                     stream, cfg);
}

int sgemm_mixed(int dtype, int trans_a, int trans_b, int M, int N, int K, float alpha,
                const void *A, int lda, const void *B, int ldb, float beta, float *C, int ldc,
                hipStream_t stream) {
    return sg::run16(dtype, trans_a, trans_b, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                     stream, nullptr);
}

int sgemm_tile_count(int variant) {
    if (variant == SGEMM_VARIANT_MFMA16) return sg::tiles16_count();
    if (variant == SGEMM_VARIANT_GENERIC16) return 1;
    int count = 0;
    sg::family(variant, &count);
    return count;
}

int sgemm_tile_info(int variant, int tile, sgemm_tile_desc *out) {
    if (!out) return sg::kBadConfig;
    if (variant == SGEMM_VARIANT_MFMA16) {
        const sgemm_tile_desc *d = sg::tile16_desc(tile);
        if (!d) return sg::kBadConfig;
        *out = *d;
        return 0;
    }
    if (variant == SGEMM_VARIANT_GENERIC16) {
        if (tile != 0) return sg::kBadConfig;
        *out = sg::kGeneric16Desc;
        return 0;
    }
    int count = 0;
    const sg::TileEntry *t = sg::family(variant, &count);
    if (!t || tile < 0 || tile >= count) return sg::kBadConfig;
    *out = t[tile].desc;
    return 0;
}

const char *sgemm_status_string(int status) {
    switch (status) {
    case 0: return "success";
    case -1: return "invalid argument 1 (M < 0)";
    case -2: return "invalid argument 2 (N < 0)";
    case -3: return "invalid argument 3 (K < 0)";
    case -5: return "invalid argument 5 (A null or not 4-byte aligned)";
    case -6: return "invalid argument 6 (lda too small: max(1, K), or max(1, M) with A transposed)";
    case -7: return "invalid argument 7 (B null or not 4-byte aligned)";
    case -8: return "invalid argument 8 (ldb too small: max(1, N), or max(1, K) with B transposed)";
    case -10: return "invalid argument 10 (C null or not 4-byte aligned)";
    case -11: return "invalid argument 11 (ldc < max(1, N))";
    case -13: return "invalid or inapplicable configuration";
    case -14: return "null output pointer";
    case -21: return "invalid trans_a (0 or 1; CBLAS: 111, 112 or 113)";
    case -22: return "invalid trans_b (0 or 1; CBLAS: 111, 112 or 113)";
    case -23: return "invalid order (CBLAS: 101 row-major or 102 column-major)";
    case -24: return "bias not 4-byte aligned";
    case -25: return "invalid activation code";
    case -26: return "negative batch stride of A";
    case -27: return "negative batch stride of B";
    case -28: return "batch stride of C lets two entries of the batch overlap";
    case -29: return "negative batch count";
    case -30: return "invalid input format (SGEMM_DTYPE_BF16 or SGEMM_DTYPE_F16)";
    case -31: return "the plan's partial sums need more memory than the static scratch holds";
    default: break;
    }
    if (status > 0) return hipGetErrorString(static_cast<hipError_t>(status));
    return "unknown status";
}

int sgemm_version(void) { return sg::kVersion; }

int sgemm_workspace_release(void) { return static_cast<int>(sg::workspace_release_all()); }

}  // extern "C"
