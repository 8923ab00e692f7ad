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

constexpr int kVersion = 200;   // 0.2.0
constexpr int kBadConfig = -13;

bool aligned4(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }
bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// 16-byte vector I/O needs every row start of A, B and C on a 16-byte
// boundary ("The GEMM Scrapbook", vectorisation chapter: 128-bit accesses
// need 16-byte alignment).
bool vector_io_ok(const float *A, int lda, const float *B, int ldb, const float *C, int ldc) {
    return aligned16(A) && aligned16(B) && aligned16(C) && (lda % 4 == 0) && (ldb % 4 == 0) &&
           (ldc % 4 == 0);
}

struct Tuned {
    int variant, tile, group_m;
};

#include "tuned_table.inc"

long long tiles_for(const TileEntry &t, int M, int N) {
    return (long long)((M + t.desc.bm - 1) / t.desc.bm) * ((N + t.desc.bn - 1) / t.desc.bn);
}

// The MFMA family: the general tiles followed by the whole-tile (direct-load)
// tiles, in one table.
const TileEntry *mfma_family(int *count) {
    static const std::vector<TileEntry> all = [] {
        std::vector<TileEntry> v;
        int n = 0;
        const TileEntry *t = mfma_tiles(&n);
        v.insert(v.end(), t, t + n);
        t = mfma_direct_tiles(&n);
        v.insert(v.end(), t, t + n);
        return v;
    }();
    *count = (int)all.size();
    return all.data();
}

// Whether tile t can run this problem (whole-tile tiles need 16-byte I/O and
// whole tiles).
bool tile_applies(const TileEntry &t, const Problem &p, bool vec) {
    if (!(t.desc.flags & SGEMM_TILE_WHOLE)) return true;
    return vec && direct_applies(p, t.desc.bm, t.desc.bn, t.desc.bk);
}

const TileEntry *family(int variant, int *count) {
    switch (variant) {
    case SGEMM_VARIANT_MFMA: return mfma_family(count);
    case SGEMM_VARIANT_VALU: return valu_tiles(count);
    case SGEMM_VARIANT_SKINNY: return skinny_tiles(count);
    default: *count = 0; return nullptr;
    }
}

int validate(int M, int N, int K, float alpha, const float *A, int lda, const float *B, int ldb,
             float *C, int ldc) {
    if (M < 0) return -1;
    if (N < 0) return -2;
    if (K < 0) return -3;
    if (lda < (K > 1 ? K : 1)) return -6;
    if (ldb < (N > 1 ? N : 1)) return -8;
    if (ldc < (N > 1 ? N : 1)) return -11;
    if (M == 0 || N == 0) return 0;
    const bool reads_ab = (alpha != 0.f) && K > 0;
    if (reads_ab && (!A || !aligned4(A))) return -5;
    if (reads_ab && (!B || !aligned4(B))) return -7;
    if (!C || !aligned4(C)) return -10;
    return 0;
}

int to_status(hipError_t e) { return e == hipSuccess ? 0 : static_cast<int>(e); }

// The general MFMA tile for a shape (never a whole-tile one): the largest tile
// that still yields about one workgroup per CU.
int general_mfma_tile(int M, int N) {
    int count = 0;
    const TileEntry *tiles = mfma_tiles(&count);
    const int order[] = {2, 5, 7};
    for (int idx : order)
        if (idx < count && tiles_for(tiles[idx], M, N) >= 200) return idx;
    return 7;
}

// The MFMA tile for a shape that is not in the tuned table: the first
// whole-tile (direct-load) configuration that applies and still yields about
// one workgroup per CU, else the general rule.
int default_mfma_tile(const Problem &p, bool vec) {
    int count = 0;
    const TileEntry *tiles = mfma_family(&count);
    for (int i = 0; i < count; ++i)
        if ((tiles[i].desc.flags & SGEMM_TILE_WHOLE) && tile_applies(tiles[i], p, vec) &&
            tiles_for(tiles[i], p.M, p.N) >= 200)
            return i;
    return general_mfma_tile(p.M, p.N);
}

// Automatic choice: the measured best configuration for this exact shape
// (tuned_table.inc), else the skinny family for memory-bound shapes, else the
// default MFMA rule.  A tuned whole-tile choice is checked against the actual
// operands in resolve().
Tuned auto_select(const Problem &p, bool vec) {
    Tuned t;
    if (lookup_tuned(p.M, p.N, p.K, t)) return t;
    if (skinny_pick(p.M, p.N, p.K) >= 0) return Tuned{SGEMM_VARIANT_SKINNY, -1, 0};
    return Tuned{SGEMM_VARIANT_MFMA, default_mfma_tile(p, vec), 0};
}

// The configuration a call runs with: explicit (sgemm_ex) or automatic, with
// a whole-tile choice replaced by the general rule where the operands do not
// allow it.  Returns 0 or kBadConfig.
struct Choice {
    int variant, tile, group_m;
    bool vec;
};

int resolve(const Problem &p, const sgemm_config *cfg, Choice &out) {
    const int flags = cfg ? cfg->flags : 0;
    const bool vec = !(flags & SGEMM_FLAG_SCALAR_IO) &&
                     vector_io_ok(p.A, (int)p.lda, p.B, (int)p.ldb, p.C, (int)p.ldc);
    int variant = cfg ? cfg->variant : SGEMM_VARIANT_AUTO;
    int tile = cfg ? cfg->tile : -1;
    int group_m = cfg ? cfg->group_m : 0;
    if (variant < 0 || variant >= SGEMM_VARIANT_COUNT) return kBadConfig;
    const bool explicit_tile = (variant != SGEMM_VARIANT_AUTO) && tile >= 0;
    if (variant == SGEMM_VARIANT_AUTO) {
        const Tuned a = auto_select(p, vec);
        variant = a.variant;
        tile = a.tile;
        if (group_m <= 0) group_m = a.group_m;
    }
    int count = 0;
    const TileEntry *tiles = family(variant, &count);
    if (!tiles) return kBadConfig;
    if (variant == SGEMM_VARIANT_SKINNY) {
        if (tile < 0) tile = skinny_pick(p.M, p.N, p.K);
        if (!skinny_fits(tile, p.M, p.N)) return kBadConfig;   // shape is not skinny
    } else if (tile < 0) {
        tile = (variant == SGEMM_VARIANT_MFMA) ? default_mfma_tile(p, vec) : 0;
    }
    if (tile >= count) {
        if (explicit_tile || variant != SGEMM_VARIANT_MFMA) return kBadConfig;
        tile = general_mfma_tile(p.M, p.N);   // a tuned row naming a tile that is not compiled
    }
    if (!tile_applies(tiles[tile], p, vec)) {
        if (explicit_tile) return kBadConfig;
        tile = general_mfma_tile(p.M, p.N);   // automatic whole-tile choice that cannot run here
    }
    if (!(vec ? tiles[tile].vec : tiles[tile].scalar)) return kBadConfig;
    out = Choice{variant, tile, group_m, vec};
    return 0;
}

int run(int M, int N, int K, float alpha, const float *A, int lda, const float *B, int ldb,
        float beta, float *C, int ldc, hipStream_t stream, const sgemm_config *cfg) {
    const int v = validate(M, N, K, alpha, A, lda, B, ldb, C, ldc);
    if (v != 0) return v;
    if (M == 0 || N == 0) return 0;

    if (alpha == 0.f || K == 0) {
        if (beta == 1.f) return 0;
        return to_status(launch_scale(M, N, beta, C, ldc, stream));
    }

    const Problem p{M, N, K, alpha, beta, A, lda, B, ldb, C, ldc};
    Choice ch;
    const int st = resolve(p, cfg, ch);
    if (st != 0) return st;
    int count = 0;
    const TileEntry &t = family(ch.variant, &count)[ch.tile];
    static const bool log = std::getenv("FP32_SGEMM_LOG") != nullptr;
    if (log)
        std::fprintf(stderr, "sgemm M=%d N=%d K=%d variant=%d tile=%d (%dx%dx%d) group_m=%d %s\n",
                     M, N, K, ch.variant, ch.tile, t.desc.bm, t.desc.bn, t.desc.bk, ch.group_m,
                     ch.vec ? "vec16" : "scalar");
    return to_status((ch.vec ? t.vec : t.scalar)(p, ch.group_m, stream));
}

}  // namespace
}  // namespace sg

extern "C" {

int sgemm(int M, int N, int K, float alpha, const float *A, int lda, const float *B, int ldb,
          float beta, float *C, int ldc, hipStream_t stream) {
    return sg::run(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream, nullptr);
}

int sgemm_ex(int M, int N, int K, float alpha, const float *A, int lda, const float *B, int ldb,
             float beta, float *C, int ldc, hipStream_t stream, const sgemm_config *cfg) {
    return sg::run(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream, cfg);
}

int sgemm_select(int M, int N, int K, const float *A, int lda, const float *B, int ldb,
                 const float *C, int ldc, sgemm_config *out) {
    if (!out) return -14;
    if (M < 0) return -1;
    if (N < 0) return -2;
    if (K < 0) return -3;
    const sg::Problem p{M, N, K, 1.f, 0.f, A, lda, B, ldb, const_cast<float *>(C), ldc};
    sg::Choice ch;
    const int st = sg::resolve(p, nullptr, ch);
    if (st != 0) return st;
    out->variant = ch.variant;
    out->tile = ch.tile;
    out->group_m = ch.group_m;
    out->flags = ch.vec ? 0 : SGEMM_FLAG_SCALAR_IO;
    return 0;
}

int sgemm_tile_count(int variant) {
    int count = 0;
    sg::family(variant, &count);
    return count;
}

int sgemm_tile_info(int variant, int tile, sgemm_tile_desc *out) {
    int count = 0;
    const sg::TileEntry *t = sg::family(variant, &count);
    if (!t || tile < 0 || tile >= count || !out) return sg::kBadConfig;
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
    case -6: return "invalid argument 6 (lda < max(1, K))";
    case -7: return "invalid argument 7 (B null or not 4-byte aligned)";
    case -8: return "invalid argument 8 (ldb < max(1, N))";
    case -10: return "invalid argument 10 (C null or not 4-byte aligned)";
    case -11: return "invalid argument 11 (ldc < max(1, N))";
    case -13: return "invalid or inapplicable configuration";
    case -14: return "null output pointer";
    default: break;
    }
    if (status > 0) return hipGetErrorString(static_cast<hipError_t>(status));
    return "unknown status";
}

int sgemm_version(void) { return sg::kVersion; }

}  // extern "C"
