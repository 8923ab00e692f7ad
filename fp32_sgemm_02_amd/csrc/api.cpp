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

// Automatic choice: the measured best configuration for this exact shape
// (tuned_table.inc), else the skinny family for memory-bound shapes, else the
// largest MFMA tile that still yields about one workgroup per CU.
Tuned auto_select(int M, int N, int K) {
    Tuned t;
    if (lookup_tuned(M, N, K, t)) return t;
    if (skinny_pick(M, N, K) >= 0) return Tuned{SGEMM_VARIANT_SKINNY, -1, 0};
    int count = 0;
    const TileEntry *tiles = mfma_tiles(&count);
    const int order[] = {2, 5, 7};
    for (int idx : order)
        if (idx < count && tiles_for(tiles[idx], M, N) >= 200)
            return Tuned{SGEMM_VARIANT_MFMA, idx, 0};
    return Tuned{SGEMM_VARIANT_MFMA, 7, 0};
}

const TileEntry *family(int variant, int *count) {
    switch (variant) {
    case SGEMM_VARIANT_MFMA: return mfma_tiles(count);
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

int run(int M, int N, int K, float alpha, const float *A, int lda, const float *B, int ldb,
        float beta, float *C, int ldc, hipStream_t stream, const sgemm_config *cfg) {
    const int v = validate(M, N, K, alpha, A, lda, B, ldb, C, ldc);
    if (v != 0) return v;
    if (M == 0 || N == 0) return 0;

    if (alpha == 0.f || K == 0) {
        if (beta == 1.f) return 0;
        return to_status(launch_scale(M, N, beta, C, ldc, stream));
    }

    Tuned choice{SGEMM_VARIANT_AUTO, -1, 0};
    int flags = 0;
    if (cfg) {
        choice = Tuned{cfg->variant, cfg->tile, cfg->group_m};
        flags = cfg->flags;
        if (choice.variant < 0 || choice.variant >= SGEMM_VARIANT_COUNT) return kBadConfig;
    }
    if (choice.variant == SGEMM_VARIANT_AUTO) {
        const Tuned a = auto_select(M, N, K);
        choice.variant = a.variant;
        if (choice.tile < 0) choice.tile = a.tile;
        if (choice.group_m <= 0) choice.group_m = a.group_m;
    }

    int count = 0;
    const TileEntry *tiles = family(choice.variant, &count);
    if (!tiles) return kBadConfig;
    if (choice.variant == SGEMM_VARIANT_SKINNY) {
        if (choice.tile < 0) choice.tile = skinny_pick(M, N, K);
        if (!skinny_fits(choice.tile, M, N)) return kBadConfig;   // shape is not skinny
    } else if (choice.tile < 0) {
        choice.tile = 0;
        if (choice.variant == SGEMM_VARIANT_MFMA) choice.tile = auto_select(M, N, K).tile;
        if (choice.tile < 0) choice.tile = 0;
    }
    if (choice.tile >= count) return kBadConfig;

    Problem p{M, N, K, alpha, beta, A, lda, B, ldb, C, ldc};
    const TileEntry &t = tiles[choice.tile];
    const bool vec = !(flags & SGEMM_FLAG_SCALAR_IO) && vector_io_ok(A, lda, B, ldb, C, ldc);
    static const bool log = std::getenv("FP32_SGEMM_LOG") != nullptr;
    if (log)
        std::fprintf(stderr, "sgemm M=%d N=%d K=%d variant=%d tile=%d (%dx%dx%d) group_m=%d %s\n",
                     M, N, K, choice.variant, choice.tile, t.desc.bm, t.desc.bn, t.desc.bk,
                     choice.group_m, vec ? "vec16" : "scalar");
    return to_status((vec ? t.vec : t.scalar)(p, choice.group_m, stream));
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
    const sg::Tuned t = sg::auto_select(M, N, K);
    out->variant = t.variant;
    out->tile = (t.variant == SGEMM_VARIANT_SKINNY && t.tile < 0) ? sg::skinny_pick(M, N, K) : t.tile;
    out->group_m = t.group_m;
    out->flags = sg::vector_io_ok(A, lda, B, ldb, C, ldc) ? 0 : SGEMM_FLAG_SCALAR_IO;
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
