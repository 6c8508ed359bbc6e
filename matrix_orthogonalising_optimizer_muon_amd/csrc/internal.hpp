// Internal interfaces between the C-ABI front end (api.cpp) and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace muon {

// Per-matrix descriptor, written into the workspace at the start of every step.
struct MatDesc {
  void* W;
  const void* G;
  void* M;
  int64_t rows, cols;     // stored shape (row-major, ld = cols)
  int32_t transposed;     // 1: canonical X is the transpose of the stored matrix
  int32_t pad_;
};

enum Kind : int { KIND_BF16 = 0, KIND_F16 = 1, KIND_F32 = 2 };
enum Epi : int { EPI_STORE = 0, EPI_APPLY = 1, EPI_UPDATE = 2 };

// Batched NT GEMM over `count` same-shape problems: acc = A * B^T with A (M x K) and
// B (N x K) row-major. Matrix i of the batch uses A + i*sA, B + i*sB, ... (element
// strides) and the device scalar s[i].
// Epilogue value: v = alpha' * acc + beta' * E + gamma * [row == col], with
//   alpha' = alpha * s[i]^alpha_spow, beta' = beta * s[i]^beta_spow, and E read at
//   (row, col) or, with e_trans, at (col, row).
//   EPI_STORE (symmetric output): C = v; only tiles with tile_m <= tile_n are computed
//     and off-diagonal tiles are also stored mirrored, so C is exactly symmetric.
//   EPI_APPLY: C = oscale * v and, if C2, C2^T = oscale * v (transposed copy).
//   EPI_UPDATE: W[desc] <- W*(1 - lr*wd) - lr*v for row < Mvalid, col < Nvalid, through
//     the descriptor's orientation.
// M, N, K are multiples of 64 (the padded canonical sizes).
struct GemmParams {
  const void* A; const void* B; void* C; void* C2; const void* E;
  int64_t lda, ldb, ldc, ldc2, lde;
  int64_t sA, sB, sC, sC2, sE;
  int32_t M, N, K;
  int32_t Mvalid, Nvalid;
  int32_t tiles_m, tiles_n, tiles;
  int32_t count;
  float alpha, beta, gamma, oscale;
  int32_t alpha_spow, beta_spow;
  int32_t e_trans;
  int32_t e_from_a;       // E is A (same buffer, lde == lda, sE == sA, K == N, !e_trans)
  const float* s;
  const MatDesc* table;   // EPI_UPDATE: descriptors of the batch (entry i = matrix i)
  float lr, wd;
  int32_t w_bf16;
};

// Stages of the GEMM family.
enum GemmOp : int {
  OP_SYRK_IN = 0,  // X X^T on the momentum output (bf16 on the bf16 path), symmetric
  OP_SYM = 1,      // A B^T with symmetric output (fp16 / fp32 operands)
  OP_APPLY = 2,    // A B^T, general output, X in both layouts
  OP_UPDATE = 3,   // A B^T, epilogue updates W
  OP_SYRK = 4,     // X X^T on the fp16 / fp32 iterate (same kernel as OP_SYM, own symbol)
};

// Workgroup tile configurations. Symmetric-output stages need BM == BN. Configurations
// 0-3 stage operands through registers; 4-13 use the CDNA4 direct global -> LDS loads
// with a multi-stage LDS ring.
enum TileCfg : int {
  TILE_64 = 0,           // 64 x 64, 4 waves, wave tile 32 x 32
  TILE_128 = 1,          // 128 x 128, 4 waves, wave tile 64 x 64
  TILE_256x128 = 2,      // 256 x 128, 8 waves, wave tile 64 x 64
  TILE_256 = 3,          // 256 x 256, 8 waves, wave tile 128 x 64
  TILE_64_DMA = 4,       // as TILE_64, 4 LDS stages
  TILE_128_DMA = 5,      // as TILE_128, 4 LDS stages
  TILE_256x128_DMA = 6,  // as TILE_256x128, 3 LDS stages
  TILE_256_DMA = 7,      // as TILE_256, 2 LDS stages
  TILE_256_DMA4 = 8,     // 256 x 256, 4 waves, wave tile 128 x 128, 2 LDS stages
  TILE_64_DMA_K2 = 9,    // as TILE_64_DMA with 8 waves: two k-groups split every slice
  TILE_128_DMA_K2 = 10,  // as TILE_128_DMA with 8 waves: two k-groups split every slice
  TILE_256_DMA_H = 11,   // as TILE_256_DMA with 64-byte slices: 4 LDS stages
  TILE_128_DMA_K2_H = 12,  // as TILE_128_DMA_K2 with 64-byte slices: 8 LDS stages
  TILE_256x192_DMA = 13,  // 256 x 192, 8 waves, wave tile 64 x 96, 2 LDS stages
  TILE_256_DMA4_H = 14,   // as TILE_256_DMA4 with 64-byte slices: 4 LDS stages
  TILE_COUNT = 15
};
inline int tile_bm(int cfg) {
  static const int bm[TILE_COUNT] = {64, 128, 256, 256, 64, 128, 256, 256, 256, 64, 128, 256, 128, 256, 256};
  return bm[cfg];
}
inline int tile_bn(int cfg) {
  static const int bn[TILE_COUNT] = {64, 128, 128, 256, 64, 128, 128, 256, 256, 64, 128, 256, 128, 192, 256};
  return bn[cfg];
}

// Whether launch_gemm has configuration `cfg` for a symmetric-output (sym) or general
// stage on the fp32 (f32) or bf16 path.
inline bool tile_available(bool sym, bool f32, int cfg) {
  if (cfg < 0 || cfg >= TILE_COUNT) return false;
  if (sym && tile_bm(cfg) != tile_bn(cfg)) return false;
  if (f32 && tile_bm(cfg) == 256) return false;
  return true;
}

// The direct-load kernels address a matrix's operands with 32-bit byte offsets. A stage
// whose operands (A: M x lda, B: N x ldb elements of `es` bytes) do not fit runs the
// register-staged tile of the same block rows instead.
inline bool dma_addressable(int64_t M, int64_t lda, int64_t N, int64_t ldb, int64_t es) {
  const int64_t lim = (int64_t{1} << 32) - 1;
  return M * lda * es <= lim && N * ldb * es <= lim;
}
inline int staged_tile(int cfg) {
  switch (cfg) {
    case TILE_64_DMA: case TILE_64_DMA_K2: return TILE_64;
    case TILE_128_DMA: case TILE_128_DMA_K2: case TILE_128_DMA_K2_H: return TILE_128;
    case TILE_256_DMA: case TILE_256_DMA4: case TILE_256_DMA_H: case TILE_256_DMA4_H: return TILE_256;
    case TILE_256x128_DMA: case TILE_256x192_DMA: return TILE_256x128;
    default: return cfg;
  }
}

// Launch one batched GEMM stage. ns_f32: fp32 kernels, else bf16/fp16 kernels.
hipError_t launch_gemm(GemmOp op, bool ns_f32, int cfg, const GemmParams& p, hipStream_t st);

// Copy up to kTableChunk descriptors (passed by value) into device memory.
constexpr int kTableChunk = 48;
struct TableChunk {
  MatDesc d[kTableChunk];
  int32_t n;
};

// The HBM-bound stages take two passes over G and M, so that the iterate is rounded once,
// from the fp32 momentum output U, after the norm is known:
//   launch_momentum_norm: per-block partial sums of U^2 (U = G + mu (mu M + G), or
//     mu M + G without Nesterov) over the stored elements; nothing is written but the
//     partials (and, with inline descriptors, the table);
//   launch_momentum_x: M <- mu M + G, and the normalised iterate X0 = xscale * s[i] * U in
//     the canonical orientation, written row-major (X, Mp x Np) and transposed (XT,
//     Np x Mp), padding included (zeros); fp16 on the bf16 path, fp32 on the fp32 path.
struct MomentumParams {
  const MatDesc* table;   // entry i = matrix i of the batch
  void* X;                // canonical padded iterate, matrix i at X + i*sX (elements)
  void* XT;               // its transpose, matrix i at XT + i*sX (ld Mp)
  int64_t sX;             // element stride between matrices (Mp * Np)
  int32_t m, n;           // canonical dims m' <= n'
  int32_t Mp, Np;         // padded canonical dims
  int32_t tiles_m, tiles_n;  // 64 x 64 canonical tiles per matrix (momentum_x grid)
  int32_t norm_blocks;    // norm_ub * kNormBlock-element blocks of the stored matrix
                          // (momentum_norm grid, one partial each)
  int32_t norm_ub;        // 1 or 4: kNormBlock-element groups per momentum_norm workgroup
                          // (4: a large group, whose momentum_x workgroups take two tiles)
  int32_t count;
  float mu;
  int32_t nesterov;
  int32_t g_bf16, m_bf16;   // storage dtypes (0: fp32)
  int32_t x_f16;            // iterate fp16 (bf16 path) or fp32
  int32_t keep_gm;          // momentum_norm: ordinary (cached) loads of G and M, so that
                            // momentum_x finds them in the caches (groups that fit)
  float xscale;             // power-of-two scale of the stored iterate
  const float* s;           // per-matrix 1 / (||U||_F + eps) (momentum_x)
  float* partials;          // [count][norm_blocks]
  // With inl.n > 0 (batches of at most kTableChunk matrices) the descriptors come in the
  // kernel arguments; momentum_norm's workgroup (0, i) also writes entry i to table_out,
  // for the later stages of the batch, so no separate table launch is needed.
  TableChunk inl;
  MatDesc* table_out;
};
hipError_t launch_momentum_norm(const MomentumParams& p, hipStream_t st);
hipError_t launch_momentum_x(const MomentumParams& p, hipStream_t st);
constexpr int kNormBlock = 4096;  // stored elements per partial sum

// Dry runs (muon_prepare): a seeded stand-in for the momentum output, U(i, r, c) =
// dry_u(i, r, c) uniform in [-1, 1) for the canonical element (r, c) of matrix i.
__host__ __device__ inline float dry_u(uint32_t mat, uint32_t r, uint32_t c) {
  uint32_t h = mat * 0x9E3779B9u ^ (r * 0x85EBCA6Bu + 0x27D4EB2Fu) ^ (c * 0xC2B2AE35u + 0x165667B1u);
  h ^= h >> 16; h *= 0x7FEB352Du; h ^= h >> 15; h *= 0x846CA68Bu; h ^= h >> 16;
  return static_cast<float>(h >> 8) * (2.0f / 16777216.0f) - 1.0f;
}
// X0 = xscale * sqrt(3 / (m n)) * dry_u (unit Frobenius norm in expectation) in both layouts,
// zero padding; the partials, s and M are not touched.
hipError_t launch_dry_x(const MomentumParams& p, hipStream_t st);

// s[i] = 1 / (sqrt(sum_j partials[i][j]) + eps), fixed-order fp64 reduction.
hipError_t launch_norm_finalize(const float* partials, int per_matrix, int count, float eps,
                                float* s, hipStream_t st);

// The whole update of each matrix of a small same-shape group in one workgroup (bf16 path,
// padded m' <= 128 and m' n' <= kSmallMaxElems): momentum, norm, the NS schedule (plain rounds or Gram segments) and the W
// update. Buffers are the group's workspace: X (Mp x Np), XT[2] (Np x Mp), S[0..3] (Mp x Mp;
// S[2], S[3] unused by plain NS), matrix i at base + i * stride (elements).
struct SmallParams {
  const MatDesc* table;
  int32_t count;
  int32_t m, n, Mp, Np;
  void* X; void* XT[2]; void* S[4];
  int64_t sX, sXT, sS;
  float mu, eps, lr, wd;
  float a, b, c;
  float xs, e;               // iterate scale (fp16 X = xs * X), Gram-space scale
  int32_t nesterov;
  int32_t plain, rounds;     // plain NS with `rounds` rounds, else Gram segments
  int32_t n_segments;
  int32_t segments[8];
  int32_t g_bf16, m_bf16, w_bf16;
  // Dry run (muon_prepare): U comes from dry_u() instead of G and M, nothing is stored to
  // M or W (the last product writes the iterate to the workspace instead).
  int32_t dry;
};
hipError_t launch_small_ns(const SmallParams& p, hipStream_t st);
constexpr int kSmallMaxElems = 64 * 1024;  // padded m' n' the single-workgroup kernel takes

// AdamW over up to kAdamChunk tensors per launch (descriptors travel in the kernel
// arguments). Tensor i covers workgroups [block0, block0 + adam_blocks(numel)).
constexpr int kAdamChunk = 24;
struct AdamTensor {
  void* W;
  const void* G;
  float* m;
  float* v;
  int64_t numel;
  int64_t block0;
  int32_t vec;      // all four arrays 16-byte aligned: 8-element vector accesses
  int32_t pad_;
};
struct AdamChunk {
  AdamTensor t[kAdamChunk];
  int32_t n;
  int32_t w_bf16, g_bf16;
  float lr, wd, b1, b2, eps;
  float bc1;        // 1 - beta1^t
  float bc2s;       // sqrt(1 - beta2^t)
};
int64_t adam_blocks(int64_t numel);
hipError_t launch_adamw(const AdamChunk& c, int64_t blocks, hipStream_t st);

hipError_t launch_write_table(const TableChunk& c, MatDesc* dst, hipStream_t st);

}  // namespace muon
