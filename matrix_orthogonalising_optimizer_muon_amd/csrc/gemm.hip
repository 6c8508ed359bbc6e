// Batched MFMA GEMM family for the Newton-Schulz products on gfx950 (CDNA4).
//
// One kernel template serves every contraction of the update:
//   * X X^T (the symmetric Gram product of the DMuon summary, section 2.2): NT operands,
//     only upper tiles computed, off-diagonal tiles stored twice (mirrored);
//   * the m' x m' products of the Gram recurrence and of A^2 (MuonX article, section
//     3.2): NT operands (every operand is exactly symmetric in storage), symmetric output;
//   * Q X / B X (the long "apply" product): NN, the row-major X tile is transposed in
//     registers on its way to LDS, so every LDS tile is K-contiguous;
//   * the last apply with the weight update fused into the epilogue.
//
// Layout: a 256-thread workgroup (4 waves of 64) owns a BM x BN output tile; each wave a
// (BM/WM) x (BN/WN) sub-tile of 32x32 MFMA blocks with fp32 accumulators. K advances in
// 128-byte slices (64 bf16/fp16 or 32 fp32 elements), double-buffered in LDS, staged
// through registers so the next slice's global loads overlap the current MFMAs. LDS rows
// are 8 chunks of 16 bytes, XOR-swizzled per row so that both the fragment reads (32
// consecutive rows, same chunk) and the transposed NN writes (rows 8 apart) spread over
// all banks.
#include "internal.hpp"

namespace muon {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int kChunks = 8;  // 16-byte chunks per 128-byte LDS row

__device__ __forceinline__ int swz(int row, int chunk) {
  return row * kChunks + (chunk ^ ((row ^ (row >> 3)) & 7));
}

__device__ __forceinline__ float bf16_to_f32(unsigned short h) {
  return __uint_as_float(static_cast<unsigned int>(h) << 16);
}
// Round-to-nearest-even fp32 -> bf16 (inputs here are finite).
__device__ __forceinline__ unsigned short f32_to_bf16(float f) {
  unsigned int u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<unsigned short>(u >> 16);
}
__device__ __forceinline__ unsigned short f32_to_f16(float f) {
  _Float16 h = static_cast<_Float16>(f);
  return __builtin_bit_cast(unsigned short, h);
}
__device__ __forceinline__ float f16_to_f32(unsigned short h) {
  return static_cast<float>(__builtin_bit_cast(_Float16, h));
}

__device__ __forceinline__ float scaled(float x, const float* s, int i, int pw) {
  if (pw == 0 || s == nullptr) return x;
  const float v = s[i];
  return pw == 1 ? x * v : x * v * v;
}

template <int KIND>
__device__ __forceinline__ void mma(f32x16& acc, const u32x4& a, const u32x4& b) {
  if constexpr (KIND == KIND_BF16) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
  } else if constexpr (KIND == KIND_F16) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                 __builtin_bit_cast(f16x8, b), acc, 0, 0, 0);
  } else {
    // fp32: each lane's 16-byte chunk holds 4 consecutive k; four 32x32x2 steps consume it.
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.x), __uint_as_float(b.x), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.y), __uint_as_float(b.y), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.z), __uint_as_float(b.z), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.w), __uint_as_float(b.w), acc, 0, 0, 0);
  }
}

// 16-bit 8x8 block transpose: in[r] holds 8 elements of row r; out[j] holds column j.
__device__ __forceinline__ void transpose8x8_16(const u32x4 (&in)[8], u32x4 (&out)[8]) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    unsigned int lo[4], hi[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const unsigned int x = in[2 * p][q];
      const unsigned int y = in[2 * p + 1][q];
      lo[p] = __builtin_amdgcn_perm(y, x, 0x05040100u);  // (x.lo, y.lo): column 2q
      hi[p] = __builtin_amdgcn_perm(y, x, 0x07060302u);  // (x.hi, y.hi): column 2q+1
    }
    out[2 * q] = u32x4{lo[0], lo[1], lo[2], lo[3]};
    out[2 * q + 1] = u32x4{hi[0], hi[1], hi[2], hi[3]};
  }
}

// 32-bit 4x4 block transpose.
__device__ __forceinline__ void transpose4x4_32(const u32x4 (&in)[4], u32x4 (&out)[4]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) out[j] = u32x4{in[0][j], in[1][j], in[2][j], in[3][j]};
}

// Tile index of this workgroup: XCD-aware remap, then grouped (8-tile-row) ordering for
// general outputs or an upper-triangle walk for symmetric ones.
template <bool SYM>
__device__ __forceinline__ void tile_coords(const GemmParams& p, int& tm, int& tn) {
  int t = blockIdx.x;
  const int nwg = gridDim.x;
  // Workgroups are dealt round-robin to the 8 XCDs; give each XCD a contiguous run of
  // logical tiles so neighbouring tiles (shared operand panels) share one L2.
  if ((nwg & 7) == 0) t = (t & 7) * (nwg >> 3) + (t >> 3);
  if constexpr (SYM) {
    int row = 0;
    int len = p.tiles_n;
    while (t >= len) { t -= len; ++row; --len; }
    tm = row;
    tn = row + t;
  } else {
    constexpr int GM = 8;
    const int group = GM * p.tiles_n;
    const int g = t / group;
    const int first = g * GM;
    const int gm = min(p.tiles_m - first, GM);
    const int r = t - g * group;
    tm = first + r % gm;
    tn = r / gm;
  }
}

template <int KIND, int BM, int BN, int WM, int WN, bool NN, bool SYM, int EPI, typename TC>
__global__ __launch_bounds__(kThreads) void gemm_kernel(const GemmParams p) {
  static_assert(WM * WN == 4, "4 waves");
  constexpr int ES = (KIND == KIND_F32) ? 4 : 2;      // element bytes in LDS / MFMA
  constexpr int VEC = 16 / ES;                         // elements per chunk
  constexpr int BK = kChunks * VEC;                    // k per LDS slice
  constexpr int TWM = BM / WM, TWN = BN / WN;          // wave tile
  constexpr int FM = TWM / 32, FN = TWN / 32;          // MFMA blocks per wave
  static_assert(FM >= 1 && FN >= 1, "wave tile");
  constexpr int A_CH = BM * kChunks / kThreads;        // A chunks per thread
  static_assert(A_CH * kThreads == BM * kChunks, "A split");
  constexpr int B_CH = BN * kChunks / kThreads;        // NT B chunks per thread
  constexpr int B_BLOCKS = (BK / VEC) * (BN / VEC);    // NN: VEC x VEC blocks
  constexpr int B_BLK = (B_BLOCKS + kThreads - 1) / kThreads;

  __shared__ u32x4 lds[2][(BM + BN) * kChunks];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int mat = blockIdx.y;

  int tm, tn;
  tile_coords<SYM>(p, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;

  const char* Ab = static_cast<const char*>(p.A) + static_cast<int64_t>(mat) * p.sA * ES;
  // NN B on the bf16 path is bf16 in memory (2 bytes) and converted to fp16.
  const char* Bb = static_cast<const char*>(p.B) + static_cast<int64_t>(mat) * p.sB * ES;

  const float bscale = scaled(p.bscale, p.s, mat, p.bscale_spow);

  u32x4 ra[A_CH];
  u32x4 rbt[NN ? 1 : B_CH];
  u32x4 rbn[NN ? B_BLK : 1][NN ? VEC : 1];

  auto load_global = [&](int k0) {
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
      const int c = tid + i * kThreads;
      const int row = c / kChunks, kc = c % kChunks;
      const int gr = m0 + row;
      if (gr < p.M) {
        ra[i] = *reinterpret_cast<const u32x4*>(Ab + (static_cast<int64_t>(gr) * p.lda + k0 + kc * VEC) * ES);
      } else {
        ra[i] = u32x4{0u, 0u, 0u, 0u};
      }
    }
    if constexpr (!NN) {
#pragma unroll
      for (int i = 0; i < B_CH; ++i) {
        const int c = tid + i * kThreads;
        const int row = c / kChunks, kc = c % kChunks;
        const int gr = n0 + row;
        if (gr < p.N) {
          rbt[i] = *reinterpret_cast<const u32x4*>(Bb + (static_cast<int64_t>(gr) * p.ldb + k0 + kc * VEC) * ES);
        } else {
          rbt[i] = u32x4{0u, 0u, 0u, 0u};
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < B_BLK; ++i) {
        const int b = tid + i * kThreads;
        if (B_BLOCKS % kThreads == 0 || b < B_BLOCKS) {
          const int kb = b / (BN / VEC), nb = b % (BN / VEC);
          const int gn = n0 + nb * VEC;
#pragma unroll
          for (int r = 0; r < VEC; ++r) {
            const int gk = k0 + kb * VEC + r;
            if (gn < p.N) {
              rbn[i][r] = *reinterpret_cast<const u32x4*>(Bb + (static_cast<int64_t>(gk) * p.ldb + gn) * ES);
            } else {
              rbn[i][r] = u32x4{0u, 0u, 0u, 0u};
            }
          }
        }
      }
    }
  };

  auto store_lds = [&](int stage) {
    u32x4* la = lds[stage];
    u32x4* lb = lds[stage] + BM * kChunks;
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
      const int c = tid + i * kThreads;
      la[swz(c / kChunks, c % kChunks)] = ra[i];
    }
    if constexpr (!NN) {
#pragma unroll
      for (int i = 0; i < B_CH; ++i) {
        const int c = tid + i * kThreads;
        lb[swz(c / kChunks, c % kChunks)] = rbt[i];
      }
    } else {
#pragma unroll
      for (int i = 0; i < B_BLK; ++i) {
        const int b = tid + i * kThreads;
        if (B_BLOCKS % kThreads == 0 || b < B_BLOCKS) {
          const int kb = b / (BN / VEC), nb = b % (BN / VEC);
          if constexpr (KIND == KIND_F16) {
            // bf16 rows -> scaled fp16 rows, then an 8x8 transpose.
            u32x4 cv[8], tr[8];
#pragma unroll
            for (int r = 0; r < 8; ++r) {
              unsigned int w[4];
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                const unsigned int x = rbn[i][r][q];
                const float lo = __uint_as_float(x << 16) * bscale;
                const float hi = __uint_as_float(x & 0xFFFF0000u) * bscale;
                w[q] = static_cast<unsigned int>(f32_to_f16(lo)) |
                       (static_cast<unsigned int>(f32_to_f16(hi)) << 16);
              }
              cv[r] = u32x4{w[0], w[1], w[2], w[3]};
            }
            transpose8x8_16(cv, tr);
#pragma unroll
            for (int j = 0; j < 8; ++j) lb[swz(nb * 8 + j, kb)] = tr[j];
          } else {
            static_assert(KIND == KIND_F32, "NN operand kinds");
            u32x4 cv[4], tr[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const u32x4 x = rbn[i][r];
              cv[r] = u32x4{__float_as_uint(__uint_as_float(x.x) * bscale),
                            __float_as_uint(__uint_as_float(x.y) * bscale),
                            __float_as_uint(__uint_as_float(x.z) * bscale),
                            __float_as_uint(__uint_as_float(x.w) * bscale)};
            }
            transpose4x4_32(cv, tr);
#pragma unroll
            for (int j = 0; j < 4; ++j) lb[swz(nb * 4 + j, kb)] = tr[j];
          }
        }
      }
    }
  };

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  const int wm0 = (wave / WN) * TWM;
  const int wn0 = (wave % WN) * TWN;
  const int nk = p.K / BK;

  load_global(0);
  store_lds(0);
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const int stage = kt & 1;
    if (kt + 1 < nk) load_global((kt + 1) * BK);
    const u32x4* la = lds[stage];
    const u32x4* lb = lds[stage] + BM * kChunks;
#pragma unroll
    for (int kk = 0; kk < kChunks / 2; ++kk) {
      const int ch = 2 * kk + (lane >> 5);
      u32x4 af[FM], bfr[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) af[i] = la[swz(wm0 + i * 32 + (lane & 31), ch)];
#pragma unroll
      for (int j = 0; j < FN; ++j) bfr[j] = lb[swz(wn0 + j * 32 + (lane & 31), ch)];
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) mma<KIND>(acc[i][j], af[i], bfr[j]);
    }
    if (kt + 1 < nk) store_lds(stage ^ 1);
    __syncthreads();
  }

  // ---- epilogue ----
  const float alpha = scaled(p.alpha, p.s, mat, p.alpha_spow);
  const float beta = scaled(p.beta, p.s, mat, p.beta_spow);
  const float gamma = p.gamma;
  const bool has_e = p.E != nullptr;
  const bool mirror = SYM && (tm != tn);

  TC* C = nullptr;
  const TC* E = nullptr;
  if (EPI == EPI_STORE) C = static_cast<TC*>(p.C) + static_cast<int64_t>(mat) * p.sC;
  if (has_e) E = static_cast<const TC*>(p.E) + static_cast<int64_t>(mat) * p.sE;

  MatDesc d{};
  float decay = 1.0f;
  if constexpr (EPI == EPI_UPDATE) {
    d = p.table[mat];
    decay = 1.0f - p.lr * p.wd;
  }

#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int c = n0 + wn0 + j * 32 + (lane & 31);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = m0 + wm0 + i * 32 + q * 8 + (lane >> 5) * 4 + e;
          if (r >= p.M || c >= p.N) continue;
          float v = alpha * acc[i][j][q * 4 + e];
          if (has_e) {
            const int64_t ei = static_cast<int64_t>(r) * p.lde + c;
            if constexpr (sizeof(TC) == 4) {
              v += beta * reinterpret_cast<const float*>(E)[ei];
            } else if constexpr (KIND == KIND_F32) {
              v += 0.0f;  // not instantiated
            } else {
              const unsigned short h = reinterpret_cast<const unsigned short*>(E)[ei];
              v += beta * ((EPI == EPI_UPDATE || !SYM) ? bf16_to_f32(h) : f16_to_f32(h));
            }
          }
          if (r == c) v += gamma;
          if constexpr (EPI == EPI_STORE) {
            const int64_t ci = static_cast<int64_t>(r) * p.ldc + c;
            const int64_t cm = static_cast<int64_t>(c) * p.ldc + r;
            if constexpr (sizeof(TC) == 4) {
              reinterpret_cast<float*>(C)[ci] = v;
              if (mirror) reinterpret_cast<float*>(C)[cm] = v;
            } else {
              const unsigned short h = SYM ? f32_to_f16(v) : f32_to_bf16(v);
              reinterpret_cast<unsigned short*>(C)[ci] = h;
              if (mirror) reinterpret_cast<unsigned short*>(C)[cm] = h;
            }
          } else {
            if (r < p.Mvalid && c < p.Nvalid) {
              const int64_t wi = d.transposed ? static_cast<int64_t>(c) * d.cols + r
                                              : static_cast<int64_t>(r) * d.cols + c;
              if (p.w_bf16) {
                unsigned short* W = static_cast<unsigned short*>(d.W);
                W[wi] = f32_to_bf16(bf16_to_f32(W[wi]) * decay - p.lr * v);
              } else {
                float* W = static_cast<float*>(d.W);
                W[wi] = W[wi] * decay - p.lr * v;
              }
            }
          }
        }
      }
    }
  }
}

template <int KIND, int T, bool NN, bool SYM, int EPI, typename TC>
hipError_t launch_cfg(const GemmParams& p, hipStream_t st) {
  dim3 grid(p.tiles, p.count);
  if (T == 128) {
    hipLaunchKernelGGL((gemm_kernel<KIND, 128, 128, 2, 2, NN, SYM, EPI, TC>), grid, dim3(kThreads), 0, st, p);
  } else {
    hipLaunchKernelGGL((gemm_kernel<KIND, 64, 64, 2, 2, NN, SYM, EPI, TC>), grid, dim3(kThreads), 0, st, p);
  }
  return hipGetLastError();
}

template <int KIND, bool NN, bool SYM, int EPI, typename TC>
hipError_t launch_tile(int tile, const GemmParams& p, hipStream_t st) {
  if (tile == 128) return launch_cfg<KIND, 128, NN, SYM, EPI, TC>(p, st);
  return launch_cfg<KIND, 64, NN, SYM, EPI, TC>(p, st);
}

}  // namespace

hipError_t launch_gemm(GemmOp op, bool ns_f32, int tile, const GemmParams& p, hipStream_t st) {
  if (p.tiles <= 0 || p.count <= 0) return hipSuccess;
  if (ns_f32) {
    switch (op) {
      case OP_SYRK:
      case OP_SQUARE: return launch_tile<KIND_F32, false, true, EPI_STORE, float>(tile, p, st);
      case OP_APPLY: return launch_tile<KIND_F32, true, false, EPI_STORE, float>(tile, p, st);
      case OP_UPDATE: return launch_tile<KIND_F32, true, false, EPI_UPDATE, float>(tile, p, st);
    }
  } else {
    switch (op) {
      case OP_SYRK: return launch_tile<KIND_BF16, false, true, EPI_STORE, unsigned short>(tile, p, st);
      case OP_SQUARE: return launch_tile<KIND_F16, false, true, EPI_STORE, unsigned short>(tile, p, st);
      case OP_APPLY: return launch_tile<KIND_F16, true, false, EPI_STORE, unsigned short>(tile, p, st);
      case OP_UPDATE: return launch_tile<KIND_F16, true, false, EPI_UPDATE, unsigned short>(tile, p, st);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace muon
