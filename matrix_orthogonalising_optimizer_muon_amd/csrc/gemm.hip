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
#include <type_traits>

#include "internal.hpp"

namespace muon {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

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
__global__ __launch_bounds__(64 * WM * WN) void gemm_kernel(const GemmParams p) {
  constexpr int NT = 64 * WM * WN;                     // threads
  constexpr int ES = (KIND == KIND_F32) ? 4 : 2;      // element bytes in LDS / MFMA
  constexpr int VEC = 16 / ES;                         // elements per 16-byte chunk
  constexpr int BK = kChunks * VEC;                    // k per LDS slice (128 bytes)
  constexpr int TWM = BM / WM, TWN = BN / WN;          // wave tile
  constexpr int FM = TWM / 32, FN = TWN / 32;          // 32x32 MFMA blocks per wave
  static_assert(FM >= 1 && FN >= 1, "wave tile");
  constexpr int A_CH = (BM * kChunks + NT - 1) / NT;   // A chunks per thread
  constexpr int B_CH = (BN * kChunks + NT - 1) / NT;   // NT B chunks per thread
  // NN: the BK x BN slice of row-major B is cut into half-blocks of VEC/2 k-rows by VEC
  // n-columns; each is transposed in registers into VEC 8-byte k-runs.
  constexpr int HR = VEC / 2;
  constexpr int N_HB = (BK / HR) * (BN / VEC);
  constexpr int HB_T = (N_HB + NT - 1) / NT;
  constexpr int KSTEPS = kChunks / 2;                  // MFMA k-steps per slice

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

  // Global offsets (bytes, without k) of the chunks this thread stages. Rows past M or N
  // are clamped to the last valid row: they only feed output rows/columns that are never
  // stored, so the loads need no branches.
  int64_t a_off[A_CH];
#pragma unroll
  for (int i = 0; i < A_CH; ++i) {
    const int c = min(tid + i * NT, BM * kChunks - 1);
    const int gr = min(m0 + c / kChunks, p.M - 1);
    a_off[i] = (static_cast<int64_t>(gr) * p.lda + (c % kChunks) * VEC) * ES;
  }
  int64_t b_off[NN ? HB_T : B_CH];
  if constexpr (!NN) {
#pragma unroll
    for (int i = 0; i < B_CH; ++i) {
      const int c = min(tid + i * NT, BN * kChunks - 1);
      const int gr = min(n0 + c / kChunks, p.N - 1);
      b_off[i] = (static_cast<int64_t>(gr) * p.ldb + (c % kChunks) * VEC) * ES;
    }
  } else {
#pragma unroll
    for (int i = 0; i < HB_T; ++i) {
      const int hb = min(tid + i * NT, N_HB - 1);
      const int nb = hb % (BN / VEC), hk = hb / (BN / VEC);
      const int gn = min(n0 + nb * VEC, p.N - VEC);
      b_off[i] = (static_cast<int64_t>(hk * HR) * p.ldb + gn) * ES;
    }
  }

  u32x4 ra[A_CH];
  u32x4 rb[NN ? HB_T * HR : B_CH];

  auto load_global = [&](int k0) {
    const int64_t ka = static_cast<int64_t>(k0) * ES;
#pragma unroll
    for (int i = 0; i < A_CH; ++i) ra[i] = *reinterpret_cast<const u32x4*>(Ab + a_off[i] + ka);
    if constexpr (!NN) {
#pragma unroll
      for (int i = 0; i < B_CH; ++i) rb[i] = *reinterpret_cast<const u32x4*>(Bb + b_off[i] + ka);
    } else {
      const int64_t kb = static_cast<int64_t>(k0) * p.ldb * ES;
#pragma unroll
      for (int i = 0; i < HB_T; ++i)
#pragma unroll
        for (int r = 0; r < HR; ++r)
          rb[i * HR + r] = *reinterpret_cast<const u32x4*>(Bb + b_off[i] + kb + static_cast<int64_t>(r) * p.ldb * ES);
    }
  };

  auto store_lds = [&](int stage) {
    u32x4* la = lds[stage];
    u32x4* lb = lds[stage] + BM * kChunks;
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
      const int c = tid + i * NT;
      if ((BM * kChunks) % NT == 0 || c < BM * kChunks) la[swz(c / kChunks, c % kChunks)] = ra[i];
    }
    if constexpr (!NN) {
#pragma unroll
      for (int i = 0; i < B_CH; ++i) {
        const int c = tid + i * NT;
        if ((BN * kChunks) % NT == 0 || c < BN * kChunks) lb[swz(c / kChunks, c % kChunks)] = rb[i];
      }
    } else {
#pragma unroll
      for (int i = 0; i < HB_T; ++i) {
        const int hb = tid + i * NT;
        if (N_HB % NT != 0 && hb >= N_HB) continue;
        const int nb = hb % (BN / VEC), hk = hb / (BN / VEC);
        const int kb = hk >> 1, half = hk & 1;
        if constexpr (KIND == KIND_F16) {
          // 4 bf16 rows of 8 -> scaled fp16, then 8 columns of 4 k-values.
          unsigned int w[4][4];
#pragma unroll
          for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const unsigned int x = rb[i * HR + r][q];
              const float lo = __uint_as_float(x << 16) * bscale;
              const float hi = __uint_as_float(x & 0xFFFF0000u) * bscale;
              w[r][q] = static_cast<unsigned int>(f32_to_f16(lo)) |
                        (static_cast<unsigned int>(f32_to_f16(hi)) << 16);
            }
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            // columns 2q (low halves) and 2q+1 (high halves) of the 4 rows
            const u32x2 lo{__builtin_amdgcn_perm(w[1][q], w[0][q], 0x05040100u),
                           __builtin_amdgcn_perm(w[3][q], w[2][q], 0x05040100u)};
            const u32x2 hi{__builtin_amdgcn_perm(w[1][q], w[0][q], 0x07060302u),
                           __builtin_amdgcn_perm(w[3][q], w[2][q], 0x07060302u)};
            reinterpret_cast<u32x2*>(&lb[swz(nb * 8 + 2 * q, kb)])[half] = lo;
            reinterpret_cast<u32x2*>(&lb[swz(nb * 8 + 2 * q + 1, kb)])[half] = hi;
          }
        } else {
          static_assert(KIND == KIND_F32, "NN operand kinds");
          // 2 fp32 rows of 4 -> 4 columns of 2 k-values.
          const u32x4 x0 = rb[i * HR], x1 = rb[i * HR + 1];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const u32x2 v{__float_as_uint(__uint_as_float(x0[j]) * bscale),
                          __float_as_uint(__uint_as_float(x1[j]) * bscale)};
            reinterpret_cast<u32x2*>(&lb[swz(nb * 4 + j, kb)])[half] = v;
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

  u32x4 fa[2][FM], fb[2][FN];
  auto load_frags = [&](int buf, const u32x4* la, const u32x4* lb, int kk) {
    const int ch = 2 * kk + (lane >> 5);
#pragma unroll
    for (int i = 0; i < FM; ++i) fa[buf][i] = la[swz(wm0 + i * 32 + (lane & 31), ch)];
#pragma unroll
    for (int j = 0; j < FN; ++j) fb[buf][j] = lb[swz(wn0 + j * 32 + (lane & 31), ch)];
  };

  // One 128-byte slice of K: fragments double-buffered across the k-steps; the staged
  // next slice goes to the other LDS buffer half-way through.
  auto slice = [&](int kt, auto has_next_tag) {
    constexpr bool HAS_NEXT = decltype(has_next_tag)::value;
    const int stage = kt & 1;
    const u32x4* la = lds[stage];
    const u32x4* lb = lds[stage] + BM * kChunks;
    if constexpr (HAS_NEXT) load_global((kt + 1) * BK);
    load_frags(0, la, lb, 0);
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) {
      if (kk + 1 < KSTEPS) load_frags((kk + 1) & 1, la, lb, kk + 1);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) mma<KIND>(acc[i][j], fa[kk & 1][i], fb[kk & 1][j]);
      if constexpr (HAS_NEXT) {
        if (kk == KSTEPS / 2 - 1) store_lds(stage ^ 1);
      }
    }
    __syncthreads();
  };

  load_global(0);
  store_lds(0);
  __syncthreads();
  for (int kt = 0; kt + 1 < nk; ++kt) slice(kt, std::true_type{});
  slice(nk - 1, std::false_type{});

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

template <int KIND, int BM, int BN, int WM, int WN, bool NN, bool SYM, int EPI, typename TC>
hipError_t launch_shape(const GemmParams& p, hipStream_t st) {
  hipLaunchKernelGGL((gemm_kernel<KIND, BM, BN, WM, WN, NN, SYM, EPI, TC>), dim3(p.tiles, p.count),
                     dim3(64 * WM * WN), 0, st, p);
  return hipGetLastError();
}

template <int KIND, bool NN, bool SYM, int EPI, typename TC>
hipError_t launch_tile(int cfg, const GemmParams& p, hipStream_t st) {
  switch (cfg) {
    case TILE_64: return launch_shape<KIND, 64, 64, 2, 2, NN, SYM, EPI, TC>(p, st);
    case TILE_128: return launch_shape<KIND, 128, 128, 2, 2, NN, SYM, EPI, TC>(p, st);
    case TILE_256:  // 8 waves (2 per SIMD), wave tile 128 x 64
      if constexpr (KIND != KIND_F32) return launch_shape<KIND, 256, 256, 2, 4, NN, SYM, EPI, TC>(p, st);
      return hipErrorInvalidValue;
    case TILE_256x128:  // 8 waves, wave tile 64 x 64
      if constexpr (!SYM && KIND != KIND_F32) return launch_shape<KIND, 256, 128, 4, 2, NN, SYM, EPI, TC>(p, st);
      return hipErrorInvalidValue;
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_gemm(GemmOp op, bool ns_f32, int cfg, const GemmParams& p, hipStream_t st) {
  if (p.tiles <= 0 || p.count <= 0) return hipSuccess;
  if (ns_f32) {
    switch (op) {
      case OP_SYRK:
      case OP_SQUARE: return launch_tile<KIND_F32, false, true, EPI_STORE, float>(cfg, p, st);
      case OP_APPLY: return launch_tile<KIND_F32, true, false, EPI_STORE, float>(cfg, p, st);
      case OP_UPDATE: return launch_tile<KIND_F32, true, false, EPI_UPDATE, float>(cfg, p, st);
    }
  } else {
    switch (op) {
      case OP_SYRK: return launch_tile<KIND_BF16, false, true, EPI_STORE, unsigned short>(cfg, p, st);
      case OP_SQUARE: return launch_tile<KIND_F16, false, true, EPI_STORE, unsigned short>(cfg, p, st);
      case OP_APPLY: return launch_tile<KIND_F16, true, false, EPI_STORE, unsigned short>(cfg, p, st);
      case OP_UPDATE: return launch_tile<KIND_F16, true, false, EPI_UPDATE, unsigned short>(cfg, p, st);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace muon
