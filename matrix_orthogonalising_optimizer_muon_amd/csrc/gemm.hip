// Batched MFMA GEMM family for the Newton-Schulz products on gfx950 (CDNA4).
//
// Every contraction of the update is an NT product C = A B^T with both operands stored
// K-contiguous (row-major, K = row length):
//   * X X^T, the Gram matrix (DMuon summary, section 2.2: the symmetric Gram product):
//     only upper tiles are computed, off-diagonal tiles are stored twice (mirrored);
//   * the m' x m' products of the Gram recurrence and A^2 (MuonX article, section 3.2):
//     every operand is exactly symmetric in storage, so A B = A B^T, and every result is
//     symmetric in exact arithmetic: symmetric output as above;
//   * the long "apply" product Q X, computed as Q (X^T)^T from the transposed copy X^T
//     the previous stage keeps; its epilogue writes X' in both layouts (and adds a*X for
//     plain NS), or, for the last product, updates W in place.
//
// Layout: a workgroup of WM x WN waves (64 lanes each) owns a BM x BN output tile; each
// wave a (BM/WM) x (BN/WN) sub-tile of 32x32x16 (bf16/fp16) or 32x32x2 (fp32) MFMA blocks
// with fp32 accumulators. K advances in 128-byte slices, double-buffered in LDS and
// staged through registers: the global loads of slice k + PF (PF = 1 or 2) are issued
// before slice k's MFMAs, and slice k + 1 is written to the other LDS buffer half-way
// through them. Fragments are double-buffered across the k-steps of a slice. LDS rows are 8 chunks of 16 bytes,
// XOR-swizzled per row so that fragment reads of 32 consecutive rows spread over all
// banks.
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

// The same for LDS rows of CH chunks (CH = 8: 128-byte rows as above; CH = 4: 64-byte
// rows, two per 128 bytes, where rows 2t and 2t+1 share the XOR term so that 8
// consecutive rows read at one logical chunk still cover all eight 16-byte positions of a
// 128-byte span).
template <int CH>
__device__ __forceinline__ int swz_bits(int row) {
  static_assert(CH == 8 || CH == 4, "chunks per row");
  return CH == 8 ? ((row ^ (row >> 3)) & 7) : ((row >> 1) & 3);
}
template <int CH>
__device__ __forceinline__ int swz_ch(int row, int chunk) {
  return row * CH + (chunk ^ swz_bits<CH>(row));
}

__device__ __forceinline__ unsigned short f32_to_f16(float f) {
  _Float16 h = static_cast<_Float16>(f);
  return __builtin_bit_cast(unsigned short, h);
}
__device__ __forceinline__ float f16_to_f32(unsigned short h) {
  return static_cast<float>(__builtin_bit_cast(_Float16, h));
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

// Output element type of a stage: fp32 on the fp32 path, fp16 on the bf16 path.
template <int KIND>
struct OutT {
  using T = typename std::conditional<KIND == KIND_F32, float, unsigned short>::type;
};

template <typename T>
__device__ __forceinline__ T to_out(float v) {
  if constexpr (sizeof(T) == 4) return v;
  else return f32_to_f16(v);
}
template <typename T>
__device__ __forceinline__ float from_out(T v) {
  if constexpr (sizeof(T) == 4) return v;
  else return f16_to_f32(v);
}

// 4 consecutive elements at p (8 or 16 bytes; offsets are multiples of 4 elements).
template <typename T>
__device__ __forceinline__ void load4(const T* p, float (&v)[4]) {
  if constexpr (sizeof(T) == 4) {
    const float4 x = *reinterpret_cast<const float4*>(p);
    v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
  } else {
    const u32x2 x = *reinterpret_cast<const u32x2*>(p);
    v[0] = f16_to_f32(x.x & 0xFFFFu); v[1] = f16_to_f32(x.x >> 16);
    v[2] = f16_to_f32(x.y & 0xFFFFu); v[3] = f16_to_f32(x.y >> 16);
  }
}
template <typename T>
__device__ __forceinline__ void store4(T* p, const float (&v)[4], float scale) {
  if constexpr (sizeof(T) == 4) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0] * scale, v[1] * scale, v[2] * scale, v[3] * scale);
  } else {
    const u32x2 x{static_cast<unsigned int>(f32_to_f16(v[0] * scale)) |
                      (static_cast<unsigned int>(f32_to_f16(v[1] * scale)) << 16),
                  static_cast<unsigned int>(f32_to_f16(v[2] * scale)) |
                      (static_cast<unsigned int>(f32_to_f16(v[3] * scale)) << 16)};
    *reinterpret_cast<u32x2*>(p) = x;
  }
}

// W element (r, c) of the canonical orientation through the descriptor: a transposed W
// holds the canonical column contiguously, so the 4 rows r0..r0+3 of a block are one
// 16-byte access when W is fp32 and aligned.
__device__ __forceinline__ int64_t w_index(const MatDesc& d, int r, int c) {
  return d.transposed ? static_cast<int64_t>(c) * d.cols + r : static_cast<int64_t>(r) * d.cols + c;
}
__device__ __forceinline__ bool w_vec(const GemmParams& p, const MatDesc& d) {
  return d.transposed && !p.w_bf16 && (d.cols % 4) == 0 && (reinterpret_cast<uintptr_t>(d.W) % 16) == 0;
}
// Load W at rows r0..r0+3 of column c (zero outside the valid region).
__device__ __forceinline__ void w_load4(const GemmParams& p, const MatDesc& d, bool vec, int r0, int c,
                                        float* w) {
  const bool cin = c < p.Nvalid;
  if (vec && cin && r0 + 3 < p.Mvalid) {
    const float4 x = *reinterpret_cast<const float4*>(static_cast<const float*>(d.W) + w_index(d, r0, c));
    w[0] = x.x; w[1] = x.y; w[2] = x.z; w[3] = x.w;
    return;
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const bool ok = cin && r0 + e < p.Mvalid;
    const int64_t wi = ok ? w_index(d, r0 + e, c) : 0;
    w[e] = !ok ? 0.0f
               : (p.w_bf16 ? bf16_to_f32(static_cast<const unsigned short*>(d.W)[wi])
                           : static_cast<const float*>(d.W)[wi]);
  }
}
// W <- W*decay - lr*o at rows r0..r0+3 of column c, given the loaded w.
__device__ __forceinline__ void w_store4(const GemmParams& p, const MatDesc& d, bool vec, float decay,
                                         int r0, int c, const float* w, const float (&o)[4]) {
  if (c >= p.Nvalid) return;
  float n[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) n[e] = w[e] * decay - p.lr * o[e];
  if (vec && r0 + 3 < p.Mvalid) {
    *reinterpret_cast<float4*>(static_cast<float*>(d.W) + w_index(d, r0, c)) = make_float4(n[0], n[1], n[2], n[3]);
    return;
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    if (r0 + e >= p.Mvalid) continue;
    const int64_t wi = w_index(d, r0 + e, c);
    if (p.w_bf16) static_cast<unsigned short*>(d.W)[wi] = f32_to_bf16(n[e]);
    else static_cast<float*>(d.W)[wi] = n[e];
  }
}

// Matrix and tile of this workgroup: XCD-aware remap, then grouped (8-tile-row) ordering for
// general outputs or an upper-triangle walk for symmetric ones.
template <bool SYM>
__device__ __forceinline__ void tile_coords(const GemmParams& p, int& mat, int& tm, int& tn) {
  // Workgroups are dealt round-robin to the 8 XCDs in the order of their linear id
  // (x fastest, then y = matrix): workgroup i runs on XCD i % 8. Give each XCD a contiguous
  // run of the launch's logical (matrix, tile) sequence, so neighbouring tiles (shared
  // operand panels) share one L2. XCD x holds nwg/8 of them, plus one if x < nwg % 8.
  const int i = blockIdx.x + blockIdx.y * gridDim.x;
  const int nwg = gridDim.x * gridDim.y;
  const int x = i & 7, q = nwg >> 3, r = nwg & 7;
  const int tt = x * q + min(x, r) + (i >> 3);
  mat = tt / p.tiles;
  int t = tt - mat * p.tiles;
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
    const int r2 = t - g * group;
    tm = first + r2 % gm;
    tn = r2 / gm;
  }
}

// Epilogue chunks: CR block rows x CC block columns of a wave's FM x FN blocks, holding
// at most V loaded values (16 per block) per lane, CR and CC dividing FM and FN.
constexpr int largest_divisor_le(int n, int cap) {
  int best = 1;
  for (int d = 1; d <= n; ++d)
    if (n % d == 0 && d <= cap) best = d;
  return best;
}
constexpr int chunk_cols(int FN, int V) { return FN * 16 <= V ? FN : largest_divisor_le(FN, V / 16); }
constexpr int chunk_rows(int FM, int FN, int V) {
  return FN * 16 <= V ? largest_divisor_le(FM, V / (FN * 16)) : 1;
}

// Epilogue shared by both kernels: per 32x32 block a lane holds column c and rows
// r0..r0+3 for q = 0..3 (acc[i][j][4q + e] is row r0 + e).
// The W update loads every W value of a chunk of block rows before computing and storing
// them, so a wave pays one memory round trip per chunk instead of one per block; a chunk
// holds at most 64 (8-wave tiles: 32) W values per lane to stay within the register file.
template <int KIND, int BM, int BN, int WM, int WN, bool SYM, int EPI, int FM, int FN, typename TO,
          bool STG = false>
__device__ __forceinline__ void epilogue(const GemmParams& p, f32x16 (&acc)[FM][FN], int mat, int tm,
                                         int tn, int m0, int n0, int wm0, int wn0, int lane,
                                         const float* ecap = nullptr, bool use_cap = false,
                                         unsigned short* stg = nullptr) {
  const float alpha = scaled(p.alpha, p.s, mat, p.alpha_spow);
  const float beta = scaled(p.beta, p.s, mat, p.beta_spow);
  const float gamma = p.gamma;
  const bool has_e = p.E != nullptr;
  const bool mirror = SYM && (tm != tn);
  // Staged transposed output of the apply (the direct-load kernels pass their LDS, 16-bit
  // outputs): block of TWN rows of TWM values per wave, rows SPITCH values apart (16-byte
  // aligned).
  constexpr int TWM = BM / WM, TWN = BN / WN;
  constexpr int SPITCH = TWM + 8;
  constexpr bool STAGED = STG && sizeof(TO) == 2 && EPI == EPI_APPLY && !SYM;
  const bool tout = (SYM && mirror) || (EPI == EPI_APPLY && p.C2 != nullptr);

  TO* C = nullptr;
  TO* C2 = nullptr;
  const TO* E = nullptr;
  if (EPI != EPI_UPDATE) C = static_cast<TO*>(p.C) + static_cast<int64_t>(mat) * p.sC;
  if (EPI == EPI_APPLY && p.C2 != nullptr) C2 = static_cast<TO*>(p.C2) + static_cast<int64_t>(mat) * p.sC2;
  if (has_e) E = static_cast<const TO*>(p.E) + static_cast<int64_t>(mat) * p.sE;

  // E at rows r0..r0+3 of column c (the caller keeps r0 < M and c < N).
  auto load_e = [&](int r0, int c, float* ev) {
    if (p.e_trans) {
      float t[4];
      load4(E + static_cast<int64_t>(c) * p.lde + r0, t);
#pragma unroll
      for (int e = 0; e < 4; ++e) ev[e] = t[e];
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) ev[e] = from_out(E[static_cast<int64_t>(r0 + e) * p.lde + c]);
    }
  };
  // v = alpha acc + beta E + gamma I for rows r0..r0+3 of column c of block (i, j), with E
  // already loaded into ev.
  auto value_ev = [&](int i, int j, int q, int r0, int c, const float* ev, float (&v)[4]) {
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = alpha * acc[i][j][q * 4 + e];
    if (has_e) {
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] += beta * ev[e];
    }
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (r0 + e == c) v[e] += gamma;
  };

  if constexpr (EPI == EPI_UPDATE) {
    const MatDesc d = p.table[mat];
    const float decay = 1.0f - p.lr * p.wd;
    const bool vec = w_vec(p, d);
    constexpr int WB = (WM * WN >= 8) ? 32 : 64;  // W values per lane per chunk
    constexpr int IG = (FN * 16 >= WB) ? 1 : largest_divisor_le(FM, WB / (FN * 16));
#pragma unroll
    for (int i0 = 0; i0 < FM; i0 += IG) {
      float w[IG][FN][16];
#pragma unroll
      for (int ii = 0; ii < IG; ++ii)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int c = n0 + wn0 + j * 32 + (lane & 31);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int r0 = m0 + wm0 + (i0 + ii) * 32 + q * 8 + (lane >> 5) * 4;
            w_load4(p, d, vec, r0, c, &w[ii][j][4 * q]);
          }
        }
#pragma unroll
      for (int ii = 0; ii < IG; ++ii)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int c = n0 + wn0 + j * 32 + (lane & 31);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int r0 = m0 + wm0 + (i0 + ii) * 32 + q * 8 + (lane >> 5) * 4;
            if (r0 >= p.M || c >= p.N) continue;
            // The E term (plain NS: a X) is loaded here, after the chunk's W loads: loading
            // it with them measured slower on the 2048 x 2048 plain-NS update.
            float ev[4] = {0.0f, 0.0f, 0.0f, 0.0f};
            if (has_e) load_e(r0, c, ev);
            float v[4];
            value_ev(i0 + ii, j, q, r0, c, ev, v);
            w_store4(p, d, vec, decay, r0, c, &w[ii][j][4 * q], v);
          }
        }
    }
  } else {
    // With an E term, every E value of a chunk of block rows is loaded before any of the
    // chunk's stores: the compiler cannot tell C from E, so a load placed after a store
    // waits for it, and block by block each wave would pay one memory round trip per block.
    // E values per lane per chunk: 64 for 4-wave tiles, 48 for 8-wave tiles, one block (16)
    // for 128 x 128 wave tiles, whose accumulators fill the register file.
    constexpr int EB = FM * FN >= 16 ? 16 : (WM * WN >= 8 ? 48 : 64);
    constexpr int EG = chunk_rows(FM, FN, EB), EJ = chunk_cols(FN, EB);
    const float os = (EPI == EPI_APPLY) ? p.oscale : 1.0f;
#pragma unroll
    for (int i0 = 0; i0 < FM; i0 += EG)
#pragma unroll
    for (int j0 = 0; j0 < FN; j0 += EJ) {
      float ev[EG][EJ][16];
      if (has_e && use_cap) {
        // E was read from LDS during the main loop (gemm_dma_kernel, E = A)
#pragma unroll
        for (int ii = 0; ii < EG; ++ii)
#pragma unroll
          for (int jj = 0; jj < EJ; ++jj)
#pragma unroll
            for (int e = 0; e < 16; ++e) ev[ii][jj][e] = ecap[((i0 + ii) * FN + j0 + jj) * 16 + e];
      } else if (has_e) {
#pragma unroll
        for (int ii = 0; ii < EG; ++ii)
#pragma unroll
          for (int jj = 0; jj < EJ; ++jj) {
            const int c = n0 + wn0 + (j0 + jj) * 32 + (lane & 31);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int r0 = m0 + wm0 + (i0 + ii) * 32 + q * 8 + (lane >> 5) * 4;
              if (r0 < p.M && c < p.N) load_e(r0, c, &ev[ii][jj][4 * q]);
            }
          }
      }
#pragma unroll
      for (int ii = 0; ii < EG; ++ii) {
        const int i = i0 + ii;
#pragma unroll
        for (int jj = 0; jj < EJ; ++jj) {
          const int j = j0 + jj;
          const int c = n0 + wn0 + j * 32 + (lane & 31);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int r0 = m0 + wm0 + i * 32 + q * 8 + (lane >> 5) * 4;
            // M and N are multiples of 4: rows r0..r0+3 are all in range or all out.
            if (r0 >= p.M || c >= p.N) continue;
            float v[4];
            value_ev(i, j, q, r0, c, &ev[ii][jj][4 * q], v);
#pragma unroll
            for (int e = 0; e < 4; ++e) C[static_cast<int64_t>(r0 + e) * p.ldc + c] = to_out<TO>(v[e] * os);
            if constexpr (STAGED) {
              // the same rounded values, transposed, into the wave's LDS block (8 bytes)
              if (tout) store4(stg + (j * 32 + (lane & 31)) * SPITCH + i * 32 + q * 8 + (lane >> 5) * 4, v, os);
            } else {
              if (SYM && mirror) store4(C + static_cast<int64_t>(c) * p.ldc + r0, v, 1.0f);
              if (EPI == EPI_APPLY && C2 != nullptr) store4(C2 + static_cast<int64_t>(c) * p.ldc2 + r0, v, os);
            }
          }
        }
      }
    }
    if constexpr (STAGED) {
      // The transposed output X'^T of an apply leaves from the wave's LDS block in whole
      // rows: 16 bytes per lane, TWM / 8 lanes per output row, instead of 8-byte pieces
      // scattered over 32 rows per instruction. Each wave reads only its own block, which
      // its own lanes wrote.
      if (tout) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        TO* dst = C2;
        const int64_t ld = p.ldc2;
        constexpr int CPR = TWM / 8;            // 16-byte chunks per output row
        constexpr int TOTAL = TWN * CPR;
        static_assert(TOTAL % 64 == 0, "whole instructions");
#pragma unroll
        for (int t = 0; t < TOTAL / 64; ++t) {
          const int idx = t * 64 + lane;
          const int cl = idx / CPR, ch = idx % CPR;
          const int grow = n0 + wn0 + cl, gcol = m0 + wm0 + ch * 8;
          if (grow < p.N && gcol < p.M) {
            const u32x4 w = *reinterpret_cast<const u32x4*>(stg + cl * SPITCH + ch * 8);
            *reinterpret_cast<u32x4*>(dst + static_cast<int64_t>(grow) * ld + gcol) = w;
          }
        }
      }
    }
  }
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding: vmcnt in bits
// 3:0 and 15:14; expcnt 6:4 and lgkmcnt 11:8 left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// The same, and every LDS access of this wave returned (lgkmcnt 0).
// Buffer resource over `bytes` bytes from `base` (raw buffer: no stride, no format
// conversion; accesses at or past `bytes` return zero instead of faulting).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes), 0x00020000);
}
// 16 bytes per lane from the buffer at voff + soff into LDS: lane l writes bytes
// [16 l, 16 l + 16) of the instruction's window at lds_dst (the M0 base).
__device__ __forceinline__ void buf_load_lds(__amdgpu_buffer_rsrc_t r, void* lds_dst, uint32_t voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_dst, 16, voff, soff, 0, 0);
}

template <int N>
__device__ __forceinline__ void wait_vmcnt_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}

// Same product as gemm_kernel, with operands moved global -> LDS by the CDNA4 direct
// loads (16 bytes per lane, lane l writing LDS bytes [16 l, 16 l + 16) of the
// instruction's 1 KB window = 64 / CH rows of CH 16-byte chunks). The XOR swizzle moves
// to the global side: lane l of a window loads logical chunk (l % CH) ^ f(row). NS LDS
// stages form a ring; while slice k is computed, slices k + 1 .. k + NS - 1 are in flight
// or landed, so no staging registers are needed. A slice is CH chunks of K per row:
// CH = 4 halves the slice, so twice as many stages fit in the same LDS and more load
// latency is covered. With KS = 2 the two k-groups of waves take alternate k-steps of
// every slice and add their partial sums through LDS at the end.
template <int KIND, int BM, int BN, int WM, int WN, int NS, int KS, int CH, bool SYM, int EPI, int TAG>
__global__ __launch_bounds__(64 * WM * WN * KS) void gemm_dma_kernel(const GemmParams p) {
  using TO = typename OutT<KIND>::T;
  constexpr int NWC = WM * WN;                             // waves per k-group (one tile each)
  constexpr int NW = NWC * KS;                             // waves
  constexpr int ES = (KIND == KIND_F32) ? 4 : 2;
  constexpr int VEC = 16 / ES;
  constexpr int BK = CH * VEC;
  constexpr int TWM = BM / WM, TWN = BN / WN;
  constexpr int FM = TWM / 32, FN = TWN / 32;
  constexpr int RPI = 64 / CH;                             // rows per load instruction
  constexpr int IA = BM / (RPI * NW), IB = BN / (RPI * NW);  // load instructions per wave
  static_assert(IA * RPI * NW == BM && IB * RPI * NW == BN, "rows per wave");
  constexpr int STAGE = (BM + BN) * CH;                    // u32x4 per stage
  constexpr int KSTEPS = CH / 2;
  constexpr int KL = KSTEPS / KS;                          // k-steps per wave per slice
  constexpr int D = NS - 1;                                // slices in flight
  static_assert(NS >= 2 && (KS == 1 || KS == 2), "stages / k-groups");
  static_assert(KS == 1 || (KS / 2) * BM * BN * 4 <= NS * STAGE * 16, "k-group reduction fits in LDS");

  // The apply epilogue reuses the LDS for its staged transposed output (X'^T, 16-bit kinds):
  // one block of TWN rows x (TWM + 8) values per wave of k-group 0. (Staging the mirror
  // tile of the symmetric products the same way measured slightly slower: 28.7 -> 29.1 us
  // for the 2560 squares, against 133.5 -> 128.6 us for the 2560 x 9728 apply.)
  constexpr bool STG = KIND != KIND_F32 && EPI == EPI_APPLY && !SYM;
  constexpr int STG_U32X4 = STG ? (NWC * TWN * (TWM + 8) * 2 + 15) / 16 : 0;
  __shared__ u32x4 lds[NS * STAGE > STG_U32X4 ? NS * STAGE : STG_U32X4];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // Wave-uniform (scalar): every LDS window address derived from it stays in SGPRs, so a
  // load's M0 is set by scalar arithmetic.
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kgrp = wave / NWC;     // which k-steps of every slice this wave computes
  const int wloc = wave % NWC;     // which wave tile of the output
  int mat, tm, tn;
  tile_coords<SYM>(p, mat, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;

  const char* Ab = static_cast<const char*>(p.A) + static_cast<int64_t>(mat) * p.sA * ES;
  const char* Bb = static_cast<const char*>(p.B) + static_cast<int64_t>(mat) * p.sB * ES;

  // Operands are read as buffers over this matrix's A and B: a lane's byte offset within
  // the matrix (32 bits; the host runs these kernels only where every operand is under
  // 4 GiB) plus the slice's K offset as the scalar offset, so a load needs no per-lane
  // address arithmetic.
  uint32_t a_off[IA], b_off[IB];
#pragma unroll
  for (int j = 0; j < IA; ++j) {
    const int row = (wave * IA + j) * RPI + lane / CH;
    const int chunk = (lane % CH) ^ swz_bits<CH>(row);
    const int gr = min(m0 + row, p.M - 1);
    a_off[j] = static_cast<uint32_t>((static_cast<int64_t>(gr) * p.lda + chunk * VEC) * ES);
  }
#pragma unroll
  for (int j = 0; j < IB; ++j) {
    const int row = (wave * IB + j) * RPI + lane / CH;
    const int chunk = (lane % CH) ^ swz_bits<CH>(row);
    const int gr = min(n0 + row, p.N - 1);
    b_off[j] = static_cast<uint32_t>((static_cast<int64_t>(gr) * p.ldb + chunk * VEC) * ES);
  }
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(Ab, static_cast<uint32_t>(static_cast<int64_t>(p.M) * p.lda * ES));
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(Bb, static_cast<uint32_t>(static_cast<int64_t>(p.N) * p.ldb * ES));

  auto issue = [&](int stage, int k0) {
    const int kb = k0 * ES;
    u32x4* sa = lds + stage * STAGE;
    u32x4* sb = sa + BM * CH;
#pragma unroll
    for (int j = 0; j < IA; ++j) buf_load_lds(ra, sa + (wave * IA + j) * RPI * CH, a_off[j], kb);
#pragma unroll
    for (int j = 0; j < IB; ++j) buf_load_lds(rb, sb + (wave * IB + j) * RPI * CH, b_off[j], kb);
  };

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  const int wm0 = (wloc / WN) * TWM;
  const int wn0 = (wloc % WN) * TWN;
  const int nk = p.K / BK;
  const int kk0 = kgrp * KL;

  // E = A (the P epilogue of R^2 and A^2, square products): the slice of A holding K
  // columns n0 + wn0 .. n0 + wn0 + TWN - 1 (one slice: BK == TWN) carries exactly the E
  // values of this wave's output block (E(r, c) = A(r, c)), so they are read from LDS while
  // that slice is resident instead of from global memory in the epilogue. Only the waves
  // that run the epilogue (k-group 0) capture; a wave whose columns lie past N stores
  // nothing and captures nothing.
  constexpr bool CAP = SYM && EPI == EPI_STORE && KIND == KIND_F16 && BK == TWN && FM * FN <= 4;
  static_assert(!CAP || KL % 2 == 0, "the capture split is written for an even k-step count");
  float ecap[CAP ? FM * FN * 16 : 1];
  const bool cap = CAP && p.e_from_a && kgrp == 0 && n0 + wn0 < p.N;
  auto capture = [&](int kt) {
    if constexpr (CAP) {
      const unsigned short* la16 = reinterpret_cast<const unsigned short*>(lds + (kt % NS) * STAGE);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int k = j * 32 + (lane & 31);  // column within the slice
#pragma unroll
          for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int row = wm0 + i * 32 + q * 8 + (lane >> 5) * 4 + e;
              ecap[(i * FN + j) * 16 + q * 4 + e] = f16_to_f32(la16[swz_ch<CH>(row, k >> 3) * 8 + (k & 7)]);
            }
        }
    }
  };

  u32x4 fa[2][FM], fb[2][FN];
  auto load_frags = [&](int buf, const u32x4* la, const u32x4* lb, int kk) {
    const int ch = 2 * kk + (lane >> 5);
#pragma unroll
    for (int i = 0; i < FM; ++i) fa[buf][i] = la[swz_ch<CH>(wm0 + i * 32 + (lane & 31), ch)];
#pragma unroll
    for (int j = 0; j < FN; ++j) fb[buf][j] = lb[swz_ch<CH>(wn0 + j * 32 + (lane & 31), ch)];
  };

  // Prologue: slices 0 .. D-1 (clamped: past the end the last slice is reloaded into a
  // stage that is never read, so every slice issues the same number of loads), then slice
  // 0 is awaited, slice D goes to the one stage still unused and the first k-step's
  // fragments are read.
#pragma unroll
  for (int s0 = 0; s0 < D; ++s0) issue(s0, min(s0, nk - 1) * BK);
  wait_vmcnt<(D - 1) * (IA + IB)>();
  __builtin_amdgcn_s_barrier();
  issue(D, min(D, nk - 1) * BK);
  load_frags(0, lds, lds + BM * CH, kk0);

  // One slice: the MFMAs of every k-step run while the fragments of the next k-step are
  // read. Before the last k-step's MFMAs the workgroup synchronises once: this wave's
  // reads of the slice have returned (lgkmcnt 0) and its loads of the next slice have
  // landed; after the barrier the slice's stage is free for the loads of slice kt + NS
  // and the next slice's first fragments are read. So LDS read latency always hides
  // behind MFMAs. P is the fragment buffer of the slice's first k-step.
  auto slice = [&](int kt, auto par_tag, auto next_tag) {
    constexpr int P = decltype(par_tag)::value;
    constexpr bool NEXT = decltype(next_tag)::value;  // a slice follows (all but the last)
    constexpr int NMF = (KIND == KIND_F32 ? 4 : 1) * FM * FN;  // MFMA instructions per k-step
    const u32x4* la = lds + (kt % NS) * STAGE;
    const u32x4* lb = la + BM * CH;
#pragma unroll
    for (int kl = 0; kl < KL; ++kl) {
      const int cur = (P + kl) & 1;
      if (kl + 1 < KL) {
        load_frags(cur ^ 1, la, lb, kk0 + kl + 1);
      } else if constexpr (NEXT) {
        // Before the barrier: M0(first MFMA) R1 M0(rest) R2 M1 ... for the k-steps before
        // the last one, then nothing may move across.
#pragma unroll
        for (int kk = 0; kk + 1 < KL; ++kk) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, FM + FN, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, NMF - 1, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        wait_vmcnt_lgkm0<(D - 1) * (IA + IB)>();
        __builtin_amdgcn_s_barrier();
        const u32x4* na = lds + ((kt + 1) % NS) * STAGE;
        load_frags(cur ^ 1, na, na + BM * CH, kk0);
        issue(kt % NS, min(kt + NS, nk - 1) * BK);
      }
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) mma<KIND>(acc[i][j], fa[cur][i], fb[cur][j]);
    }
    // After the barrier: the next slice's first fragment reads, then the loads of slice
    // kt + NS one by one between the last k-step's MFMAs, so the MFMA pipe is fed while
    // the loads and their address and M0 set-up issue (issuing the loads as one block
    // ahead of the MFMAs left the pipe idle at every slice boundary: 3584 x 18944 apply
    // 505 -> 474 us, 3584 Gram product over K = 18944 390 -> 347 us). The fragment reads
    // come first in program order because the direct loads write LDS, which the compiler
    // does not move reads across. The last slice: the same pattern as before the barrier,
    // without the reads of a next slice. The first MFMA of a k-step goes ahead of the
    // reads because its fragments may still be in flight and the compiler waits for every
    // read issued before it.
    if constexpr (NEXT) {
      constexpr int NL = IA + IB;                  // load instructions per wave and slice
      constexpr int NP = NL < NMF ? NL : NMF;
      __builtin_amdgcn_sched_group_barrier(0x100, FM + FN, 0);
#pragma unroll
      for (int q = 0; q < NP; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      }
      if constexpr (NL > NP) __builtin_amdgcn_sched_group_barrier(0x010, NL - NP, 0);
      if constexpr (NMF > NP) __builtin_amdgcn_sched_group_barrier(0x008, NMF - NP, 0);
    } else {
#pragma unroll
      for (int kk = 0; kk + 1 < KL; ++kk) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, FM + FN, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, NMF - 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, NMF, 0);
    }
  };
  // The last slice is peeled off, so the steady-state loop has no branch around its
  // barrier (a control-flow join there makes the compiler wait for every LDS read,
  // including the next slice's, before the last k-step's MFMAs).
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using YES = std::true_type;
  using NO = std::false_type;
  if constexpr (KL % 2 == 0) {
    if (CAP && cap) {
      // The same slices and barriers as below, with the E reads before slice kcap. Slice
      // kcap has landed: the barrier of the slice before it (or of the prologue) waited for it.
      const int kcap = (n0 + wn0) / BK;  // < nk, as n0 + wn0 < N = K
      int kt = 0;
      for (; kt < kcap; ++kt) slice(kt, I0{}, YES{});
      capture(kcap);
      __builtin_amdgcn_sched_barrier(0);
      if (kcap + 1 < nk) {
        slice(kcap, I0{}, YES{});
        for (kt = kcap + 1; kt + 1 < nk; ++kt) slice(kt, I0{}, YES{});
      }
      slice(nk - 1, I0{}, NO{});
    } else {
      for (int kt = 0; kt + 1 < nk; ++kt) slice(kt, I0{}, YES{});
      slice(nk - 1, I0{}, NO{});
    }
  } else {
    int kt = 0;
    for (; kt + 2 < nk; kt += 2) {
      slice(kt, I0{}, YES{});
      slice(kt + 1, I1{}, YES{});
    }
    if (kt + 2 == nk) {
      slice(kt, I0{}, YES{});
      slice(kt + 1, I1{}, NO{});
    } else {
      slice(kt, I0{}, NO{});
    }
  }
  wait_vmcnt<0>();

  if constexpr (KS > 1) {
    // Tree reduction of the k-groups' partial sums through LDS: in each round the upper
    // half of the remaining k-groups writes its partials, the lower half adds them
    // ((g0 + g2) + (g1 + g3) for four groups: a fixed order).
    float* red = reinterpret_cast<float*>(lds);
    constexpr int REG = BM * BN;  // floats per k-group partial
#pragma unroll
    for (int half = KS / 2; half >= 1; half /= 2) {
      __syncthreads();
      if (kgrp >= half && kgrp < 2 * half) {
        float* r = red + (kgrp - half) * REG;
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) r[((i * FN + j) * 16 + e) * (64 * NWC) + wloc * 64 + lane] = acc[i][j][e];
      }
      __syncthreads();
      if (kgrp < half) {
        const float* r = red + kgrp * REG;
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] += r[((i * FN + j) * 16 + e) * (64 * NWC) + wloc * 64 + lane];
      }
    }
    if constexpr (STG) __syncthreads();  // every wave is done with the partials before the epilogue reuses the LDS
    if (kgrp != 0) return;
  } else if constexpr (STG) {
    __syncthreads();  // every wave is done with the last slice before the epilogue reuses the LDS
  }

  epilogue<KIND, BM, BN, WM, WN, SYM, EPI, FM, FN, TO, STG>(
      p, acc, mat, tm, tn, m0, n0, wm0, wn0, lane, ecap, cap,
      reinterpret_cast<unsigned short*>(lds) + wloc * TWN * (TWM + 8));
}

template <int KIND, int BM, int BN, int WM, int WN, int PF, bool SYM, int EPI, int TAG>
__global__ __launch_bounds__(64 * WM * WN) void gemm_kernel(const GemmParams p) {
  static_assert(PF == 1 || PF == 2, "prefetch distance");
  using TO = typename OutT<KIND>::T;
  constexpr int NT = 64 * WM * WN;                     // threads
  constexpr int ES = (KIND == KIND_F32) ? 4 : 2;      // operand element bytes
  constexpr int VEC = 16 / ES;                         // elements per 16-byte chunk
  constexpr int BK = kChunks * VEC;                    // k per LDS slice (128 bytes)
  constexpr int TWM = BM / WM, TWN = BN / WN;          // wave tile
  constexpr int FM = TWM / 32, FN = TWN / 32;          // 32x32 MFMA blocks per wave
  static_assert(FM >= 1 && FN >= 1, "wave tile");
  constexpr int A_CH = (BM * kChunks + NT - 1) / NT;   // staged A chunks per thread
  constexpr int B_CH = (BN * kChunks + NT - 1) / NT;   // staged B chunks per thread
  constexpr int KSTEPS = kChunks / 2;                  // MFMA k-steps per slice

  __shared__ u32x4 lds[2][(BM + BN) * kChunks];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  int mat, tm, tn;
  tile_coords<SYM>(p, mat, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;

  const char* Ab = static_cast<const char*>(p.A) + static_cast<int64_t>(mat) * p.sA * ES;
  const char* Bb = static_cast<const char*>(p.B) + static_cast<int64_t>(mat) * p.sB * ES;

  // Byte offsets (without k) of the chunks this thread stages. Rows past M or N are
  // clamped to the last valid row: they only feed output rows/columns that are never
  // stored, so the loads need no branches. K is a multiple of BK.
  int64_t a_off[A_CH], b_off[B_CH];
#pragma unroll
  for (int i = 0; i < A_CH; ++i) {
    const int c = min(tid + i * NT, BM * kChunks - 1);
    const int gr = min(m0 + c / kChunks, p.M - 1);
    a_off[i] = (static_cast<int64_t>(gr) * p.lda + (c % kChunks) * VEC) * ES;
  }
#pragma unroll
  for (int i = 0; i < B_CH; ++i) {
    const int c = min(tid + i * NT, BN * kChunks - 1);
    const int gr = min(n0 + c / kChunks, p.N - 1);
    b_off[i] = (static_cast<int64_t>(gr) * p.ldb + (c % kChunks) * VEC) * ES;
  }

  // PF staging register sets: slice k lands in set k % PF.
  u32x4 ra[PF][A_CH], rb[PF][B_CH];
  auto load_global = [&](int set, int k0) {
    const int64_t kb = static_cast<int64_t>(k0) * ES;
#pragma unroll
    for (int i = 0; i < A_CH; ++i) ra[set][i] = *reinterpret_cast<const u32x4*>(Ab + a_off[i] + kb);
#pragma unroll
    for (int i = 0; i < B_CH; ++i) rb[set][i] = *reinterpret_cast<const u32x4*>(Bb + b_off[i] + kb);
  };
  auto store_lds = [&](int set, int stage) {
    u32x4* la = lds[stage];
    u32x4* lb = lds[stage] + BM * kChunks;
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
      const int c = tid + i * NT;
      if ((BM * kChunks) % NT == 0 || c < BM * kChunks) la[swz(c / kChunks, c % kChunks)] = ra[set][i];
    }
#pragma unroll
    for (int i = 0; i < B_CH; ++i) {
      const int c = tid + i * NT;
      if ((BN * kChunks) % NT == 0 || c < BN * kChunks) lb[swz(c / kChunks, c % kChunks)] = rb[set][i];
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

  // One 128-byte slice of K, read from LDS buffer kt % 2, fragments double-buffered
  // across its k-steps. LOAD: issue the global loads of slice kt + PF into staging set
  // kt % PF. STORE: half-way through, write slice kt + 1 (staging set (kt + 1) % PF) to
  // the other LDS buffer. PH = kt % PF (a compile-time index into the staging sets).
  auto slice = [&](int kt, auto load_tag, auto store_tag, auto ph_tag) {
    constexpr bool LOAD = decltype(load_tag)::value;
    constexpr bool STORE = decltype(store_tag)::value;
    constexpr int PH = decltype(ph_tag)::value;
    const int stage = kt & 1;
    const u32x4* la = lds[stage];
    const u32x4* lb = lds[stage] + BM * kChunks;
    if constexpr (LOAD) load_global(PH, (kt + PF) * BK);
    load_frags(0, la, lb, 0);
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) {
      if (kk + 1 < KSTEPS) load_frags((kk + 1) & 1, la, lb, kk + 1);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) mma<KIND>(acc[i][j], fa[kk & 1][i], fb[kk & 1][j]);
      if constexpr (STORE) {
        if (kk == KSTEPS / 2 - 1) store_lds((PH + 1) % PF, stage ^ 1);
      }
    }
    __syncthreads();
  };
  using T_ = std::true_type;
  using F_ = std::false_type;
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, (PF > 1) ? 1 : 0>;

  if constexpr (PF == 1) {
    load_global(0, 0);
    store_lds(0, 0);
    __syncthreads();
    for (int kt = 0; kt + 1 < nk; ++kt) slice(kt, T_{}, T_{}, P0{});
    slice(nk - 1, F_{}, F_{}, P0{});
  } else {
    load_global(0, 0);
    load_global(1, min(1, nk - 1) * BK);
    store_lds(0, 0);
    __syncthreads();
    int kt = 0;
    for (; kt + 3 < nk; kt += 2) {
      slice(kt, T_{}, T_{}, P0{});
      slice(kt + 1, T_{}, T_{}, P1{});
    }
    const int left = nk - kt;  // 1, 2 or 3 slices, kt even
    if (left == 3) {
      slice(kt, T_{}, T_{}, P0{});
      slice(kt + 1, F_{}, T_{}, P1{});
      slice(kt + 2, F_{}, F_{}, P0{});
    } else if (left == 2) {
      slice(kt, F_{}, T_{}, P0{});
      slice(kt + 1, F_{}, F_{}, P1{});
    } else {
      slice(kt, F_{}, F_{}, P0{});
    }
  }

  epilogue<KIND, BM, BN, WM, WN, SYM, EPI, FM, FN, TO>(p, acc, mat, tm, tn, m0, n0, wm0, wn0, lane);
}

// TAG only gives otherwise identical instantiations their own symbol (profiles tell the
// Gram product of the iterate from the m' x m' products).
template <int KIND, int BM, int BN, int WM, int WN, int PF, bool SYM, int EPI, int TAG>
hipError_t launch_shape(const GemmParams& p, hipStream_t st) {
  hipLaunchKernelGGL((gemm_kernel<KIND, BM, BN, WM, WN, PF, SYM, EPI, TAG>), dim3(p.tiles, p.count),
                     dim3(64 * WM * WN), 0, st, p);
  return hipGetLastError();
}

template <int KIND, int BM, int BN, int WM, int WN, int NS, bool SYM, int EPI, int TAG, int KS = 1, int CH = 8>
hipError_t launch_dma(const GemmParams& p, hipStream_t st) {
  hipLaunchKernelGGL((gemm_dma_kernel<KIND, BM, BN, WM, WN, NS, KS, CH, SYM, EPI, TAG>), dim3(p.tiles, p.count),
                     dim3(64 * WM * WN * KS), 0, st, p);
  return hipGetLastError();
}

template <int KIND, bool SYM, int EPI, int TAG = 0>
hipError_t launch_tile(int cfg, const GemmParams& p, hipStream_t st) {
  switch (cfg) {
    // 64 and 128 tiles keep two slices of loads in flight (few workgroups per CU must
    // hide the load latency themselves); the 8-wave 256 tiles keep one.
    case TILE_64: return launch_shape<KIND, 64, 64, 2, 2, 2, SYM, EPI, TAG>(p, st);
    case TILE_128: return launch_shape<KIND, 128, 128, 2, 2, 2, SYM, EPI, TAG>(p, st);
    case TILE_256:  // 8 waves (2 per SIMD), wave tile 128 x 64
      if constexpr (KIND != KIND_F32) return launch_shape<KIND, 256, 256, 2, 4, 1, SYM, EPI, TAG>(p, st);
      return hipErrorInvalidValue;
    case TILE_256x128:  // 8 waves, wave tile 64 x 64
      if constexpr (!SYM && KIND != KIND_F32) return launch_shape<KIND, 256, 128, 4, 2, 1, SYM, EPI, TAG>(p, st);
      return hipErrorInvalidValue;
    case TILE_64_DMA: return launch_dma<KIND, 64, 64, 2, 2, 4, SYM, EPI, TAG>(p, st);
    case TILE_128_DMA: return launch_dma<KIND, 128, 128, 2, 2, 4, SYM, EPI, TAG>(p, st);
    case TILE_256x128_DMA:
      if constexpr (!SYM && KIND != KIND_F32) return launch_dma<KIND, 256, 128, 4, 2, 3, SYM, EPI, TAG>(p, st);
      return hipErrorInvalidValue;
    case TILE_256_DMA:
      if constexpr (KIND != KIND_F32) return launch_dma<KIND, 256, 256, 2, 4, 2, SYM, EPI, TAG>(p, st);
      return hipErrorInvalidValue;
    case TILE_256_DMA4:
      if constexpr (KIND != KIND_F32) return launch_dma<KIND, 256, 256, 2, 2, 2, SYM, EPI, TAG>(p, st);
      return hipErrorInvalidValue;
    case TILE_64_DMA_K2: return launch_dma<KIND, 64, 64, 2, 2, 4, SYM, EPI, TAG, 2>(p, st);
    case TILE_128_DMA_K2: return launch_dma<KIND, 128, 128, 2, 2, 4, SYM, EPI, TAG, 2>(p, st);
    case TILE_256_DMA_H:  // 64-byte slices: 4 stages, three slices in flight
      if constexpr (KIND != KIND_F32) return launch_dma<KIND, 256, 256, 2, 4, 4, SYM, EPI, TAG, 1, 4>(p, st);
      return hipErrorInvalidValue;
    case TILE_128_DMA_K2_H: return launch_dma<KIND, 128, 128, 2, 2, 8, SYM, EPI, TAG, 2, 4>(p, st);
    case TILE_256_DMA4_H:  // 4 waves of 128 x 128, 64-byte slices: 4 stages, three slices in flight
      if constexpr (KIND != KIND_F32) return launch_dma<KIND, 256, 256, 2, 2, 4, SYM, EPI, TAG, 1, 4>(p, st);
      return hipErrorInvalidValue;
    case TILE_256x192_DMA:  // 8 waves, wave tile 64 x 96: 2560 x 9728 is 510 tiles, two full rounds of 256 CUs
      if constexpr (!SYM && KIND != KIND_F32) return launch_dma<KIND, 256, 192, 4, 2, 2, SYM, EPI, TAG>(p, st);
      return hipErrorInvalidValue;
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_gemm(GemmOp op, bool ns_f32, int cfg, const GemmParams& p, hipStream_t st) {
  if (p.tiles <= 0 || p.count <= 0) return hipSuccess;
  if (ns_f32) {
    switch (op) {
      case OP_SYRK_IN:
      case OP_SYRK: return launch_tile<KIND_F32, true, EPI_STORE, 1>(cfg, p, st);
      case OP_SYM: return launch_tile<KIND_F32, true, EPI_STORE>(cfg, p, st);
      case OP_APPLY: return launch_tile<KIND_F32, false, EPI_APPLY>(cfg, p, st);
      case OP_UPDATE: return launch_tile<KIND_F32, false, EPI_UPDATE>(cfg, p, st);
    }
  } else {
    switch (op) {
      case OP_SYRK_IN: return launch_tile<KIND_BF16, true, EPI_STORE>(cfg, p, st);
      case OP_SYRK: return launch_tile<KIND_F16, true, EPI_STORE, 1>(cfg, p, st);
      case OP_SYM: return launch_tile<KIND_F16, true, EPI_STORE>(cfg, p, st);
      case OP_APPLY: return launch_tile<KIND_F16, false, EPI_APPLY>(cfg, p, st);
      case OP_UPDATE: return launch_tile<KIND_F16, false, EPI_UPDATE>(cfg, p, st);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace muon
