// Whole update of one small matrix per workgroup: momentum, Frobenius normalisation, every
// Newton-Schulz product of the schedule and the weight update in a single launch for a
// same-shape group (one workgroup per matrix).
//
// Small shapes (m' <= 128) leave the GPU idle between the ~20 launches the staged path
// needs per group; the pages batch such matrices and pick kernels per shape (DMuon
// summary, section 2.2: batching of similar shapes; section 2.4: per-shape kernel
// configurations). Here the whole schedule of one matrix runs inside one workgroup:
//   * the m' x m' matrices of the recurrence (R, Q and two temporaries; A and B for plain
//     NS) live in LDS for the whole kernel;
//   * the iterate X (m' x n') stays in the group's workspace (L2-resident), row-major and
//     transposed, and is streamed through an LDS staging buffer 64 columns (Gram product)
//     or 64 rows of X^T (apply) at a time, the next slice's global loads in flight while
//     the current one is multiplied.
// Arithmetic and scaling follow the staged bf16 path: the iterate kept in fp16 as xs * X
// (X0 rounded once from the fp32 momentum output), Gram-space matrices in fp16 scaled by e
// (polynomial coefficients b / e and c / e^2), fp32 MFMA accumulation (32x32x16 fp16).
// Products are dense.
#include "internal.hpp"

namespace muon {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16;

__device__ __forceinline__ float bf16_to_f32(u16 h) { return __uint_as_float(static_cast<unsigned int>(h) << 16); }
__device__ __forceinline__ u16 f32_to_bf16(float f) {
  unsigned int u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<u16>(u >> 16);
}
__device__ __forceinline__ u16 f32_to_f16(float f) { return __builtin_bit_cast(u16, static_cast<_Float16>(f)); }
__device__ __forceinline__ float f16_to_f32(u16 h) { return static_cast<float>(__builtin_bit_cast(_Float16, h)); }

__device__ __forceinline__ float load_elem(const void* base, int64_t i, int bf16) {
  return bf16 ? bf16_to_f32(static_cast<const u16*>(base)[i]) : static_cast<const float*>(base)[i];
}
__device__ __forceinline__ void store_elem(void* base, int64_t i, float v, int bf16) {
  if (bf16) static_cast<u16*>(base)[i] = f32_to_bf16(v);
  else static_cast<float*>(base)[i] = v;
}

// LDS matrices of fp16 rows holding CH 16-byte chunks (8 elements each); chunk j of row r
// sits at position j ^ (r mod CH), so the 32 rows one MFMA fragment read touches (same
// logical chunk) spread over all banks.
template <int CH>
__device__ __forceinline__ int chunk_at(int r, int j) { return r * CH + (j ^ (r & (CH - 1))); }
template <int CH>
__device__ __forceinline__ int elem_at(int r, int c) { return chunk_at<CH>(r, c >> 3) * 8 + (c & 7); }

// acc += A[rows a0.., k-step kk] * B[rows b0.., k-step kk]^T from two swizzled LDS matrices.
template <int CHA, int CHB>
__device__ __forceinline__ void mma_step(f32x16& acc, const u32x4* A, int a0, const u32x4* B, int b0, int kk,
                                         int lane) {
  const int j = 2 * kk + (lane >> 5);
  const u32x4 fa = A[chunk_at<CHA>(a0 + (lane & 31), j)];
  const u32x4 fb = B[chunk_at<CHB>(b0 + (lane & 31), j)];
  acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, fa), __builtin_bit_cast(f16x8, fb),
                                               acc, 0, 0, 0);
}

// The value of x, opaque to the optimiser: per-lane index math derived from it is
// recomputed inside each product instead of being hoisted out of the whole schedule
// (which would keep hundreds of LDS addresses live across the kernel).
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding: vmcnt in bits
// 3:0 and 15:14; expcnt 6:4 and lgkmcnt 11:8 left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// acc[t] += A[rows a0 + t * astride ..] * B[rows b0 ..]^T at k-step kk: NBLK output blocks in
// one block column share the B fragment.
template <int CHA, int CHB, int NBLK>
__device__ __forceinline__ void mma_col(f32x16 (&acc)[NBLK], const u32x4* A, int a0, int astride,
                                        const u32x4* B, int b0, int kk, int lane) {
  const int j = 2 * kk + (lane >> 5);
  const f16x8 fb = __builtin_bit_cast(f16x8, B[chunk_at<CHB>(b0 + (lane & 31), j)]);
#pragma unroll
  for (int t = 0; t < NBLK; ++t) {
    const f16x8 fa = __builtin_bit_cast(f16x8, A[chunk_at<CHA>(a0 + t * astride + (lane & 31), j)]);
    acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa, fb, acc[t], 0, 0, 0);
  }
}

__device__ __forceinline__ void zero(f32x16& a) {
#pragma unroll
  for (int e = 0; e < 16; ++e) a[e] = 0.0f;
}

template <int MP, int NT, int NPMAX>
__global__ __launch_bounds__(NT) void small_ns_kernel(const SmallParams p) {
  constexpr int NW = NT / 64;                 // waves
  constexpr int CS = MP / 8;                  // chunks per row of an m' x m' matrix
  constexpr int NB = (MP / 32) * (MP / 32);   // 32 x 32 blocks of an m' x m' product
  constexpr int BPW = NB / NW;                // ... per wave
  static_assert(BPW * NW == NB && BPW >= 1, "blocks per wave");
  constexpr int SQ = MP * CS;                 // u32x4 per m' x m' matrix
  // staging slice: 64 columns of X (MP rows x 8 chunks) or 64 rows of X^T (64 x CS chunks)
  constexpr int STG = MP * 8;
  static_assert(64 * CS == STG, "slice sizes");
  constexpr int LPW = MP / 8 / NW;            // direct-load instructions per wave per slice
  static_assert(LPW * NW * 8 == MP && LPW >= 1, "loads per wave");
  constexpr int APB = (MP / 32) * 2 / NW;     // apply blocks per wave per 64-column slice
  static_assert(APB * NW == (MP / 32) * 2 && APB >= 1, "apply blocks");
  // A wave's blocks of an m' x m' output form one block column (same B rows): block t sits
  // at block row bi0 + t * NW / (MP / 32), block column bj (likewise for the apply's two
  // block columns per slice).
  static_assert(NW % (MP / 32) == 0 && NW % 2 == 0, "block columns");
  constexpr int SQ_ASTRIDE = 32 * NW / (MP / 32);
  constexpr int AP_ASTRIDE = 32 * NW / 2;

  // LDS: the four m' x m' matrices and the staging slice; before the recurrence starts
  // the same space holds xs * X0 (MP x NPMAX fp16 values at most). Sizing it by the group's
  // n' lets several workgroups of a short-row group share a CU.
  static_assert(MP * NPMAX <= kSmallMaxElems, "single-workgroup size bound");
  constexpr int SMQ = (4 * SQ + STG) > MP * NPMAX / 8 ? (4 * SQ + STG) : MP * NPMAX / 8;
  static_assert(SMQ % STG == 0 && SQ % STG == 0, "stage slots");
  constexpr int NR0 = SMQ / STG - SQ / STG;   // staging slices besides one m' x m' matrix
  constexpr int NR = NR0 > 8 ? 8 : NR0;
  static_assert(NR >= 3 && (NR - 2) * LPW < 64, "ring");
  __shared__ u32x4 sm[SMQ];
  __shared__ double red[NT];
  u32x4* S[4] = {sm, sm + SQ, sm + 2 * SQ, sm + 3 * SQ};

  const int mat = blockIdx.x;
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const MatDesc d = p.table[mat];
  const int Np = p.Np;
  u16* X = static_cast<u16*>(p.X) + static_cast<int64_t>(mat) * p.sX;
  u16* XT[2] = {static_cast<u16*>(p.XT[0]) + static_cast<int64_t>(mat) * p.sXT,
                static_cast<u16*>(p.XT[1]) + static_cast<int64_t>(mat) * p.sXT};

  // 1. Momentum in the stored layout, 8 consecutive stored elements per thread (16-byte
  //    accesses when rows allow), in two passes over G and M as on the staged path: the
  //    first sums the squares of the fp32 U (fixed-order tree over the threads: the norm is
  //    deterministic), the second stores M' and writes X0 = xs * s * U, rounded once to
  //    fp16, to LDS in the canonical layout (the recurrence's LDS is free until step 3).
  u16* U = reinterpret_cast<u16*>(sm);   // MP x Np fp16, row-major: xs * X0
  static_assert(sizeof(sm) >= static_cast<size_t>(MP) * NPMAX * 2, "X0 fits in LDS");
  {
    const int total = MP * Np;
    for (int i = tid * 8; i < total; i += NT * 8) *reinterpret_cast<uint4*>(U + i) = make_uint4(0, 0, 0, 0);
  }
  const int rows = static_cast<int>(d.rows), cols = static_cast<int>(d.cols);
  const int gpr = (cols + 7) / 8;            // groups of 8 per stored row
  const bool vec = (cols % 8) == 0 && (reinterpret_cast<uintptr_t>(d.G) % 16) == 0 &&
                   (reinterpret_cast<uintptr_t>(d.M) % 16) == 0;
  // G and M of stored group gi (zero past the row end), the new momentum and U.
  auto load_gm = [&](int gi, float (&g)[8], float (&m)[8]) {
    const int sr = gi / gpr, sc0 = (gi % gpr) * 8;
    const int64_t base = static_cast<int64_t>(sr) * cols + sc0;
    if (vec) {
      if (p.g_bf16) {
        const uint4 w = *reinterpret_cast<const uint4*>(static_cast<const u16*>(d.G) + base);
        const unsigned int ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) { g[2 * q] = __uint_as_float(ws[q] << 16); g[2 * q + 1] = __uint_as_float(ws[q] & 0xFFFF0000u); }
      } else {
        const float4 x0 = *reinterpret_cast<const float4*>(static_cast<const float*>(d.G) + base);
        const float4 x1 = *reinterpret_cast<const float4*>(static_cast<const float*>(d.G) + base + 4);
        g[0] = x0.x; g[1] = x0.y; g[2] = x0.z; g[3] = x0.w; g[4] = x1.x; g[5] = x1.y; g[6] = x1.z; g[7] = x1.w;
      }
      if (p.m_bf16) {
        const uint4 w = *reinterpret_cast<const uint4*>(static_cast<const u16*>(d.M) + base);
        const unsigned int ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) { m[2 * q] = __uint_as_float(ws[q] << 16); m[2 * q + 1] = __uint_as_float(ws[q] & 0xFFFF0000u); }
      } else {
        const float4 x0 = *reinterpret_cast<const float4*>(static_cast<const float*>(d.M) + base);
        const float4 x1 = *reinterpret_cast<const float4*>(static_cast<const float*>(d.M) + base + 4);
        m[0] = x0.x; m[1] = x0.y; m[2] = x0.z; m[3] = x0.w; m[4] = x1.x; m[5] = x1.y; m[6] = x1.z; m[7] = x1.w;
      }
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const bool ok = sc0 + k < cols;
        g[k] = ok ? load_elem(d.G, base + k, p.g_bf16) : 0.0f;
        m[k] = ok ? load_elem(d.M, base + k, p.m_bf16) : 0.0f;
      }
    }
  };
  auto momentum8 = [&](const float (&g)[8], const float (&m)[8], float (&mn)[8], float (&u)[8]) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      mn[k] = p.mu * m[k] + g[k];
      u[k] = p.nesterov ? g[k] + p.mu * mn[k] : mn[k];
    }
  };
  // U of stored group gi: from G and M, or in a dry run (muon_prepare) the seeded stand-in
  // (G and M are then neither read nor written).
  auto momentum_u = [&](int gi, float (&mn)[8], float (&u)[8]) {
    if (p.dry) {
      const int sr = gi / gpr, sc0 = (gi % gpr) * 8;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int r = d.transposed ? sc0 + k : sr, c = d.transposed ? sr : sc0 + k;
        u[k] = sc0 + k < cols ? dry_u(mat, r, c) : 0.0f;
        mn[k] = 0.0f;
      }
      return;
    }
    float g[8], m[8];
    load_gm(gi, g, m);
    momentum8(g, m, mn, u);
  };
  // Each pass takes UB groups of 8 per thread and iteration, every load of the batch issued
  // before any arithmetic (indices past the end are clamped and their values dropped), so a
  // thread has UB * 2 loads in flight instead of one round trip per group.
  constexpr int UB = 4;
  const int ngr = rows * gpr;
  float sq = 0.0f;
  for (int g0 = tid; g0 < ngr; g0 += NT * UB) {
    float mn[UB][8], u[UB][8];
#pragma unroll
    for (int b = 0; b < UB; ++b) momentum_u(min(g0 + b * NT, ngr - 1), mn[b], u[b]);
#pragma unroll
    for (int b = 0; b < UB; ++b)
      if (g0 + b * NT < ngr) {
#pragma unroll
        for (int k = 0; k < 8; ++k) sq += u[b][k] * u[b][k];   // zero past the row end
      }
  }
  red[tid] = static_cast<double>(sq);
  __syncthreads();
  for (int w = NT / 2; w > 0; w >>= 1) {  // fixed-order tree: deterministic
    if (tid < w) red[tid] += red[tid + w];
    __syncthreads();
  }
  const float s = static_cast<float>(1.0 / (sqrt(red[0]) + static_cast<double>(p.eps)));
  const float xsc = p.xs * s;
  for (int g0 = tid; g0 < ngr; g0 += NT * UB) {
    float mn[UB][8], u[UB][8];
#pragma unroll
    for (int b = 0; b < UB; ++b) momentum_u(min(g0 + b * NT, ngr - 1), mn[b], u[b]);
#pragma unroll
    for (int b = 0; b < UB; ++b) {
      const int gi = g0 + b * NT;
      if (gi >= ngr) continue;
      const int sr = gi / gpr, sc0 = (gi % gpr) * 8;
      const int64_t base = static_cast<int64_t>(sr) * cols + sc0;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        if (sc0 + k >= cols) continue;
        if (!p.dry) store_elem(d.M, base + k, mn[b][k], p.m_bf16);
        const int r = d.transposed ? sc0 + k : sr, c = d.transposed ? sr : sc0 + k;
        U[r * Np + c] = f32_to_f16(xsc * u[b][k]);
      }
    }
  }
  __syncthreads();

  // 2. The iterate (already xs * X0 in fp16) to the workspace, row-major and transposed,
  //    8 elements (16 bytes) per store.
  {
    for (int i = tid * 8; i < MP * Np; i += NT * 8) {
      const int r = i / Np, c0 = i % Np;
      *reinterpret_cast<uint4*>(X + static_cast<int64_t>(r) * Np + c0) = *reinterpret_cast<const uint4*>(U + i);
    }
    for (int i = tid * 8; i < MP * Np; i += NT * 8) {   // X^T: row c holds column c of X
      const int c = i / MP, r0 = i % MP;
      unsigned int w[4];
#pragma unroll
      for (int q = 0; q < 4; ++q)
        w[q] = U[(r0 + 2 * q) * Np + c] | (static_cast<unsigned int>(U[(r0 + 2 * q + 1) * Np + c]) << 16);
      *reinterpret_cast<uint4*>(XT[0] + static_cast<int64_t>(c) * MP + r0) = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
  __syncthreads();

  const float e = p.e;
  const float b1 = p.b / e, c1 = p.c / (e * e);
  const float gram_alpha = e / (p.xs * p.xs);
  const float decay = 1.0f - p.lr * p.wd;
  const float inv_xs = 1.0f / p.xs;

  // X and X^T are streamed through a ring of NR staging slices in the LDS the live m' x m'
  // operand does not occupy, filled by the CDNA4 direct global -> LDS loads (16 bytes per
  // lane; lane l of an instruction writes bytes [16 l, 16 l + 16) of a 1 KB window). NR - 1
  // slices are in flight. A slice is 64 columns of X (MP rows of 8 chunks) or 64 rows of
  // X^T (64 rows of CS chunks); the XOR swizzle is applied on the global side (lane l
  // fetches the logical chunk that belongs at its position).
  typedef __attribute__((address_space(3))) void* lds_ptr;
  typedef const __attribute__((address_space(1))) void* glb_ptr;
  // stage k of the ring, skipping the SQ/STG slots of the m' x m' matrix at `keep`
  auto stage = [&](int k, const u32x4* keep) -> u32x4* {
    const int ks = static_cast<int>(keep - sm) / STG;
    return sm + STG * (k < ks ? k : k + SQ / STG);
  };
  auto issue_x = [&](u32x4* dst, const u16* src, int sl) {   // 64 columns of X
    const int lane = opaque(tid & 63);
#pragma unroll
    for (int t = 0; t < LPW; ++t) {
      const int ins = wave + t * NW;                 // 8 rows per instruction
      const int row = ins * 8 + (lane >> 3);
      const int ch = (lane & 7) ^ (row & 7);
      __builtin_amdgcn_global_load_lds((glb_ptr)(src + static_cast<int64_t>(row) * Np + sl * 64 + ch * 8),
                                       (lds_ptr)(dst + ins * 64), 16, 0, 0);
    }
  };
  auto issue_xt = [&](u32x4* dst, const u16* src, int sl) {  // 64 rows of X^T
    const int lane = opaque(tid & 63);
#pragma unroll
    for (int t = 0; t < LPW; ++t) {
      const int ins = wave + t * NW;                 // 64 / CS rows per instruction
      const int row = ins * (64 / CS) + lane / CS;
      const int ch = (lane % CS) ^ (row & (CS - 1));
      __builtin_amdgcn_global_load_lds((glb_ptr)(src + static_cast<int64_t>(sl * 64 + row) * MP + ch * 8),
                                       (lds_ptr)(dst + ins * 64), 16, 0, 0);
    }
  };
  // m' x m' output element writes / reads in LDS.
  auto sq_put = [&](u32x4* M, int r, int c, float v) { reinterpret_cast<u16*>(M)[elem_at<CS>(r, c)] = f32_to_f16(v); };
  auto sq_get = [&](const u32x4* M, int r, int c) { return f16_to_f32(reinterpret_cast<const u16*>(M)[elem_at<CS>(r, c)]); };

  // Gram product: C = alpha X X^T into LDS matrix C (X streamed in 64-column slices).
  auto gram = [&](u32x4* C, float alpha) {
    const int lane = opaque(tid & 63);
    f32x16 acc[BPW];
#pragma unroll
    for (int t = 0; t < BPW; ++t) zero(acc[t]);
    const int ns = Np / 64;
#pragma unroll
    for (int k = 0; k < NR - 1; ++k) issue_x(stage(k, C), X, min(k, ns - 1));
    for (int sl = 0; sl < ns; ++sl) {
      wait_vmcnt<(NR - 2) * LPW>();   // this wave's part of slice sl has landed
      __builtin_amdgcn_s_barrier();   // ... and every wave's; slice sl - 1's stage is free
      issue_x(stage((sl + NR - 1) % NR, C), X, min(sl + NR - 1, ns - 1));
      const u32x4* st = stage(sl % NR, C);
#pragma unroll 2
      for (int kk = 0; kk < 4; ++kk)
        mma_col<8, 8, BPW>(acc, st, (wave / (MP / 32)) * 32, SQ_ASTRIDE, st, (wave % (MP / 32)) * 32, kk, lane);
    }
    wait_vmcnt<0>();
#pragma unroll
    for (int t = 0; t < BPW; ++t) {
      const int bi = wave / (MP / 32) + t * (NW / (MP / 32)), bj = wave % (MP / 32);
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int k = 0; k < 4; ++k)
          sq_put(C, bi * 32 + q * 8 + (lane >> 5) * 4 + k, bj * 32 + (lane & 31), alpha * acc[t][4 * q + k]);
    }
    __syncthreads();
  };
  // m' x m' product in LDS: C = alpha A B^T + beta E + gamma I (C distinct from A, B, E).
  auto square = [&](u32x4* C, const u32x4* A, const u32x4* B, const u32x4* E, float alpha, float beta,
                    float gamma) {
    const int lane = opaque(tid & 63);
    f32x16 acc[BPW];
#pragma unroll
    for (int t = 0; t < BPW; ++t) zero(acc[t]);
#pragma unroll 2
    for (int kk = 0; kk < MP / 16; ++kk)
      mma_col<CS, CS, BPW>(acc, A, (wave / (MP / 32)) * 32, SQ_ASTRIDE, B, (wave % (MP / 32)) * 32, kk, lane);
#pragma unroll
    for (int t = 0; t < BPW; ++t) {
      const int bi = wave / (MP / 32) + t * (NW / (MP / 32)), bj = wave % (MP / 32);
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int r = bi * 32 + q * 8 + (lane >> 5) * 4 + k, c = bj * 32 + (lane & 31);
          float v = alpha * acc[t][4 * q + k] + (r == c ? gamma : 0.0f);
          if (E) v += beta * sq_get(E, r, c);
          sq_put(C, r, c, v);
        }
    }
    __syncthreads();
  };
  // Long product v = Q X (Q in LDS, X^T streamed in 64-row slices); per 32 x 32 block
  // epi(rb, c, acc) with acc[4q + k] the value at row rb + 8q + k of column c.
  auto apply = [&](const u32x4* Q, const u16* xt, auto&& epi) {
    const int ns = Np / 64;
    const int lane = opaque(tid & 63);
#pragma unroll
    for (int k = 0; k < NR - 1; ++k) issue_xt(stage(k, Q), xt, min(k, ns - 1));
    for (int sl = 0; sl < ns; ++sl) {
      wait_vmcnt<(NR - 2) * LPW>();
      __builtin_amdgcn_s_barrier();
      issue_xt(stage((sl + NR - 1) % NR, Q), xt, min(sl + NR - 1, ns - 1));
      const u32x4* st = stage(sl % NR, Q);
      f32x16 acc[APB];
#pragma unroll
      for (int t = 0; t < APB; ++t) zero(acc[t]);
#pragma unroll 2
      for (int kk = 0; kk < MP / 16; ++kk)
        mma_col<CS, CS, APB>(acc, Q, (wave / 2) * 32, AP_ASTRIDE, st, (wave % 2) * 32, kk, lane);
#pragma unroll 1
      for (int t = 0; t < APB; ++t)
        epi((wave / 2) * 32 + t * AP_ASTRIDE + (lane >> 5) * 4, sl * 64 + (wave % 2) * 32 + (lane & 31), acc[t]);
    }
    wait_vmcnt<0>();
    __syncthreads();
  };
  // W <- W * decay - lr * O with O = v / xs, through the orientation; all 16 W values of
  // the block are loaded before any is stored.
  auto update = [&](int rb, int c, const f32x16& v) {
    float w[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int r = rb + (e >> 2) * 8 + (e & 3);
      const bool ok = r < p.m && c < p.n;
      const int64_t wi = !ok ? 0 : d.transposed ? static_cast<int64_t>(c) * d.cols + r : static_cast<int64_t>(r) * d.cols + c;
      w[e] = !ok ? 0.0f : p.w_bf16 ? bf16_to_f32(static_cast<const u16*>(d.W)[wi]) : static_cast<const float*>(d.W)[wi];
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int r = rb + (e >> 2) * 8 + (e & 3);
      if (r >= p.m || c >= p.n) continue;
      const int64_t wi = d.transposed ? static_cast<int64_t>(c) * d.cols + r : static_cast<int64_t>(r) * d.cols + c;
      const float nw = w[e] * decay - p.lr * (v[e] * inv_xs);
      if (p.w_bf16) static_cast<u16*>(d.W)[wi] = f32_to_bf16(nw);
      else static_cast<float*>(d.W)[wi] = nw;
    }
  };
  // New iterate: X row-major and X^T (both from the same fp32 value).
  auto store_x = [&](u16* xtn, int rb, int c, const f32x16& v) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      u16 h[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        h[k] = f32_to_f16(v[4 * q + k]);
        X[static_cast<int64_t>(rb + 8 * q + k) * Np + c] = h[k];
      }
      *reinterpret_cast<uint2*>(xtn + static_cast<int64_t>(c) * MP + rb + 8 * q) =
          make_uint2(h[0] | (static_cast<unsigned int>(h[1]) << 16), h[2] | (static_cast<unsigned int>(h[3]) << 16));
    }
  };

  int cur = 0;
  if (p.plain) {
    for (int round = 0; round < p.rounds; ++round) {
      const bool last = round + 1 == p.rounds;
      gram(S[0], gram_alpha);                         // A_e = e X X^T
      square(S[1], S[0], S[0], S[0], c1, b1, 0.0f);   // B = b A + c A^2
      u16* xtn = XT[cur ^ 1];
      // X' = a X + B X; a X reads the same fp16 X the products consume. Each element of X is
      // read and then written by the same lane, and the apply reads only X^T.
      apply(S[1], XT[cur], [&](int rb, int c, const f32x16& v) {
        f32x16 o;
#pragma unroll
        for (int e = 0; e < 16; ++e) o[e] = f16_to_f32(X[static_cast<int64_t>(rb + (e >> 2) * 8 + (e & 3)) * Np + c]);
#pragma unroll
        for (int e = 0; e < 16; ++e) o[e] = v[e] + p.a * o[e];
        if (last && !p.dry) update(rb, c, o);
        else store_x(xtn, rb, c, o);
      });
      cur ^= 1;
    }
    return;
  }

  for (int sg = 0; sg < p.n_segments; ++sg) {
    const bool last = sg + 1 == p.n_segments;
    u32x4* R = S[0];
    u32x4* Q = S[1];
    u32x4* T1 = S[2];
    u32x4* T2 = S[3];
    gram(R, gram_alpha);                     // R_e = e X X^T
    square(Q, R, R, R, c1, b1, p.a);         // Q = P(R)
    for (int k = 1; k < p.segments[sg]; ++k) {
      square(T1, Q, R, nullptr, 1.0f, 0.0f, 0.0f);    // T1 = Q R_e
      square(T2, T1, Q, nullptr, 1.0f, 0.0f, 0.0f);   // A_e = Q R_e Q^T
      square(T1, T2, T2, T2, c1, b1, p.a);            // P = P(A)
      square(T2, T1, Q, nullptr, 1.0f, 0.0f, 0.0f);   // Q' = P Q
      u32x4* t = Q; Q = T2; T2 = t;
    }
    u16* xtn = XT[cur ^ 1];
    apply(Q, XT[cur], [&](int rb, int c, const f32x16& v) {
      if (last && !p.dry) update(rb, c, v);
      else store_x(xtn, rb, c, v);
    });
    cur ^= 1;
  }
}

}  // namespace

hipError_t launch_small_ns(const SmallParams& p, hipStream_t st) {
  if (p.count <= 0) return hipSuccess;
  // m' = 64: LDS sized for n' <= 256 (three workgroups per CU) or for the largest n';
  // m' = 128: eight waves (two per SIMD), one workgroup per CU.
  if (p.Mp == 64 && p.Np <= 256) {
    hipLaunchKernelGGL((small_ns_kernel<64, 256, 256>), dim3(p.count), dim3(256), 0, st, p);
  } else if (p.Mp == 64) {
    hipLaunchKernelGGL((small_ns_kernel<64, 256, kSmallMaxElems / 64>), dim3(p.count), dim3(256), 0, st, p);
  } else if (p.Mp == 128) {
    hipLaunchKernelGGL((small_ns_kernel<128, 512, kSmallMaxElems / 128>), dim3(p.count), dim3(512), 0, st, p);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace muon
