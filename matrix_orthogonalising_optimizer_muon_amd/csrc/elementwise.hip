// HBM-bound stages of the update: momentum + Nesterov look-ahead, the write of U in the
// canonical (short side first) orientation, and the Frobenius norm.
//
// MuonX article, section 2: Muon first smooths the gradient with momentum, then
// orthogonalises; the momentum form (heavy-ball sum, Nesterov look-ahead
// U = G + mu*M') and the normalisation X0 = U / (||U||_F + eps) are the plain readings of
// the pages. The norm is reduced deterministically: per-workgroup partial sums of squares
// (wavefront shuffles, then LDS), then one fixed-order fp64 pass per matrix.
#include "internal.hpp"

namespace muon {
namespace {

constexpr int kTile = 64;      // canonical 64 x 64 tile per workgroup
constexpr int kThreads = 256;  // 8 threads per 64-element row, 32 rows per pass

__device__ __forceinline__ float bf16_to_f32(unsigned short h) {
  return __uint_as_float(static_cast<unsigned int>(h) << 16);
}
__device__ __forceinline__ unsigned short f32_to_bf16(float f) {
  unsigned int u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<unsigned short>(u >> 16);
}

__device__ __forceinline__ float load_elem(const void* base, int64_t i, int bf16) {
  return bf16 ? bf16_to_f32(static_cast<const unsigned short*>(base)[i])
              : static_cast<const float*>(base)[i];
}
__device__ __forceinline__ void store_elem(void* base, int64_t i, float v, int bf16) {
  if (bf16) static_cast<unsigned short*>(base)[i] = f32_to_bf16(v);
  else static_cast<float*>(base)[i] = v;
}
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// 16-byte global access; NT marks it non-temporal (streamed data that is not read again
// in this step).
template <bool NT>
__device__ __forceinline__ u32x4 ld16(const void* p) {
  if constexpr (NT) return __builtin_nontemporal_load(static_cast<const u32x4*>(p));
  else return *static_cast<const u32x4*>(p);
}
template <bool NT>
__device__ __forceinline__ void st16(void* p, u32x4 v) {
  if constexpr (NT) __builtin_nontemporal_store(v, static_cast<u32x4*>(p));
  else *static_cast<u32x4*>(p) = v;
}

template <bool NT = false>
__device__ __forceinline__ void load8(const void* base, int64_t i, int bf16, float (&v)[8]) {
  if (bf16) {
    const u32x4 w = ld16<NT>(static_cast<const unsigned short*>(base) + i);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v[2 * q] = __uint_as_float(w[q] << 16);
      v[2 * q + 1] = __uint_as_float(w[q] & 0xFFFF0000u);
    }
  } else {
    const float* f = static_cast<const float*>(base) + i;
    const u32x4 a = ld16<NT>(f), b = ld16<NT>(f + 4);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v[q] = __uint_as_float(a[q]);
      v[4 + q] = __uint_as_float(b[q]);
    }
  }
}
template <bool NT = false>
__device__ __forceinline__ void store8(void* base, int64_t i, int bf16, const float (&v)[8]) {
  if (bf16) {
    u32x4 w;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      w[q] = static_cast<unsigned int>(f32_to_bf16(v[2 * q])) |
             (static_cast<unsigned int>(f32_to_bf16(v[2 * q + 1])) << 16);
    st16<NT>(static_cast<unsigned short*>(base) + i, w);
  } else {
    float* f = static_cast<float*>(base) + i;
    st16<NT>(f, u32x4{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3])});
    st16<NT>(f + 4, u32x4{__float_as_uint(v[4]), __float_as_uint(v[5]), __float_as_uint(v[6]), __float_as_uint(v[7])});
  }
}
// Value as it will be stored (rounded to bf16 if the store is bf16).
__device__ __forceinline__ float round_as(float v, int bf16) {
  return bf16 ? bf16_to_f32(f32_to_bf16(v)) : v;
}

// Block partial of sum(u^2): wavefront butterfly, then the 4 wave sums in order.
__device__ __forceinline__ void write_partial(float sq, float* wsum, float* dst) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) sq += __shfl_xor(sq, off, 64);
  if ((tid & 63) == 0) wsum[tid >> 6] = sq;
  __syncthreads();
  if (tid == 0) *dst = (wsum[0] + wsum[1]) + (wsum[2] + wsum[3]);
}

// Stores 8 values of U (bf16 or fp32) at element offset off of U.
__device__ __forceinline__ void store_u8(void* U, int64_t off, int bf16, const float (&v)[8]) {
  if (bf16) {
    unsigned int w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
      w[q] = static_cast<unsigned int>(f32_to_bf16(v[2 * q])) |
             (static_cast<unsigned int>(f32_to_bf16(v[2 * q + 1])) << 16);
    *reinterpret_cast<uint4*>(static_cast<unsigned short*>(U) + off) = make_uint4(w[0], w[1], w[2], w[3]);
  } else {
    float4* dst = reinterpret_cast<float4*>(static_cast<float*>(U) + off);
    dst[0] = make_float4(v[0], v[1], v[2], v[3]);
    dst[1] = make_float4(v[4], v[5], v[6], v[7]);
  }
}

// Momentum, Nesterov look-ahead and the U store for one 8-element chunk at (r, c) of the
// canonical U of a matrix stored in canonical orientation; g and m hold the chunk's G and
// M when full (16-byte path), otherwise the chunk is read element by element (zero in the
// padding). Returns the sum of squares of the stored U values.
__device__ __forceinline__ float momentum_chunk(const MomentumParams& p, const MatDesc& d, int mat, int64_t r,
                                                int64_t c, bool full, const float (&g)[8], const float (&m)[8]) {
  float u[8];
  if (full) {
    float mn[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      mn[e] = p.mu * m[e] + g[e];
      u[e] = p.nesterov ? g[e] + p.mu * mn[e] : mn[e];
    }
    store8<true>(d.M, r * d.cols + c, p.m_bf16, mn);
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int64_t sc = c + e;
      u[e] = 0.0f;
      if (r < d.rows && sc < d.cols) {
        const int64_t idx = r * d.cols + sc;
        const float gv = load_elem(d.G, idx, p.g_bf16);
        const float mv = load_elem(d.M, idx, p.m_bf16);
        const float mn = p.mu * mv + gv;
        store_elem(d.M, idx, mn, p.m_bf16);
        u[e] = p.nesterov ? gv + p.mu * mn : mn;
      }
    }
  }
  float sq = 0.0f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    u[e] = round_as(u[e], p.u_bf16);
    sq += u[e] * u[e];
  }
  store_u8(p.U, static_cast<int64_t>(mat) * p.sU + r * p.ldu + c, p.u_bf16, u);
  return sq;
}

// Batches with a matrix stored transposed (rows > cols): one workgroup per canonical
// 64 x 64 tile of the padded U (so one partial per 4096 elements, as in the flat kernel
// below). A transposed matrix's tile is walked in the stored layout (coalesced along
// stored columns) and written transposed through LDS; a matrix of the same batch stored
// in canonical orientation takes the 4096 elements of U in row-major order instead (512
// consecutive 8-element chunks; Np is a multiple of 64, so no chunk crosses a row), with
// both of a thread's chunks loaded before any store. G and M are streamed (non-temporal):
// nothing reads them again in the step.
__global__ __launch_bounds__(kThreads) void momentum_kernel(const MomentumParams p) {
  __shared__ float tile[kTile][kTile + 1];
  __shared__ float wsum[kThreads / 64];

  const int mat = blockIdx.y;
  const MatDesc d = p.inl.n > 0 ? p.inl.d[mat] : p.table[mat];
  if (p.inl.n > 0 && blockIdx.x == 0 && threadIdx.x == 0) p.table_out[mat] = d;
  const int tid = threadIdx.x;
  // 16-byte accesses when every row start is 16-byte aligned (row length a multiple of
  // 8 elements and aligned base pointers); otherwise element by element.
  const bool vec_ok = (d.cols % 8) == 0 && (reinterpret_cast<uintptr_t>(d.G) % 16) == 0 &&
                      (reinterpret_cast<uintptr_t>(d.M) % 16) == 0;
  float* part = p.partials + static_cast<int64_t>(mat) * (p.tiles_m * p.tiles_n);

  if (!d.transposed) {
    const int t = blockIdx.x;
    const int cpr = p.Np / 8;  // chunks per row of U
    float g[2][8], m[2][8];
    int64_t r[2], c[2];
    bool full[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int64_t q = static_cast<int64_t>(t) * 512 + k * 256 + tid;
      r[k] = q / cpr;
      c[k] = (q % cpr) * 8;
      full[k] = vec_ok && r[k] < d.rows && c[k] + 8 <= d.cols;
      if (full[k]) {
        const int64_t idx = r[k] * d.cols + c[k];
        load8<true>(d.G, idx, p.g_bf16, g[k]);
        load8<true>(d.M, idx, p.m_bf16, m[k]);
      }
    }
    float sq = 0.0f;
#pragma unroll
    for (int k = 0; k < 2; ++k) sq += momentum_chunk(p, d, mat, r[k], c[k], full[k], g[k], m[k]);
    write_partial(sq, wsum, part + t);
    return;
  }

  const int t = blockIdx.x;
  const int ti = t / p.tiles_n, tj = t % p.tiles_n;
  const int i0 = ti * kTile, j0 = tj * kTile;   // canonical tile origin
  const int cr = tid >> 3;          // local row within a pass
  const int cc = (tid & 7) * 8;     // local first column (8 consecutive)

  // Phase 1: walk the tile in the STORED layout: stored rows are canonical columns. Both
  // passes' loads are issued before any store.
  const int64_t srow0 = j0, scol0 = i0;
  float g[2][8], m[2][8];
  bool full[2];
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int64_t sr = srow0 + cr + pass * 32;
    const int64_t sc0 = scol0 + cc;
    full[pass] = vec_ok && sr < d.rows && sc0 + 8 <= d.cols;
    if (full[pass]) {
      load8<true>(d.G, sr * d.cols + sc0, p.g_bf16, g[pass]);
      load8<true>(d.M, sr * d.cols + sc0, p.m_bf16, m[pass]);
    }
  }
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int lr = cr + pass * 32;
    const int64_t sr = srow0 + lr;
    const int64_t sc0 = scol0 + cc;
    if (full[pass]) {
      float mn[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        mn[e] = p.mu * m[pass][e] + g[pass][e];
        tile[lr][cc + e] = p.nesterov ? g[pass][e] + p.mu * mn[e] : mn[e];
      }
      store8<true>(d.M, sr * d.cols + sc0, p.m_bf16, mn);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int64_t sc = sc0 + e;
        float u = 0.0f;
        if (sr < d.rows && sc < d.cols) {
          const int64_t idx = sr * d.cols + sc;
          const float gv = load_elem(d.G, idx, p.g_bf16);
          const float mv = load_elem(d.M, idx, p.m_bf16);
          const float mn = p.mu * mv + gv;
          store_elem(d.M, idx, mn, p.m_bf16);
          u = p.nesterov ? gv + p.mu * mn : mn;
        }
        tile[lr][cc + e] = u;
      }
    }
  }
  __syncthreads();

  // Phase 2: write U in the canonical layout (coalesced along canonical columns),
  // including the zero padding up to Mp x Np; sum the squares of the stored values.
  float sq = 0.0f;
#pragma unroll
  for (int pass = 0; pass < kTile / 32; ++pass) {
    const int lr = cr + pass * 32;
    const int64_t gi = i0 + lr;
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      v[e] = round_as(tile[cc + e][lr], p.u_bf16);
      sq += v[e] * v[e];
    }
    store_u8(p.U, static_cast<int64_t>(mat) * p.sU + gi * p.ldu + j0 + cc, p.u_bf16, v);
  }
  write_partial(sq, wsum, part + t);
}

// Batches with every matrix stored in canonical orientation (rows <= cols): no LDS tile,
// 512 threads, one 8-element chunk each, so a workgroup covers 4096 consecutive elements
// of the padded U in row-major order and writes one partial. More workgroups per CU keep
// more loads in flight than the tiled kernel (measured on one MI355X: 2560 x 9728 bf16,
// 5.2 TB/s against 4.9 TB/s).
constexpr int kFlatThreads = 512;
__global__ __launch_bounds__(kFlatThreads) void momentum_flat_kernel(const MomentumParams p) {
  __shared__ float wsum[kFlatThreads / 64];
  const int mat = blockIdx.y;
  const int t = blockIdx.x;
  const MatDesc d = p.inl.n > 0 ? p.inl.d[mat] : p.table[mat];
  if (p.inl.n > 0 && blockIdx.x == 0 && threadIdx.x == 0) p.table_out[mat] = d;
  const int tid = threadIdx.x;
  const bool vec_ok = (d.cols % 8) == 0 && (reinterpret_cast<uintptr_t>(d.G) % 16) == 0 &&
                      (reinterpret_cast<uintptr_t>(d.M) % 16) == 0;
  const int cpr = p.Np / 8;
  const int64_t q = static_cast<int64_t>(t) * 512 + tid;
  const int64_t r = q / cpr, c = (q % cpr) * 8;
  const bool full = vec_ok && r < d.rows && c + 8 <= d.cols;
  float g[8], m[8];
  if (full) {
    load8<true>(d.G, r * d.cols + c, p.g_bf16, g);
    load8<true>(d.M, r * d.cols + c, p.m_bf16, m);
  }
  float sq = momentum_chunk(p, d, mat, r, c, full, g, m);
  // Wavefront butterfly, then the 8 wave sums in a fixed order.
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) sq += __shfl_xor(sq, off, 64);
  if ((tid & 63) == 0) wsum[tid >> 6] = sq;
  __syncthreads();
  if (tid == 0) {
    const float tot = ((wsum[0] + wsum[1]) + (wsum[2] + wsum[3])) + ((wsum[4] + wsum[5]) + (wsum[6] + wsum[7]));
    p.partials[static_cast<int64_t>(mat) * (p.tiles_m * p.tiles_n) + t] = tot;
  }
}

constexpr int kFinThreads = 1024;

__global__ __launch_bounds__(kFinThreads) void norm_finalize_kernel(const float* partials, int per_matrix,
                                                                    float eps, float* s) {
  __shared__ double wred[kFinThreads / 64];
  const int mat = blockIdx.x;
  const int tid = threadIdx.x;
  const float* src = partials + static_cast<int64_t>(mat) * per_matrix;
  // Thread tid adds partials tid, tid + 1024, ... in that order, their loads issued eight
  // at a time (the partials come from every XCD's workgroups, so each load goes past this
  // XCD's L2; 8192 partials, a 32768 x 16384 matrix, take one batch); the zero padding
  // past the end leaves the sum unchanged. Then a wavefront butterfly and the 16 wave
  // sums in order: a fixed summation order.
  double acc = 0.0;
  for (int base = tid; base < per_matrix; base += kFinThreads * 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = base + u * kFinThreads;
      v[u] = i < per_matrix ? src[i] : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) acc += static_cast<double>(v[u]);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if ((tid & 63) == 0) wred[tid >> 6] = acc;
  __syncthreads();
  if (tid == 0) {
    double total = 0.0;
#pragma unroll
    for (int w = 0; w < kFinThreads / 64; ++w) total += wred[w];
    s[mat] = static_cast<float>(1.0 / (sqrt(total) + static_cast<double>(eps)));
  }
}

// 64 x 64 tile transpose through LDS: coalesced reads of U rows, coalesced writes of
// X^T rows; the value is scaled by scale * s[mat] and converted (bf16 -> fp16 path).
constexpr int kTransThreads = 512;  // 8 threads per 64-element row: the whole tile in one pass
__global__ __launch_bounds__(kTransThreads) void transpose_scale_kernel(const TransposeParams p) {
  constexpr int kRowsPerPass = kTransThreads / 8;
  __shared__ float tile[kTile][kTile + 1];
  const int mat = blockIdx.y;
  const int tiles_n = p.Np / kTile;
  const int ti = blockIdx.x / tiles_n, tj = blockIdx.x % tiles_n;
  const int i0 = ti * kTile, j0 = tj * kTile;
  const int tid = threadIdx.x;
  const int cr = tid >> 3, cc = (tid & 7) * 8;
  const float sc = p.scale * p.s[mat];
  const int64_t ubase = static_cast<int64_t>(mat) * p.sU;
#pragma unroll
  for (int pass = 0; pass < kTile / kRowsPerPass; ++pass) {
    const int lr = cr + pass * kRowsPerPass;
    float v[8];
    load8(p.U, ubase + static_cast<int64_t>(i0 + lr) * p.Np + j0 + cc, p.u_bf16, v);
#pragma unroll
    for (int e = 0; e < 8; ++e) tile[lr][cc + e] = v[e] * sc;
  }
  __syncthreads();
  const int64_t xbase = static_cast<int64_t>(mat) * p.sXT;
#pragma unroll
  for (int pass = 0; pass < kTile / kRowsPerPass; ++pass) {
    const int lr = cr + pass * kRowsPerPass;   // row of X^T = column of U
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = tile[cc + e][lr];
    const int64_t off = xbase + static_cast<int64_t>(j0 + lr) * p.Mp + i0 + cc;
    if (p.u_bf16) {
      unsigned int w[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const _Float16 lo = static_cast<_Float16>(v[2 * q]), hi = static_cast<_Float16>(v[2 * q + 1]);
        w[q] = static_cast<unsigned int>(__builtin_bit_cast(unsigned short, lo)) |
               (static_cast<unsigned int>(__builtin_bit_cast(unsigned short, hi)) << 16);
      }
      *reinterpret_cast<uint4*>(static_cast<unsigned short*>(p.XT) + off) = make_uint4(w[0], w[1], w[2], w[3]);
    } else {
      float4* dst = reinterpret_cast<float4*>(static_cast<float*>(p.XT) + off);
      dst[0] = make_float4(v[0], v[1], v[2], v[3]);
      dst[1] = make_float4(v[4], v[5], v[6], v[7]);
    }
  }
}

__global__ void write_table_kernel(const TableChunk c, MatDesc* dst) {
  const int i = threadIdx.x;
  if (i < c.n) dst[i] = c.d[i];
}

}  // namespace

hipError_t launch_momentum(const MomentumParams& p, hipStream_t st) {
  if (p.count <= 0) return hipSuccess;
  dim3 grid(p.tiles_m * p.tiles_n, p.count);
  if (p.has_tall) hipLaunchKernelGGL(momentum_kernel, grid, dim3(kThreads), 0, st, p);
  else hipLaunchKernelGGL(momentum_flat_kernel, grid, dim3(kFlatThreads), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_norm_finalize(const float* partials, int per_matrix, int count, float eps,
                                float* s, hipStream_t st) {
  if (count <= 0) return hipSuccess;
  hipLaunchKernelGGL(norm_finalize_kernel, dim3(count), dim3(kFinThreads), 0, st, partials, per_matrix, eps, s);
  return hipGetLastError();
}

hipError_t launch_transpose_scale(const TransposeParams& p, hipStream_t st) {
  if (p.count <= 0) return hipSuccess;
  dim3 grid((p.Mp / kTile) * (p.Np / kTile), p.count);
  hipLaunchKernelGGL(transpose_scale_kernel, grid, dim3(kTransThreads), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_write_table(const TableChunk& c, MatDesc* dst, hipStream_t st) {
  if (c.n <= 0) return hipSuccess;
  hipLaunchKernelGGL(write_table_kernel, dim3(1), dim3(64), 0, st, c, dst);
  return hipGetLastError();
}

}  // namespace muon
