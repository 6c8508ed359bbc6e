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
__device__ __forceinline__ void load8(const void* base, int64_t i, int bf16, float (&v)[8]) {
  if (bf16) {
    const uint4 w = *reinterpret_cast<const uint4*>(static_cast<const unsigned short*>(base) + i);
    const unsigned int ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v[2 * q] = __uint_as_float(ws[q] << 16);
      v[2 * q + 1] = __uint_as_float(ws[q] & 0xFFFF0000u);
    }
  } else {
    const float4* f = reinterpret_cast<const float4*>(static_cast<const float*>(base) + i);
    const float4 a = f[0], b = f[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
}
__device__ __forceinline__ void store8(void* base, int64_t i, int bf16, const float (&v)[8]) {
  if (bf16) {
    unsigned int w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
      w[q] = static_cast<unsigned int>(f32_to_bf16(v[2 * q])) |
             (static_cast<unsigned int>(f32_to_bf16(v[2 * q + 1])) << 16);
    *reinterpret_cast<uint4*>(static_cast<unsigned short*>(base) + i) = make_uint4(w[0], w[1], w[2], w[3]);
  } else {
    float4* f = reinterpret_cast<float4*>(static_cast<float*>(base) + i);
    f[0] = make_float4(v[0], v[1], v[2], v[3]);
    f[1] = make_float4(v[4], v[5], v[6], v[7]);
  }
}
// Value as it will be stored (rounded to bf16 if the store is bf16).
__device__ __forceinline__ float round_as(float v, int bf16) {
  return bf16 ? bf16_to_f32(f32_to_bf16(v)) : v;
}

__global__ __launch_bounds__(kThreads) void momentum_kernel(const MomentumParams p) {
  __shared__ float tile[kTile][kTile + 1];
  __shared__ float wsum[kThreads / 64];

  const int mat = blockIdx.y;
  const int t = blockIdx.x;
  const int ti = t / p.tiles_n, tj = t % p.tiles_n;
  const int i0 = ti * kTile, j0 = tj * kTile;   // canonical tile origin
  const MatDesc d = p.table[mat];
  const int tid = threadIdx.x;
  const int cr = tid >> 3;          // local row within a pass
  const int cc = (tid & 7) * 8;     // local first column (8 consecutive)

  // Phase 1: walk the tile in the STORED layout (coalesced along stored columns).
  // Stored rows of this tile: canonical rows if not transposed, else canonical columns.
  const int64_t srow0 = d.transposed ? j0 : i0;
  const int64_t scol0 = d.transposed ? i0 : j0;
  // 16-byte accesses when every row start is 16-byte aligned (row length a multiple of
  // 8 elements and aligned base pointers); otherwise element by element.
  const bool vec_ok = (d.cols % 8) == 0 && (reinterpret_cast<uintptr_t>(d.G) % 16) == 0 &&
                      (reinterpret_cast<uintptr_t>(d.M) % 16) == 0;
#pragma unroll
  for (int pass = 0; pass < kTile / 32; ++pass) {
    const int lr = cr + pass * 32;
    const int64_t sr = srow0 + lr;
    const int64_t sc0 = scol0 + cc;
    if (vec_ok && sr < d.rows && sc0 + 8 <= d.cols) {
      const int64_t idx = sr * d.cols + sc0;
      float g[8], m[8];
      load8(d.G, idx, p.g_bf16, g);
      load8(d.M, idx, p.m_bf16, m);
      float mn[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        mn[e] = p.mu * m[e] + g[e];
        tile[lr][cc + e] = p.nesterov ? g[e] + p.mu * mn[e] : mn[e];
      }
      store8(d.M, idx, p.m_bf16, mn);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int64_t sc = sc0 + e;
        float u = 0.0f;
        if (sr < d.rows && sc < d.cols) {
          const int64_t idx = sr * d.cols + sc;
          const float g = load_elem(d.G, idx, p.g_bf16);
          const float m = load_elem(d.M, idx, p.m_bf16);
          const float mn = p.mu * m + g;
          store_elem(d.M, idx, mn, p.m_bf16);
          u = p.nesterov ? g + p.mu * mn : mn;
        }
        tile[lr][cc + e] = u;
      }
    }
  }
  __syncthreads();

  // Phase 2: write U in the canonical layout (coalesced along canonical columns),
  // including the zero padding up to Mp x Np; sum the squares of the stored values.
  float sq = 0.0f;
  const char* ub = static_cast<const char*>(p.U);
#pragma unroll
  for (int pass = 0; pass < kTile / 32; ++pass) {
    const int lr = cr + pass * 32;
    const int64_t gi = i0 + lr;
    if (gi >= p.Mp) continue;
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float u = d.transposed ? tile[cc + e][lr] : tile[lr][cc + e];
      v[e] = round_as(u, p.u_bf16);
      sq += v[e] * v[e];
    }
    const int64_t gj = j0 + cc;
    if (gj >= p.Np) continue;
    const int64_t off = static_cast<int64_t>(mat) * p.sU + gi * p.ldu + gj;
    if (p.u_bf16) {
      unsigned int w[4];
#pragma unroll
      for (int q = 0; q < 4; ++q)
        w[q] = static_cast<unsigned int>(f32_to_bf16(v[2 * q])) |
               (static_cast<unsigned int>(f32_to_bf16(v[2 * q + 1])) << 16);
      *reinterpret_cast<uint4*>(const_cast<char*>(ub) + off * 2) = make_uint4(w[0], w[1], w[2], w[3]);
    } else {
      float4* dst = reinterpret_cast<float4*>(const_cast<char*>(ub) + off * 4);
      dst[0] = make_float4(v[0], v[1], v[2], v[3]);
      dst[1] = make_float4(v[4], v[5], v[6], v[7]);
    }
  }

  // Block partial of sum(u^2): wavefront butterfly, then the 4 wave sums in order.
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) sq += __shfl_xor(sq, off, 64);
  if ((tid & 63) == 0) wsum[tid >> 6] = sq;
  __syncthreads();
  if (tid == 0) {
    const float total = (wsum[0] + wsum[1]) + (wsum[2] + wsum[3]);
    p.partials[static_cast<int64_t>(mat) * (p.tiles_m * p.tiles_n) + t] = total;
  }
}

__global__ __launch_bounds__(256) void norm_finalize_kernel(const float* partials, int per_matrix,
                                                            float eps, float* s) {
  __shared__ double red[256];
  const int mat = blockIdx.x;
  const float* src = partials + static_cast<int64_t>(mat) * per_matrix;
  // Partials i = tid, tid + 256, ... are added in that order; their loads are issued
  // eight at a time (the partials come from every XCD's workgroups, so each load goes
  // past this XCD's L2), and the zero padding past the end leaves the sum unchanged.
  double acc = 0.0;
  for (int base = threadIdx.x; base < per_matrix; base += 256 * 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = base + u * 256;
      v[u] = i < per_matrix ? src[i] : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) acc += static_cast<double>(v[u]);
  }
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) s[mat] = static_cast<float>(1.0 / (sqrt(red[0]) + static_cast<double>(eps)));
}

// 64 x 64 tile transpose through LDS: coalesced reads of U rows, coalesced writes of
// X^T rows; the value is scaled by scale * s[mat] and converted (bf16 -> fp16 path).
__global__ __launch_bounds__(kThreads) void transpose_scale_kernel(const TransposeParams p) {
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
  for (int pass = 0; pass < kTile / 32; ++pass) {
    const int lr = cr + pass * 32;
    float v[8];
    load8(p.U, ubase + static_cast<int64_t>(i0 + lr) * p.Np + j0 + cc, p.u_bf16, v);
#pragma unroll
    for (int e = 0; e < 8; ++e) tile[lr][cc + e] = v[e] * sc;
  }
  __syncthreads();
  const int64_t xbase = static_cast<int64_t>(mat) * p.sXT;
#pragma unroll
  for (int pass = 0; pass < kTile / 32; ++pass) {
    const int lr = cr + pass * 32;   // row of X^T = column of U
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
  hipLaunchKernelGGL(momentum_kernel, grid, dim3(kThreads), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_norm_finalize(const float* partials, int per_matrix, int count, float eps,
                                float* s, hipStream_t st) {
  if (count <= 0) return hipSuccess;
  hipLaunchKernelGGL(norm_finalize_kernel, dim3(count), dim3(256), 0, st, partials, per_matrix, eps, s);
  return hipGetLastError();
}

hipError_t launch_transpose_scale(const TransposeParams& p, hipStream_t st) {
  if (p.count <= 0) return hipSuccess;
  dim3 grid((p.Mp / kTile) * (p.Np / kTile), p.count);
  hipLaunchKernelGGL(transpose_scale_kernel, grid, dim3(kThreads), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_write_table(const TableChunk& c, MatDesc* dst, hipStream_t st) {
  if (c.n <= 0) return hipSuccess;
  hipLaunchKernelGGL(write_table_kernel, dim3(1), dim3(64), 0, st, c, dst);
  return hipGetLastError();
}

}  // namespace muon
