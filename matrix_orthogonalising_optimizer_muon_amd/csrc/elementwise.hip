// HBM-bound stages of the update: momentum + Nesterov look-ahead, the Frobenius norm, and
// the normalised iterate in the canonical (short side first) orientation.
//
// MuonX article, section 2: Muon first smooths the gradient with momentum, then
// orthogonalises; the momentum form (heavy-ball sum, Nesterov look-ahead
// U = G + mu*M') and the normalisation X0 = U / (||U||_F + eps) are the plain readings of
// the pages. Two passes over G and M: the first only sums U^2 (per-workgroup partials from
// wavefront shuffles, then one fixed-order fp64 pass per matrix: deterministic); the
// second stores M' and rounds X0 once, from the fp32 U, to the iterate's storage type.
// Rounding U to a 16-bit type before the norm is known would add an error of the size of
// that type's half ulp to every element, which Newton-Schulz amplifies in the small
// singular directions of a low-rank-plus-noise gradient.
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
// The momentum update of 8 stored elements: mn = mu m + g (the new momentum) and the
// Nesterov look-ahead u = g + mu mn (or u = mn). Both passes evaluate exactly this, so the
// norm pass sums the squares of the same fp32 values the iterate pass scales.
struct Mom8 {
  float mn[8], u[8];
};
__device__ __forceinline__ Mom8 momentum8(const MomentumParams& p, const float (&g)[8], const float (&m)[8]) {
  Mom8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    r.mn[e] = p.mu * m[e] + g[e];
    r.u[e] = p.nesterov ? g[e] + p.mu * r.mn[e] : r.mn[e];
  }
  return r;
}

// Pass 1: partial sums of U^2 over blocks of UB * kNormBlock consecutive stored elements
// (the sum does not depend on the layout, so the stored matrix is read as one flat array:
// UB groups of 8 elements per thread, all loads of a thread issued before its arithmetic,
// 16-byte loads when the base pointers allow). Wavefront butterfly, then the 8 wave sums
// in a fixed order: deterministic. UB = 4 for groups that stream G and M past the caches
// (7B list's 3584 x 18944 group 4.29 -> 3.69 ms, 6.2 TB/s); UB = 1 for the small ones,
// which need the workgroups (2560 x 9728: 25.1 us against 27.3 with UB = 4).
constexpr int kNormThreads = kNormBlock / 8;
template <int UB>
__global__ __launch_bounds__(kNormThreads) void momentum_norm_kernel(const MomentumParams p) {
  __shared__ float wsum[kNormThreads / 64];
  const int mat = blockIdx.y;
  const int t = blockIdx.x;
  const MatDesc d = p.inl.n > 0 ? p.inl.d[mat] : p.table[mat];
  if (p.inl.n > 0 && blockIdx.x == 0 && threadIdx.x == 0) p.table_out[mat] = d;
  const int tid = threadIdx.x;
  const int64_t numel = d.rows * d.cols;
  const bool al = (reinterpret_cast<uintptr_t>(d.G) % 16) == 0 && (reinterpret_cast<uintptr_t>(d.M) % 16) == 0;
  float g[UB][8], m[UB][8];
#pragma unroll
  for (int b = 0; b < UB; ++b) {
    const int64_t e0 = (static_cast<int64_t>(t) * UB + b) * kNormBlock + tid * 8;
    const bool vec = al && e0 + 8 <= numel;
    if (vec && p.keep_gm) {
      load8<false>(d.G, e0, p.g_bf16, g[b]);
      load8<false>(d.M, e0, p.m_bf16, m[b]);
    } else if (vec) {
      load8<true>(d.G, e0, p.g_bf16, g[b]);
      load8<true>(d.M, e0, p.m_bf16, m[b]);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const bool ok = e0 + e < numel;
        g[b][e] = ok ? load_elem(d.G, e0 + e, p.g_bf16) : 0.0f;
        m[b][e] = ok ? load_elem(d.M, e0 + e, p.m_bf16) : 0.0f;
      }
    }
  }
  float sq = 0.0f;
#pragma unroll
  for (int b = 0; b < UB; ++b) {
    const Mom8 r = momentum8(p, g[b], m[b]);
#pragma unroll
    for (int e = 0; e < 8; ++e) sq += r.u[e] * r.u[e];
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) sq += __shfl_xor(sq, off, 64);
  if ((tid & 63) == 0) wsum[tid >> 6] = sq;
  __syncthreads();
  if (tid == 0) {
    const float tot = ((wsum[0] + wsum[1]) + (wsum[2] + wsum[3])) + ((wsum[4] + wsum[5]) + (wsum[6] + wsum[7]));
    p.partials[static_cast<int64_t>(mat) * p.norm_blocks + t] = tot;
  }
}

// 8 iterate values (already scaled) at element offset off: fp16 or fp32.
__device__ __forceinline__ void store_x8(void* X, int64_t off, int f16, const float (&v)[8]) {
  if (f16) {
    unsigned int w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const _Float16 lo = static_cast<_Float16>(v[2 * q]), hi = static_cast<_Float16>(v[2 * q + 1]);
      w[q] = static_cast<unsigned int>(__builtin_bit_cast(unsigned short, lo)) |
             (static_cast<unsigned int>(__builtin_bit_cast(unsigned short, hi)) << 16);
    }
    *reinterpret_cast<uint4*>(static_cast<unsigned short*>(X) + off) = make_uint4(w[0], w[1], w[2], w[3]);
  } else {
    float4* dst = reinterpret_cast<float4*>(static_cast<float*>(X) + off);
    dst[0] = make_float4(v[0], v[1], v[2], v[3]);
    dst[1] = make_float4(v[4], v[5], v[6], v[7]);
  }
}

// Pass 2: TPW canonical 64 x 64 tiles of the padded iterate per workgroup. A tile is read
// in the STORED layout (coalesced along stored rows; the loads of all TPW tiles issued
// before any store), M' is stored back, and x = xscale * s * u goes out twice:
//   * in the stored layout straight from registers: for a matrix stored in canonical
//     orientation that is X (row-major), for a tall one (stored as the transpose) X^T;
//   * through an LDS tile, transposed, as the other layout.
// Tiles over the padding write zeros, so both layouts are zero outside m' x n'. TPW = 2 for
// the groups whose first pass streams (more loads in flight per thread: 7B list's 84-matrix
// pass 11.8 -> 10.7 ms and 9.73 -> 9.60 ms on two boxes, decoder 2048 x 8192 group 2.49 ->
// 2.38 ms, 2048^2 group 0.83 -> 0.73 ms); a past-the-end second tile (odd tile counts)
// loads the last tile again and stores nothing.
template <int TPW>
__global__ __launch_bounds__(kThreads) void momentum_x_kernel(const MomentumParams p) {
  __shared__ float tile[kTile][kTile + 1];
  const int mat = blockIdx.y;
  const MatDesc d = p.inl.n > 0 ? p.inl.d[mat] : p.table[mat];
  const int tid = threadIdx.x;
  const bool vec_ok = (d.cols % 8) == 0 && (reinterpret_cast<uintptr_t>(d.G) % 16) == 0 &&
                      (reinterpret_cast<uintptr_t>(d.M) % 16) == 0;
  const int ntiles = p.tiles_m * p.tiles_n;
  const int cr = tid >> 3;          // local row within a pass
  const int cc = (tid & 7) * 8;     // local first column (8 consecutive)
  const float sc = p.xscale * p.s[mat];
  void* direct = d.transposed ? p.XT : p.X;     // layout that follows the stored rows
  void* other = d.transposed ? p.X : p.XT;
  const int64_t ld_direct = d.transposed ? p.Mp : p.Np, ld_other = d.transposed ? p.Np : p.Mp;
  const int64_t base = static_cast<int64_t>(mat) * p.sX;

  float g[TPW][2][8], m[TPW][2][8];
  bool full[TPW][2];
  int64_t srow0[TPW], scol0[TPW];
  bool valid[TPW];
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    const int t0 = blockIdx.x * TPW + u;
    valid[u] = t0 < ntiles;
    const int t = valid[u] ? t0 : ntiles - 1;
    const int ti = t / p.tiles_n, tj = t % p.tiles_n;
    const int i0 = ti * kTile, j0 = tj * kTile;
    srow0[u] = d.transposed ? j0 : i0;
    scol0[u] = d.transposed ? i0 : j0;
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
      const int64_t sr = srow0[u] + cr + pass * 32;
      const int64_t sc0 = scol0[u] + cc;
      full[u][pass] = vec_ok && sr < d.rows && sc0 + 8 <= d.cols;
      if (full[u][pass]) {
        load8<true>(d.G, sr * d.cols + sc0, p.g_bf16, g[u][pass]);
        load8<true>(d.M, sr * d.cols + sc0, p.m_bf16, m[u][pass]);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const bool ok = sr < d.rows && sc0 + e < d.cols;
          g[u][pass][e] = ok ? load_elem(d.G, sr * d.cols + sc0 + e, p.g_bf16) : 0.0f;
          m[u][pass][e] = ok ? load_elem(d.M, sr * d.cols + sc0 + e, p.m_bf16) : 0.0f;
        }
      }
    }
  }
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    if (u > 0) __syncthreads();   // the previous tile's LDS reads are done
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
      const int lr = cr + pass * 32;
      const int64_t sr = srow0[u] + lr;
      const int64_t sc0 = scol0[u] + cc;
      const Mom8 r = momentum8(p, g[u][pass], m[u][pass]);
      if (valid[u]) {
        if (full[u][pass]) {
          store8<true>(d.M, sr * d.cols + sc0, p.m_bf16, r.mn);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (sr < d.rows && sc0 + e < d.cols) store_elem(d.M, sr * d.cols + sc0 + e, r.mn[e], p.m_bf16);
        }
      }
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        x[e] = sc * r.u[e];
        tile[lr][cc + e] = x[e];
      }
      if (valid[u]) store_x8(direct, base + (srow0[u] + lr) * ld_direct + scol0[u] + cc, p.x_f16, x);
    }
    __syncthreads();
    if (valid[u]) {
#pragma unroll
      for (int pass = 0; pass < 2; ++pass) {
        const int lr = cr + pass * 32;
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = tile[cc + e][lr];
        const int64_t off = (scol0[u] + lr) * ld_other + srow0[u] + cc;
        store_x8(other, base + off, p.x_f16, v);
      }
    }
  }
}

// Dry-run iterate: each thread writes 8 consecutive elements of X (row-major) and 8 of X^T,
// computing every value from its canonical position, so both layouts agree exactly.
__global__ __launch_bounds__(kThreads) void dry_x_kernel(const MomentumParams p) {
  const int mat = blockIdx.y;
  const int t = blockIdx.x;
  const int ti = t / p.tiles_n, tj = t % p.tiles_n;
  const int i0 = ti * kTile, j0 = tj * kTile;
  const int tid = threadIdx.x;
  const int cr = tid >> 3, cc = (tid & 7) * 8;
  const float sc = p.xscale * sqrtf(3.0f / (static_cast<float>(p.m) * static_cast<float>(p.n)));
  const int64_t base = static_cast<int64_t>(mat) * p.sX;
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int lr = cr + pass * 32;
    float v[8], w[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int r = i0 + lr, c = j0 + cc + e;            // X row i0 + lr
      v[e] = (r < p.m && c < p.n) ? sc * dry_u(mat, r, c) : 0.0f;
      const int r2 = i0 + cc + e, c2 = j0 + lr;          // X^T row j0 + lr
      w[e] = (r2 < p.m && c2 < p.n) ? sc * dry_u(mat, r2, c2) : 0.0f;
    }
    store_x8(p.X, base + static_cast<int64_t>(i0 + lr) * p.Np + j0 + cc, p.x_f16, v);
    store_x8(p.XT, base + static_cast<int64_t>(j0 + lr) * p.Mp + i0 + cc, p.x_f16, w);
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

__global__ void write_table_kernel(const TableChunk c, MatDesc* dst) {
  const int i = threadIdx.x;
  if (i < c.n) dst[i] = c.d[i];
}

}  // namespace

hipError_t launch_momentum_norm(const MomentumParams& p, hipStream_t st) {
  if (p.count <= 0 || p.norm_blocks <= 0) return hipSuccess;
  if (p.norm_ub == 4)
    hipLaunchKernelGGL(momentum_norm_kernel<4>, dim3(p.norm_blocks, p.count), dim3(kNormThreads), 0, st, p);
  else if (p.norm_ub == 1)
    hipLaunchKernelGGL(momentum_norm_kernel<1>, dim3(p.norm_blocks, p.count), dim3(kNormThreads), 0, st, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_momentum_x(const MomentumParams& p, hipStream_t st) {
  if (p.count <= 0) return hipSuccess;
  const int nt = p.tiles_m * p.tiles_n;
  if (p.norm_ub == 4)   // the large groups (G and M past the caches)
    hipLaunchKernelGGL(momentum_x_kernel<2>, dim3((nt + 1) / 2, p.count), dim3(kThreads), 0, st, p);
  else
    hipLaunchKernelGGL(momentum_x_kernel<1>, dim3(nt, p.count), dim3(kThreads), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_norm_finalize(const float* partials, int per_matrix, int count, float eps,
                                float* s, hipStream_t st) {
  if (count <= 0) return hipSuccess;
  hipLaunchKernelGGL(norm_finalize_kernel, dim3(count), dim3(kFinThreads), 0, st, partials, per_matrix, eps, s);
  return hipGetLastError();
}

hipError_t launch_dry_x(const MomentumParams& p, hipStream_t st) {
  if (p.count <= 0) return hipSuccess;
  hipLaunchKernelGGL(dry_x_kernel, dim3(p.tiles_m * p.tiles_n, p.count), dim3(kThreads), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_write_table(const TableChunk& c, MatDesc* dst, hipStream_t st) {
  if (c.n <= 0) return hipSuccess;
  hipLaunchKernelGGL(write_table_kernel, dim3(1), dim3(64), 0, st, c, dst);
  return hipGetLastError();
}

}  // namespace muon
